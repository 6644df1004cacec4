// Projection GEMMs of the step: C[M][N] = A[M][K] . B[N][K]^T (+ Res[M][N]).
// A = activation rows (X or O), B = output-major weight (linear layer), both
// K-contiguous, so MFMA operands load straight from global memory.
#include "dg_common.h"

namespace dg {

// bf16 path.  Computed as C^T = B . A^T on 32x32x16 MFMA tiles so that each
// lane ends up holding 4 consecutive output columns of one output row
// (8-byte stores).  Workgroup = 4 waves, tile 64 (m) x 64 (n), wave tile
// 32 x 32; the K loop is double-buffered in registers, 4 K-steps per stage.
constexpr int GU = 4;  // K-steps of 16 per stage

__global__ void __launch_bounds__(256) k_gemm_nt_bf16(int M, int N, int K, const u16* __restrict__ A,
                                                      const u16* __restrict__ B,
                                                      const u16* __restrict__ Res,
                                                      u16* __restrict__ C) {
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63, h = l >> 5, l32 = l & 31;
  const int m0 = blockIdx.y * 64 + (w >> 1) * 32;
  const int n0 = blockIdx.x * 64 + (w & 1) * 32;
  const int am = m0 + l32, bn = n0 + l32;
  const bool aok = am < M, bok = bn < N;
  const u16* ap = A + (size_t)(aok ? am : 0) * K + h * 8;
  const u16* bp = B + (size_t)(bok ? bn : 0) * K + h * 8;
  const u32x4 z4 = {0u, 0u, 0u, 0u};

  f32x16 acc = zero16();
  u32x4 xa[GU], wa[GU], xb[GU], wb[GU];
#pragma unroll
  for (int u = 0; u < GU; ++u) {
    xa[u] = aok ? ldg128(ap + u * 16) : z4;
    wa[u] = bok ? ldg128(bp + u * 16) : z4;
  }
  const int KS = 16 * GU;
  for (int k = 0; k < K; k += 2 * KS) {
    if (k + KS < K) {
#pragma unroll
      for (int u = 0; u < GU; ++u) {
        xb[u] = aok ? ldg128(ap + k + KS + u * 16) : z4;
        wb[u] = bok ? ldg128(bp + k + KS + u * 16) : z4;
      }
    }
#pragma unroll
    for (int u = 0; u < GU; ++u) acc = mfma32(wa[u], xa[u], acc);
    if (k + KS >= K) break;
    if (k + 2 * KS < K) {
#pragma unroll
      for (int u = 0; u < GU; ++u) {
        xa[u] = aok ? ldg128(ap + k + 2 * KS + u * 16) : z4;
        wa[u] = bok ? ldg128(bp + k + 2 * KS + u * 16) : z4;
      }
    }
#pragma unroll
    for (int u = 0; u < GU; ++u) acc = mfma32(wb[u], xb[u], acc);
  }
  if (!aok) return;
  // lane holds C[am][n0 + 8j + 4h + i], i = 0..3
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = n0 + 8 * j + 4 * h;
    if (n >= N) continue;
    float v[4] = {acc[4 * j], acc[4 * j + 1], acc[4 * j + 2], acc[4 * j + 3]};
    const size_t o = (size_t)am * N + n;
    if (n + 4 <= N) {
      if (Res) {
        u32x2 r = *(const u32x2*)(Res + o);
        v[0] += bf16_to_f32(r[0] & 0xFFFFu); v[1] += bf16_to_f32(r[0] >> 16);
        v[2] += bf16_to_f32(r[1] & 0xFFFFu); v[3] += bf16_to_f32(r[1] >> 16);
      }
      u32x2 out = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      *(u32x2*)(C + o) = out;
    } else {
      for (int i = 0; i < 4 && n + i < N; ++i) {
        float x = v[i];
        if (Res) x += bf16_to_f32(Res[o + i]);
        C[o + i] = (u16)f32_to_bf16(x);
      }
    }
  }
}

// fp32-storage path: classic 16x16 LDS-tiled GEMM accumulating in fp64 (one
// rounding of the stored output), sequential over K.
__global__ void __launch_bounds__(256) k_gemm_nt_f32(int M, int N, int K, const float* __restrict__ A,
                                                     const float* __restrict__ B,
                                                     const float* __restrict__ Res,
                                                     float* __restrict__ C) {
  __shared__ float As[16][17], Bs[16][17];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int m = blockIdx.y * 16 + ty, n = blockIdx.x * 16 + tx;
  double acc = 0.0;
  for (int k0 = 0; k0 < K; k0 += 16) {
    const int ka = k0 + tx;
    As[ty][tx] = (m < M && ka < K) ? A[(size_t)m * K + ka] : 0.f;
    const int nb = blockIdx.x * 16 + ty;
    Bs[ty][tx] = (nb < N && ka < K) ? B[(size_t)nb * K + ka] : 0.f;
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) acc = fma((double)As[ty][kk], (double)Bs[tx][kk], acc);
    __syncthreads();
  }
  if (m < M && n < N) {
    if (Res) acc += (double)Res[(size_t)m * N + n];
    C[(size_t)m * N + n] = (float)acc;
  }
}

hipError_t launch_gemm_nt(int dtype, int M, int N, int K, const void* A, const void* B,
                          const void* Res, void* C, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (dtype == 1) {
    dim3 grid((N + 63) / 64, (M + 63) / 64);
    hipLaunchKernelGGL(k_gemm_nt_bf16, grid, dim3(256), 0, s, M, N, K, (const u16*)A,
                       (const u16*)B, (const u16*)Res, (u16*)C);
  } else {
    dim3 grid((N + 15) / 16, (M + 15) / 16);
    hipLaunchKernelGGL(k_gemm_nt_f32, grid, dim3(256), 0, s, M, N, K, (const float*)A,
                       (const float*)B, (const float*)Res, (float*)C);
  }
  return hipGetLastError();
}

}  // namespace dg
