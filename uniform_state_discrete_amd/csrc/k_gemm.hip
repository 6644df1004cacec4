// Projection GEMMs of the step: C[M][N] = A[M][K] . B[N][K]^T (+ Res[M][N]).
// A = activation rows (X or O), B = output-major weight (linear layer), both
// K-contiguous, so MFMA operands load straight from global memory.
#include "dg_common.h"

namespace dg {

// bf16 path.  Output tile TM (m) x 64 (n), wave tile 32 x 32: 4 waves for
// TM = 64; 2 waves for TM = 32, which the host picks when 64-row tiles would
// leave CUs without a workgroup (256 rows of a 2048-wide output: 128 tiles
// of 64 x 64; 32-row tiles give 256 workgroups, 12.2 against 13.9 us).
// K advances in slices of 64 staged through LDS (double-buffered): 8 threads
// load one 128-byte row segment with 16-byte loads, so every global load
// instruction reads whole contiguous rows; global loads run four slices
// (64 or 48 KiB per workgroup) ahead of the products, enough bytes in flight
// to cover the latency of the weight stream from HBM.  Computed as
// C^T = B . A^T on 32x32x16 MFMA tiles (A operand: weight rows, B operand:
// activation rows, both read from LDS with one 16-byte read per lane), so
// each lane ends up holding 4 consecutive output columns of one output row
// (8-byte stores).  Two accumulators take alternate K-steps: two independent
// chains keep the matrix core busy.  Up to three (weight, output) segments
// share one launch (the Q, K and V projections read the same activations).
constexpr int GKS = 64, GLD = GKS + 8;  // K slice; LDS row of 144 bytes: conflict-free

// The cache copy of output element(s) of row am, columns n .. n+cnt-1 (within
// one head: dh is a multiple of 4 and n of 4): cache[b][g][L + i][e] with
// am = b Cn + i, n = g dh + e (the prefill-append's cache write, fused into
// the projection's epilogue).
__device__ __forceinline__ u16* cache_row(u16* cache, const CacheGeom& cg, int N, int am, int n) {
  const int b = am / cg.Cn, i = am - b * cg.Cn;
  const int g = n / cg.dh, e = n - g * cg.dh;
  return cache + (((size_t)b * (N / cg.dh) + g) * cg.cap + cg.L + i) * cg.dh + e;
}

template <int TM>
__global__ void __launch_bounds__(TM * 4) k_gemm_nt_bf16(int M, int K, const u16* __restrict__ A, GemmSeg s0,
                                                         GemmSeg s1, GemmSeg s2, u32x4* __restrict__ zp,
                                                         size_t zn16, CacheGeom cg) {
  static_assert(TM == 64 || TM == 32, "row tile of 64 (4 waves) or 32 (2 waves)");
  constexpr int RS = TM / 2;                 // rows per loader pass: 8 threads per 128-byte row segment
  constexpr int JA = TM / RS, JB = 64 / RS;  // loader passes over the A and B tiles
  if (zp) {
    // a region a later kernel needs zeroed, spread over every thread of the grid
    const size_t nth = (size_t)gridDim.x * gridDim.y * blockDim.x;
    for (size_t i = ((size_t)blockIdx.y * gridDim.x + blockIdx.x) * blockDim.x + threadIdx.x; i < zn16; i += nth)
      zp[i] = u32x4{0u, 0u, 0u, 0u};
  }
  __shared__ __attribute__((aligned(16))) u16 As[2][TM][GLD];
  __shared__ __attribute__((aligned(16))) u16 Bs[2][64][GLD];
  int tile = blockIdx.x;
  GemmSeg sg = s0;
  if (tile >= s0.tiles) {
    tile -= s0.tiles;
    sg = s1;
    if (tile >= s1.tiles) {
      tile -= s1.tiles;
      sg = s2;
    }
  }
  const int N = sg.N;
  const u16* __restrict__ B = sg.B;
  const int m0 = blockIdx.y * TM, n0 = tile * 64;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, h = l >> 5, l32 = l & 31;
  const int lr = tid >> 3, lc = (tid & 7) * 8;  // loader: rows lr + RS j; columns lc .. lc+7
  const int nk = K / GKS;                       // K is a multiple of 64
  // Buffer resources end at the operands: rows past M or N load zeros, with
  // no branch around the loads.
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(const_cast<u16*>(A), (short)0,
                                                                      (int)((size_t)M * K * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(const_cast<u16*>(B), (short)0,
                                                                      (int)((size_t)N * K * 2), 0x00020000);
  const uint32_t oa = (uint32_t)(((size_t)(m0 + lr) * K + lc) * 2), ob = (uint32_t)(((size_t)(n0 + lr) * K + lc) * 2);
  const uint32_t rowRS = (uint32_t)(RS * K * 2);
  constexpr int GPF = 4;           // slices in flight
  u32x4 ga[GPF][JA], gb[GPF][JB];  // [slot][loader pass]
  auto gload = [&](int slot, int ks) {
    const uint32_t k2 = (uint32_t)(ks * GKS * 2);
#pragma unroll
    for (int j = 0; j < JA; ++j)
      ga[slot][j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ra, oa + j * rowRS + k2, 0, 0));
#pragma unroll
    for (int j = 0; j < JB; ++j)
      gb[slot][j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rb, ob + j * rowRS + k2, 0, 0));
  };
  auto lstore = [&](int slot, int buf) {
#pragma unroll
    for (int j = 0; j < JA; ++j) *(DG_LDS u32x4*)&As[buf][lr + RS * j][lc] = ga[slot][j];
#pragma unroll
    for (int j = 0; j < JB; ++j) *(DG_LDS u32x4*)&Bs[buf][lr + RS * j][lc] = gb[slot][j];
  };
  f32x16 acc0 = zero16(), acc1 = zero16();
  const int wm = TM == 64 ? (w >> 1) * 32 : 0, wn = TM == 64 ? (w & 1) * 32 : w * 32;
#pragma unroll
  for (int s = 0; s < GPF; ++s) gload(s, s);
  lstore(0, 0);
  __syncthreads();
  // one slice: products from LDS buffer (slot & 1), prefetch of slice
  // ks + GPF into the register slot just emptied, the next slice to LDS
  auto slice = [&](int u, int ks) {
    const int buf = u & 1;
    gload(u, ks + GPF);  // slot u's slice went to LDS in the last iteration
#pragma unroll
    for (int kk = 0; kk < GKS / 16; ++kk) {
      const u32x4 a = *(const DG_LDS u32x4*)&Bs[buf][wn + l32][kk * 16 + 8 * h];
      const u32x4 b = *(const DG_LDS u32x4*)&As[buf][wm + l32][kk * 16 + 8 * h];
      if (kk & 1)
        acc1 = mfma32(a, b, acc1);
      else
        acc0 = mfma32(a, b, acc0);
    }
    if (ks + 1 < nk) lstore((u + 1) & (GPF - 1), buf ^ 1);
    __syncthreads();
  };
  // unrolled by GPF so that every register slot index is a constant; slices
  // past the end are loaded (in bounds of the resource) but never stored
  const int nfull = nk & ~(GPF - 1);
  for (int ks0 = 0; ks0 < nfull; ks0 += GPF) {
#pragma unroll
    for (int u = 0; u < GPF; ++u) slice(u, ks0 + u);
  }
#pragma unroll
  for (int u = 0; u < GPF - 1; ++u)
    if (nfull + u < nk) slice(u, nfull + u);
  const int am = m0 + wm + l32;
  if (am >= M) return;
  const u16* __restrict__ Res = sg.Res;
  u16* __restrict__ C = sg.C;
  // lane holds C[am][n0 + wn + 8j + 4h + i], i = 0..3
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = n0 + wn + 8 * j + 4 * h;
    if (n >= N) continue;
    float v[4] = {acc0[4 * j] + acc1[4 * j], acc0[4 * j + 1] + acc1[4 * j + 1], acc0[4 * j + 2] + acc1[4 * j + 2],
                  acc0[4 * j + 3] + acc1[4 * j + 3]};
    const size_t o = (size_t)am * N + n;
    if (n + 4 <= N) {
      if (Res) {
        u32x2 r = *(const u32x2*)(Res + o);
        v[0] += bf16_to_f32(r[0] & 0xFFFFu); v[1] += bf16_to_f32(r[0] >> 16);
        v[2] += bf16_to_f32(r[1] & 0xFFFFu); v[3] += bf16_to_f32(r[1] >> 16);
      }
      u32x2 out = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      *(u32x2*)(C + o) = out;
      if (sg.cache) *(u32x2*)cache_row(sg.cache, cg, N, am, n) = out;
    } else {
      for (int i = 0; i < 4 && n + i < N; ++i) {
        float x = v[i];
        if (Res) x += bf16_to_f32(Res[o + i]);
        C[o + i] = (u16)f32_to_bf16(x);
        if (sg.cache) *cache_row(sg.cache, cg, N, am, n + i) = (u16)f32_to_bf16(x);
      }
    }
  }
}

// bf16 path for many rows (M >= 1024: prompt prefill, many canvases): output
// tile 128 x 128, wave tile 64 x 64 (2 x 2 products of 32 x 32 per 16-deep K
// step).  Per K slice a wave reads 16 KiB of LDS for 16 products, half the
// LDS bytes per product of the 64 x 64 tile, whose waves are bound by LDS
// reads at large M.  Same operand layout, loads and epilogue convention;
// two slices in flight through registers.
__global__ void __launch_bounds__(256) k_gemm_nt_bf16_t128(int M, int K, const u16* __restrict__ A, GemmSeg s0,
                                                           GemmSeg s1, GemmSeg s2, u32x4* __restrict__ zp,
                                                           size_t zn16, CacheGeom cg) {
  if (zp) {
    const size_t nth = (size_t)gridDim.x * gridDim.y * blockDim.x;
    for (size_t i = ((size_t)blockIdx.y * gridDim.x + blockIdx.x) * blockDim.x + threadIdx.x; i < zn16; i += nth)
      zp[i] = u32x4{0u, 0u, 0u, 0u};
  }
  __shared__ __attribute__((aligned(16))) u16 As[2][128][GLD];
  __shared__ __attribute__((aligned(16))) u16 Bs[2][128][GLD];
  int tile = blockIdx.x;
  GemmSeg sg = s0;
  if (tile >= s0.tiles) {
    tile -= s0.tiles;
    sg = s1;
    if (tile >= s1.tiles) {
      tile -= s1.tiles;
      sg = s2;
    }
  }
  const int N = sg.N;
  const u16* __restrict__ B = sg.B;
  const int m0 = blockIdx.y * 128, n0 = tile * 128;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, h = l >> 5, l32 = l & 31;
  const int lr = tid >> 3, lc = (tid & 7) * 8;  // loader: rows lr + 32 j (j < 4); columns lc .. lc+7
  const int nk = K / GKS;                       // K is a multiple of 64
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(const_cast<u16*>(A), (short)0,
                                                                      (int)((size_t)M * K * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(const_cast<u16*>(B), (short)0,
                                                                      (int)((size_t)N * K * 2), 0x00020000);
  const uint32_t oa = (uint32_t)(((size_t)(m0 + lr) * K + lc) * 2), ob = (uint32_t)(((size_t)(n0 + lr) * K + lc) * 2);
  const uint32_t row32 = (uint32_t)(32 * K * 2);
  u32x4 ga[2][4], gb[2][4];  // [slot][row group]
  auto gload = [&](int slot, int ks) {
    const uint32_t k2 = (uint32_t)(ks * GKS * 2);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ga[slot][j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ra, oa + j * row32 + k2, 0, 0));
      gb[slot][j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rb, ob + j * row32 + k2, 0, 0));
    }
  };
  auto lstore = [&](int slot, int buf) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      *(DG_LDS u32x4*)&As[buf][lr + 32 * j][lc] = ga[slot][j];
      *(DG_LDS u32x4*)&Bs[buf][lr + 32 * j][lc] = gb[slot][j];
    }
  };
  f32x16 acc[2][2] = {{zero16(), zero16()}, {zero16(), zero16()}};  // [m half][n half]
  const int wm = (w >> 1) * 64, wn = (w & 1) * 64;
  gload(0, 0);
  gload(1, 1);
  lstore(0, 0);
  __syncthreads();
  // slice ks: products from LDS buffer u (= slot u), slot u refilled with
  // slice ks + 2, slice ks + 1 (slot u ^ 1) to the other LDS buffer
  auto slice = [&](int u, int ks) {
    gload(u, ks + 2);
#pragma unroll
    for (int kk = 0; kk < GKS / 16; ++kk) {
      u32x4 a[2], b[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        a[q] = *(const DG_LDS u32x4*)&Bs[u][wn + 32 * q + l32][kk * 16 + 8 * h];
        b[q] = *(const DG_LDS u32x4*)&As[u][wm + 32 * q + l32][kk * 16 + 8 * h];
      }
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) acc[mi][ni] = mfma32(a[ni], b[mi], acc[mi][ni]);
    }
    if (ks + 1 < nk) lstore(u ^ 1, u ^ 1);
    __syncthreads();
  };
  // unrolled by 2 so that the slot indexes are constants; slices past the
  // end are loaded (in bounds of the resource) but never stored
  const int nfull = nk & ~1;
  for (int ks0 = 0; ks0 < nfull; ks0 += 2) {
    slice(0, ks0);
    slice(1, ks0 + 1);
  }
  if (nfull < nk) slice(0, nfull);
  const u16* __restrict__ Res = sg.Res;
  u16* __restrict__ C = sg.C;
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) {
    const int am = m0 + wm + 32 * mi + l32;
    if (am >= M) continue;
    // lane holds C[am][n0 + wn + 32 ni + 8j + 4h + i], i = 0..3
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int n = n0 + wn + 32 * ni + 8 * j + 4 * h;
        if (n >= N) continue;
        float v[4] = {acc[mi][ni][4 * j], acc[mi][ni][4 * j + 1], acc[mi][ni][4 * j + 2], acc[mi][ni][4 * j + 3]};
        const size_t o = (size_t)am * N + n;
        if (n + 4 <= N) {
          if (Res) {
            u32x2 r = *(const u32x2*)(Res + o);
            v[0] += bf16_to_f32(r[0] & 0xFFFFu); v[1] += bf16_to_f32(r[0] >> 16);
            v[2] += bf16_to_f32(r[1] & 0xFFFFu); v[3] += bf16_to_f32(r[1] >> 16);
          }
          u32x2 out = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
          *(u32x2*)(C + o) = out;
          if (sg.cache) *(u32x2*)cache_row(sg.cache, cg, N, am, n) = out;
        } else {
          for (int i = 0; i < 4 && n + i < N; ++i) {
            float x = v[i];
            if (Res) x += bf16_to_f32(Res[o + i]);
            C[o + i] = (u16)f32_to_bf16(x);
            if (sg.cache) *cache_row(sg.cache, cg, N, am, n + i) = (u16)f32_to_bf16(x);
          }
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

// Row count from which the 128 x 128 tile kernel runs.
constexpr int kGemmBigM = 1024;
// Below it, 64 x 64 tiles unless they leave CUs of an MI355X (256) without a
// workgroup: then 32 x 64 tiles with two waves each.
constexpr int kGemmFill = 256;

static hipError_t launch_gemm_small(int M, int K, const void* A, const GemmSeg& s0, const GemmSeg& s1,
                                    const GemmSeg& s2, void* zero, size_t zero_bytes, const CacheGeom& cg,
                                    hipStream_t s) {
  const int tiles = s0.tiles + s1.tiles + s2.tiles;
  if ((size_t)tiles * (size_t)((M + 63) / 64) >= (size_t)kGemmFill) {
    hipLaunchKernelGGL(k_gemm_nt_bf16<64>, dim3((unsigned)tiles, (M + 63) / 64), dim3(256), 0, s, M, K,
                       (const u16*)A, s0, s1, s2, (u32x4*)zero, zero_bytes / 16, cg);
  } else {
    hipLaunchKernelGGL(k_gemm_nt_bf16<32>, dim3((unsigned)tiles, (M + 31) / 32), dim3(128), 0, s, M, K,
                       (const u16*)A, s0, s1, s2, (u32x4*)zero, zero_bytes / 16, cg);
  }
  return hipGetLastError();
}

static GemmSeg gemm_seg(const void* B, const void* Res, void* C, int N, int tn, void* cache = nullptr) {
  return GemmSeg{(const u16*)B, (const u16*)Res, (u16*)C, N, (N + tn - 1) / tn, (u16*)cache};
}

hipError_t launch_gemm_nt(int dtype, int M, int N, int K, const void* A, const void* B,
                          const void* Res, void* C, hipStream_t s, void* zero, size_t zero_bytes) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (dtype == 1) {
    const int tn = M >= kGemmBigM ? 128 : 64;
    const GemmSeg s0 = gemm_seg(B, Res, C, N, tn), none = GemmSeg{nullptr, nullptr, nullptr, 0, 0, nullptr};
    const CacheGeom cg{1, 0, 1, 1};
    if (tn != 128) return launch_gemm_small(M, K, A, s0, none, none, zero, zero_bytes, cg, s);
    dim3 grid((unsigned)s0.tiles, (M + tn - 1) / tn);
    hipLaunchKernelGGL(k_gemm_nt_bf16_t128, grid, dim3(256), 0, s, M, K, (const u16*)A, s0, none, none,
                       (u32x4*)zero, zero_bytes / 16, cg);
  } else {
    dim3 grid((N + 15) / 16, (M + 15) / 16);
    hipLaunchKernelGGL(k_gemm_nt_f32, grid, dim3(256), 0, s, M, N, K, (const float*)A,
                       (const float*)B, (const float*)Res, (float*)C);
  }
  return hipGetLastError();
}

hipError_t launch_gemm_qkv(int dtype, int M, int K, const void* A, const void* Wq, int Nq, void* Q,
                           const void* Wk, const void* Wv, int Nkv, void* Kn, void* Vn, hipStream_t s,
                           void* k_cache, void* v_cache, CacheGeom g) {
  if (M <= 0) return hipSuccess;
  if (dtype != 1) {
    hipError_t e = launch_gemm_nt(dtype, M, Nq, K, A, Wq, nullptr, Q, s);
    if (e == hipSuccess) e = launch_gemm_nt(dtype, M, Nkv, K, A, Wk, nullptr, Kn, s);
    if (e == hipSuccess) e = launch_gemm_nt(dtype, M, Nkv, K, A, Wv, nullptr, Vn, s);
    if (e == hipSuccess && k_cache)
      e = launch_cache_append(dtype, M / g.Cn, g.Cn, g.L, g.cap, Nkv / g.dh, g.dh, Kn, k_cache, s);
    if (e == hipSuccess && v_cache)
      e = launch_cache_append(dtype, M / g.Cn, g.Cn, g.L, g.cap, Nkv / g.dh, g.dh, Vn, v_cache, s);
    return e;
  }
  const int tn = M >= kGemmBigM ? 128 : 64;
  const GemmSeg sq = gemm_seg(Wq, nullptr, Q, Nq, tn), sk = gemm_seg(Wk, nullptr, Kn, Nkv, tn, k_cache),
                sv = gemm_seg(Wv, nullptr, Vn, Nkv, tn, v_cache);
  if (tn != 128) return launch_gemm_small(M, K, A, sq, sk, sv, nullptr, 0, g, s);
  dim3 grid((unsigned)(sq.tiles + sk.tiles + sv.tiles), (M + tn - 1) / tn);
  hipLaunchKernelGGL(k_gemm_nt_bf16_t128, grid, dim3(256), 0, s, M, K, (const u16*)A, sq, sk, sv, nullptr,
                     (size_t)0, g);
  return hipGetLastError();
}

}  // namespace dg
