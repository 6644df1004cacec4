// Small kernels of the denoise step: assemble X = H + E[x] + S, uniform-state
// renoise with Philox4x64-10, and the cache append of a finished block.
#include "dg_common.h"

namespace dg {

// ---------------------------------------------------------------------------
// Assemble: X[r] = H[r] + E[x_r] + S[r] (S may be NULL).  The denoiser reads
// the canvas tokens' embeddings on top of the hidden rows plus the
// self-conditioning vector handed over from the previous step
// (DiffusionGemma explainer, "Autocondizionamento").  One rounding to the
// storage type (bf16: fp32 sum; fp32: fp64 sum).  One workgroup per row.
// bf16 reads the token's row from the tiled table (the only copy of E the
// bf16 path keeps): columns 32c + 8g .. +7 of id 16 vb + i are the 16 bytes at
// lane position 16 g + i of 1 KiB block (vb, c), the two 8-byte halves
// swapped for odd g.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) k_assemble_bf16(int d, int V, const u16* __restrict__ H,
                                                       const u16* __restrict__ Et,
                                                       const int32_t* __restrict__ x,
                                                       const u16* __restrict__ S,
                                                       u16* __restrict__ X) {
  const int r = blockIdx.x;
  int tok = x[r];
  if (tok < 0 || tok >= V) tok = 0;
  const size_t ro = (size_t)r * d;
  const size_t vb = (size_t)(tok >> 4) * (d >> 5), id = (size_t)(tok & 15);
  for (int e = threadIdx.x * 8; e < d; e += 256 * 8) {
    const int c = e >> 5, g = (e >> 3) & 3;
    u32x4 h = ldg128(H + ro + e);
    u32x4 em = ldg128(Et + (vb + c) * 512 + 8 * (16 * g + id));
    if (g & 1) em = u32x4{em[2], em[3], em[0], em[1]};
    u32x4 s = {0u, 0u, 0u, 0u};
    if (S) s = ldg128(S + ro + e);
    u32x4 o;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float lo = bf16_to_f32(h[k] & 0xFFFFu) + bf16_to_f32(em[k] & 0xFFFFu) + bf16_to_f32(s[k] & 0xFFFFu);
      float hi = bf16_to_f32(h[k] >> 16) + bf16_to_f32(em[k] >> 16) + bf16_to_f32(s[k] >> 16);
      o[k] = pack_bf16x2(lo, hi);
    }
    *(u32x4*)(X + ro + e) = o;
  }
}

__global__ void __launch_bounds__(256) k_assemble_f32(int d, int V, const float* __restrict__ H,
                                                      const float* __restrict__ E,
                                                      const int32_t* __restrict__ x,
                                                      const float* __restrict__ S,
                                                      float* __restrict__ X) {
  const int r = blockIdx.x;
  int tok = x[r];
  if (tok < 0 || tok >= V) tok = 0;
  const size_t ro = (size_t)r * d;
  const size_t eo = (size_t)tok * d;
  for (int e = threadIdx.x; e < d; e += 256) {
    double v = (double)H[ro + e] + (double)E[eo + e];
    if (S) v += (double)S[ro + e];
    X[ro + e] = (float)v;
  }
}

hipError_t launch_assemble(int dtype, int R, int d, int V, const void* H, const void* E,
                           const int32_t* x, const void* S, void* X, hipStream_t s) {
  if (R <= 0) return hipSuccess;
  if (dtype == 1)
    hipLaunchKernelGGL(k_assemble_bf16, dim3(R), dim3(256), 0, s, d, V, (const u16*)H,
                       (const u16*)E, x, (const u16*)S, (u16*)X);
  else
    hipLaunchKernelGGL(k_assemble_f32, dim3(R), dim3(256), 0, s, d, V, (const float*)H,
                       (const float*)E, x, (const float*)S, (float*)X);
  return hipGetLastError();
}

// Uniform-state renoise (explainer, "Diffusione dello stato uniforme"): a
// position whose confidence is below tau gets a fresh uniform vocabulary
// token; the others take the argmax.  conf == NULL draws every position
// (a block's initial canvas).  Token = floor(w0 * V / 2^64).
__global__ void k_renoise(int rows, int canvas, int V, const int32_t* __restrict__ argmax,
                          const float* __restrict__ conf, float tau, uint64_t seed, uint32_t t,
                          uint32_t block, int32_t* __restrict__ out, uint8_t* __restrict__ mask) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= rows) return;
  const RenoiseArgs rn{out, mask, tau, seed, t, block, canvas, V};
  if (conf == nullptr) {
    // every position draws (conf = -inf is below any tau)
    renoise_row(rn, r, 0, -INFINITY);
    return;
  }
  renoise_row(rn, r, argmax[r], conf[r]);
}
hipError_t launch_renoise(int rows, int canvas, int V, const int32_t* argmax, const float* conf,
                          float tau, uint64_t seed, uint32_t t, uint32_t block, int32_t* out,
                          uint8_t* mask, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_renoise, dim3((rows + 255) / 256), dim3(256), 0, s, rows, canvas, V,
                     argmax, conf, tau, seed, t, block, out, mask);
  return hipGetLastError();
}

// Masked diffusion (explainer, "Diffusione mascherata"): a position holding
// the mask id takes the model's prediction when the confidence meets tau and
// the prediction is not the mask id itself; every other position keeps its
// token, so a committed token is locked.  in == NULL writes a fully masked
// canvas.  commit (may be NULL) flags the positions unmasked by this call.
__global__ void k_unmask(int rows, const int32_t* __restrict__ argmax, const float* __restrict__ conf,
                         float tau, int32_t mask_id, const int32_t* in, int32_t* out,
                         uint8_t* __restrict__ commit) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= rows) return;
  int tok = mask_id;
  bool take = false;
  if (in) {
    tok = in[r];
    if (tok == mask_id) {
      const int a = argmax[r];
      take = (conf[r] >= tau) && (a != mask_id);
      tok = take ? a : tok;
    }
  }
  out[r] = tok;
  if (commit) commit[r] = take ? 1 : 0;
}

hipError_t launch_unmask(int rows, const int32_t* argmax, const float* conf, float tau, int32_t mask_id,
                         const int32_t* in, int32_t* out, uint8_t* commit, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_unmask, dim3((rows + 255) / 256), dim3(256), 0, s, rows, argmax, conf, tau, mask_id,
                     in, out, commit);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Cache append: canvas rows kn[b][i][g][:] -> cache[b][g][L + i][:].
// One 16-byte (bf16) or 4-byte (fp32) element group per lane.
// ---------------------------------------------------------------------------
template <typename T>
__global__ void k_cache_append(int B, int C, int L, int cap, int Hkv, int dh, const T* __restrict__ kn,
                               T* __restrict__ cache, int vec) {
  const size_t n = (size_t)B * C * Hkv * dh / vec;
  for (size_t e = blockIdx.x * (size_t)blockDim.x + threadIdx.x; e < n; e += (size_t)gridDim.x * blockDim.x) {
    const size_t el = e * vec;
    const int f = (int)(el % dh);
    const size_t rest = el / dh;
    const int g = (int)(rest % Hkv);
    const size_t bi = rest / Hkv;
    const int i = (int)(bi % C), b = (int)(bi / C);
    T* dst = cache + (((size_t)b * Hkv + g) * cap + L + i) * dh + f;
    if (vec == 8) {
      *(u32x4*)dst = *(const u32x4*)(kn + el);
    } else {
      *dst = kn[el];
    }
  }
}

hipError_t launch_cache_append(int dtype, int B, int C, int L, int cap, int Hkv, int dh,
                               const void* kn, void* cache, hipStream_t s) {
  const size_t n = (size_t)B * C * Hkv * dh;
  if (n == 0) return hipSuccess;
  if (dtype == 1) {
    const size_t nv = n / 8;
    const int grid = (int)((nv + 255) / 256 < 4096 ? (nv + 255) / 256 : 4096);
    hipLaunchKernelGGL(k_cache_append<u16>, dim3(grid), dim3(256), 0, s, B, C, L, cap, Hkv, dh,
                       (const u16*)kn, (u16*)cache, 8);
  } else {
    const int grid = (int)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096);
    hipLaunchKernelGGL(k_cache_append<float>, dim3(grid), dim3(256), 0, s, B, C, L, cap, Hkv, dh,
                       (const float*)kn, (float*)cache, 1);
  }
  return hipGetLastError();
}

}  // namespace dg
