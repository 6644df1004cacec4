// Internal helpers shared by the gfx950 kernels of libdg (not part of the ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace dg {

typedef uint16_t u16;
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // 8 bf16
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));  // 4 bf16

#define DG_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// float -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}
// bf16 value of the rounded float (used to keep sums consistent with the packed operand).
__device__ __forceinline__ float round_bf16(float f) { return __uint_as_float(f32_to_bf16(f) << 16); }

// D = A.B + C on a 32x32x16 bf16 tile.  Lane l supplies A[m = l%32][k = 8(l/32)+i],
// B[k = 8(l/32)+i][n = l%32] (i = 0..7); D lane l holds D[8j + 4(l/32) + i][l%32]
// at element 4j + i.
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Transposing LDS read: within each 16-lane group, lane p points at 4
// consecutive bf16 of row p/4 (cols 4(p%4)..+3) of a 4 x 16 block; lane p then
// receives column p of that block (rows 0..3).
__device__ __forceinline__ u32x2 lds_read_tr16(const DG_LDS u16* p) {
  bf16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((DG_LDS bf16x4_t*)p);
  return __builtin_bit_cast(u32x2, v);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

__device__ __forceinline__ u32x4 ldg128(const u16* p) { return *(const u32x4*)p; }

// ---------------------------------------------------------------------------
// Philox4x64-10 (Salmon et al., SC'11, "Parallel random numbers: as easy as
// 1, 2, 3"): 10 rounds of two 64x64->128 multiplies with the round constants
// below, the key bumped by the Weyl constants between rounds.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint64_t philox4x64_w0(uint64_t c0, uint64_t c1, uint64_t c2, uint64_t c3,
                                              uint64_t k0, uint64_t k1) {
  const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) { k0 += W0; k1 += W1; }
    const uint64_t hi0 = __umul64hi(M0, c0), lo0 = M0 * c0;
    const uint64_t hi1 = __umul64hi(M1, c2), lo1 = M1 * c2;
    const uint64_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
  }
  return c0;
}

// The uniform-state renoise of one row (explainer, "Diffusione dello stato
// uniforme"): conf < tau draws floor(w0 V / 2^64) from Philox4x64-10 at
// counter (position, t, canvas, block), key (seed, 0); else the argmax.
struct RenoiseArgs {
  int32_t* out;    // NULL: no renoise
  uint8_t* mask;   // may be NULL
  float tau;
  uint64_t seed;
  uint32_t t, block;
  int canvas, V;
};
__device__ __forceinline__ void renoise_row(const RenoiseArgs& rn, int r, int32_t argmax, float conf) {
  const bool draw = conf < rn.tau;
  int tok = argmax;
  if (draw) {
    const uint32_t b = (uint32_t)(r / rn.canvas), i = (uint32_t)(r % rn.canvas);
    tok = (int)__umul64hi(philox4x64_w0(i, rn.t, b, rn.block, rn.seed, 0), (uint64_t)rn.V);
  }
  rn.out[r] = tok;
  if (rn.mask) rn.mask[r] = draw ? 1 : 0;
}

}  // namespace dg

// Launch wrappers (host side), implemented next to their kernels.  Each returns
// the hipError_t of its launch.  Pointers and sizes are already validated.
namespace dg {
struct VocabPlan {
  // variant: 0 fp32 rowwise, 1 bf16 32-row, 2 bf16 16-row, 3 bf16 64-row CU
  // groups of `group` workgroups (2 for d = 2048, 4 for d = 4096)
  int rows, d, V, nrb, nsplit, split_len, variant, group;
  size_t part_S_bytes, part_stat_bytes, part_X_bytes;  // X: group exchange (variant 3)
};
VocabPlan vocab_plan(int rows, int d, int V, int dtype);
// Poll bound of the CU-group handshake of later launches (< 0: the default).
void set_group_wait(int32_t polls);
// ev_begin / ev_end (may be NULL) are recorded around the main kernel only.
// rn (may be NULL): the uniform-state renoise of every row, done by the split
// combine from the row's own argmax and confidence (a separate launch on the
// fp32 path, which has no combine).
hipError_t launch_vocab(const VocabPlan& p, const void* z, const void* E, float* max_logit,
                        int32_t* argmax, float* conf, float* lse, void* selfcond, void* ws,
                        hipStream_t s, hipEvent_t ev_begin = nullptr, hipEvent_t ev_end = nullptr,
                        const RenoiseArgs* rn = nullptr, bool exchange_cleared = false);
// The region of ws that the CU-group kernel needs zeroed before it runs
// (tickets, flags, group words and exchange records): its bytes (a multiple of 16), 0 for
// the other variants.  launch_vocab clears it itself unless exchange_cleared.
size_t vocab_exchange_region(const VocabPlan& p, void* ws, void** region);

struct AttnPlan {
  int B, C, L, cap, Hq, Hkv, dh, dtype, causal, nrb, nsplit, keys_per_split;
  int merge_first;  // first canvas position whose rows the split combine merges
  size_t part_bytes;
};
AttnPlan attn_plan(int B, int C, int L, int cap, int Hq, int Hkv, int dh, int dtype, int causal);
hipError_t launch_attn(const AttnPlan& p, const void* q, const void* kc, const void* vc,
                       const void* kn, const void* vn, void* out, float* lse, void* ws,
                       hipStream_t s, hipEvent_t ev_begin = nullptr, hipEvent_t ev_end = nullptr);

// Tiled bf16 embedding table (16-id x 32-column blocks of 1 KiB in operand
// lane order); see dg_pack_embedding.
hipError_t launch_pack_embedding(int V, int d, const void* E, void* E_tiled, hipStream_t s);

// C[M][N] = A[M][K] . B[N][K]^T (+ Res[M][N]); dtype 0 fp32, 1 bf16.
// One (weight, residual, output, N) segment of a projection launch.
struct GemmSeg {
  const u16* B;
  const u16* Res;
  u16* C;
  int N, tiles;
  // optional second destination of the output: a KV cache [B][N/dh][cap][dh]
  // whose rows [L, L + Cn) of every (canvas, head) take output rows
  // b Cn + i (the cache write of a prefill-append); NULL: none
  u16* cache;
};
// Geometry of GemmSeg::cache (canvas length Cn, first row L, capacity, head dim).
struct CacheGeom {
  int Cn, L, cap, dh;
};
// bf16: zero_bytes (a multiple of 16) at zero are also cleared by the same
// launch, for a kernel later on the stream.
hipError_t launch_gemm_nt(int dtype, int M, int N, int K, const void* A, const void* B,
                          const void* Res, void* C, hipStream_t s, void* zero = nullptr,
                          size_t zero_bytes = 0);
// Q, K and V projections of the same activations in one launch (bf16), or
// three launches (fp32).  bf16 with k_cache / v_cache set: the K and V
// outputs are also written to those caches at rows [g.L, g.L + g.Cn) by the
// same launch (fp32: by separate cache-append launches).
hipError_t launch_gemm_qkv(int dtype, int M, int K, const void* A, const void* Wq, int Nq, void* Q,
                           const void* Wk, const void* Wv, int Nkv, void* Kn, void* Vn, hipStream_t s,
                           void* k_cache = nullptr, void* v_cache = nullptr, CacheGeom g = CacheGeom{1, 0, 1, 1});

hipError_t launch_assemble(int dtype, int R, int d, int V, const void* H, const void* E,
                           const int32_t* x, const void* S, void* X, hipStream_t s);
hipError_t launch_renoise(int rows, int canvas, int V, const int32_t* argmax, const float* conf,
                          float tau, uint64_t seed, uint32_t t, uint32_t block, int32_t* out,
                          uint8_t* mask, hipStream_t s);
// Masked diffusion: unmask-and-lock (in == NULL: a fully masked canvas).
hipError_t launch_unmask(int rows, const int32_t* argmax, const float* conf, float tau, int32_t mask_id,
                         const int32_t* in, int32_t* out, uint8_t* commit, hipStream_t s);
// Scatter canvas rows kn[B][C][Hkv][dh] into cache[B][Hkv][cap][dh] at rows [L, L+C).
hipError_t launch_cache_append(int dtype, int B, int C, int L, int cap, int Hkv, int dh,
                               const void* kn, void* cache, hipStream_t s);
}  // namespace dg
