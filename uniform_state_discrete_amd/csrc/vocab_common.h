// Device helpers shared by the vocabulary-head kernels (flash-vocab): the
// rescale threshold, MFMA and DPP wrappers, buffer loads, and the block order
// of the split-V grid.  Included by k_vocab.hip and k_vocab16.hip.
#pragma once
#include "dg_common.h"
#include <math.h>

namespace dg {

// Rescale threshold (natural-log units): a row's reference max only moves
// when a new logit exceeds it by more than this.  P = exp(l - m_ref) then
// stays <= e^40, and a sum of up to 2^24 such terms times |E| stays far below
// FLT_MAX; terms more than ~87 below the reference underflow, and they are
// then more than 87 below the row's maximum too (negligible in fp32).
constexpr float kLazyTh = 40.0f;

// LDS row of E-tile row m.  Rows are padded by 16 bytes, so the 64 banks see
// (row + 16-byte unit) mod 16; permuting each group of 16 rows (even rows of
// the group first, then odd) keeps both access patterns conflict-free: 16
// lanes writing one 16-byte unit of 16 consecutive tile rows, and the
// transposing reads of 8 consecutive tile rows x 32 bytes per 32 lanes.
// Column offsets stay compile-time.
__device__ __forceinline__ int prow16(int m) { return 2 * (m & 7) + (m >> 3); }

typedef __bf16 bf16x4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x4 mfma16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16(u32x2 a, u32x2 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4v, a),
                                                   __builtin_bit_cast(bf16x4v, b), c, 0, 0, 0);
}

// D += A.B on a 16x16x32 tile with D in VGPRs.  The products whose
// accumulators live in the AGPR file (the self-conditioning sums fill all 256
// of them) go through the builtin; the per-tile logits accumulate in VGPRs
// through this form, so the register allocator never has to move
// accumulators between the two files.  The compiler does not track the
// hazards of inline assembly: the leading s_nop gives the 2 wait states a
// product needs after a VALU write of any of its operands (the zeroed
// accumulator at the start of a tile); a chain of these products on one
// accumulator needs none; reads of the result by other instructions wait in
// mfma_v_settle.
__device__ __forceinline__ void mfma16x32_v(u32x4 a, u32x4 b, f32x4& d) {
  asm("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
// The same product without the leading wait states, for operands that no
// VALU instruction wrote (loaded from memory, constant, or the accumulator of
// the chain itself), and the first product of a chain, whose accumulator
// input is the inline constant 0 (no zeroing instructions, no wait states).
__device__ __forceinline__ void mfma16x32_vn(u32x4 a, u32x4 b, f32x4& d) {
  asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma16x32_v0(u32x4 a, u32x4 b, f32x4& d) {
  asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=v"(d) : "v"(a), "v"(b));
}
// Wait states between the last VGPR-form product and any other reader of its
// result.
__device__ __forceinline__ void mfma_v_settle(f32x4 (&lg)[2][2]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(lg[0][0]), "+v"(lg[0][1]), "+v"(lg[1][0]), "+v"(lg[1][1]));
}
__device__ __forceinline__ void mfma_v_settle(f32x4 (&lg)[4]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(lg[0]), "+v"(lg[1]), "+v"(lg[2]), "+v"(lg[3]));
}
__device__ __forceinline__ void mfma_v_settle(f32x4& a, f32x4& b) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(a), "+v"(b));
}

// The tiled table stores the 16 bytes of a lane with odd g (columns
// 8g..8g+7 of a chunk) as columns 8g+4..8g+7 then 8g..8g+3: those lanes
// write their first 8 bytes to LDS column 8g+4, the others to 8g, so each
// LDS store instruction covers all 64 banks without selecting data.  The
// matrix-core contraction sees the same permuted k-slots on both operands:
// the Z fragments of odd-g lanes get their halves swapped once, at load.
__device__ __forceinline__ u32x4 swap_halves(u32x4 v, bool sw) {
  return sw ? u32x4{v[2], v[3], v[0], v[1]} : v;
}

// Workgroup -> (row block, vocab split).  Workgroups are dispatched round-robin
// over the 8 XCDs (blockIdx % 8); consecutive linear ids are given to one XCD,
// so the row blocks that share a vocab split share that XCD's L2.
__device__ __forceinline__ void vocab_block(int nrb, int& rb, int& split) {
  const int nblk = gridDim.x, bid = blockIdx.x;
  const int lin = (nblk & 7) == 0 ? (bid & 7) * (nblk >> 3) + (bid >> 3) : bid;
  split = lin / nrb;
  rb = lin % nrb;
}

#ifndef DG_VOCAB32_PF
#define DG_VOCAB32_PF 8
#endif
// Buffer resource over [base, base + bytes): loads past the end return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 buffer_ld128(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
}
// LDS row of a 16-row tile row m: the 16-lane writes of one 16-byte unit of 16
// consecutive rows and the transposing reads of 4 rows x 4 units per 32 lanes
// fall on distinct banks (rows are padded by 16 bytes).
__device__ __forceinline__ int prow16t(int m) { return 4 * (m & 3) + (m >> 2); }
// max with the lowest id on ties, and sums, over 8 consecutive lanes (DPP:
// swap neighbours, swap pairs, mirror the two quads)
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xF, 0xF, false);
}
// max(x, x of the lane 1 apart / 2 apart within each group of 4 lanes), one
// DPP instruction each.  The compiler's own form adds NaN-quieting moves around
// every max; these operands are never NaN (finite logits or -inf).  The leading
// wait states cover a VALU write of x just before the DPP read.
__device__ __forceinline__ float dpp_max_x1(float x) {
  float r;
  asm("s_nop 1\n\tv_max_f32_dpp %0, %1, %1 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf" : "=v"(r) : "v"(x));
  return r;
}
__device__ __forceinline__ float dpp_max_x2(float x) {
  float r;
  asm("s_nop 1\n\tv_max_f32_dpp %0, %1, %1 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf" : "=v"(r) : "v"(x));
  return r;
}
// max of four values in two instructions (never NaN here, as above)
__device__ __forceinline__ float max4_f(float a, float b, float c, float d) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3\n\tv_max_f32 %0, %0, %4" : "=&v"(r) : "v"(a), "v"(b), "v"(c), "v"(d));
  return r;
}
template <int CTRL>
__device__ __forceinline__ void argmax_step(float& m, int& a) {
  const float om = dpp_f<CTRL>(m);
  const int oa = dpp_i<CTRL>(a);
  const bool take = (om > m) | ((om == m) & (oa < a));  // branch-free
  m = take ? om : m;
  a = take ? oa : a;
}
__device__ __forceinline__ float sum8(float s) {
  s += dpp_f<0xB1>(s);
  s += dpp_f<0x4E>(s);
  s += dpp_f<0x141>(s);
  return s;
}


// Launches the 16-row kernel (d = 4096, SLICE 1024) of k_vocab16.hip, which is
// compiled with its own scheduler flags.
hipError_t launch_vocab16_1024(dim3 grid, hipStream_t s, const u16* Z, const u16* E, int R, int d, int V,
                               int nrb, int split_len, float* pS, f32x4* pstat);

}  // namespace dg
