// Flash-vocab: the tied vocabulary head, its full-vocabulary softmax with the
// per-row max probability ("confidence"), and self-conditioning S = P . E
// (DiffusionGemma explainer, "Autocondizionamento": the probability matrix
// times the token-embedding table is handed to the next step), in one pass
// over the embedding table E that never stores the rows x V probabilities.
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
// (row + 16-byte unit) mod 16; permuting the rows keeps both access patterns
// conflict-free: 16 lanes writing one unit of 16 consecutive tile rows, and
// the transposing reads of 4 (32-row tiles) or 8 (16-row tiles) consecutive
// tile rows x 32 bytes per 32 lanes.  Column offsets stay compile-time.
__device__ __forceinline__ int prow32(int m) { return 4 * (m & 3) + ((m >> 2) & 3) + 16 * (m >> 4); }
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

// Workgroup -> (row block, vocab split).  Workgroups are dispatched round-robin
// over the 8 XCDs (blockIdx % 8); consecutive linear ids are given to one XCD,
// so the row blocks that share a vocab split share that XCD's L2.
__device__ __forceinline__ void vocab_block(int nrb, int& rb, int& split) {
  const int nblk = gridDim.x, bid = blockIdx.x;
  const int lin = (nblk & 7) == 0 ? (bid & 7) * (nblk >> 3) + (bid >> 3) : bid;
  split = lin / nrb;
  rb = lin % nrb;
}

// ---------------------------------------------------------------------------
// Variant 32 (d = 4*SLICE <= 2048).  Workgroup = 4 waves, 32 rows of Z, one
// vocab split; wave w owns the d-slice [w*SLICE, (w+1)*SLICE).
//
// Per 32-id vocab tile, wave w computes the partial logits^T over its d-slice
//   lg^T[v][row] = E[v, slice] . Z[row, slice]^T   (A = E rows from global,
//                                                    B = Z fragments in VGPRs)
// the 4 partials are summed through LDS (fixed order), every wave then runs
// the same max / argmax / sum on the full logits, and accumulates its slice of
//   S^T[slice][row] += E[tile, slice]^T . P^T       (A = E tile read back
//                                                    transposed from LDS,
//                                                    B = P in registers)
// The E tile is staged in LDS by the same wave that loaded it (no barrier);
// the product for tile t-1 is interleaved chunk by chunk with the logits of
// tile t, and tile t's chunk c overwrites tile t-1's chunk c right after it
// is consumed, so one tile of LDS per wave suffices.  Each lane owns one row
// (row = lane % 32) in every layout, so the softmax state stays in-lane.
//
// P = exp(l - m_seg) uses a reference m_seg per row that is fixed for a
// "segment" of tiles; only when a logit exceeds it by more than kLazyTh does
// the segment end: the accumulator is folded into the split's partial in
// global memory, G = G e^(m_G - m) + acc e^(m_seg - m), and a new segment
// starts from a zero accumulator.  The accumulator is therefore never
// rescaled inside the tile loop (it stays in the AGPR file).
// Output: G (unnormalised, relative to m_G) and per-row (m_G, sum, max,
// argmax) for the combine.
// ---------------------------------------------------------------------------
template <int SLICE>
__global__ void __launch_bounds__(256, 1)
    k_vocab32(const u16* __restrict__ Z, const u16* __restrict__ E, int R, int d, int V, int nrb,
              int split_len, float* __restrict__ pS, f32x4* __restrict__ pstat) {
  constexpr int NCH = SLICE / 32, KSN = SLICE / 16, EP = SLICE + 8;
  constexpr int PF = NCH < 4 ? NCH : (SLICE >= 512 ? 2 : 4);  // chunks of E in flight
  __shared__ __attribute__((aligned(16))) u16 Et[4][32][EP];
  __shared__ __attribute__((aligned(16))) f32x4 xch[4][4][64];  // [wave][16-byte chunk][lane]

  const int w = threadIdx.x >> 6, l = threadIdx.x & 63, h = l >> 5, l32 = l & 31;
  int rb, split;
  vocab_block(nrb, rb, split);
  const int r0 = rb * 32;
  const int vs = split * split_len, ve = min(V, vs + split_len);
  const int dbase = w * SLICE;
  const u32x4 z4 = {0u, 0u, 0u, 0u};

  const int zr = r0 + l32;
  const bool zok = zr < R;
  // Rows past R load a copy of row R-1 (branch-free); their results are never stored.
  u32x4 zf[KSN];
  {
    const u16* zp = Z + (size_t)(zok ? zr : R - 1) * d + dbase + h * 8;
#pragma unroll
    for (int ks = 0; ks < KSN; ++ks) zf[ks] = ldg128(zp + ks * 16);
  }
  float* gp = pS + ((size_t)split * R + (zok ? zr : 0)) * d + dbase + 4 * h;
  const size_t tofs = (size_t)gridDim.x / nrb * R * d;  // temp area follows the nsplit partials
  DG_LDS u16* et = (DG_LDS u16*)&Et[w][0][0];
  const int nt = ve > vs ? (ve - vs + 31) / 32 : 0;
  for (int e = l * 8; e < 32 * EP; e += 64 * 8) *(DG_LDS u32x4*)(et + e) = z4;
  // transposing-read addresses of this lane: tile rows tr_r + {0, 8, 16, 24},
  // column 16*((l>>4)&1) + 4*(l&3) inside each 32-column chunk
  const int tr_r = 4 * h + ((l & 15) >> 2);
  const int tr_c = 16 * ((l >> 4) & 1) + (l & 3) * 4;
  const DG_LDS u16* trb[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) trb[s] = et + prow32(tr_r + 8 * s) * EP + tr_c;
  DG_LDS u16* wrb = et + prow32(l32) * EP + h * 8;

  // E fragments of chunk c (columns [32c, 32c+32) of the slice) of a tile live
  // in ring slot c % PF; they are issued PF chunks ahead of their use.
  u32x4 ring0[PF], ring1[PF];
  // Ids past the split or V load a copy of row V-1 (branch-free): their logits
  // are masked to -inf, so their probabilities are exactly 0.
  auto issue = [&](int slot, int tile, int c) {
    const int ev = min(vs + tile * 32 + l32, V - 1);
    const u16* ep = E + (size_t)ev * d + dbase + h * 8 + c * 32;
    ring0[slot] = ldg128(ep);
    ring1[slot] = ldg128(ep + 16);
  };
#pragma unroll
  for (int c = 0; c < PF; ++c) issue(c, 0, c);

  float m_seg = -INFINITY, lsum = 0.f;        // current segment
  float m_G = -INFINITY, l_G = 0.f;           // folded partial
  bool g_valid = false;
  float m_true = -INFINITY, tmax = -INFINITY;
  int amax = 0;
  u32x4 pf0 = z4, pf1 = z4;

  // full logits of the current tile from the exchange buffer (fixed order)
  auto gather_logits = [&](int v0, float* L) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      f32x4 a = xch[0][q][l];
      a += xch[1][q][l];
      a += xch[2][q][l];
      a += xch[3][q][l];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int v = v0 + 8 * q + 4 * h + i;  // element 4q+i is id v0 + 8q + 4h + i
        L[4 * q + i] = v < ve ? a[i] : -INFINITY;
      }
    }
  };
  auto make_p = [&](const float* L) {
    float pv[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      // the normaliser sums the fp32 probabilities; bf16 copies feed P.E
      pv[e] = L[e] == -INFINITY ? 0.f : exp2f((L[e] - m_seg) * kLog2e);
      lsum += pv[e];
    }
    pf0 = u32x4{pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]), pack_bf16x2(pv[4], pv[5]),
                pack_bf16x2(pv[6], pv[7])};
    pf1 = u32x4{pack_bf16x2(pv[8], pv[9]), pack_bf16x2(pv[10], pv[11]),
                pack_bf16x2(pv[12], pv[13]), pack_bf16x2(pv[14], pv[15])};
  };

  int t = 0;
  for (;;) {  // segments
    f32x16 acc[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) acc[c] = zero16();
    bool rescale = false;
    for (;; ++t) {  // tiles
      const bool have = t < nt;
      f32x16 lg = zero16();
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const int slot = c % PF;
        // Branch-free body: on the first tile P = 0 and the LDS tile is zero;
        // on the drain pass (t == nt) the logits are computed and discarded.
        const u32x4 e0 = ring0[slot], e1 = ring1[slot];
        lg = mfma32(e0, zf[2 * c], lg);
        lg = mfma32(e1, zf[2 * c + 1], lg);
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          const u32x2 a0 = lds_read_tr16(trb[2 * p] + c * 32);
          const u32x2 a1 = lds_read_tr16(trb[2 * p + 1] + c * 32);
          acc[c] = mfma32(u32x4{a0[0], a0[1], a1[0], a1[1]}, p ? pf1 : pf0, acc[c]);
        }
        *(DG_LDS u32x4*)(wrb + c * 32) = e0;
        *(DG_LDS u32x4*)(wrb + c * 32 + 16) = e1;
        if (c + PF < NCH)
          issue(slot, t, c + PF);
        else
          issue(slot, t + 1, c + PF - NCH);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (!have) break;

      // sum the four d-slice partials
#pragma unroll
      for (int q = 0; q < 4; ++q)
        xch[w][q][l] = f32x4{lg[4 * q], lg[4 * q + 1], lg[4 * q + 2], lg[4 * q + 3]};
      __syncthreads();
      const int v0 = vs + t * 32;
      float L[16];
      gather_logits(v0, L);
      __syncthreads();

      tmax = -INFINITY;
      int targ = 0x7fffffff;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int v = v0 + 8 * (e >> 2) + 4 * h + (e & 3);
        const bool gt = L[e] > tmax;  // ids increase with e: the first maximum is kept
        tmax = gt ? L[e] : tmax;
        targ = gt ? v : targ;
      }
      {
        const float om = __shfl_xor(tmax, 32);
        const int oa = __shfl_xor(targ, 32);
        const bool take = om > tmax || (om == tmax && oa < targ);
        tmax = take ? om : tmax;
        targ = take ? oa : targ;
      }
      amax = tmax > m_true ? targ : amax;  // earlier tiles win ties
      m_true = fmaxf(m_true, tmax);
      if (m_seg == -INFINITY) {
        m_seg = tmax;  // first tile of the split
      } else if (__any(tmax > m_seg + kLazyTh)) {
        rescale = true;  // fold and restart before this tile's P
        break;
      }
      make_p(L);
    }

    // Fold the segment into G.  The accumulator is only ever stored raw (never
    // touched by VALU code, so it stays in AGPRs): the first fold makes it G
    // (reference m_seg); a later fold stores it to the temp area T and merges
    // G = G e^(m_G - m) + T e^(m_seg - m) with plain loads and stores.
    const float m_new = rescale ? fmaxf(m_seg, tmax) : m_seg;
    float* dst = g_valid ? gp + tofs : gp;
    if (zok) {
#pragma unroll
      for (int c = 0; c < NCH; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *(f32x4*)(dst + 32 * c + 8 * j) =
              f32x4{acc[c][4 * j], acc[c][4 * j + 1], acc[c][4 * j + 2], acc[c][4 * j + 3]};
    }
    if (!g_valid) {
      m_G = m_seg;
      l_G = lsum;
      g_valid = true;
    } else {
      const float gs = m_G == -INFINITY ? 0.f : exp2f((m_G - m_new) * kLog2e);
      const float as = m_seg == -INFINITY ? 0.f : exp2f((m_seg - m_new) * kLog2e);
      if (zok) {
        for (int c = 0; c < NCH; ++c)
          for (int j = 0; j < 4; ++j) {
            float* g = gp + 32 * c + 8 * j;
            *(f32x4*)g = *(const f32x4*)g * gs + *(const f32x4*)(g + tofs) * as;
          }
      }
      l_G = l_G * gs + lsum * as;
      m_G = m_new;
    }
    if (!rescale) break;
    m_seg = m_new;
    lsum = 0.f;
    float L[16];
    gather_logits(vs + t * 32, L);  // the exchange buffer still holds tile t
    make_p(L);
    ++t;
  }

  l_G += __shfl_xor(l_G, 32);
  if (zok && w == 0 && h == 0) pstat[(size_t)split * R + zr] = f32x4{m_G, l_G, m_true, __int_as_float(amax)};
}

// ---------------------------------------------------------------------------
// Variant 16 (d = 4*SLICE up to 4096): the same algorithm on 16-row tiles and
// 16-id vocab tiles, so that one E tile (16 x d) fits in LDS at d = 4096.
// Logits^T use 16x16x32 MFMAs; the P.E product uses 16x16x16 MFMAs, whose
// 4-deep K slice lines up with the logits' output layout (no permutation).
// ---------------------------------------------------------------------------
template <int SLICE>
__global__ void __launch_bounds__(256, 1)
    k_vocab16(const u16* __restrict__ Z, const u16* __restrict__ E, int R, int d, int V, int nrb,
              int split_len, float* __restrict__ pS, f32x4* __restrict__ pstat) {
  constexpr int NCH = SLICE / 32, EP = SLICE + 8;
  constexpr int PF = NCH < 8 ? NCH : 8;
  __shared__ __attribute__((aligned(16))) u16 Et[4][16][EP];
  __shared__ __attribute__((aligned(16))) f32x4 xch[4][64];

  const int w = threadIdx.x >> 6, l = threadIdx.x & 63, g4 = l >> 4, l16 = l & 15;
  int rb, split;
  vocab_block(nrb, rb, split);
  const int r0 = rb * 16;
  const int vs = split * split_len, ve = min(V, vs + split_len);
  const int dbase = w * SLICE;
  const u32x4 z4 = {0u, 0u, 0u, 0u};

  const int zr = r0 + l16;
  const bool zok = zr < R;
  u32x4 zf[NCH];
  {
    const u16* zp = Z + (size_t)(zok ? zr : R - 1) * d + dbase + g4 * 8;
#pragma unroll
    for (int ks = 0; ks < NCH; ++ks) zf[ks] = ldg128(zp + ks * 32);
  }
  float* gp = pS + ((size_t)split * R + (zok ? zr : 0)) * d + dbase + 4 * g4;
  const size_t tofs = (size_t)gridDim.x / nrb * R * d;
  DG_LDS u16* et = (DG_LDS u16*)&Et[w][0][0];
  const int nt = ve > vs ? (ve - vs + 15) / 16 : 0;
  for (int e = l * 8; e < 16 * EP; e += 64 * 8) *(DG_LDS u32x4*)(et + e) = z4;
  const int tr_r = 4 * g4 + (l16 >> 2);
  const DG_LDS u16* trb = et + prow16(tr_r) * EP + (l & 3) * 4;
  DG_LDS u16* wrb = et + prow16(l16) * EP + g4 * 8;

  u32x4 ring0[PF];
  auto issue = [&](int slot, int tile, int c) {
    const int ev = min(vs + tile * 16 + l16, V - 1);
    ring0[slot] = ldg128(E + (size_t)ev * d + dbase + g4 * 8 + c * 32);
  };
#pragma unroll
  for (int c = 0; c < PF; ++c) issue(c, 0, c);

  float m_seg = -INFINITY, lsum = 0.f, m_G = -INFINITY, l_G = 0.f;
  bool g_valid = false;
  float m_true = -INFINITY, tmax = -INFINITY;
  int amax = 0;
  u32x2 pf = {0u, 0u};

  auto gather_logits = [&](int v0, float* L) {
    f32x4 a = xch[0][l];
    a += xch[1][l];
    a += xch[2][l];
    a += xch[3][l];
#pragma unroll
    for (int i = 0; i < 4; ++i) L[i] = (v0 + 4 * g4 + i) < ve ? a[i] : -INFINITY;  // id v0 + 4*g4 + i
  };
  auto make_p = [&](const float* L) {
    float pv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pv[i] = L[i] == -INFINITY ? 0.f : exp2f((L[i] - m_seg) * kLog2e);
      lsum += pv[i];
    }
    pf = u32x2{pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3])};
  };

  int t = 0;
  for (;;) {
    f32x4 acc[2 * NCH];
#pragma unroll
    for (int c = 0; c < 2 * NCH; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    bool rescale = false;
    for (;; ++t) {
      const bool have = t < nt;
      f32x4 lg = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const int slot = c % PF;
        const u32x4 e0 = ring0[slot];
        lg = mfma16x32(e0, zf[c], lg);
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          const u32x2 a = lds_read_tr16(trb + c * 32 + 16 * p);
          acc[2 * c + p] = mfma16x16(a, pf, acc[2 * c + p]);
        }
        *(DG_LDS u32x4*)(wrb + c * 32) = e0;
        if (c + PF < NCH)
          issue(slot, t, c + PF);
        else
          issue(slot, t + 1, c + PF - NCH);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (!have) break;

      xch[w][l] = lg;
      __syncthreads();
      const int v0 = vs + t * 16;
      float L[4];
      gather_logits(v0, L);
      __syncthreads();

      tmax = -INFINITY;
      int targ = 0x7fffffff;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool gt = L[i] > tmax;
        tmax = gt ? L[i] : tmax;
        targ = gt ? v0 + 4 * g4 + i : targ;
      }
#pragma unroll
      for (int o = 16; o <= 32; o <<= 1) {
        const float om = __shfl_xor(tmax, o);
        const int oa = __shfl_xor(targ, o);
        const bool take = om > tmax || (om == tmax && oa < targ);
        tmax = take ? om : tmax;
        targ = take ? oa : targ;
      }
      amax = tmax > m_true ? targ : amax;
      m_true = fmaxf(m_true, tmax);
      if (m_seg == -INFINITY) {
        m_seg = tmax;
      } else if (__any(tmax > m_seg + kLazyTh)) {
        rescale = true;
        break;
      }
      make_p(L);
    }

    const float m_new = rescale ? fmaxf(m_seg, tmax) : m_seg;
    float* dst = g_valid ? gp + tofs : gp;
    if (zok) {
#pragma unroll
      for (int c = 0; c < 2 * NCH; ++c) *(f32x4*)(dst + 16 * c) = acc[c];
    }
    if (!g_valid) {
      m_G = m_seg;
      l_G = lsum;
      g_valid = true;
    } else {
      const float gs = m_G == -INFINITY ? 0.f : exp2f((m_G - m_new) * kLog2e);
      const float as = m_seg == -INFINITY ? 0.f : exp2f((m_seg - m_new) * kLog2e);
      if (zok) {
        for (int c = 0; c < 2 * NCH; ++c) {
          float* g = gp + 16 * c;
          *(f32x4*)g = *(const f32x4*)g * gs + *(const f32x4*)(g + tofs) * as;
        }
      }
      l_G = l_G * gs + lsum * as;
      m_G = m_new;
    }
    if (!rescale) break;
    m_seg = m_new;
    lsum = 0.f;
    float L[4];
    gather_logits(vs + t * 16, L);
    make_p(L);
    ++t;
  }

  l_G += __shfl_xor(l_G, 16);
  l_G += __shfl_xor(l_G, 32);
  if (zok && w == 0 && g4 == 0) pstat[(size_t)split * R + zr] = f32x4{m_G, l_G, m_true, __int_as_float(amax)};
}

// ---------------------------------------------------------------------------
// Combine of the vocab splits, one workgroup per row, splits in increasing
// vocab order:  max = max_s max_s,  argmax = that of the first split
// attaining it (lowest id),  mu = max_s m_ref_s,  Lt = sum_s e^(m_ref_s - mu) sum_s,
// lse = mu + ln Lt,  conf = e^(max - mu) / Lt,  S = sum_s e^(m_ref_s - mu) S_s / Lt.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) k_vocab_combine(int R, int d, int nsplit, const float* __restrict__ pS,
                                                       const f32x4* __restrict__ pstat,
                                                       float* __restrict__ max_logit,
                                                       int32_t* __restrict__ argmax,
                                                       float* __restrict__ conf, float* __restrict__ lse,
                                                       void* __restrict__ S, int out_bf16) {
  __shared__ float wgt[1024];
  __shared__ float sh[4];
  const int r = blockIdx.x;
  if (threadIdx.x == 0) {
    float M = -INFINITY, mu = -INFINITY;
    int A = 0;
    for (int s = 0; s < nsplit; ++s) {
      const f32x4 st = pstat[(size_t)s * R + r];
      if (st[2] > M) { M = st[2]; A = __float_as_int(st[3]); }
      mu = fmaxf(mu, st[0]);
    }
    float Lt = 0.f;
    for (int s = 0; s < nsplit; ++s) {
      const f32x4 st = pstat[(size_t)s * R + r];
      const float ws = st[0] == -INFINITY ? 0.f : expf(st[0] - mu);
      wgt[s] = ws;
      Lt += ws * st[1];
    }
    sh[0] = 1.f / Lt;
    max_logit[r] = M;
    argmax[r] = A;
    conf[r] = expf(M - mu) / Lt;
    if (lse) lse[r] = mu + logf(Lt);
  }
  __syncthreads();
  const float invL = sh[0];
  for (int e = threadIdx.x * 4; e < d; e += 256 * 4) {
    f32x4 a = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < nsplit; ++s) a += wgt[s] * *(const f32x4*)(pS + ((size_t)s * R + r) * d + e);
    a *= invL;
    if (out_bf16) {
      u32x2 o = {pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3])};
      *(u32x2*)((u16*)S + (size_t)r * d + e) = o;
    } else {
      *(f32x4*)((float*)S + (size_t)r * d + e) = a;
    }
  }
}

// ---------------------------------------------------------------------------
// fp32-storage path: one workgroup per row, vocab ids in chunks of 256 (one
// per lane), online softmax in fp64 (exp/log in double), lane k accumulates S
// columns k, k+256, ... in fp64; only the stored outputs are rounded.
// ---------------------------------------------------------------------------
constexpr int kF32MaxD = 4096;
__global__ void __launch_bounds__(256) k_vocab_f32(int R, int d, int V, const float* __restrict__ Z,
                                                   const float* __restrict__ E,
                                                   float* __restrict__ max_logit,
                                                   int32_t* __restrict__ argmax,
                                                   float* __restrict__ conf, float* __restrict__ lse,
                                                   float* __restrict__ S) {
  __shared__ float zs[kF32MaxD];
  __shared__ double ps[256], rv[256];
  __shared__ int ri[256];
  const int r = blockIdx.x, tid = threadIdx.x;
  for (int e = tid; e < d; e += 256) zs[e] = Z[(size_t)r * d + e];
  __syncthreads();
  double sacc[kF32MaxD / 256];
#pragma unroll
  for (int k = 0; k < kF32MaxD / 256; ++k) sacc[k] = 0.0;
  double m = -INFINITY, lsum = 0.0;
  int am = 0;
  for (int v0 = 0; v0 < V; v0 += 256) {
    const int v = v0 + tid;
    double lgv = -INFINITY;
    if (v < V) {
      const float* er = E + (size_t)v * d;
      double a = 0.0;
      for (int e = 0; e < d; ++e) a = fma((double)zs[e], (double)er[e], a);
      lgv = a;
    }
    rv[tid] = lgv;
    ri[tid] = v;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
      if (tid < o) {
        const double x = rv[tid + o];
        const int xi = ri[tid + o];
        if (x > rv[tid] || (x == rv[tid] && xi < ri[tid])) { rv[tid] = x; ri[tid] = xi; }
      }
      __syncthreads();
    }
    const double cm = rv[0];
    const int ca = ri[0];
    __syncthreads();
    double mnew = m;
    if (cm > m) { mnew = cm; am = ca; }
    const double alpha = (m == -INFINITY) ? 0.0 : exp(m - mnew);
    const double p = v < V ? exp(lgv - mnew) : 0.0;
    ps[tid] = p;
    rv[tid] = p;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
      if (tid < o) rv[tid] += rv[tid + o];
      __syncthreads();
    }
    lsum = lsum * alpha + rv[0];
    m = mnew;
    const int vn = min(256, V - v0);
#pragma unroll
    for (int k = 0; k < kF32MaxD / 256; ++k) {
      const int e = tid + 256 * k;
      if (e < d) {
        double a = sacc[k] * alpha;
        for (int jj = 0; jj < vn; ++jj) a = fma(ps[jj], (double)E[(size_t)(v0 + jj) * d + e], a);
        sacc[k] = a;
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int k = 0; k < kF32MaxD / 256; ++k) {
    const int e = tid + 256 * k;
    if (e < d) S[(size_t)r * d + e] = (float)(sacc[k] / lsum);
  }
  if (tid == 0) {
    max_logit[r] = (float)m;
    argmax[r] = am;
    conf[r] = (float)(1.0 / lsum);
    if (lse) lse[r] = (float)(m + log(lsum));
  }
}

// ---------------------------------------------------------------------------
VocabPlan vocab_plan(int rows, int d, int V, int dtype) {
  VocabPlan p{};
  p.rows = rows; p.d = d; p.V = V;
  if (dtype != 1) {
    p.variant = 0; p.nrb = rows; p.nsplit = 1; p.split_len = V;
    return p;
  }
  int rw, vt;
  if (d <= 2048) { p.variant = 1; rw = 32; vt = 32; }
  else { p.variant = 2; rw = 16; vt = 16; }
  p.nrb = (rows + rw - 1) / rw;
  const int tiles = (V + vt - 1) / vt;
  int ns = (256 + p.nrb / 2) / p.nrb;              // one workgroup per CU
  ns = ns < 1 ? 1 : (ns > tiles ? tiles : ns);
  p.split_len = (tiles + ns - 1) / ns * vt;
  p.nsplit = (V + p.split_len - 1) / p.split_len;
  // nsplit partials of S, then an equal temp area used only when a row's
  // reference max has to move during a split
  p.part_S_bytes = 2 * (size_t)p.nsplit * rows * d * sizeof(float);
  p.part_stat_bytes = (size_t)p.nsplit * rows * sizeof(f32x4);
  return p;
}

hipError_t launch_vocab(const VocabPlan& p, const void* z, const void* E, float* max_logit,
                        int32_t* argmax, float* conf, float* lse, void* selfcond, void* ws,
                        hipStream_t s, hipEvent_t ev_begin, hipEvent_t ev_end) {
  if (p.rows <= 0) return hipSuccess;
  if (p.variant == 0) {
    hipLaunchKernelGGL(k_vocab_f32, dim3(p.rows), dim3(256), 0, s, p.rows, p.d, p.V,
                       (const float*)z, (const float*)E, max_logit, argmax, conf, lse,
                       (float*)selfcond);
    return hipGetLastError();
  }
  float* pS = (float*)ws;
  f32x4* pstat = (f32x4*)((char*)ws + p.part_S_bytes);
  const dim3 grid((unsigned)(p.nrb * p.nsplit));
  const u16* Zb = (const u16*)z;
  const u16* Eb = (const u16*)E;
  const int sl = p.d / 4;
  bool launched = true;
  if (ev_begin) {
    hipError_t e = hipEventRecord(ev_begin, s);
    if (e != hipSuccess) return e;
  }
  if (p.variant == 1) {
    switch (sl) {
      case 32: hipLaunchKernelGGL(k_vocab32<32>, grid, dim3(256), 0, s, Zb, Eb, p.rows, p.d, p.V, p.nrb, p.split_len, pS, pstat); break;
      case 64: hipLaunchKernelGGL(k_vocab32<64>, grid, dim3(256), 0, s, Zb, Eb, p.rows, p.d, p.V, p.nrb, p.split_len, pS, pstat); break;
      case 128: hipLaunchKernelGGL(k_vocab32<128>, grid, dim3(256), 0, s, Zb, Eb, p.rows, p.d, p.V, p.nrb, p.split_len, pS, pstat); break;
      case 256: hipLaunchKernelGGL(k_vocab32<256>, grid, dim3(256), 0, s, Zb, Eb, p.rows, p.d, p.V, p.nrb, p.split_len, pS, pstat); break;
      case 512: hipLaunchKernelGGL(k_vocab32<512>, grid, dim3(256), 0, s, Zb, Eb, p.rows, p.d, p.V, p.nrb, p.split_len, pS, pstat); break;
      default: launched = false;
    }
  } else {
    switch (sl) {
      case 1024: hipLaunchKernelGGL(k_vocab16<1024>, grid, dim3(256), 0, s, Zb, Eb, p.rows, p.d, p.V, p.nrb, p.split_len, pS, pstat); break;
      default: launched = false;
    }
  }
  if (!launched) return hipErrorInvalidValue;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (ev_end && (e = hipEventRecord(ev_end, s)) != hipSuccess) return e;
  hipLaunchKernelGGL(k_vocab_combine, dim3(p.rows), dim3(256), 0, s, p.rows, p.d, p.nsplit, pS,
                     pstat, max_logit, argmax, conf, lse, selfcond, 1);
  return hipGetLastError();
}

}  // namespace dg
