// Canvas attention over [KV cache || canvas] (DiffusionGemma explainer,
// "Architettura: il prefill incrementale e il denoising"): bidirectional in
// denoising (every canvas query sees every canvas token and the whole cache),
// causal in the incremental prefill of a finished block (query i sees the
// cache and canvas keys 0..i).
#include "dg_common.h"
#include <math.h>

#include <algorithm>
#include <functional>
#include <vector>

namespace dg {

// ---------------------------------------------------------------------------
// bf16 path.  One workgroup = one (canvas b, KV head g), 128 packed query rows
// (row = canvas position * G + head-in-group: the G query heads sharing a KV
// head share every K/V tile), and one split of the keys.  4 waves x 32 rows.
//
// Both products are computed transposed so that each lane owns one query row:
//   S^T[key][row] = K . Q^T   (A = K tile from LDS, B = Q fragments in VGPRs)
//   O^T[dh][row] += V^T . P^T (A = V tile read transposed from LDS with
//                              ds_read_b64_tr_b16, B = P straight from S^T)
// The key order inside a 16-deep MFMA step is permuted identically on both
// operands, so P never leaves registers.  Online softmax in the log2 domain.
// K/V tiles of 64 keys are double-buffered in LDS through registers; one
// barrier per tile.  Rows of the K tile are padded by 16 B and of the V tile
// by 64 B so that the row-wise and the transposing reads are conflict-free.
// KSPLIT (launches of at most 64 packed rows): waves w and w + 2 take the same
// 32 rows and the two 32-key halves of every tile, so all four SIMDs work
// (otherwise waves 2 and 3 only move tiles); the halves merge their running
// max, sum and accumulators through LDS after the last tile.
// ---------------------------------------------------------------------------
constexpr float kAttnLazy = 8.0f;

// Keys seen by the packed row block rb (128 rows): all L + C of them in
// denoising; in a causal pass none past L + (the block's last query's
// position), so the block's key range stops there.
__host__ __device__ inline int attn_key_limit(int causal, int L, int C, int G, int rb) {
  const int nkeys = L + C, M = C * G;
  if (!causal) return nkeys;
  const int last = (M < rb * 128 + 128 ? M : rb * 128 + 128) - 1;
  const int lim = L + last / G + 1;
  return lim < nkeys ? lim : nkeys;
}

template <int DH, bool KSPLIT>
__global__ void __launch_bounds__(256, 2)
    k_attn_bf16(int B, int C, int L, int cap, int Hq, int Hkv, int G, int causal, int nrb,
                int nsplit, int kps, const u16* __restrict__ Q, const u16* __restrict__ Kc,
                const u16* __restrict__ Vc, const u16* __restrict__ Kn, const u16* __restrict__ Vn,
                u16* __restrict__ O, float* __restrict__ lse_out, float* __restrict__ Opart,
                float* __restrict__ mpart, float* __restrict__ lpart) {
  constexpr int KP = DH + 8, VP = DH + 32, KS = DH / 16, MB = DH / 32;
  constexpr int CPR = DH / 8, NLD = 64 * CPR / 256;
  __shared__ __attribute__((aligned(16))) u16 Ks[2][64][KP];
  __shared__ __attribute__((aligned(16))) u16 Vs[2][64][VP];

  const int w = threadIdx.x >> 6, l = threadIdx.x & 63, h = l >> 5, l32 = l & 31;
  // Workgroups are dealt to the 8 XCDs in turn, each with its own L2.  The
  // logical order puts the nrb row blocks that read the same keys next to
  // each other on one XCD, so the K/V tiles come from that XCD's L2 after the
  // first of them has fetched it.  The grid is padded to a multiple of 8.
  int bid = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
  if (bid >= nrb * nsplit * Hkv * B) return;
  // causal: the last row blocks see the most keys; dispatched first, their
  // splits finish while the short blocks' workgroups fill the freed slots
  const int rb = causal ? nrb - 1 - bid % nrb : bid % nrb;
  bid /= nrb;
  const int split = bid % nsplit;
  bid /= nsplit;
  const int g = bid % Hkv, b = bid / Hkv;
  const int M = C * G;
  const int k_lim = attn_key_limit(causal, L, C, G, rb);
  // A row block whose keys all lie in the first split writes its output
  // directly; its other splits have nothing to do.  A longer one leaves a
  // partial per split (an empty one, m = -inf and l = 0, for a split past
  // its key limit) for the combine.
  const bool direct = k_lim <= kps;
  if (direct && split > 0) return;
  const int k_begin = split * kps;
  const int k_end = min(k_lim, k_begin + kps);
  const int wr = KSPLIT ? (w & 1) : w;  // this wave's group of 32 packed rows
  const int kh = KSPLIT ? (w >> 1) : 0;  // KSPLIT: this wave's 32-key half of each tile
  constexpr int NKB = KSPLIT ? 1 : 2;    // 32-key chains of S^T per wave
  const int row = rb * 128 + wr * 32 + l32;
  const bool rok = row < M;
  const bool wave_live = rb * 128 + wr * 32 < M;  // uniform over the wave
  const int qi = rok ? row / G : 0, qh = g * G + (rok ? row % G : 0);
  const u32x4 z4 = {0u, 0u, 0u, 0u};

  u32x4 qf[KS];
  {
    const u16* qp = Q + (((size_t)b * C + qi) * Hq + qh) * DH + h * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = rok ? ldg128(qp + ks * 16) : z4;
  }
  f32x16 oacc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) oacc[mb] = zero16();
  float m = -INFINITY, lsum = 0.f;
  const float sl2 = kLog2e * rsqrtf((float)DH);
  const int qlim = L + qi;  // causal: key <= L + i
  // causal: every row of the block sees keys up to L + (its first position)
  const int kvis = L + rb * 128 / G;

  u32x4 kreg[NLD], vreg[NLD];
  // Tiles that lie in the cache and inside the split (all but the last one
  // or two) load through buffer resources over this (b, g) cache slab: a
  // fixed per-lane offset plus a scalar tile offset, no address arithmetic.
  constexpr int RPU = 256 / CPR;  // tile rows per load instruction
  const int kfast = min(L, k_end);
  const __amdgpu_buffer_rsrc_t rsK = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<u16*>(Kc + ((size_t)b * Hkv + g) * cap * DH), (short)0, (int)((size_t)cap * DH * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t rsV = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<u16*>(Vc + ((size_t)b * Hkv + g) * cap * DH), (short)0, (int)((size_t)cap * DH * 2), 0x00020000);
  const uint32_t voff = (uint32_t)(((threadIdx.x / CPR) * DH + (threadIdx.x % CPR) * 8) * 2);
  auto load_tile = [&](int t0) {
    if (t0 + 64 <= kfast) {
#pragma unroll
      for (int u = 0; u < NLD; ++u) {
        const uint32_t so = (uint32_t)((t0 + u * RPU) * DH * 2);
        kreg[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsK, voff, so, 0));
        vreg[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsV, voff, so, 0));
      }
      return;
    }
#pragma unroll
    for (int u = 0; u < NLD; ++u) {
      const int idx = threadIdx.x + u * 256;
      const int rr = idx / CPR, cc = (idx % CPR) * 8;
      // keys past the split load a valid key's row instead (finite data; the
      // scores of those keys are masked, so their P is 0): no select on the
      // loaded value, which would wait for the load right here
      const int key = min(t0 + rr, k_end - 1);
      size_t o;
      const u16 *kp, *vp;
      if (key < L) {
        o = (((size_t)b * Hkv + g) * cap + key) * DH + cc;
        kp = Kc + o;
        vp = Vc + o;
      } else {
        o = (((size_t)b * C + (key - L)) * Hkv + g) * DH + cc;
        kp = Kn + o;
        vp = Vn + o;
      }
      kreg[u] = ldg128(kp);
      vreg[u] = ldg128(vp);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int u = 0; u < NLD; ++u) {
      const int idx = threadIdx.x + u * 256;
      const int rr = idx / CPR, cc = (idx % CPR) * 8;
      *(u32x4*)&Ks[buf][rr][cc] = kreg[u];
      *(u32x4*)&Vs[buf][rr][cc] = vreg[u];
    }
  };

  const int ntiles = k_end > k_begin ? (k_end - k_begin + 63) / 64 : 0;
  if (ntiles > 0) {
    load_tile(k_begin);
    store_tile(0);
  }
  // The Q fragments are complete on every path into the loop.  Without this
  // use, the path with no tiles leaves their loads pending at the loop head,
  // and the first product of every tile would then wait for all vector
  // loads, including the K/V prefetch issued just before it.
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) asm volatile("" ::"v"(qf[ks]));
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    const int t0 = k_begin + t * 64;
    if (t + 1 < ntiles) load_tile(t0 + 64);
    // a wave whose 32 packed rows are all past the canvas (few queries per
    // KV head) only helps move the tiles: no products, no softmax
    if (wave_live) {
      // S^T for keys 0..31 and 32..63: two independent chains interleaved, K
      // fragments read two steps ahead of their products
      f32x16 sacc[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) sacc[kb] = zero16();
      {
        u32x4 ka[3][NKB];
        auto kread = [&](int ks) {
  #pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
            ka[ks % 3][kb] = *(const u32x4*)&Ks[buf][(kh + kb) * 32 + l32][ks * 16 + h * 8];
        };
        kread(0);
        kread(1);
  #pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          if (ks + 2 < KS) kread(ks + 2);
  #pragma unroll
          for (int kb = 0; kb < NKB; ++kb) sacc[kb] = mfma32(ka[ks % 3][kb], qf[ks], sacc[kb]);
        }
      }
      // scores stay unscaled: p = 2^(s sl2 - m) with m in the scaled (log2) domain
      if (!(t0 + 64 <= k_end && (!causal || t0 + 63 <= kvis))) {
        // a ragged tile or one that crosses the causal diagonal (uniform
        // branch): masked keys get -inf
  #pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
  #pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int key = t0 + (kh + kb) * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
            const bool valid = key < k_end && (!causal || key <= qlim);
            sacc[kb][e] = valid ? sacc[kb][e] : -INFINITY;
          }
      }
      float tmax = -INFINITY;
  #pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
  #pragma unroll
        for (int e = 0; e < 16; e += 2) tmax = fmaxf(tmax, fmaxf(sacc[kb][e], sacc[kb][e + 1]));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32)) * sl2;  // sl2 > 0 keeps the order
      // Lazy reference: it moves only when a score exceeds it by more than
      // kAttnLazy (log2 units), so p <= 2^kAttnLazy and the accumulators are
      // rescaled a few times per row instead of on most tiles.
      if (tmax > m + kAttnLazy) {
        const float alpha = __builtin_amdgcn_exp2f(m - tmax);  // m = -inf gives 0
        lsum *= alpha;
  #pragma unroll
        for (int mb = 0; mb < MB; ++mb) oacc[mb] *= alpha;
        m = tmax;
      }
      // a row with no valid key yet keeps m = -inf: its scores are all -inf
      const float mu = m == -INFINITY ? 0.f : m;
      typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
      typedef float f32x2v __attribute__((ext_vector_type(2)));
      const bf16x2v one2 = __builtin_bit_cast(bf16x2v, 0x3f803f80u);  // (1, 1)
      constexpr int NQ = 2 * NKB;  // 16-key groups of this wave's keys
      u32x4 pf[NQ];
  #pragma unroll
      for (int q = 0; q < NQ; ++q) {
        uint32_t pk[4];
  #pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const float s0 = sacc[q >> 1][8 * (q & 1) + e], s1 = sacc[q >> 1][8 * (q & 1) + e + 1];
          const float p0 = __builtin_amdgcn_exp2f(fmaf(s0, sl2, -mu)), p1 = __builtin_amdgcn_exp2f(fmaf(s1, sl2, -mu));
          // P enters the product in bf16: the normaliser sums the same rounded
          // values (a dot product of the packed pair with (1, 1))
          const bf16x2v pb = __builtin_convertvector(f32x2v{p0, p1}, bf16x2v);
          lsum = __builtin_amdgcn_fdot2_f32_bf16(pb, one2, lsum, false);
          pk[e >> 1] = __builtin_bit_cast(uint32_t, pb);
        }
        pf[q] = u32x4{pk[0], pk[1], pk[2], pk[3]};
      }
      // O^T += V^T P^T: the MB output chains interleaved, V^T fragments of the
      // next key group read one step ahead of their products
      const DG_LDS u16* vbase = (const DG_LDS u16*)&Vs[buf][0][0];
      {
        u32x4 va[2][MB];
        auto vread = [&](int q) {
  #pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
            const int r0 = 32 * kh + 16 * q + 4 * h + ((l & 15) >> 2);
            const int c0 = mb * 32 + 16 * ((l >> 4) & 1) + (l & 3) * 4;
            const u32x2 a0 = lds_read_tr16(vbase + r0 * VP + c0);
            const u32x2 a1 = lds_read_tr16(vbase + (r0 + 8) * VP + c0);
            va[q & 1][mb] = u32x4{a0[0], a0[1], a1[0], a1[1]};
          }
        };
        vread(0);
  #pragma unroll
        for (int q = 0; q < NQ; ++q) {
          if (q + 1 < NQ) vread(q + 1);
  #pragma unroll
          for (int mb = 0; mb < MB; ++mb) oacc[mb] = mfma32(va[q & 1][mb], pf[q], oacc[mb]);
        }
      }
    }
    if (t + 1 < ntiles) store_tile(buf ^ 1);
    __syncthreads();
  }
  lsum += __shfl_xor(lsum, 32);
  if constexpr (KSPLIT) {
    // Wave w + 2 hands its reference, sum and accumulators (in its own lane
    // layout) to wave w through the K buffers, free after the last tile's
    // barrier; wave w merges them under the larger reference.
    constexpr int NX = MB * 16 + 2;  // floats per lane
    float* xs = (float*)&Ks[0][0][0] + (size_t)wr * NX * 64 + l;
    if (kh == 1 && wave_live) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) xs[(mb * 16 + i) * 64] = oacc[mb][i];
      xs[(MB * 16) * 64] = m;
      xs[(MB * 16 + 1) * 64] = lsum;
    }
    __syncthreads();
    if (kh == 1) return;
    if (wave_live) {
      const float m2 = xs[(MB * 16) * 64], l2 = xs[(MB * 16 + 1) * 64];
      const float mn = fmaxf(m, m2);
      const float a = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - mn);
      const float a2 = m2 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m2 - mn);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[mb][i] = oacc[mb][i] * a + xs[(mb * 16 + i) * 64] * a2;
      lsum = lsum * a + l2 * a2;
      m = mn;
    }
  }
  if (!rok) return;
  const size_t orow = ((size_t)b * C + qi) * Hq + qh;
  if (direct) {
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int f = mb * 32 + 8 * j + 4 * h;
        u32x2 o2 = {pack_bf16x2(oacc[mb][4 * j] * inv, oacc[mb][4 * j + 1] * inv),
                    pack_bf16x2(oacc[mb][4 * j + 2] * inv, oacc[mb][4 * j + 3] * inv)};
        *(u32x2*)(O + orow * DH + f) = o2;
      }
    if (lse_out && h == 0) lse_out[orow] = (m + log2f(lsum)) * kLn2;
  } else {
    const size_t nrows = (size_t)B * C * Hq;
    float* op = Opart + ((size_t)split * nrows + orow) * DH;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int f = mb * 32 + 8 * j + 4 * h;
        *(f32x4*)(op + f) = f32x4{oacc[mb][4 * j], oacc[mb][4 * j + 1], oacc[mb][4 * j + 2],
                                  oacc[mb][4 * j + 3]};
      }
    if (h == 0) {
      mpart[split * nrows + orow] = m;
      lpart[split * nrows + orow] = lsum;
    }
  }
}

// Merge of the key splits: O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s,
// splits in a fixed order (deterministic).  Rows (b, i, h) of the canvas
// positions i >= first (the rows before are written directly); a row of a row
// block that was written directly is skipped.
constexpr int kAttnMaxSplits = 512;  // attn_plan makes at most 512 splits
constexpr int kAttnFewSplits = 8;    // at most this many: k_attn_combine_few

__device__ __forceinline__ bool attn_merge_row(int ridx, int mrows, int C, int L, int Hq, int G, int causal,
                                               int kps, int first, int& r) {
  if (ridx >= mrows) return false;
  const int span = (C - first) * Hq;
  const int bb = ridx / span, rem = ridx % span;
  const int i = first + rem / Hq, hq = rem % Hq;
  r = (bb * C + i) * Hq + hq;
  return attn_key_limit(causal, L, C, G, (i * G + hq % G) / 128) > kps;
}

// Many splits (few rows): one row per workgroup of 128 threads; one wave
// computes the split weights into LDS, every thread then merges one feature.
__global__ void __launch_bounds__(128)
    k_attn_combine_bf16(int nrows, int mrows, int nsplit, int dh, int C, int L, int Hq, int G, int causal,
                        int kps, int first, const float* __restrict__ Opart, const float* __restrict__ mpart,
                        const float* __restrict__ lpart, u16* __restrict__ O, float* __restrict__ lse_out) {
  __shared__ float wgt[kAttnMaxSplits];
  __shared__ float sh[2];
  const int ridx = blockIdx.x;
  const int span = (C - first) * Hq;
  const int bb = ridx / span, rem = ridx % span;
  const int i = first + rem / Hq, hq = rem % Hq;
  const bool live = ridx < mrows && attn_key_limit(causal, L, C, G, (i * G + hq % G) / 128) > kps;
  const int r = (bb * C + i) * Hq + hq;
  if (live && threadIdx.x < 64) {
    // one wave: lane l takes splits l, l+64, ...; fixed-pattern reductions
    const int l = threadIdx.x;
    float M = -INFINITY;
    for (int s = l; s < nsplit; s += 64) M = fmaxf(M, mpart[(size_t)s * nrows + r]);
    for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
    float part = 0.f;
    for (int s = l; s < nsplit; s += 64) {
      const float ms = mpart[(size_t)s * nrows + r];
      const float ws = ms == -INFINITY ? 0.f : exp2f(ms - M);
      wgt[s] = ws;
      part += ws == 0.f ? 0.f : ws * lpart[(size_t)s * nrows + r];
    }
    for (int o = 32; o > 0; o >>= 1) part += __shfl_xor(part, o);
    if (l == 0) {
      sh[0] = part > 0.f ? 1.f / part : 0.f;
      sh[1] = (M + log2f(part)) * kLn2;
    }
  }
  __syncthreads();
  if (!live) return;
  const float inv = sh[0];
  // splits in a fixed order; 8 independent loads in flight per thread
  for (int f = threadIdx.x; f < dh; f += 128) {
    float acc = 0.f;
    const float* op = Opart + (size_t)r * dh + f;
    const size_t st = (size_t)nrows * dh;
    int s = 0;
    for (; s + 8 <= nsplit; s += 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = op[(size_t)(s + u) * st];
#pragma unroll
      for (int u = 0; u < 8; ++u) acc += wgt[s + u] == 0.f ? 0.f : wgt[s + u] * v[u];
    }
    for (; s < nsplit; ++s) acc += wgt[s] == 0.f ? 0.f : wgt[s] * op[(size_t)s * st];
    O[(size_t)r * dh + f] = (u16)f32_to_bf16(acc * inv);
  }
  if (lse_out && threadIdx.x == 0) lse_out[r] = sh[1];
}

// Few splits (many rows): one row per wave, four per workgroup.  Every lane
// issues all its loads at once (the split maxima and sums, and its dh / 64
// features of every split), so a row costs one memory round trip; every lane
// forms the same weights from the same values, with no LDS and no barrier.
__global__ void __launch_bounds__(256)
    k_attn_combine_few(int nrows, int mrows, int nsplit, int dh, int C, int L, int Hq, int G, int causal,
                       int kps, int first, const float* __restrict__ Opart, const float* __restrict__ mpart,
                       const float* __restrict__ lpart, u16* __restrict__ O, float* __restrict__ lse_out) {
  int r = 0;
  if (!attn_merge_row(blockIdx.x * 4 + (threadIdx.x >> 6), mrows, C, L, Hq, G, causal, kps, first, r)) return;
  const int l = threadIdx.x & 63;
  const size_t st = (size_t)nrows * dh;
  float ms[kAttnFewSplits], ls[kAttnFewSplits], v[kAttnFewSplits][2];
#pragma unroll
  for (int s = 0; s < kAttnFewSplits; ++s) {
    if (s < nsplit) {
      ms[s] = mpart[(size_t)s * nrows + r];
      ls[s] = lpart[(size_t)s * nrows + r];
#pragma unroll
      for (int j = 0; j < 2; ++j)
        v[s][j] = 64 * j + l < dh ? Opart[(size_t)s * st + (size_t)r * dh + 64 * j + l] : 0.f;
    }
  }
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < kAttnFewSplits; ++s)
    if (s < nsplit) M = fmaxf(M, ms[s]);
  float part = 0.f, acc[2] = {0.f, 0.f};
#pragma unroll
  for (int s = 0; s < kAttnFewSplits; ++s) {
    if (s < nsplit) {
      const float ws = ms[s] == -INFINITY ? 0.f : exp2f(ms[s] - M);
      if (ws != 0.f) {
        part += ws * ls[s];
        acc[0] += ws * v[s][0];
        acc[1] += ws * v[s][1];
      }
    }
  }
  const float inv = part > 0.f ? 1.f / part : 0.f;
#pragma unroll
  for (int j = 0; j < 2; ++j)
    if (64 * j + l < dh) O[(size_t)r * dh + 64 * j + l] = (u16)f32_to_bf16(acc[j] * inv);
  if (lse_out && l == 0) lse_out[r] = (M + log2f(part)) * kLn2;
}

// ---------------------------------------------------------------------------
// fp32-storage path: one workgroup per (b, i, h) query row, keys in chunks of
// 256 (one per lane), online softmax in fp64 (exp/log in double), lane f < dh
// accumulates output feature f in fp64; only the stored O is rounded.  For
// the small fp32 workloads.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) k_attn_f32(int B, int C, int L, int cap, int Hq, int Hkv,
                                                  int G, int dh, int causal,
                                                  const float* __restrict__ Q,
                                                  const float* __restrict__ Kc,
                                                  const float* __restrict__ Vc,
                                                  const float* __restrict__ Kn,
                                                  const float* __restrict__ Vn,
                                                  float* __restrict__ O, float* __restrict__ lse_out) {
  __shared__ double qs[256], ps[256], red[256];
  const int r = blockIdx.x;
  const int hq = r % Hq, i = (r / Hq) % C, b = r / (Hq * C);
  const int g = hq / G;
  const int tid = threadIdx.x;
  if (tid < dh) qs[tid] = (double)Q[(size_t)r * dh + tid];
  __syncthreads();
  const double scale = 1.0 / sqrt((double)dh);
  const int nkeys = causal ? L + i + 1 : L + C;  // causal: keys past L + i are masked
  double m = -INFINITY, lsum = 0.0, oacc = 0.0;
  for (int j0 = 0; j0 < nkeys; j0 += 256) {
    const int j = j0 + tid;
    double s = -INFINITY;
    if (j < nkeys && (!causal || j <= L + i)) {
      const float* kp = j < L ? Kc + (((size_t)b * Hkv + g) * cap + j) * dh
                              : Kn + (((size_t)b * C + (j - L)) * Hkv + g) * dh;
      double acc = 0.0;
      for (int f = 0; f < dh; ++f) acc = fma(qs[f], (double)kp[f], acc);
      s = acc * scale;
    }
    red[tid] = s;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
      if (tid < o) red[tid] = fmax(red[tid], red[tid + o]);
      __syncthreads();
    }
    const double mnew = fmax(m, red[0]);
    __syncthreads();
    const double alpha = (mnew == -INFINITY) ? 1.0 : exp(m - mnew);
    const double p = (s == -INFINITY) ? 0.0 : exp(s - mnew);
    ps[tid] = p;
    red[tid] = p;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
      if (tid < o) red[tid] += red[tid + o];
      __syncthreads();
    }
    lsum = lsum * alpha + red[0];
    m = mnew;
    if (tid < dh) {
      double acc = oacc * alpha;
      const int jn = min(256, nkeys - j0);
      for (int jj = 0; jj < jn; ++jj) {
        const int jk = j0 + jj;
        const float* vp = jk < L ? Vc + (((size_t)b * Hkv + g) * cap + jk) * dh
                                 : Vn + (((size_t)b * C + (jk - L)) * Hkv + g) * dh;
        acc = fma(ps[jj], (double)vp[tid], acc);
      }
      oacc = acc;
    }
    __syncthreads();
  }
  if (tid < dh) O[(size_t)r * dh + tid] = (float)(oacc / lsum);
  if (lse_out && tid == 0) lse_out[r] = (float)(m + log(lsum));
}

// ---------------------------------------------------------------------------
// Causal passes: row block rb sees about L + (rb + 1) 64 keys, so the last
// blocks set the critical path.  Candidate split counts from ns0 up are
// scored in units of one tile's time: list scheduling in dispatch order
// (longest row blocks first, split by split), each XCD taking its eighth of
// the grid on its own 64 slots (32 CUs, two workgroups each), with one tile
// of fixed cost per workgroup that has keys, plus the partials'
// write and read at kAttnTileBytes per tile time (the chip moves about
// 12 MB from HBM in the ~3 us a workgroup spends on one tile).  The lowest
// score wins, the fewest splits on a tie.
constexpr double kAttnTileBytes = 12e6;
static int attn_causal_splits(int B, int C, int L, int Hq, int Hkv, int G, int dh, int nrb, int ns0,
                              int maxs) {
  const int nkeys = L + C;
  int best = ns0;
  double best_span = 1e300;
  std::vector<double> slot;
  for (int ns = ns0; ns <= maxs && ns <= 4 * ns0; ++ns) {
    const int kps = ((nkeys + ns - 1) / ns + 63) / 64 * 64;
    const int nsp = (nkeys + kps - 1) / kps;
    const long total = (long)nrb * nsp * Hkv * B, chunk = (total + 7) / 8;
    // per XCD, a min-heap of the times at which its 64 slots come free
    slot.assign(8 * 64, 0.0);
    auto put = [&](int x, double len) {
      auto b0 = slot.begin() + 64 * x, b1 = b0 + 64;
      std::pop_heap(b0, b1, std::greater<double>());
      *(b1 - 1) += len;
      std::push_heap(b0, b1, std::greater<double>());
    };
    long idx = 0;
    for (int bg = 0; bg < B * Hkv; ++bg)
      for (int sp = 0; sp < nsp; ++sp)
        for (int k = 0; k < nrb; ++k, ++idx) {
          const int rb = nrb - 1 - k;
          const int lim = attn_key_limit(1, L, C, G, rb);
          const int kb = sp * kps, ke = lim < kb + kps ? lim : kb + kps;
          const double len = (lim <= kps && sp > 0) ? 0.0 : (ke > kb ? 1.0 + (ke - kb + 63) / 64 : 0.25);
          put((int)(idx / chunk), len);
        }
    int rb0 = 0;
    while (rb0 < nrb && attn_key_limit(1, L, C, G, rb0) <= kps) ++rb0;
    const double merged = nsp > 1 ? (double)B * (C - (rb0 < nrb ? rb0 * 128 / G : C)) * Hq : 0.0;
    const double span = *std::max_element(slot.begin(), slot.end()) +
                        2.0 * merged * nsp * (dh + 2) * 4.0 / kAttnTileBytes;
    if (span < best_span) {
      best_span = span;
      best = ns;
    }
  }
  return best;
}

AttnPlan attn_plan(int B, int C, int L, int cap, int Hq, int Hkv, int dh, int dtype, int causal) {
  AttnPlan p{};
  p.B = B; p.C = C; p.L = L; p.cap = cap; p.Hq = Hq; p.Hkv = Hkv; p.dh = dh; p.dtype = dtype;
  p.causal = causal;
  const int nkeys = L + C;
  if (dtype == 1) {
    const int G = Hq / Hkv;
    p.nrb = (C * G + 127) / 128;
    const int pairs = B * Hkv * p.nrb;
    int ns = (512 + pairs - 1) / pairs;             // about two workgroups per CU
    const int maxs = (nkeys + 127) / 128;           // at least two 64-key tiles per split
    ns = ns < 1 ? 1 : (ns > maxs ? maxs : ns);
    // At most kAttnFewSplits splits when that still gives every CU a
    // workgroup: the merge then takes one memory round trip per row
    // (k_attn_combine_few).  At 256 queries over 8448 keys, 8 splits measured
    // 40.0 us (kernel + combine) against 41.7 us for 15.
    if (ns > kAttnFewSplits && pairs * kAttnFewSplits >= 256) ns = kAttnFewSplits;
    if (causal) ns = attn_causal_splits(B, C, L, Hq, Hkv, G, dh, p.nrb, ns, maxs);
    p.keys_per_split = ((nkeys + ns - 1) / ns + 63) / 64 * 64;
    p.nsplit = (nkeys + p.keys_per_split - 1) / p.keys_per_split;
    if (p.nsplit < 1) p.nsplit = 1;
    // the first canvas position with a row in a split row block (row blocks
    // past it see at least as many keys)
    int rb0 = 0;
    while (rb0 < p.nrb && attn_key_limit(causal, L, C, G, rb0) <= p.keys_per_split) ++rb0;
    p.merge_first = rb0 < p.nrb ? rb0 * 128 / G : C;
    p.part_bytes = p.merge_first < C ? (size_t)p.nsplit * B * C * Hq * (dh + 2) * sizeof(float) : 0;
  } else {
    p.nrb = 1; p.nsplit = 1; p.keys_per_split = nkeys; p.part_bytes = 0; p.merge_first = C;
  }
  return p;
}

hipError_t launch_attn(const AttnPlan& p, const void* q, const void* kc, const void* vc,
                       const void* kn, const void* vn, void* out, float* lse, void* ws,
                       hipStream_t s, hipEvent_t ev_begin, hipEvent_t ev_end) {
  const int G = p.Hq / p.Hkv;
  const size_t nrows = (size_t)p.B * p.C * p.Hq;
  if (nrows == 0) return hipSuccess;
  if (ev_begin) {
    hipError_t e = hipEventRecord(ev_begin, s);
    if (e != hipSuccess) return e;
  }
  if (p.dtype != 1) {
    hipLaunchKernelGGL(k_attn_f32, dim3((unsigned)nrows), dim3(256), 0, s, p.B, p.C, p.L, p.cap,
                       p.Hq, p.Hkv, G, p.dh, p.causal, (const float*)q, (const float*)kc,
                       (const float*)vc, (const float*)kn, (const float*)vn, (float*)out, lse);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess && ev_end) e = hipEventRecord(ev_end, s);
    return e;
  }
  float* Opart = (float*)ws;
  float* mpart = Opart + (size_t)p.nsplit * nrows * p.dh;
  float* lpart = mpart + (size_t)p.nsplit * nrows;
  const dim3 grid((unsigned)((p.nrb * p.nsplit * p.Hkv * p.B + 7) / 8 * 8));
  const bool ksplit = p.C * G <= 64;  // one row block with at most two row groups
#define DG_ATTN_LAUNCH(DHV, KSPLITV)                                                              \
  hipLaunchKernelGGL((k_attn_bf16<DHV, KSPLITV>), grid, dim3(256), 0, s, p.B, p.C, p.L, p.cap, p.Hq, p.Hkv, \
                     G, p.causal, p.nrb, p.nsplit, p.keys_per_split, (const u16*)q,                \
                     (const u16*)kc, (const u16*)vc, (const u16*)kn, (const u16*)vn, (u16*)out,    \
                     lse, Opart, mpart, lpart)
  if (p.dh == 128 && ksplit)
    DG_ATTN_LAUNCH(128, true);
  else if (p.dh == 128)
    DG_ATTN_LAUNCH(128, false);
  else if (ksplit)
    DG_ATTN_LAUNCH(64, true);
  else
    DG_ATTN_LAUNCH(64, false);
#undef DG_ATTN_LAUNCH
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && ev_end) e = hipEventRecord(ev_end, s);
  if (e != hipSuccess || p.merge_first >= p.C) return e;
  const size_t mrows = (size_t)p.B * (p.C - p.merge_first) * p.Hq;
  if (p.nsplit <= kAttnFewSplits)
    hipLaunchKernelGGL(k_attn_combine_few, dim3((unsigned)((mrows + 3) / 4)), dim3(256), 0, s, (int)nrows,
                       (int)mrows, p.nsplit, p.dh, p.C, p.L, p.Hq, G, p.causal, p.keys_per_split,
                       p.merge_first, Opart, mpart, lpart, (u16*)out, lse);
  else
    hipLaunchKernelGGL(k_attn_combine_bf16, dim3((unsigned)mrows), dim3(128), 0, s, (int)nrows,
                       (int)mrows, p.nsplit, p.dh, p.C, p.L, p.Hq, G, p.causal, p.keys_per_split,
                       p.merge_first, Opart, mpart, lpart, (u16*)out, lse);
  return hipGetLastError();
}

}  // namespace dg
