// Flash-vocab: the tied vocabulary head, its full-vocabulary softmax with the
// per-row max probability ("confidence"), and self-conditioning S = P . E
// (DiffusionGemma explainer, "Autocondizionamento": the probability matrix
// times the token-embedding table is handed to the next step), in one pass
// over the embedding table E that never stores the rows x V probabilities.
#include "vocab_common.h"

#include <atomic>

namespace dg {

// ---------------------------------------------------------------------------
// Variant 32 (d = 4*SLICE <= 2048).  Workgroup = 4 waves, 32 rows of Z, one
// vocab split; wave w owns the d-slice [w*SLICE, (w+1)*SLICE).  Vocab tiles
// hold 16 ids, and three tiles are in flight: iteration t computes the
// logits of tile t, the softmax of tile t-1 and the self-conditioning
// product of tile t-2, so the softmax work runs between the matrix-core
// instructions instead of stalling them.  Lane l = 16 g + r.
//
// Per tile and 32-column chunk c of its slice, wave w accumulates the partial
//   lg^T[v][row] += E[v, chunk] . Z[row, chunk]^T        (16x16x32, rows 16h..)
// with A = one block of the tiled E (16 ids x 32 columns, 1 KiB read by one
// load instruction) and B = Z fragments in VGPRs.  The block is also written
// to LDS (buffer t & 1, over tile t-2's data right after it was read) and
// later read back transposed for
//   S^T[col][row] += E[tile, col]^T . P^T                (32x32x16)
// whose B operand, P^T, comes from an LDS tile that the softmax step writes in
// operand order.
//
// Softmax of a tile: the four d-slice partials are exchanged through LDS (at
// rotated lane positions: conflict-free); wave w owns rows 8w..8w+7, sums
// their partials (lane 8 rho + q: ids 2q, 2q+1 of row 8w + rho), reduces max /
// first argmax over the 8 lanes of a row with DPP, keeps the row's reference
// m_seg, running max / argmax and part of the running sum, and writes P
// (bf16) and the row's fold factor to LDS.
//
// P = exp(l - m_seg) uses a reference that only moves when a logit exceeds it
// by more than kLazyTh; then s = e^(m_old - m_new) rescales the running sum
// at once and, after the product of the tile before has been accumulated,
// every wave folds its accumulator into the split's partial in global memory,
// G = (G + acc) s, and starts a zero accumulator (the accumulator is only
// ever stored raw, so it stays in the AGPR file).  Output: G (unnormalised,
// relative to the final m_seg) and per-row (m_seg, sum, max, argmax).
// ---------------------------------------------------------------------------
template <int SLICE>
__global__ void __launch_bounds__(256, 1)
    k_vocab32(const u16* __restrict__ Z, const u16* __restrict__ E, int R, int d, int V, int nrb,
              int split_len, float* __restrict__ pS, f32x4* __restrict__ pstat) {
  constexpr int NCH = SLICE / 32, EP = SLICE + 8;
  constexpr int PF = NCH < DG_VOCAB32_PF ? NCH : DG_VOCAB32_PF;  // chunks of E in flight
  // chunk c of every tile lives in ring slot c % PF, which needs PF | NCH
  static_assert(NCH % PF == 0, "the prefetch depth must divide the chunks per tile");
  // chunks at which the softmax steps of the previous tile run: every LDS
  // result is consumed two chunks after it was requested, so its latency
  // hides behind matrix-core work instead of stalling the wave's issue
  constexpr int kRdX = 0;                      // request the partials
  constexpr int kSum = NCH > 2 ? 2 : NCH - 1;  // sum them, first reductions
  constexpr int kRed = NCH > 3 ? 3 : NCH - 1;  // finish max / argmax
  constexpr int kExp = NCH > 4 ? 4 : NCH - 1;  // reference, P, fold factor
  __shared__ __attribute__((aligned(16))) u16 Et[2][4][16][EP];
  // softmax exchange buffers, double-buffered by tile parity so that one
  // barrier per iteration suffices
  __shared__ __attribute__((aligned(16))) f32x4 xch[2][4][2][64];  // [tile & 1][wave][h][rotated lane]
  __shared__ __attribute__((aligned(16))) u32x4 Pbuf[2][2][32];     // [tile & 1]: P of row m, ids 8k..8k+7
  __shared__ float Sbuf[2][32];                                     // [tile & 1]: per-row fold factor
  __shared__ int flags[2][4];

  const int w = threadIdx.x >> 6, l = threadIdx.x & 63, g = l >> 4, r = l & 15;
  const int h2 = l >> 5, m32 = l & 31;
  int rb, split;
  vocab_block(nrb, rb, split);
  const int r0 = rb * 32;
  const int vs = split * split_len, ve = min(V, vs + split_len);
  const int dbase = w * SLICE;
  const u32x4 z4 = {0u, 0u, 0u, 0u};
  const size_t tofs = (size_t)gridDim.x / nrb * R * d;  // temp area follows the nsplit partials

  // Rows 16h + r of the block.  Rows past R load a copy of row R-1
  // (branch-free); their results are never stored.
  u32x4 zf[2][NCH];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const u16* zp = Z + (size_t)min(r0 + 16 * h + r, R - 1) * d + dbase + 8 * g;
#pragma unroll
    for (int c = 0; c < NCH; ++c) zf[h][c] = swap_halves(ldg128(zp + 32 * c), g & 1);
  }

  const int nt = ve > vs ? (ve - vs + 15) / 16 : 0;
  // Tile order: the 8 row blocks of a split stream the same E tiles.  In
  // lockstep every workgroup would wait the full HBM latency on every load,
  // with only one workgroup's worth of distinct bytes in flight per split.
  // Instead, within each round of 8 tiles, row block rb starts at tile
  // (rb + s) % 8 of the round: the first step of a round fetches 8 tiles
  // at once, the other 7 find their tiles in L2.  A last partial round goes
  // in order.
  const int nt8 = nt & ~7;
  auto phys = [&](int s) { return s < nt8 ? (s & ~7) | ((s + rb) & 7) : s; };
  {
    DG_LDS u16* e0p = (DG_LDS u16*)&Et[0][w][0][0];
    DG_LDS u16* e1p = (DG_LDS u16*)&Et[1][w][0][0];
    for (int e = l * 8; e < 16 * EP; e += 64 * 8) {
      *(DG_LDS u32x4*)(e0p + e) = z4;
      *(DG_LDS u32x4*)(e1p + e) = z4;
    }
  }
  // this lane's LDS offsets (elements) inside a wave's tile: the 16 bytes it
  // loaded (id r, columns 8g..8g+7 of a chunk), and the transposing reads of
  // ids 8 h2 + 4k + (0..3) at column m32 of a chunk (k = 0, 1)
  const int wr_a = prow16t(r) * EP + 8 * g + ((g & 1) ? 4 : 0), wr_b = wr_a ^ 4;
  int tr_off[2];
#pragma unroll
  for (int k = 0; k < 2; ++k)
    tr_off[k] = prow16t(8 * h2 + 4 * k + ((l & 15) >> 2)) * EP + 16 * ((l >> 4) & 1) + 4 * (l & 3);

  // E blocks of chunk c live in ring slot c % PF, issued PF chunks ahead.
  // E is the tiled table: the 16 bytes this lane needs sit at lane position l
  // of a contiguous 1 KiB block.  The buffer resource ends at the table's end
  // (ids past it read zeros); ids outside the split are masked to -inf.
  const uint32_t blk_row = (uint32_t)d * 32u;  // bytes of the d/32 blocks of 16 ids
  const __amdgpu_buffer_rsrc_t erc = buffer_rsrc(E, (uint32_t)(((size_t)V + 15) / 16 * blk_row));
  const uint32_t lane_off = (uint32_t)((size_t)(vs / 16) * blk_row + (size_t)(w * NCH) * 1024u + l * 16u);
  u32x4 ring[PF];
  auto issue = [&](int slot, int step, int c) {
    ring[slot] = buffer_ld128(erc, lane_off + (uint32_t)phys(step) * blk_row + 1024u * c);
  };
#pragma unroll
  for (int c = 0; c < PF; ++c) issue(c, 0, c);

  // A operands of the P.E product: ids 8 h2 .. 8 h2 + 7 at column m32 of a
  // chunk; chunk c's sits in slot c & 1 and is read two chunks ahead
  u32x4 tra[2];
  auto tr_load = [&](const DG_LDS u16* tile, int c, int slot) {
    const u32x2 a = lds_read_tr16(tile + tr_off[0] + 32 * c);
    const u32x2 b = lds_read_tr16(tile + tr_off[1] + 32 * c);
    tra[slot] = u32x4{a[0], a[1], b[0], b[1]};
  };
  // zeros: tile -2 adds 0 * 0
  tr_load((const DG_LDS u16*)&Et[0][w][0][0], 0, 0);
  tr_load((const DG_LDS u16*)&Et[0][w][0][0], NCH > 1 ? 1 : 0, 1);

  // softmax state of the owned row 8w + rho (lane 8 rho + q holds ids 2q, 2q+1)
  const int rho = l >> 3, q = l & 7, orow = 8 * w + rho;
  float m_seg = -INFINITY, lsum = 0.f, m_true = -INFINITY;
  int amax = 0;
  bool g_valid = false;
  u32x4 pf = z4;  // P^T operand of tile t-2
  f32x4 lg[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
  // partial-logit exchange positions: lane (g, r) writes at 16g + ((r + 4g) & 15)
  const int xw = 16 * g + ((r + 4 * g) & 15);
  const int xr = 16 * (q >> 1) + ((8 * (w & 1) + rho + 4 * (q >> 1)) & 15);

  for (int e = threadIdx.x; e < 2 * 2 * 32; e += 256) (&Pbuf[0][0][0])[e] = z4;
  if (threadIdx.x < 8) (&flags[0][0])[threadIdx.x] = 0;
  int t = 0;
  bool top_done = false;  // iteration t's barrier and reads already ran (it stopped for a fold)
  bool fold_now = false;
  for (;;) {  // segments
    f32x16 acc[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) acc[c] = zero16();
    bool last = false;
    for (;; ++t) {  // iterations: logits(t), softmax(t-1), P.E(t-2)
      if (!top_done) {
        // every wave's partial logits of tile t-1 (written at the end of the
        // previous iteration) and the softmax of tile t-2 become visible
        __syncthreads();
        pf = Pbuf[t & 1][h2][m32];
        const int* fl = flags[t & 1];
        fold_now = t >= 2 && (fl[0] | fl[1] | fl[2] | fl[3]) != 0;
        if (fold_now) {
          top_done = true;  // fold before P.E(t-2), then run iteration t
          break;
        }
      }
      top_done = false;
      const bool more = t <= nt;  // an iteration t = nt + 1 only finishes P.E(nt - 1)
      DG_LDS u16* tile = (DG_LDS u16*)&Et[t & 1][w][0][0];
      const int tp = (t - 1) & 1;                            // parity of tile t-1
      const bool prev_ok = t >= 1 && t - 1 < nt;             // step t-1 is a real tile
      const int v1 = vs + 16 * (prev_ok ? phys(t - 1) : 0);  // its first id
      float x0 = 0.f, x1 = 0.f, tm = -INFINITY;
      int ta = 0;
      f32x4 xa[4];
      lg[0] = f32x4{0.f, 0.f, 0.f, 0.f};
      lg[1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const int slot = c % PF;
        const u32x4 e = ring[slot];
        mfma16x32_v(e, zf[0][c], lg[0]);
        mfma16x32_v(e, zf[1][c], lg[1]);
        acc[c] = mfma32(tra[c & 1], pf, acc[c]);
        // chunk c+2 of tile t-2 (overwritten only two chunks later, after
        // this read), or chunks 0 and 1 of tile t-1 for the next iteration
        if (c + 2 < NCH)
          tr_load(tile, c + 2, c & 1);
        else if (NCH > 1)
          tr_load((const DG_LDS u16*)&Et[(t + 1) & 1][w][0][0], c + 2 - NCH, c & 1);
        else
          tr_load((const DG_LDS u16*)&Et[(t + 1) & 1][w][0][0], 0, 0);
        // 8-byte LDS writes run at twice the rate of 16-byte ones (the tiled
        // layout puts each lane's halves in the order that keeps them
        // conflict-free)
        *(DG_LDS u32x2*)(tile + wr_a + 32 * c) = u32x2{e[0], e[1]};
        *(DG_LDS u32x2*)(tile + wr_b + 32 * c) = u32x2{e[2], e[3]};
        if (c + PF < NCH)
          issue(slot, t, c + PF);
        else
          issue(slot, t + 1, c + PF - NCH);

        // ---- softmax of tile t-1, spread over the chunks ----
        if (c == kRdX) {
#pragma unroll
          for (int s = 0; s < 4; ++s) xa[s] = xch[tp][s][w >> 1][xr];
        }
        if (c == kSum) {
          const f32x4 a = ((xa[0] + xa[1]) + xa[2]) + xa[3];
          const bool hi2 = q & 1;  // ids 2q, 2q+1 are elements 2(q & 1) + (0, 1)
          const int id = v1 + 2 * q;
          x0 = prev_ok && id < ve ? (hi2 ? a[2] : a[0]) : -INFINITY;
          x1 = prev_ok && id + 1 < ve ? (hi2 ? a[3] : a[1]) : -INFINITY;
          const bool second = x1 > x0;
          tm = second ? x1 : x0;
          ta = second ? id + 1 : id;
          argmax_step<0xB1>(tm, ta);
        }
        if (c == kRed) {
          argmax_step<0x4E>(tm, ta);
          argmax_step<0x141>(tm, ta);
        }
        if (c == kExp) {
          // tiles come out of id order: ties go to the lower id
          const bool better = (tm > m_true) | ((tm == m_true) & (tm != -INFINITY) & (ta < amax));
          amax = better ? ta : amax;
          m_true = fmaxf(m_true, tm);
          // Lazy reference: it only moves when a logit exceeds it by more than
          // kLazyTh; the running sum is then rescaled by s = e^(m_old - m_new).
          const bool first = m_seg == -INFINITY;
          const bool over = !first & (tm > m_seg + kLazyTh);
          const float s = over ? exp2f((m_seg - tm) * kLog2e) : 1.f;
          m_seg = (first | over) ? tm : m_seg;
          // the normaliser sums the fp32 probabilities; bf16 copies feed P.E
          const float p0 = x0 == -INFINITY ? 0.f : exp2f((x0 - m_seg) * kLog2e);
          const float p1 = x1 == -INFINITY ? 0.f : exp2f((x1 - m_seg) * kLog2e);
          lsum = lsum * s + (p0 + p1);
          *(DG_LDS uint32_t*)((DG_LDS char*)&Pbuf[tp][q >> 2][orow] + 4 * (q & 3)) = pack_bf16x2(p0, p1);
          if (q == 0) Sbuf[tp][orow] = s;
          const bool need_w = __any(s != 1.f);
          if (l == 0) flags[tp][w] = need_w ? 1 : 0;
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      mfma_v_settle(lg[0], lg[1]);
      // this tile's partial logits, for the owners in the next iteration
#pragma unroll
      for (int h = 0; h < 2; ++h) xch[t & 1][w][h][xw] = lg[h];
      if (!more) {
        last = true;
        break;
      }
    }

    // Fold the segment into G with the per-row factor s: G = (G + acc) s
    // (G = acc s on the first fold; s = 1 at the end of the split).  The first
    // fold stores the raw accumulator to G, a later one to the temp area T,
    // which is then merged with plain loads and stores.
    const int zr = r0 + m32;
    const float s = fold_now ? Sbuf[t & 1][m32] : 1.f;
    if (zr < R) {
      float* gp = pS + ((size_t)split * R + zr) * d + dbase + 4 * h2;
      float* dst = g_valid ? gp + tofs : gp;
#pragma unroll
      for (int c = 0; c < NCH; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *(f32x4*)(dst + 32 * c + 8 * j) =
              f32x4{acc[c][4 * j], acc[c][4 * j + 1], acc[c][4 * j + 2], acc[c][4 * j + 3]};
      if (g_valid || fold_now) {
        for (int c = 0; c < NCH; ++c)
          for (int j = 0; j < 4; ++j) {
            float* p = gp + 32 * c + 8 * j;
            f32x4 v = *(const f32x4*)p;
            if (g_valid) v += *(const f32x4*)(p + tofs);
            *(f32x4*)p = v * s;
          }
      }
    }
    g_valid = true;
    if (last) break;
    fold_now = false;
  }

  const float tot = sum8(lsum);
  if (r0 + orow < R && q == 0)
    pstat[(size_t)split * R + r0 + orow] = f32x4{m_seg, tot, m_true, __int_as_float(amax)};
}

// ---------------------------------------------------------------------------
// Variant 64g (d = Q * 1024, Q = 2 or 4): a group of Q workgroups on one XCD
// shares 64 rows.  With 32 rows per workgroup every E byte feeds too little
// matrix-core work: one 64-cycle chunk needs 4 KiB of E from L2 and 8 KiB of
// LDS traffic per CU, more than either path delivers.  Here a workgroup (a
// member of the group) owns 64 rows and 1024 of the columns of S = P.E (so
// its accumulators still fit the AGPR file): per 16-id tile it reads only its
// 1024 columns of E (32 KiB) for 2x the rows.  The logits need the full-width
// contraction, so the members swap their partial logits through the XCD's
// L2: each writes its 64 x 16 partial as tagged records and polls the
// others' until all tags match (no ordering between stores is needed; every
// member adds the Q partials in member order, so all compute bit-identical
// softmax results).  Every poll loop is bounded: on timeout it raises an
// error flag (the combine then writes NaN statistics) and stops waiting, so
// no wave can hang.
//
// Grouping: workgroup = 4 waves, one per SIMD, one per CU (LDS).  A workgroup
// reads its XCD id from the hardware and takes a ticket from that XCD's
// counter; tickets Qk .. Qk+Q-1 on XCD x form group x * (grid/8/Q) + k
// (member = ticket % Q), so members always share an L2 whatever the dispatch
// order.  The exchange needs every member of a group resident at once, which
// another kernel on the GPU can prevent; so the members first agree, through
// one word per group, whether the group runs paired or solo: each sets its
// bit; a member that finds every bit set runs paired; one that waits longer
// than a bound for the others marks the group solo (compare-and-swap on the
// same word, so the decision is the same for every member).  A solo member
// computes the other members' partial logits itself, with the same products
// in the same order, and produces the same bits as a paired run.
// The counters, tags and group words are cleared before each launch.
//
// Pipeline of the paired run (iteration t, 8 chunks of 32 columns per wave):
//   logits of tile t            all chunks (E streamed through registers)
//   partial of tile t-1         LDS exchange of the 4 waves, summed, stored
//   softmax of tile t-2         after the other members' partials arrived
//   P.E of tile t-3             from the 4-deep LDS ring of E tiles
// Barriers sit at chunk boundaries where the LDS operations before them were
// issued a full chunk of matrix-core work earlier.
// ---------------------------------------------------------------------------
constexpr int kPairSlots = 4;                // exchange ring depth, in tiles
constexpr uint32_t kPairSpin = 1u << 20;     // poll bound of one exchange
constexpr uint32_t kGroupSpin = 1u << 14;    // poll bound of the start handshake
// header words: 0-7 tickets per XCD, 8 error flag, 9 exchange waits that
// had to poll, 10 poll timeouts, 11 workgroups without a ticket, 12-15 the
// first timeout (group, iteration, member | wave << 4, lane 0's generation
// bit), 16 solo members; words kGroupWord + g: the handshake word of group g
constexpr int kGroupWord = 64;
constexpr int kMaxGroups = 128;
constexpr int kPairHdrWords = kGroupWord + kMaxGroups;   // 768 bytes
constexpr uint32_t kGroupSolo = 1u << 8;
// exchange records of one member: kPairSlots slots of 256 lanes x 16 bytes
constexpr size_t kMemberRecBytes = (size_t)kPairSlots * 256 * 16;

// Exchange record of a lane: its 4 partial logits, each fp32 carrying the
// slot generation of its tile in its lowest mantissa bit.  A slot is reused
// every 4 tiles and a reader is never more than one generation behind, so one
// bit tells the wanted tile from the one before it.  The first generation has
// bit 1, so a slot that still holds the launch's cleared zeros never matches.
// Each 4-byte word is single-copy atomic, so a reader accepts the record once
// all four bits match.  The bit moves a partial by at most one ulp, and every
// member adds the same tagged values in the same order.  The members share
// an XCD: the store (through a buffer resource: no 64-bit lane address)
// reaches that XCD's L2, the vector L1 being write-through; the load is a
// device-scope global load, which misses the L1.  (A device-scope buffer load
// kept returning the L1's stale line on gfx950, in a ping-pong probe between
// paired workgroups.)
__device__ __forceinline__ uint32_t pair_gen(int tile) { return (uint32_t)((tile >> 2) + 1) & 1u; }
__device__ __forceinline__ f32x4 pair_tagged(f32x4 v, uint32_t gen) {
  f32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = __uint_as_float((__float_as_uint(v[i]) & ~1u) | gen);
  return o;
}
// all four tag bits equal gen: with m = gen - 1 (0, or all ones for gen 0),
// bit 0 of the AND of the words xor m is set
// (v_bitop3 truth table 0x42: (s0 ^ s2) & (s1 ^ s2))
__device__ __forceinline__ bool pair_gen_ok(u32x4 w, uint32_t gen) {
  const uint32_t m = gen - 1u;
  uint32_t a, b;
  asm("v_bitop3_b32 %0, %2, %3, %6 bitop3:0x42\n\tv_bitop3_b32 %1, %4, %5, %6 bitop3:0x42"
      : "=&v"(a), "=&v"(b)
      : "v"(w[0]), "v"(w[1]), "v"(w[2]), "v"(w[3]), "s"(m));
  return (a & b & 1u) != 0;
}
// true when ok holds in every lane of the wave (all lanes are active here)
__device__ __forceinline__ bool wave_all(bool ok) { return __builtin_amdgcn_ballot_w64(!ok) == 0; }
__device__ __forceinline__ u32x4 pair_load(const char* base, uint32_t off) {
  uint64_t* p = (uint64_t*)(const_cast<char*>(base) + off);
  const uint64_t a = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint64_t b = __hip_atomic_load(p + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return u32x4{(uint32_t)a, (uint32_t)(a >> 32), (uint32_t)b, (uint32_t)(b >> 32)};
}

// 16-byte unit, inside a 1 KiB LDS block of 16 ids x 32 columns, holding id i,
// columns 8gp..8gp+7 (gp < 4) as one lane of the tiled table stores them:
// 16 gp + (i ^ 4 gp).  Each 16-lane group of the staging stores (lanes
// 16g + r, one 16-byte store each) fills 16 distinct units of 4 banks, and
// each 32-lane group of the transposing reads (ids 4k + 0..3 or 8 + 4k +
// 0..3, all 8 column groups, 8 bytes each) covers the 64 banks once.  A
// padded row layout written with two 8-byte stores per lane conflicted on
// the stores.
__device__ __forceinline__ int pair_lds_unit(int i, int gp) { return 16 * gp + (i ^ (4 * gp)); }

// The start handshake of a group (thread 0 of each member): returns true when
// the group runs solo.  Every member's decision is read from the same word:
// paired iff all Q arrival bits were set before the solo mark.
// A bound of 0 marks the group solo at once (every member, deterministically).
template <int Q>
__device__ __forceinline__ bool group_handshake(uint32_t* word, int member, uint32_t spin) {
  const uint32_t full = (1u << Q) - 1u, mine = 1u << member;
  if (spin == 0) {
    __hip_atomic_fetch_or(word, mine | kGroupSolo, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return true;
  }
  uint32_t v = __hip_atomic_fetch_or(word, mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) | mine;
  for (uint32_t n = 0;; ++n) {
    if ((v & kGroupSolo) || (v & full) == full) break;
    if (n >= spin) {
      // mark the group solo unless the word changed since it was read
      uint32_t expect = v;
      if (__hip_atomic_compare_exchange_strong(word, &expect, v | kGroupSolo, __ATOMIC_RELAXED,
                                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
        v |= kGroupSolo;
        break;
      }
      v = expect;  // another member arrived meanwhile: decide again
      continue;
    }
    v = __hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  return (v & kGroupSolo) != 0;
}

template <int Q, bool PIN, bool MARK>
__global__ void __launch_bounds__(256, 1)
    k_vocab_group(const u16* __restrict__ Z, const u16* __restrict__ E, int R, int d, int V, int nrb,
                  int split_len, float* __restrict__ pS, f32x4* __restrict__ pstat,
                  uint32_t* __restrict__ xhdr, uint64_t* __restrict__ xrec, uint32_t group_spin) {
  constexpr int SLICE = 256, NCH = SLICE / 32;
  static_assert(Q == 2 || Q == 4, "groups of 2 or 4 workgroups");
  // [tile & 3][wave][chunk]: 1 KiB per chunk of 16 ids x 32 columns in 16-byte
  // units (pair_lds_unit), no padding
  __shared__ __attribute__((aligned(16))) u16 Et[4][4][NCH][512];
  __shared__ __attribute__((aligned(16))) f32x4 xch[4][4][64];      // [writer wave][row group][rotated lane]
  __shared__ __attribute__((aligned(16))) u32x4 Pbuf[2][64];        // P of row m, ids 8k..8k+7
  __shared__ float Sbuf[64];                                        // per-row fold factor
  __shared__ __attribute__((aligned(16))) int flags[4];
  __shared__ __attribute__((aligned(16))) f32x4 ownb[256];          // this member's partial, owner lane
  __shared__ int role[3];

  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), l = threadIdx.x & 63, g = l >> 4, r = l & 15;
  const int h2 = l >> 5, m32 = l & 31;
  if (threadIdx.x == 0) {
    const uint32_t xcc = __builtin_amdgcn_s_getreg((15 << 11) | 20) & 0xFu;  // HW_REG_XCC_ID
    const uint32_t quota = gridDim.x / 8;
    int grp = -1, mb = 0, solo = 0;
    if (xcc < 8) {
      const uint32_t tk = __hip_atomic_fetch_add(&xhdr[xcc], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (tk < quota) {
        grp = (int)(xcc * (quota / Q) + tk / Q);
        mb = (int)(tk % Q);
      }
    }
    if (grp < 0) {
      __hip_atomic_store(&xhdr[8], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_fetch_add(&xhdr[11], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      solo = group_handshake<Q>(&xhdr[kGroupWord + grp], mb, group_spin) ? 1 : 0;
      if (solo) __hip_atomic_fetch_add(&xhdr[16], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    role[0] = grp;
    role[1] = mb;
    role[2] = solo;
  }
  const u32x4 z4 = {0u, 0u, 0u, 0u};
  for (int e = threadIdx.x; e < 2 * 64; e += 256) (&Pbuf[0][0])[e] = z4;
  if (threadIdx.x < 4) flags[threadIdx.x] = 0;
  {
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      DG_LDS u16* ep = (DG_LDS u16*)&Et[b][w][0][0];
      for (int e = l * 8; e < NCH * 512; e += 64 * 8) *(DG_LDS u32x4*)(ep + e) = z4;
    }
  }
  __syncthreads();
  const int grp = __builtin_amdgcn_readfirstlane(role[0]), mb = __builtin_amdgcn_readfirstlane(role[1]);
  const bool solo = __builtin_amdgcn_readfirstlane(role[2]) != 0;
  if (grp < 0) return;  // the whole workgroup: no ticket (error raised)
  const int rb = grp % nrb, split = grp / nrb;
  const int r0 = rb * 64;
  const int vs = split * split_len, ve = min(V, vs + split_len);
  const int dq = d / Q;  // columns per member
  const int dbase = mb * dq + w * SLICE;
  const size_t tofs = (size_t)gridDim.x / Q / nrb * R * d;  // temp area follows the nsplit partials

  const int nt = ve > vs ? (ve - vs + 15) / 16 : 0;
  // the 4 row blocks that stream one split start at different tiles of each
  // round of 4, so one step fetches 4 distinct tiles from HBM
  const int nt4 = nt & ~3;
  auto phys = [&](int s) { return s < nt4 ? (s & ~3) | ((s + rb) & 3) : s; };

  // this lane's 16 bytes (id r, columns 8g..8g+7 of a chunk, in the tiled
  // table's order) go to one unit; the transposing reads take ids
  // 8 h2 + 4k + p/4, column group cg = 4 b4 + p % 4 (p = l % 16, b4 = bit 4
  // of l) from the 8-byte half of unit (id, cg / 2) that holds it (the odd
  // pairs store their upper half first).  Ids 4 apart flip bit 2 of the
  // unit's low part: the second read offset is the first with bit 5 flipped.
  const int wr = 8 * pair_lds_unit(r, g);
  int tr_off0;  // the second read is at tr_off0 ^ 32
  {
    const int p = l & 15, cg = 4 * ((l >> 4) & 1) + (p & 3), gp = cg >> 1;
    tr_off0 = 8 * pair_lds_unit(8 * h2 + (p >> 2), gp) + 4 * ((cg & 1) ^ (gp & 1));
  }

  const uint32_t blk_row = (uint32_t)d * 32u;
  const __amdgpu_buffer_rsrc_t erc = buffer_rsrc(E, (uint32_t)(((size_t)V + 15) / 16 * blk_row));
  const uint32_t lane_off = (uint32_t)((size_t)(vs / 16) * blk_row + (size_t)(dbase / 32) * 1024u + l * 16u);

  u32x4 tra[2];
  auto tr_load = [&](const DG_LDS u16* tile, int c, int slot) {
    const u32x2 a = lds_read_tr16(tile + tr_off0 + 512 * c);
    const u32x2 b = lds_read_tr16(tile + (tr_off0 ^ 32) + 512 * c);
    tra[slot] = u32x4{a[0], a[1], b[0], b[1]};
  };

  // softmax owner: row 16w + rho, ids 4q .. 4q+3 (lane 4 rho + q)
  const int rho = l >> 2, q = l & 3, orow = 16 * w + rho;
  float m_seg = -INFINITY, lsum = 0.f, m_true = -INFINITY;
  int amax = 0;
  bool g_valid = false;
  int broken = 0;  // an exchange wait timed out (uniform; an int, not a lane mask)
  u32x4 pf[2] = {z4, z4};
  const int xw = 16 * g + ((r + 4 * g) & 15);
  const int xr = 16 * q + ((rho + 4 * q) & 15);

  // G = (G + acc) s (G = acc s on the first fold; the first fold stores the
  // raw accumulator to G, a later one to the temp area T, merged after)
  auto fold = [&](f32x16 (&acc)[2][NCH], float s, bool scale) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int zr = r0 + 32 * hh + m32;
      if (zr < R) {
        float* gp = pS + ((size_t)split * R + zr) * d + dbase + 4 * h2;
        float* dst = g_valid ? gp + tofs : gp;
#pragma unroll
        for (int c = 0; c < NCH; ++c)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            *(f32x4*)(dst + 32 * c + 8 * j) =
                f32x4{acc[hh][c][4 * j], acc[hh][c][4 * j + 1], acc[hh][c][4 * j + 2], acc[hh][c][4 * j + 3]};
      }
    }
    if (g_valid || scale) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int zr = r0 + 32 * hh + m32;
        const float sr = scale ? Sbuf[32 * hh + m32] : 1.f;
        if (zr < R) {
          float* gp = pS + ((size_t)split * R + zr) * d + dbase + 4 * h2;
          for (int c = 0; c < NCH; ++c)
            for (int j = 0; j < 4; ++j) {
              float* p = gp + 32 * c + 8 * j;
              f32x4 v = *(const f32x4*)p;
              if (g_valid) v += *(const f32x4*)(p + tofs);
              *(f32x4*)p = v * sr;
            }
        }
      }
    }
    g_valid = true;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int c = 0; c < NCH; ++c) acc[hh][c] = zero16();
  };
  // after the last tile: the final fold and the row statistics (member 0)
  auto finish = [&](f32x16 (&acc)[2][NCH]) {
    fold(acc, 1.f, false);
    const float tot = lsum + dpp_f<0xB1>(lsum);
    const float tot4 = tot + dpp_f<0x4E>(tot);
    if (mb == 0 && r0 + orow < R && q == 0)
      pstat[(size_t)split * R + r0 + orow] = f32x4{m_seg, tot4, m_true, __int_as_float(amax)};
  };

  if (solo) {
    f32x16 acc[2][NCH];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int c = 0; c < NCH; ++c) acc[hh][c] = zero16();
    // ---- solo run: every member's partial computed here, then the same
    // softmax and P.E as the paired run, one tile at a time ----
    DG_LDS u16* tile = (DG_LDS u16*)&Et[0][w][0][0];
    for (int s = 0; s < nt; ++s) {
      const int ph = phys(s);
      const int v2 = vs + 16 * ph;
      f32x4 x4 = {0.f, 0.f, 0.f, 0.f};
      for (int m = 0; m < Q; ++m) {
        const int cb = m * dq + w * SLICE;  // member m's columns of this wave
        const uint32_t moff = (uint32_t)((size_t)(vs / 16) * blk_row + (size_t)(cb / 32) * 1024u + l * 16u) +
                              (uint32_t)ph * blk_row;
        f32x4 lg[4] = {};
#pragma unroll 1
        for (int c = 0; c < NCH; ++c) {
          const u32x4 e = buffer_ld128(erc, moff + 1024u * c);
          if (m == mb) *(DG_LDS u32x4*)(tile + wr + 512 * c) = e;
#pragma unroll
          for (int h = 0; h < 4; ++h) {
            const u32x4 zf = swap_halves(ldg128(Z + (size_t)min(r0 + 16 * h + r, R - 1) * d + cb + 32 * c + 8 * g),
                                         g & 1);
            lg[h] = mfma16x32(e, zf, c == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : lg[h]);
          }
        }
#pragma unroll
        for (int h = 0; h < 4; ++h) xch[w][h][xw] = lg[h];
        __syncthreads();
        f32x4 xa[4];
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) xa[s4] = xch[s4][w][xr];
        f32x4 own = xa[0] + xa[1];
        own = (own + xa[2]) + xa[3];
        own = pair_tagged(own, pair_gen(s));
        x4 = m == 0 ? own : x4 + own;
        __syncthreads();
      }
      float x[4] = {x4[0], x4[1], x4[2], x4[3]};
      if (!(v2 + 16 <= ve)) {
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = v2 + 4 * q + i < ve ? x[i] : -INFINITY;
      }
      float tm = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
      tm = fmaxf(tm, dpp_f<0xB1>(tm));
      tm = fmaxf(tm, dpp_f<0x4E>(tm));
      if (__any(tm >= m_true)) {
        int cand = 0x7FFFFFFF;
#pragma unroll
        for (int i = 3; i >= 0; --i) cand = x[i] == tm ? v2 + 4 * q + i : cand;
        cand = min(cand, dpp_i<0xB1>(cand));
        cand = min(cand, dpp_i<0x4E>(cand));
        const bool better = (tm > m_true) | ((tm == m_true) & (tm != -INFINITY) & (cand < amax));
        amax = better ? cand : amax;
        m_true = fmaxf(m_true, tm);
      }
      const bool first = m_seg == -INFINITY;
      const bool over = !first & (tm > m_seg + kLazyTh);
      const float sc = over ? __builtin_amdgcn_exp2f((m_seg - tm) * kLog2e) : 1.f;
      m_seg = (first | over) ? tm : m_seg;
      const float ms = m_seg == -INFINITY ? 0.f : m_seg;
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = __builtin_amdgcn_exp2f((x[i] - ms) * kLog2e);
      lsum = fmaf(lsum, sc, (x[0] + x[1]) + (x[2] + x[3]));
      {
        typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
        typedef float f32x2v __attribute__((ext_vector_type(2)));
        const uint32_t lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2v{x[0], x[1]}, bf16x2v));
        const uint32_t hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2v{x[2], x[3]}, bf16x2v));
        *(DG_LDS u32x2*)((DG_LDS char*)&Pbuf[q >> 1][orow] + 8 * (q & 1)) = u32x2{lo, hi};
      }
      Sbuf[threadIdx.x >> 2] = sc;
      flags[w] = __any(sc != 1.f) ? 1 : 0;
      __syncthreads();
      pf[0] = Pbuf[h2][m32];
      pf[1] = Pbuf[h2][32 + m32];
      if ((flags[0] | flags[1] | flags[2] | flags[3]) != 0) fold(acc, 0.f, true);
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        tr_load(tile, c, 0);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) acc[hh][c] = mfma32(tra[0], pf[hh], acc[hh][c]);
        __builtin_amdgcn_sched_barrier(0);
      }
      __syncthreads();  // the tile, P and the flags are rewritten next tile
    }
    finish(acc);
    return;
  }
  {
    // ---- paired run ----
    f32x16 acc[2][NCH];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int c = 0; c < NCH; ++c) acc[hh][c] = zero16();
    // Z fragments of rows 16h + r, columns dbase + 32c + 8g .. +7
    u32x4 zf[4][NCH];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const u16* zp = Z + (size_t)min(r0 + 16 * h + r, R - 1) * d + dbase + 8 * g;
#pragma unroll
      for (int c = 0; c < NCH; ++c) zf[h][c] = swap_halves(ldg128(zp + 32 * c), g & 1);
    }
    // E chunks stream through a register ring of PF slots: chunk c of a tile
    // sits in slot c % PF and is loaded PF chunks ahead (a whole tile ahead
    // for pairs; half a tile for quads, whose three exchange records leave
    // no room for eight slots)
    constexpr int PF = Q == 2 ? NCH : NCH / 2;
    u32x4 ring[PF];
    auto issue = [&](int c, int step) {
      ring[c % PF] = buffer_ld128(erc, lane_off + (uint32_t)phys(step) * blk_row + 1024u * c);
    };
#pragma unroll
    for (int c = 0; c < PF; ++c) issue(c, 0);
    tr_load((const DG_LDS u16*)&Et[1][w][0][0], 0, 0);  // tile -3: zeros
    tr_load((const DG_LDS u16*)&Et[1][w][0][0], 1, 1);

    f32x4 lg[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) lg[h] = f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 own_old = {0.f, 0.f, 0.f, 0.f};
    u32x4 xp[Q - 1];
#pragma unroll
    for (int k = 0; k < Q - 1; ++k) xp[k] = z4;
    // exchange records: [group][member][slot][256 lanes][4 words]; uniform
    // bases plus a 32-bit lane offset
    const __amdgpu_buffer_rsrc_t xrc = buffer_rsrc(xrec, (uint32_t)(gridDim.x * kMemberRecBytes));
    const uint32_t xo_out = (uint32_t)(((size_t)grp * Q + mb) * kMemberRecBytes);
    // other member k (k < Q - 1) is member k + (k >= mb); its records are
    // addressed as the uniform base plus a 32-bit offset (the region is a
    // few MiB), so no 64-bit lane addresses stay live across the loop
    const char* const xbase = (const char*)xrec;
    auto xo_in = [&](int k) {
      return (uint32_t)(((size_t)grp * Q + k + (k >= mb ? 1 : 0)) * kMemberRecBytes);
    };
    const uint32_t xlane = threadIdx.x * 16u;

    // MARK marks the rare paths (a fold, an exchange poll, a ragged tile, a
    // new running maximum) unlikely, so that their code moves out of the loop's
    // straight line.  Only pair launches of four row blocks or more use it (2% faster
    // there).  With two row blocks the same layout made each exchange poll
    // costly: once the members fell into polling, the launch took 75% longer
    // (the default layout, in the same state, 10%).  Quads keep the default
    // layout too: marked, the d = 4096 launch slowed down by 20% and more.
    constexpr bool kMarkRare = MARK;
    // The same instances store chunk 0's partial logits one row group at a
    // time, each just before the product that overwrites it, instead of all
    // four (and the E chunk) ahead of the products: the products start while
    // the stores drain.  1% faster at 256 rows (0.596-0.603 against
    // 0.606-0.611 ms), 2% at V = 32768; the quads fell into polling with it.
    constexpr bool kC0Interleave = MARK;
    // A late partner record is waited for in a poll loop whose every reload
    // also waits for the E loads issued before it (vector loads complete in
    // order).  With one row block E comes straight from HBM and that wait is
    // most of a tile: the waiting member falls behind by more than the
    // exchange margin, its partner then finds a late record in turn, and the
    // pair keeps alternating (about 16% of waits poll, 385 us at 1-64 rows).
    // kDefer re-loads a late record in chunk 4 and waits for it only at the
    // start of chunk 7, where the loads issued before it are 3-4 chunks old,
    // and runs the skipped softmax steps there: 281-318 us, 5% of waits late.
    // Launches with several row blocks read E mostly from L2, where a wait
    // is short, and keep the plain loop.
    constexpr bool kDefer = PIN;
    bool defer = false;  // uniform: a late record's softmax steps wait for chunk 7
    // a wait that hit its bound: raise the error flag, record the first one
    auto exchange_timeout = [&](int k, int t) {
      broken = 1;
      if (l == 0) {
        __hip_atomic_store(&xhdr[8], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (__hip_atomic_fetch_add(&xhdr[10], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0) {
          xhdr[12] = (uint32_t)grp;
          xhdr[13] = (uint32_t)t;
          xhdr[14] = (uint32_t)(mb | (w << 4));
          xhdr[15] = xp[k][0] & 1u;
        }
      }
    };
    for (int t = 0; t <= nt + 2; ++t) {
      // Tile t-1's partial logits and tile t-3's softmax output (written in
      // the previous iteration) become visible.
      __syncthreads();
      pf[0] = Pbuf[h2][m32];
      pf[1] = Pbuf[h2][32 + m32];
      typedef int i32x4_t __attribute__((ext_vector_type(4)));
      i32x4_t flv = *(const DG_LDS i32x4_t*)flags;  // combined after chunk 0's logit products
      const bool own_ok = (uint32_t)(t - 1) < (uint32_t)nt;  // tile t-1 is exchanged
      const bool sm_ok = (uint32_t)(t - 2) < (uint32_t)nt;   // tile t-2 gets its softmax
      const int v2 = vs + 16 * (sm_ok ? phys(t - 2) : 0);
      DG_LDS u16* tile = (DG_LDS u16*)&Et[t & 3][w][0][0];
      const DG_LDS u16* tpe = (const DG_LDS u16*)&Et[(t + 1) & 3][w][0][0];   // tile t-3
      const DG_LDS u16* tnx = (const DG_LDS u16*)&Et[(t + 2) & 3][w][0][0];   // tile t-2
      f32x4 xa[4], own;
      float x[4];
      float tm = -INFINITY, s = 1.f, ms = 0.f;
      bool over = false, first = false;
      // The softmax of tile t-2 and the exchange of tile t-1, cut into small
      // steps: step (c, j) is placed after matrix-core instruction j of chunk
      // c (j = 0..3 logits, 4..5 self-conditioning), so the latency of its
      // dependent vector instructions overlaps the products in flight instead
      // of idling the matrix core.  PIN = false lets the compiler move the steps
      // between the products of a chunk (2-5% faster from 128 rows up); PIN =
      // true pins each step after its product (faster for a single 64-row
      // block, where streaming E dominates: 10-16% at 1 row).  The chunks
      // themselves stay in order either way.
      auto stage = [&](int c, int j) {
        const bool live = !(kDefer && defer);  // false: this tile's softmax steps run in chunk 7
        if (c == 2 && j == 0) {
#pragma unroll
          for (int s4 = 0; s4 < 4; ++s4) xa[s4] = xch[s4][w][xr];
        }
        if (c == 3 && j == 0) {
          own_old = ownb[threadIdx.x];  // this member's partial of tile t-2, parked last iteration
          own = xa[0] + xa[1];
        }
        if (c == 3 && j == 1) own = (own + xa[2]) + xa[3];
        if (c == 3 && j == 2) {
          own = pair_tagged(own, pair_gen(t - 1));
          ownb[threadIdx.x] = own;
        }
        if (c == 3 && j == 3 && own_ok)
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, own), xrc, xlane,
                                                 xo_out + ((t - 1) & 3) * 4096u, 0);
        if (c == 4 && j == 0 && sm_ok) {
          const uint32_t want = pair_gen(t - 2);
#pragma unroll
          for (int k = 0; k < Q - 1; ++k) {
            const bool late = !wave_all(pair_gen_ok(xp[k], want));
            if (kMarkRare ? __builtin_expect(late, 0) : late) {
              if (broken) continue;  // a partner already timed out: no more waiting
              if (l == 0) __hip_atomic_fetch_add(&xhdr[9], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              uint32_t xl = xlane;
              asm volatile("" : "+v"(xl));
              const uint32_t so = xo_in(k) + ((t - 2) & 3) * 4096u + xl;
              if constexpr (kDefer) {
                xp[k] = pair_load(xbase, so);  // waited for in chunk 7
                defer = true;
                continue;
              }
              for (uint32_t n = 0;; ++n) {
                xp[k] = pair_load(xbase, so);
                if (wave_all(pair_gen_ok(xp[k], want))) break;
                if (n >= kPairSpin) {
                  exchange_timeout(k, t);
                  break;
                }
              }
            }
          }
        }
        if (c == 4 && j == 1 && live) {
          // every member adds the Q partials in member order (for two members
          // own + other is that sum: the addition commutes exactly)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if constexpr (Q == 2) {
              x[i] = own_old[i] + __uint_as_float(xp[0][i]);
            } else {
              float a = mb == 0 ? own_old[i] : __uint_as_float(xp[0][i]);
#pragma unroll
              for (int m = 1; m < Q; ++m)
                a += m == mb ? own_old[i] : __uint_as_float(xp[m - (m > mb ? 1 : 0)][i]);
              x[i] = a;
            }
          }
        }
        if (c == 4 && j == 2 && live &&
            (kMarkRare ? __builtin_expect(!(sm_ok && v2 + 16 <= ve), 0) : !(sm_ok && v2 + 16 <= ve))) {
          // a ragged or absent tile (uniform): ids past the split are -inf
          const int lim = sm_ok ? ve - v2 : 0;
#pragma unroll
          for (int i = 0; i < 4; ++i) x[i] = 4 * q + i < lim ? x[i] : -INFINITY;
        }
        if (c == 4 && j == 3 && live) tm = max4_f(x[0], x[1], x[2], x[3]);
        if (c == 4 && j == 4 && live) tm = dpp_max_x1(tm);
        if (c == 4 && j == 5 && live) tm = dpp_max_x2(tm);  // the row's tile max, in all 4 lanes
        if (c == 5 && j == 0 && live && (kMarkRare ? __builtin_expect(__any(tm >= m_true), 0) : __any(tm >= m_true))) {
          // the running max may move (uniform branch, rare after a split's
          // first tiles): lowest id attaining the tile max; tiles come out of
          // id order, so a tie goes to the lower id.  The offset within the
          // tile is reduced, then the tile's first id added.
          int cand = 0x7FFFFFFF;
#pragma unroll
          for (int i = 3; i >= 0; --i) cand = x[i] == tm ? 4 * q + i : cand;
          cand = min(cand, dpp_i<0xB1>(cand));
          cand = min(cand, dpp_i<0x4E>(cand));
          cand += v2;
          const bool better = (tm > m_true) | ((tm == m_true) & (tm != -INFINITY) & (cand < amax));
          amax = better ? cand : amax;
          m_true = fmaxf(m_true, tm);
        }
        if (c == 5 && j == 1 && live) {
          // Lazy reference: it only moves when a logit exceeds it by more than
          // kLazyTh; the running sum is then rescaled by s = e^(m_old - m_new).
          first = m_seg == -INFINITY;
          over = !first & (tm > m_seg + kLazyTh);
          s = over ? __builtin_amdgcn_exp2f((m_seg - tm) * kLog2e) : 1.f;
        }
        if (c == 5 && j == 2 && live) {
          m_seg = (first | over) ? tm : m_seg;
          ms = m_seg == -INFINITY ? 0.f : m_seg;  // a row with no valid logit yet: all p are 0
        }
        // p = 2^((x - m) log2 e): exact 1 at the maximum, 0 for a masked -inf;
        // results below 2^-126 flush to 0 (more than 87 below the reference)
        if (c == 5 && j == 3 && live) {
          x[0] = __builtin_amdgcn_exp2f((x[0] - ms) * kLog2e);
          x[1] = __builtin_amdgcn_exp2f((x[1] - ms) * kLog2e);
        }
        if (c == 5 && j == 4 && live) {
          x[2] = __builtin_amdgcn_exp2f((x[2] - ms) * kLog2e);
          x[3] = __builtin_amdgcn_exp2f((x[3] - ms) * kLog2e);
        }
        if (c == 5 && j == 5 && live) lsum = fmaf(lsum, s, (x[0] + x[1]) + (x[2] + x[3]));
        if (c == 6 && j == 0 && live) {
          typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
          typedef float f32x2v __attribute__((ext_vector_type(2)));
          const uint32_t lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2v{x[0], x[1]}, bf16x2v));
          const uint32_t hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2v{x[2], x[3]}, bf16x2v));
          *(DG_LDS u32x2*)((DG_LDS char*)&Pbuf[q >> 1][orow] + 8 * (q & 1)) = u32x2{lo, hi};
        }
        if (c == 6 && j == 1 && live) {
          // every lane of a row writes the same factor, every lane of the wave
          // the same flag (no branch; orow = threadIdx.x / 4)
          Sbuf[threadIdx.x >> 2] = s;
          flags[w] = __any(s != 1.f) ? 1 : 0;
        }
      };
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const u32x4 e = ring[c % PF];
        if (c == 0 && !kC0Interleave) {
          // tile t-1's partial logits of this wave (finished last iteration)
#pragma unroll
          for (int h = 0; h < 4; ++h) xch[w][h][xw] = lg[h];
        }
        if (!(kC0Interleave && c == 0)) *(DG_LDS u32x4*)(tile + wr + 512 * c) = e;
        if (kDefer && c == 7 && defer) {
          // the late record of tile t-2, re-loaded in chunk 4: wait for it
          // here, then run the softmax steps skipped in chunks 4-6
          const uint32_t want = pair_gen(t - 2);
          uint32_t xl = xlane;
          asm volatile("" : "+v"(xl));
#pragma unroll
          for (int k = 0; k < Q - 1; ++k) {
            const uint32_t so = xo_in(k) + ((t - 2) & 3) * 4096u + xl;
            for (uint32_t n = 0; !broken && !wave_all(pair_gen_ok(xp[k], want)); ++n) {
              if (n >= kPairSpin) {
                exchange_timeout(k, t);
                break;
              }
              xp[k] = pair_load(xbase, so);
            }
          }
          defer = false;
#pragma unroll
          for (int jj = 1; jj < 6; ++jj) stage(4, jj);
#pragma unroll
          for (int jj = 0; jj < 6; ++jj) stage(5, jj);
          stage(6, 0);
          stage(6, 1);
        }
        if (c == 7 && own_ok) {
          // the other members' partials of tile t-1 (stored at chunk 3 of
          // this iteration), consumed at chunk 4 of the next; the lane offset
          // is made opaque here, so the per-member offsets are added at each
          // load instead of being kept live across the loop
          uint32_t xl = xlane;
          asm volatile("" : "+v"(xl));
#pragma unroll
          for (int k = 0; k < Q - 1; ++k) xp[k] = pair_load(xbase, xo_in(k) + ((t - 1) & 3) * 4096u + xl);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          // e comes from memory, zf is constant: no VALU write precedes
          if (c == 0) {
            if constexpr (kC0Interleave) xch[w][h][xw] = lg[h];  // tile t-1's, row group h
            mfma16x32_v0(e, zf[h][c], lg[h]);  // a new tile's chain starts from 0
            if constexpr (kC0Interleave) {
              if (h == 3) *(DG_LDS u32x4*)(tile + wr) = e;
              __builtin_amdgcn_sched_barrier(0);
            }
          } else {
            mfma16x32_vn(e, zf[h][c], lg[h]);
          }
          stage(c, h);
          if constexpr (PIN) __builtin_amdgcn_sched_barrier(0);
        }
        if (c == 0) {
          // the flags' LDS latency hides behind the products above: their
          // first use is pinned after them
          asm volatile("" : "+v"(flv));
          const bool fl = t >= 3 && __builtin_amdgcn_readfirstlane(flv[0] | flv[1] | flv[2] | flv[3]) != 0;
          if (kMarkRare ? __builtin_expect(fl, 0) : fl) {
            // tile t-3's softmax moved a reference: fold the products of the
            // tiles before it under the old one
            fold(acc, 0.f, true);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          acc[hh][c] = mfma32(tra[c & 1], pf[hh], acc[hh][c]);
          stage(c, 4 + hh);
          if constexpr (PIN) __builtin_amdgcn_sched_barrier(0);
        }
        if (c == NCH - 1) mfma_v_settle(lg);
        if (c == 1) __syncthreads();  // tile t-1's partials are in LDS; tile t-3's P is read
        // A operand of chunk c+2 of tile t-3 (slot c & 1 was just consumed), or
        // of chunks 0, 1 of tile t-2 for the next iteration
        if (c + 2 < NCH)
          tr_load(tpe, c + 2, c & 1);
        else
          tr_load(tnx, c + 2 - NCH, c & 1);
        // the chunk PF ahead (of this tile or of tile t+1) into the slot this
        // chunk's products just read
        if (c + PF < NCH)
          issue(c + PF, t);
        else
          issue(c + PF - NCH, t + 1);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    finish(acc);
  }
}

// Zeroes the pair tickets, error flag and exchange tags (a kernel, so that
// the launch sequence can be captured in a graph).
__global__ void __launch_bounds__(256) k_vocab_pair_clear(u32x4* __restrict__ p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256)
    p[i] = u32x4{0u, 0u, 0u, 0u};
}

// ---------------------------------------------------------------------------
// Combine of the vocab splits, one workgroup per row, splits in increasing
// vocab order:  max = max_s max_s,  argmax = that of the first split
// attaining it (lowest id),  mu = max_s m_ref_s,  Lt = sum_s e^(m_ref_s - mu) sum_s,
// lse = mu + ln Lt,  conf = e^(max - mu) / Lt,  S = sum_s e^(m_ref_s - mu) S_s / Lt.
// err (may be NULL): the paired kernel's error flag; when set, the outputs are
// NaN (argmax -1) instead of a silently wrong result.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) k_vocab_combine(int R, int d, int nsplit, const float* __restrict__ pS,
                                                       const f32x4* __restrict__ pstat,
                                                       float* __restrict__ max_logit,
                                                       int32_t* __restrict__ argmax,
                                                       float* __restrict__ conf, float* __restrict__ lse,
                                                       void* __restrict__ S, int out_bf16,
                                                       const uint32_t* __restrict__ err, RenoiseArgs rn) {
  __shared__ float wgt[1024];
  __shared__ float sh[4];
  const int r = blockIdx.x;
  if (err && *err) {
    // a resident group member stopped answering (its exchange timed out):
    // the statistics and S of every row are NaN (argmax -1), and the row's
    // token is drawn as for a renoised position, so the token stream stays
    // within [0, V)
    if (threadIdx.x == 0) {
      max_logit[r] = NAN;
      argmax[r] = -1;
      conf[r] = NAN;
      if (lse) lse[r] = NAN;
      if (rn.out) renoise_row(rn, r, 0, -INFINITY);
    }
    for (int e = threadIdx.x; e < d; e += 256) {
      if (out_bf16) ((u16*)S)[(size_t)r * d + e] = 0x7FC0;
      else ((float*)S)[(size_t)r * d + e] = NAN;
    }
    return;
  }
  if (threadIdx.x < 64) {
    // one wave: lane l takes splits l, l+64, ... (independent loads), then
    // fixed-pattern reductions across the wave
    const int l = threadIdx.x;
    float M = -INFINITY, mu = -INFINITY;
    int A = 0, Sfirst = 0x7FFFFFFF;
    for (int s = l; s < nsplit; s += 64) {
      const f32x4 st = pstat[(size_t)s * R + r];
      if (st[2] > M) { M = st[2]; A = __float_as_int(st[3]); Sfirst = s; }
      mu = fmaxf(mu, st[0]);
    }
    // max logit; argmax of the first (lowest-id) split attaining it
    for (int o = 32; o > 0; o >>= 1) {
      const float oM = __shfl_xor(M, o);
      const int oA = __shfl_xor(A, o), oS = __shfl_xor(Sfirst, o);
      const bool take = (oM > M) | ((oM == M) & (oS < Sfirst));
      M = take ? oM : M;
      A = take ? oA : A;
      Sfirst = take ? oS : Sfirst;
      mu = fmaxf(mu, __shfl_xor(mu, o));
    }
    float part = 0.f;
    for (int s = l; s < nsplit; s += 64) {
      const f32x4 st = pstat[(size_t)s * R + r];
      const float ws = st[0] == -INFINITY ? 0.f : expf(st[0] - mu);
      wgt[s] = ws;
      part += ws * st[1];
    }
    for (int o = 32; o > 0; o >>= 1) part += __shfl_xor(part, o);
    const float Lt = part;
    if (l == 0) {
      sh[0] = 1.f / Lt;
      max_logit[r] = M;
      argmax[r] = A;
      const float cf = expf(M - mu) / Lt;
      conf[r] = cf;
      if (lse) lse[r] = mu + logf(Lt);
      if (rn.out) renoise_row(rn, r, A, cf);   // the stored confidence decides
    }
  }
  __syncthreads();
  const float invL = sh[0];
  for (int e = threadIdx.x * 4; e < d; e += 256 * 4) {
    f32x4 a = {0.f, 0.f, 0.f, 0.f};
    // splits in a fixed order; 8 independent loads in flight per thread
    const float* sp = pS + (size_t)r * d + e;
    const size_t st = (size_t)R * d;
    int s = 0;
    for (; s + 8 <= nsplit; s += 8) {
      f32x4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = *(const f32x4*)(sp + (size_t)(s + u) * st);
#pragma unroll
      for (int u = 0; u < 8; ++u) a += wgt[s + u] * v[u];
    }
    for (; s < nsplit; ++s) a += wgt[s] * *(const f32x4*)(sp + (size_t)s * st);
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
// Tiled table: thread q writes 16 bytes of block q / 64 at lane position
// q % 64 = 16 g + r: id 16 vb + r, columns 32 c + 8 g .. +7 (for odd g the
// two 8-byte halves swapped), where the block is (vb, c) =
// (q / 64 / (d/32), q / 64 % (d/32)); ids past V are zero.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) k_pack_embedding(int V, int d, size_t n16, const u16* __restrict__ E,
                                                        u32x4* __restrict__ out) {
  const size_t q = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (q >= n16) return;
  const size_t b = q >> 6;
  const int lane = (int)(q & 63), g = lane >> 4, r = lane & 15;
  const size_t cpb = (size_t)d / 32;
  const size_t vb = b / cpb, c = b % cpb;
  const size_t id = vb * 16 + r;
  out[q] = id < (size_t)V ? swap_halves(ldg128(E + id * d + c * 32 + g * 8), g & 1) : u32x4{0u, 0u, 0u, 0u};
}

hipError_t launch_pack_embedding(int V, int d, const void* E, void* E_tiled, hipStream_t s) {
  const size_t n16 = ((size_t)V + 15) / 16 * 16 * (size_t)d / 8;
  const size_t nb = (n16 + 255) / 256;
  hipLaunchKernelGGL(k_pack_embedding, dim3((unsigned)nb), dim3(256), 0, s, V, d, n16, (const u16*)E,
                     (u32x4*)E_tiled);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// CU groups need all 8 XCDs of a full MI355X (256 CUs, one workgroup each).
static bool group_capable() {
  static std::atomic<int> cached[64];  // 0 unknown, 1 no, 2 yes
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return false;
  int c = cached[dev].load(std::memory_order_relaxed);
  if (c == 0) {
    int n = 0;
    c = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n == 256 ? 2 : 1;
    cached[dev].store(c, std::memory_order_relaxed);
  }
  return c == 2;
}

// Poll bound of the group handshake (a test hook can set it to 0, which
// makes every group run solo).
static std::atomic<uint32_t> g_group_spin{kGroupSpin};
void set_group_wait(int32_t polls) { g_group_spin.store(polls < 0 ? kGroupSpin : (uint32_t)polls); }

VocabPlan vocab_plan(int rows, int d, int V, int dtype) {
  VocabPlan p{};
  p.rows = rows; p.d = d; p.V = V;
  if (dtype != 1) {
    p.variant = 0; p.nrb = rows; p.nsplit = 1; p.split_len = V;
    return p;
  }
  const int vt = 16, tiles = (V + vt - 1) / vt;
  const int Q = d / 1024;
  if ((d == 2048 || d == 4096) && group_capable()) {
    // CU groups of Q = d / 1024 workgroups, 64 rows: Q nrb nsplit = 256
    // workgroups at most, with nrb nsplit a multiple of 8 so that every XCD
    // holds whole groups
    const int nrb = (rows + 63) / 64;
    int ns = 256 / Q / nrb;
    while (ns > 0 && (nrb * ns) % 8 != 0) --ns;
    if (ns > tiles) {
      ns = tiles;
      while (ns > 0 && (nrb * ns) % 8 != 0) --ns;
    }
    if (ns > 0) {
      p.variant = 3;
      p.group = Q;
      p.nrb = nrb;
      p.split_len = (tiles + ns - 1) / ns * vt;
      p.nsplit = ns;  // trailing splits may be empty: they contribute nothing
      p.part_S_bytes = 2 * (size_t)p.nsplit * rows * d * sizeof(float);
      p.part_stat_bytes = (size_t)p.nsplit * rows * sizeof(f32x4);
      p.part_X_bytes = 256 + kPairHdrWords * 4 + (size_t)nrb * ns * Q * kMemberRecBytes;
      return p;
    }
  }
  int rw;
  if (d <= 2048) { p.variant = 1; rw = 32; }
  else { p.variant = 2; rw = 16; }
  p.nrb = (rows + rw - 1) / rw;
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

size_t vocab_exchange_region(const VocabPlan& p, void* ws, void** region) {
  *region = nullptr;
  if (p.rows <= 0 || p.variant != 3) return 0;
  *region = (void*)(((uintptr_t)ws + p.part_S_bytes + p.part_stat_bytes + 255) & ~(uintptr_t)255);
  return kPairHdrWords * 4 + (size_t)p.nrb * p.nsplit * p.group * kMemberRecBytes;
}

hipError_t launch_vocab(const VocabPlan& p, const void* z, const void* E, float* max_logit,
                        int32_t* argmax, float* conf, float* lse, void* selfcond, void* ws,
                        hipStream_t s, hipEvent_t ev_begin, hipEvent_t ev_end, const RenoiseArgs* rn,
                        bool exchange_cleared) {
  if (p.rows <= 0) return hipSuccess;
  if (p.variant == 0) {
    hipLaunchKernelGGL(k_vocab_f32, dim3(p.rows), dim3(256), 0, s, p.rows, p.d, p.V,
                       (const float*)z, (const float*)E, max_logit, argmax, conf, lse,
                       (float*)selfcond);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess && rn && rn->out)
      e = launch_renoise(p.rows, rn->canvas, rn->V, argmax, conf, rn->tau, rn->seed, rn->t, rn->block, rn->out,
                         rn->mask, s);
    return e;
  }
  const RenoiseArgs no_rn{nullptr, nullptr, 0.f, 0, 0, 0, 1, 1};
  float* pS = (float*)ws;
  f32x4* pstat = (f32x4*)((char*)ws + p.part_S_bytes);
  const dim3 grid((unsigned)(p.nrb * p.nsplit));
  const u16* Zb = (const u16*)z;
  const u16* Eb = (const u16*)E;
  const int sl = p.d / 4;
  bool launched = true;
  uint32_t* xhdr = nullptr;
  if (p.variant == 3) {
    void* region = nullptr;
    const size_t xbytes = vocab_exchange_region(p, ws, &region);
    xhdr = (uint32_t*)region;
    if (!exchange_cleared) {
      hipLaunchKernelGGL(k_vocab_pair_clear, dim3(512), dim3(256), 0, s, (u32x4*)xhdr, xbytes / 16);
      if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    }
  }
  if (ev_begin) {
    hipError_t e = hipEventRecord(ev_begin, s);
    if (e != hipSuccess) return e;
  }
  if (p.variant == 3) {
    const dim3 pgrid((unsigned)(p.group * p.nrb * p.nsplit));
    uint64_t* xrec = (uint64_t*)(xhdr + kPairHdrWords);
    const uint32_t spin = g_group_spin.load();
    if (p.group == 4)
      hipLaunchKernelGGL((k_vocab_group<4, false, false>), pgrid, dim3(256), 0, s, Zb, Eb, p.rows, p.d, p.V,
                         p.nrb, p.split_len, pS, pstat, xhdr, xrec, spin);
    else if (p.nrb == 1)  // at most 64 rows
      hipLaunchKernelGGL((k_vocab_group<2, true, false>), pgrid, dim3(256), 0, s, Zb, Eb, p.rows, p.d, p.V,
                         p.nrb, p.split_len, pS, pstat, xhdr, xrec, spin);
    else if (p.nrb < 4)  // 65 to 192 rows
      hipLaunchKernelGGL((k_vocab_group<2, false, false>), pgrid, dim3(256), 0, s, Zb, Eb, p.rows, p.d, p.V,
                         p.nrb, p.split_len, pS, pstat, xhdr, xrec, spin);
    else
      hipLaunchKernelGGL((k_vocab_group<2, false, true>), pgrid, dim3(256), 0, s, Zb, Eb, p.rows, p.d, p.V,
                         p.nrb, p.split_len, pS, pstat, xhdr, xrec, spin);
  } else if (p.variant == 1) {
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
      case 1024: launch_vocab16_1024(grid, s, Zb, Eb, p.rows, p.d, p.V, p.nrb, p.split_len, pS, pstat); break;
      default: launched = false;
    }
  }
  if (!launched) return hipErrorInvalidValue;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (ev_end && (e = hipEventRecord(ev_end, s)) != hipSuccess) return e;
  hipLaunchKernelGGL(k_vocab_combine, dim3(p.rows), dim3(256), 0, s, p.rows, p.d, p.nsplit, pS,
                     pstat, max_logit, argmax, conf, lse, selfcond, 1, xhdr ? xhdr + 8 : nullptr,
                     rn ? *rn : no_rn);
  return hipGetLastError();
}

}  // namespace dg
