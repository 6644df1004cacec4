// Flash-vocab, 16-row variant for d = 4096 (DiffusionGemma explainer,
// "Autocondizionamento": the probability matrix times the token-embedding
// table).  Its own translation unit, so that the build can give it its own
// scheduler flags.
#include "vocab_common.h"

namespace dg {

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
    for (int ks = 0; ks < NCH; ++ks) zf[ks] = swap_halves(ldg128(zp + ks * 32), g4 & 1);
  }
  float* gp = pS + ((size_t)split * R + (zok ? zr : 0)) * d + dbase + 4 * g4;
  const size_t tofs = (size_t)gridDim.x / nrb * R * d;
  DG_LDS u16* et = (DG_LDS u16*)&Et[w][0][0];
  const int nt = ve > vs ? (ve - vs + 15) / 16 : 0;
  for (int e = l * 8; e < 16 * EP; e += 64 * 8) *(DG_LDS u32x4*)(et + e) = z4;
  const int tr_r = 4 * g4 + (l16 >> 2);
  const DG_LDS u16* trb = et + prow16(tr_r) * EP + (l & 3) * 4;
  DG_LDS u16* wrb = et + prow16(l16) * EP + g4 * 8;

  // E is the tiled table (one 1 KiB block of 16 ids x 32 columns per load
  // instruction, in operand lane order); ids past the table read zeros
  const uint32_t blk_row = (uint32_t)d * 32u;
  const __amdgpu_buffer_rsrc_t erc = buffer_rsrc(E, (uint32_t)(((size_t)V + 15) / 16 * blk_row));
  const uint32_t lane_off = (uint32_t)((size_t)(vs / 16) * blk_row + (size_t)(dbase / 32) * 1024u + l * 16u);
  u32x4 ring0[PF];
  auto issue = [&](int slot, int tile, int c) {
    ring0[slot] = buffer_ld128(erc, lane_off + (uint32_t)tile * blk_row + 1024u * c);
  };
#pragma unroll
  for (int c = 0; c < PF; ++c) issue(c, 0, c);

  float m_seg = -INFINITY, lsum = 0.f, m_G = -INFINITY, l_G = 0.f;
  bool g_valid = false;
  float m_true = -INFINITY, tmax = -INFINITY;
  int amax = 0;
  u32x2 pf = {0u, 0u};
  float L[4];  // logits of ids v0 + 4*g4 + i of the current tile

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
        *(DG_LDS u32x2*)(wrb + c * 32 + ((g4 & 1) ? 4 : 0)) = u32x2{e0[0], e0[1]};
        *(DG_LDS u32x2*)(wrb + c * 32 + ((g4 & 1) ? 0 : 4)) = u32x2{e0[2], e0[3]};
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
    make_p(L);  // this tile's P against the new reference (L still holds it)
    ++t;
  }

  l_G += __shfl_xor(l_G, 16);
  l_G += __shfl_xor(l_G, 32);
  if (zok && w == 0 && g4 == 0) pstat[(size_t)split * R + zr] = f32x4{m_G, l_G, m_true, __int_as_float(amax)};
}

hipError_t launch_vocab16_1024(dim3 grid, hipStream_t s, const u16* Z, const u16* E, int R, int d, int V,
                               int nrb, int split_len, float* pS, f32x4* pstat) {
  hipLaunchKernelGGL(k_vocab16<1024>, grid, dim3(256), 0, s, Z, E, R, d, V, nrb, split_len, pS, pstat);
  return hipGetLastError();
}

}  // namespace dg
