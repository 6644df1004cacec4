// C ABI of libdg: argument checks (before anything is enqueued), workspace
// layout and the launch sequence of the canvas denoise step.
#include "../../include/dg.h"
#include "dg_common.h"

#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <new>

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return status;
}

int hip_fail(hipError_t e, const char* where) {
  return fail(DG_EHIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

size_t esize(int dtype) { return dtype == DG_BF16 ? 2 : 4; }

size_t round_up(size_t x) { return (x + 255) & ~(size_t)255; }

// Limits of what is implemented.
constexpr int kMaxSplits = 1024;

int check_dims(const dg_dims* d, bool need_vocab) {
  if (!d) return fail(DG_EINVAL, "dims is NULL");
  if (d->dtype != DG_F32 && d->dtype != DG_BF16) return fail(DG_EINVAL, "dtype %d is not DG_F32 or DG_BF16", d->dtype);
  if (d->B <= 0 || d->C <= 0 || d->d <= 0 || d->n_q_heads <= 0 || d->n_kv_heads <= 0 ||
      d->head_dim <= 0 || (need_vocab && d->V <= 0))
    return fail(DG_EINVAL, "sizes must be positive (B=%d C=%d d=%d Hq=%d Hkv=%d dh=%d V=%d)", d->B, d->C,
                d->d, d->n_q_heads, d->n_kv_heads, d->head_dim, d->V);
  if (d->L < 0 || d->cap < d->L) return fail(DG_EINVAL, "need 0 <= L <= cap (L=%d cap=%d)", d->L, d->cap);
  if (d->n_q_heads % d->n_kv_heads) return fail(DG_EINVAL, "n_q_heads %% n_kv_heads != 0 (%d, %d)", d->n_q_heads, d->n_kv_heads);
  if ((long long)d->B * d->C > (1 << 24) || (long long)d->L + d->C > (1 << 28))
    return fail(DG_EUNSUPPORTED, "B*C or L+C too large");
  if (d->dtype == DG_BF16) {
    if (d->head_dim != 64 && d->head_dim != 128) return fail(DG_EUNSUPPORTED, "bf16 head_dim must be 64 or 128 (got %d)", d->head_dim);
    if (d->n_kv_heads * d->head_dim % 64) return fail(DG_EUNSUPPORTED, "bf16 needs n_kv_heads*head_dim %% 64 == 0");
    if ((size_t)d->cap * d->head_dim * 2 > 0x7FFFFFFFu)
      return fail(DG_EUNSUPPORTED, "bf16 cache slab of one (canvas, KV head) must be under 2 GiB (cap=%d)", d->cap);
  } else {
    if (d->head_dim > 256) return fail(DG_EUNSUPPORTED, "fp32 head_dim must be <= 256 (got %d)", d->head_dim);
  }
  return DG_OK;
}

int check_vocab_shape(int rows, int d, int V, int dtype) {
  if (rows <= 0 || d <= 0 || V <= 0) return fail(DG_EINVAL, "rows, d, V must be positive (%d, %d, %d)", rows, d, V);
  if (dtype != DG_F32 && dtype != DG_BF16) return fail(DG_EINVAL, "dtype %d is not DG_F32 or DG_BF16", dtype);
  if (dtype == DG_BF16) {
    if (!(d == 128 || d == 256 || d == 512 || d == 1024 || d == 2048 || d == 4096))
      return fail(DG_EUNSUPPORTED, "bf16 vocab head needs d in {128,256,512,1024,2048,4096} (got %d)", d);
    if (((size_t)V + 15) / 16 * 16 * (size_t)d * 2 > 0xFFFF0000u)
      return fail(DG_EUNSUPPORTED, "bf16 vocab head needs a table under 4 GiB (V=%d d=%d)", V, d);
    dg::VocabPlan p = dg::vocab_plan(rows, d, V, dtype);
    if (p.nsplit > kMaxSplits) return fail(DG_EUNSUPPORTED, "too many vocab splits");
  } else {
    if (d > 4096) return fail(DG_EUNSUPPORTED, "fp32 vocab head needs d <= 4096 (got %d)", d);
  }
  return DG_OK;
}

size_t vocab_ws(int rows, int d, int V, int dtype) {
  dg::VocabPlan p = dg::vocab_plan(rows, d, V, dtype);
  return round_up(p.part_S_bytes) + round_up(p.part_stat_bytes) + round_up(p.part_X_bytes);
}

size_t attn_ws(const dg_dims* d, int causal) {
  dg::AttnPlan p = dg::attn_plan(d->B, d->C, d->L, d->cap, d->n_q_heads, d->n_kv_heads, d->head_dim,
                                 d->dtype, causal);
  return round_up(p.part_bytes);
}

// Step workspace: X | Q | Kn | Vn | O | Z | scratch (max of attention and vocab partials).
struct StepLayout {
  size_t X, Q, Kn, Vn, O, Z, scratch, total;
};
StepLayout step_layout(const dg_dims* d) {
  const size_t R = (size_t)d->B * d->C, es = esize(d->dtype);
  StepLayout s{};
  size_t off = 0;
  s.X = off; off += round_up(R * d->d * es);
  s.Q = off; off += round_up(R * d->n_q_heads * d->head_dim * es);
  s.Kn = off; off += round_up(R * d->n_kv_heads * d->head_dim * es);
  s.Vn = off; off += round_up(R * d->n_kv_heads * d->head_dim * es);
  s.O = off; off += round_up(R * d->n_q_heads * d->head_dim * es);
  s.Z = off; off += round_up(R * d->d * es);
  s.scratch = off;
  size_t sc = attn_ws(d, 0);
  const size_t sc1 = attn_ws(d, 1);
  if (sc1 > sc) sc = sc1;
  if (d->V > 0) {
    const size_t sv = vocab_ws((int)R, d->d, d->V, d->dtype);
    if (sv > sc) sc = sv;
  }
  s.total = off + sc;
  return s;
}

int check_bf16_align(const dg_dims* d, const void* const* ptrs, int n) {
  if (d->dtype != DG_BF16) return DG_OK;
  for (int i = 0; i < n; ++i)
    if (ptrs[i] && !aligned16(ptrs[i])) return fail(DG_EINVAL, "bf16 tensor pointer #%d is not 16-byte aligned", i);
  return DG_OK;
}

char* at(void* ws, size_t off) { return (char*)ws + off; }

int check_step(const dg_dims* dims, const dg_weights* w, const dg_step_io* io, const void* ws,
               size_t ws_bytes) {
  int st = check_dims(dims, true);
  if (st != DG_OK) return st;
  if (!w || !io) return fail(DG_EINVAL, "weights and io must be non-NULL");
  if (!w->Wq || !w->Wk || !w->Wv || !w->Wo || !w->E)
    return fail(DG_EINVAL, "every weight pointer must be non-NULL");
  if (!io->H || !io->tokens_in || !io->tokens_out || !io->selfcond_out || !io->max_logit ||
      !io->conf || !io->argmax || (dims->L > 0 && (!io->k_cache || !io->v_cache)))
    return fail(DG_EINVAL, "H, tokens_in/out, selfcond_out, max_logit, conf, argmax (and the caches when L > 0) must be non-NULL");
  const int R = dims->B * dims->C;
  if ((st = check_vocab_shape(R, dims->d, dims->V, dims->dtype)) != DG_OK) return st;
  if (dims->dtype == DG_BF16 && (dims->d % 128 || dims->n_q_heads * dims->head_dim % 64))
    return fail(DG_EUNSUPPORTED, "bf16 step needs d %% 128 == 0 and n_q_heads*head_dim %% 64 == 0");
  const void* ptrs[] = {w->Wq, w->Wk, w->Wv, w->Wo, w->E, io->H, io->k_cache, io->v_cache,
                        io->selfcond_in, io->selfcond_out, io->x_out, io->q_out, io->k_new_out,
                        io->v_new_out, io->attn_out, io->z_out};
  if ((st = check_bf16_align(dims, ptrs, 16)) != DG_OK) return st;
  const StepLayout L = step_layout(dims);
  if (!ws || ws_bytes < L.total)
    return fail(DG_EWORKSPACE, "step workspace needs %zu bytes (got %zu)", L.total, ws ? ws_bytes : 0);
  if (!aligned16(ws)) return fail(DG_EINVAL, "workspace must be 16-byte aligned");
  return DG_OK;
}

// The model pass of a step, then the sampler: uniform-state renoise
// (mask_id < 0) or the masked sampler's unmask-and-lock (mask_id >= 0).
int enqueue_step(const dg_dims* dims, const dg_weights* w, const dg_step_io* io, float tau,
                 uint64_t seed, uint32_t t, uint32_t block, void* ws, hipStream_t s,
                 int32_t mask_id = -1) {
  const StepLayout L = step_layout(dims);
  const int R = dims->B * dims->C;
  const int dt = dims->dtype, d = dims->d, Hq = dims->n_q_heads, Hkv = dims->n_kv_heads, dh = dims->head_dim;
  void* X = io->x_out ? io->x_out : at(ws, L.X);
  void* Q = io->q_out ? io->q_out : at(ws, L.Q);
  void* Kn = io->k_new_out ? io->k_new_out : at(ws, L.Kn);
  void* Vn = io->v_new_out ? io->v_new_out : at(ws, L.Vn);
  void* O = io->attn_out ? io->attn_out : at(ws, L.O);
  void* Z = io->z_out ? io->z_out : at(ws, L.Z);
  void* scratch = at(ws, L.scratch);
  hipError_t e;
  if ((e = dg::launch_assemble(dt, R, d, dims->V, io->H, w->E, io->tokens_in, io->selfcond_in, X, s)) != hipSuccess)
    return hip_fail(e, "assemble");
  if ((e = dg::launch_gemm_qkv(dt, R, d, X, w->Wq, Hq * dh, Q, w->Wk, w->Wv, Hkv * dh, Kn, Vn, s)) != hipSuccess)
    return hip_fail(e, "Q/K/V projections");
  dg::AttnPlan ap = dg::attn_plan(dims->B, dims->C, dims->L, dims->cap, Hq, Hkv, dh, dt, 0);
  if ((e = dg::launch_attn(ap, Q, io->k_cache, io->v_cache, Kn, Vn, O, nullptr, scratch, s,
                           (hipEvent_t)io->ev_attn_begin, (hipEvent_t)io->ev_attn_end)) != hipSuccess)
    return hip_fail(e, "attention");
  dg::VocabPlan vp = dg::vocab_plan(R, d, dims->V, dt);
  // the output projection also zeroes what the vocabulary head's CU-pair
  // kernel needs cleared (the attention's partials there are consumed by now)
  void* xregion = nullptr;
  const size_t xbytes = dt == DG_BF16 ? dg::vocab_exchange_region(vp, scratch, &xregion) : 0;
  if ((e = dg::launch_gemm_nt(dt, R, d, Hq * dh, O, w->Wo, X, Z, s, xregion, xbytes)) != hipSuccess)
    return hip_fail(e, "output projection");
  // the uniform-state renoise rides on the vocabulary head's split combine
  const dg::RenoiseArgs rn{io->tokens_out, io->mask, tau, seed, t, block, dims->C, dims->V};
  if ((e = dg::launch_vocab(vp, Z, w->E, io->max_logit, io->argmax, io->conf, io->lse, io->selfcond_out,
                            scratch, s, (hipEvent_t)io->ev_vocab_begin, (hipEvent_t)io->ev_vocab_end,
                            mask_id >= 0 ? nullptr : &rn, xbytes > 0)) != hipSuccess)
    return hip_fail(e, "vocab/self-conditioning/renoise");
  if (mask_id >= 0) {
    if ((e = dg::launch_unmask(R, io->argmax, io->conf, tau, mask_id, io->tokens_in, io->tokens_out, io->mask,
                               s)) != hipSuccess)
      return hip_fail(e, "unmask");
  }
  return DG_OK;
}

int check_append(const dg_dims* dims, const dg_weights* w, const void* H, const int32_t* tokens_final,
                 const void* k_cache, const void* v_cache, const void* attn_out, const void* ws,
                 size_t ws_bytes) {
  int st = check_dims(dims, true);
  if (st != DG_OK) return st;
  if (!w || !w->Wq || !w->Wk || !w->Wv || !w->E || !H || !tokens_final || !k_cache || !v_cache)
    return fail(DG_EINVAL, "weights (Wq, Wk, Wv, E), H, tokens_final and the caches must be non-NULL");
  if (dims->L + dims->C > dims->cap)
    return fail(DG_EINVAL, "append needs L + C <= cap (L=%d C=%d cap=%d)", dims->L, dims->C, dims->cap);
  if (dims->dtype == DG_BF16 && dims->d % 64)
    return fail(DG_EUNSUPPORTED, "bf16 append needs d %% 64 == 0");
  const void* ptrs[] = {w->Wq, w->Wk, w->Wv, w->E, H, k_cache, v_cache, attn_out};
  if ((st = check_bf16_align(dims, ptrs, 8)) != DG_OK) return st;
  const StepLayout L = step_layout(dims);
  if (!ws || ws_bytes < L.total)
    return fail(DG_EWORKSPACE, "append workspace needs %zu bytes (got %zu)", L.total, ws ? ws_bytes : 0);
  return DG_OK;
}

int enqueue_append(const dg_dims* dims, const dg_weights* w, const void* H, const int32_t* tokens_final,
                   void* k_cache, void* v_cache, void* attn_out, void* ws, hipStream_t s) {
  const StepLayout L = step_layout(dims);
  const int dt = dims->dtype, d = dims->d, Hq = dims->n_q_heads, Hkv = dims->n_kv_heads, dh = dims->head_dim;
  const int R = dims->B * dims->C;
  void* X = at(ws, L.X);
  void* Q = at(ws, L.Q);
  void* Kn = at(ws, L.Kn);
  void* Vn = at(ws, L.Vn);
  void* O = attn_out ? attn_out : at(ws, L.O);
  hipError_t e;
  if ((e = dg::launch_assemble(dt, R, d, dims->V, H, w->E, tokens_final, nullptr, X, s)) != hipSuccess)
    return hip_fail(e, "assemble");
  // the projection's epilogue also writes K_new / V_new into cache rows [L, L + C)
  if ((e = dg::launch_gemm_qkv(dt, R, d, X, w->Wq, Hq * dh, Q, w->Wk, w->Wv, Hkv * dh, Kn, Vn, s, k_cache, v_cache,
                               dg::CacheGeom{dims->C, dims->L, dims->cap, dh})) != hipSuccess)
    return hip_fail(e, "Q/K/V projections and cache write");
  dg::AttnPlan ap = dg::attn_plan(dims->B, dims->C, dims->L, dims->cap, Hq, Hkv, dh, dt, 1);
  if ((e = dg::launch_attn(ap, Q, k_cache, v_cache, Kn, Vn, O, nullptr, at(ws, L.scratch), s)) != hipSuccess)
    return hip_fail(e, "causal attention");
  return DG_OK;
}

// The per-step tensors of step s of block k in the block loop.
dg_step_io block_step_io(const dg_dims* dims, const dg_block_io* io, int steps, int k, int s) {
  const size_t R = (size_t)dims->B * dims->C, es = esize(dims->dtype);
  const size_t slab = R * dims->d * es;
  const size_t n = (size_t)k * steps + s;  // record index of this step
  dg_step_io o{};
  o.H = (const char*)io->H + (size_t)k * slab;
  o.k_cache = io->k_cache;
  o.v_cache = io->v_cache;
  if (io->trace_tokens) {
    o.tokens_in = s == 0 ? io->canvas : io->trace_tokens + (n - 1) * R;
    o.tokens_out = io->trace_tokens + n * R;
  } else {
    o.tokens_in = io->canvas + (size_t)(s & 1) * R;
    o.tokens_out = io->canvas + (size_t)((s + 1) & 1) * R;
  }
  if (io->trace_selfcond) {
    o.selfcond_in = s == 0 ? nullptr : (const char*)io->trace_selfcond + (n - 1) * slab;
    o.selfcond_out = (char*)io->trace_selfcond + n * slab;
  } else {
    o.selfcond_in = s == 0 ? nullptr : (const char*)io->selfcond + (size_t)(s & 1) * slab;
    o.selfcond_out = (char*)io->selfcond + (size_t)((s + 1) & 1) * slab;
  }
  o.max_logit = io->max_logit;
  o.conf = io->trace_conf ? io->trace_conf + n * R : io->conf;
  o.argmax = s == steps - 1 ? io->tokens + (size_t)k * R : io->argmax;
  o.mask = io->mask;
  return o;
}

int check_block_loop(const dg_dims* dims, const dg_weights* w, const dg_block_io* io, const float* taus,
                     int steps, int blocks, const void* ws, size_t ws_bytes) {
  int st = check_dims(dims, true);
  if (st != DG_OK) return st;
  if (!io || !taus) return fail(DG_EINVAL, "io and taus must be non-NULL");
  if (steps <= 0 || blocks <= 0) return fail(DG_EINVAL, "steps and blocks must be positive (%d, %d)", steps, blocks);
  if ((long long)dims->L + (long long)blocks * dims->C > dims->cap)
    return fail(DG_EINVAL, "block loop needs L + blocks*C <= cap (L=%d C=%d blocks=%d cap=%d)", dims->L,
                dims->C, blocks, dims->cap);
  if (!io->H || !io->k_cache || !io->v_cache || !io->tokens || !io->max_logit || !io->argmax ||
      !io->canvas || (!io->selfcond && !io->trace_selfcond) || (!io->conf && !io->trace_conf))
    return fail(DG_EINVAL, "H, the caches, tokens, canvas, selfcond (or trace_selfcond), max_logit, conf (or trace_conf) and argmax must be non-NULL");
  const void* ptrs[] = {io->H, io->selfcond, io->trace_selfcond};
  if ((st = check_bf16_align(dims, ptrs, 3)) != DG_OK) return st;
  // every step and append of the loop, checked before anything is enqueued
  for (int k = 0; k < blocks; ++k) {
    dg_dims dk = *dims;
    dk.L = dims->L + k * dims->C;
    for (int s = 0; s < steps; s += (steps > 1 ? steps - 1 : 1)) {
      const dg_step_io o = block_step_io(&dk, io, steps, k, s);
      if ((st = check_step(&dk, w, &o, ws, ws_bytes)) != DG_OK) return st;
    }
    if ((st = check_append(&dk, w, block_step_io(&dk, io, steps, k, 0).H, io->tokens + (size_t)k * dims->B * dims->C,
                           io->k_cache, io->v_cache, nullptr, ws, ws_bytes)) != DG_OK)
      return st;
  }
  return DG_OK;
}

int enqueue_block_loop(const dg_dims* dims, const dg_weights* w, const dg_block_io* io, const float* taus,
                       int steps, int blocks, uint64_t seed, void* ws, hipStream_t s) {
  const int R = dims->B * dims->C;
  int st;
  for (int k = 0; k < blocks; ++k) {
    dg_dims dk = *dims;
    dk.L = dims->L + k * dims->C;
    hipError_t e = dg::launch_renoise(R, dims->C, dims->V, nullptr, nullptr, 0.f, seed, 0, (uint32_t)k,
                                      io->canvas, nullptr, s);
    if (e != hipSuccess) return hip_fail(e, "initial canvas");
    for (int t = 0; t < steps; ++t) {
      const dg_step_io o = block_step_io(&dk, io, steps, k, t);
      if ((st = enqueue_step(&dk, w, &o, taus[t], seed, (uint32_t)t + 1, (uint32_t)k, ws, s)) != DG_OK) return st;
    }
    const dg_step_io o = block_step_io(&dk, io, steps, k, 0);
    if ((st = enqueue_append(&dk, w, o.H, io->tokens + (size_t)k * R, io->k_cache, io->v_cache, nullptr, ws, s)) != DG_OK)
      return st;
  }
  return DG_OK;
}

int check_attn(const dg_dims* dims, const void* q, const void* k_cache, const void* v_cache,
               const void* k_new, const void* v_new, const void* out) {
  int st = check_dims(dims, false);
  if (st != DG_OK) return st;
  if (!q || !k_new || !v_new || !out || (dims->L > 0 && (!k_cache || !v_cache)))
    return fail(DG_EINVAL, "q, k_new, v_new, out (and the caches when L > 0) must be non-NULL");
  const void* ptrs[] = {q, k_cache, v_cache, k_new, v_new, out};
  return check_bf16_align(dims, ptrs, 6);
}

// Device scratch of dg_attn_bidir_noalloc: the split partials of the
// attention live in this file-scope array instead of a caller workspace, so
// that entry point allocates nothing.  Every GPU the library runs on holds
// its own copy until the process ends.  Host code never passes the array's
// name to a kernel (on the host it is only a stand-in for the symbol): the
// device address of the copy on each device is looked up once, with that
// device current, and kept in g_scratch.
constexpr size_t kNoAllocScratchBytes = DG_ATTN_NOALLOC_MAX_BYTES;
__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];

int scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(DG_EUNSUPPORTED, "device ordinal %d is out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(DG_EHIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return DG_OK;
}

}  // namespace

struct dg_graph_s {
  hipGraphExec_t exec;
};

extern "C" {

const char* dg_status_str(int status) {
  switch (status) {
    case DG_OK: return "DG_OK";
    case DG_EINVAL: return "DG_EINVAL: invalid argument";
    case DG_EUNSUPPORTED: return "DG_EUNSUPPORTED: valid but not implemented";
    case DG_EWORKSPACE: return "DG_EWORKSPACE: workspace missing or too small";
    case DG_EHIP: return "DG_EHIP: HIP call failed";
    default: return "unknown dg_status";
  }
}

const char* dg_last_error(void) { return g_err; }

void dg_test_set_group_wait(int32_t polls) { dg::set_group_wait(polls); }

size_t dg_workspace_bytes(const dg_dims* dims) {
  if (check_dims(dims, true) != DG_OK) return 0;
  return step_layout(dims).total;
}

size_t dg_attn_workspace_bytes(const dg_dims* dims) {
  if (check_dims(dims, false) != DG_OK) return 0;
  const size_t a = attn_ws(dims, 0), b = attn_ws(dims, 1);
  return a > b ? a : b;
}

size_t dg_vocab_workspace_bytes(int32_t rows, int32_t d, int32_t V, int32_t dtype) {
  if (check_vocab_shape(rows, d, V, dtype) != DG_OK) return 0;
  return vocab_ws(rows, d, V, dtype);
}

int dg_renoise(int32_t rows, int32_t canvas, int32_t V, const int32_t* argmax, const float* conf,
               float tau, uint64_t seed, uint32_t t, uint32_t block, int32_t* tokens_out,
               uint8_t* mask_out, void* stream) {
  if (rows <= 0 || canvas <= 0 || V <= 0) return fail(DG_EINVAL, "rows, canvas, V must be positive (%d, %d, %d)", rows, canvas, V);
  if (!argmax || !conf || !tokens_out) return fail(DG_EINVAL, "argmax, conf and tokens_out must be non-NULL");
  hipError_t e = dg::launch_renoise(rows, canvas, V, argmax, conf, tau, seed, t, block, tokens_out,
                                    mask_out, (hipStream_t)stream);
  return e == hipSuccess ? DG_OK : hip_fail(e, "dg_renoise");
}

int dg_init_canvas(int32_t rows, int32_t canvas, int32_t V, uint64_t seed, uint32_t block,
                   int32_t* tokens_out, void* stream) {
  if (rows <= 0 || canvas <= 0 || V <= 0) return fail(DG_EINVAL, "rows, canvas, V must be positive (%d, %d, %d)", rows, canvas, V);
  if (!tokens_out) return fail(DG_EINVAL, "tokens_out must be non-NULL");
  hipError_t e = dg::launch_renoise(rows, canvas, V, nullptr, nullptr, 0.f, seed, 0, block,
                                    tokens_out, nullptr, (hipStream_t)stream);
  return e == hipSuccess ? DG_OK : hip_fail(e, "dg_init_canvas");
}

size_t dg_tiled_embedding_bytes(int32_t V, int32_t d, int32_t dtype) {
  if (dtype != DG_BF16 || V <= 0 || d <= 0 || d % 32) return 0;
  return ((size_t)V + 15) / 16 * 16 * (size_t)d * 2;
}

int dg_pack_embedding(int32_t V, int32_t d, int32_t dtype, const void* E, void* E_tiled, void* stream) {
  if (dtype != DG_BF16) return fail(DG_EUNSUPPORTED, "only bf16 tables have a tiled layout");
  if (V <= 0 || d <= 0 || d % 32) return fail(DG_EINVAL, "need V > 0 and d %% 32 == 0 (V=%d d=%d)", V, d);
  if (!E || !E_tiled) return fail(DG_EINVAL, "E and E_tiled must be non-NULL");
  if (!aligned16(E) || !aligned16(E_tiled)) return fail(DG_EINVAL, "E and E_tiled must be 16-byte aligned");
  const size_t n = dg_tiled_embedding_bytes(V, d, dtype);
  const char *a = (const char*)E, *b = (const char*)E_tiled;
  if (a < b + n && b < a + (size_t)V * d * 2) return fail(DG_EINVAL, "E_tiled must not overlap E");
  hipError_t e = dg::launch_pack_embedding(V, d, E, E_tiled, (hipStream_t)stream);
  return e == hipSuccess ? DG_OK : hip_fail(e, "dg_pack_embedding");
}

int dg_vocab_selfcond(int32_t rows, int32_t d, int32_t V, int32_t dtype, const void* z,
                      const void* E, float* max_logit, int32_t* argmax, float* conf, float* lse,
                      void* selfcond, void* ws, size_t ws_bytes, void* stream) {
  int st = check_vocab_shape(rows, d, V, dtype);
  if (st != DG_OK) return st;
  if (!z || !E || !max_logit || !argmax || !conf || !selfcond)
    return fail(DG_EINVAL, "z, E, max_logit, argmax, conf and selfcond must be non-NULL");
  if (dtype == DG_BF16 && (!aligned16(z) || !aligned16(E) || !aligned16(selfcond)))
    return fail(DG_EINVAL, "bf16 z, E and selfcond must be 16-byte aligned");
  const size_t need = vocab_ws(rows, d, V, dtype);
  if (need && (!ws || ws_bytes < need))
    return fail(DG_EWORKSPACE, "vocab workspace needs %zu bytes (got %zu)", need, ws ? ws_bytes : 0);
  dg::VocabPlan p = dg::vocab_plan(rows, d, V, dtype);
  hipError_t e = dg::launch_vocab(p, z, E, max_logit, argmax, conf, lse, selfcond, ws, (hipStream_t)stream);
  return e == hipSuccess ? DG_OK : hip_fail(e, "dg_vocab_selfcond");
}

int dg_attn_bidir(const dg_dims* dims, const void* q, const void* k_cache, const void* v_cache,
                  const void* k_new, const void* v_new, void* out, float* lse_out, int causal,
                  void* ws, size_t ws_bytes, void* stream) {
  int st = check_attn(dims, q, k_cache, v_cache, k_new, v_new, out);
  if (st != DG_OK) return st;
  const size_t need = attn_ws(dims, causal ? 1 : 0);
  if (need && (!ws || ws_bytes < need))
    return fail(DG_EWORKSPACE, "attention workspace needs %zu bytes (got %zu)", need, ws ? ws_bytes : 0);
  dg::AttnPlan p = dg::attn_plan(dims->B, dims->C, dims->L, dims->cap, dims->n_q_heads, dims->n_kv_heads,
                                 dims->head_dim, dims->dtype, causal ? 1 : 0);
  hipError_t e = dg::launch_attn(p, q, k_cache, v_cache, k_new, v_new, out, lse_out, ws, (hipStream_t)stream);
  return e == hipSuccess ? DG_OK : hip_fail(e, "dg_attn_bidir");
}

int dg_attn_bidir_noalloc(const dg_dims* dims, const void* q, const void* k_cache, const void* v_cache,
                          const void* k_new, const void* v_new, void* out, float* lse_out, int causal,
                          void* stream) {
  int st = check_attn(dims, q, k_cache, v_cache, k_new, v_new, out);
  if (st != DG_OK) return st;
  const size_t need = attn_ws(dims, causal ? 1 : 0);
  if (need > kNoAllocScratchBytes)
    return fail(DG_EWORKSPACE, "this shape needs %zu bytes of split partials; the built-in scratch holds %zu",
                need, kNoAllocScratchBytes);
  void* sc = nullptr;
  if (need && (st = scratch_of_current_device(&sc)) != DG_OK) return st;
  dg::AttnPlan p = dg::attn_plan(dims->B, dims->C, dims->L, dims->cap, dims->n_q_heads, dims->n_kv_heads,
                                 dims->head_dim, dims->dtype, causal ? 1 : 0);
  hipError_t e = dg::launch_attn(p, q, k_cache, v_cache, k_new, v_new, out, lse_out, sc, (hipStream_t)stream);
  return e == hipSuccess ? DG_OK : hip_fail(e, "dg_attn_bidir_noalloc");
}

int dg_denoise_step(const dg_dims* dims, const dg_weights* w, const dg_step_io* io, float tau,
                    uint64_t seed, uint32_t t, uint32_t block, void* ws, size_t ws_bytes,
                    void* stream) {
  int st = check_step(dims, w, io, ws, ws_bytes);
  if (st != DG_OK) return st;
  return enqueue_step(dims, w, io, tau, seed, t, block, ws, (hipStream_t)stream);
}

int dg_denoise_step_masked(const dg_dims* dims, const dg_weights* w, const dg_step_io* io, float tau,
                           int32_t mask_id, void* ws, size_t ws_bytes, void* stream) {
  int st = check_step(dims, w, io, ws, ws_bytes);
  if (st != DG_OK) return st;
  if (mask_id < 0 || mask_id >= dims->V) return fail(DG_EINVAL, "mask_id must lie in [0, V) (got %d, V=%d)", mask_id, dims->V);
  return enqueue_step(dims, w, io, tau, 0, 0, 0, ws, (hipStream_t)stream, mask_id);
}

int dg_unmask(int32_t rows, const int32_t* argmax, const float* conf, float tau, int32_t mask_id,
              const int32_t* tokens_in, int32_t* tokens_out, uint8_t* commit_out, void* stream) {
  if (rows <= 0 || mask_id < 0) return fail(DG_EINVAL, "rows must be positive and mask_id non-negative (%d, %d)", rows, mask_id);
  if (!argmax || !conf || !tokens_in || !tokens_out)
    return fail(DG_EINVAL, "argmax, conf, tokens_in and tokens_out must be non-NULL");
  hipError_t e = dg::launch_unmask(rows, argmax, conf, tau, mask_id, tokens_in, tokens_out, commit_out,
                                   (hipStream_t)stream);
  return e == hipSuccess ? DG_OK : hip_fail(e, "dg_unmask");
}

int dg_init_masked(int32_t rows, int32_t mask_id, int32_t* tokens_out, void* stream) {
  if (rows <= 0 || mask_id < 0) return fail(DG_EINVAL, "rows must be positive and mask_id non-negative (%d, %d)", rows, mask_id);
  if (!tokens_out) return fail(DG_EINVAL, "tokens_out must be non-NULL");
  hipError_t e = dg::launch_unmask(rows, nullptr, nullptr, 0.f, mask_id, nullptr, tokens_out, nullptr,
                                   (hipStream_t)stream);
  return e == hipSuccess ? DG_OK : hip_fail(e, "dg_init_masked");
}

int dg_prefill_append(const dg_dims* dims, const dg_weights* w, const void* H,
                      const int32_t* tokens_final, void* k_cache, void* v_cache, void* attn_out,
                      void* ws, size_t ws_bytes, void* stream) {
  int st = check_append(dims, w, H, tokens_final, k_cache, v_cache, attn_out, ws, ws_bytes);
  if (st != DG_OK) return st;
  return enqueue_append(dims, w, H, tokens_final, k_cache, v_cache, attn_out, ws, (hipStream_t)stream);
}

int dg_block_loop(const dg_dims* dims, const dg_weights* w, const dg_block_io* io, const float* taus,
                  int32_t steps, int32_t blocks, uint64_t seed, void* ws, size_t ws_bytes,
                  void* stream) {
  int st = check_block_loop(dims, w, io, taus, steps, blocks, ws, ws_bytes);
  if (st != DG_OK) return st;
  return enqueue_block_loop(dims, w, io, taus, steps, blocks, seed, ws, (hipStream_t)stream);
}

int dg_graph_capture_block_loop(const dg_dims* dims, const dg_weights* w, const dg_block_io* io,
                                const float* taus, int32_t steps, int32_t blocks, uint64_t seed,
                                void* ws, size_t ws_bytes, void* stream, dg_graph* graph) {
  if (!graph) return fail(DG_EINVAL, "graph must be non-NULL");
  *graph = nullptr;
  if (!stream) return fail(DG_EINVAL, "graph capture needs a created stream, not the NULL stream");
  int st = check_block_loop(dims, w, io, taus, steps, blocks, ws, ws_bytes);
  if (st != DG_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal);
  if (e != hipSuccess) return hip_fail(e, "hipStreamBeginCapture");
  st = enqueue_block_loop(dims, w, io, taus, steps, blocks, seed, ws, s);
  hipGraph_t g = nullptr;
  e = hipStreamEndCapture(s, &g);
  if (st != DG_OK) {
    if (g) hipGraphDestroy(g);
    return st;
  }
  if (e != hipSuccess) {
    if (g) hipGraphDestroy(g);
    return hip_fail(e, "hipStreamEndCapture");
  }
  hipGraphExec_t x = nullptr;
  e = hipGraphInstantiateWithFlags(&x, g, 0);
  hipGraphDestroy(g);
  if (e != hipSuccess) return hip_fail(e, "hipGraphInstantiate");
  dg_graph out = new (std::nothrow) dg_graph_s;
  if (!out) {
    hipGraphExecDestroy(x);
    return fail(DG_EINVAL, "out of host memory");
  }
  out->exec = x;
  *graph = out;
  return DG_OK;
}

int dg_graph_launch(dg_graph graph, void* stream) {
  if (!graph || !graph->exec) return fail(DG_EINVAL, "graph is NULL");
  hipError_t e = hipGraphLaunch(graph->exec, (hipStream_t)stream);
  return e == hipSuccess ? DG_OK : hip_fail(e, "hipGraphLaunch");
}

void dg_graph_destroy(dg_graph graph) {
  if (!graph) return;
  if (graph->exec) hipGraphExecDestroy(graph->exec);
  delete graph;
}

}  // extern "C"
