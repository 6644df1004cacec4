/*
 * dg.h -- C ABI of the canvas denoise step for uniform-state text diffusion,
 * hand-written HIP kernels for AMD Instinct MI355X (gfx950).
 *
 * The method is the one the DiffusionGemma explainer describes
 * (ai.google.dev, "DiffusionGemma explained"; sections cited by their Italian
 * headings).  One denoise step over a canvas of C tokens:
 *
 *   X   = H + E[x] + S_prev                     self-conditioning input
 *   Q,K,V = X Wq^T, X Wk^T, X Wv^T              projections
 *   O   = attention(Q; [cache || canvas])       bidirectional, no mask
 *   Z   = X + O Wo^T
 *   l   = Z E^T;  m = max l;  a = argmax l;  c = exp(m - lse)
 *   S   = softmax(l) E                          P.E, P never stored
 *   x'  = c < tau ? uniform token : a           uniform-state renoise
 *
 * Conventions shared by every entry point
 * ----------------------------------------
 *  - Every pointer argument is a DEVICE pointer owned by the caller; the
 *    library never allocates, frees, copies to the host or synchronises.
 *    Every call only enqueues kernels on `stream` (a hipStream_t; NULL is the
 *    default stream), so calls can be captured in a HIP graph.
 *  - Tensors are dense row-major in the index order written next to them.
 *    Floating tensors are float32 (DG_F32) or bfloat16 bit patterns
 *    (DG_BF16) as selected by `dtype`; statistics (max_logit, conf, lse) are
 *    always float32, token ids int32, masks uint8.  bf16 inputs are multiplied
 *    exactly and accumulated in float32; bf16 outputs are rounded to nearest
 *    even.
 *  - Base pointers of bf16 tensors must be 16-byte aligned.
 *  - Outputs must not alias inputs except where an entry point says so.
 *  - Arguments are checked before anything is enqueued: a failed check returns
 *    a negative dg_status, enqueues nothing and leaves outputs untouched; the
 *    reason is in dg_last_error() (per calling thread).  A HIP launch failure
 *    returns DG_EHIP.  Nothing aborts, prints or throws across the ABI.
 *  - Token ids read by a kernel must lie in [0, V); an id outside that range
 *    is read as id 0 (never out of bounds).
 *  - The library is stateless and reentrant; concurrent calls on different
 *    streams must use different workspaces.
 */
#ifndef DG_H
#define DG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { DG_F32 = 0, DG_BF16 = 1 } dg_dtype;

typedef enum {
  DG_OK = 0,
  DG_EINVAL = -1,        /* NULL pointer, bad size, bad alignment, Hq % Hkv != 0 ... */
  DG_EUNSUPPORTED = -2,  /* valid but not implemented (e.g. bf16 head_dim not 64/128) */
  DG_EWORKSPACE = -3,    /* workspace NULL or smaller than the *_workspace_bytes figure */
  DG_EHIP = -4           /* a HIP call failed; text in dg_last_error() */
} dg_status;

/* Sizes of one step.  B canvases of C tokens; the cache holds `cap` rows per
 * (canvas, KV head), of which rows [0, L) are valid.  GQA: query head h reads
 * KV head h / (n_q_heads / n_kv_heads). */
typedef struct {
  int32_t B, C, L, cap, d, n_q_heads, n_kv_heads, head_dim, V;
  int32_t dtype; /* dg_dtype */
} dg_dims;

/* Model tensors.  Projection weights are stored output-major, like a linear
 * layer's weight: Wq[Hq*dh][d], Wk[Hkv*dh][d], Wv[Hkv*dh][d], Wo[d][Hq*dh].
 * E is the token-embedding table, also the tied vocabulary head: for DG_F32
 * the row-major E[V][d]; for DG_BF16 the same table in the tiled layout of
 * dg_pack_embedding (the only copy the bf16 path needs: the vocabulary head
 * streams it and the token gathers read their rows from it). */
typedef struct {
  const void *Wq, *Wk, *Wv, *Wo, *E;
} dg_weights;

/* Per-step tensors (R = B*C rows, row r = canvas r / C, position r % C). */
typedef struct {
  const void *H;            /* [B][C][d] canvas hidden rows */
  const void *k_cache;      /* [B][Hkv][cap][dh]; rows [0, L) are read */
  const void *v_cache;      /* [B][Hkv][cap][dh] */
  const int32_t *tokens_in; /* [B][C] canvas tokens x_t */
  const void *selfcond_in;  /* [B][C][d] S from the previous step; NULL reads 0 */
  int32_t *tokens_out;      /* [B][C] x_{t+1}; may equal tokens_in */
  void *selfcond_out;       /* [B][C][d] S of this step; may equal selfcond_in */
  float *max_logit;         /* [R] m */
  float *conf;              /* [R] c = max probability */
  float *lse;               /* [R] log-sum-exp of the logits; may be NULL */
  int32_t *argmax;          /* [R] lowest id attaining m */
  uint8_t *mask;            /* [R] 1 where the position was renoised; may be NULL */
  /* Optional copies of the intermediates (NULL: kept in the workspace). */
  void *x_out;              /* [R][d]        X */
  void *q_out;              /* [R][Hq][dh]   Q */
  void *k_new_out;          /* [R][Hkv][dh]  canvas keys */
  void *v_new_out;          /* [R][Hkv][dh]  canvas values */
  void *attn_out;           /* [R][Hq][dh]   O */
  void *z_out;              /* [R][d]        Z */
  /* Optional profiling hooks: hipEvent_t handles recorded on `stream` right
   * before and right after the main attention kernel and the main flash-vocab
   * kernel (split combines excluded).  NULL: nothing is recorded. */
  void *ev_attn_begin, *ev_attn_end;
  void *ev_vocab_begin, *ev_vocab_end;
} dg_step_io;

/* Workspace bytes needed by dg_denoise_step and dg_prefill_append for dims. */
size_t dg_workspace_bytes(const dg_dims *dims);

/* One denoise step for all B canvases ("Diffusione dello stato uniforme" and
 * "Autocondizionamento"; attention as in "Architettura: il prefill
 * incrementale e il denoising", denoising mode).  The cache is only read.
 * tau: renoise threshold (a position is renoised iff conf < tau).
 * seed, t, block: Philox4x64-10 key (seed, 0) and counter words (position i,
 * draw index t, canvas b, block); the initial canvas of a block is draw 0,
 * so denoise step s of a block should pass t = s + 1.
 * ws/ws_bytes: device workspace of at least dg_workspace_bytes(dims). */
int dg_denoise_step(const dg_dims *dims, const dg_weights *w, const dg_step_io *io,
                    float tau, uint64_t seed, uint32_t t, uint32_t block,
                    void *ws, size_t ws_bytes, void *stream);

/* Canvas attention ("Architettura..."): for canvas b, query head h, position
 * i, O = softmax_j(q.k_j / sqrt(dh)) v_j over keys j in
 * [k_cache[b][g][0..L) || k_new[b][0..C)[g]], g = h / (Hq/Hkv).
 * causal = 0: every key (denoising).  causal = 1: key j is kept iff
 * j < L + i + 1 (prefill of a block after an L-row cache).
 * q[B][C][Hq][dh], k_new/v_new[B][C][Hkv][dh], caches as in dg_step_io,
 * out[B][C][Hq][dh]; lse_out[B][C][Hq] (natural log, float32) may be NULL.
 * Only dims->{B,C,L,cap,n_q_heads,n_kv_heads,head_dim,dtype} are used.
 * bf16 needs head_dim 64 or 128 and cap * head_dim * 2 < 2^31 (one cache
 * slab is addressed with 32-bit offsets); otherwise DG_EUNSUPPORTED. */
size_t dg_attn_workspace_bytes(const dg_dims *dims);
int dg_attn_bidir(const dg_dims *dims, const void *q, const void *k_cache, const void *v_cache,
                  const void *k_new, const void *v_new, void *out, float *lse_out, int causal,
                  void *ws, size_t ws_bytes, void *stream);

/* dg_attn_bidir for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation and kernels, with the split partials kept in a
 * scratch array built into the library instead of a caller workspace.  The
 * call allocates nothing and frees nothing; the caller still passes the
 * inputs and outputs.  Each GPU the library runs on holds one copy of the
 * array (DG_ATTN_NOALLOC_MAX_BYTES, 64 MiB) from the first call on
 * that device until the process ends.  A shape whose partials need more
 * (dg_attn_workspace_bytes(dims) larger than that) returns DG_EWORKSPACE
 * and enqueues nothing; the single-canvas 256-token denoising shapes with up
 * to 32 query heads and the 16-query long-cache shape fit.  All calls on one
 * GPU share its array: calls that may overlap in time on one GPU (different
 * streams, or different host threads) race on it and must be serialised by
 * the caller; consecutive calls on one stream are safe.  Arguments and
 * errors as for dg_attn_bidir. */
#define DG_ATTN_NOALLOC_MAX_BYTES ((size_t)64 << 20)
int dg_attn_bidir_noalloc(const dg_dims *dims, const void *q, const void *k_cache, const void *v_cache,
                          const void *k_new, const void *v_new, void *out, float *lse_out, int causal,
                          void *stream);

/* Tiled layout of a bf16 embedding table (the form dg_weights.E takes for
 * DG_BF16; convert once per model, then the row-major table can be freed).
 * E[V][d]
 * (row-major) is cut into blocks of 16 ids x 32 columns; block (vb, c) is
 * 1 KiB at byte offset (vb * (d / 32) + c) * 1024, and inside it entry
 * (id 16 vb + r, column 32 c + 8 g + e) sits at element 8 (16 g + r) + e'
 * with e' = e for even g and e' = e ^ 4 for odd g (g < 4, r < 16, e < 8).
 * Ids in [V, 16 ceil(V/16)) read as zero.  The
 * vocabulary kernels load one block per instruction, 1 KiB contiguous, in
 * the lane order of their matrix-core operands.  Needs d % 32 == 0.
 * dg_tiled_embedding_bytes returns 16 ceil(V/16) d 2 (0 for invalid sizes or
 * DG_F32, which has no tiled layout); dg_pack_embedding writes E_tiled
 * (that many bytes, 16-byte aligned, not overlapping E) from E. */
size_t dg_tiled_embedding_bytes(int32_t V, int32_t d, int32_t dtype);
int dg_pack_embedding(int32_t V, int32_t d, int32_t dtype, const void *E, void *E_tiled,
                      void *stream);

/* Vocabulary head, confidence and self-conditioning ("Autocondizionamento";
 * confidence as in "Diffusione dello stato uniforme"): for each of `rows`
 * rows of z[rows][d] and the table E[V][d]: logits l = z E^T,
 * max_logit = max l, argmax = lowest id attaining it, lse = log sum exp l,
 * conf = exp(max_logit - lse), selfcond[rows][d] = softmax(l) E.
 * The rows x V probability matrix is never stored.  lse may be NULL.
 * E is the row-major table for DG_F32 and the tiled table of
 * dg_pack_embedding for DG_BF16. */
size_t dg_vocab_workspace_bytes(int32_t rows, int32_t d, int32_t V, int32_t dtype);
int dg_vocab_selfcond(int32_t rows, int32_t d, int32_t V, int32_t dtype, const void *z,
                      const void *E, float *max_logit, int32_t *argmax, float *conf, float *lse,
                      void *selfcond, void *ws, size_t ws_bytes, void *stream);

/* Uniform-state renoise ("Diffusione dello stato uniforme"): row r (canvas
 * b = r / canvas, position i = r % canvas) becomes
 *   conf[r] < tau ? floor(w0 * V / 2^64) : argmax[r],
 * w0 = word 0 of Philox4x64-10(counter (i, t, b, block), key (seed, 0)).
 * mask_out[r] = 1 where a token was drawn (may be NULL).  tokens_out may
 * equal argmax. */
int dg_renoise(int32_t rows, int32_t canvas, int32_t V, const int32_t *argmax, const float *conf,
               float tau, uint64_t seed, uint32_t t, uint32_t block, int32_t *tokens_out,
               uint8_t *mask_out, void *stream);

/* A block's starting canvas ("Il problema con i modelli autoregressivi":
 * random vocabulary tokens): every row drawn as in dg_renoise with t = 0. */
int dg_init_canvas(int32_t rows, int32_t canvas, int32_t V, uint64_t seed, uint32_t block,
                   int32_t *tokens_out, void *stream);

/* Masked diffusion ("Diffusione mascherata"), the sampler the pages contrast
 * with uniform-state diffusion: noise is an explicit [MASK] token, here the
 * caller-chosen vocabulary id mask_id.  Row r becomes
 *   tokens_in[r] == mask_id && conf[r] >= tau && argmax[r] != mask_id
 *       ? argmax[r] : tokens_in[r]
 * so a committed token is locked (never changed again) and a prediction of
 * the mask id itself commits nothing.  commit_out[r] = 1 where this call
 * unmasked the row (may be NULL).  tokens_out may equal tokens_in. */
int dg_unmask(int32_t rows, const int32_t *argmax, const float *conf, float tau, int32_t mask_id,
              const int32_t *tokens_in, int32_t *tokens_out, uint8_t *commit_out, void *stream);

/* A fully masked canvas: every row of tokens_out[rows] set to mask_id. */
int dg_init_masked(int32_t rows, int32_t mask_id, int32_t *tokens_out, void *stream);

/* One step of the masked sampler: the model pass of dg_denoise_step (same
 * dims, weights, io and workspace), then dg_unmask instead of the
 * uniform-state renoise.  io->mask receives the commit flags.  mask_id must
 * lie in [0, V). */
int dg_denoise_step_masked(const dg_dims *dims, const dg_weights *w, const dg_step_io *io,
                           float tau, int32_t mask_id, void *ws, size_t ws_bytes, void *stream);

/* Incremental prefill of a finished block ("Architettura...", causal
 * prefill; "Campionamento multi-canvas (diffusione a blocchi)"):
 * X = H + E[tokens_final] (no self-conditioning), canvas keys/values
 * X Wk^T, X Wv^T are written to cache rows [L, L+C) of every (canvas, KV
 * head), and causal attention of X Wq^T over [cache rows 0..L) || canvas] is
 * written to attn_out[B][C][Hq][dh] (may be NULL: then it goes to the
 * workspace).  Requires L + C <= cap.  The caller then uses L + C as the
 * cache length. */
int dg_prefill_append(const dg_dims *dims, const dg_weights *w, const void *H,
                      const int32_t *tokens_final, void *k_cache, void *v_cache, void *attn_out,
                      void *ws, size_t ws_bytes, void *stream);

/* Block diffusion ("Campionamento multi-canvas (diffusione a blocchi)"):
 * `blocks` canvases diffused one after another, each for `steps` denoise
 * steps and then appended to the KV cache by the causal prefill
 * ("Architettura: il prefill incrementale e il denoising").  For block k
 * (cache length L_k = dims->L + k C):
 *   canvas = dg_init_canvas(draw 0 of block k)
 *   for s in 0..steps-1: dg_denoise_step(tau = taus[s], t = s + 1, block = k,
 *       cache length L_k; the first step reads no self-conditioning vector)
 *   tokens[k] = argmax of the last step (the finished canvas, not renoised)
 *   dg_prefill_append(H[k], tokens[k]): cache rows [L_k, L_k + C) are written
 * Needs dims->cap >= dims->L + blocks C.  Every pointer is a caller-owned
 * device pointer; R = B C. */
typedef struct {
  const void *H;            /* [blocks][B][C][d] hidden rows of each block's canvas */
  void *k_cache, *v_cache;  /* [B][Hkv][cap][dh]; rows [0, L) valid on entry */
  int32_t *tokens;          /* [blocks][B][C] finished canvas of every block */
  int32_t *canvas;          /* [2][B][C] working canvases; the initial canvas of a
                               block is drawn into the first [B][C] (with
                               trace_tokens set only that part is used) */
  void *selfcond;           /* [2][B][C][d] working self-conditioning vectors
                               (unused when trace_selfcond is set) */
  float *max_logit, *conf;  /* [R] statistics of the latest step (conf unused when trace_conf is set) */
  int32_t *argmax;          /* [R] argmax of the latest step but the last of a block */
  uint8_t *mask;            /* [R] renoise mask of the latest step; may be NULL */
  /* Optional per-step records (NULL: not kept).  When set, each step writes
   * its outputs there and the next step reads them from there. */
  int32_t *trace_tokens;    /* [blocks][steps][B][C] tokens after each step */
  float *trace_conf;        /* [blocks][steps][R] confidence of each step */
  void *trace_selfcond;     /* [blocks][steps][B][C][d] S of each step */
} dg_block_io;

/* Enqueues the whole block loop on `stream`.  taus is a HOST array of
 * `steps` thresholds, read during the call.  ws: dg_workspace_bytes(dims). */
int dg_block_loop(const dg_dims *dims, const dg_weights *w, const dg_block_io *io,
                  const float *taus, int32_t steps, int32_t blocks, uint64_t seed,
                  void *ws, size_t ws_bytes, void *stream);

/* The same sequence captured once into an instantiated HIP graph, replayed
 * with dg_graph_launch: one launch per whole sequence instead of one per
 * kernel.  The graph holds the pointers and scalars of the capture call, so
 * every buffer must stay allocated until dg_graph_destroy.  stream must be a
 * created stream (not NULL): capture runs on it, nothing executes during the
 * capture.  On failure *graph is NULL and nothing was launched.  Replays on
 * one graph must not overlap (they share the workspace). */
typedef struct dg_graph_s *dg_graph;
int dg_graph_capture_block_loop(const dg_dims *dims, const dg_weights *w, const dg_block_io *io,
                                const float *taus, int32_t steps, int32_t blocks, uint64_t seed,
                                void *ws, size_t ws_bytes, void *stream, dg_graph *graph);
int dg_graph_launch(dg_graph graph, void *stream);
void dg_graph_destroy(dg_graph graph);

/* Test hook of the vocabulary head at d = 2048 and 4096 on a 256-CU device.
 * There the head runs each 64-row block on a group of d/1024 workgroups that
 * exchange partial logits, which needs every member of a group resident at
 * the same time; a member that waits more than `polls` polls for the others
 * at the start makes its group compute alone ("solo": each member computes
 * the others' partial logits itself, with the same bits as a paired run).
 * This sets the bound for later launches of the calling process (< 0
 * restores the default); 0 makes every group run solo.  Results are the same
 * either way; only the speed differs.  If a resident member stops answering
 * in the middle of a launch (its exchange poll times out), the statistics and
 * S of every row are NaN and argmax is -1, and each row's token is drawn as
 * for a renoised position, so tokens stay within [0, V). */
void dg_test_set_group_wait(int32_t polls);

/* Text of a dg_status; text of the last failure on the calling thread. */
const char *dg_status_str(int status);
const char *dg_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* DG_H */
