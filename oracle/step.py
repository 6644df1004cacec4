"""numpy float64 oracle of one canvas denoise step (and the causal append).

Each function follows a passage of the DiffusionGemma explainer; readings of
what the pages leave open are stated where they are used.  Shapes:

  H      [B, C, d]        canvas hidden states (the backbone's input rows)
  E      [V, d]           token-embedding table, also the (tied) vocabulary head
  Wq     [Hq*dh, d]       projection weights stored output-major (linear layer)
  Wk, Wv [Hkv*dh, d]
  Wo     [d, Hq*dh]
  Kc, Vc [B, Hkv, cap, dh] KV cache, rows [0, L) valid
  x      [B, C] int       canvas tokens
  S      [B, C, d]        self-conditioning vector from the previous step

All float inputs are float64 arrays holding the stored (already rounded)
values; ``dtype`` names the storage precision that API-visible results are
rounded to.
"""
import math

import numpy as np

from .numerics import round_store
from .philox import draw_tokens


# -- assemble -------------------------------------------------------------------

def assemble(H, E, x, S_prev, dtype):
    """The denoiser reads the canvas (its tokens' embeddings) on top of the
    hidden rows, plus the self-conditioning vector handed over from the
    previous step ("Autocondizionamento": the result is passed directly to the
    next step).  Reading taken: X = H + E[x] + S_prev with S_prev = 0 on a
    block's first step; no embedding scale."""
    X = H + E[x]
    if S_prev is not None:
        X = X + S_prev
    return round_store(X, dtype)


def linear(X, W, dtype):
    """Y = X . W^T for an output-major weight W[out, in]; stored rounding."""
    return round_store(X @ W.T, dtype)


# -- attention --------------------------------------------------------------------

def attention(Q, Kc, Vc, Kn, Vn, L, causal, dtype=None):
    """Canvas attention over [cache rows 0..L) || canvas rows 0..C).

    Denoise mode ("Architettura...", bidirectional denoising): every canvas
    query attends to every canvas token and to the whole KV cache -- no mask.
    Prefill mode (same section, causal prefill): query i sees the whole cache
    and canvas keys 0..i, i.e. key j is kept iff j < L + i + 1.

    GQA: query head h uses KV head floor(h / (Hq/Hkv)).  Scores are scaled by
    1/sqrt(dh) (reading: the standard scale; the pages give none).
    Returns O [B, C, Hq, dh] (rounded to dtype when given) and the natural-log
    sum-exp of the scaled scores, lse [B, C, Hq] (float64).
    """
    B, C, Hq, dh = Q.shape
    Hkv = Kn.shape[2]
    G = Hq // Hkv
    O = np.empty((B, C, Hq, dh))
    lse = np.empty((B, C, Hq))
    scale = 1.0 / math.sqrt(dh)
    if causal:
        j = np.arange(L + C)[None, :]
        i = np.arange(C)[:, None]
        keep = j < (L + i + 1)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            keys = np.concatenate([Kc[b, g, :L], Kn[b, :, g]], axis=0)   # [L+C, dh]
            vals = np.concatenate([Vc[b, g, :L], Vn[b, :, g]], axis=0)
            s = (Q[b, :, h] @ keys.T) * scale                              # [C, L+C]
            if causal:
                s = np.where(keep, s, -np.inf)
            m = s.max(axis=1, keepdims=True)
            p = np.exp(s - m)
            l = p.sum(axis=1, keepdims=True)
            O[b, :, h] = (p @ vals) / l
            lse[b, :, h] = (m + np.log(l))[:, 0]
    if dtype is not None:
        O = round_store(O, dtype)
    return O, lse


def attention_row(q, b, g, i, Kc, Vc, Kn, Vn, L, causal):
    """The same attention for one query vector q [dh] of canvas b at position
    i, read against KV head g (used to check sampled rows at full size).
    Returns (o [dh], lse)."""
    keys = np.concatenate([Kc[b, g, :L], Kn[b, :, g]], axis=0)
    vals = np.concatenate([Vc[b, g, :L], Vn[b, :, g]], axis=0)
    if causal:
        keys = keys[:L + i + 1]
        vals = vals[:L + i + 1]
    s = (keys @ q) / math.sqrt(q.shape[0])
    m = s.max()
    p = np.exp(s - m)
    l = p.sum()
    return (p @ vals) / l, m + math.log(l)


# -- vocabulary head, confidence and self-conditioning ----------------------------

def vocab_selfcond(Z, E, dtype=None, rows=256):
    """Full-vocabulary softmax of the tied head l = Z . E^T, per row:

      m   = max_v l_v                  a = lowest v attaining m
      lse = m + ln sum_v exp(l_v - m)  c = exp(m - lse)  (max probability)
      S   = sum_v P_v E_v with P = exp(l - lse)
      gap = m - max_{v != a} l_v       (top-2 logit gap; +inf when V = 1)

    The confidence compared with the threshold is read as the largest
    probability of the row, i.e. how sure the model is of its own prediction
    ("Diffusione dello stato uniforme").  S is the probability matrix times
    the embedding table ("Autocondizionamento").  For each block of `rows`
    rows the whole logits row is formed once and every statistic is read
    from it directly.  The gap is not part of the method: the parity tests
    use it to recognise near-ties of the argmax.
    Z [R, d], E [V, d] -> m, a, lse, c, gap [R] and S [R, d] (S rounded to
    dtype when given).
    """
    R = Z.shape[0]
    V = E.shape[0]
    m = np.empty(R)
    a = np.empty(R, np.int64)
    lse = np.empty(R)
    gap = np.empty(R)
    S = np.empty((R, E.shape[1]))
    for r0 in range(0, R, rows):
        lg = Z[r0:r0 + rows] @ E.T                   # [n, V] logits
        n = lg.shape[0]
        idx = np.arange(n)
        ai = lg.argmax(axis=1)                       # first index among equal maxima
        mi = lg[idx, ai]
        if V > 1:
            lg[idx, ai] = -np.inf                    # the best logit of the other ids
            gap[r0:r0 + n] = mi - lg.max(axis=1)
            lg[idx, ai] = mi
        else:
            gap[r0:r0 + n] = np.inf
        p = np.exp(lg - mi[:, None])
        l = p.sum(axis=1)
        m[r0:r0 + n] = mi
        a[r0:r0 + n] = ai
        lse[r0:r0 + n] = mi + np.log(l)
        S[r0:r0 + n] = (p @ E) / l[:, None]
    c = np.exp(m - lse)
    if dtype is not None:
        S = round_store(S, dtype)
    return m, a, lse, c, S, gap


# -- uniform-state renoise ---------------------------------------------------------

def renoise(a, c, tau, seed, t, block, B, C, V):
    """"Diffusione dello stato uniforme": a position whose probability drops
    below the threshold is renoised with a new random vocabulary token; the
    others keep the model's prediction.  Readings: the probability is the
    confidence c (max probability); "below" is strict (c < tau, the threshold
    taken as a float32 as the kernel receives it); a kept position takes the
    argmax a; the replacement is uniform over all V ids (Philox draw t).
    a, c: [B*C] -> new tokens [B*C] int64, mask [B*C] uint8."""
    tau32 = float(np.float32(tau))
    mask = (np.asarray(c, np.float64) < tau32)
    U = draw_tokens(seed, t, block, B, C, V).reshape(-1)
    x_new = np.where(mask, U, np.asarray(a, np.int64))
    return x_new, mask.astype(np.uint8)


def init_canvas(seed, block, B, C, V):
    """A block's canvas starts as random vocabulary tokens ("Il problema con i
    modelli autoregressivi": 256 random tokens; table row "Punto iniziale").
    Draw index t = 0."""
    return draw_tokens(seed, 0, block, B, C, V)


# -- masked diffusion --------------------------------------------------------------

def unmask(a, c, tau, x, mask_id):
    """"Diffusione mascherata": noise is an explicit [MASK] token; in the
    reverse process the model predicts the token behind each mask and the
    prediction replaces the mask where its confidence meets the threshold.
    A replaced token is locked: later steps never change it.  Readings: the
    confidence is c (max probability) and "meets" is c >= tau (tau taken as a
    float32, the complement of the uniform-state "below"); the committed
    token is the argmax a; a prediction equal to the mask id commits nothing
    (the position stays masked); [MASK] is a caller-chosen vocabulary id.
    a, c, x: [B*C] -> new tokens [B*C] int64, newly committed [B*C] uint8."""
    tau32 = float(np.float32(tau))
    x = np.asarray(x, np.int64).reshape(-1)
    a = np.asarray(a, np.int64).reshape(-1)
    commit = (x == mask_id) & (np.asarray(c, np.float64).reshape(-1) >= tau32) & (a != mask_id)
    return np.where(commit, a, x), commit.astype(np.uint8)


def init_masked(B, C, mask_id):
    """A masked-diffusion canvas starts fully masked (all noise)."""
    return np.full((B, C), mask_id, np.int64)


# -- the step -------------------------------------------------------------------

def forward(H, E, W, Kc, Vc, L, x, S_prev, dtype):
    """Steps 1-5 of a denoise step, shared by both samplers: the model reads
    the canvas and returns every intermediate, the prediction a, its
    confidence c and the self-conditioning vector S."""
    B, C, d = H.shape
    dh = Kc.shape[3]
    Hq = W["Wq"].shape[0] // dh
    Hkv = W["Wk"].shape[0] // dh
    X = assemble(H, E, x, S_prev, dtype)
    Xf = X.reshape(B * C, d)
    Q = linear(Xf, W["Wq"], dtype).reshape(B, C, Hq, dh)
    Kn = linear(Xf, W["Wk"], dtype).reshape(B, C, Hkv, dh)
    Vn = linear(Xf, W["Wv"], dtype).reshape(B, C, Hkv, dh)
    O, lse_att = attention(Q, Kc, Vc, Kn, Vn, L, causal=False, dtype=dtype)
    Z = round_store(Xf + O.reshape(B * C, Hq * dh) @ W["Wo"].T, dtype)
    m, a, lse, c, S, gap = vocab_selfcond(Z, E, dtype)
    return dict(X=X, Q=Q, Kn=Kn, Vn=Vn, O=O, lse_att=lse_att, Z=Z.reshape(B, C, d),
                m=m, a=a, lse=lse, c=c, S=S.reshape(B, C, d), gap=gap)


def denoise_step_masked(H, E, W, Kc, Vc, L, x, S_prev, tau, mask_id, dtype):
    """One step of the masked-diffusion sampler: the same model pass as
    denoise_step, then unmask-and-lock instead of the uniform renoise.
    Returns the intermediates plus x_new and `commit` (newly unmasked)."""
    B, C, _ = H.shape
    r = forward(H, E, W, Kc, Vc, L, x, S_prev, dtype)
    x_new, commit = unmask(r["a"], r["c"], tau, x, mask_id)
    r.update(x_new=x_new.reshape(B, C), commit=commit.reshape(B, C))
    return r


def denoise_step(H, E, W, Kc, Vc, L, x, S_prev, tau, seed, t, block, dtype):
    """One denoise step over all B canvases.  W = dict(Wq, Wk, Wv, Wo).

    1 X = H + E[x] + S_prev                  (assemble)
    2 Q, K_new, V_new = X Wq^T, X Wk^T, X Wv^T
    3 O = bidirectional attention over [cache || canvas]
    4 Z = X + O Wo^T                          (residual)
    5 m, a, lse, c, S = vocab head and self-conditioning of Z
    6 x', mask = renoise(a, c)                (draw index t)
    The cache is only read (denoise never writes it; only prefill does,
    "Architettura...").  Returns a dict of every intermediate.
    """
    B, C, _ = H.shape
    V = E.shape[0]
    r = forward(H, E, W, Kc, Vc, L, x, S_prev, dtype)
    x_new, mask = renoise(r["a"], r["c"], tau, seed, t, block, B, C, V)
    r.update(x_new=x_new.reshape(B, C), mask=mask.reshape(B, C))
    return r


def prefill_append(H, E, W, Kc, Vc, L, x_final, dtype):
    """Incremental prefill of a finished block ("Architettura...": causal
    attention writes the KV cache, once per block, before the next canvas;
    "Campionamento multi-canvas": the completed block joins the context).
    X = H + E[x_final] (no self-conditioning), K_new/V_new written at cache
    rows [L, L+C), then causal attention (query i sees the cache and canvas
    keys 0..i).  Returns (Kc', Vc', O, lse) with copies of the caches."""
    B, C, d = H.shape
    dh = Kc.shape[3]
    Hq = W["Wq"].shape[0] // dh
    Hkv = W["Wk"].shape[0] // dh
    X = assemble(H, E, x_final, None, dtype).reshape(B * C, d)
    Q = linear(X, W["Wq"], dtype).reshape(B, C, Hq, dh)
    Kn = linear(X, W["Wk"], dtype).reshape(B, C, Hkv, dh)
    Vn = linear(X, W["Wv"], dtype).reshape(B, C, Hkv, dh)
    O, lse = attention(Q, Kc, Vc, Kn, Vn, L, causal=True, dtype=dtype)
    Kc2 = Kc.copy()
    Vc2 = Vc.copy()
    Kc2[:, :, L:L + C] = Kn.transpose(0, 2, 1, 3)
    Vc2[:, :, L:L + C] = Vn.transpose(0, 2, 1, 3)
    return Kc2, Vc2, O, lse
