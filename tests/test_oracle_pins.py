"""Pins for the CPU oracle against things other than itself: library routines
(numpy's Philox, torch SDPA / linear in float64, scipy's logsumexp), closed
forms, invariants the pages fix, and an independently written pure-Python
brute force.  All CPU-only."""
import math

import numpy as np
import pytest
import scipy.special
import scipy.stats
import torch

from oracle import brute, numerics, philox, step
from synth import config_by_name, from_storage, gen_problem

rng0 = np.random.default_rng(12345)


# ---- Philox4x64-10 and the uniform draw ----------------------------------------

@pytest.mark.parametrize("ctr,key", [
    ((0, 0, 0, 0), (0, 0)),
    ((5, 7, 11, 13), (1234, 0)),
    ((2**64 - 5, 3, 2**63, 9), (2**64 - 1, 2**40 + 17)),
    ((255, 31, 7, 3), (1002, 0)),
])
def test_philox_block_matches_numpy(ctr, key):
    # numpy's Philox increments its 256-bit counter before producing a block,
    # so a generator started at counter c yields block(c + 1) first.
    g = np.random.Philox(counter=np.array(ctr, dtype=np.uint64), key=np.array(key, dtype=np.uint64))
    raw = [int(v) for v in g.random_raw(4)]
    c = list(ctr)
    c[0] += 1
    for w in range(4):                       # carry like a 256-bit integer
        if c[w] >= 2**64:
            c[w] -= 2**64
            if w < 3:
                c[w + 1] += 1
    assert list(philox.philox4x64_10(c, key)) == raw


def test_philox_vectorised_matches_scalar():
    r = np.random.default_rng(1)
    n = 200
    c = r.integers(0, 2**63, size=(4, n), dtype=np.uint64) * np.uint64(2) + r.integers(0, 2, size=(4, n), dtype=np.uint64)
    k = r.integers(0, 2**63, size=(2, n), dtype=np.uint64)
    out = philox.philox4x64_10_np(c[0], c[1], c[2], c[3], k[0], k[1])
    for j in range(n):
        ref = philox.philox4x64_10([int(c[w, j]) for w in range(4)], (int(k[0, j]), int(k[1, j])))
        assert tuple(int(out[w][j]) for w in range(4)) == ref


def test_uniform_token_is_top_bits_and_uniform():
    V = 512
    n = 1 << 20
    i = np.arange(n, dtype=np.uint64)
    u = philox.uniform_tokens_np(1000, 3, 0, 0, i, V)
    # for V a power of two the draw is the top log2(V) bits of word 0
    w0 = philox.philox4x64_10_np(i, np.full(n, 3, np.uint64), np.zeros(n, np.uint64),
                                 np.zeros(n, np.uint64), np.full(n, 1000, np.uint64),
                                 np.zeros(n, np.uint64))[0]
    assert np.array_equal(u, (w0 >> np.uint64(55)).astype(np.int64))
    assert u.min() >= 0 and u.max() < V
    counts = np.bincount(u, minlength=V)
    chi2 = ((counts - n / V) ** 2 / (n / V)).sum()
    assert scipy.stats.chi2.sf(chi2, V - 1) > 1e-4
    # non-power-of-two V stays in range
    u7 = philox.uniform_tokens_np(5, 1, 2, 3, np.arange(10000, dtype=np.uint64), 7)
    assert u7.min() == 0 and u7.max() == 6
    # scalar and vectorised draws agree, and the key (seed, t, b, k, i) decides
    for j in (0, 1, 77, 4095):
        assert philox.uniform_token(1000, 3, 0, 0, j, V) == u[j]
    assert philox.uniform_token(1, 2, 3, 4, 5, V) == philox.uniform_token(1, 2, 3, 4, 5, V)
    draws = {philox.uniform_token(1, t, b, k, 5, 2**18) for t in range(3) for b in range(3) for k in range(3)}
    assert len(draws) > 20


# ---- storage rounding -------------------------------------------------------------

def test_round_bf16_cases_and_torch():
    r = numerics.round_bf16
    one = 1.0
    assert r(one + 2**-8) == 1.0                 # halfway, ties to even (down)
    assert r(one + 3 * 2**-8) == 1.0 + 2**-6     # halfway, ties to even (up)
    assert r(one + 2**-8 + 2**-20) == 1.0 + 2**-7
    assert r(-(one + 2**-8 + 2**-20)) == -(1.0 + 2**-7)
    assert r(255.5) == 256.0 and r(0.0) == 0.0
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 10
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(r(x.astype(np.float64)), ref)


# ---- projections -------------------------------------------------------------------

def test_linear_matches_torch():
    X = rng0.standard_normal((7, 12))
    W = rng0.standard_normal((5, 12))
    ref = torch.nn.functional.linear(torch.from_numpy(X), torch.from_numpy(W)).numpy()
    out = step.linear(X, W, "f32")
    assert np.allclose(out, ref.astype(np.float32), rtol=0, atol=0)


# ---- attention ------------------------------------------------------------------------

def _attn_inputs(B=2, C=6, L=5, Hq=4, Hkv=2, dh=8, cap=None, seed=0, scale=1.0):
    r = np.random.default_rng(seed)
    cap = cap or L + 3
    Q = r.standard_normal((B, C, Hq, dh)) * scale
    Kc = r.standard_normal((B, Hkv, cap, dh))
    Vc = r.standard_normal((B, Hkv, cap, dh))
    Kn = r.standard_normal((B, C, Hkv, dh))
    Vn = r.standard_normal((B, C, Hkv, dh))
    return Q, Kc, Vc, Kn, Vn


def _sdpa(Q, K, V, causal, mask=None):
    # Q [C, H, dh] -> torch [1, H, C, dh]
    q = torch.from_numpy(Q).permute(1, 0, 2)[None]
    k = torch.from_numpy(K).permute(1, 0, 2)[None]
    v = torch.from_numpy(V).permute(1, 0, 2)[None]
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask, is_causal=causal)
    return o[0].permute(1, 0, 2).numpy()


@pytest.mark.parametrize("G", [1, 2, 4])
def test_attention_empty_cache_is_full_attention(G):
    Hkv = 2
    Q, Kc, Vc, Kn, Vn = _attn_inputs(L=0, Hq=Hkv * G, Hkv=Hkv, seed=G, scale=3.0)
    O, lse = step.attention(Q, Kc, Vc, Kn, Vn, 0, causal=False)
    Oc, _ = step.attention(Q, Kc, Vc, Kn, Vn, 0, causal=True)
    for b in range(Q.shape[0]):
        K = np.repeat(Kn[b], G, axis=1)
        Vv = np.repeat(Vn[b], G, axis=1)
        assert np.allclose(O[b], _sdpa(Q[b], K, Vv, False), atol=1e-12)
        assert np.allclose(Oc[b], _sdpa(Q[b], K, Vv, True), atol=1e-12)
        # lse: natural log-sum-exp of the scaled scores
        s = np.einsum("chd,khd->hck", Q[b], K) / math.sqrt(Q.shape[3])
        assert np.allclose(lse[b], scipy.special.logsumexp(s, axis=2).T, atol=1e-12)
    # the two masks agree on the last canvas row only (it sees every key)
    assert np.allclose(O[:, -1], Oc[:, -1], atol=1e-12)
    assert not np.allclose(O[:, 0], Oc[:, 0])


def test_attention_with_cache_matches_masked_sdpa():
    B, C, L, G = 2, 6, 5, 2
    Q, Kc, Vc, Kn, Vn = _attn_inputs(B=B, C=C, L=L, Hq=4, Hkv=2, seed=9, scale=2.0)
    for causal in (False, True):
        O, _ = step.attention(Q, Kc, Vc, Kn, Vn, L, causal=causal)
        for b in range(B):
            K = np.repeat(np.concatenate([Kc[b, :, :L].transpose(1, 0, 2), Kn[b]], 0), G, axis=1)
            Vv = np.repeat(np.concatenate([Vc[b, :, :L].transpose(1, 0, 2), Vn[b]], 0), G, axis=1)
            mask = None
            if causal:   # query i keeps key j iff j <= L + i (diagonal offset by the cache)
                mask = torch.from_numpy(np.arange(L + C)[None, :] <= (L + np.arange(C))[:, None])
            assert np.allclose(O[b], _sdpa(Q[b], K, Vv, False, mask), atol=1e-12)


def test_attention_special_cases():
    Q, Kc, Vc, Kn, Vn = _attn_inputs(B=1, C=1, L=0, Hq=2, Hkv=1, seed=3)
    O, _ = step.attention(Q, Kc, Vc, Kn, Vn, 0, causal=False)       # one key -> O = v
    assert np.allclose(O[0, 0, 0], Vn[0, 0, 0]) and np.allclose(O[0, 0, 1], Vn[0, 0, 0])
    Q, Kc, Vc, Kn, Vn = _attn_inputs(B=1, C=4, L=3, Hq=2, Hkv=1, seed=4)
    Kc[:] = 0.7
    Kn[:] = 0.7                                                       # identical keys -> mean(v)
    O, _ = step.attention(Q, Kc, Vc, Kn, Vn, 3, causal=False)
    mean_v = np.concatenate([Vc[0, 0, :3], Vn[0, :, 0]]).mean(0)
    assert np.allclose(O[0, :, 0], mean_v[None], atol=1e-12)


def test_attention_permutations():
    B, C, L = 1, 7, 9
    Q, Kc, Vc, Kn, Vn = _attn_inputs(B=B, C=C, L=L, Hq=4, Hkv=2, seed=5, scale=2.0)
    O, _ = step.attention(Q, Kc, Vc, Kn, Vn, L, causal=False)
    pc = np.random.default_rng(1).permutation(L)                     # cache order is irrelevant
    Kc2, Vc2 = Kc.copy(), Vc.copy()
    Kc2[:, :, :L] = Kc[:, :, pc]
    Vc2[:, :, :L] = Vc[:, :, pc]
    O2, _ = step.attention(Q, Kc2, Vc2, Kn, Vn, L, causal=False)
    assert np.allclose(O, O2, atol=1e-12)
    pq = np.random.default_rng(2).permutation(C)                     # no positions: equivariant
    O3, _ = step.attention(Q[:, pq], Kc, Vc, Kn[:, pq], Vn[:, pq], L, causal=False)
    assert np.allclose(O3, O[:, pq], atol=1e-12)


@pytest.mark.parametrize("L,Hq,Hkv,causal", [(0, 2, 2, False), (0, 4, 1, True), (5, 3, 1, False),
                                             (5, 4, 2, True), (5, 4, 4, False), (0, 4, 2, False)])
def test_attention_row_matches_attention(L, Hq, Hkv, causal):
    """attention_row (one query against its KV head) equals the batched
    attention on every canvas, head and position, with the lse."""
    B, C = 2, 6
    Q, Kc, Vc, Kn, Vn = _attn_inputs(B=B, C=C, L=L, Hq=Hq, Hkv=Hkv, seed=20 + L + Hq, scale=1.5)
    O, lse = step.attention(Q, Kc, Vc, Kn, Vn, L, causal=causal)
    G = Hq // Hkv
    for b in range(B):
        for h in range(Hq):
            for i in range(C):
                o, l = step.attention_row(Q[b, i, h], b, h // G, i, Kc, Vc, Kn, Vn, L, causal)
                assert np.allclose(o, O[b, i, h], atol=1e-13, rtol=0)
                assert abs(l - lse[b, i, h]) < 1e-12


# ---- vocabulary head, confidence, self-conditioning -------------------------------------------

def _emb(V=300, d=16, seed=0):
    return np.random.default_rng(seed).standard_normal((V, d)) * 0.3


def test_vocab_matches_full_softmax_and_logsumexp():
    E = _emb()
    Z = np.random.default_rng(1).standard_normal((9, 16)) * 3
    m, a, lse, c, S, gap = step.vocab_selfcond(Z, E, rows=4)            # several row blocks
    lg = Z @ E.T
    P = scipy.special.softmax(lg, axis=1)
    assert np.array_equal(a, lg.argmax(1))
    assert np.allclose(m, lg.max(1), atol=0)
    assert np.allclose(lse, scipy.special.logsumexp(lg, axis=1), atol=1e-12)
    assert np.allclose(c, P.max(1), atol=1e-14)
    assert np.allclose(S, P @ E, atol=1e-13)
    assert np.all((c >= 1.0 / E.shape[0]) & (c <= 1.0))
    # one row at a time gives the same rows
    for r in (0, 4, 8):
        u = step.vocab_selfcond(Z[r:r + 1], E)
        for x, w in zip(u, (m, a, lse, c, S, gap)):
            assert np.allclose(x[0], w[r], atol=1e-12)


def _fsum_logits(Z, E):
    """Logits by scalar loops with exactly rounded sums (math.fsum)."""
    return [[math.fsum(z * e for z, e in zip(zr, er)) for er in E] for zr in Z]


def test_vocab_top2_gap_brute_force():
    E = _emb(V=97, d=8, seed=5)
    Z = np.random.default_rng(6).standard_normal((7, 8)) * 2
    *_, gap = step.vocab_selfcond(Z, E, rows=3)
    for r, row in enumerate(_fsum_logits(Z.tolist(), E.tolist())):
        top = sorted(row, reverse=True)
        assert abs(gap[r] - (top[0] - top[1])) < 1e-12
    # a planted near-tie: two ids whose logits differ by exactly 2^-20 in every row
    E2 = np.zeros((6, 2))
    E2[:, 0] = [0.1, 0.5, 0.25, 0.5 - 2.0 ** -20, -1.0, 0.0]
    m, a, lse, c, S, gap2 = step.vocab_selfcond(np.array([[1.0, 0.0], [1.0, 3.0]]), E2)
    assert np.array_equal(a, [1, 1]) and np.all(gap2 == 2.0 ** -20)
    # exact ties: the gap is 0 and the lowest id wins
    E3 = np.array([[0.0], [2.0], [1.0], [2.0]])
    m, a, *_, gap3 = step.vocab_selfcond(np.array([[1.0]]), E3)
    assert a[0] == 1 and gap3[0] == 0.0
    # a single id has no runner-up
    *_, gap4 = step.vocab_selfcond(np.array([[1.0, 2.0]]), np.array([[0.5, 0.5]]))
    assert gap4[0] == np.inf


def test_vocab_rows_sum_to_one_via_ones_column():
    E = _emb(V=257)
    E[:, 5] = 1.0                                                       # S[:,5] = sum_v P_v = 1
    Z = np.random.default_rng(2).standard_normal((6, 16))
    S = step.vocab_selfcond(Z, E, rows=4)[4]
    assert np.allclose(S[:, 5], 1.0, atol=1e-14)


def test_vocab_one_hot_is_embedding_lookup():
    E = np.round(_emb(V=512, d=32) * 64) / 64
    y = np.array([3, 100, 511, 0])
    Z = 1000.0 * E[y]
    m, a, lse, c, S, gap = step.vocab_selfcond(Z, E, dtype="bf16", rows=3)
    assert np.array_equal(a, y)
    assert np.all(c == 1.0)
    assert np.array_equal(S, numerics.round_bf16(E[y]))


def test_vocab_zero_input_closed_form():
    E = _emb(V=1024, d=8)
    Z = np.zeros((3, 8))
    m, a, lse, c, S, gap = step.vocab_selfcond(Z, E, rows=2)
    assert np.all(a == 0) and np.all(m == 0)                           # ties -> lowest index
    assert np.all(gap == 0)
    assert np.allclose(c, 1.0 / 1024, rtol=1e-15)
    assert np.allclose(lse, math.log(1024), rtol=1e-15)
    assert np.allclose(S, E.mean(0)[None], atol=1e-15)


def test_vocab_ties_take_lowest_index():
    E = np.zeros((10, 2))
    E[:, 0] = [0, 1, 3, 2, 3, 1, 3, 0, 0, 0]
    m, a, *_ = step.vocab_selfcond(np.array([[1.0, 0.0]]), E)
    assert a[0] == 2 and m[0] == 3.0


# ---- renoise -------------------------------------------------------------------------------

def test_renoise_keeps_confident_and_draws_the_rest():
    B, C, V = 2, 8, 64
    a = np.arange(B * C) % V
    c = np.linspace(0.0, 1.0, B * C)
    tau = 0.5
    x, mask = step.renoise(a, c, tau, seed=7, t=3, block=1, B=B, C=C, V=V)
    keep = c >= np.float32(tau)
    assert np.array_equal(mask, (~keep).astype(np.uint8))
    assert np.array_equal(x[keep], a[keep])
    for r in np.nonzero(~keep)[0]:
        b, i = divmod(int(r), C)
        assert x[r] == philox.uniform_token(7, 3, b, 1, i, V)
    x0 = step.init_canvas(7, 1, B, C, V)
    assert x0.shape == (B, C) and x0[1, 2] == philox.uniform_token(7, 0, 1, 1, 2, V)
    # tau is compared as the float32 the kernel receives
    x, mask = step.renoise(np.array([1]), np.array([float(np.float32(0.9))]), 0.9, 1, 1, 0, 1, 1, 8)
    assert mask[0] == 0


# ---- the whole step against the brute force ----------------------------------------------------

def _tolist(a):
    return np.asarray(a).tolist()


def _compare_step(ref, br, rel=1e-12):
    for k in ("X", "Q", "Kn", "Vn", "O", "Z", "S"):
        u = np.asarray(ref[k], np.float64).reshape(-1)
        w = np.asarray(br[k], np.float64).reshape(-1)
        assert np.allclose(u, w, rtol=rel, atol=rel * max(1.0, np.abs(u).max())), k
    for k in ("m", "lse", "c"):
        assert np.allclose(np.asarray(ref[k]), np.asarray(br[k]), rtol=rel, atol=rel), k
    assert np.array_equal(np.asarray(ref["a"]), np.asarray(br["a"]))
    assert np.array_equal(np.asarray(ref["x_new"]).reshape(-1), np.asarray(br["x_new"]))
    assert np.array_equal(np.asarray(ref["mask"]).reshape(-1), np.asarray(br["mask"]))


def test_step_matches_brute_force_tiny_workload():
    cfg = config_by_name("tiny_c16_L32_d64_V512_f32")
    p = gen_problem(cfg)
    f = lambda a: from_storage(a, cfg.dtype).astype(np.float64)
    E, H, Kc, Vc = f(p.E), f(p.H[0]), f(p.Kc), f(p.Vc)
    W = {k: f(v) for k, v in p.W.items()}
    x = step.init_canvas(cfg.seed, 0, cfg.B, cfg.C, cfg.V)
    S = None
    kept = []
    for s in range(2):
        ref = step.denoise_step(H, E, W, Kc, Vc, cfg.L, x, S, cfg.tau[0], cfg.seed, s + 1, 0, cfg.dtype)
        br = brute.step(_tolist(H), _tolist(E), {k: _tolist(v) for k, v in W.items()},
                        _tolist(Kc), _tolist(Vc), cfg.L, _tolist(x),
                        None if S is None else _tolist(S), cfg.tau[0], cfg.seed, s + 1, 0, cfg.dtype)
        _compare_step(ref, br)
        kept.append(1 - ref["mask"].mean())
        x, S = ref["x_new"], ref["S"]
    # the calibrated signal gives a mix of kept and renoised positions
    assert 0.0 < kept[0] < 1.0


@pytest.mark.parametrize("L,Hq,Hkv,V,dtype,seed", [
    (0, 2, 2, 7, "f32", 1), (5, 4, 2, 64, "bf16", 2), (3, 4, 1, 33, "f32", 3), (8, 2, 1, 16, "bf16", 4)])
def test_step_matches_brute_force_random_shapes(L, Hq, Hkv, V, dtype, seed):
    r = np.random.default_rng(seed)
    B, C, d, dh = 2, 5, 8, 4
    q = (lambda a: numerics.round_store(a, dtype))
    E = q(r.standard_normal((V, d)))
    W = {"Wq": q(r.standard_normal((Hq * dh, d)) * 0.5), "Wk": q(r.standard_normal((Hkv * dh, d)) * 0.5),
         "Wv": q(r.standard_normal((Hkv * dh, d)) * 0.5), "Wo": q(r.standard_normal((d, Hq * dh)) * 0.5)}
    H = q(r.standard_normal((B, C, d)))
    Kc = q(r.standard_normal((B, Hkv, L + 2, dh)))
    Vc = q(r.standard_normal((B, Hkv, L + 2, dh)))
    x = r.integers(0, V, size=(B, C))
    S = q(r.standard_normal((B, C, d)) * 0.1)
    ref = step.denoise_step(H, E, W, Kc, Vc, L, x, S, 0.3, 99, 2, 1, dtype)
    br = brute.step(_tolist(H), _tolist(E), {k: _tolist(v) for k, v in W.items()}, _tolist(Kc),
                    _tolist(Vc), L, _tolist(x), _tolist(S), 0.3, 99, 2, 1, dtype)
    _compare_step(ref, br, rel=1e-12 if dtype == "f32" else 1e-9)


def test_prefill_append_writes_cache_rows_and_is_causal():
    r = np.random.default_rng(11)
    B, C, d, dh, Hq, Hkv, V, L = 2, 4, 8, 4, 2, 1, 16, 3
    E = r.standard_normal((V, d))
    W = {"Wq": r.standard_normal((Hq * dh, d)), "Wk": r.standard_normal((Hkv * dh, d)),
         "Wv": r.standard_normal((Hkv * dh, d)), "Wo": r.standard_normal((d, Hq * dh))}
    H = r.standard_normal((B, C, d))
    Kc = r.standard_normal((B, Hkv, L + C, dh))
    Vc = r.standard_normal((B, Hkv, L + C, dh))
    xf = r.integers(0, V, (B, C))
    K2, V2, O, _ = step.prefill_append(H, E, W, Kc, Vc, L, xf, "f32")
    X = numerics.round_store((H + E[xf]).reshape(B * C, d), "f32")
    Kn = numerics.round_store(X @ W["Wk"].T, "f32").reshape(B, C, Hkv, dh)
    assert np.array_equal(K2[:, :, :L], Kc[:, :, :L])                # old rows untouched
    assert np.array_equal(K2[:, :, L:], Kn.transpose(0, 2, 1, 3))    # new rows appended
    # the last query sees every key: equals the bidirectional result for that row
    Q = numerics.round_store(X @ W["Wq"].T, "f32").reshape(B, C, Hq, dh)
    Vn = numerics.round_store(X @ W["Wv"].T, "f32").reshape(B, C, Hkv, dh)
    Ob, _ = step.attention(Q, Kc, Vc, Kn, Vn, L, causal=False, dtype="f32")
    assert np.allclose(O[:, -1], Ob[:, -1]) and not np.allclose(O[:, 0], Ob[:, 0])
