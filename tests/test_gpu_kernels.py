"""Parity of each C-ABI entry point with the CPU oracle, element by element, at
sizes that span several tiles with ragged tails, plus the special cases the
method has (one-hot probabilities, flat logits, empty cache, causal prefill)."""
import math

import numpy as np
import pytest
import torch

from oracle import numerics, philox, step
from tests.gpu_util import (ATOL, RELF, argmax_match, as_f64, close, dev, f64, need_gpu,
                            renoise_match, say, stored)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()
    import uniform_state_discrete_amd as dg
    dg.lib()
    yield


# ---- renoise / initial canvas ---------------------------------------------------------

@pytest.mark.parametrize("B,C,V", [(1, 16, 512), (8, 256, 262144), (3, 37, 7), (2, 100, 32768)])
def test_renoise_bit_exact(B, C, V):
    import uniform_state_discrete_amd as dg
    say(f"renoise B={B} C={C} V={V}")
    r = np.random.default_rng(B * 1000 + C)
    R = B * C
    a = r.integers(0, V, R).astype(np.int32)
    c = r.random(R).astype(np.float32)
    c[::7] = np.float32(0.9)                         # exactly tau: kept (strict <)
    c[1::11] = np.nextafter(np.float32(0.9), np.float32(0))   # just below: renoised
    tau, seed, t, blk = 0.9, 1002, 5, 3
    out = torch.empty(R, dtype=torch.int32, device="cuda")
    mask = torch.empty(R, dtype=torch.uint8, device="cuda")
    dg.dg_renoise(R, C, V, dev(a), dev(c), tau, seed, t, blk, out, mask)
    torch.cuda.synchronize()
    ref_x, ref_m = step.renoise(a, c.astype(np.float64), tau, seed, t, blk, B, C, V)
    assert np.array_equal(mask.cpu().numpy(), ref_m)
    assert np.array_equal(out.cpu().numpy(), ref_x)
    # the initial canvas is draw 0
    dg.dg_init_canvas(R, C, V, seed, blk, out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().reshape(B, C), step.init_canvas(seed, blk, B, C, V))


# ---- vocabulary head / confidence / self-conditioning ------------------------------------

def _vocab_inputs(R, d, V, dtype, seed, signal=None):
    r = np.random.default_rng(seed)
    if signal is None:   # planted-row amplitude that puts the median confidence near 1/2
        signal = (math.sqrt(d) - math.sqrt(d - 2 * math.log(V - 1))) / 0.02
    E = stored(r.standard_normal((V, d)).astype(np.float32) * 0.02, dtype)
    Ef = as_f64(E, dtype)
    y = r.integers(0, V, R)
    amp = signal * (1 + 0.2 * r.standard_normal(R))
    Z = amp[:, None] * Ef[y] / np.linalg.norm(Ef[y], axis=1, keepdims=True) + 0.5 * r.standard_normal((R, d))
    Z = stored(Z, dtype)
    return E, Z


def _run_vocab(R, d, V, E, Z, dtype):
    import uniform_state_discrete_amd as dg
    Ed, Zd = dev(E), dev(Z)
    m = torch.empty(R, dtype=torch.float32, device="cuda")
    c = torch.empty_like(m)
    lse = torch.empty_like(m)
    a = torch.empty(R, dtype=torch.int32, device="cuda")
    S = torch.empty((R, d), dtype=Zd.dtype, device="cuda")
    ws = dg.workspace(dg.dg_vocab_workspace_bytes(R, d, V, Zd.dtype))
    Et = dg.tiled_embedding(Ed)
    dg.dg_vocab_selfcond(R, d, V, Zd, Ed if Et is None else Et, m, a, c, lse, S, ws)
    torch.cuda.synchronize()
    return f64(m), a.cpu().numpy(), f64(c), f64(lse), f64(S)


@pytest.mark.parametrize("V,d", [(37, 64), (3000, 256), (16, 4096)])
def test_tiled_embedding_layout(V, d):
    """The tiled table holds, at element 8(16g + r) + e' of 1 KiB block
    (vb, c), entry (16 vb + r, 32 c + 8 g + e) of E (e' = e for even g,
    e ^ 4 for odd g), zero past V."""
    import uniform_state_discrete_amd as dg
    say(f"tiled embedding V={V} d={d}")
    r = np.random.default_rng(V + d)
    E = stored(r.standard_normal((V, d)).astype(np.float32), "bf16")
    Et = dg.tiled_embedding(dev(E))
    torch.cuda.synchronize()
    got = Et.view(torch.int16).cpu().numpy().view(np.uint16)
    Vp = -(-V // 16) * 16
    ref = np.zeros((Vp, d), dtype=np.uint16)
    ref[:V] = E
    # blocks [vb][c][g][r][e'] <- ref[16 vb + r][32 c + 8 g + e]
    blk = ref.reshape(Vp // 16, 16, d // 32, 4, 8).transpose(0, 2, 3, 1, 4).copy()
    blk[:, :, 1::2] = np.concatenate([blk[:, :, 1::2, :, 4:], blk[:, :, 1::2, :, :4]], axis=-1)
    ref = blk.reshape(-1)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("R,d,V,dtype", [
    (16, 64, 512, "f32"), (33, 100, 777, "f32"),          # fp32 path
    (40, 256, 1000, "bf16"),                              # 32-row tiles: ragged rows and ids
    (70, 128, 4133, "bf16"),
    (256, 2048, 32768, "bf16"),                           # the 32k-vocab step's shape, every row
    (100, 2048, 5000, "bf16"),                            # CU pairs: ragged 64-row block
    (1, 2048, 200, "bf16"),                               # splits of 2, 1 and 0 tiles
    (130, 2048, 7001, "bf16"),                            # 3 row blocks x 40 splits, ragged ids
    (300, 2048, 9001, "bf16"),                            # 5 row blocks (the marked layout), ragged rows and ids
    (37, 4096, 3000, "bf16"),                             # 16-row tiles (d = 4096)
])
def test_vocab_matches_oracle(R, d, V, dtype):
    say(f"vocab R={R} d={d} V={V} {dtype}")
    E, Z = _vocab_inputs(R, d, V, dtype, seed=R + d + V)
    m, a, c, lse, S = _run_vocab(R, d, V, E, Z, dtype)
    Ef, Zf = as_f64(E, dtype), as_f64(Z, dtype)
    rm, ra, rlse, rc, rS, gap = step.vocab_selfcond(Zf, Ef, dtype)
    tol, rel = ATOL[dtype], RELF[dtype]
    close("m", m, rm, tol)
    close("lse", lse, rlse, tol)
    close("c", c, rc, tol)
    close("S", S, rS, tol, rel)
    argmax_match("argmax", a, ra, gap, rm)
    if R >= 16:
        assert 0.1 < rc.mean() < 0.95   # the inputs exercise a non-trivial softmax


@pytest.mark.parametrize("d,V,rows", [(2048, 262144, 256), (4096, 262144, 256), (2048, 262144, 2048),
                                      (2048, 262144, 8), (2048, 262144, 1)])  # one 64-row CU-pair block
def test_vocab_full_vocab_every_row(d, V, rows):
    """The full 262144-id table at the workloads' widths, every row against
    the oracle (which forms each row's whole logits row)."""
    say(f"vocab full-size d={d} V={V} R={rows} (every row)")
    E, Z = _vocab_inputs(rows, d, V, "bf16", seed=d + rows)
    m, a, c, lse, S = _run_vocab(rows, d, V, E, Z, "bf16")
    Ef, Zf = as_f64(E, "bf16"), as_f64(Z, "bf16")
    del E
    rm, ra, rlse, rc, rS, gap = step.vocab_selfcond(Zf, Ef, "bf16")
    close("m", m, rm, ATOL["bf16"])
    close("lse", lse, rlse, ATOL["bf16"])
    close("c", c, rc, ATOL["bf16"])
    close("S", S, rS, ATOL["bf16"], RELF["bf16"])
    argmax_match("argmax", a, ra, gap, rm)
    assert np.all((c >= 1.0 / V * 0.999) & (c <= 1.0 + 1e-6)) and np.all(lse >= m - 1e-4)


@pytest.mark.parametrize("R,d,V", [(100, 2048, 5000), (1, 2048, 200), (130, 2048, 7001), (37, 4096, 3000),
                                   (256, 2048, 262144), (256, 4096, 262144)])
def test_vocab_group_solo_equals_paired(R, d, V):
    """The CU-group vocabulary head computing solo (each member computes the
    other members' partial logits itself) gives the same bits as the paired
    run: with the handshake bound 0 every group runs solo, with a bound of 1
    some groups pair and some do not.  The small shapes are also checked
    against the oracle."""
    import uniform_state_discrete_amd as dg
    say(f"vocab solo vs paired R={R} d={d} V={V}")
    E, Z = _vocab_inputs(R, d, V, "bf16", seed=R + d + V + 1)
    ref = _run_vocab(R, d, V, E, Z, "bf16")
    try:
        for polls in (0, 1):
            dg.dg_test_set_group_wait(polls)
            got = _run_vocab(R, d, V, E, Z, "bf16")
            for name, u, w in zip(("m", "a", "c", "lse", "S"), got, ref):
                assert np.array_equal(u, w), f"bound {polls}: {name} differs from the paired run"
    finally:
        dg.dg_test_set_group_wait(-1)
    if V <= 8000:
        Ef, Zf = as_f64(E, "bf16"), as_f64(Z, "bf16")
        rm, ra, rlse, rc, rS, gap = step.vocab_selfcond(Zf, Ef, "bf16")
        close("m", got[0], rm, ATOL["bf16"])
        close("c", got[2], rc, ATOL["bf16"])
        close("S", got[4], rS, ATOL["bf16"], RELF["bf16"])
        argmax_match("argmax", got[1], ra, gap, rm)


def test_vocab_group_beside_a_concurrent_kernel():
    """A long matrix product on another stream holds CUs while the vocabulary
    head starts, so the members of a CU group are dispatched as CUs free up
    and may wait for each other; whatever the handshake then decides (on this
    box the members arrived within its bound: paired), the outputs are the
    bits of an undisturbed run.  The number of members that ran solo is read
    from the exchange header (word 16) and reported."""
    import uniform_state_discrete_amd as dg
    R, d, V = 256, 2048, 262144
    say("vocab beside a concurrent kernel")
    E, Z = _vocab_inputs(R, d, V, "bf16", seed=77)
    Ed, Zd = dev(E), dev(Z)
    Et = dg.tiled_embedding(Ed)
    del Ed
    nbytes = dg.dg_vocab_workspace_bytes(R, d, V, Zd.dtype)
    ws = dg.workspace(nbytes)

    def run(stream):
        out = [torch.empty(R, device="cuda") for _ in range(3)]
        a = torch.empty(R, dtype=torch.int32, device="cuda")
        S = torch.empty((R, d), dtype=torch.bfloat16, device="cuda")
        dg.dg_vocab_selfcond(R, d, V, Zd, Et, out[0], a, out[1], out[2], S, ws, stream)
        return out + [a, S]

    ref = run(torch.cuda.current_stream())
    torch.cuda.synchronize()
    # exchange header: after the partials of S (2 nsplit R d fp32) and the
    # per-row split statistics (nsplit R x 16 bytes), 256-byte aligned; 32
    # splits of 8192 ids at these sizes
    nsplit = 32
    hdr = (2 * nsplit * R * d * 4 + nsplit * R * 16 + 255) // 256 * 256
    side = torch.cuda.Stream()
    g = torch.Generator(device="cuda").manual_seed(5)
    A = torch.randn(8192, 8192, generator=g, device="cuda").to(torch.bfloat16)
    solo = []
    for rep in range(4):
        torch.cuda.synchronize()
        with torch.cuda.stream(side):
            for _ in range(2):
                C = A @ A                              # holds CUs for milliseconds
        got = run(torch.cuda.current_stream())      # not ordered after the side stream
        torch.cuda.synchronize()
        solo.append(int(ws[hdr + 64:hdr + 68].view(torch.int32).item()))
        for name, u, v in zip(("max_logit", "conf", "lse", "argmax", "S"), got, ref):
            assert torch.equal(u, v), f"run {rep}: {name} differs from the undisturbed run"
        del C
    say(f"members that ran solo per run: {solo} (of 256)")


@pytest.mark.parametrize("d,dtype", [(256, "bf16"), (2048, "bf16"), (4096, "bf16"), (64, "f32")])
def test_vocab_one_hot_is_exact_embedding_lookup(d, dtype):
    V, R = 3000, 40
    r = np.random.default_rng(d)
    E = stored(np.round(r.standard_normal((V, d)) * 0.02 * 64) / 64, dtype)
    Ef = as_f64(E, dtype)
    y = r.integers(0, V, R)
    y[:4] = [0, V - 1, 1234, 31]
    # Z = alpha * E[y] with alpha a power of two (exact) large enough that every
    # other logit sits more than 110 below the planted one: exp underflows to 0
    lg = Ef[y] @ Ef.T
    own = lg[np.arange(R), y]
    lg[np.arange(R), y] = -np.inf
    margin = float((own - lg.max(1)).min())
    assert margin > 0
    alpha = 2.0 ** math.ceil(math.log2(110.0 / margin))
    Z = stored(alpha * Ef[y], dtype)
    assert np.array_equal(as_f64(Z, dtype), alpha * Ef[y])
    m, a, c, lse, S = _run_vocab(R, d, V, E, Z, dtype)
    assert np.array_equal(a, y)
    assert np.all(c == 1.0)
    assert np.array_equal(S, Ef[y])              # bit-exact lookup


def test_vocab_flat_logits_closed_form():
    V, d, R = 32768, 256, 33
    r = np.random.default_rng(0)
    E = stored(r.standard_normal((V, d)) * 0.02, "bf16")
    Z = stored(np.zeros((R, d)), "bf16")
    m, a, c, lse, S = _run_vocab(R, d, V, E, Z, "bf16")
    assert np.all(a == 0) and np.all(m == 0)
    assert np.all(c == np.float32(1.0 / V))     # exact: 1/V, V a power of two
    close("lse", lse, np.full(R, math.log(V)), 1e-5)
    close("S=mean(E)", S, np.repeat(as_f64(E, "bf16").mean(0)[None], R, 0), 2e-3)


def test_vocab_probabilities_sum_to_one():
    V, d, R = 5000, 512, 64
    E, Z = _vocab_inputs(R, d, V, "bf16", seed=3)
    Ef = as_f64(E, "bf16")
    Ef[:, 7] = 1.0
    E = stored(Ef, "bf16")
    *_, S = _run_vocab(R, d, V, E, Z, "bf16")
    close("sum_v P", S[:, 7], np.ones(R), 8e-3)


# ---- attention ----------------------------------------------------------------------------

def _attn_inputs(B, C, L, cap, Hq, Hkv, dh, dtype, seed, qscale=1.0):
    r = np.random.default_rng(seed)
    q = stored(r.standard_normal((B, C, Hq, dh)) * qscale, dtype)
    Kc = stored(r.standard_normal((B, Hkv, cap, dh)), dtype)
    Vc = stored(r.standard_normal((B, Hkv, cap, dh)), dtype)
    Kn = stored(r.standard_normal((B, C, Hkv, dh)), dtype)
    Vn = stored(r.standard_normal((B, C, Hkv, dh)), dtype)
    return q, Kc, Vc, Kn, Vn


def _run_attn(B, C, L, cap, Hq, Hkv, dh, dtype, arrs, causal):
    import uniform_state_discrete_amd as dg
    q, Kc, Vc, Kn, Vn = (dev(x) for x in arrs)
    dims = dg.make_dims(B, C, L, cap, 64, Hq, Hkv, dh, 1, dg.DG_BF16 if dtype == "bf16" else dg.DG_F32)
    out = torch.empty((B, C, Hq, dh), dtype=q.dtype, device="cuda")
    lse = torch.empty((B, C, Hq), dtype=torch.float32, device="cuda")
    ws = dg.workspace(dg.dg_attn_workspace_bytes(dims))
    dg.dg_attn_bidir(dims, q, Kc, Vc, Kn, Vn, out, lse, causal, ws)
    torch.cuda.synchronize()
    return f64(out), f64(lse)


@pytest.mark.parametrize("B,C,L,Hq,Hkv,dh,dtype,qscale", [
    (1, 16, 32, 2, 1, 32, "f32", 1.0),         # the fp32 workload's shape
    (2, 37, 100, 4, 2, 64, "bf16", 1.0),       # ragged canvas and keys, GQA 2
    (2, 37, 100, 4, 2, 64, "bf16", 3.0),       # sharp scores (std about 3)
    (1, 50, 0, 8, 2, 128, "bf16", 3.0),        # empty cache, GQA 4
    (3, 70, 333, 4, 4, 128, "bf16", 2.0),      # MHA
    (1, 256, 1024, 16, 8, 128, "bf16", 1.0),   # the 32k-vocab step's attention shape
    (1, 300, 0, 8, 2, 128, "bf16", 2.0),       # 10 row blocks x 3 splits: causal blocks skip splits
    (2, 200, 150, 4, 2, 64, "bf16", 1.0),      # causal key limit inside a split, non-empty cache
    (1, 40, 20, 2, 1, 32, "f32", 1.0),         # fp32 rows stop at their own key limit
    # at most 64 packed rows (one row block, half its waves idle)
    (2, 13, 100, 4, 2, 64, "bf16", 1.0),       # 26 rows, one split of two tiles
    (1, 16, 2000, 8, 2, 128, "bf16", 2.0),     # 64 rows, 16 splits, ragged last split
    (3, 5, 700, 6, 2, 128, "bf16", 1.0),       # GQA 3, ragged last split
    (1, 20, 40, 2, 1, 64, "bf16", 1.0),        # one tile, no split
    # causal, GQA 3: row blocks 0-1 fit one split (written directly), row
    # block 2 is split; position 85 has rows in both kinds of row block
    (1, 100, 40, 6, 2, 64, "bf16", 1.0),
    # caches of whole 64-key tiles: the three-tile ring when not causal
    (2, 37, 128, 4, 2, 64, "bf16", 1.0),       # two cache tiles, then a ragged canvas tile
    (1, 16, 2048, 8, 2, 128, "bf16", 2.0),     # 17 splits of two tiles (many-splits combine)
    (3, 100, 192, 6, 2, 64, "bf16", 1.0),      # a split that runs from cache tiles into canvas tiles
])
@pytest.mark.parametrize("causal", [0, 1])
def test_attention_matches_oracle(B, C, L, Hq, Hkv, dh, dtype, qscale, causal):
    say(f"attention B={B} C={C} L={L} Hq={Hq} Hkv={Hkv} dh={dh} {dtype} q*{qscale} causal={causal}")
    cap = L + 5
    arrs = _attn_inputs(B, C, L, cap, Hq, Hkv, dh, dtype, seed=B + C + L + dh, qscale=qscale)
    O, lse = _run_attn(B, C, L, cap, Hq, Hkv, dh, dtype, arrs, causal)
    q, Kc, Vc, Kn, Vn = (as_f64(x, dtype) for x in arrs)
    rO, rlse = step.attention(q, Kc, Vc, Kn, Vn, L, causal=bool(causal), dtype=dtype)
    close("O", O, rO, ATOL[dtype], RELF[dtype])
    close("lse", lse, rlse, ATOL[dtype])


def test_attention_long_cache_every_row():
    """The 32k-token cache, 32/8-head shape (K/V ~ N(0,1)), every row."""
    B, C, L, Hq, Hkv, dh = 1, 256, 32768, 32, 8, 128
    say("attention long cache, every row")
    arrs = _attn_inputs(B, C, L, L, Hq, Hkv, dh, "bf16", seed=7, qscale=1.0)
    O, lse = _run_attn(B, C, L, L, Hq, Hkv, dh, "bf16", arrs, 0)
    q, Kc, Vc, Kn, Vn = (as_f64(x, "bf16") for x in arrs)
    rO, rlse = step.attention(q, Kc, Vc, Kn, Vn, L, causal=False, dtype="bf16")
    close("O", O, rO, ATOL["bf16"], RELF["bf16"])
    close("lse", lse, rlse, ATOL["bf16"])
    # a few rows also through the one-query form
    G = Hq // Hkv
    for (i, h) in [(0, 0), (255, 17), (128, 8)]:
        ro, rl = step.attention_row(q[0, i, h], 0, h // G, i, Kc, Vc, Kn, Vn, L, False)
        close(f"O[{i},{h}] one query", O[0, i, h], numerics.round_bf16(ro), ATOL["bf16"])
