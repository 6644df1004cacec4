"""The oracle against the hand-worked examples in tests/golden/worked_examples.txt:
exact fractions and logs derived on paper from the operations as the
explainer defines them ("DiffusionGemma explained": "Diffusione dello stato
uniforme", "Diffusione mascherata", "Autocondizionamento", "Architettura: il
prefill incrementale e il denoising").  CPU only."""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import philox, step

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.txt")
DRAW = object()  # "*": a renoised position (its Philox draw)


def _value(tok):
    if tok == "*":
        return DRAW
    if tok.startswith("ln(") and tok.endswith(")"):
        return math.log(float(Fraction(tok[3:-1])))
    return float(Fraction(tok))


def _parse(path):
    cases, cur = {}, None
    for raw in open(path, encoding="utf-8"):
        line = raw.split("#", 1)[0].strip()
        if not line:
            continue
        if line.startswith("[") and line.endswith("]"):
            cur = cases.setdefault(line[1:-1], {})
            continue
        key, rhs = (s.strip() for s in line.split("=", 1))
        rows = [[_value(t) for t in r.split()] for r in rhs.split(";")]
        cur[key] = rows
    return cases


CASES = _parse(GOLDEN)


def arr(case, key):
    """Rows of floats as an array: a single column or a single row -> 1-D, a
    single value -> a scalar."""
    a = np.array(CASES[case][key], np.float64)
    if a.shape[1] == 1:
        a = a[:, 0]
    elif a.shape[0] == 1:
        a = a[0]
    return a[0] if a.shape == (1,) else a


def test_every_section_is_present():
    assert set(CASES) == {"vocab", "renoise", "unmask", "assemble", "attention", "attention_scale"}


def test_vocab_worked_rows():
    Z, E = arr("vocab", "Z"), arr("vocab", "E")
    m, a, lse, c, S, gap = step.vocab_selfcond(Z, E)
    np.testing.assert_allclose(m, arr("vocab", "m"), rtol=1e-14, atol=1e-14)
    assert a.tolist() == arr("vocab", "a").astype(np.int64).tolist()
    np.testing.assert_allclose(lse, arr("vocab", "lse"), rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(c, arr("vocab", "c"), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(S, arr("vocab", "S"), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(gap, arr("vocab", "gap"), rtol=1e-14, atol=1e-14)


def test_renoise_worked_positions():
    g = CASES["renoise"]
    tau, seed, t, block, V = (g[k][0][0] for k in ("tau", "seed", "t", "block", "V"))
    seed, t, block, V = int(seed), int(t), int(block), int(V)
    a = np.array(g["a"][0], np.int64)
    c = np.array(g["c"][0], np.float64)
    x_new, mask = step.renoise(a, c, tau, seed, t, block, 1, len(a), V)
    assert mask.tolist() == [int(v) for v in g["mask"][0]]
    for i, want in enumerate(g["x_new"][0]):
        if want is DRAW:
            assert x_new[i] == philox.uniform_token(seed, t, 0, block, i, V)
        else:
            assert x_new[i] == int(want)


def test_unmask_worked_positions():
    g = CASES["unmask"]
    x_new, commit = step.unmask(np.array(g["a"][0], np.int64), np.array(g["c"][0]), g["tau"][0][0],
                                np.array(g["x"][0], np.int64), int(g["mask_id"][0][0]))
    assert x_new.tolist() == [int(v) for v in g["x_new"][0]]
    assert commit.tolist() == [int(v) for v in g["commit"][0]]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_assemble_worked_rows(dtype):
    E, H, S_prev = arr("assemble", "E"), arr("assemble", "H"), arr("assemble", "S_prev")
    x = arr("assemble", "x").astype(np.int64)
    X = step.assemble(H[None], E, x[None], S_prev[None], dtype)[0]
    # every value of the example is exact in both storage types
    assert X.tolist() == arr("assemble", "X").tolist()


def _attn_inputs(case):
    g = CASES[case]
    q = np.array(g["q"][0], np.float64)
    Kc = np.array(g["Kc"], np.float64)
    Vc = np.array(g["Vc"], np.float64)
    Kn = np.array(g["Kn"], np.float64)
    Vn = np.array(g["Vn"], np.float64)
    return q, Kc, Vc, Kn, Vn


def test_attention_worked_heads_bidirectional_and_causal():
    q, Kc, Vc, Kn, Vn = _attn_inputs("attention")
    C, Hq, dh, L = Kn.shape[0], q.shape[0], 1, Kc.shape[0]
    Q = np.broadcast_to(q[None, None, :, None], (1, C, Hq, dh)).copy()   # every position, head h queries q[h]
    Kc4, Vc4 = Kc.reshape(1, 1, L, dh), Vc.reshape(1, 1, L, dh)         # [B, Hkv, cap, dh]
    Kn4, Vn4 = Kn.reshape(1, C, 1, dh), Vn.reshape(1, C, 1, dh)         # [B, C, Hkv, dh]
    for causal, suffix in ((False, "bidir"), (True, "causal")):
        O, lse = step.attention(Q, Kc4, Vc4, Kn4, Vn4, L, causal)
        np.testing.assert_allclose(O[0, :, :, 0], arr("attention", "O_" + suffix), rtol=1e-14, atol=1e-14)
        np.testing.assert_allclose(lse[0], arr("attention", "lse_" + suffix), rtol=1e-14, atol=1e-14)
        for i in range(C):
            for h in range(Hq):
                o, l1 = step.attention_row(Q[0, i, h], 0, 0, i, Kc4, Vc4, Kn4, Vn4, L, causal)
                np.testing.assert_allclose(o[0], arr("attention", "O_" + suffix)[i, h], rtol=1e-14, atol=1e-14)
                assert math.isclose(l1, arr("attention", "lse_" + suffix)[i, h], rel_tol=1e-14)


def test_attention_worked_scale():
    q, Kc, Vc, Kn, Vn = _attn_inputs("attention_scale")
    dh, L = q.shape[0], Kc.shape[0]
    Q = q.reshape(1, 1, 1, dh)
    O, lse = step.attention(Q, Kc.reshape(1, 1, L, dh), Vc.reshape(1, 1, L, dh), Kn.reshape(1, 1, 1, dh),
                            Vn.reshape(1, 1, 1, dh), L, False)
    np.testing.assert_allclose(O[0, 0, 0], arr("attention_scale", "O"), rtol=1e-14, atol=1e-14)
    assert math.isclose(lse[0, 0, 0], arr("attention_scale", "lse"), rel_tol=1e-14)
