"""Pins of the oracle's masked-diffusion sampler ("Diffusione mascherata": the
model predicts the token behind each [MASK]; the prediction replaces the mask
where its confidence meets the threshold; a replaced token is locked and is
never corrected later).  CPU only."""
import numpy as np
import pytest

from oracle import brute, step
from synth import config_by_name, Config, from_storage, gen_problem

M = 9  # the [MASK] id of the hand-worked cases


def test_unmask_hand_worked_positions():
    """Each position is one case of the rule, worked out by hand:
    0 masked, confident (0.9 >= 0.5)            -> commits its prediction 5
    1 masked, not confident (0.4 < 0.5)         -> stays masked
    2 already committed (token 2), confident    -> locked: stays 2, not 7
    3 masked, confident, but predicts [MASK]     -> nothing to commit, stays masked
    4 masked, confidence exactly the threshold   -> commits ("meets" includes equality)
    5 masked, confidence one float32 step below  -> stays masked
    6 already committed, not confident          -> locked: stays 4 (no renoise)
    """
    tau = 0.5
    below = float(np.nextafter(np.float32(0.5), np.float32(0)))
    a = [5, 3, 7, M, 6, 8, 1]
    c = [0.9, 0.4, 0.95, 0.99, 0.5, below, 0.1]
    x = [M, M, 2, M, M, M, 4]
    x_new, commit = step.unmask(a, c, tau, x, M)
    assert x_new.tolist() == [5, M, 2, M, 6, M, 4]
    assert commit.tolist() == [1, 0, 0, 0, 1, 0, 0]


def test_unmask_threshold_is_compared_in_float32():
    """tau = 0.9 is not a float32; the kernel receives float32(0.9), which is
    just below 0.9.  A confidence between the two commits (it meets the
    float32 threshold although it is below 0.9); one under float32(0.9) does
    not."""
    t32 = float(np.float32(0.9))
    assert t32 < 0.899999985 < 0.9
    x_new, commit = step.unmask([3, 3], [0.899999985, 0.8999999], 0.9, [M, M], M)
    assert commit.tolist() == [1, 0] and x_new.tolist() == [3, M]


def test_unmask_threshold_extremes():
    rng = np.random.default_rng(1)
    V, R = 50, 400
    a = rng.integers(0, V, R)
    c = rng.uniform(1.0 / V, 1.0, R)
    x = np.where(rng.uniform(size=R) < 0.6, M, rng.integers(0, V, R))
    # tau = 0: every masked position whose prediction is not [MASK] commits
    x0, k0 = step.unmask(a, c, 0.0, x, M)
    assert np.array_equal(k0.astype(bool), (x == M) & (a != M))
    assert np.array_equal(x0[x != M], x[x != M])
    # tau above 1: nothing commits, the canvas is unchanged
    x1, k1 = step.unmask(a, c, 1.5, x, M)
    assert not k1.any() and np.array_equal(x1, x)


def tiny_masked_cfg():
    c = config_by_name("tiny_c16_L32_d64_V512_f32")
    return Config("tiny_masked", 93, c.B, c.C, c.L, c.d, c.Hq, c.Hkv, c.dh, c.V, c.dtype, 6, 1,
                  (0.3, 0.3))


def test_masked_chain_locks_and_only_unmasks():
    """A chain of masked steps on the tiny workload from a fully masked canvas:
    the number of masks never grows, a committed token never changes, and
    every commit is a masked position whose confidence met tau."""
    cfg = tiny_masked_cfg()
    p = gen_problem(cfg)
    f = lambda a: from_storage(a, cfg.dtype).astype(np.float64)
    E, H, Kc, Vc = f(p.E), f(p.H[0]), f(p.Kc), f(p.Vc)
    W = {k: f(v) for k, v in p.W.items()}
    mask_id = cfg.V - 1
    x = step.init_masked(cfg.B, cfg.C, mask_id)
    assert (x == mask_id).all()
    S = None
    n_masked = [int((x == mask_id).sum())]
    for s in range(cfg.steps):
        r = step.denoise_step_masked(H, E, W, Kc, Vc, cfg.L, x, S, cfg.tau[0], mask_id, cfg.dtype)
        xn = r["x_new"].reshape(-1)
        xo = x.reshape(-1)
        locked = xo != mask_id
        assert np.array_equal(xn[locked], xo[locked])
        k = r["commit"].reshape(-1).astype(bool)
        assert np.array_equal(k, (xo == mask_id) & (xn != mask_id))
        assert np.all(r["c"][k] >= np.float32(cfg.tau[0])) and np.array_equal(xn[k], r["a"][k])
        x, S = r["x_new"], r["S"]
        n_masked.append(int((x == mask_id).sum()))
    assert all(b <= a for a, b in zip(n_masked, n_masked[1:]))
    assert n_masked[-1] < n_masked[0], n_masked


def test_masked_step_model_pass_matches_brute_force():
    """The masked sampler runs the same model pass as the uniform-state step:
    on a fully masked tiny canvas its prediction, confidence and S agree with
    the scalar brute force, and its commits follow from them."""
    cfg = tiny_masked_cfg()
    p = gen_problem(cfg)
    f = lambda a: from_storage(a, cfg.dtype).astype(np.float64)
    E, H, Kc, Vc = f(p.E), f(p.H[0]), f(p.Kc), f(p.Vc)
    W = {k: f(v) for k, v in p.W.items()}
    mask_id = cfg.V - 1
    x = step.init_masked(cfg.B, cfg.C, mask_id)
    r = step.denoise_step_masked(H, E, W, Kc, Vc, cfg.L, x, None, cfg.tau[0], mask_id, cfg.dtype)
    b = brute.step(H, E, W, Kc, Vc, cfg.L, x, None, cfg.tau[0], cfg.seed, 1, 0, cfg.dtype)
    assert np.array_equal(np.asarray(b["a"]).reshape(-1), r["a"])
    np.testing.assert_allclose(np.asarray(b["c"]).reshape(-1), r["c"], rtol=1e-12, atol=0)
    np.testing.assert_allclose(np.asarray(b["S"]).reshape(cfg.R, -1), r["S"].reshape(cfg.R, -1),
                               rtol=0, atol=1e-14)
    want = [int(ai) if (ci >= np.float32(cfg.tau[0]) and ai != mask_id) else mask_id
            for ai, ci in zip(np.asarray(b["a"]).reshape(-1), np.asarray(b["c"]).reshape(-1))]
    assert r["x_new"].reshape(-1).tolist() == want
