"""Edge and degenerate cases of the step on the GPU against the oracle: a
one-id vocabulary (the softmax is a point mass), a tiny ragged vocabulary, the
HBM-bound attention shape the bench times (every row), thresholds that renoise
nothing or everything, an empty cache and one-token canvases."""
import numpy as np
import pytest
import torch

from oracle import step
from synth import Config, gen_problem
from tests.gpu_util import ATOL, RELF, as_f64, close, need_gpu, say
from tests.test_gpu_kernels import _attn_inputs, _run_attn, _run_vocab, _vocab_inputs
from tests.test_gpu_step import Dev, compare_full, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()
    import uniform_state_discrete_amd as dg
    dg.lib()
    yield


@pytest.mark.parametrize("R,d,dtype", [(5, 2048, "bf16"), (3, 256, "bf16"), (4, 64, "f32")])
def test_vocab_single_id(R, d, dtype):
    """V = 1: every probability is exactly 1, so conf = 1, argmax = 0,
    lse = the logit and S = E[0] exactly (one product by 1, one rounding of
    an already representable value)."""
    say(f"vocab V=1 R={R} d={d} {dtype}")
    E, Z = _vocab_inputs(R, d, 1, dtype, seed=R + d, signal=5.0)
    m, a, c, lse, S = _run_vocab(R, d, 1, E, Z, dtype)
    Ef = as_f64(E, dtype)
    assert np.all(c == 1.0) and np.all(a == 0)
    assert np.array_equal(S, np.repeat(Ef[:1], R, axis=0))
    rm, _, rlse, *_ = step.vocab_selfcond(as_f64(Z, dtype), Ef, dtype)
    close("m", m, rm, ATOL[dtype])
    close("lse", lse, rlse, ATOL[dtype])


@pytest.mark.parametrize("R,d,V", [(9, 256, 7), (70, 2048, 17)])
def test_vocab_tiny_ragged_vocabulary(R, d, V):
    say(f"vocab tiny V={V} R={R} d={d}")
    E, Z = _vocab_inputs(R, d, V, "bf16", seed=R * V + d)
    m, a, c, lse, S = _run_vocab(R, d, V, E, Z, "bf16")
    Ef, Zf = as_f64(E, "bf16"), as_f64(Z, "bf16")
    rm, ra, rlse, rc, rS, _ = step.vocab_selfcond(Zf, Ef, "bf16")
    close("m", m, rm, ATOL["bf16"])
    close("c", c, rc, ATOL["bf16"])
    close("lse", lse, rlse, ATOL["bf16"])
    close("S", S, rS, ATOL["bf16"], RELF["bf16"], bf16_ulp=True)
    assert np.array_equal(a, ra)


def test_attention_hbm_shape_every_row():
    """The bench's HBM-bound shape: 16 canvas queries of 32 heads over a
    32768-row cache of 8 KV heads (K/V ~ N(0, 1)), every output row."""
    B, C, L, Hq, Hkv, dh = 1, 16, 32768, 32, 8, 128
    say("attention HBM shape, every row")
    arrs = _attn_inputs(B, C, L, L + C, Hq, Hkv, dh, "bf16", seed=32768)
    O, lse = _run_attn(B, C, L, L + C, Hq, Hkv, dh, "bf16", arrs, 0)
    q, Kc, Vc, Kn, Vn = (as_f64(x, "bf16") for x in arrs)
    rO, rlse = step.attention(q, Kc, Vc, Kn, Vn, L, causal=False, dtype="bf16")
    close("O", O, rO, ATOL["bf16"], RELF["bf16"], bf16_ulp=True)
    close("lse", lse, rlse, ATOL["bf16"])


SMALL = Config("edge_small_bf16", 97, B=2, C=40, L=70, d=256, Hq=4, Hkv=2, dh=64, V=3000,
               dtype="bf16", steps=2, blocks=1, tau=(0.6, 0.6))
TINY = Config("edge_tiny_f32", 98, B=1, C=16, L=32, d=64, Hq=2, Hkv=1, dh=32, V=512,
              dtype="f32", steps=2, blocks=1, tau=(0.5, 0.5))


@pytest.mark.parametrize("cfg", [TINY, SMALL], ids=lambda c: c.name)
def test_step_thresholds_renoise_nothing_or_everything(cfg):
    """tau = 0: no confidence falls below it, so every token is the argmax and
    the mask is empty.  tau = 1.5: every confidence falls below it, so every
    token is the Philox draw of its position, bit for bit, whatever the
    floats."""
    import uniform_state_discrete_amd as dg
    say(f"step thresholds {cfg.name}")
    p = gen_problem(cfg)
    g = Dev(p)
    h = host(p)
    x = torch.empty((cfg.B, cfg.C), dtype=torch.int32, device="cuda")
    dg.dg_init_canvas(cfg.R, cfg.C, cfg.V, cfg.seed, 0, x)
    o = g.step(x, None, 0.0, 1, 0)
    assert not o["mask"].cpu().numpy().any()
    assert np.array_equal(o["tokens_out"].cpu().numpy().reshape(-1), o["argmax"].cpu().numpy())
    ref = step.denoise_step(h["H"][0], h["E"], h["W"], h["Kc"], h["Vc"], cfg.L, x.cpu().numpy(), None, 0.0,
                            cfg.seed, 1, 0, cfg.dtype)
    compare_full(cfg, o, ref, h["E"], 0.0, "tau 0")
    o = g.step(x, None, 1.5, 2, 0)
    assert o["mask"].cpu().numpy().all()
    draws, _ = step.renoise(np.zeros(cfg.R, np.int64), np.zeros(cfg.R), 1.5, cfg.seed, 2, 0, cfg.B, cfg.C, cfg.V)
    assert np.array_equal(o["tokens_out"].cpu().numpy().reshape(-1), draws)


@pytest.mark.parametrize("cfg", [
    Config("edge_empty_cache", 99, B=3, C=40, L=0, d=256, Hq=4, Hkv=2, dh=64, V=3000,
           dtype="bf16", steps=1, blocks=1, tau=(0.6, 0.6)),
    Config("edge_one_token_canvas", 100, B=3, C=1, L=70, d=256, Hq=4, Hkv=2, dh=64, V=3000,
           dtype="bf16", steps=1, blocks=1, tau=(0.6, 0.6)),
    Config("edge_one_token_no_cache", 101, B=2, C=1, L=0, d=64, Hq=2, Hkv=1, dh=32, V=512,
           dtype="f32", steps=1, blocks=1, tau=(0.5, 0.5)),
], ids=lambda c: c.name)
def test_step_empty_cache_and_one_token_canvas(cfg):
    import uniform_state_discrete_amd as dg
    say(f"step {cfg.name}")
    p = gen_problem(cfg)
    g = Dev(p)
    h = host(p)
    x = torch.empty((cfg.B, cfg.C), dtype=torch.int32, device="cuda")
    dg.dg_init_canvas(cfg.R, cfg.C, cfg.V, cfg.seed, 0, x)
    o = g.step(x, None, cfg.tau[0], 1, 0)
    ref = step.denoise_step(h["H"][0], h["E"], h["W"], h["Kc"], h["Vc"], cfg.L, x.cpu().numpy(), None,
                            cfg.tau[0], cfg.seed, 1, 0, cfg.dtype)
    compare_full(cfg, o, ref, h["E"], cfg.tau[0], cfg.name)
