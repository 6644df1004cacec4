"""dg_denoise_step and dg_prefill_append against the oracle, in lockstep: step t
of the oracle consumes the GPU's inputs to step t (tokens and self-conditioning
vector), so an excluded near-tie cannot cascade.  Every workload, the
full-size ones included, is compared on every element of every step run."""
import math

import numpy as np
import pytest
import torch

from oracle import step
from synth import config_by_name, Config, gen_problem, tau_schedule
from tests.gpu_util import (ATOL, RELF, argmax_match, as_f64, close, close_rel, dev, f64, need_gpu,
                            renoise_match, say)

pytestmark = pytest.mark.gpu

SMALL_BF16 = Config("test_small_bf16", 90, B=2, C=40, L=70, d=256, Hq=4, Hkv=2, dh=64, V=3000,
                    dtype="bf16", steps=3, blocks=2, tau=(0.6, 0.8))
# 1100 rows (5 canvases of 220): the projections run the 128 x 128 tile GEMM,
# with a ragged last row tile (1100 = 8 x 128 + 76)
MANY_ROWS_BF16 = Config("test_many_rows_bf16", 91, B=5, C=220, L=40, d=256, Hq=4, Hkv=2, dh=64, V=3000,
                        dtype="bf16", steps=2, blocks=1, tau=(0.6, 0.6))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()
    import uniform_state_discrete_amd as dg
    dg.lib()
    yield


class Dev:
    """A workload's tensors on the GPU."""

    def __init__(self, p):
        import uniform_state_discrete_amd as dg
        c = p.cfg
        self.cfg = c
        self.W = {k: dev(v) for k, v in p.W.items()}
        self.W["E"] = dg.model_embedding(dev(p.E))
        self.Kc = dev(p.Kc)
        self.Vc = dev(p.Vc)
        self.H = [dev(h) for h in p.H]
        self.dt = dg.DG_BF16 if c.dtype == "bf16" else dg.DG_F32
        self.dims = dg.make_dims(c.B, c.C, c.L, c.cap, c.d, c.Hq, c.Hkv, c.dh, c.V, self.dt)
        self.ws = dg.workspace(dg.dg_workspace_bytes(self.dims))

    def step(self, x, S, tau, t, block, L=None):
        import uniform_state_discrete_amd as dg
        c = self.cfg
        R = c.B * c.C
        fdt = self.W["E"].dtype
        o = dict(
            H=self.H[block], k_cache=self.Kc, v_cache=self.Vc, tokens_in=x, selfcond_in=S,
            tokens_out=torch.empty_like(x), selfcond_out=torch.empty((c.B, c.C, c.d), dtype=fdt, device="cuda"),
            max_logit=torch.empty(R, dtype=torch.float32, device="cuda"),
            conf=torch.empty(R, dtype=torch.float32, device="cuda"),
            lse=torch.empty(R, dtype=torch.float32, device="cuda"),
            argmax=torch.empty(R, dtype=torch.int32, device="cuda"),
            mask=torch.empty(R, dtype=torch.uint8, device="cuda"),
            x_out=torch.empty((R, c.d), dtype=fdt, device="cuda"),
            q_out=torch.empty((R, c.Hq * c.dh), dtype=fdt, device="cuda"),
            k_new_out=torch.empty((R, c.Hkv * c.dh), dtype=fdt, device="cuda"),
            v_new_out=torch.empty((R, c.Hkv * c.dh), dtype=fdt, device="cuda"),
            attn_out=torch.empty((R, c.Hq * c.dh), dtype=fdt, device="cuda"),
            z_out=torch.empty((R, c.d), dtype=fdt, device="cuda"))
        dims = self.dims if L is None else dg.make_dims(c.B, c.C, L, c.cap, c.d, c.Hq, c.Hkv, c.dh, c.V, self.dt)
        dg.dg_denoise_step(dims, self.W, o, tau, c.seed, t, block, self.ws)
        torch.cuda.synchronize()
        return o


def host(p):
    c = p.cfg
    f = lambda a: as_f64(a, c.dtype)
    return dict(E=f(p.E), W={k: f(v) for k, v in p.W.items()}, Kc=f(p.Kc), Vc=f(p.Vc),
                H=[f(h) for h in p.H])


def compare_full(c, o, ref, E, tau, tag):
    dt = c.dtype
    R = c.B * c.C
    rel_ulp = 2.0 ** -7 if dt == "bf16" else 1e-6
    close_rel(f"{tag} X", f64(o["x_out"]), ref["X"].reshape(R, -1), rel_ulp)
    close_rel(f"{tag} Q", f64(o["q_out"]), ref["Q"].reshape(R, -1), 2 * rel_ulp)
    close_rel(f"{tag} Kn", f64(o["k_new_out"]), ref["Kn"].reshape(R, -1), 2 * rel_ulp)
    close_rel(f"{tag} Vn", f64(o["v_new_out"]), ref["Vn"].reshape(R, -1), 2 * rel_ulp)
    bu = dt == "bf16"
    close(f"{tag} O", f64(o["attn_out"]), ref["O"].reshape(R, -1), ATOL[dt], RELF[dt], bf16_ulp=bu)
    close(f"{tag} Z", f64(o["z_out"]), ref["Z"].reshape(R, -1), ATOL[dt], bf16_ulp=bu)
    close(f"{tag} m", f64(o["max_logit"]), ref["m"], ATOL[dt])
    close(f"{tag} lse", f64(o["lse"]), ref["lse"], ATOL[dt])
    close(f"{tag} c", f64(o["conf"]), ref["c"], ATOL[dt])
    close(f"{tag} S", f64(o["selfcond_out"]).reshape(R, -1), ref["S"].reshape(R, -1), ATOL[dt], RELF[dt],
          bf16_ulp=bu)
    gap = ref["gap"]
    argmax_match(f"{tag} argmax", o["argmax"].cpu().numpy(), ref["a"], gap, ref["m"])
    tie = gap < 1e-3 * np.maximum(1.0, np.abs(ref["m"]))
    renoise_match(f"{tag} renoise", o["tokens_out"].cpu().numpy(), o["mask"].cpu().numpy(),
                  ref["x_new"], ref["mask"], ref["c"], tau, extra_excl=tie)


@pytest.mark.parametrize("cfg", [config_by_name("tiny_c16_L32_d64_V512_f32"), SMALL_BF16, MANY_ROWS_BF16,
                                 config_by_name("canvas256_L1024_d2048_V32768")], ids=lambda c: c.name)
def test_step_lockstep_every_element(cfg):
    import uniform_state_discrete_amd as dg
    say(f"step lockstep {cfg.name}")
    p = gen_problem(cfg)
    g = Dev(p)
    h = host(p)
    taus = tau_schedule(cfg)
    x = torch.empty((cfg.B, cfg.C), dtype=torch.int32, device="cuda")
    dg.dg_init_canvas(cfg.R, cfg.C, cfg.V, cfg.seed, 0, x)
    S = None
    nsteps = min(cfg.steps, 4)
    kept = []
    for s in range(nsteps):
        o = g.step(x, S, taus[s], s + 1, 0)
        xin = x.cpu().numpy()
        Sin = None if S is None else f64(S)
        ref = step.denoise_step(h["H"][0], h["E"], h["W"], h["Kc"], h["Vc"], cfg.L, xin, Sin,
                                taus[s], cfg.seed, s + 1, 0, cfg.dtype)
        compare_full(cfg, o, ref, h["E"], taus[s], f"step {s}")
        kept.append(1 - ref["mask"].mean())
        x, S = o["tokens_out"], o["selfcond_out"]
    say("kept fraction per step", np.round(kept, 3))


# ---- full-size workloads, every element -----------------------------------------------

@pytest.mark.parametrize("name", ["canvas256_L8192_d2048_V262144", "canvas256_L32768_d4096_V262144"])
def test_step_full_size_every_row(name):
    """Four chained steps of a full-size workload, every element of every
    intermediate and output against the oracle step in lockstep."""
    import uniform_state_discrete_amd as dg
    c = config_by_name(name)
    say(f"full-size step {c.name}, every row")
    p = gen_problem(c)
    g = Dev(p)
    h = host(p)
    del p
    taus = tau_schedule(c)
    x = torch.empty((c.B, c.C), dtype=torch.int32, device="cuda")
    dg.dg_init_canvas(c.R, c.C, c.V, c.seed, 0, x)
    S = None
    kept = []
    for s in range(4):
        o = g.step(x, S, taus[s], s + 1, 0)
        ref = step.denoise_step(h["H"][0], h["E"], h["W"], h["Kc"], h["Vc"], c.L, x.cpu().numpy(),
                                None if S is None else f64(S), taus[s], c.seed, s + 1, 0, c.dtype)
        compare_full(c, o, ref, h["E"], taus[s], f"step {s}")
        kept.append(1 - ref["mask"].mean())
        # properties of the outputs that hold at any size
        tok = o["tokens_out"].cpu().numpy().reshape(-1)
        assert tok.min() >= 0 and tok.max() < c.V
        x, S = o["tokens_out"], o["selfcond_out"]
    say("kept fraction per step", np.round(kept, 3))


@pytest.mark.parametrize("cfg", [config_by_name("tiny_c16_L32_d64_V512_f32"), SMALL_BF16], ids=lambda c: c.name)
def test_block_append_and_next_block(cfg):
    """Finish block 0, append it through the causal prefill, then run a step of
    block 1 against the grown cache."""
    import uniform_state_discrete_amd as dg
    say(f"block append {cfg.name}")
    c = cfg if cfg.blocks > 1 else Config(cfg.name + "_2blk", cfg.index, cfg.B, cfg.C, cfg.L, cfg.d,
                                          cfg.Hq, cfg.Hkv, cfg.dh, cfg.V, cfg.dtype, cfg.steps, 2, cfg.tau)
    p = gen_problem(c)
    g = Dev(p)
    h = host(p)
    x = torch.empty((c.B, c.C), dtype=torch.int32, device="cuda")
    dg.dg_init_canvas(c.R, c.C, c.V, c.seed, 0, x)
    o = g.step(x, None, c.tau[0], 1, 0)
    xf = o["argmax"].view(c.B, c.C).contiguous()        # the finalized canvas: argmax of the last step
    attn = torch.empty((c.B, c.C, c.Hq, c.dh), dtype=g.W["E"].dtype, device="cuda")
    Kc0, Vc0 = f64(g.Kc), f64(g.Vc)
    dg.dg_prefill_append(g.dims, g.W, g.H[0], xf, g.Kc, g.Vc, attn, g.ws)
    torch.cuda.synchronize()
    K2, V2, rO, _ = step.prefill_append(h["H"][0], h["E"], h["W"], Kc0, Vc0, c.L, xf.cpu().numpy(), c.dtype)
    assert np.array_equal(f64(g.Kc)[:, :, :c.L], Kc0[:, :, :c.L])
    close_rel("appended K", f64(g.Kc)[:, :, c.L:c.L + c.C], K2[:, :, c.L:c.L + c.C], 2.0 ** -6)
    close_rel("appended V", f64(g.Vc)[:, :, c.L:c.L + c.C], V2[:, :, c.L:c.L + c.C], 2.0 ** -6)
    close("causal O", f64(attn), rO, ATOL[c.dtype], RELF[c.dtype], bf16_ulp=c.dtype == "bf16")
    # block 1 starts from a fresh canvas (draw 0 of block 1) over the grown cache
    L1 = c.L + c.C
    dg.dg_init_canvas(c.R, c.C, c.V, c.seed, 1, x)
    assert np.array_equal(x.cpu().numpy(), step.init_canvas(c.seed, 1, c.B, c.C, c.V))
    o = g.step(x, None, c.tau[1], 1, 1, L=L1)
    ref = step.denoise_step(h["H"][1], h["E"], h["W"], f64(g.Kc), f64(g.Vc), L1, x.cpu().numpy(), None,
                            c.tau[1], c.seed, 1, 1, c.dtype)
    compare_full(c, o, ref, h["E"], c.tau[1], "block 1 step 0")


def test_prefill_append_prompt4096_every_element():
    """The causal prefill of a 4096-token prompt into an empty cache, the shape
    bench.py times (the full-vocabulary workload's model: d = 2048, 16/8 heads
    of 128): every appended K/V cache row and every element of the causal
    attention output against the oracle's prefill-append."""
    import uniform_state_discrete_amd as dg
    c = config_by_name("canvas256_L8192_d2048_V262144")
    n = 4096
    say(f"prefill-append of a {n}-token prompt, every element")
    p = gen_problem(c)
    W = {k: dev(v) for k, v in p.W.items()}
    W["E"] = dg.model_embedding(dev(p.E))
    rng = np.random.default_rng(4096)
    Hs = np.tile(p.H[0].reshape(c.C, c.d), (n // c.C, 1)).reshape(1, n, c.d)   # stored bf16 bits
    toks = rng.integers(0, c.V, (1, n)).astype(np.int32)
    dims = dg.make_dims(1, n, 0, n, c.d, c.Hq, c.Hkv, c.dh, c.V, dg.DG_BF16)
    ws = dg.workspace(dg.dg_workspace_bytes(dims))
    Kc = torch.zeros((1, c.Hkv, n, c.dh), dtype=torch.bfloat16, device="cuda")
    Vc = torch.zeros_like(Kc)
    attn = torch.empty((1, n, c.Hq, c.dh), dtype=torch.bfloat16, device="cuda")
    dg.dg_prefill_append(dims, W, dev(Hs), dev(toks), Kc, Vc, attn, ws)
    torch.cuda.synchronize()
    f = lambda a: as_f64(a, c.dtype)
    E = f(p.E)
    Wf = {k: f(v) for k, v in p.W.items()}
    del p
    z = np.zeros((1, c.Hkv, n, c.dh))
    K2, V2, rO, _ = step.prefill_append(f(Hs), E, Wf, z, z, 0, toks, c.dtype)
    close_rel("appended K, 4096 rows", f64(Kc), K2, 2.0 ** -6)
    close_rel("appended V, 4096 rows", f64(Vc), V2, 2.0 ** -6)
    close("causal O", f64(attn), rO, ATOL[c.dtype], RELF[c.dtype], bf16_ulp=True)
