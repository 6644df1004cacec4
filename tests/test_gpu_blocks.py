"""dg_block_loop and its HIP graph (block diffusion, "Campionamento
multi-canvas (diffusione a blocchi)"): every step of every block against the
oracle in lockstep (step s of the oracle consumes the GPU's tokens and
self-conditioning vector of step s-1, and a cache the oracle grows itself from
the GPU's finished canvases), and graph replays equal to the eager sequence
bit for bit, including the full-size 8-canvas block workload.  At full size
(8 canvases, V = 262144) the whole 4-block sequence runs once with per-step
records; every row of all 32 steps of block 0, every appended cache row of
the 4 blocks, and every row of the first and last step of blocks 1-3 are
compared with the oracle (the other 60 steps of blocks 1-3 run but are not
compared; each costs the oracle about 5 s)."""
import numpy as np
import pytest
import torch

from oracle import step
from synth import config_by_name, Config, gen_problem, tau_schedule
from tests.gpu_util import ATOL, RELF, as_f64, close, close_rel, f64, need_gpu, renoise_match, say

pytestmark = pytest.mark.gpu

SMALL_BF16_3BLK = Config("blocks_small_bf16", 91, B=2, C=40, L=70, d=256, Hq=4, Hkv=2, dh=64, V=3000,
                         dtype="bf16", steps=3, blocks=3, tau=(0.6, 0.8))
TINY_2BLK = Config("blocks_tiny_f32", 92, B=1, C=16, L=32, d=64, Hq=2, Hkv=1, dh=32, V=512,
                   dtype="f32", steps=4, blocks=2, tau=(0.5, 0.7))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()
    import uniform_state_discrete_amd as dg
    dg.lib()
    yield


class Loop:
    """A workload's tensors on the GPU plus the block loop's buffers."""

    def __init__(self, p, blocks, steps, trace):
        import uniform_state_discrete_amd as dg
        c = p.cfg
        self.cfg, self.blocks, self.steps = c, blocks, steps
        fdt = torch.bfloat16 if c.dtype == "bf16" else torch.float32
        self.W = {k: dg.to_device(v) for k, v in p.W.items()}
        self.W["E"] = dg.model_embedding(dg.to_device(p.E))
        self.Kc0 = dg.to_device(p.Kc)
        self.Vc0 = dg.to_device(p.Vc)
        self.Kc, self.Vc = self.Kc0.clone(), self.Vc0.clone()
        self.H = torch.stack([dg.to_device(h) for h in p.H[:blocks]]).contiguous()
        self.dims = dg.make_dims(c.B, c.C, c.L, c.cap, c.d, c.Hq, c.Hkv, c.dh, c.V,
                                 dg.DG_BF16 if c.dtype == "bf16" else dg.DG_F32)
        self.ws = dg.workspace(dg.dg_workspace_bytes(self.dims))
        R = c.R
        i32 = dict(dtype=torch.int32, device="cuda")
        f32 = dict(dtype=torch.float32, device="cuda")
        self.io = dict(H=self.H, k_cache=self.Kc, v_cache=self.Vc,
                       tokens=torch.zeros((blocks, c.B, c.C), **i32),
                       canvas=torch.zeros((2, c.B, c.C), **i32),
                       selfcond=torch.zeros((2, c.B, c.C, c.d), dtype=fdt, device="cuda"),
                       max_logit=torch.zeros(R, **f32), conf=torch.zeros(R, **f32),
                       argmax=torch.zeros(R, **i32), mask=torch.zeros(R, dtype=torch.uint8, device="cuda"))
        if trace:
            self.io.update(trace_tokens=torch.zeros((blocks, steps, c.B, c.C), **i32),
                           trace_conf=torch.zeros((blocks, steps, R), **f32),
                           trace_selfcond=torch.zeros((blocks, steps, c.B, c.C, c.d), dtype=fdt, device="cuda"))
        self.taus = tau_schedule(c)[:steps] if steps == c.steps else \
            [c.tau[0] + (c.tau[1] - c.tau[0]) * s / max(1, steps - 1) for s in range(steps)]

    def outputs(self):
        """Host copies of everything the loop writes."""
        keys = ["tokens", "trace_tokens", "trace_conf", "trace_selfcond"]
        out = {k: self.io[k].cpu().clone() for k in keys if k in self.io}
        c = self.cfg
        out["k_cache"] = self.Kc[:, :, c.L:c.L + self.blocks * c.C].cpu().clone()
        out["v_cache"] = self.Vc[:, :, c.L:c.L + self.blocks * c.C].cpu().clone()
        return out

    def clear_outputs(self):
        c = self.cfg
        for k in ("tokens", "trace_tokens", "trace_conf", "trace_selfcond"):
            if k in self.io:
                self.io[k].zero_()
        self.Kc[:, :, c.L:].zero_()
        self.Vc[:, :, c.L:].zero_()


def lockstep(c, lp, p):
    """Every step of every block of the GPU trace against the oracle."""
    f = lambda a: as_f64(a, c.dtype)
    E = f(p.E)
    W = {k: f(v) for k, v in p.W.items()}
    Kc, Vc = f(p.Kc), f(p.Vc)
    R = c.R
    tt = lp.io["trace_tokens"].cpu().numpy()
    tc = lp.io["trace_conf"].cpu().numpy()
    ts = lp.io["trace_selfcond"].float().cpu().numpy().astype(np.float64)
    toks = lp.io["tokens"].cpu().numpy()
    L = c.L
    excluded = 0
    for k in range(lp.blocks):
        H = f(p.H[k])
        x = step.init_canvas(c.seed, k, c.B, c.C, c.V)
        S = None
        for s in range(lp.steps):
            tag = f"block {k} step {s}"
            ref = step.denoise_step(H, E, W, Kc, Vc, L, x, S, lp.taus[s], c.seed, s + 1, k, c.dtype)
            close(f"{tag} c", tc[k, s], ref["c"], ATOL[c.dtype])
            close(f"{tag} S", ts[k, s].reshape(R, -1), ref["S"].reshape(R, -1), ATOL[c.dtype], RELF[c.dtype],
                  bf16_ulp=c.dtype == "bf16")
            gap = ref["gap"]
            tie = gap < 1e-3 * np.maximum(1.0, np.abs(ref["m"]))
            # the kernel renoises where its fp32 confidence is below the fp32 tau
            got_mask = (tc[k, s] < np.float32(lp.taus[s])).astype(np.uint8)
            excluded += renoise_match(f"{tag} renoise", tt[k, s], got_mask, ref["x_new"], ref["mask"], ref["c"],
                                      lp.taus[s], extra_excl=tie)
            if s == lp.steps - 1:
                bad = (toks[k].reshape(-1) != ref["a"]) & ~tie
                say(f"{tag} finished canvas: {int(bad.sum())} argmax mismatches, {int(tie.sum())} near-ties")
                assert not bad.any()
            # lockstep: the next step consumes the GPU's outputs of this one
            x = tt[k, s]
            S = ts[k, s]
        # the oracle grows its own cache from the GPU's finished canvas
        Kc, Vc, _, _ = step.prefill_append(H, E, W, Kc, Vc, L, toks[k], c.dtype)
        L += c.C
    got_K = f64(lp.Kc)
    got_V = f64(lp.Vc)
    close_rel("appended K rows", got_K[:, :, c.L:L], Kc[:, :, c.L:L], 2.0 ** -6)
    close_rel("appended V rows", got_V[:, :, c.L:L], Vc[:, :, c.L:L], 2.0 ** -6)
    assert np.array_equal(got_K[:, :, :c.L], f(p.Kc)[:, :, :c.L])
    say(f"lockstep done, {excluded} positions excluded near tau")


@pytest.mark.parametrize("cfg", [TINY_2BLK, SMALL_BF16_3BLK], ids=lambda c: c.name)
def test_block_loop_lockstep_and_graph(cfg):
    import uniform_state_discrete_amd as dg
    say(f"block loop {cfg.name}")
    p = gen_problem(cfg)
    lp = Loop(p, cfg.blocks, cfg.steps, trace=True)
    dg.dg_block_loop(lp.dims, lp.W, lp.io, lp.taus, lp.steps, lp.blocks, cfg.seed, lp.ws)
    torch.cuda.synchronize()
    lockstep(cfg, lp, p)
    eager = lp.outputs()
    # the same loop as one graph, replayed several times with eager work and
    # synchronisation in between; every replay equals the eager run
    side = torch.cuda.Stream()
    g = dg.dg_graph_capture_block_loop(lp.dims, lp.W, lp.io, lp.taus, lp.steps, lp.blocks, cfg.seed, lp.ws, side)
    for rep in range(3):
        lp.clear_outputs()
        torch.cuda.synchronize()
        g.launch(side)
        side.synchronize()
        got = lp.outputs()
        for k, v in eager.items():
            assert torch.equal(got[k], v), f"graph replay {rep}: {k} differs from the eager run"
        say(f"graph replay {rep} equals the eager run")
    g.close()


def test_block_loop_graph_full_size():
    """The 8-canvas block workload at full size (V = 262144, 4096-row caches):
    two blocks of two steps captured in one graph equal the eager sequence bit
    for bit, the appended cache rows of block 0 match the oracle's append of
    the GPU's finished canvas, and every step's outputs are valid."""
    import uniform_state_discrete_amd as dg
    c = config_by_name("blocks4_canvas8x256_L4096_d2048_V262144")
    say(f"full-size block loop graph {c.name}")
    p = gen_problem(c)
    blocks, steps = 2, 2
    lp = Loop(p, blocks, steps, trace=False)
    dg.dg_block_loop(lp.dims, lp.W, lp.io, lp.taus, steps, blocks, c.seed, lp.ws)
    torch.cuda.synchronize()
    eager = lp.outputs()
    tok = eager["tokens"].numpy()
    assert tok.min() >= 0 and tok.max() < c.V
    side = torch.cuda.Stream()
    g = dg.dg_graph_capture_block_loop(lp.dims, lp.W, lp.io, lp.taus, steps, blocks, c.seed, lp.ws, side)
    for rep in range(2):
        lp.clear_outputs()
        torch.cuda.synchronize()
        g.launch(side)
        side.synchronize()
        got = lp.outputs()
        for k, v in eager.items():
            assert torch.equal(got[k], v), f"graph replay {rep}: {k} differs from the eager run"
        say(f"graph replay {rep} equals the eager run")
    g.close()
    # block 0's append for canvas 0, from the GPU's finished canvas: K/V rows are
    # linear in X = H + E[x] (no self-conditioning), so one canvas suffices
    f = lambda a: as_f64(a, c.dtype)
    ids = tok[0, 0]
    X = step.assemble(f(p.H[0][:1]), f(p.E[ids]), np.arange(c.C)[None, :], None, c.dtype).reshape(c.C, c.d)
    Kn = step.linear(X, f(p.W["Wk"]), c.dtype).reshape(c.C, c.Hkv, c.dh).transpose(1, 0, 2)
    Vn = step.linear(X, f(p.W["Wv"]), c.dtype).reshape(c.C, c.Hkv, c.dh).transpose(1, 0, 2)
    close_rel("block 0 appended K rows, canvas 0", f64(lp.Kc[0, :, c.L:c.L + c.C]), Kn, 2.0 ** -6)
    close_rel("block 0 appended V rows, canvas 0", f64(lp.Vc[0, :, c.L:c.L + c.C]), Vn, 2.0 ** -6)


# ---- the full-size 8-canvas block workload, in lockstep with the oracle ---------------------

FULL = "blocks4_canvas8x256_L4096_d2048_V262144"


@pytest.fixture(scope="module")
def full_run():
    """The whole 4 x 32-step sequence of the 8-canvas workload run once on the
    GPU with per-step records, and the oracle's inputs: the stored tensors in
    float64 and a cache the oracle grows itself from the GPU's finished
    canvases (rows [L, L + 4 C) hold the 4 appended blocks; a block's step
    reads only the rows before its own)."""
    import uniform_state_discrete_amd as dg
    c = config_by_name(FULL)
    say(f"full-size block loop {c.name}: GPU run")
    p = gen_problem(c)
    lp = Loop(p, c.blocks, c.steps, trace=True)
    dg.dg_block_loop(lp.dims, lp.W, lp.io, lp.taus, lp.steps, lp.blocks, c.seed, lp.ws)
    torch.cuda.synchronize()
    out = dict(cfg=c, taus=lp.taus,
               tt=lp.io["trace_tokens"].cpu().numpy(), tc=lp.io["trace_conf"].cpu().numpy(),
               ts=lp.io["trace_selfcond"].cpu(), toks=lp.io["tokens"].cpu().numpy(),
               gK=lp.Kc[:, :, c.L:c.L + c.blocks * c.C].float().cpu().numpy(),
               gV=lp.Vc[:, :, c.L:c.L + c.blocks * c.C].float().cpu().numpy())
    tok = out["tt"]
    assert tok.min() >= 0 and tok.max() < c.V
    del lp
    torch.cuda.empty_cache()
    f = lambda a: as_f64(a, c.dtype)
    out.update(E=f(p.E), W={k: f(v) for k, v in p.W.items()}, H=[f(h) for h in p.H])
    Kc, Vc = f(p.Kc), f(p.Vc)
    L = c.L
    for k in range(c.blocks):
        say(f"oracle append of block {k}")
        Kc, Vc, _, _ = step.prefill_append(out["H"][k], out["E"], out["W"], Kc, Vc, L, out["toks"][k], c.dtype)
        L += c.C
    out.update(Kc=Kc, Vc=Vc)
    return out


def _full_step(run, k, s):
    c = run["cfg"]
    R = c.R
    tag = f"block {k} step {s}"
    say(f"full-size {tag}: oracle")
    x = step.init_canvas(c.seed, k, c.B, c.C, c.V) if s == 0 else run["tt"][k, s - 1]
    S = None if s == 0 else run["ts"][k, s - 1].float().numpy().astype(np.float64)
    ref = step.denoise_step(run["H"][k], run["E"], run["W"], run["Kc"], run["Vc"], c.L + k * c.C, x, S,
                            run["taus"][s], c.seed, s + 1, k, c.dtype)
    close(f"{tag} c", run["tc"][k, s], ref["c"], ATOL[c.dtype])
    got_S = run["ts"][k, s].float().numpy().astype(np.float64).reshape(R, -1)
    close(f"{tag} S", got_S, ref["S"].reshape(R, -1), ATOL[c.dtype], RELF[c.dtype], bf16_ulp=True)
    tie = ref["gap"] < 1e-3 * np.maximum(1.0, np.abs(ref["m"]))
    got_mask = (run["tc"][k, s] < np.float32(run["taus"][s])).astype(np.uint8)
    renoise_match(f"{tag} renoise", run["tt"][k, s], got_mask, ref["x_new"], ref["mask"], ref["c"],
                  run["taus"][s], extra_excl=tie)
    if s == c.steps - 1:
        bad = (run["toks"][k].reshape(-1) != ref["a"]) & ~tie
        say(f"{tag} finished canvas: {int(bad.sum())} argmax mismatches, {int(tie.sum())} near-ties")
        assert not bad.any()


@pytest.mark.parametrize("s", range(32), ids=lambda s: f"step{s:02d}")
def test_full_block0_every_step(full_run, s):
    _full_step(full_run, 0, s)


def test_full_appended_cache_rows(full_run):
    c = full_run["cfg"]
    n = c.blocks * c.C
    close_rel("appended K rows, 4 blocks", full_run["gK"], full_run["Kc"][:, :, c.L:c.L + n], 2.0 ** -6)
    close_rel("appended V rows, 4 blocks", full_run["gV"], full_run["Vc"][:, :, c.L:c.L + n], 2.0 ** -6)


@pytest.mark.parametrize("k,s", [(k, s) for k in (1, 2, 3) for s in (0, 31)], ids=lambda v: str(v))
def test_full_later_blocks_first_and_last_step(full_run, k, s):
    _full_step(full_run, k, s)
