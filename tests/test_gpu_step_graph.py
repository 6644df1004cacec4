"""The chained denoise steps captured into one HIP graph (as bench.py times
them) give the same bits as the eager steps: the graph is replayed several
times, each time from the same starting canvas restored by eager work with a
synchronisation between replays, and every replay's tokens, confidences and
self-conditioning vector are compared with the eager run."""
import pytest
import torch

from synth import config_by_name, Config, gen_problem, tau_schedule
from tests.gpu_util import need_gpu, say

pytestmark = pytest.mark.gpu

SMALL = Config("graph_small_bf16", 93, B=2, C=40, L=70, d=256, Hq=4, Hkv=2, dh=64, V=3000,
               dtype="bf16", steps=4, blocks=1, tau=(0.6, 0.6))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()
    import uniform_state_discrete_amd as dg
    dg.lib()
    yield


@pytest.mark.parametrize("cfg", [SMALL, config_by_name("canvas256_L8192_d2048_V262144"),
                                 config_by_name("canvas256_L32768_d4096_V262144")], ids=lambda c: c.name)
def test_step_graph_replays_equal_eager(cfg):
    import uniform_state_discrete_amd as dg
    say(f"step graph {cfg.name}")
    p = gen_problem(cfg)
    W = {k: dg.to_device(v) for k, v in p.W.items()}
    W["E"] = dg.model_embedding(dg.to_device(p.E))
    Kc, Vc, H = dg.to_device(p.Kc), dg.to_device(p.Vc), dg.to_device(p.H[0])
    del p
    dims = dg.make_dims(cfg.B, cfg.C, cfg.L, cfg.cap, cfg.d, cfg.Hq, cfg.Hkv, cfg.dh, cfg.V, dg.DG_BF16)
    ws = dg.workspace(dg.dg_workspace_bytes(dims))
    R = cfg.R
    tok = [torch.empty((cfg.B, cfg.C), dtype=torch.int32, device="cuda") for _ in range(2)]
    sc = [torch.zeros((cfg.B, cfg.C, cfg.d), dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    conf = [torch.empty(R, device="cuda") for _ in range(4)]
    stats = dict(max_logit=torch.empty(R, device="cuda"), lse=torch.empty(R, device="cuda"),
                 argmax=torch.empty(R, dtype=torch.int32, device="cuda"),
                 mask=torch.empty(R, dtype=torch.uint8, device="cuda"))
    taus = tau_schedule(cfg)
    steps = 4
    start = torch.empty((cfg.B, cfg.C), dtype=torch.int32, device="cuda")
    dg.dg_init_canvas(R, cfg.C, cfg.V, cfg.seed, 0, start)

    def run(s, strm):
        a, b = s % 2, (s + 1) % 2
        io = dict(H=H, k_cache=Kc, v_cache=Vc, tokens_in=tok[a], selfcond_in=None if s == 0 else sc[a],
                  tokens_out=tok[b], selfcond_out=sc[b], conf=conf[s], **stats)
        dg.dg_denoise_step(dims, W, io, taus[s], cfg.seed, s + 1, 0, ws, strm)

    def outputs():
        return [tok[steps % 2].clone(), sc[steps % 2].clone()] + [c.clone() for c in conf]

    tok[0].copy_(start)
    for s in range(steps):
        run(s, torch.cuda.current_stream())
    torch.cuda.synchronize()
    eager = outputs()

    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=cap, capture_error_mode="relaxed"):
        for s in range(steps):
            run(s, cap)
    torch.cuda.synchronize()
    for rep in range(3):
        for t in [tok[1], sc[0], sc[1]] + conf:   # eager work between the replays
            t.zero_()
        tok[0].copy_(start)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = outputs()
        for name, u, v in zip(["tokens", "S"] + [f"conf step {s}" for s in range(steps)], got, eager):
            assert torch.equal(u, v), f"replay {rep}: {name} differs from the eager steps"
        say(f"replay {rep} equals the eager steps")
