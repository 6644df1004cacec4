"""The masked-diffusion sampler ("Diffusione mascherata") on the GPU against
the oracle: dg_unmask bit for bit, and dg_denoise_step_masked in lockstep
from a fully masked canvas (step s of the oracle consumes the GPU's tokens and
self-conditioning vector of step s-1)."""
import numpy as np
import pytest
import torch

from oracle import step
from synth import config_by_name, Config, gen_problem
from tests.gpu_util import ATOL, RELF, TAU_BAND, argmax_match, as_f64, close, f64, need_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()
    import uniform_state_discrete_amd as dg
    dg.lib()
    yield


@pytest.mark.parametrize("rows,V", [(1, 7), (37, 100), (256, 32768), (2048 * 8 + 5, 262144)])
@pytest.mark.parametrize("alias", [False, True])
def test_unmask_bit_exact(rows, V, alias):
    import uniform_state_discrete_amd as dg
    rng = np.random.default_rng(rows + V)
    mask_id = V - 1
    a = rng.integers(0, V, rows).astype(np.int32)
    a[rng.uniform(size=rows) < 0.05] = mask_id          # some predictions are the mask id
    c = rng.uniform(1.0 / V, 1.0, rows).astype(np.float32)
    tau = 0.6
    c[rng.uniform(size=rows) < 0.05] = np.float32(tau)  # exactly at the threshold
    x = np.where(rng.uniform(size=rows) < 0.7, mask_id, rng.integers(0, V, rows)).astype(np.int32)
    ref_x, ref_k = step.unmask(a, c.astype(np.float64), tau, x, mask_id)
    ta, tc, tx = (torch.from_numpy(v).cuda() for v in (a, c, x))
    out = tx if alias else torch.empty_like(tx)
    k = torch.empty(rows, dtype=torch.uint8, device="cuda")
    dg.dg_unmask(rows, ta, tc, tau, mask_id, tx, out, k)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), ref_x)
    assert np.array_equal(k.cpu().numpy(), ref_k)
    dg.dg_init_masked(rows, mask_id, out)
    torch.cuda.synchronize()
    assert (out.cpu().numpy() == mask_id).all()


SMALL_BF16 = Config("masked_small_bf16", 94, B=2, C=40, L=70, d=256, Hq=4, Hkv=2, dh=64, V=3000,
                    dtype="bf16", steps=4, blocks=1, tau=(0.5, 0.5))


def tiny(cfg, name, idx, tau):
    return Config(name, idx, cfg.B, cfg.C, cfg.L, cfg.d, cfg.Hq, cfg.Hkv, cfg.dh, cfg.V, cfg.dtype, 4, 1,
                  (tau, tau))


def full_vocab(steps):
    """The full-vocabulary workload (V = 262144, 8192-row cache) with tau 0.8
    and the given number of steps."""
    c = config_by_name("canvas256_L8192_d2048_V262144")
    return Config("masked_v262144", c.index, c.B, c.C, c.L, c.d, c.Hq, c.Hkv, c.dh, c.V, c.dtype, steps, 1,
                  (0.8, 0.8))


@pytest.mark.parametrize("cfg", [tiny(config_by_name("tiny_c16_L32_d64_V512_f32"), "masked_tiny", 95, 0.3), SMALL_BF16,
                                 tiny(config_by_name("canvas256_L1024_d2048_V32768"), "masked_v32768", 96, 0.9),
                                 full_vocab(2)], ids=lambda c: c.name)
def test_masked_step_lockstep(cfg):
    import uniform_state_discrete_amd as dg
    say(f"masked step lockstep {cfg.name}")
    p = gen_problem(cfg)
    f = lambda a: as_f64(a, cfg.dtype)
    E, H, Kc, Vc = f(p.E), f(p.H[0]), f(p.Kc), f(p.Vc)
    W = {k: f(v) for k, v in p.W.items()}
    Wd = {k: dg.to_device(v) for k, v in p.W.items()}
    Wd["E"] = dg.model_embedding(dg.to_device(p.E))
    dt = dg.DG_BF16 if cfg.dtype == "bf16" else dg.DG_F32
    dims = dg.make_dims(cfg.B, cfg.C, cfg.L, cfg.cap, cfg.d, cfg.Hq, cfg.Hkv, cfg.dh, cfg.V, dt)
    ws = dg.workspace(dg.dg_workspace_bytes(dims))
    fdt = Wd["E"].dtype
    R = cfg.R
    mask_id = cfg.V - 1
    x = torch.empty((cfg.B, cfg.C), dtype=torch.int32, device="cuda")
    dg.dg_init_masked(R, mask_id, x)
    S = None
    masked = [R]
    for s in range(cfg.steps):
        io = dict(H=dg.to_device(p.H[0]), k_cache=dg.to_device(p.Kc), v_cache=dg.to_device(p.Vc),
                  tokens_in=x, selfcond_in=S, tokens_out=torch.empty_like(x),
                  selfcond_out=torch.empty((cfg.B, cfg.C, cfg.d), dtype=fdt, device="cuda"),
                  max_logit=torch.empty(R, device="cuda"), conf=torch.empty(R, device="cuda"),
                  lse=torch.empty(R, device="cuda"), argmax=torch.empty(R, dtype=torch.int32, device="cuda"),
                  mask=torch.empty(R, dtype=torch.uint8, device="cuda"),
                  z_out=torch.empty((R, cfg.d), dtype=fdt, device="cuda"))
        dg.dg_denoise_step_masked(dims, Wd, io, cfg.tau[0], mask_id, ws)
        torch.cuda.synchronize()
        xin = x.cpu().numpy()
        ref = step.denoise_step_masked(H, E, W, Kc, Vc, cfg.L, xin, None if S is None else f64(S),
                                       cfg.tau[0], mask_id, cfg.dtype)
        tag = f"step {s}"
        close(f"{tag} c", f64(io["conf"]), ref["c"], ATOL[cfg.dtype])
        close(f"{tag} S", f64(io["selfcond_out"]).reshape(R, -1), ref["S"].reshape(R, -1), ATOL[cfg.dtype],
              RELF[cfg.dtype], bf16_ulp=cfg.dtype == "bf16")
        gap = ref["gap"]
        argmax_match(f"{tag} argmax", io["argmax"].cpu().numpy(), ref["a"], gap, ref["m"])
        tie = gap < 1e-3 * np.maximum(1.0, np.abs(ref["m"]))
        band = (np.abs(ref["c"] - float(np.float32(cfg.tau[0]))) < TAU_BAND) | tie
        got_x = io["tokens_out"].cpu().numpy().reshape(-1)
        got_k = io["mask"].cpu().numpy()
        bad = ((got_x != ref["x_new"].reshape(-1)) | (got_k != ref["commit"].reshape(-1))) & ~band
        say(f"{tag}: {int(bad.sum())} token/commit mismatches, {int(band.sum())} excluded, "
            f"{int(ref['commit'].sum())} committed")
        assert not bad.any()
        # locked positions never change, on the GPU's own inputs
        locked = xin.reshape(-1) != mask_id
        assert np.array_equal(got_x[locked], xin.reshape(-1)[locked])
        x, S = io["tokens_out"], io["selfcond_out"]
        masked.append(int((got_x == mask_id).sum()))
    say(f"masked positions per step: {masked}")
    assert all(b <= a for a, b in zip(masked, masked[1:]))
