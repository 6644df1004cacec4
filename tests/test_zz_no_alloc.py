"""dg_attn_bidir_noalloc (the attention entry point that allocates nothing:
its split partials live in the library's built-in scratch) against
dg_attn_bidir with a caller workspace, bit for bit, on two calls in a row, the
second on a smaller input, plus the oracle on the smaller case.  Collected
last, so a failure here hides no other test."""
import numpy as np
import pytest
import torch

from oracle import step
from tests.gpu_util import ATOL, RELF, as_f64, close, dev, f64, need_gpu, say, stored

pytestmark = pytest.mark.gpu


def _inputs(B, C, L, cap, Hq, Hkv, dh, seed):
    r = np.random.default_rng(seed)
    q = stored(r.standard_normal((B, C, Hq, dh)), "bf16")
    Kc = stored(r.standard_normal((B, Hkv, cap, dh)), "bf16")
    Vc = stored(r.standard_normal((B, Hkv, cap, dh)), "bf16")
    Kn = stored(r.standard_normal((B, C, Hkv, dh)), "bf16")
    Vn = stored(r.standard_normal((B, C, Hkv, dh)), "bf16")
    return q, Kc, Vc, Kn, Vn


def _both(B, C, L, Hq, Hkv, dh, causal, seed):
    """Runs the shape through dg_attn_bidir (fresh workspace) and through
    dg_attn_bidir_noalloc; returns both outputs and the inputs."""
    import uniform_state_discrete_amd as dg
    cap = L + 3
    arrs = _inputs(B, C, L, cap, Hq, Hkv, dh, seed)
    q, Kc, Vc, Kn, Vn = (dev(x) for x in arrs)
    dims = dg.make_dims(B, C, L, cap, 64, Hq, Hkv, dh, 1, dg.DG_BF16)
    need = dg.dg_attn_workspace_bytes(dims)
    assert 0 < need <= dg.ATTN_NOALLOC_MAX_BYTES
    outs = []
    for noalloc in (False, True):
        out = torch.full((B, C, Hq, dh), float("nan"), dtype=torch.bfloat16, device="cuda")
        lse = torch.full((B, C, Hq), float("nan"), dtype=torch.float32, device="cuda")
        if noalloc:
            dg.dg_attn_bidir_noalloc(dims, q, Kc, Vc, Kn, Vn, out, lse, causal)
        else:
            ws = dg.workspace(need)
            dg.dg_attn_bidir(dims, q, Kc, Vc, Kn, Vn, out, lse, causal, ws)
        torch.cuda.synchronize()
        outs.append((out, lse))
    return outs, arrs


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()
    import uniform_state_discrete_amd as dg
    dg.lib()
    yield


def test_noalloc_attention_equals_workspace_attention_twice():
    # first call: the 256-token denoising shape over an 8192-row cache (8 key
    # splits, 17 MB of partials); second call: a smaller causal shape whose
    # partials cover only part of what the first call left in the scratch
    for (B, C, L, Hq, Hkv, dh, causal, seed) in [(1, 256, 8192, 16, 8, 128, 0, 1),
                                                 (1, 100, 700, 6, 2, 128, 1, 2)]:
        say(f"no-alloc attention B={B} C={C} L={L} Hq={Hq} Hkv={Hkv} causal={causal}")
        (ref, got), arrs = _both(B, C, L, Hq, Hkv, dh, causal, seed)
        assert torch.equal(got[0], ref[0]), "O differs from dg_attn_bidir"
        assert torch.equal(got[1], ref[1]), "lse differs from dg_attn_bidir"
        if C <= 100:
            q, Kc, Vc, Kn, Vn = (as_f64(x, "bf16") for x in arrs)
            rO, rlse = step.attention(q, Kc, Vc, Kn, Vn, L, causal=bool(causal), dtype="bf16")
            close("O vs oracle", f64(got[0]), rO, ATOL["bf16"], RELF["bf16"])
            close("lse vs oracle", f64(got[1]), rlse, ATOL["bf16"])


def test_noalloc_attention_rejects_shapes_beyond_its_scratch():
    """The causal prefill of a 4096-token prompt needs 65 MiB of partials, more
    than the 64 MiB scratch: the call is refused before anything is enqueued
    (the tensors are full size all the same)."""
    import uniform_state_discrete_amd as dg
    B, C, L, Hq, Hkv, dh = 1, 4096, 0, 16, 8, 128
    dims = dg.make_dims(B, C, L, L + C, 64, Hq, Hkv, dh, 1, dg.DG_BF16)
    assert dg.dg_attn_workspace_bytes(dims) > dg.ATTN_NOALLOC_MAX_BYTES
    bf = dict(dtype=torch.bfloat16, device="cuda")
    q = torch.zeros((B, C, Hq, dh), **bf)
    Kc = torch.zeros((B, Hkv, L + C, dh), **bf)
    kn = torch.zeros((B, C, Hkv, dh), **bf)
    out = torch.zeros((B, C, Hq, dh), **bf)
    with pytest.raises(dg.DgError) as ei:
        dg.dg_attn_bidir_noalloc(dims, q, Kc, Kc, kn, kn, out, None, 1)
    assert ei.value.status == dg.DG_EWORKSPACE
