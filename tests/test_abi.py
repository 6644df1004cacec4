"""The C-ABI library loads, exports every entry point include/dg.h declares,
and rejects bad arguments before anything touches the GPU (these calls return
from the argument checks, so they run on a machine without a GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dg.h")


@pytest.fixture(scope="module")
def L():
    import uniform_state_discrete_amd as dg
    if not os.path.exists(dg.LIB_PATH):
        from uniform_state_discrete_amd import build
        build.build()
    return dg


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dg_[a-z_0-9]+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("dg_denoise_step", "dg_attn_bidir", "dg_vocab_selfcond", "dg_renoise",
              "dg_prefill_append", "dg_init_canvas", "dg_workspace_bytes", "dg_status_str",
              "dg_last_error"):
        assert n in names


def test_library_exports_every_declared_symbol(L):
    raw = ctypes.CDLL(L.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(raw, n)]
    assert not missing, missing


def test_status_strings(L):
    lib = L.lib()
    for code in (0, -1, -2, -3, -4):
        assert lib.dg_status_str(code).decode().startswith("DG_")
    assert b"unknown" in lib.dg_status_str(7)


FAKE = 0x10000  # never dereferenced: every call below fails its argument checks


def dims(**kw):
    import uniform_state_discrete_amd as dg
    base = dict(B=1, C=256, L=1024, cap=1024, d=2048, n_q_heads=16, n_kv_heads=8, head_dim=128,
                V=32768, dtype=dg.DG_BF16)
    base.update(kw)
    return dg.make_dims(**base)


def test_workspace_sizes(L):
    from synth import CONFIGS
    for c in CONFIGS:
        d = L.make_dims(c.B, c.C, c.L, c.cap, c.d, c.Hq, c.Hkv, c.dh, c.V,
                        L.DG_BF16 if c.dtype == "bf16" else L.DG_F32)
        assert L.dg_workspace_bytes(d) > 0, c.name
    assert L.dg_workspace_bytes(dims(n_kv_heads=7)) == 0
    assert L.dg_vocab_workspace_bytes(256, 2048, 262144, L.DG_BF16) > 256 * 2048 * 4
    assert L.dg_vocab_workspace_bytes(16, 64, 512, L.DG_F32) == 0


@pytest.mark.parametrize("B,C,Lk,Hq,Hkv,dh", [
    (1, 1, 0, 2, 1, 64), (1, 4096, 0, 16, 8, 128), (8, 256, 4096, 16, 8, 128),
    (1, 16, 1 << 20, 32, 8, 128), (2, 32768, 0, 32, 8, 128), (3, 300, 77, 12, 4, 64),
    (1, 100, 40, 6, 2, 64)])
def test_attention_plan_bounds(L, B, C, Lk, Hq, Hkv, dh):
    """The host plan of the bf16 attention (both the denoising and the causal
    split choice, which list-schedules the dispatch order) stays within 512
    key splits, sizes the workspace as whole per-split partial slabs, and
    takes little host time even for long prompts and caches."""
    import time
    d = dims(B=B, C=C, L=Lk, cap=Lk + C, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=dh)
    t0 = time.perf_counter()
    by = L.dg_attn_workspace_bytes(d)
    assert time.perf_counter() - t0 < 2.0
    slab = B * C * Hq * (dh + 2) * 4
    if by:  # no workspace when every row block fits in one split
        ns = by // slab  # the size is rounded up to 256 bytes
        assert ns * slab <= by < ns * slab + 256
        assert 2 <= ns <= 512


@pytest.mark.parametrize("C,Lc,Hq,Hkv", [(16, 32768, 32, 8), (256, 1024, 16, 8), (5, 700, 6, 2)])
def test_attention_workspace_holds_the_split_partials(L, C, Lc, Hq, Hkv):
    """Keys this long are split over several workgroups; every split leaves
    an fp32 partial row (dh outputs, max and sum) per query head, so the
    workspace holds at least two of them (one and several row blocks per KV
    head)."""
    dh = 128
    d = dims(C=C, L=Lc, cap=Lc + C, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=dh)
    assert L.dg_attn_workspace_bytes(d) >= 2 * C * Hq * (dh + 2) * 4


def _step(L, d, ws_bytes=1 << 40, null=(), weights_null=(), ws=FAKE):
    lib = L.lib()
    w = L.Weights(*[None if k in weights_null else FAKE for k in L.WEIGHT_FIELDS])
    io = L.StepIO(*[None if (k in null or k in ("selfcond_in", "lse", "mask", "x_out", "q_out",
                                                 "k_new_out", "v_new_out", "attn_out", "z_out"))
                    else FAKE for k in L.STEP_IO_FIELDS])
    return lib.dg_denoise_step(ctypes.byref(d), ctypes.byref(w), ctypes.byref(io), 0.9, 1, 1, 0,
                               ws, ws_bytes, None)


def test_step_argument_checks(L):
    lib = L.lib()
    assert _step(L, dims(), null=("H",)) == L.DG_EINVAL
    assert _step(L, dims(), weights_null=("E",)) == L.DG_EINVAL
    assert _step(L, dims(n_kv_heads=3)) == L.DG_EINVAL
    assert _step(L, dims(B=0)) == L.DG_EINVAL
    assert _step(L, dims(L=2000, cap=1024)) == L.DG_EINVAL
    assert _step(L, dims(dtype=5)) == L.DG_EINVAL
    assert _step(L, dims(head_dim=96)) == L.DG_EUNSUPPORTED
    assert _step(L, dims(d=1000)) == L.DG_EUNSUPPORTED
    assert _step(L, dims(), ws_bytes=1000) == L.DG_EWORKSPACE
    assert _step(L, dims(), ws=None) == L.DG_EWORKSPACE
    assert b"workspace" in lib.dg_last_error()
    # misaligned bf16 tensor
    w = L.Weights(FAKE, FAKE + 2, FAKE, FAKE, FAKE)
    io = L.StepIO(*[FAKE if k in ("H", "k_cache", "v_cache", "tokens_in", "tokens_out", "selfcond_out",
                                  "max_logit", "conf", "argmax") else None for k in L.STEP_IO_FIELDS])
    st = lib.dg_denoise_step(ctypes.byref(dims()), ctypes.byref(w), ctypes.byref(io), 0.9, 1, 1, 0,
                             FAKE, 1 << 40, None)
    assert st == L.DG_EINVAL and b"aligned" in lib.dg_last_error()


def test_component_argument_checks(L):
    lib = L.lib()
    vp = ctypes.c_void_p
    # vocab
    assert lib.dg_vocab_selfcond(0, 2048, 100, L.DG_BF16, *[vp(FAKE)] * 7, vp(FAKE), 1 << 40, None) == L.DG_EINVAL
    assert lib.dg_vocab_selfcond(4, 2048, 100, L.DG_BF16, None, *[vp(FAKE)] * 6, vp(FAKE), 1 << 40, None) == L.DG_EINVAL
    assert lib.dg_vocab_selfcond(4, 3000, 100, L.DG_BF16, *[vp(FAKE)] * 7, vp(FAKE), 1 << 40, None) == L.DG_EUNSUPPORTED
    assert lib.dg_vocab_selfcond(4, 2048, 100, L.DG_BF16, *[vp(FAKE)] * 7, vp(FAKE), 16, None) == L.DG_EWORKSPACE
    # attention
    d = dims()
    assert lib.dg_attn_bidir(ctypes.byref(d), None, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, FAKE, 1 << 40, None) == L.DG_EINVAL
    assert lib.dg_attn_bidir(ctypes.byref(dims(head_dim=32)), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0,
                             FAKE, 1 << 40, None) == L.DG_EUNSUPPORTED
    # renoise / init
    assert lib.dg_renoise(0, 256, 100, FAKE, FAKE, 0.5, 1, 1, 0, FAKE, None, None) == L.DG_EINVAL
    assert lib.dg_renoise(16, 16, 100, None, FAKE, 0.5, 1, 1, 0, FAKE, None, None) == L.DG_EINVAL
    assert lib.dg_init_canvas(16, 16, 0, 1, 0, FAKE, None) == L.DG_EINVAL
    # append beyond the cache capacity
    w = L.Weights(FAKE, FAKE, FAKE, FAKE, FAKE)
    assert lib.dg_prefill_append(ctypes.byref(dims(L=1000, cap=1024)), ctypes.byref(w), FAKE, FAKE, FAKE,
                                 FAKE, None, FAKE, 1 << 40, None) == L.DG_EINVAL
    assert b"cap" in lib.dg_last_error()


def test_tiled_embedding_sizes_and_checks(L):
    lib = L.lib()
    vp = ctypes.c_void_p
    # 16-id x 32-column blocks: V rounds up to a multiple of 16
    assert L.dg_tiled_embedding_bytes(262144, 2048, L.DG_BF16) == 262144 * 2048 * 2
    assert L.dg_tiled_embedding_bytes(3000, 256, L.DG_BF16) == 3008 * 256 * 2
    assert L.dg_tiled_embedding_bytes(100, 2048, L.DG_F32) == 0      # no tiled fp32 layout
    assert L.dg_tiled_embedding_bytes(100, 100, L.DG_BF16) == 0      # d % 32 != 0
    assert lib.dg_pack_embedding(100, 64, L.DG_F32, vp(FAKE), vp(FAKE * 4), None) == L.DG_EUNSUPPORTED
    assert lib.dg_pack_embedding(100, 100, L.DG_BF16, vp(FAKE), vp(FAKE * 4), None) == L.DG_EINVAL
    assert lib.dg_pack_embedding(100, 64, L.DG_BF16, None, vp(FAKE * 4), None) == L.DG_EINVAL
    assert lib.dg_pack_embedding(100, 64, L.DG_BF16, vp(FAKE), vp(FAKE + 8), None) == L.DG_EINVAL  # aligned
    assert lib.dg_pack_embedding(100, 64, L.DG_BF16, vp(FAKE), vp(FAKE + 4096), None) == L.DG_EINVAL  # overlap
    assert b"overlap" in lib.dg_last_error()


def test_block_loop_and_graph_argument_checks(L):
    lib = L.lib()
    w = L.Weights(FAKE, FAKE, FAKE, FAKE, FAKE)
    io = L.BlockIO(*[FAKE if k not in ("mask", "trace_tokens", "trace_conf", "trace_selfcond") else None
                     for k in L.BLOCK_IO_FIELDS])
    taus = (ctypes.c_float * 4)(0.5, 0.6, 0.7, 0.8)
    tp = ctypes.cast(taus, ctypes.c_void_p)
    # the cache has no room for the appended blocks
    st = lib.dg_block_loop(ctypes.byref(dims(L=1024, cap=1024 + 256)), ctypes.byref(w), ctypes.byref(io),
                           tp, 4, 2, 1, FAKE, 1 << 40, None)
    assert st == L.DG_EINVAL and b"cap" in lib.dg_last_error()
    d = dims(L=1024, cap=1024 + 2 * 256)
    assert lib.dg_block_loop(ctypes.byref(d), ctypes.byref(w), ctypes.byref(io), tp, 0, 2, 1, FAKE, 1 << 40,
                             None) == L.DG_EINVAL
    assert lib.dg_block_loop(ctypes.byref(d), ctypes.byref(w), ctypes.byref(io), None, 4, 2, 1, FAKE, 1 << 40,
                             None) == L.DG_EINVAL
    assert lib.dg_block_loop(ctypes.byref(d), ctypes.byref(w), ctypes.byref(io), tp, 4, 2, 1, FAKE, 1000,
                             None) == L.DG_EWORKSPACE
    io_nocanvas = L.BlockIO(*[FAKE if k not in ("canvas", "mask", "trace_tokens", "trace_conf", "trace_selfcond")
                              else None for k in L.BLOCK_IO_FIELDS])
    assert lib.dg_block_loop(ctypes.byref(d), ctypes.byref(w), ctypes.byref(io_nocanvas), tp, 4, 2, 1, FAKE,
                             1 << 40, None) == L.DG_EINVAL
    # graph capture needs a created stream and an output handle
    h = ctypes.c_void_p(FAKE)
    st = lib.dg_graph_capture_block_loop(ctypes.byref(d), ctypes.byref(w), ctypes.byref(io), tp, 4, 2, 1,
                                         FAKE, 1 << 40, None, ctypes.byref(h))
    assert st == L.DG_EINVAL and h.value is None and b"stream" in lib.dg_last_error()
    assert lib.dg_graph_capture_block_loop(ctypes.byref(d), ctypes.byref(w), ctypes.byref(io), tp, 4, 2, 1,
                                           FAKE, 1 << 40, FAKE, None) == L.DG_EINVAL
    assert lib.dg_graph_launch(None, None) == L.DG_EINVAL
    lib.dg_graph_destroy(None)


def test_masked_sampler_argument_checks(L):
    lib = L.lib()
    assert lib.dg_unmask(0, FAKE, FAKE, 0.5, 3, FAKE, FAKE, None, None) == L.DG_EINVAL
    assert lib.dg_unmask(16, FAKE, FAKE, 0.5, -1, FAKE, FAKE, None, None) == L.DG_EINVAL
    assert lib.dg_unmask(16, None, FAKE, 0.5, 3, FAKE, FAKE, None, None) == L.DG_EINVAL
    assert lib.dg_unmask(16, FAKE, FAKE, 0.5, 3, None, FAKE, None, None) == L.DG_EINVAL
    assert lib.dg_init_masked(16, 3, None, None) == L.DG_EINVAL
    assert lib.dg_init_masked(0, 3, FAKE, None) == L.DG_EINVAL
    w = L.Weights(FAKE, FAKE, FAKE, FAKE, FAKE)
    io = L.StepIO(*[FAKE if k in ("H", "k_cache", "v_cache", "tokens_in", "tokens_out", "selfcond_out",
                                  "max_logit", "conf", "argmax") else None for k in L.STEP_IO_FIELDS])
    for mid in (-1, 32768):   # outside [0, V)
        st = lib.dg_denoise_step_masked(ctypes.byref(dims()), ctypes.byref(w), ctypes.byref(io), 0.9, mid,
                                        FAKE, 1 << 40, None)
        assert st == L.DG_EINVAL and b"mask_id" in lib.dg_last_error()
