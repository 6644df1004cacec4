"""ctypes binding of libdg (include/dg.h): argument marshalling only.

Every function here has the name of the C entry point it calls and takes
torch tensors that already live on the GPU; it checks dtype / device /
contiguity, passes raw pointers and sizes, and raises DgError on a negative
status.  No step of the computation runs in Python.  torch is used for device
memory and streams only.
"""
import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
# DG_LIB names another build of the same library (for example the host-side
# AddressSanitizer build of `python -m uniform_state_discrete_amd.build
# --host-asan PATH`); by default the in-tree build is loaded.
LIB_PATH = os.environ.get("DG_LIB") or os.path.join(HERE, "libdg.so")

DG_F32, DG_BF16 = 0, 1
DG_OK, DG_EINVAL, DG_EUNSUPPORTED, DG_EWORKSPACE, DG_EHIP = 0, -1, -2, -3, -4


class DgError(RuntimeError):
    def __init__(self, status, where, detail):
        self.status = status
        super().__init__(f"{where}: status {status}: {detail}")


class Dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("B", "C", "L", "cap", "d", "n_q_heads", "n_kv_heads", "head_dim", "V", "dtype")]


WEIGHT_FIELDS = ("Wq", "Wk", "Wv", "Wo", "E")


class Weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in WEIGHT_FIELDS]


STEP_IO_FIELDS = ("H", "k_cache", "v_cache", "tokens_in", "selfcond_in", "tokens_out",
                  "selfcond_out", "max_logit", "conf", "lse", "argmax", "mask",
                  "x_out", "q_out", "k_new_out", "v_new_out", "attn_out", "z_out",
                  "ev_attn_begin", "ev_attn_end", "ev_vocab_begin", "ev_vocab_end")
EVENT_FIELDS = ("ev_attn_begin", "ev_attn_end", "ev_vocab_begin", "ev_vocab_end")


class StepIO(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in STEP_IO_FIELDS]


BLOCK_IO_FIELDS = ("H", "k_cache", "v_cache", "tokens", "canvas", "selfcond", "max_logit", "conf",
                   "argmax", "mask", "trace_tokens", "trace_conf", "trace_selfcond")


class BlockIO(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in BLOCK_IO_FIELDS]


_lib = None


def lib():
    """The loaded libdg.so.  Raises if it has not been built: there is no
    fallback implementation."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m uniform_state_discrete_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, sz, i32, u32, u64, f32 = (ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32,
                                      ctypes.c_uint32, ctypes.c_uint64, ctypes.c_float)
        pd = ctypes.POINTER(Dims)
        sig = {
            "dg_workspace_bytes": (sz, [pd]),
            "dg_attn_workspace_bytes": (sz, [pd]),
            "dg_vocab_workspace_bytes": (sz, [i32, i32, i32, i32]),
            "dg_tiled_embedding_bytes": (sz, [i32, i32, i32]),
            "dg_pack_embedding": (ctypes.c_int, [i32, i32, i32, vp, vp, vp]),
            "dg_denoise_step": (ctypes.c_int, [pd, ctypes.POINTER(Weights), ctypes.POINTER(StepIO),
                                               f32, u64, u32, u32, vp, sz, vp]),
            "dg_attn_bidir": (ctypes.c_int, [pd, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int, vp, sz, vp]),
            "dg_attn_bidir_noalloc": (ctypes.c_int, [pd, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int, vp]),
            "dg_vocab_selfcond": (ctypes.c_int, [i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp,
                                                 vp, sz, vp]),
            "dg_renoise": (ctypes.c_int, [i32, i32, i32, vp, vp, f32, u64, u32, u32, vp, vp, vp]),
            "dg_init_canvas": (ctypes.c_int, [i32, i32, i32, u64, u32, vp, vp]),
            "dg_prefill_append": (ctypes.c_int, [pd, ctypes.POINTER(Weights), vp, vp, vp, vp, vp,
                                                 vp, sz, vp]),
            "dg_block_loop": (ctypes.c_int, [pd, ctypes.POINTER(Weights), ctypes.POINTER(BlockIO), vp,
                                             i32, i32, u64, vp, sz, vp]),
            "dg_graph_capture_block_loop": (ctypes.c_int, [pd, ctypes.POINTER(Weights), ctypes.POINTER(BlockIO),
                                                           vp, i32, i32, u64, vp, sz, vp,
                                                           ctypes.POINTER(ctypes.c_void_p)]),
            "dg_graph_launch": (ctypes.c_int, [vp, vp]),
            "dg_graph_destroy": (None, [vp]),
            "dg_unmask": (ctypes.c_int, [i32, vp, vp, f32, i32, vp, vp, vp, vp]),
            "dg_init_masked": (ctypes.c_int, [i32, i32, vp, vp]),
            "dg_denoise_step_masked": (ctypes.c_int, [pd, ctypes.POINTER(Weights), ctypes.POINTER(StepIO),
                                                      f32, i32, vp, sz, vp]),
            "dg_test_set_group_wait": (None, [i32]),
            "dg_status_str": (ctypes.c_char_p, [ctypes.c_int]),
            "dg_last_error": (ctypes.c_char_p, []),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(status, where):
    if status != DG_OK:
        L = lib()
        raise DgError(status, where, f"{L.dg_status_str(status).decode()} -- {L.dg_last_error().decode()}")


def dtype_code(t):
    if t == torch.bfloat16:
        return DG_BF16
    if t == torch.float32:
        return DG_F32
    raise TypeError(f"unsupported dtype {t}")


def ptr(t, dtype=None):
    """Device pointer of a contiguous GPU tensor (None -> NULL)."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"expected {dtype}, got {t.dtype}")
    return t.data_ptr()


def event_handle(ev):
    """hipEvent_t of a torch.cuda.Event (None -> NULL).  torch creates the
    underlying event lazily, so the event must have been recorded once."""
    if ev is None:
        return None
    h = int(ev.cuda_event)
    if h == 0:
        raise ValueError("torch.cuda.Event has no HIP event yet: record it once first")
    return h


def stream_handle(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def make_dims(B, C, L, cap, d, n_q_heads, n_kv_heads, head_dim, V, dtype):
    code = dtype if isinstance(dtype, int) else dtype_code(dtype)
    return Dims(B, C, L, cap, d, n_q_heads, n_kv_heads, head_dim, V, code)


def workspace(nbytes, device="cuda"):
    return torch.empty(max(1, int(nbytes)), dtype=torch.uint8, device=device)


# ---- entry points ----------------------------------------------------------------

def dg_workspace_bytes(dims):
    return lib().dg_workspace_bytes(ctypes.byref(dims))


def dg_attn_workspace_bytes(dims):
    return lib().dg_attn_workspace_bytes(ctypes.byref(dims))


def dg_vocab_workspace_bytes(rows, d, V, dtype):
    return lib().dg_vocab_workspace_bytes(rows, d, V, dtype if isinstance(dtype, int) else dtype_code(dtype))


def dg_tiled_embedding_bytes(V, d, dtype):
    return lib().dg_tiled_embedding_bytes(int(V), int(d), dtype if isinstance(dtype, int) else dtype_code(dtype))


def dg_pack_embedding(V, d, E, E_tiled, stream=None):
    st = lib().dg_pack_embedding(int(V), int(d), dtype_code(E.dtype), ptr(E), ptr(E_tiled), stream_handle(stream))
    _check(st, "dg_pack_embedding")


def tiled_embedding(E, stream=None):
    """A new device tensor holding bf16 table E[V][d] in the tiled layout the
    vocabulary head reads (dg_pack_embedding); None for a float32 table."""
    if E.dtype != torch.bfloat16:
        return None
    V, d = E.shape
    n = dg_tiled_embedding_bytes(V, d, E.dtype)
    if n == 0:
        raise DgError(DG_EUNSUPPORTED, "tiled_embedding", f"no tiled layout for V={V} d={d}")
    out = torch.empty(n // 2, dtype=torch.bfloat16, device=E.device)
    dg_pack_embedding(V, d, E, out, stream)
    return out


def model_embedding(E, stream=None):
    """The embedding table in the form dg_weights.E takes: the tiled table
    for a bf16 E[V][d] (a new tensor; the row-major one can then be freed),
    E itself for float32."""
    return tiled_embedding(E, stream) if E.dtype == torch.bfloat16 else E


_FLOAT_IO = ("H", "k_cache", "v_cache", "selfcond_in", "selfcond_out", "x_out", "q_out",
             "k_new_out", "v_new_out", "attn_out", "z_out")


def _check_float_dtype(dims, tensors):
    want = torch.bfloat16 if dims.dtype == DG_BF16 else torch.float32
    for name, t in tensors:
        if t is not None and t.dtype != want:
            raise TypeError(f"{name}: expected {want}, got {t.dtype}")


def dg_denoise_step(dims, weights, io, tau, seed, t, block, ws, stream=None):
    """weights: dict Wq, Wk, Wv, Wo, E (E as model_embedding returns it: the
    tiled table for bf16); io: dict with the dg_step_io fields (missing keys
    -> NULL).  ws: uint8 workspace tensor."""
    _check_float_dtype(dims, [(k, weights.get(k)) for k in WEIGHT_FIELDS] +
                       [(k, io.get(k)) for k in _FLOAT_IO])
    for k in ("tokens_in", "tokens_out", "argmax"):
        if io.get(k) is not None and io[k].dtype != torch.int32:
            raise TypeError(f"{k}: expected torch.int32")
    w = Weights(*(ptr(weights.get(k)) for k in WEIGHT_FIELDS))
    s = StepIO(*((event_handle(io.get(k)) if k in EVENT_FIELDS else ptr(io.get(k))) for k in STEP_IO_FIELDS))
    st = lib().dg_denoise_step(ctypes.byref(dims), ctypes.byref(w), ctypes.byref(s), float(tau),
                               int(seed), int(t), int(block), ptr(ws), ws.numel() if ws is not None else 0,
                               stream_handle(stream))
    _check(st, "dg_denoise_step")


def dg_attn_bidir(dims, q, k_cache, v_cache, k_new, v_new, out, lse_out, causal, ws, stream=None):
    st = lib().dg_attn_bidir(ctypes.byref(dims), ptr(q), ptr(k_cache), ptr(v_cache), ptr(k_new),
                             ptr(v_new), ptr(out), ptr(lse_out, torch.float32), int(bool(causal)),
                             ptr(ws), ws.numel() if ws is not None else 0, stream_handle(stream))
    _check(st, "dg_attn_bidir")


# DG_ATTN_NOALLOC_MAX_BYTES of include/dg.h: the built-in scratch of dg_attn_bidir_noalloc
ATTN_NOALLOC_MAX_BYTES = 64 << 20


def dg_attn_bidir_noalloc(dims, q, k_cache, v_cache, k_new, v_new, out, lse_out, causal, stream=None):
    st = lib().dg_attn_bidir_noalloc(ctypes.byref(dims), ptr(q), ptr(k_cache), ptr(v_cache), ptr(k_new),
                                     ptr(v_new), ptr(out), ptr(lse_out, torch.float32), int(bool(causal)),
                                     stream_handle(stream))
    _check(st, "dg_attn_bidir_noalloc")


def dg_test_set_group_wait(polls):
    """Test hook: the start-handshake poll bound of the CU-group vocabulary
    head (0: every group computes solo; negative: the default)."""
    lib().dg_test_set_group_wait(int(polls))


def dg_vocab_selfcond(rows, d, V, z, E, max_logit, argmax, conf, lse, selfcond, ws, stream=None):
    """E: the row-major float32 table, or for bf16 the tiled table of
    tiled_embedding."""
    st = lib().dg_vocab_selfcond(int(rows), int(d), int(V), dtype_code(z.dtype), ptr(z), ptr(E),
                                 ptr(max_logit, torch.float32), ptr(argmax, torch.int32),
                                 ptr(conf, torch.float32), ptr(lse, torch.float32), ptr(selfcond),
                                 ptr(ws), ws.numel() if ws is not None else 0, stream_handle(stream))
    _check(st, "dg_vocab_selfcond")


def dg_renoise(rows, canvas, V, argmax, conf, tau, seed, t, block, tokens_out, mask_out, stream=None):
    st = lib().dg_renoise(int(rows), int(canvas), int(V), ptr(argmax, torch.int32),
                          ptr(conf, torch.float32), float(tau), int(seed), int(t), int(block),
                          ptr(tokens_out, torch.int32), ptr(mask_out, torch.uint8), stream_handle(stream))
    _check(st, "dg_renoise")


def dg_init_canvas(rows, canvas, V, seed, block, tokens_out, stream=None):
    st = lib().dg_init_canvas(int(rows), int(canvas), int(V), int(seed), int(block),
                              ptr(tokens_out, torch.int32), stream_handle(stream))
    _check(st, "dg_init_canvas")


def dg_prefill_append(dims, weights, H, tokens_final, k_cache, v_cache, attn_out, ws, stream=None):
    w = Weights(*(ptr(weights.get(k)) for k in WEIGHT_FIELDS))
    st = lib().dg_prefill_append(ctypes.byref(dims), ctypes.byref(w), ptr(H), ptr(tokens_final, torch.int32),
                                 ptr(k_cache), ptr(v_cache), ptr(attn_out), ptr(ws),
                                 ws.numel() if ws is not None else 0, stream_handle(stream))
    _check(st, "dg_prefill_append")


def _block_args(dims, weights, io, taus, steps):
    _check_float_dtype(dims, [(k, weights.get(k)) for k in WEIGHT_FIELDS] +
                       [(k, io.get(k)) for k in ("H", "k_cache", "v_cache", "selfcond", "trace_selfcond")])
    for k in ("tokens", "canvas", "argmax", "trace_tokens"):
        if io.get(k) is not None and io[k].dtype != torch.int32:
            raise TypeError(f"{k}: expected torch.int32")
    if len(taus) != steps:
        raise ValueError(f"need {steps} thresholds, got {len(taus)}")
    w = Weights(*(ptr(weights.get(k)) for k in WEIGHT_FIELDS))
    b = BlockIO(*(ptr(io.get(k)) for k in BLOCK_IO_FIELDS))
    t = (ctypes.c_float * steps)(*[float(x) for x in taus])
    return w, b, t


def dg_block_loop(dims, weights, io, taus, steps, blocks, seed, ws, stream=None):
    """io: dict with the dg_block_io fields (missing keys -> NULL); taus: the
    `steps` thresholds of a block (host floats)."""
    w, b, t = _block_args(dims, weights, io, taus, steps)
    st = lib().dg_block_loop(ctypes.byref(dims), ctypes.byref(w), ctypes.byref(b), ctypes.cast(t, ctypes.c_void_p),
                             int(steps), int(blocks), int(seed), ptr(ws), ws.numel() if ws is not None else 0,
                             stream_handle(stream))
    _check(st, "dg_block_loop")


class Graph:
    """An instantiated HIP graph of the block loop (dg_graph).  Holds the
    tensors it was captured on, so they outlive it."""

    def __init__(self, handle, keep):
        self._h = handle
        self._keep = keep

    def launch(self, stream=None):
        _check(lib().dg_graph_launch(self._h, stream_handle(stream)), "dg_graph_launch")

    def close(self):
        if self._h:
            lib().dg_graph_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def dg_graph_capture_block_loop(dims, weights, io, taus, steps, blocks, seed, ws, stream):
    """Capture the block loop on `stream` (a torch.cuda.Stream, not the NULL
    stream) into a Graph; nothing runs until Graph.launch."""
    w, b, t = _block_args(dims, weights, io, taus, steps)
    h = ctypes.c_void_p()
    st = lib().dg_graph_capture_block_loop(ctypes.byref(dims), ctypes.byref(w), ctypes.byref(b),
                                           ctypes.cast(t, ctypes.c_void_p), int(steps), int(blocks), int(seed),
                                           ptr(ws), ws.numel() if ws is not None else 0, stream_handle(stream),
                                           ctypes.byref(h))
    _check(st, "dg_graph_capture_block_loop")
    return Graph(h.value, (dict(weights), dict(io), ws))


def dg_unmask(rows, argmax, conf, tau, mask_id, tokens_in, tokens_out, commit_out, stream=None):
    st = lib().dg_unmask(int(rows), ptr(argmax, torch.int32), ptr(conf, torch.float32), float(tau), int(mask_id),
                         ptr(tokens_in, torch.int32), ptr(tokens_out, torch.int32), ptr(commit_out, torch.uint8),
                         stream_handle(stream))
    _check(st, "dg_unmask")


def dg_init_masked(rows, mask_id, tokens_out, stream=None):
    st = lib().dg_init_masked(int(rows), int(mask_id), ptr(tokens_out, torch.int32), stream_handle(stream))
    _check(st, "dg_init_masked")


def dg_denoise_step_masked(dims, weights, io, tau, mask_id, ws, stream=None):
    """As dg_denoise_step, with the masked sampler; io["mask"] receives the
    commit flags."""
    _check_float_dtype(dims, [(k, weights.get(k)) for k in WEIGHT_FIELDS] +
                       [(k, io.get(k)) for k in _FLOAT_IO])
    for k in ("tokens_in", "tokens_out", "argmax"):
        if io.get(k) is not None and io[k].dtype != torch.int32:
            raise TypeError(f"{k}: expected torch.int32")
    w = Weights(*(ptr(weights.get(k)) for k in WEIGHT_FIELDS))
    s = StepIO(*((event_handle(io.get(k)) if k in EVENT_FIELDS else ptr(io.get(k))) for k in STEP_IO_FIELDS))
    st = lib().dg_denoise_step_masked(ctypes.byref(dims), ctypes.byref(w), ctypes.byref(s), float(tau),
                                      int(mask_id), ptr(ws), ws.numel() if ws is not None else 0,
                                      stream_handle(stream))
    _check(st, "dg_denoise_step_masked")
