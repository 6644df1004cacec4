"""MI355X-native canvas denoise step of uniform-state text diffusion.

The computation lives in libdg.so (hand-written HIP kernels for gfx950 behind
the C ABI of include/dg.h); this package is its Python binding.  Importing it
does not touch the GPU; the library is loaded on first use and a missing
library is an error, never a fallback.
"""
from ._lib import (  # noqa: F401
    DG_BF16, DG_F32, DG_OK, DG_EINVAL, DG_EUNSUPPORTED, DG_EWORKSPACE, DG_EHIP,
    DgError, Dims, Weights, StepIO, STEP_IO_FIELDS, LIB_PATH,
    lib, make_dims, workspace, ptr, dtype_code, stream_handle,
    dg_workspace_bytes, dg_attn_workspace_bytes, dg_vocab_workspace_bytes,
    dg_denoise_step, dg_attn_bidir, dg_vocab_selfcond, dg_renoise, dg_init_canvas,
    dg_prefill_append, dg_tiled_embedding_bytes, dg_pack_embedding, tiled_embedding, model_embedding,
    WEIGHT_FIELDS, BlockIO, BLOCK_IO_FIELDS, Graph, dg_block_loop, dg_graph_capture_block_loop,
    dg_unmask, dg_init_masked, dg_denoise_step_masked,
    dg_attn_bidir_noalloc, ATTN_NOALLOC_MAX_BYTES, dg_test_set_group_wait,
)
from .device import to_device, torch_dtype  # noqa: F401
