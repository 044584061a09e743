"""Latent-KV chunk attention (VideoMLA's streaming attention step) for MI355X.

The compute lives in libmla355.so (HIP kernels for gfx950 behind the C ABI in
include/mla.h); this package only binds it. See `_lib` for the calls and
`layer` for a device-resident layer state that strings them together.
"""
from ._lib import (  # noqa: F401
    MLA_BF16, MLA_F32, MlaError, MlaShape, EXPORTS, LIB_PATH,
    abi_version, shape_check, qabs_dim, make_shape, lib,
    rope3d_table_floats, rope3d_tables, cache_write, absorb_q, flash_workspace_bytes, flash_attend,
    flash_attend_frame_causal, flash_attend_noalloc, NOALLOC_SCRATCH_BYTES,
    up_v, chunk_attend_workspace_bytes, chunk_attend, chunk_attend_latent, chunk_attend_form, FORM_LATENT, FORM_HEADS, chunk_attend_heads_workspace_bytes, chunk_attend_heads,
    chunk_attend_frame_causal, chunk_attend_latent_frame_causal, chunk_attend_heads_frame_causal, query_project, output_project, MlaLayerWeights, layer_weights_struct,
    layer_step_workspace_bytes, layer_step, query_absorb_weights, query_project_absorbed,
)
