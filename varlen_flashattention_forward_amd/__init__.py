"""MI355X-native packed variable-length attention, forward and backward.

O = softmax(scale * Q K^T) V per packed segment, plus the log-sum-exp, and the
gradients dQ, dK, dV for an upstream dO, computed by hand-written gfx950 HIP
kernels behind the C ABI of include/attn_varlen.h (libattn_varlen.so). This
package is the thin Python binding over it.
"""
from ._binding import (  # noqa: F401
    CAUSAL, AttnVarlenError, BatchedLayout, BwdLayout, Layout, async_grid, async_status, async_workspace,
    async_workspace_bytes, attn_fwd, attn_varlen_bwd, attn_varlen_fwd, attn_varlen_fwd_async, attn_varlen_fwd_async_noalloc,
    attn_varlen_fwd_fp8,
    fp8_workspace_bytes, fp8_workspace_offsets,
    block_m, bwd_grid_plan, bwd_preprocess, count_tiles, decode_tile, element_offset, grid_plan, last_error, lib,
    num_tiles,
    one_stage_keys, short_stage_keys,
    segments_per_launch, validate, validate_batched, validate_bwd,
)
