"""MI355X-native packed variable-length attention forward.

O = softmax(scale * Q K^T) V per packed segment, plus the log-sum-exp, computed
by hand-written gfx950 HIP kernels behind the C ABI of include/attn_varlen.h
(libattn_varlen.so). This package is the thin Python binding over it.
"""
from ._binding import (  # noqa: F401
    CAUSAL, AttnVarlenError, BatchedLayout, Layout, attn_fwd, attn_varlen_fwd, block_m, count_tiles,
    decode_tile, element_offset, grid_plan, last_error, lib, segments_per_launch, validate,
    validate_batched,
)
