"""MI355X-native (gfx950) AWQ W4A16 hot path: quantize + pack, activation-aware scale
search, and the W4A16 linear, as hand-written HIP kernels behind a small C ABI
(include/awq.h, lib/libawq_mi355x.so)."""

from ._abi import AwqError, load as load_library  # noqa: F401
from .awq import (  # noqa: F401
    PackedLinear, SearchResult, SearchWorkspace, activation_stats, alloc_packed, apply_inverse_scale,
    candidate_scales, clip_search, gemv_max_m, linear_w4a16, linear_w4a16_gated_silu, quantize_pack,
    search_scales,
)
