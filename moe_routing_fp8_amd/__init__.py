"""MI355X-native MoE dispatch path: top-k gating, token->expert map (plain, or
padded and expert-local), fused expand + per-token e4m3 cast, SwiGLU + e4m3 cast, and the combine back to
token order.

The compute lives in hand-written gfx950 HIP kernels behind the C ABI of
libmoe_fp8.so (include/moe_fp8.h); this package is its thin Python binding
(same names as the C entry points).  The seeded synthetic inputs live outside
the package, in the top-level ``workloads`` module.
"""
from ._native import (  # noqa: F401
    MOE_DISPATCH_AUTO,
    MOE_DISPATCH_SINGLE_LAUNCH,
    MOE_DISPATCH_SPLIT,
    MOE_FMT_E2M1,
    MOE_FMT_E4M3,
    CHECK_FLAGS,
    MoeError,
    check_flag_names,
    debug_enabled,
    moe_check_activations,
    moe_check_dispatch,
    moe_check_pos,
    moe_check_scores,
    moe_check_topk_idx,
    moe_combine,
    moe_dispatch,
    moe_dispatch_workspace_bytes,
    moe_cast_format,
    moe_expand_cast,
    moe_expand_cast_fp8,
    moe_expand_cast_fp8_padded,
    moe_token_map,
    moe_token_map_aligned,
    moe_token_map_aligned_rows,
    moe_token_map_noalloc,
    moe_token_map_workspace_bytes,
    moe_topk_gate,
    swiglu_cast,
    swiglu_cast_fp8,
)

__all__ = [
    "MoeError",
    "moe_topk_gate",
    "moe_token_map",
    "moe_token_map_workspace_bytes",
    "moe_token_map_noalloc",
    "moe_expand_cast_fp8",
    "swiglu_cast_fp8",
    "moe_combine",
    "moe_token_map_aligned_rows",
    "moe_token_map_aligned",
    "moe_expand_cast_fp8_padded",
    "moe_dispatch_workspace_bytes",
    "moe_dispatch",
    "MOE_DISPATCH_AUTO",
    "MOE_DISPATCH_SINGLE_LAUNCH",
    "MOE_DISPATCH_SPLIT",
    "moe_cast_format",
    "moe_expand_cast",
    "swiglu_cast",
    "MOE_FMT_E4M3",
    "MOE_FMT_E2M1",
    "moe_check_scores",
    "moe_check_topk_idx",
    "moe_check_pos",
    "moe_check_activations",
    "moe_check_dispatch",
    "CHECK_FLAGS",
    "check_flag_names",
    "debug_enabled",
]
