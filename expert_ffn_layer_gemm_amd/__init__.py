"""MI355X-native MoE expert-FFN layer: ctypes binding of libmoe.so (HIP kernels for gfx950)."""
from ._binding import (  # noqa: F401
    MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP,
    MOE_BF16, MOE_FP8_E4M3_BLOCK128, MOE_MXFP8, MoeShape, MoeError, lib, make_shape, shape_of,
    moe_last_error, moe_abi_version, moe_forward_workspace_bytes, moe_workspace_bytes,
    moe_ffn_workspace_bytes,
    moe_route_workspace_bytes, moe_route, moe_route_from_logits,
    moe_permute_workspace_bytes, moe_permute, moe_grouped_ffn, moe_combine, moe_forward,
    moe_forward_noalloc, NOALLOC_SCRATCH_BYTES,
    moe_profile_start, moe_profile_count, moe_profile_read, moe_profile_stop,
)
