"""Sparse Mixture-of-Experts layer forward on AMD Instinct MI355X (gfx950).

The layer runs in libmoe.so (hand-written HIP kernels behind the C ABI in
include/moe.h); this package is its thin Python binding. Importing it loads
the library and raises if it is missing: there is no CPU fallback.
"""
from ._lib import (  # noqa: F401
    EXPORTED,
    LIB_PATH,
    MOE_BF16,
    MOE_F32,
    MOE_FLAG_EXPERT_CHOICE,
    MOE_FLAG_FIRST_COME,
    MOE_FLAG_HIDDEN_SPLIT,
    MOE_FLAG_IDENTITY_FALLBACK,
    MOE_FLAG_PACKED_WEIGHTS,
    MOE_FLAG_RENORM_SURVIVORS,
    MOE_FLAG_Y_F32,
    MOE_NOALLOC_SCRATCH_BYTES,
    MoeError,
    alloc_workspace,
    moe_capacity,
    moe_combine,
    moe_dispatch,
    moe_expert_ffn,
    moe_forward,
    moe_forward_noalloc,
    moe_pack_weights,
    moe_route,
    moe_routing_stats,
    moe_set_profile_events,
    moe_shared_expert,
    moe_shared_workspace_bytes,
    moe_version,
    moe_workspace_bytes,
)
