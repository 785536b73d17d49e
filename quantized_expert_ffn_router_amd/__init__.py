"""MI355X (gfx950) decode-time MoE expert FFN: thin Python binding of libmoe.

Every function here marshals arguments and calls the C ABI of libmoe.so
(declared in include/moe.h) under the same name; all arithmetic of the
decode path runs in the library's HIP kernels.  Device buffers are torch
tensors on the current HIP device; streams are torch streams (the current
stream by default).  There is no fallback: if libmoe.so is missing or fails
to load, importing the binding's functions raises.
"""
from ._lib import (  # noqa: F401
    MOE_Q4_K,
    MOE_Q6_K,
    MOE_Q8_0,
    Cache,
    ExpertDesc,
    MoeError,
    lib,
    lib_path,
    MOE_PLACE_ALL_CACHED,
    MOE_PLACE_FIT,
    moe_cache_plan,
    moe_placement_plan,
    moe_down_k,
    moe_expert_bytes,
    moe_expert_ffn,
    moe_group_tokens,
    moe_layer_ffn,
    moe_layer_chain_supported,
    moe_layer_forward,
    moe_layer_forward_chain,
    moe_layer_forward_noalloc,
    moe_layer_route,
    moe_repack_expert,
    moe_rmsnorm,
    moe_route_topk,
    moe_workspace_bytes,
    moe_workspace_init,
    moe_workspace_status,
    moe_set_spin_limit,
    MOE_WS_KEYS_TIMEOUT,
    MOE_WS_TOPK_TIMEOUT,
    MOE_WS_STATUS_OFFSET,
    EXPORTED,
)
