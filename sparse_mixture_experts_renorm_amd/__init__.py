"""MI355X (gfx950) top-k routed Mixture-of-Experts layer, forward pass.

The computation lives in the HIP library libmoe_mi355x.so behind the C ABI
of include/moe.h; this package only builds it and binds it with ctypes.
"""
from ._lib import (  # noqa: F401
    MOE_BF16, MOE_F32, MoEError, MoeOptions, declared_symbols, lib, moe_expert_ffn, moe_forward,
    moe_forward_ext, moe_forward_ext_workspace_size, moe_forward_no_alloc, moe_permute,
    moe_route, moe_route_logits, moe_router_stats, moe_workspace_size, stage_events, status_string,
    workspace,
)
