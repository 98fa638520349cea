"""MI355X (gfx950) sparse Mixture-of-Experts layer forward pass.

The layer runs in hand-written HIP kernels behind the C ABI of include/moe.h
(libmoe_hip.so, built in-tree by ``python -m sparse_mixture_experts_gating_amd.build``);
``binding`` exposes the same entry points to Python with torch tensors.
"""
from .binding import (MoEError, alloc_routing, alloc_workspace, config_from_spec, load, make_config,  # noqa: F401
                      make_routing, make_weights, moe_capacity, moe_combine, moe_expert_ffn, moe_forward,
                      moe_kernel_names, moe_last_error, moe_permute, moe_permute_noalloc, moe_route, moe_route_from_logits,
                      moe_route_noisy, moe_router_losses, STAGE_LOSSES,
                      moe_timing_enable, moe_timing_read, moe_timing_reset, moe_workspace_size,
                      STAGE_FORWARD, STAGE_PERMUTE, STAGE_FFN)
