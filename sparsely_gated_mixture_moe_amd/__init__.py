"""MI355X-native (gfx950) forward pass of the sparsely-gated Mixture-of-Experts
layer: noisy top-k gating, stable per-expert routing, grouped expert FFNs on
the matrix cores, the gate-weighted combine and the Importance/Load balancing
losses, flat or two-level (hierarchical), and the batchwise-gated variant,
behind the C ABI of include/moe.h (libmoe_mi355x.so, built in-tree by ``python -m sparsely_gated_mixture_moe_amd.build``).

PyTorch is used only for device memory and streams.
"""
from ._binding import (  # noqa: F401
    LIB_PATH, MOE_BF16, MOE_F32, MoeBatchwiseForward, MoeDims, MoeError, MoeForward, MoeGateOpts,
    MoeHierDims, MoeHierForward, MoeHierOutputs, lib, make_dims, make_opts, moe_aux_losses,
    moe_backward, moe_batchwise_forward, moe_combine, moe_expert_ffn, moe_ffn_timing, moe_ffn_timing_read,
    moe_forward, moe_forward_noalloc, moe_gate, moe_hier_forward, moe_pack_expert_weights, moe_route,
    moe_workspace_size,
    workspace, NOALLOC_SCRATCH_BYTES,
)
