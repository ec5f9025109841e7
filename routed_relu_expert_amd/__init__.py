"""routed_relu_expert_amd: the forward pass of a routed ReLU^2 MoE layer
(Nemotron-style) as hand-written HIP kernels for AMD MI355X (gfx950),
behind the C ABI of libmoe (include/moe.h).

The binding loads libmoe.so on first use; see ``_lib`` for the calls
(moe_pack_weight, moe_quantize_fp8, moe_router_logits, moe_route,
moe_dispatch, moe_experts, moe_experts_fp8, moe_experts_mxfp4, moe_combine,
moe_layer_forward, moe_layer_backward, moe_quantize_mxfp4, moe_workspace_routing).
"""
from ._lib import (  # noqa: F401
    EXPORTS, LIB_PATH, MOE_BF16, MOE_F32, MOE_FP8_E4M3, MOE_FLAG_ACCUMULATE_OUT, MOE_FLAG_FP8_EXPERTS,
    MOE_FLAG_PRENORM_RESIDUAL, MOE_FLAG_ZERO_SKIP_DOWN,
    MOE_PACK_NEURON_MAJOR, MOE_PACK_OUT_IN, PACK_KIND, STAGES, LayerDesc, LayerWeights, MoeError, device_weights, lib, make_desc,
    make_weights_struct, moe_combine, moe_dispatch, moe_experts, moe_layer_forward, moe_route,
    moe_capacity_slots, moe_dispatch_capacity, moe_experts_fp8, moe_pack_weight, moe_quantize_fp8,
    moe_rmsnorm, moe_router_logits, moe_workspace_size, LayerGrads, LayerWeightsBwd, device_weights_bwd,
    moe_backward_workspace_size, moe_layer_backward, moe_layer_forward_train, BWD_STAGES,
    MOE_MXFP4, MOE_FLAG_MXFP4_EXPERTS, moe_quantize_mxfp4, moe_experts_mxfp4, fp4_transpose,
    moe_workspace_routing, routing_views, RoutingLayout, moe_layer_forward_noalloc, NOALLOC_SCRATCH_BYTES,
    MOE_FLAG_MXFP8_ACTIVATIONS, moe_quantize_mxfp8,
)
