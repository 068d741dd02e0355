"""DeepSeekMoE layer forward + aux-loss-free bias update on AMD MI355X (gfx950).

The compute lives in libmoe_mi355x.so (hand-written HIP kernels behind the C
ABI in include/moe.h); this package only builds and binds it.
"""

from .binding import (  # noqa: F401
    ExpertWeights,
    LayerShape,
    MoEError,
    alloc_routing,
    alloc_train_workspace,
    alloc_weight_grads,
    alloc_workspace,
    load_library,
    moe_forward,
    moe_backward,
    moe_forward_static,
    moe_forward_train,
    moe_quantize_act_e4m3,
    moe_quantize_weight_e4m3,
    moe_route,
    moe_update_bias,
    prepare_weights,
    status_str,
    version,
    workspace_layout,
    train_workspace_size,
    workspace_size,
)
