"""MI355X (gfx950) MoE expert layer: HIP kernels behind a C ABI, with a thin torch binding.

The Python names mirror the C entry points of ``include/moe.h``.
"""
from ._lib import (  # noqa: F401
    MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EWORKSPACE, MOE_EHIP, MOE_EDEVICE,
    MOE_F32, MOE_BF16, MOE_FP8_E4M3, MOE_INT8, MOE_INT4, MoEError, moe_shape, moe_weights, shape, shape_of, weights, weights_of,
    lib, moe_workspace_bytes, moe_grouped_ffn_workspace_bytes, moe_gate_topk, moe_init_routing,
    moe_grouped_ffn, moe_finalize_routing, moe_layer, moe_layer_overlap, moe_layer_profiled,
    moe_get_error, moe_router, router, moe_gate_topk_ex, moe_layer_ex,
    moe_status_str, EV_NAMES, moe_layer_plan_of, moe_grouped_ffn_gathered, moe_layer_static,
    MOE_STATIC_SCRATCH_BYTES,
)
