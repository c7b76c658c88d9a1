"""MI355X (gfx950) DeepSeekMoE layer forward: HIP kernels behind a C ABI.

``binding`` mirrors include/moe.h call for call; ``layer.MoELayer`` composes
the five calls into one layer forward plus the step-end bias update.
"""
from . import binding  # noqa: F401
from .binding import (  # noqa: F401
    MoEError, moe_shape, moe_route, moe_permute, moe_grouped_ffn, moe_combine, moe_bias_update,
    moe_quantize_weights, moe_workspace_bytes, moe_ffn_gate_up, moe_ffn_down, MOE_F32, MOE_BF16, MOE_F8E4M3, MOE_ROWS_DIRECT,
    MOE_ROWS_GATHER, MOE_ROWS_SEGMENT,
)
from .layer import MoELayer, StepGraph  # noqa: F401
