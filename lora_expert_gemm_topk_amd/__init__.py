"""Fused MoE-LoRA layer for MI355X (gfx950).

The layer (top-k routing with shared-expert slots, expert/adapter alignment,
grouped gate_up/SwiGLU/down GEMMs with each token's LoRA shrink and expand
fused in, weighted top-k combine) runs entirely in the HIP kernels of
``libmoelora.so``; ``moe_lora`` is its ctypes binding and ``synth`` draws the
seeded synthetic inputs.
"""
from .moe_lora import (  # noqa: F401
    MOE_LORA_BAD_ADAPTER, MOE_LORA_BAD_LOGIT, MOE_LORA_BAD_MXFP8, MOE_LORA_BF16, MOE_LORA_EHIP, MOE_LORA_EINVAL, MOE_LORA_EUNSUPPORTED, MOE_LORA_EWORKSPACE,
    MOE_LORA_F32, MOE_LORA_OK, MoeLoraArgs, MoeLoraDims, MoeLoraError, Mxfp8Weights, PackedWeights, Workspace,
    forward_inputs, make_dims, moe_lora_align, moe_lora_check_args, moe_lora_check_inputs, moe_lora_forward,
    moe_lora_forward_static, moe_lora_packed_mxfp8_bytes, moe_lora_packed_weight_bytes, moe_lora_plan_query, moe_lora_route, moe_lora_strerror,
    moe_lora_workspace_bytes,
)
