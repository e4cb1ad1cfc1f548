"""Oracle for the fused LoRA linear layer: plain, slow, float64 CPU code.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import it.  The HIP library never calls it, and the two
share no code.
"""
from .lora_oracle import (  # noqa: F401
    lora_forward,
    lora_backward,
    lora_grad_x,
    lora_grad_ab,
    lora_panel,
    rope_angles,
    rope_rotate,
    qk_rope_forward,
    qk_rope_backward,
    round_f32,
    round_bf16,
    nf4_unpack,
    nf4_dequant,
    nf4_encode,
    nf4_lora_forward,
    nf4_lora_backward,
    merged_weight,
    dropout_keep,
    philox4x32_10,
    dropout_threshold,
    dropout_mask_philox,
    dropout_mask_philox_np,
    dropout_pack,
    lora_dropout_forward,
    lora_dropout_backward,
    silu,
    swiglu_forward,
    swiglu_grad,
    swiglu_backward,
    rel_err,
)
