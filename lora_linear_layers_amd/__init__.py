"""MI355X (gfx950) fused LoRA linear layer: C-ABI HIP library + thin binding.

    y = W x + s B (A x)   (frozen W, s = alpha / r)

Forward folds the rank-r update into the base GEMM's accumulator; optional
RoPE epilogue for q/k projections; optional NF4 base weight dequantised in
the GEMM load stage.  Backward returns dX, dA, dB, recomputes X A^T and never
forms dW.
"""
from ._lib import (  # noqa: F401
    EXPORTS,
    GROUP_MAX,
    GroupMember,
    LIB_PATH,
    LORA_BF16,
    LORA_F32,
    OP_BWD,
    OP_DROPOUT_BWD,
    OP_DROPOUT_FWD,
    OP_FWD,
    OP_MERGE,
    OP_NF4_BWD,
    OP_NF4_FWD,
    OP_ROPE_BWD,
    OP_ROPE_FWD,
    LoraError,
    lib,
    load,
    workspace_bytes,
)
from .functional import (  # noqa: F401
    LoraLinearFunction,
    lora_dropout_bwd,
    lora_dropout_fwd,
    lora_dropout_mask,
    lora_dropout_philox_bwd,
    lora_dropout_philox_fwd,
    lora_group_bwd,
    lora_group_fwd,
    lora_linear_bwd,
    lora_linear_fwd,
    lora_linear_fwd_noalloc,
    lora_merge,
    lora_qk_rope_bwd,
    lora_qk_rope_fwd,
    lora_swiglu_bwd,
    lora_swiglu_fwd,
    lora_transpose,
    nf4_dequant,
    nf4_lora_linear_bwd,
    nf4_lora_linear_fwd,
    rope_cache,
)
