"""Seeded synthetic inputs for the fused LoRA linear layer.

This package only draws random numbers and rounds them to the storage type
(fp32 or bf16).  It holds none of the method's arithmetic: the oracle under
``oracle/`` and the HIP library under ``lora_linear_layers_amd/`` both take
their inputs from here and from nowhere else.
"""
from .gen import (  # noqa: F401
    splitmix64_uniform,
    normal,
    uniform_sym,
    to_storage,
    nf4_table,
    nf4_random_codes,
    nf4_random_absmax,
    positions_mod,
)
from .configs import CONFIGS, Projection, Config, tensor_seed  # noqa: F401
