"""Shared test helpers: seeded inputs on the device and oracle comparisons."""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle as O
from synth import gen

TOL = {"f32": 1e-5, "bf16": 2e-2}
TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def draw(seed, shape, kind, scale, dtype, device="cuda"):
    n = int(np.prod(shape))
    if kind == "normal":
        x = gen.normal(seed, n, scale)
    elif kind == "uniform":
        x = gen.uniform_sym(seed, n, scale)
    else:
        raise ValueError(kind)
    return gen.to_storage(x, shape, dtype).to(device)


def lora_inputs(seed, M, d_in, d_out, r, dtype, device="cuda"):
    """X, W, A, B, dY with the workload distributions (variance reading)."""
    X = draw(seed + 0, (M, d_in), "normal", 1.0, dtype, device)
    W = draw(seed + 1, (d_out, d_in), "normal", 1.0 / math.sqrt(d_in), dtype, device)
    A = draw(seed + 2, (r, d_in), "uniform", 1.0 / math.sqrt(d_in), dtype, device)
    B = draw(seed + 3, (d_out, r), "normal", math.sqrt(0.02), dtype, device)
    dY = draw(seed + 4, (M, d_out), "normal", 1.0, dtype, device)
    return X, W, A, B, dY


def int_inputs(seed, M, d_in, d_out, r, dtype, lo=-1, hi=1, device="cuda"):
    """Small-integer tensors: every product and sum below is exact."""
    g = torch.Generator().manual_seed(seed)
    mk = lambda *s: torch.randint(lo, hi + 1, s, generator=g).to(TORCH_DT[dtype]).to(device)  # noqa: E731
    return mk(M, d_in), mk(d_out, d_in), mk(r, d_in), mk(d_out, r), mk(M, d_out)


def cpu64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def rel(got, ref):
    return O.rel_err(cpu64(got) if torch.is_tensor(got) else got, ref)
