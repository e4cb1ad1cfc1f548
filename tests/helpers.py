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


def sample_rows(M, seq_len, batch, n=256, seed=99):
    """n seeded token rows of an [M, .] output, every sequence's first and last
    token among them (all rows when M <= n)."""
    if M <= n:
        return np.arange(M)
    must = sorted({b * seq_len for b in range(batch)} | {b * seq_len + seq_len - 1 for b in range(batch)})
    rng = np.random.default_rng(seed)
    rest = rng.choice(np.setdiff1d(np.arange(M), must), n - len(must), replace=False)
    return np.sort(np.concatenate([must, rest]))


def few_path(bwd, nf4, M, d_in, d_out, r, rope=False):
    """Whether the library takes the few-token path (its dispatch rule): bf16
    activations, 1 <= M <= 128, r a multiple of 8 up to 64, d_in and d_out
    multiples of 64 (d_out of 128 with RoPE, d_in of 128 in the backward and
    with NF4), at most 256 column tiles of 128; the backward, the forward with
    NF4, and the forward with a bf16 W up to 64 tokens with RoPE, more than 16
    tokens, a rank above 16 or W of 2^25 elements or more."""
    if not (1 <= M <= 128 and r % 8 == 0 and r <= 64 and d_in % 64 == 0 and d_out % 64 == 0):
        return False
    if (rope and d_out % 128) or ((bwd or nf4) and d_in % 128):
        return False
    if -(-(d_in if bwd else d_out) // 128) > 256:
        return False
    return bwd or nf4 or (M <= 64 and (rope or M > 16 or r > 16 or d_in * d_out >= 1 << 25))


def fwd_kind(M, d_in, d_out, r, rope=False):
    """The launch that computes a bf16 forward's product at few tokens: the
    few-token stream, else the one-launch skinny kernel (up to 64 tokens, r a
    multiple of 8 up to 64, d_in a multiple of 8, d_out of 128 with RoPE), else
    the split GEMM."""
    if few_path(False, False, M, d_in, d_out, r, rope):
        return "few_fwd"
    if 1 <= M <= 64 and r % 8 == 0 and r <= 64 and d_in % 8 == 0 and not (rope and d_out % 128):
        return "skinny_fwd"
    return "gemm_bf16_128x128_nt_split"
