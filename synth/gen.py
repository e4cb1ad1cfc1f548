"""Counter-based random draws for the synthetic LoRA workloads.

Generator: splitmix64 (Steele, Lea and Flood, "Fast splittable pseudorandom
number generators", OOPSLA 2014).  Draw i of a stream with seed S is
mix64(mix64(S) + (i + 1) * 0x9E3779B97F4A7C15), and its top 53 bits give a
uniform double in [0, 1).  Normals use the Box-Muller transform on draws 2i
and 2i+1 of the stream (cosine branch only).  Every tensor has its own
stream, so a tensor never depends on the order in which tensors are drawn.

The integer part runs as wrapping int64 arithmetic in torch, which gives the
same bits on the CPU and on a GPU; values are drawn in float64 and then
rounded to the storage type with torch's round-to-nearest-even conversion.
Both the oracle and the GPU library read the stored values; the oracle widens
them to float64 exactly.
"""
from __future__ import annotations

import os

import numpy as np
import torch

_CHUNK = 1 << 24


def _s64(u: int) -> int:
    u &= (1 << 64) - 1
    return u - (1 << 64) if u >= (1 << 63) else u


_GAMMA = _s64(0x9E3779B97F4A7C15)
_M1 = _s64(0xBF58476D1CE4E5B9)
_M2 = _s64(0x94D049BB133111EB)


def _shr(z: torch.Tensor, k: int) -> torch.Tensor:
    """Logical right shift of int64 bit patterns."""
    return (z >> k) & ((1 << (64 - k)) - 1)


def _mix64(z: torch.Tensor) -> torch.Tensor:
    z = z ^ _shr(z, 30)
    z = z * _M1
    z = z ^ _shr(z, 27)
    z = z * _M2
    return z ^ _shr(z, 31)


def _mix64_int(x: int) -> int:
    m = (1 << 64) - 1
    x &= m
    x ^= x >> 30
    x = (x * 0xBF58476D1CE4E5B9) & m
    x ^= x >> 27
    x = (x * 0x94D049BB133111EB) & m
    return x ^ (x >> 31)


def _raw(seed: int, start: int, n: int, device) -> torch.Tensor:
    base = _s64(_mix64_int(seed))
    ctr = torch.arange(start + 1, start + n + 1, dtype=torch.int64, device=device)
    return _mix64(ctr * _GAMMA + base)


def _uniform_chunk(seed, start, n, device):
    return _shr(_raw(seed, start, n, device), 11).to(torch.float64) * (1.0 / 9007199254740992.0)


def splitmix64_uniform(seed: int, n: int, start: int = 0, device="cpu") -> torch.Tensor:
    """n uniform doubles in [0, 1) from draws start..start+n-1 of stream `seed`."""
    out = torch.empty(n, dtype=torch.float64, device=device)
    for lo in range(0, n, _CHUNK):
        hi = min(n, lo + _CHUNK)
        out[lo:hi] = _uniform_chunk(seed, start + lo, hi - lo, device)
    return out


def normal(seed: int, n: int, std: float, start: int = 0, device="cpu") -> torch.Tensor:
    """Draws start..start+n-1 of N(0, std^2); element i uses uniforms 2i and 2i+1."""
    out = torch.empty(n, dtype=torch.float64, device=device)
    for lo in range(0, n, _CHUNK // 2):
        hi = min(n, lo + _CHUNK // 2)
        u = _uniform_chunk(seed, 2 * (start + lo), 2 * (hi - lo), device).view(-1, 2)
        u1 = 1.0 - u[:, 0]  # (0, 1]: log is finite
        out[lo:hi] = torch.sqrt(-2.0 * torch.log(u1)) * torch.cos((2.0 * np.pi) * u[:, 1]) * std
    return out


def uniform_sym(seed: int, n: int, bound: float, device="cpu") -> torch.Tensor:
    """n draws of U(-bound, +bound)."""
    return (2.0 * splitmix64_uniform(seed, n, device=device) - 1.0) * bound


def to_storage(x: torch.Tensor, shape, dtype: str) -> torch.Tensor:
    """Round float64 draws to the storage dtype ('f32' or 'bf16')."""
    t = x.reshape(shape)
    if dtype == "f32":
        return t.to(torch.float32)
    if dtype == "bf16":
        return t.to(torch.float32).to(torch.bfloat16)
    raise ValueError(dtype)


def nf4_table() -> np.ndarray:
    """The 16 NormalFloat-4 code values (fp32), read from nf4_table.txt beside this file."""
    path = os.path.join(os.path.dirname(__file__), "nf4_table.txt")
    vals = []
    with open(path) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                vals.append(float(line))
    if len(vals) != 16:
        raise ValueError("nf4_table.txt must hold 16 values")
    return np.array(vals, dtype=np.float32)


def nf4_random_codes(seed: int, n_elems: int, device="cpu") -> torch.Tensor:
    """Packed uint8 codes for n_elems 4-bit values drawn uniformly from 0..15.

    Element 2j sits in the high nibble of byte j, element 2j+1 in the low
    nibble; each byte takes the top 8 bits of one draw.
    """
    if n_elems % 2:
        raise ValueError("n_elems must be even")
    nb = n_elems // 2
    out = torch.empty(nb, dtype=torch.uint8, device=device)
    for lo in range(0, nb, _CHUNK):
        hi = min(nb, lo + _CHUNK)
        out[lo:hi] = _shr(_raw(seed, lo, hi - lo, device), 56).to(torch.uint8)
    return out


def nf4_random_absmax(seed: int, n_blocks: int, std: float, blocksize: int = 64,
                      device="cpu") -> torch.Tensor:
    """Per-block absmax distributed as max |N(0, std^2)| over `blocksize` draws.

    Drawn through the order statistic: for U ~ U(0,1),
    std * Phi^{-1}((1 + U^(1/blocksize)) / 2) has the law of that maximum.
    Stored as fp32.
    """
    u = splitmix64_uniform(seed, n_blocks, device=device).clamp_min(1e-300)
    m = std * torch.special.ndtri(0.5 * (1.0 + u ** (1.0 / blocksize)))
    return m.to(torch.float32)


def positions_mod(M: int, seq_len: int) -> np.ndarray:
    """Token positions for M = batch * seq_len flattened rows: pos[t] = t mod seq_len."""
    return (np.arange(M, dtype=np.int64) % seq_len).astype(np.int32)
