"""The five synthetic workloads and the per-tensor seeds.

Shapes follow the pages' workloads: Llama-3-8B attention and SwiGLU MLP
projections (4 sequences of 2048 tokens, or 1 of 8192 for long context) and a
Qwen1.5-32B-shaped QLoRA case with an NF4 base weight.  Distributions, with
the second argument of N(.,.) read as a variance:

  X, dY ~ N(0, 1);  W ~ N(0, 1/d_in);  A ~ U(-1/sqrt(d_in), +1/sqrt(d_in));
  B ~ N(0, 0.02);   NF4: codes uniform on 0..15, absmax = max|N(0, 1/d_in)|
  over each block of 64.

Seeds: 3407 + 100 * config + 1000 * slot + index, where slot names the tensor
kind and index the projection (or, for X, the input group: projections that
read the same activations share X).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np
import torch

from . import gen

BASE_SEED = 3407
SLOTS = {"X": 0, "W": 1, "A": 2, "B": 3, "dY": 4, "codes": 5, "absmax": 6}


def tensor_seed(cfg_id: int, slot: str, index: int) -> int:
    return BASE_SEED + 100 * cfg_id + 1000 * SLOTS[slot] + index


@dataclass(frozen=True)
class Projection:
    name: str
    d_in: int
    d_out: int
    rope: bool = False
    x_group: int = 0  # projections with the same group read the same X


@dataclass(frozen=True)
class Config:
    cfg_id: int
    name: str
    dtype: str  # 'f32' or 'bf16'
    batch: int
    seq_len: int
    r: int
    alpha: float
    projections: List[Projection] = field(default_factory=list)
    nf4: bool = False
    rope_theta: float = 500000.0
    head_dim: int = 128

    @property
    def M(self) -> int:
        return self.batch * self.seq_len

    @property
    def scale(self) -> float:
        return self.alpha / self.r

    def useful_flop(self, M: Optional[int] = None) -> float:
        """Forward + backward useful FLOP over all projections: 2M(2dk + 3r(d+k))."""
        M = self.M if M is None else M
        tot = 0.0
        for p in self.projections:
            tot += 2.0 * M * (2.0 * p.d_in * p.d_out + 3.0 * self.r * (p.d_in + p.d_out))
        return tot


def _attn(h, kv):
    return [
        Projection("q_proj", h, h, rope=True, x_group=0),
        Projection("k_proj", h, kv, rope=True, x_group=0),
        Projection("v_proj", h, kv, x_group=0),
        Projection("o_proj", h, h, x_group=1),
    ]


def _mlp(h, inter):
    return [
        Projection("gate_proj", h, inter, x_group=2),
        Projection("up_proj", h, inter, x_group=2),
        Projection("down_proj", inter, h, x_group=3),
    ]


CONFIGS = {
    1: Config(1, "single-fp32-256", "f32", 1, 128, 8, 16.0,
              [Projection("linear", 256, 256)]),
    2: Config(2, "llama3-8b-attn-4x2048-r16", "bf16", 4, 2048, 16, 16.0, _attn(4096, 1024)),
    3: Config(3, "llama3-8b-mlp-4x2048-r64", "bf16", 4, 2048, 64, 16.0, _mlp(4096, 14336)),
    4: Config(4, "llama3-8b-attn-1x8192-r64", "bf16", 1, 8192, 64, 16.0, _attn(4096, 1024)),
    5: Config(5, "qwen15-32b-nf4-4x2048-r64", "bf16", 4, 2048, 64, 16.0,
              [Projection("q_proj", 5120, 5120, x_group=0),
               Projection("k_proj", 5120, 1024, x_group=0),
               Projection("v_proj", 5120, 1024, x_group=0),
               Projection("o_proj", 5120, 5120, x_group=1)] + _mlp(5120, 27392), nf4=True),
}


def _rows(M, rows):
    return np.arange(M) if rows is None else np.asarray(rows, dtype=np.int64)


class Inputs:
    """Inputs of one config, drawn on demand.  Tensors are torch tensors in the
    storage dtype on `device`.  X and dY may be drawn for a subset of rows
    (tokens) only: such a draw holds exactly the values the full tensor holds
    in those rows."""

    def __init__(self, cfg: Config, M: Optional[int] = None, device="cpu"):
        self.cfg = cfg
        self.M = cfg.M if M is None else M
        self.device = device

    # -- activations -----------------------------------------------------
    def _act(self, slot, index, width, rows):
        seed = tensor_seed(self.cfg.cfg_id, slot, index)
        if rows is None:
            x = gen.normal(seed, self.M * width, 1.0, device=self.device)
            return gen.to_storage(x, (self.M, width), self.cfg.dtype)
        rows = _rows(self.M, rows)
        parts = [gen.normal(seed, width, 1.0, start=int(t) * width, device=self.device) for t in rows]
        x = torch.cat(parts) if parts else torch.zeros(0, dtype=torch.float64, device=self.device)
        return gen.to_storage(x, (len(rows), width), self.cfg.dtype)

    def X(self, p: Projection, rows=None):
        return self._act("X", p.x_group, p.d_in, rows)

    def dY(self, p: Projection, rows=None):
        return self._act("dY", self.cfg.projections.index(p), p.d_out, rows)

    # -- weights ---------------------------------------------------------
    def W(self, p: Projection):
        i = self.cfg.projections.index(p)
        w = gen.normal(tensor_seed(self.cfg.cfg_id, "W", i), p.d_in * p.d_out,
                       1.0 / math.sqrt(p.d_in), device=self.device)
        return gen.to_storage(w, (p.d_out, p.d_in), self.cfg.dtype)

    def A(self, p: Projection):
        i = self.cfg.projections.index(p)
        a = gen.uniform_sym(tensor_seed(self.cfg.cfg_id, "A", i), self.cfg.r * p.d_in,
                            1.0 / math.sqrt(p.d_in), device=self.device)
        return gen.to_storage(a, (self.cfg.r, p.d_in), self.cfg.dtype)

    def B(self, p: Projection):
        i = self.cfg.projections.index(p)
        b = gen.normal(tensor_seed(self.cfg.cfg_id, "B", i), p.d_out * self.cfg.r,
                       math.sqrt(0.02), device=self.device)
        return gen.to_storage(b, (p.d_out, self.cfg.r), self.cfg.dtype)

    def nf4(self, p: Projection):
        """(packed codes uint8 [d_out*d_in/2], absmax fp32 [d_out*d_in/64])."""
        i = self.cfg.projections.index(p)
        n = p.d_in * p.d_out
        codes = gen.nf4_random_codes(tensor_seed(self.cfg.cfg_id, "codes", i), n, device=self.device)
        absmax = gen.nf4_random_absmax(tensor_seed(self.cfg.cfg_id, "absmax", i), n // 64,
                                       1.0 / math.sqrt(p.d_in), device=self.device)
        return codes, absmax

    def positions(self, rows=None):
        pos = gen.positions_mod(self.M, self.cfg.seq_len)
        pos = pos if rows is None else pos[_rows(self.M, rows)]
        return torch.from_numpy(pos).to(self.device)
