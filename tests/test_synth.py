"""The seeded input generator: published splitmix64 draws, row-subset consistency."""
import numpy as np
import torch

from synth import CONFIGS, gen
from synth.configs import Inputs


def _splitmix64_ref(seed, i):
    m = (1 << 64) - 1

    def mix(x):
        x ^= x >> 30
        x = (x * 0xBF58476D1CE4E5B9) & m
        x ^= x >> 27
        x = (x * 0x94D049BB133111EB) & m
        return x ^ (x >> 31)

    return mix((mix(seed) + (i + 1) * 0x9E3779B97F4A7C15) & m)


def test_uniform_matches_scalar_splitmix64():
    u = gen.splitmix64_uniform(3407, 9, start=1000)
    ref = [(_splitmix64_ref(3407, 1000 + i) >> 11) / 2.0 ** 53 for i in range(9)]
    assert u.tolist() == ref


def test_normal_moments_and_rows():
    inp = Inputs(CONFIGS[2], M=64)
    p = CONFIGS[2].projections[0]
    X = inp.X(p)
    assert X.dtype == torch.bfloat16 and X.shape == (64, 4096)
    x = X.double()
    assert abs(x.mean().item()) < 0.01 and abs(x.std().item() - 1.0) < 0.01
    rows = [0, 17, 63]
    assert torch.equal(inp.X(p, rows=rows), X[rows])


def test_weight_scales_and_seeds_distinct():
    c = CONFIGS[1]
    inp = Inputs(c)
    p = c.projections[0]
    W, A, B = inp.W(p), inp.A(p), inp.B(p)
    assert W.dtype == torch.float32 and W.shape == (256, 256)
    assert abs(W.double().std().item() * 16 - 1.0) < 0.02           # var 1/d_in
    assert A.abs().max().item() <= 1.0 / 16                          # U(+-1/sqrt(d_in))
    assert abs(B.double().std().item() - np.sqrt(0.02)) < 0.02       # var 0.02
    assert not torch.equal(inp.X(p)[:1], inp.dY(p)[:1])


def test_nf4_codes_and_absmax():
    codes = gen.nf4_random_codes(11, 1 << 16)
    assert codes.dtype == torch.uint8 and codes.numel() == 1 << 15
    hist = torch.bincount((codes >> 4).long(), minlength=16).double()
    assert (hist / hist.mean() - 1).abs().max() < 0.1
    am = gen.nf4_random_absmax(12, 4096, 1.0 / 64)
    # E max|N(0,1)| over 64 draws is about 2.4
    assert 2.2 < am.double().mean().item() * 64 < 2.6


def test_positions_and_config_flops():
    pos = gen.positions_mod(8192, 2048)
    assert pos[0] == 0 and pos[2047] == 2047 and pos[2048] == 0 and pos.dtype == np.int32
    assert abs(CONFIGS[3].useful_flop() / 1e12 - 5.946) < 1e-3
    assert abs(CONFIGS[1].useful_flop() - 3.670016e7) < 1
