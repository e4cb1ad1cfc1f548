"""GPU parity of the one-launch few-token forward (skinny_fwd: up to 64
tokens, rank a multiple of 8 up to 64, bf16 W) against the float64 oracle:
ragged token counts, outputs that are not a multiple of 16 wide,
contractions that are not a multiple of 32, both rank widths and both strip
widths (4 strips from 12288 outputs on), RoPE.  Integer inputs make the
plain case exact.  Skinny keeps the shapes the few-token stream does not
take (small plain problems, d_in or d_out off a multiple of 64), so the cases
with RoPE, more than 16 tokens or a rank above 16 have such a dimension."""
import math

import numpy as np
import pytest
import torch

import oracle as O
from lora_linear_layers_amd import _lib
from synth import gen
from tests.helpers import TOL, cpu64, lora_inputs, rel

pytestmark = pytest.mark.gpu


def _kinds(fn):
    _lib.profile_begin(64)
    out = fn()
    torch.cuda.synchronize()
    _lib.profile_end()
    return out, set(_lib.profile_report())


# (M, d_in, d_out, r)
PLAIN = [(1, 4096, 4096, 16), (5, 2048, 520, 8), (16, 4104, 1024, 24), (17, 1032, 2048, 64),
         (33, 2056, 776, 16), (64, 4104, 1024, 64), (12, 1024, 12288, 16), (64, 512, 12296, 64)]


@pytest.mark.parametrize("shape", PLAIN, ids=[f"{m}x{i}x{o}r{r}" for m, i, o, r in PLAIN])
def test_skinny_plain_parity(lib, shape):
    M, d_in, d_out, r = shape
    s = 16.0 / r
    X, W, A, B, _ = lora_inputs(900 + M + r, M, d_in, d_out, r, "bf16")
    Y, kinds = _kinds(lambda: lib.lora_linear_fwd(X, W, A, B, s))
    assert kinds == {"skinny_fwd"}, kinds
    err = rel(Y, O.lora_forward(X, W, A, B, s))
    print(shape, err)
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("M,d_in,d_out,r", [(16, 2048, 1024, 8), (64, 1032, 512, 64)])
def test_skinny_integer_exact(lib, M, d_in, d_out, r):
    # sparse {-1, 0, 1} inputs: every product, panel entry and sum is a small
    # integer, so the fused forward must equal the oracle exactly
    g = torch.Generator().manual_seed(31 + M)

    def sp(shape, density):
        v = torch.randint(-1, 2, shape, generator=g)
        return (v * (torch.rand(shape, generator=g) < density)).to(torch.bfloat16).cuda()
    X, W, A, B = sp((M, d_in), 1 / 16), sp((d_out, d_in), 1.0), sp((r, d_in), 1.0), sp((d_out, r), 1 / 4)
    Y, kinds = _kinds(lambda: lib.lora_linear_fwd(X, W, A, B, 1.0))
    assert kinds == {"skinny_fwd"}
    Yr = O.lora_forward(X, W, A, B, 1.0)
    assert np.abs(O.lora_panel(X, A)).max() <= 256 and np.abs(Yr).max() <= 256
    assert np.array_equal(cpu64(Y), Yr)


@pytest.mark.parametrize("M,d_in,d_out,r,seq", [(1, 4104, 4096, 16, 2048), (40, 2056, 1024, 64, 40),
                                                (64, 1032, 512, 8, 8192)])
def test_skinny_rope_parity(lib, M, d_in, d_out, r, seq):
    X, W, A, B, _ = lora_inputs(70 + M, M, d_in, d_out, r, "bf16")
    pos = torch.from_numpy(gen.positions_mod(M, seq)).cuda()
    cos, sin = lib.rope_cache(seq, 128, 500000.0)
    s = 16.0 / r
    Y, kinds = _kinds(lambda: lib.lora_qk_rope_fwd(X, W, A, B, s, pos, cos, sin))
    assert kinds == {"skinny_fwd"}, kinds
    err = rel(Y, O.qk_rope_forward(X, W, A, B, s, pos.cpu().numpy()))
    print(M, err)
    assert err <= TOL["bf16"]


def test_skinny_not_taken_for_nf4(lib):
    # an NF4 W beyond the few-token path's 128 tokens keeps the split path (its
    # load stage dequantises in LDS tiles)
    M, d_in, d_out, r = 200, 1024, 2048, 16
    tab = gen.nf4_table()
    X, _, A, B, _ = lora_inputs(12, M, d_in, d_out, r, "bf16")
    codes = gen.nf4_random_codes(13, d_out * d_in).cuda()
    absmax = gen.nf4_random_absmax(14, d_out * d_in // 64, 1.0 / math.sqrt(d_in)).cuda()
    Y, kinds = _kinds(lambda: lib.nf4_lora_linear_fwd(X, codes, absmax, tab, A, B, 1.0, d_out))
    assert "skinny_fwd" not in kinds and "gemm_nf4_128x128_nt_split" in kinds, kinds


def test_skinny_not_taken_outside_its_range(lib):
    # 65 tokens, a rank that is not a multiple of 8, a rank above 64: split path
    for M, r in ((65, 16), (16, 12), (16, 72)):
        X, W, A, B, _ = lora_inputs(3, M, 1024, 1024, r, "bf16")
        Y, kinds = _kinds(lambda: lib.lora_linear_fwd(X, W, A, B, 1.0))
        assert "skinny_fwd" not in kinds, (M, r, kinds)
        assert rel(Y, O.lora_forward(X, W, A, B, 1.0)) <= TOL["bf16"]
