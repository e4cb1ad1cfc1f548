"""GPU parity at few tokens.  Outside the few-token path's range (its own
tests cover it) the dX GEMM (and the forward beyond 64 tokens, or with a rank
that is not a multiple of 8 or above 64) splits its contraction into fp32
partials (the 128x128 tiles alone would leave most CUs idle) and a
fixed-order sum finishes them (with the RoPE rotation for q/k); up to 64
tokens the bf16 forward is one fused launch (skinny_fwd) where the few-token
stream does not take it.  The profiler
confirms which path ran; the oracle is the float64 reference as everywhere
else."""
import math

import numpy as np
import pytest
import torch

import oracle as O
from lora_linear_layers_amd import _lib
from synth import gen
from tests.helpers import TOL, cpu64, few_path, fwd_kind, lora_inputs, rel

pytestmark = pytest.mark.gpu


def _kinds(lib, fn):
    _lib.profile_begin(256)
    out = fn()
    torch.cuda.synchronize()
    _lib.profile_end()
    return out, set(_lib.profile_report())


# (M, d_in, d_out, r): contraction splits of 2..16, ragged splits and ranks
SMALL = [(1, 4096, 1024, 16), (7, 2048, 4096, 3), (16, 4096, 4096, 16), (64, 1024, 520, 8),
         (128, 5120, 1024, 64), (256, 1024, 2048, 100)]


@pytest.mark.parametrize("shape", SMALL, ids=[f"{m}x{i}x{o}r{r}" for m, i, o, r in SMALL])
def test_small_token_parity(lib, shape):
    M, d_in, d_out, r = shape
    s = 16.0 / r
    X, W, A, B, dY = lora_inputs(300 + M, M, d_in, d_out, r, "bf16")
    (Y, (dX, dA, dB)), kinds = _kinds(lib, lambda: (lib.lora_linear_fwd(X, W, A, B, s),
                                                   lib.lora_linear_bwd(X, W, A, B, s, dY)))
    if few_path(True, False, M, d_in, d_out, r):
        assert "few_bwd" in kinds, kinds
    else:
        assert {"gemm_bf16_128x128_nn_split", "split_finish"} <= kinds, kinds
    assert fwd_kind(M, d_in, d_out, r) in kinds, kinds
    Yr = O.lora_forward(X, W, A, B, s)
    dXr, dAr, dBr = O.lora_backward(X, W, A, B, s, dY)
    errs = dict(Y=rel(Y, Yr), dX=rel(dX, dXr), dA=rel(dA, dAr), dB=rel(dB, dBr))
    print(shape, errs)
    assert all(e <= TOL["bf16"] for e in errs.values()), errs
    # fixed-order reductions: repeats are bitwise equal
    Y2 = lib.lora_linear_fwd(X, W, A, B, s)
    dX2, dA2, dB2 = lib.lora_linear_bwd(X, W, A, B, s, dY)
    torch.cuda.synchronize()
    for a, b in ((Y, Y2), (dX, dX2), (dA, dA2), (dB, dB2)):
        assert torch.equal(a, b)


@pytest.mark.parametrize("M,d_in,d_out,r,seq", [(64, 4096, 4096, 16, 2048), (200, 1024, 1024, 64, 100),
                                                (5, 2048, 1024, 8, 7)])
def test_small_token_rope_parity(lib, M, d_in, d_out, r, seq):
    X, W, A, B, dY = lora_inputs(77 + M, M, d_in, d_out, r, "bf16")
    pos = torch.from_numpy(gen.positions_mod(M, seq)).cuda()
    cos, sin = lib.rope_cache(seq, 128, 500000.0)
    s = 16.0 / r
    (Y, (dX, dA, dB)), kinds = _kinds(lib, lambda: (lib.lora_qk_rope_fwd(X, W, A, B, s, pos, cos, sin),
                                                   lib.lora_qk_rope_bwd(X, W, A, B, s, pos, cos, sin, dY)))
    assert ("few_bwd" if few_path(True, False, M, d_in, d_out, r, rope=True) else "split_finish") in kinds, kinds
    assert fwd_kind(M, d_in, d_out, r, rope=True) in kinds, kinds
    p = pos.cpu().numpy()
    Yr = O.qk_rope_forward(X, W, A, B, s, p)
    dXr, dAr, dBr = O.qk_rope_backward(X, W, A, B, s, p, dY)
    errs = dict(Y=rel(Y, Yr), dX=rel(dX, dXr), dA=rel(dA, dAr), dB=rel(dB, dBr))
    print(M, errs)
    assert all(e <= TOL["bf16"] for e in errs.values()), errs


@pytest.mark.parametrize("M,d_in,d_out,r", [(16, 1024, 2048, 16), (128, 5120, 1024, 64), (3, 2048, 512, 5)])
def test_small_token_nf4_parity(lib, M, d_in, d_out, r):
    tab = gen.nf4_table()
    X, _, A, B, dY = lora_inputs(51 + M, M, d_in, d_out, r, "bf16")
    codes = gen.nf4_random_codes(53 + M, d_out * d_in).cuda()
    absmax = gen.nf4_random_absmax(54 + M, d_out * d_in // 64, 1.0 / math.sqrt(d_in)).cuda()
    s = 16.0 / r
    (Y, (dX, dA, dB)), kinds = _kinds(lib, lambda: (
        lib.nf4_lora_linear_fwd(X, codes, absmax, tab, A, B, s, d_out),
        lib.nf4_lora_linear_bwd(X, codes, absmax, tab, A, B, s, dY)))
    fwd_few, bwd_few = few_path(False, True, M, d_in, d_out, r), few_path(True, True, M, d_in, d_out, r)
    assert ("few_fwd" if fwd_few else "gemm_nf4_128x128_nt_split") in kinds, kinds
    assert ("few_bwd" if bwd_few else "gemm_nf4_128x128_nn_split") in kinds, kinds
    c, am = codes.cpu().numpy(), absmax.cpu().numpy()
    Yr = O.nf4_lora_forward(X, c, am, tab, A, B, s, d_out, d_in)
    dXr, dAr, dBr = O.nf4_lora_backward(X, c, am, tab, A, B, s, dY, d_out, d_in)
    errs = dict(Y=rel(Y, Yr), dX=rel(dX, dXr), dA=rel(dA, dAr), dB=rel(dB, dBr))
    print("nf4", M, errs)
    assert all(e <= TOL["bf16"] for e in errs.values()), errs


def test_small_token_integer_exact(lib):
    # Sparse {-1, 0, 1} inputs: every partial, panel and output is a small
    # integer, so the fixed-order sums must equal the oracle exactly.
    M, d_in, d_out, r, s = 64, 2048, 1024, 16, 1.0
    g = torch.Generator().manual_seed(91)

    def sp(shape, density):
        v = torch.randint(-1, 2, shape, generator=g)
        keep = torch.rand(shape, generator=g) < density
        return (v * keep).to(torch.bfloat16).cuda()
    X, W, A, B, dY = sp((M, d_in), 1 / 16), sp((d_out, d_in), 1.0), sp((r, d_in), 1.0), sp((d_out, r), 1 / 4), \
        sp((M, d_out), 1 / 8)
    (Y, (dX, dA, dB)), kinds = _kinds(lib, lambda: (lib.lora_linear_fwd(X, W, A, B, s),
                                                   lib.lora_linear_bwd(X, W, A, B, s, dY)))
    assert {fwd_kind(M, d_in, d_out, r), "few_bwd"} <= kinds, kinds
    Yr = O.lora_forward(X, W, A, B, s)
    dXr, dAr, dBr = O.lora_backward(X, W, A, B, s, dY)
    assert np.abs(O.lora_panel(X, A)).max() <= 256 and np.abs(cpu64(dY) @ cpu64(B)).max() <= 256
    assert np.abs(Yr).max() <= 256 and np.abs(dXr).max() <= 256
    for got, ref in ((Y, Yr), (dX, dXr), (dA, dAr), (dB, dBr)):
        assert np.array_equal(cpu64(got), ref)
