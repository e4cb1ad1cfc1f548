"""GPU parity of the few-token path (1 to 128 tokens, bf16 activations, r a
multiple of 8 up to 64; the backward, the NF4 forward and the bf16 forward
where the dispatch rule takes it): a panel-partials launch (the backward
then sums the panels), then one launch that streams W (bf16, or NF4 codes
expanded on the fly) in 256 equal ranges of the column tiles' contraction stages; the last
block to arrive at a tile sums its partials in block order, adds the rank term
and stores (or rotates, RoPE).  Against the float64 oracle at the bf16 bar;
repeats are bitwise equal (the arrival order of blocks must not change a bit);
small-integer inputs are exact."""
import math

import numpy as np
import pytest
import torch

import oracle as O
from lora_linear_layers_amd import _lib
from synth import gen
from tests.helpers import TOL, cpu64, few_path, lora_inputs, rel

pytestmark = pytest.mark.gpu


def _kinds(fn):
    _lib.profile_only(None)
    _lib.profile_begin(256)
    out = fn()
    torch.cuda.synchronize()
    _lib.profile_end()
    return out, set(_lib.profile_report())


def _check_path(kinds, nf4, M, d_in, d_out, r, rope=False):
    """The few-token launches ran exactly where the dispatch rule takes them."""
    fwd, bwd = few_path(False, nf4, M, d_in, d_out, r, rope), few_path(True, nf4, M, d_in, d_out, r, rope)
    assert ("few_fwd" in kinds) == fwd and ("few_bwd" in kinds) == bwd, kinds
    if not nf4 and not fwd:
        assert ("skinny_fwd" in kinds) == (M <= 64), kinds
    assert ("few_panel" in kinds) == (fwd or bwd), kinds
    assert fwd or bwd, "a case outside the few-token path"


# (M, d_in, d_out, r): every 16-row block count, ranges of one to many stages
# per block, ranks 8 / 16 / 64, panels summed in the stream (fold) or between
# the launches
SHAPES = [(1, 256, 512, 8), (5, 384, 576, 16), (16, 4096, 4096, 16), (17, 1024, 2048, 64),
          (33, 2048, 1024, 8), (64, 4096, 1024, 64), (49, 512, 4096, 16), (100, 512, 4096, 16),
          (128, 5120, 1024, 64)]


@pytest.mark.parametrize("shape", SHAPES, ids=[f"{m}x{i}x{o}r{r}" for m, i, o, r in SHAPES])
def test_few_parity(lib, shape):
    M, d_in, d_out, r = shape
    s = 16.0 / r
    X, W, A, B, dY = lora_inputs(700 + M, M, d_in, d_out, r, "bf16")
    (Y, (dX, dA, dB)), kinds = _kinds(lambda: (lib.lora_linear_fwd(X, W, A, B, s),
                                               lib.lora_linear_bwd(X, W, A, B, s, dY)))
    _check_path(kinds, False, M, d_in, d_out, r)
    Yr = O.lora_forward(X, W, A, B, s)
    dXr, dAr, dBr = O.lora_backward(X, W, A, B, s, dY)
    errs = dict(Y=rel(Y, Yr), dX=rel(dX, dXr), dA=rel(dA, dAr), dB=rel(dB, dBr))
    print(shape, errs, flush=True)
    assert all(e <= TOL["bf16"] for e in errs.values()), errs
    Y2 = lib.lora_linear_fwd(X, W, A, B, s)
    dX2, dA2, dB2 = lib.lora_linear_bwd(X, W, A, B, s, dY)
    torch.cuda.synchronize()
    for a, b in ((Y, Y2), (dX, dX2), (dA, dA2), (dB, dB2)):
        assert torch.equal(a, b)


@pytest.mark.parametrize("M,d_in,d_out,r,seq", [(1, 1024, 512, 8, 64), (16, 4096, 4096, 16, 2048),
                                                (64, 2048, 1024, 64, 100), (40, 1024, 4096, 16, 4096),
                                                (128, 1024, 4096, 16, 4096)])
def test_few_rope_parity(lib, M, d_in, d_out, r, seq):
    X, W, A, B, dY = lora_inputs(730 + M, M, d_in, d_out, r, "bf16")
    pos = torch.from_numpy(gen.positions_mod(M, seq)).cuda()
    cos, sin = lib.rope_cache(seq, 128, 500000.0)
    s = 16.0 / r
    (Y, (dX, dA, dB)), kinds = _kinds(lambda: (lib.lora_qk_rope_fwd(X, W, A, B, s, pos, cos, sin),
                                               lib.lora_qk_rope_bwd(X, W, A, B, s, pos, cos, sin, dY)))
    _check_path(kinds, False, M, d_in, d_out, r, rope=True)
    p = pos.cpu().numpy()
    Yr = O.qk_rope_forward(X, W, A, B, s, p)
    dXr, dAr, dBr = O.qk_rope_backward(X, W, A, B, s, p, dY)
    errs = dict(Y=rel(Y, Yr), dX=rel(dX, dXr), dA=rel(dA, dAr), dB=rel(dB, dBr))
    print(M, errs, flush=True)
    assert all(e <= TOL["bf16"] for e in errs.values()), errs


# NF4: a ragged forward tile (704 = 5.5 tiles of 128), up to 128 tokens
@pytest.mark.parametrize("M,d_in,d_out,r", [(1, 512, 704, 8), (16, 5120, 2048, 64), (40, 1024, 4096, 16),
                                            (100, 1024, 2048, 16), (128, 2048, 1024, 64)])
def test_few_nf4_parity(lib, M, d_in, d_out, r):
    tab = gen.nf4_table()
    X, _, A, B, dY = lora_inputs(760 + M, M, d_in, d_out, r, "bf16")
    codes = gen.nf4_random_codes(761 + M, d_out * d_in).cuda()
    absmax = gen.nf4_random_absmax(762 + M, d_out * d_in // 64, 1.0 / math.sqrt(d_in)).cuda()
    s = 16.0 / r
    (Y, (dX, dA, dB)), kinds = _kinds(lambda: (
        lib.nf4_lora_linear_fwd(X, codes, absmax, tab, A, B, s, d_out),
        lib.nf4_lora_linear_bwd(X, codes, absmax, tab, A, B, s, dY)))
    _check_path(kinds, True, M, d_in, d_out, r)
    c, am = codes.cpu().numpy(), absmax.cpu().numpy()
    Yr = O.nf4_lora_forward(X, c, am, tab, A, B, s, d_out, d_in)
    dXr, dAr, dBr = O.nf4_lora_backward(X, c, am, tab, A, B, s, dY, d_out, d_in)
    errs = dict(Y=rel(Y, Yr), dX=rel(dX, dXr), dA=rel(dA, dAr), dB=rel(dB, dBr))
    print("nf4", M, errs, flush=True)
    assert all(e <= TOL["bf16"] for e in errs.values()), errs


@pytest.mark.parametrize("nf4", [False, True])
def test_few_integer_exact(lib, nf4):
    # Sparse {-1, 0, 1} activations and adapters with W in {-1, 0, 1} (NF4:
    # codes of -1, 0 and 1 with absmax 1): every partial, panel and output is
    # a small integer, so the split sums must equal the oracle exactly.
    M, d_in, d_out, r, s = 48, 2048, 1024, 16, 1.0
    g = torch.Generator().manual_seed(93)

    def sp(shape, density):
        v = torch.randint(-1, 2, shape, generator=g)
        keep = torch.rand(shape, generator=g) < density
        return (v * keep).to(torch.bfloat16).cuda()
    X, A, B, dY = sp((M, d_in), 1 / 16), sp((r, d_in), 1.0), sp((d_out, r), 1 / 4), sp((M, d_out), 1 / 8)
    tab = gen.nf4_table()
    if nf4:
        pick = torch.tensor([0, 7, 15], dtype=torch.int64)  # table values -1, 0, 1
        c = pick[torch.randint(0, 3, (d_out * d_in,), generator=g)]
        codes = ((c[0::2] << 4) | c[1::2]).to(torch.uint8).cuda()
        absmax = torch.ones(d_out * d_in // 64, dtype=torch.float32).cuda()
        W = torch.from_numpy(O.nf4_dequant(codes.cpu().numpy(), absmax.cpu().numpy(), tab, d_out, d_in))
        assert set(np.unique(W.numpy())) <= {-1.0, 0.0, 1.0}
        (Y, (dX, dA, dB)), kinds = _kinds(lambda: (
            lib.nf4_lora_linear_fwd(X, codes, absmax, tab, A, B, s, d_out),
            lib.nf4_lora_linear_bwd(X, codes, absmax, tab, A, B, s, dY)))
    else:
        W = sp((d_out, d_in), 1.0)
        (Y, (dX, dA, dB)), kinds = _kinds(lambda: (lib.lora_linear_fwd(X, W, A, B, s),
                                                   lib.lora_linear_bwd(X, W, A, B, s, dY)))
    _check_path(kinds, nf4, M, d_in, d_out, r)
    Yr = O.lora_forward(X, W, A, B, s)
    dXr, dAr, dBr = O.lora_backward(X, W, A, B, s, dY)
    assert np.abs(O.lora_panel(X, A)).max() <= 256 and np.abs(cpu64(dY) @ cpu64(B)).max() <= 256
    assert np.abs(Yr).max() <= 256 and np.abs(dXr).max() <= 256
    for got, ref in ((Y, Yr), (dX, dXr), (dA, dAr), (dB, dBr)):
        assert np.array_equal(cpu64(got), ref)
