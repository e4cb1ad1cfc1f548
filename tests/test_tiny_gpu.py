"""GPU parity of the one-launch fp32 path for tiny problems (the whole forward
in one launch, the whole backward in another) against the float64 oracle, at
ragged shapes on both sides of the size rule that selects it, and its run-to-run
bit equality.  The size rule is restated here so that each case checks which
path it took."""
import numpy as np
import pytest
import torch

import oracle as O
from lora_linear_layers_amd import _lib
from tests.helpers import cpu64, int_inputs, lora_inputs, rel

pytestmark = pytest.mark.gpu


def tiny_path(M, d_in, d_out, r):
    mx = max(d_in, d_out)
    return (1 <= r <= 32 and M * r <= 4096 and mx <= 4096 and M * r * mx <= 2 ** 21
            and M * d_in * d_out <= 2 ** 25)


def _kinds(fn):
    _lib.profile_begin(256)
    out = fn()
    torch.cuda.synchronize()
    _lib.profile_end()
    return out, _lib.profile_report()


# (M, d_in, d_out, r): one partial tile, ragged tiles on every side, the
# fp32 workload (128 tokens, 256 -> 256, r 8), the M r and work limits, and
# shapes just past them
TINY = [(1, 8, 8, 1), (7, 136, 72, 3), (33, 40, 104, 5), (128, 256, 256, 8), (129, 264, 392, 16),
        (128, 4096, 8, 32), (512, 8, 4096, 1), (4096, 8, 8, 1), (4097, 8, 8, 1), (129, 264, 392, 33),
        (300, 1000, 24, 8)]


@pytest.mark.parametrize("shape", TINY, ids=[f"{m}x{i}x{o}r{r}" for m, i, o, r in TINY])
def test_tiny_parity(lib, shape):
    M, d_in, d_out, r = shape
    s = 16.0 / r
    X, W, A, B, dY = lora_inputs(700 + M + r, M, d_in, d_out, r, "f32")
    (Y, (dX, dA, dB)), kinds = _kinds(lambda: (lib.lora_linear_fwd(X, W, A, B, s),
                                               lib.lora_linear_bwd(X, W, A, B, s, dY)))
    want = tiny_path(M, d_in, d_out, r)
    assert ("tiny_f32" in kinds) == want, kinds
    if want:
        assert kinds["tiny_f32"][1] == 2  # one launch each way, and nothing else
        assert set(kinds) == {"tiny_f32"}, kinds
    Yr = O.lora_forward(X, W, A, B, s)
    dXr, dAr, dBr = O.lora_backward(X, W, A, B, s, dY)
    errs = dict(Y=rel(Y, Yr), dX=rel(dX, dXr), dA=rel(dA, dAr), dB=rel(dB, dBr))
    print(shape, want, errs)
    assert all(e <= 1e-5 for e in errs.values()), errs


def test_tiny_integer_exact(lib):
    # integer inputs: every partial sum is an integer below 2^24, so any
    # summation order gives the exact result
    M, d_in, d_out, r = 77, 136, 200, 7
    assert tiny_path(M, d_in, d_out, r)
    X, W, A, B, dY = int_inputs(31, M, d_in, d_out, r, "f32")
    Y = lib.lora_linear_fwd(X, W, A, B, 2.0)
    dX, dA, dB = lib.lora_linear_bwd(X, W, A, B, 2.0, dY)
    torch.cuda.synchronize()
    Yr = O.lora_forward(X, W, A, B, 2.0)
    dXr, dAr, dBr = O.lora_backward(X, W, A, B, 2.0, dY)
    for got, ref in ((Y, Yr), (dX, dXr), (dA, dAr), (dB, dBr)):
        assert np.array_equal(cpu64(got), ref)


def test_tiny_without_dx_and_repeats(lib):
    M, d_in, d_out, r = 128, 256, 256, 8
    X, W, A, B, dY = lora_inputs(5, M, d_in, d_out, r, "f32")
    g1 = lib.lora_linear_bwd(X, W, A, B, 2.0, dY)
    g2 = lib.lora_linear_bwd(X, W, A, B, 2.0, dY)
    dXn, dAn, dBn = lib.lora_linear_bwd(X, W, A, B, 2.0, dY, need_dX=False)
    Y1 = lib.lora_linear_fwd(X, W, A, B, 2.0)
    Y2 = lib.lora_linear_fwd(X, W, A, B, 2.0)
    torch.cuda.synchronize()
    assert dXn is None
    assert torch.equal(Y1, Y2)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)
    # the gradients of A and B do not depend on whether dX is formed
    assert torch.equal(dAn, g1[1]) and torch.equal(dBn, g1[2])
