"""GPU parity of LoRA dropout on the adapter's input against the float64
oracle.  The keep mask is an input drawn here (seeded) and packed to bits;
the same mask feeds the oracle.  Under dropout the rank-r term of dX is added
after the base term, so dX is rounded twice (still within the bar)."""
import numpy as np
import pytest
import torch

import oracle as O
from tests.helpers import TOL, cpu64, lora_inputs, rel

pytestmark = pytest.mark.gpu


def _keep(seed, M, d_in, p):
    g = torch.Generator().manual_seed(seed)
    bits = (torch.rand(M, d_in, generator=g) >= p).to(torch.uint8)
    packed = (bits.view(M, d_in // 8, 8) << torch.arange(8, dtype=torch.uint8)).sum(-1).to(torch.uint8)
    return packed.contiguous().cuda(), bits.bool().numpy()


SHAPES = [(300, 264, 392, 16, 0.1), (2048, 1024, 4096, 64, 0.05), (4096, 4096, 1024, 16, 0.5),
          (16, 4096, 1024, 16, 0.1), (129, 520, 136, 3, 0.3)]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", SHAPES, ids=[f"{m}x{i}x{o}r{r}p{p}" for m, i, o, r, p in SHAPES])
def test_dropout_parity(lib, dtype, shape):
    M, d_in, d_out, r, p = shape
    s = 16.0 / r
    X, W, A, B, dY = lora_inputs(500 + M, M, d_in, d_out, r, dtype)
    keep, kb = _keep(7 + M, M, d_in, p)
    Y = lib.lora_dropout_fwd(X, W, A, B, s, p, keep)
    dX, dA, dB = lib.lora_dropout_bwd(X, W, A, B, s, p, keep, dY)
    torch.cuda.synchronize()
    Yr = O.lora_dropout_forward(X, W, A, B, s, p, kb)
    dXr, dAr, dBr = O.lora_dropout_backward(X, W, A, B, s, p, kb, dY)
    errs = dict(Y=rel(Y, Yr), dX=rel(dX, dXr), dA=rel(dA, dAr), dB=rel(dB, dBr))
    print(dtype, shape, errs)
    assert all(e <= TOL[dtype] for e in errs.values()), errs
    # the packed mask is read the way the oracle reads it
    assert np.array_equal(O.dropout_keep(keep.cpu().numpy(), M, d_in), kb)


def test_dropout_p0_all_kept_equals_plain_layer(lib):
    M, d_in, d_out, r = 1000, 1024, 520, 8
    X, W, A, B, dY = lora_inputs(3, M, d_in, d_out, r, "bf16")
    keep = torch.full((M, d_in // 8), 255, dtype=torch.uint8, device="cuda")
    Y = lib.lora_dropout_fwd(X, W, A, B, 2.0, 0.0, keep)
    dX, dA, dB = lib.lora_dropout_bwd(X, W, A, B, 2.0, 0.0, keep, dY)
    Y0 = lib.lora_linear_fwd(X, W, A, B, 2.0)
    dX0, dA0, dB0 = lib.lora_linear_bwd(X, W, A, B, 2.0, dY)
    torch.cuda.synchronize()
    # same panel inputs and scale: the forward and the adapter gradients are bit-equal
    assert torch.equal(Y, Y0) and torch.equal(dA, dA0) and torch.equal(dB, dB0)
    assert rel(dX, cpu64(dX0)) <= 2 ** -7


def test_dropout_nothing_kept(lib):
    M, d_in, d_out, r = 300, 264, 392, 16
    X, W, A, B, dY = lora_inputs(9, M, d_in, d_out, r, "bf16")
    keep = torch.zeros(M, d_in // 8, dtype=torch.uint8, device="cuda")
    Y = lib.lora_dropout_fwd(X, W, A, B, 1.0, 0.2, keep)
    dX, dA, dB = lib.lora_dropout_bwd(X, W, A, B, 1.0, 0.2, keep, dY)
    torch.cuda.synchronize()
    assert rel(Y, cpu64(X) @ cpu64(W).T) <= TOL["bf16"]
    assert rel(dX, cpu64(dY) @ cpu64(W)) <= TOL["bf16"]
    assert torch.count_nonzero(dA) == 0 and torch.count_nonzero(dB) == 0


# ---------------------------------------------------------------------------
# The mask drawn on the device from Philox4x32-10 (seed, offset)
# ---------------------------------------------------------------------------

MASKS = [(1, 8, 0.5, 0, 0), (3, 520, 0.1, 3407, 0), (129, 264, 0.3, 2 ** 40 + 17, 2 ** 33 + 5),
         (4096, 4096, 0.05, 0xFFFFFFFFFFFFFFFF, 0xFFFFFFFF00000001)]


@pytest.mark.parametrize("case", MASKS, ids=[f"{m}x{k}p{p}" for m, k, p, _, _ in MASKS])
def test_philox_mask_bit_exact(lib, case):
    M, d_in, p, seed, off = case
    keep = lib.lora_dropout_mask(M, d_in, p, seed, off)
    torch.cuda.synchronize()
    ref = O.dropout_pack(O.dropout_mask_philox_np(M * d_in, p, seed, off)).reshape(M, d_in // 8)
    assert np.array_equal(keep.cpu().numpy(), ref)


PHILOX = [(300, 264, 392, 16, 0.1), (2048, 1024, 4096, 64, 0.05), (129, 520, 136, 3, 0.3)]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", PHILOX, ids=[f"{m}x{i}x{o}r{r}p{p}" for m, i, o, r, p in PHILOX])
def test_philox_dropout_parity(lib, dtype, shape):
    # the oracle draws its own mask from its own Philox; the library draws it
    # again in the backward from the same (seed, offset)
    M, d_in, d_out, r, p = shape
    s, seed, off = 16.0 / r, 3407 + M, 11
    X, W, A, B, dY = lora_inputs(900 + M, M, d_in, d_out, r, dtype)
    Y = lib.lora_dropout_philox_fwd(X, W, A, B, s, p, seed, off)
    dX, dA, dB = lib.lora_dropout_philox_bwd(X, W, A, B, s, p, seed, dY, off)
    torch.cuda.synchronize()
    kb = O.dropout_mask_philox_np(M * d_in, p, seed, off).reshape(M, d_in)
    Yr = O.lora_dropout_forward(X, W, A, B, s, p, kb)
    dXr, dAr, dBr = O.lora_dropout_backward(X, W, A, B, s, p, kb, dY)
    errs = dict(Y=rel(Y, Yr), dX=rel(dX, dXr), dA=rel(dA, dAr), dB=rel(dB, dBr))
    print(dtype, shape, errs)
    assert all(e <= TOL[dtype] for e in errs.values()), errs


def test_philox_entry_points_equal_mask_entry_points(lib):
    # drawing the mask inside the call changes nothing but where it comes from
    M, d_in, d_out, r, p, seed = 1000, 1024, 520, 8, 0.1, 99
    X, W, A, B, dY = lora_inputs(21, M, d_in, d_out, r, "bf16")
    keep = lib.lora_dropout_mask(M, d_in, p, seed, 4)
    Y0 = lib.lora_dropout_fwd(X, W, A, B, 2.0, p, keep)
    g0 = lib.lora_dropout_bwd(X, W, A, B, 2.0, p, keep, dY)
    Y1 = lib.lora_dropout_philox_fwd(X, W, A, B, 2.0, p, seed, 4)
    g1 = lib.lora_dropout_philox_bwd(X, W, A, B, 2.0, p, seed, dY, 4)
    torch.cuda.synchronize()
    assert torch.equal(Y0, Y1)
    for a, b in zip(g0, g1):
        assert torch.equal(a, b)
    # another offset draws another mask
    Y2 = lib.lora_dropout_philox_fwd(X, W, A, B, 2.0, p, seed, 5)
    torch.cuda.synchronize()
    assert not torch.equal(Y1, Y2)
