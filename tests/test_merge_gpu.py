"""GPU parity of lora_merge (W + s B A folded into the weight for inference)
against the float64 oracle: within one rounding of the output type for bf16,
1e-5 for fp32, exact for integer inputs; in place equals out of place;
unmerging restores W up to the rounding the merge did; the merged weight's
forward equals the unmerged fused forward."""
import numpy as np
import pytest
import torch

import oracle as O
from tests.helpers import TOL, cpu64, int_inputs, lora_inputs, rel

pytestmark = pytest.mark.gpu

SHAPES = [(4096, 4096, 16), (1032, 520, 3), (14336, 4096, 64), (64, 8, 1), (520, 1032, 256)]


def _bf16_ulp(x):
    # spacing of bf16 values at |x| (normal range): 2^(e - 7)
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -126)))
    return 2.0 ** (e - 7)


def _merge_bound(W, A, B, s, ref):
    # one bf16 rounding of the result, plus the fp32 accumulation of r
    # products and W (each step rounds relative to the operands, which matters
    # where W and s B A nearly cancel)
    r = A.shape[0]
    mag = np.abs(cpu64(W)) + abs(s) * (np.abs(cpu64(B)) @ np.abs(cpu64(A)))
    return _bf16_ulp(ref) + (r + 2) * 2.0 ** -24 * mag


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", SHAPES, ids=[f"{o}x{i}r{r}" for o, i, r in SHAPES])
def test_merge_parity(lib, dtype, shape):
    d_out, d_in, r = shape
    s = 16.0 / r
    _, W, A, B, _ = lora_inputs(700 + r, 1, d_in, d_out, r, dtype)
    Wm = lib.lora_merge(W, A, B, s)
    torch.cuda.synchronize()
    ref = O.merged_weight(W, A, B, s)
    got = cpu64(Wm)
    err = rel(got, ref)
    print(dtype, shape, err)
    assert err <= TOL[dtype]
    if dtype == "bf16":
        # one fp32 accumulation then one rounding: within one bf16 step of the
        # exact value, and equal to its correctly rounded value almost always
        assert np.all(np.abs(got - ref) <= _merge_bound(W, A, B, s, ref))
        assert np.mean(got == O.round_bf16(ref)) > 0.99


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_merge_in_place_and_unmerge(lib, dtype):
    d_out, d_in, r = 2048, 1024, 16
    s = 1.0
    _, W, A, B, _ = lora_inputs(11, 1, d_in, d_out, r, dtype)
    Wm = lib.lora_merge(W, A, B, s)
    Wi = W.clone()
    lib.lora_merge(Wi, A, B, s, out=Wi)
    torch.cuda.synchronize()
    assert torch.equal(Wm, Wi)
    Wu = lib.lora_merge(Wm, A, B, -s)
    torch.cuda.synchronize()
    # the unmerge removes exactly the merged term up to two roundings
    w0, wu = cpu64(W), cpu64(Wu)
    if dtype == "bf16":
        # two roundings (merge, then unmerge), each within the merge bound
        b = _merge_bound(W, A, B, s, O.merged_weight(W, A, B, s)) + _merge_bound(Wm, A, B, s, w0)
        assert np.all(np.abs(wu - w0) <= b)
    else:
        assert rel(wu, w0) <= 1e-5


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_merge_integer_exact(lib, dtype):
    _, W, A, B, _ = int_inputs(5, 1, 264, 136, 7, dtype)
    Wm = lib.lora_merge(W, A, B, 2.0)
    torch.cuda.synchronize()
    assert np.array_equal(cpu64(Wm), O.merged_weight(W, A, B, 2.0))


def test_merged_forward_equals_fused_forward(lib):
    # fp32, so that only accumulation order separates the two paths
    M, d_in, d_out, r = 300, 520, 1032, 16
    X, W, A, B, _ = lora_inputs(19, M, d_in, d_out, r, "f32")
    s = 2.0
    Y = lib.lora_linear_fwd(X, W, A, B, s)
    Wm = lib.lora_merge(W, A, B, s)
    torch.cuda.synchronize()
    Ym = cpu64(X) @ cpu64(Wm).T  # the merged weight applied exactly
    assert rel(Y, Ym) <= 1e-5
