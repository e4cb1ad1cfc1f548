"""GPU parity of the SwiGLU entry points (gate / up pair -> silu(G) * U and its
backward) against the float64 oracle.  Whole-tile bf16 shapes run gate and up
as one GEMM with the SwiGLU epilogue; other shapes (ragged, fp32, NF4 with few
tokens) form G and U with the group path and H elementwise.  The GPU backward
uses the G and U its forward stored; the oracle uses its own exact G and U."""
import math

import numpy as np
import pytest
import torch

import oracle as O
from lora_linear_layers_amd import _lib
from synth import gen
from tests.helpers import TOL, cpu64, draw, rel

pytestmark = pytest.mark.gpu


def _pair(seed, M, d_in, d_ff, rg, ru, dtype, nf4=False):
    X = draw(seed, (M, d_in), "normal", 1.0, dtype)
    dH = draw(seed + 1, (M, d_ff), "normal", 1.0, dtype)
    members, dense = [], []
    for g, r in enumerate((rg, ru)):
        base = seed + 10 * (g + 1)
        A = draw(base + 2, (r, d_in), "uniform", 1.0 / math.sqrt(d_in), dtype)
        B = draw(base + 3, (d_ff, r), "normal", math.sqrt(0.02), dtype)
        m = dict(A=A, B=B, scale=(16.0 if g == 0 else 8.0) / r)
        if nf4:
            m["codes"] = gen.nf4_random_codes(base + 4, d_ff * d_in).cuda()
            m["absmax"] = gen.nf4_random_absmax(base + 5, d_ff * d_in // 64, 1.0 / math.sqrt(d_in)).cuda()
            W = O.nf4_dequant(m["codes"].cpu().numpy(), m["absmax"].cpu().numpy(), gen.nf4_table(), d_ff, d_in)
        else:
            m["W"] = draw(base + 1, (d_ff, d_in), "normal", 1.0 / math.sqrt(d_in), dtype)
            W = m["W"]
        members.append(m)
        dense.append(W)
    return X, dH, members, dense


def _kinds(fn):
    _lib.profile_begin(512)
    out = fn()
    torch.cuda.synchronize()
    _lib.profile_end()
    return out, set(_lib.profile_report())


def _check(lib, X, dH, members, dense, dtype, fused, table=None):
    (H, G, U), kinds = _kinds(lambda: lib.lora_swiglu_fwd(X, members, table16=table))
    assert ("gemm_bf16_256x256_swiglu" in kinds) == fused, kinds
    (dX, grads), _ = _kinds(lambda: lib.lora_swiglu_bwd(X, members, dH, G, U, table16=table))
    mg, mu = members
    args = (X, dense[0], mg["A"], mg["B"], mg["scale"], dense[1], mu["A"], mu["B"], mu["scale"])
    Hr, Gr, Ur = O.swiglu_forward(*args)
    dXr, dAgr, dBgr, dAur, dBur = O.swiglu_backward(*args, dH)
    errs = dict(H=rel(H, Hr), G=rel(G, Gr), U=rel(U, Ur), dX=rel(dX, dXr), dAg=rel(grads[0][0], dAgr),
                dBg=rel(grads[0][1], dBgr), dAu=rel(grads[1][0], dAur), dBu=rel(grads[1][1], dBur))
    print(dtype, X.shape, "fused" if fused else "elementwise", errs)
    assert all(e <= TOL[dtype] for e in errs.values()), errs
    return H, G, U


@pytest.mark.parametrize("M,d_in,d_ff,rg,ru", [(2048, 1024, 2048, 16, 8), (1024, 512, 1024, 5, 12),
                                               (512, 2048, 4096, 64, 64)])
def test_swiglu_fused_parity(lib, M, d_in, d_ff, rg, ru):
    X, dH, members, dense = _pair(3 + M, M, d_in, d_ff, rg, ru, "bf16")
    _check(lib, X, dH, members, dense, "bf16", fused=True)


def test_swiglu_fused_gu_equal_group_projections(lib):
    # At sizes where the group path also runs the whole-tile kernel, the G and
    # U that the fused GEMM stores equal the group's projections bit for bit:
    # the contraction order is the same and the other member's rank columns
    # only add exact zeros.  H then agrees with silu(G) U to bf16 rounding.
    M, d_in, d_ff = 4096, 1024, 4096
    X, dH, members, dense = _pair(17, M, d_in, d_ff, 16, 8, "bf16")
    (H, G, U), kinds = _kinds(lambda: lib.lora_swiglu_fwd(X, members))
    assert "gemm_bf16_256x256_swiglu" in kinds
    (Yg, Yu), kinds = _kinds(lambda: lib.lora_group_fwd(X, [dict(members[0]), dict(members[1])]))
    # the group's whole-tile GEMM: one launch per member, or every member's
    # tiles in one launch (same main loop, same contraction order)
    assert kinds & {"gemm_bf16_256x256_nt_store", "gemm_bf16_256x256_nt_group"}, kinds
    assert torch.equal(G, Yg) and torch.equal(U, Yu)
    Hs = O.silu(cpu64(G)) * cpu64(U)
    assert rel(H, Hs) <= 2 ** -7


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("M,d_in,d_ff,rg,ru", [(300, 264, 520, 16, 3), (129, 1024, 2048, 64, 8)])
def test_swiglu_elementwise_parity(lib, dtype, M, d_in, d_ff, rg, ru):
    X, dH, members, dense = _pair(40 + M, M, d_in, d_ff, rg, ru, dtype)
    _check(lib, X, dH, members, dense, dtype, fused=False)


@pytest.mark.parametrize("M,fused", [(512, True), (100, False)])
def test_swiglu_nf4_parity(lib, M, fused):
    tab = gen.nf4_table()
    X, dH, members, dense = _pair(70 + M, M, 1024, 1024, 16, 16, "bf16", nf4=True)
    _check(lib, X, dH, members, dense, "bf16", fused=fused, table=tab)


def test_swiglu_without_stored_gu_and_without_dx(lib):
    M, d_in, d_ff = 1024, 512, 1024
    X, dH, members, dense = _pair(91, M, d_in, d_ff, 8, 8, "bf16")
    H1, G, U = lib.lora_swiglu_fwd(X, members)
    H2, G2, U2 = lib.lora_swiglu_fwd(X, members, store_gu=False)
    dX1, g1 = lib.lora_swiglu_bwd(X, members, dH, G, U)
    dX2, g2 = lib.lora_swiglu_bwd(X, members, dH, G, U, need_dX=False)
    torch.cuda.synchronize()
    assert G2 is None and U2 is None and dX2 is None
    assert torch.equal(H1, H2)
    for a, b in zip(g1, g2):
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_swiglu_m_zero(lib):
    X, dH, members, dense = _pair(5, 0, 256, 512, 8, 8, "bf16")
    H, G, U = lib.lora_swiglu_fwd(X, members)
    dX, grads = lib.lora_swiglu_bwd(X, members, dH, G, U)
    torch.cuda.synchronize()
    assert H.shape == (0, 512) and dX.shape == (0, 256)
    for dA, dB in grads:
        assert torch.count_nonzero(dA) == 0 and torch.count_nonzero(dB) == 0
