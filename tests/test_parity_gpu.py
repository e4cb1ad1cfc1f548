"""GPU parity of the HIP library against the float64 oracle, at sizes the
oracle finishes in seconds (several tiles plus ragged tails), through the
C ABI via the thin binding.  Bar: max|gpu - ref| / max|ref| <= 1e-5 (fp32
inputs) or 2e-2 (bf16 inputs, fp32 accumulate); exact for integer inputs;
bit-exact for NF4 dequantisation and for run-to-run repeats."""
import math

import numpy as np
import pytest
import torch

import oracle as O
from synth import gen
from tests.helpers import TOL, cpu64, int_inputs, lora_inputs, rel

pytestmark = pytest.mark.gpu

SHAPES = [
    # (M, d_in, d_out, r)
    (1, 64, 64, 1),
    (7, 136, 72, 3),
    (129, 264, 392, 16),
    (300, 520, 1032, 64),
    (1000, 1024, 520, 8),
    (2088, 520, 7680, 64),   # 256x256 tiles with ragged M and contraction tails
    (4100, 4096, 1024, 16),
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", SHAPES)
def test_fwd_bwd_parity(lib, dtype, shape):
    M, d_in, d_out, r = shape
    s = 16.0 / r
    X, W, A, B, dY = lora_inputs(100 + M, M, d_in, d_out, r, dtype)
    Y = lib.lora_linear_fwd(X, W, A, B, s)
    dX, dA, dB = lib.lora_linear_bwd(X, W, A, B, s, dY)
    torch.cuda.synchronize()
    Yr = O.lora_forward(X, W, A, B, s)
    dXr, dAr, dBr = O.lora_backward(X, W, A, B, s, dY)
    tol = TOL[dtype]
    errs = dict(Y=rel(Y, Yr), dX=rel(dX, dXr), dA=rel(dA, dAr), dB=rel(dB, dBr))
    print(dtype, shape, errs)
    assert all(e <= tol for e in errs.values()), errs


def test_config1_fp32_full(lib):
    from synth import CONFIGS
    from synth.configs import Inputs

    c = CONFIGS[1]
    inp = Inputs(c, device="cuda")
    p = c.projections[0]
    X, W, A, B, dY = inp.X(p), inp.W(p), inp.A(p), inp.B(p), inp.dY(p)
    Y = lib.lora_linear_fwd(X, W, A, B, c.scale)
    dX, dA, dB = lib.lora_linear_bwd(X, W, A, B, c.scale, dY)
    torch.cuda.synchronize()
    Yr = O.lora_forward(X, W, A, B, c.scale)
    dXr, dAr, dBr = O.lora_backward(X, W, A, B, c.scale, dY)
    errs = dict(Y=rel(Y, Yr), dX=rel(dX, dXr), dA=rel(dA, dAr), dB=rel(dB, dBr))
    print("config1", errs)
    assert all(e <= 1e-5 for e in errs.values()), errs


@pytest.mark.parametrize("dtype,M,d_in,d_out,r", [("bf16", 1000, 40, 40, 2), ("bf16", 67, 32, 136, 1),
                                                  ("f32", 530, 264, 136, 5), ("bf16", 3000, 40, 48, 2)])
def test_integer_inputs_exact(lib, dtype, M, d_in, d_out, r):
    # |values| <= 1 and small contractions keep every result an integer that the
    # output type (bf16: up to 256) and the bf16 panels hold exactly.
    X, W, A, B, dY = int_inputs(7 + M, M, d_in, d_out, r, dtype)
    s = 2.0
    Y = lib.lora_linear_fwd(X, W, A, B, s)
    dX, dA, dB = lib.lora_linear_bwd(X, W, A, B, s, dY)
    torch.cuda.synchronize()
    Yr = O.lora_forward(X, W, A, B, s)
    dXr, dAr, dBr = O.lora_backward(X, W, A, B, s, dY)
    if dtype == "bf16":
        assert np.abs(Yr).max() <= 256 and np.abs(dXr).max() <= 256
    assert np.array_equal(cpu64(Y), Yr)
    assert np.array_equal(cpu64(dX), dXr)
    assert np.array_equal(cpu64(dA), dAr)
    assert np.array_equal(cpu64(dB), dBr)


# Whole-tile shapes: M, d_out and d_in multiples of 256 with at least 256
# tiles of 256 x 256 in the forward and in the input gradient, so both run on
# the whole-tile ping-pong kernel; ragged ranks exercise its masked rank-r
# segment.  Y and dX are compared on 256 sampled rows, dA and dB in full.
WHOLE = [(4096, 4096, 4096, 1), (4096, 4096, 4096, 24), (4096, 4096, 4096, 100),
         (4096, 4096, 4096, 256), (8192, 4096, 2048, 64)]


def _sample_rows(M, n=256, seed=5):
    rng = np.random.default_rng(seed)
    return np.sort(np.concatenate([[0, M - 1], rng.choice(np.arange(1, M - 1), n - 2, replace=False)]))


@pytest.mark.parametrize("shape", WHOLE, ids=[f"{m}x{i}x{o}r{r}" for m, i, o, r in WHOLE])
def test_whole_tile_parity(lib, shape):
    M, d_in, d_out, r = shape
    s = 16.0 / r
    X, W, A, B, dY = lora_inputs(900 + r, M, d_in, d_out, r, "bf16")
    Y = lib.lora_linear_fwd(X, W, A, B, s)
    dX, dA, dB = lib.lora_linear_bwd(X, W, A, B, s, dY)
    torch.cuda.synchronize()
    rows = _sample_rows(M)
    tr = torch.from_numpy(rows).cuda()
    Yr = O.lora_forward(X[tr], W, A, B, s)
    dXr = O.lora_grad_x(W, A, B, s, dY[tr])
    dAr, dBr = O.lora_grad_ab(X, A, B, s, dY)
    errs = dict(Y=rel(Y[tr], Yr), dX=rel(dX[tr], dXr), dA=rel(dA, dAr), dB=rel(dB, dBr))
    print(shape, errs)
    assert all(e <= TOL["bf16"] for e in errs.values()), errs


def _sparse_int(g, shape, density, device="cuda"):
    v = torch.randint(-1, 2, shape, generator=g)
    keep = torch.rand(shape, generator=g) < density
    return (v * keep).to(torch.bfloat16).to(device)


def test_whole_tile_integer_exact(lib):
    # Sparse {-1, 0, 1} inputs keep every sum, panel and output a small
    # integer (checked below), so the whole-tile kernel must match exactly.
    M, d_in, d_out, r, s = 4096, 4096, 4096, 16, 1.0
    g = torch.Generator().manual_seed(77)
    X = _sparse_int(g, (M, d_in), 1 / 16)
    W = _sparse_int(g, (d_out, d_in), 1.0)
    A = _sparse_int(g, (r, d_in), 1.0)
    B = _sparse_int(g, (d_out, r), 1 / 4)
    dY = _sparse_int(g, (M, d_out), 1 / 16)
    Y = lib.lora_linear_fwd(X, W, A, B, s)
    dX, dA, dB = lib.lora_linear_bwd(X, W, A, B, s, dY)
    torch.cuda.synchronize()
    rows = _sample_rows(M, 512, 6)
    tr = torch.from_numpy(rows).cuda()
    Yr = O.lora_forward(X[tr], W, A, B, s)
    dXr = O.lora_grad_x(W, A, B, s, dY[tr])
    dAr, dBr = O.lora_grad_ab(X, A, B, s, dY)
    P, Q = O.lora_panel(X, A), cpu64(dY) @ cpu64(B)
    assert np.abs(P).max() <= 256 and np.abs(Q).max() <= 256
    assert np.abs(Yr).max() <= 256 and np.abs(dXr).max() <= 256
    assert np.array_equal(cpu64(Y[tr]), Yr)
    assert np.array_equal(cpu64(dX[tr]), dXr)
    assert np.array_equal(cpu64(dA), dAr)
    assert np.array_equal(cpu64(dB), dBr)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_w_zero_isolates_lora_term(lib, dtype):
    M, d_in, d_out, r = 777, 512, 640, 16
    X, W, A, B, dY = lora_inputs(5, M, d_in, d_out, r, dtype)
    W = torch.zeros_like(W)
    Y = lib.lora_linear_fwd(X, W, A, B, 1.0)
    dX, dA, dB = lib.lora_linear_bwd(X, W, A, B, 1.0, dY)
    torch.cuda.synchronize()
    Yr = O.lora_forward(X, W, A, B, 1.0)
    dXr, dAr, dBr = O.lora_backward(X, W, A, B, 1.0, dY)
    tol = TOL[dtype]
    assert rel(Y, Yr) <= tol and rel(dX, dXr) <= tol
    assert rel(dA, dAr) <= tol and rel(dB, dBr) <= tol


def test_b_zero_gives_zero_dA(lib):
    X, W, A, B, dY = lora_inputs(9, 300, 256, 384, 8, "bf16")
    B = torch.zeros_like(B)
    Y = lib.lora_linear_fwd(X, W, A, B, 2.0)
    dX, dA, dB = lib.lora_linear_bwd(X, W, A, B, 2.0, dY)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dA).item() == 0
    assert rel(Y, O.lora_forward(X, W, A, B, 2.0)) <= 2e-2


def test_dx_optional_and_m_zero(lib):
    X, W, A, B, dY = lora_inputs(11, 200, 128, 256, 8, "bf16")
    dX, dA, dB = lib.lora_linear_bwd(X, W, A, B, 2.0, dY, need_dX=False)
    assert dX is None
    _, dAr, dBr = O.lora_backward(X, W, A, B, 2.0, dY)
    assert rel(dA, dAr) <= 2e-2 and rel(dB, dBr) <= 2e-2
    # M = 0: empty output, zero gradients of A and B
    X0, dY0 = X[:0], dY[:0]
    Y0 = lib.lora_linear_fwd(X0, W, A, B, 2.0)
    dA0 = torch.full_like(dA, 7.0)
    dB0 = torch.full_like(dB, 7.0)
    lib.lora_linear_bwd(X0, W, A, B, 2.0, dY0, out=(None, dA0, dB0))
    torch.cuda.synchronize()
    assert Y0.shape == (0, 256)
    assert torch.count_nonzero(dA0).item() == 0 and torch.count_nonzero(dB0).item() == 0


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_deterministic_repeats(lib, dtype):
    X, W, A, B, dY = lora_inputs(13, 2050, 1024, 1536, 64, dtype)
    outs = []
    for _ in range(2):
        Y = lib.lora_linear_fwd(X, W, A, B, 0.25)
        dX, dA, dB = lib.lora_linear_bwd(X, W, A, B, 0.25, dY)
        outs.append([Y, dX, dA, dB])
    torch.cuda.synchronize()
    for a, b in zip(*outs):
        assert torch.equal(a, b)


# ---------------------------------------------------------------------------
# RoPE
# ---------------------------------------------------------------------------

def test_rope_cache_values(lib):
    cos, sin = lib.rope_cache(2048, 128, 500000.0)
    torch.cuda.synchronize()
    a = O.rope_angles(np.arange(2048), 128, 500000.0)
    # fp64 on both sides, rounded once to fp32: equal up to one fp32 rounding step
    assert np.abs(cpu64(cos) - O.round_f32(np.cos(a))).max() <= 2.0 ** -24
    assert np.abs(cpu64(sin) - O.round_f32(np.sin(a))).max() <= 2.0 ** -24
    assert np.mean(cpu64(cos) == O.round_f32(np.cos(a))) > 0.999


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("M,d_in,d_out,r,seq", [(300, 264, 256, 16, 100), (2100, 1024, 4096, 64, 2048),
                                              (4096, 1024, 4096, 40, 2048),
                                                (4096, 512, 1024, 8, 4096), (4100, 256, 4096, 16, 2048)])
def test_rope_fwd_bwd_parity(lib, dtype, M, d_in, d_out, r, seq):
    X, W, A, B, dY = lora_inputs(17 + M, M, d_in, d_out, r, dtype)
    pos = torch.from_numpy(gen.positions_mod(M, seq)).cuda()
    cos, sin = lib.rope_cache(seq, 128, 500000.0)
    s = 16.0 / r
    Y = lib.lora_qk_rope_fwd(X, W, A, B, s, pos, cos, sin)
    dX, dA, dB = lib.lora_qk_rope_bwd(X, W, A, B, s, pos, cos, sin, dY)
    torch.cuda.synchronize()
    p = pos.cpu().numpy()
    Yr = O.qk_rope_forward(X, W, A, B, s, p)
    dXr, dAr, dBr = O.qk_rope_backward(X, W, A, B, s, p, dY)
    tol = TOL[dtype]
    errs = dict(Y=rel(Y, Yr), dX=rel(dX, dXr), dA=rel(dA, dAr), dB=rel(dB, dBr))
    print(dtype, M, errs)
    assert all(e <= tol for e in errs.values()), errs


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_rope_position_zero_is_identity(lib, dtype):
    M, d_in, d_out, r = 700, 256, 512, 16
    X, W, A, B, dY = lora_inputs(23, M, d_in, d_out, r, dtype)
    pos = torch.zeros(M, dtype=torch.int32, device="cuda")
    cos, sin = lib.rope_cache(4, 128, 500000.0)
    Y = lib.lora_qk_rope_fwd(X, W, A, B, 1.0, pos, cos, sin)
    Y0 = lib.lora_linear_fwd(X, W, A, B, 1.0)
    g = lib.lora_qk_rope_bwd(X, W, A, B, 1.0, pos, cos, sin, dY)
    g0 = lib.lora_linear_bwd(X, W, A, B, 1.0, dY)
    torch.cuda.synchronize()
    assert torch.equal(Y, Y0)
    for a, b in zip(g, g0):
        assert torch.equal(a, b)


# each RoPE path: one-launch few-token forward, few-token split partials,
# generic 128 x 128 tiles, whole 256 x 256 tiles
@pytest.mark.parametrize("M,d_out", [(40, 512), (200, 512), (2048, 2048), (4096, 4096)])
def test_rope_out_of_range_positions_give_zero_rows(lib, M, d_out):
    # positions just outside [0, max_pos) read no cache row: their rows of Y
    # are zeros and their gradient is taken as zero; every other row is the
    # plain RoPE layer's
    d_in, r, seq = 256, 16, 64
    X, W, A, B, dY = lora_inputs(29 + M, M, d_in, d_out, r, "bf16")
    p = gen.positions_mod(M, seq).astype(np.int32)
    bad = np.array([1, M // 2, M - 1])
    p[bad] = [seq, -1, seq + 3]
    pos = torch.from_numpy(p).cuda()
    cos, sin = lib.rope_cache(seq, 128, 500000.0)
    s = 1.0
    Y = lib.lora_qk_rope_fwd(X, W, A, B, s, pos, cos, sin)
    dX, dA, dB = lib.lora_qk_rope_bwd(X, W, A, B, s, pos, cos, sin, dY)
    torch.cuda.synchronize()
    good = np.setdiff1d(np.arange(M), bad)
    pc = np.where((p >= 0) & (p < seq), p, 0)
    assert np.all(cpu64(Y)[bad] == 0.0)
    assert rel(Y[torch.from_numpy(good).cuda()], O.qk_rope_forward(X[torch.from_numpy(good).cuda()], W, A, B, s,
                                                                      pc[good])) <= TOL["bf16"]
    dY0 = cpu64(dY)
    dY0[bad] = 0.0
    dXr, dAr, dBr = O.qk_rope_backward(X, W, A, B, s, pc, dY0)
    assert np.all(cpu64(dX)[bad] == 0.0)
    errs = dict(dX=rel(dX, dXr), dA=rel(dA, dAr), dB=rel(dB, dBr))
    print(M, d_out, errs)
    assert all(e <= TOL["bf16"] for e in errs.values()), errs


def test_rope_largest_cache_top_rows(lib):
    # the largest cache the q/k projections accept (2^23 - 1 rows, more than
    # 1 GiB each for cos and sin): positions in its top rows, where the
    # whole-tile epilogue's 32-bit byte offsets into the cache are largest,
    # one position on the last row, one just past it and one negative (zero
    # rows), one at 0
    from lora_linear_layers_amd import _lib

    M, d_in, d_out, r = 4096, 256, 4096, 16
    max_pos = (1 << 23) - 1
    X, W, A, B, dY = lora_inputs(41, M, d_in, d_out, r, "bf16")
    p = (max_pos - 1 - (np.arange(M) % 97)).astype(np.int32)
    p[5], p[M // 3], p[M // 2], p[M - 2] = max_pos - 1, max_pos, -7, 0
    pos = torch.from_numpy(p).cuda()
    cos, sin = lib.rope_cache(max_pos, 128, 500000.0)
    _lib.profile_begin(64)
    Y = lib.lora_qk_rope_fwd(X, W, A, B, 1.0, pos, cos, sin)
    torch.cuda.synchronize()
    _lib.profile_end()
    assert "gemm_bf16_256x256_nt_rope" in _lib.profile_report()
    dX, dA, dB = lib.lora_qk_rope_bwd(X, W, A, B, 1.0, pos, cos, sin, dY)
    torch.cuda.synchronize()
    del cos, sin
    bad = np.array([M // 3, M // 2])
    good = np.setdiff1d(np.arange(M), bad)
    pc = np.where((p >= 0) & (p < max_pos), p, 0)
    assert np.all(cpu64(Y)[bad] == 0.0)
    gi = torch.from_numpy(good).cuda()
    assert rel(Y[gi], O.qk_rope_forward(X[gi], W, A, B, 1.0, pc[good])) <= TOL["bf16"]
    dY0 = cpu64(dY)
    dY0[bad] = 0.0
    dXr, dAr, dBr = O.qk_rope_backward(X, W, A, B, 1.0, pc, dY0)
    errs = dict(dX=rel(dX, dXr), dA=rel(dA, dAr), dB=rel(dB, dBr))
    print(errs)
    assert all(e <= TOL["bf16"] for e in errs.values()), errs


# ---------------------------------------------------------------------------
# NF4
# ---------------------------------------------------------------------------

def _nf4_weight(seed, d_out, d_in):
    codes = gen.nf4_random_codes(seed, d_out * d_in).cuda()
    absmax = gen.nf4_random_absmax(seed + 1, d_out * d_in // 64, 1.0 / math.sqrt(d_in)).cuda()
    return codes, absmax


def test_nf4_dequant_bit_exact(lib):
    tab = gen.nf4_table()
    d_out, d_in = 96, 1024
    codes, absmax = _nf4_weight(31, d_out, d_in)
    w = lib.nf4_dequant(codes, absmax, tab, d_out * d_in)
    torch.cuda.synchronize()
    ref = O.nf4_dequant(codes.cpu().numpy(), absmax.cpu().numpy(), tab, d_out, d_in).reshape(-1)
    got = cpu64(w)
    assert np.array_equal(got, ref)
    # and on hand-made extremes: every code with a few absmax values
    codes = torch.tensor(np.tile(np.arange(256, dtype=np.uint8), 4), device="cuda")
    absmax = torch.tensor([1.0, 0.5, 3.0e-3, 7.25], dtype=torch.float32, device="cuda").repeat_interleave(8)
    w = lib.nf4_dequant(codes, absmax, tab, 2048)
    torch.cuda.synchronize()
    ref = O.nf4_dequant(codes.cpu().numpy(), absmax.cpu().numpy(), tab, 1, 2048).reshape(-1)
    assert np.array_equal(cpu64(w), ref)


@pytest.mark.parametrize("M,d_in,d_out,r", [(129, 256, 264, 8), (1500, 1024, 1032, 64), (2056, 640, 7424, 16),
                                             (4100, 4096, 512, 8)])
def test_nf4_fwd_bwd_parity(lib, M, d_in, d_out, r):
    tab = gen.nf4_table()
    X, _, A, B, dY = lora_inputs(41 + M, M, d_in, d_out, r, "bf16")
    codes, absmax = _nf4_weight(43 + M, d_out, d_in)
    s = 16.0 / r
    Y = lib.nf4_lora_linear_fwd(X, codes, absmax, tab, A, B, s, d_out)
    dX, dA, dB = lib.nf4_lora_linear_bwd(X, codes, absmax, tab, A, B, s, dY)
    torch.cuda.synchronize()
    c, am = codes.cpu().numpy(), absmax.cpu().numpy()
    Yr = O.nf4_lora_forward(X, c, am, tab, A, B, s, d_out, d_in)
    dXr, dAr, dBr = O.nf4_lora_backward(X, c, am, tab, A, B, s, dY, d_out, d_in)
    errs = dict(Y=rel(Y, Yr), dX=rel(dX, dXr), dA=rel(dA, dAr), dB=rel(dB, dBr))
    print("nf4", M, errs)
    assert all(e <= 2e-2 for e in errs.values()), errs
    # the NF4 GEMM equals the bf16 GEMM on the dequantised weight, to rounding
    Wd = lib.nf4_dequant(codes, absmax, tab, d_out * d_in).view(d_out, d_in)
    Yb = lib.lora_linear_fwd(X, Wd, A, B, s)
    torch.cuda.synchronize()
    assert torch.equal(Y, Yb)


@pytest.mark.parametrize("M,d_in,d_out,r", [(512, 1024, 1024, 16), (768, 640, 512, 64), (512, 128, 768, 8),
                                             (512, 64, 256, 3), (1024, 320, 512, 200), (4096, 1024, 4096, 16)])
def test_nf4_load_stage_forward(lib, M, d_in, d_out, r):
    # the whole-tile GEMM that expands NF4 codes in its load stage (one and
    # two stages of W, several rank stages, a ragged rank): within the bar of
    # the oracle; and where the dequantise-once path also runs whole 256 x 256
    # tiles (at least 256 of them), bit-equal to it: the same tile, stage and
    # MFMA order on the same W values
    from lora_linear_layers_amd import _lib
    tab = gen.nf4_table()
    X, _, A, B, _ = lora_inputs(61 + M + r, M, d_in, d_out, r, "bf16")
    codes, absmax = _nf4_weight(63 + d_in, d_out, d_in)
    s = 16.0 / r
    prev = _lib.set_nf4_fwd_path("load_stage")
    try:
        _lib.profile_only(None)
        _lib.profile_begin(64)
        Y = lib.nf4_lora_linear_fwd(X, codes, absmax, tab, A, B, s, d_out)
        torch.cuda.synchronize()
        _lib.profile_end()
        kinds = set(_lib.profile_report())
        _lib.set_nf4_fwd_path("dequant")
        Yd = lib.nf4_lora_linear_fwd(X, codes, absmax, tab, A, B, s, d_out)
        torch.cuda.synchronize()
    finally:
        _lib.set_nf4_fwd_path(prev)
    assert "gemm_nf4_256x256_nt_whole" in kinds, kinds
    Yr = O.nf4_lora_forward(X, codes.cpu().numpy(), absmax.cpu().numpy(), tab, A, B, s, d_out, d_in)
    e = rel(Y, Yr)
    print("nf4 load stage", M, d_in, d_out, r, e)
    assert e <= 2e-2
    if (M // 256) * (d_out // 256) >= 256:
        assert torch.equal(Y, Yd)
    else:
        assert rel(Yd, Yr) <= 2e-2


def test_nf4_whole_tile_backward_equals_bf16_on_dequantised(lib):
    # from 512 tokens on whole tiles the NF4 backward dequantises straight
    # into W^T; the result must equal, bit for bit, the bf16 backward on the
    # dequantised weight (which transposes W itself)
    tab = gen.nf4_table()
    M, d_in, d_out, r = 4096, 4096, 1024, 16
    X, _, A, B, dY = lora_inputs(8, M, d_in, d_out, r, "bf16")
    codes, absmax = _nf4_weight(9, d_out, d_in)
    g = lib.nf4_lora_linear_bwd(X, codes, absmax, tab, A, B, 2.0, dY)
    Wd = lib.nf4_dequant(codes, absmax, tab, d_out * d_in).view(d_out, d_in)
    g0 = lib.lora_linear_bwd(X, Wd, A, B, 2.0, dY)
    torch.cuda.synchronize()
    for a, b in zip(g, g0):
        assert torch.equal(a, b)
