"""Pins of the float64 oracle against what the pages and the mathematics fix.

None of these re-type the oracle's matrix formulas: they use hand-worked
values, brute-force scalar sums on tiny inputs, exact integer arithmetic,
finite differences, invariants of the rotation group, and library routines on
special cases.  CPU only.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle as O

RNG = np.random.default_rng(3407)


def _rand(*shape):
    return RNG.standard_normal(shape)


# ---------------------------------------------------------------------------
# forward
# ---------------------------------------------------------------------------

def test_hand_worked_2x2():
    # X = [1 2], W = I, A = [1 1] (r = 1), B = [1; 2], s = 2.
    # A x = 3, B A x = [3, 6], y = W x + s B A x = [1, 2] + [6, 12] = [7, 14].
    X = np.array([[1.0, 2.0]])
    W = np.eye(2)
    A = np.array([[1.0, 1.0]])
    B = np.array([[1.0], [2.0]])
    Y = O.lora_forward(X, W, A, B, 2.0)
    assert Y.tolist() == [[7.0, 14.0]]
    # dY = [1 1]: dY B = 3; dX = dY W + s (dY B) A = [1,1] + 6 [1,1] = [7, 7];
    # dB = s dY^T (X A^T) = 2 [1;1] 3 = [6; 6]; dA = s (dY B)^T X = 6 [1, 2].
    dX, dA, dB = O.lora_backward(X, W, A, B, 2.0, np.array([[1.0, 1.0]]))
    assert dX.tolist() == [[7.0, 7.0]]
    assert dA.tolist() == [[6.0, 12.0]]
    assert dB.tolist() == [[6.0], [6.0]]


def _brute_forward(X, W, A, B, s):
    """y_t[i] = sum_j W[i][j] x_t[j] + s sum_q B[i][q] sum_j A[q][j] x_t[j], exact."""
    M, k = len(X), len(X[0])
    d, r = len(W), len(A)
    Y = []
    for t in range(M):
        ax = [sum(Fraction(A[q][j]) * Fraction(X[t][j]) for j in range(k)) for q in range(r)]
        row = []
        for i in range(d):
            base = sum(Fraction(W[i][j]) * Fraction(X[t][j]) for j in range(k))
            low = sum(Fraction(B[i][q]) * ax[q] for q in range(r))
            row.append(base + Fraction(s) * low)
        Y.append(row)
    return Y


def _brute_backward(X, W, A, B, s, G):
    """Scalar-sum gradients of L = sum_t sum_i G[t][i] y_t[i], exact."""
    M, k = len(X), len(X[0])
    d, r = len(W), len(A)
    F = Fraction
    ax = [[sum(F(A[q][j]) * F(X[t][j]) for j in range(k)) for q in range(r)] for t in range(M)]
    gb = [[sum(F(G[t][i]) * F(B[i][q]) for i in range(d)) for q in range(r)] for t in range(M)]
    dX = [[sum(F(G[t][i]) * F(W[i][j]) for i in range(d)) + F(s) * sum(gb[t][q] * F(A[q][j]) for q in range(r))
           for j in range(k)] for t in range(M)]
    dB = [[F(s) * sum(F(G[t][i]) * ax[t][q] for t in range(M)) for q in range(r)] for i in range(d)]
    dA = [[F(s) * sum(gb[t][q] * F(X[t][j]) for t in range(M)) for j in range(k)] for q in range(r)]
    return dX, dA, dB


def _small_ints(shape, lo=-3, hi=3):
    return RNG.integers(lo, hi + 1, size=shape).astype(np.float64)


@pytest.mark.parametrize("M,k,d,r", [(3, 5, 4, 2), (1, 8, 8, 1), (4, 3, 7, 3)])
def test_integer_brute_force_exact(M, k, d, r):
    X, W, A, B, G = (_small_ints(s) for s in [(M, k), (d, k), (r, k), (d, r), (M, d)])
    s = 2.0
    Y = O.lora_forward(X, W, A, B, s)
    assert Y.tolist() == [[float(v) for v in row] for row in _brute_forward(X.tolist(), W.tolist(), A.tolist(), B.tolist(), s)]
    dX, dA, dB = O.lora_backward(X, W, A, B, s, G)
    bX, bA, bB = _brute_backward(X.tolist(), W.tolist(), A.tolist(), B.tolist(), s, G.tolist())
    assert dX.tolist() == [[float(v) for v in row] for row in bX]
    assert dA.tolist() == [[float(v) for v in row] for row in bA]
    assert dB.tolist() == [[float(v) for v in row] for row in bB]


def test_panel_brute_force_exact():
    # P[t][q] = sum_j X[t][j] A[q][j]: the rank-r projection A x of each token,
    # summed exactly over Fractions on small integers, and a hand value.
    X, A = _small_ints((4, 7)), _small_ints((3, 7))
    ref = [[float(sum(Fraction(A[q][j]) * Fraction(X[t][j]) for j in range(7))) for q in range(3)] for t in range(4)]
    assert O.lora_panel(X, A).tolist() == ref
    # x = [1, 2, 3], A = [[1, 0, -1], [2, 1, 0]]: A x = [1 - 3, 2 + 2] = [-2, 4]
    P = O.lora_panel(np.array([[1.0, 2.0, 3.0]]), np.array([[1.0, 0.0, -1.0], [2.0, 1.0, 0.0]]))
    assert P.tolist() == [[-2.0, 4.0]]


def test_brute_force_float_shapes():
    X, W, A, B = _rand(2, 6), _rand(5, 6), _rand(3, 6), _rand(5, 3)
    ref = np.array([[float(v) for v in row] for row in _brute_forward(X.tolist(), W.tolist(), A.tolist(), B.tolist(), 0.25)])
    assert np.abs(O.lora_forward(X, W, A, B, 0.25) - ref).max() < 1e-12


def test_special_cases_B_zero_and_A_zero():
    X, W, A, B, G = _rand(4, 6), _rand(5, 6), _rand(2, 6), _rand(5, 2), _rand(4, 5)
    base = np.array([[sum(W[i, j] * X[t, j] for j in range(6)) for i in range(5)] for t in range(4)])
    # B = 0: y = W x, dA = 0 exactly
    Y = O.lora_forward(X, W, A, np.zeros_like(B), 0.5)
    assert np.abs(Y - base).max() < 1e-12
    dX, dA, dB = O.lora_backward(X, W, A, np.zeros_like(B), 0.5, G)
    assert np.all(dA == 0.0)
    # A = 0: y = W x, dB = 0 exactly
    Y = O.lora_forward(X, W, np.zeros_like(A), B, 0.5)
    assert np.abs(Y - base).max() < 1e-12
    dX, dA, dB = O.lora_backward(X, W, np.zeros_like(A), B, 0.5, G)
    assert np.all(dB == 0.0)


def test_merged_weight_equals_unmerged():
    # Folding the branch into the weight gives the same output (P2 5.1, P5 3.2).
    X, W, A, B = _rand(7, 9), _rand(6, 9), _rand(4, 9), _rand(6, 4)
    s = 4.0
    Wm = O.merged_weight(W, A, B, s)
    merged = np.array([[sum(Wm[i, j] * X[t, j] for j in range(9)) for i in range(6)] for t in range(7)])
    unmerged = O.lora_forward(X, W, A, B, s)
    assert np.abs(merged - unmerged).max() / np.abs(unmerged).max() < 1e-12


def test_scale_enters_linearly():
    X, W, A, B = _rand(3, 5), _rand(4, 5), _rand(2, 5), _rand(4, 2)
    y0 = O.lora_forward(X, W, A, B, 0.0)
    y1 = O.lora_forward(X, W, A, B, 1.0)
    y3 = O.lora_forward(X, W, A, B, 3.0)
    assert np.abs((y3 - y0) - 3.0 * (y1 - y0)).max() < 1e-12


def test_parameter_count_4096_r16():
    # A in R^{r x k}, B in R^{d x r}: 4096 x 4096 with r = 16 trains 2*4096*16 = 131072 values.
    d = k = 4096
    r = 16
    assert r * k + d * r == 131072


# ---------------------------------------------------------------------------
# backward: finite differences and invariants
# ---------------------------------------------------------------------------

def _loss(X, W, A, B, s, G):
    return float(np.sum(G * O.lora_forward(X, W, A, B, s)))


def _fd(f, P, h=1e-3):
    g = np.zeros_like(P)
    for idx in np.ndindex(P.shape):
        old = P[idx]
        P[idx] = old + h
        fp = f()
        P[idx] = old - h
        fm = f()
        P[idx] = old
        g[idx] = (fp - fm) / (2 * h)
    return g


@pytest.mark.parametrize("s", [2.0, 0.25])
def test_backward_matches_finite_differences(s):
    M, k, d, r = 3, 5, 4, 2
    X, W, A, B, G = _rand(M, k), _rand(d, k), _rand(r, k), _rand(d, r), _rand(M, d)
    dX, dA, dB = O.lora_backward(X, W, A, B, s, G)
    f = lambda: _loss(X, W, A, B, s, G)  # noqa: E731
    # L is linear in each of X, A, B separately: central differences are exact up to rounding.
    assert np.abs(_fd(f, X) - dX).max() < 1e-9
    assert np.abs(_fd(f, A) - dA).max() < 1e-9
    assert np.abs(_fd(f, B) - dB).max() < 1e-9


def test_backward_inner_product_identities():
    # Y is homogeneous of degree 1 in X, in A and in B, so
    #   <dX, X> = <G, Y>,  <dA, A> = <dB, B> = <G, Y - X W^T>.
    M, k, d, r = 6, 7, 5, 3
    X, W, A, B, G = _rand(M, k), _rand(d, k), _rand(r, k), _rand(d, r), _rand(M, d)
    s = 0.5
    Y = O.lora_forward(X, W, A, B, s)
    dX, dA, dB = O.lora_backward(X, W, A, B, s, G)
    lora_part = Y - O.lora_forward(X, W, A, np.zeros_like(B), s)
    assert abs(np.sum(dX * X) - np.sum(G * Y)) < 1e-10
    assert abs(np.sum(dA * A) - np.sum(G * lora_part)) < 1e-10
    assert abs(np.sum(dB * B) - np.sum(G * lora_part)) < 1e-10


# ---------------------------------------------------------------------------
# RoPE (P1 RoPE缓存集成; pairing and base are readings)
# ---------------------------------------------------------------------------

def test_rope_hand_values_rotate_half():
    # head_dim 4: pairs are (0, 2) and (1, 3); frequency 0 is 1, frequency 1 is theta^(-2/4).
    Z = np.array([[1.0, 0.0, 0.0, 0.0], [0.0, 1.0, 0.0, 0.0]])
    pos = np.array([1, 2])
    Y = O.rope_rotate(Z, pos, 4, 10000.0)
    assert np.allclose(Y[0], [math.cos(1.0), 0.0, math.sin(1.0), 0.0], atol=1e-15)
    a = 2 * 10000.0 ** -0.5
    assert np.allclose(Y[1], [0.0, math.cos(a), 0.0, math.sin(a)], atol=1e-15)


def test_rope_angles_closed_form():
    a = O.rope_angles(np.array([0, 1, 7, 8191]), 128, 500000.0)
    assert np.all(a[:, 0] == np.array([0, 1, 7, 8191], dtype=np.float64))  # theta^0 = 1
    assert a[2, 63] == pytest.approx(7 * math.pow(500000.0, -126.0 / 128.0), rel=1e-15)
    assert a[3, 1] == pytest.approx(8191 * math.pow(500000.0, -2.0 / 128.0), rel=1e-15)


def test_rope_identity_norm_inverse_composition():
    Z = _rand(5, 256)
    zero = np.zeros(5, dtype=np.int64)
    assert np.array_equal(O.rope_rotate(Z, zero, 128, 5e5), Z)
    pos = np.array([0, 1, 100, 2047, 8191])
    Y = O.rope_rotate(Z, pos, 128, 5e5)
    zn = Z.reshape(5, 2, 2, 64)
    yn = Y.reshape(5, 2, 2, 64)
    assert np.abs((zn ** 2).sum(2) - (yn ** 2).sum(2)).max() < 1e-12  # per-pair norm
    assert np.abs(O.rope_rotate(Y, pos, 128, 5e5, inverse=True) - Z).max() < 1e-12
    p2 = np.array([3, 4, 5, 6, 7])
    both = O.rope_rotate(O.rope_rotate(Z, pos, 128, 5e5), p2, 128, 5e5)
    assert np.abs(both - O.rope_rotate(Z, pos + p2, 128, 5e5)).max() < 1e-10


def test_rope_relative_position():
    q, k = _rand(1, 128), _rand(1, 128)
    for m, n in [(3, 10), (100, 40), (0, 2047)]:
        lhs = np.sum(O.rope_rotate(q, [m], 128, 5e5) * O.rope_rotate(k, [n], 128, 5e5))
        rhs = np.sum(q * O.rope_rotate(k, [n - m], 128, 5e5))
        assert abs(lhs - rhs) < 1e-10


def test_qk_rope_projection_hand_worked():
    # head_dim 4, position 1, theta = 4 / pi^2: pair (0, 2) turns by 1 rad and
    # pair (1, 3) by theta^(-1/2) = pi / 2.  x = [1, 2, 3, 4], W = I,
    # A = [1, 0, 0, 0] (r = 1, A x = 1), B = e_3, s = 2: before the rotation
    # z = x + s B (A x) = [1, 2, 3, 6].  Rotating (z_i, z_{i+2}) by +a gives
    # (z_i cos a - z_{i+2} sin a, z_{i+2} cos a + z_i sin a):
    #   pair 0: (cos 1 - 3 sin 1, 3 cos 1 + sin 1);  pair 1: (-6, 2).
    theta = 4.0 / math.pi ** 2
    X = np.array([[1.0, 2.0, 3.0, 4.0]])
    W = np.eye(4)
    A = np.array([[1.0, 0.0, 0.0, 0.0]])
    B = np.array([[0.0], [0.0], [0.0], [1.0]])
    c, sn = math.cos(1.0), math.sin(1.0)
    Y = O.qk_rope_forward(X, W, A, B, 2.0, [1], head_dim=4, theta=theta)
    assert np.abs(Y - np.array([[c - 3 * sn, -6.0, 3 * c + sn, 2.0]])).max() < 1e-14
    # Backward, dY = [1, 1, 0, 0]: G rotates each pair by -a,
    # (g_i cos a + g_{i+2} sin a, g_{i+2} cos a - g_i sin a):
    #   G = [cos 1, 0, -sin 1, -1];  G B = G[3] = -1;  A x = 1
    #   dX = G W + s (G B) A = [cos 1 - 2, 0, -sin 1, -1]
    #   dA = s (G B)^T x = -2 [1, 2, 3, 4];  dB = s G^T (A x) = 2 G^T
    dX, dA, dB = O.qk_rope_backward(X, W, A, B, 2.0, [1], np.array([[1.0, 1.0, 0.0, 0.0]]), head_dim=4,
                                    theta=theta)
    assert np.abs(dX - np.array([[c - 2.0, 0.0, -sn, -1.0]])).max() < 1e-14
    assert np.abs(dA - np.array([[-2.0, -4.0, -6.0, -8.0]])).max() < 1e-14
    assert np.abs(dB - np.array([[2 * c], [0.0], [-2 * sn], [-2.0]])).max() < 1e-14


def test_rope_backward_matches_finite_differences():
    M, k, d, r = 2, 4, 8, 2
    X, W, A, B, dY = _rand(M, k), _rand(d, k), _rand(r, k), _rand(d, r), _rand(M, d)
    pos = np.array([3, 11])
    s = 0.5
    dX, dA, dB = O.qk_rope_backward(X, W, A, B, s, pos, dY, head_dim=4, theta=10.0)
    f = lambda: float(np.sum(dY * O.qk_rope_forward(X, W, A, B, s, pos, head_dim=4, theta=10.0)))  # noqa: E731
    assert np.abs(_fd(f, X) - dX).max() < 1e-9
    assert np.abs(_fd(f, A) - dA).max() < 1e-9
    assert np.abs(_fd(f, B) - dB).max() < 1e-9


# ---------------------------------------------------------------------------
# rounding and NF4
# ---------------------------------------------------------------------------

def test_round_bf16_ties_and_library_agreement():
    import torch

    one = 1.0
    assert O.round_bf16([one + 2 ** -8])[0] == 1.0                 # tie, even stays
    assert O.round_bf16([one + 3 * 2 ** -8])[0] == 1.0 + 2 ** -6    # tie, rounds to even above
    assert O.round_bf16([one + 2 ** -8 + 2 ** -20])[0] == 1.0 + 2 ** -7
    assert O.round_bf16([-(one + 3 * 2 ** -8)])[0] == -(1.0 + 2 ** -6)
    x = np.concatenate([RNG.standard_normal(20000) * 10.0 ** RNG.integers(-6, 6, 20000),
                        np.array([0.0, -0.0, 65504.0, 1e-40])]).astype(np.float32)
    lib = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O.round_bf16(x), lib)


def test_nf4_table_matches_normal_quantile_construction():
    from scipy.stats import norm

    from synth import nf4_table

    t = nf4_table().astype(np.float64)
    assert len(t) == 16 and np.all(np.diff(t) > 0)
    assert t[0] == -1.0 and t[7] == 0.0 and t[15] == 1.0
    assert np.sum(t < 0) == 7 and np.sum(t > 0) == 8
    # Quantiles of N(0,1): 8 positive levels and 7 negative ones, from
    # offset delta = (1 - 1/(2*15) + 1 - 1/(2*16)) / 2 towards the median, plus zero.
    delta = 0.5 * ((1 - 1 / 30) + (1 - 1 / 32))
    pos = norm.ppf(np.linspace(delta, 0.5, 9)[:-1])
    neg = -norm.ppf(np.linspace(delta, 0.5, 8)[:-1])
    v = np.sort(np.concatenate([pos, [0.0], neg]))
    v /= v.max()
    assert np.abs(v - t).max() < 5e-7


def test_nf4_unpack_order_high_nibble_first():
    codes = O.nf4_unpack(np.array([0xAB, 0x0F], dtype=np.uint8), 4)
    assert codes.tolist() == [10, 11, 0, 15]


def test_nf4_dequant_hand_and_fp32_multiply():
    from synth import nf4_table

    t = nf4_table()
    # byte 0xF0: element 0 is code 15 (+1), element 1 is code 0 (-1); absmax 0.5
    w = O.nf4_dequant(np.array([0xF0] * 32, dtype=np.uint8), np.array([0.5], np.float32), t, 1, 64)
    assert w[0, 0] == 0.5 and w[0, 1] == -0.5
    # general case: fp32 multiply (numpy float32) then bf16 rounding
    codes = RNG.integers(0, 256, 64 * 8, dtype=np.uint8)
    am = (np.abs(RNG.standard_normal(16)) * 0.03).astype(np.float32)
    w = O.nf4_dequant(codes, am, t, 8, 128)
    c = O.nf4_unpack(codes, 1024)
    prod32 = (t[c] * np.repeat(am, 64)).astype(np.float32)  # fp32 * fp32 in fp32
    assert prod32.dtype == np.float32
    import torch
    ref = torch.from_numpy(prod32).to(torch.bfloat16).to(torch.float64).numpy().reshape(8, 128)
    assert np.array_equal(w, ref)


def test_nf4_round_trip_all_codes():
    from synth import nf4_table

    t = nf4_table()
    codes = np.arange(16)
    packed = ((codes[0::2] << 4) | codes[1::2]).astype(np.uint8)
    packed = np.tile(packed, 8)  # one block of 64
    w = O.nf4_dequant(packed, np.array([1.0], np.float32), t, 1, 64)
    # with absmax 1 the decode is the table (rounded to bf16); -1, 0, +1 are exact
    assert w[0, 0] == -1.0 and w[0, 7] == 0.0 and w[0, 15] == 1.0
    assert np.abs(w[0, :16] - t).max() < 2 ** -8
    re, am = O.nf4_encode(w, t)
    assert am[0] == 1.0
    assert np.array_equal(O.nf4_unpack(re, 64), np.tile(codes, 4))


def test_nf4_encode_zero_block_and_ties():
    from synth import nf4_table

    t = nf4_table()
    packed, am = O.nf4_encode(np.zeros((1, 64)), t)
    assert am[0] == 0.0
    assert np.all(O.nf4_unpack(packed, 64) == 7)
    # a value exactly midway between codes 7 (0.0) and 8 goes to the lower code
    mid = float(t[8]) / 2
    w = np.zeros((1, 64))
    w[0, 0] = 1.0  # sets absmax = 1
    w[0, 1] = mid
    packed, am = O.nf4_encode(w, t)
    assert O.nf4_unpack(packed, 64)[1] == 7


def test_rel_err():
    assert O.rel_err(np.array([1.0, 2.0]), np.array([1.0, 4.0])) == 0.5
    assert O.rel_err(np.zeros(3), np.zeros(3)) == 0.0


# ---------------------------------------------------------------------------
# SwiGLU on the gate / up pair
# ---------------------------------------------------------------------------

def test_silu_closed_forms():
    e = math.e
    assert O.silu(np.array([0.0]))[0] == 0.0
    assert abs(O.silu(np.array([1.0]))[0] - e / (1 + e)) < 1e-16
    assert abs(O.silu(np.array([-1.0]))[0] + 1 / (1 + e)) < 1e-16
    # large |z|: silu(z) -> z, silu(-z) -> -z e^-z
    assert O.silu(np.array([40.0]))[0] == 40.0
    assert abs(O.silu(np.array([-40.0]))[0] / (-40.0 * math.exp(-40.0)) - 1) < 1e-12
    # the minimum: silu'(z*) = 0 means sigmoid(z*) = 1 + 1/z*, so silu(z*) = z* + 1;
    # z* = -1 - W0(1/e) with the principal Lambert W value W0(1/e) = 0.2784645427610738
    z = -1.2784645427610738
    assert abs(O.silu(np.array([z]))[0] - (z + 1)) < 1e-15
    dG, _ = O.swiglu_grad(np.array([1.0]), np.array([z]), np.array([1.0]))
    assert abs(dG[0]) < 1e-15


def test_swiglu_hand_worked_1x1():
    # x = 2, gate: w = 1, a = 1, b = 0.5, s = 2 -> g = 2 + 2 * 0.5 * 2 = 4;
    # up: w = -1, a = b = 0 -> u = -2; h = silu(4) u = -2 * 4 / (1 + e^-4)
    X = np.array([[2.0]])
    H, G, U = O.swiglu_forward(X, [[1.0]], [[1.0]], [[0.5]], 2.0, [[-1.0]], [[0.0]], [[0.0]], 1.0)
    assert G[0, 0] == 4.0 and U[0, 0] == -2.0
    assert abs(H[0, 0] - (-8.0 / (1.0 + math.exp(-4.0)))) < 1e-15


def test_swiglu_grad_matches_finite_differences():
    G, U, dH = _rand(4, 6) * 3, _rand(4, 6), _rand(4, 6)
    dG, dU = O.swiglu_grad(dH, G, U)
    h = 1e-6
    # elementwise: perturb one entry at a time
    num_g = np.zeros_like(G)
    num_u = np.zeros_like(U)
    for idx in np.ndindex(G.shape):
        Gp, Gm = G.copy(), G.copy()
        Gp[idx] += h
        Gm[idx] -= h
        num_g[idx] = (np.sum(dH * O.silu(Gp) * U) - np.sum(dH * O.silu(Gm) * U)) / (2 * h)
        Up, Um = U.copy(), U.copy()
        Up[idx] += h
        Um[idx] -= h
        num_u[idx] = (np.sum(dH * O.silu(G) * Up) - np.sum(dH * O.silu(G) * Um)) / (2 * h)
    assert np.abs(num_g - dG).max() < 1e-8
    assert np.abs(num_u - dU).max() < 1e-8


def test_swiglu_backward_matches_finite_differences():
    M, k, d, rg, ru = 3, 5, 4, 2, 3
    X = _rand(M, k)
    Wg, Ag, Bg = _rand(d, k), _rand(rg, k), _rand(d, rg)
    Wu, Au, Bu = _rand(d, k), _rand(ru, k), _rand(d, ru)
    sg, su = 2.0, 0.5
    dH = _rand(M, d)
    dX, dAg, dBg, dAu, dBu = O.swiglu_backward(X, Wg, Ag, Bg, sg, Wu, Au, Bu, su, dH)

    def f():
        H, _, _ = O.swiglu_forward(X, Wg, Ag, Bg, sg, Wu, Au, Bu, su)
        return float(np.sum(dH * H))
    # the loss is smooth but not linear: central differences, O(h^2) error
    for P, g in ((X, dX), (Ag, dAg), (Bg, dBg), (Au, dAu), (Bu, dBu)):
        assert np.abs(_fd(f, P, h=1e-5) - g).max() < 1e-6 * max(1.0, np.abs(g).max())


def test_swiglu_zero_up_adapter_has_zero_gradients():
    # Au = Bu = 0: dAu = su (dU Bu)^T X and dBu = su dU^T (X Au^T) vanish
    # whatever dU is, while the gate adapter still receives a gradient
    M, k, d = 2, 3, 4
    X, Wg, Ag, Bg, Wu = _rand(M, k), _rand(d, k), _rand(1, k), _rand(d, 1), _rand(d, k)
    Z = np.zeros
    dX, dAg, dBg, dAu, dBu = O.swiglu_backward(X, Wg, Ag, Bg, 1.0, Wu, Z((1, k)), Z((d, 1)), 1.0, _rand(M, d))
    assert np.all(dAu == 0.0) and np.all(dBu == 0.0)
    assert np.abs(dAg).max() > 0 and np.abs(dBg).max() > 0


# ---------------------------------------------------------------------------
# LoRA dropout on the adapter's input
# ---------------------------------------------------------------------------

def test_dropout_keep_bit_order():
    # byte 0b00000101 keeps elements 0 and 2; 0x80 keeps element 7 of its group
    k = O.dropout_keep(np.array([[0b00000101, 0x80]], dtype=np.uint8), 1, 16)
    assert k.tolist() == [[True, False, True] + [False] * 12 + [True]]


def test_dropout_hand_worked():
    # x = [2, 4], W = [[1, 1]], A = [[1, 1]], B = [[1]], s = 1, p = 0.5, keep = [1, 0]:
    # D = [4, 0], A D = 4, y = 6 + 4 = 10
    Y = O.lora_dropout_forward([[2.0, 4.0]], [[1.0, 1.0]], [[1.0, 1.0]], [[1.0]], 1.0, 0.5, [[True, False]])
    assert Y[0, 0] == 10.0


def test_dropout_special_cases():
    M, k, d, r = 4, 8, 5, 2
    X, W, A, B, G = _rand(M, k), _rand(d, k), _rand(r, k), _rand(d, r), _rand(M, d)
    ones, zeros = np.ones((M, k), bool), np.zeros((M, k), bool)
    # p = 0 and every element kept: the plain layer
    assert np.abs(O.lora_dropout_forward(X, W, A, B, 2.0, 0.0, ones) - O.lora_forward(X, W, A, B, 2.0)).max() < 1e-12
    for a, b in zip(O.lora_dropout_backward(X, W, A, B, 2.0, 0.0, ones, G), O.lora_backward(X, W, A, B, 2.0, G)):
        assert np.abs(a - b).max() < 1e-12
    # nothing kept: the adapter sees zeros, so it contributes nothing and gets no gradient
    assert np.abs(O.lora_dropout_forward(X, W, A, B, 2.0, 0.3, zeros) - X @ W.T).max() < 1e-12
    dX, dA, dB = O.lora_dropout_backward(X, W, A, B, 2.0, 0.3, zeros, G)
    assert np.abs(dX - G @ W).max() < 1e-12 and np.all(dA == 0) and np.all(dB == 0)


def test_dropout_backward_matches_finite_differences():
    M, k, d, r = 3, 8, 4, 2
    X, W, A, B, G = _rand(M, k), _rand(d, k), _rand(r, k), _rand(d, r), _rand(M, d)
    keep = RNG.random((M, k)) < 0.7
    s, p = 2.0, 0.3
    dX, dA, dB = O.lora_dropout_backward(X, W, A, B, s, p, keep, G)
    f = lambda: float(np.sum(G * O.lora_dropout_forward(X, W, A, B, s, p, keep)))  # noqa: E731
    # linear in each of X, A, B for a fixed mask: central differences are exact up to rounding
    assert np.abs(_fd(f, X) - dX).max() < 1e-9
    assert np.abs(_fd(f, A) - dA).max() < 1e-9
    assert np.abs(_fd(f, B) - dB).max() < 1e-9


def test_dropout_is_unbiased_over_masks():
    # inverted dropout keeps the expectation: the mean over many masks tends to
    # the plain layer (tolerance 5 standard errors of the mean)
    M, k, d, r, p = 2, 6, 3, 2, 0.4
    X, W, A, B = _rand(M, k), _rand(d, k), _rand(r, k), _rand(d, r)
    rng = np.random.default_rng(11)
    ys = np.stack([O.lora_dropout_forward(X, W, A, B, 1.0, p, rng.random((M, k)) >= p) for _ in range(20000)])
    se = ys.std(axis=0) / np.sqrt(len(ys))
    assert np.all(np.abs(ys.mean(axis=0) - O.lora_forward(X, W, A, B, 1.0)) <= 5 * se + 1e-12)


# ---------------------------------------------------------------------------
# Philox4x32-10 dropout mask
# ---------------------------------------------------------------------------

def _philox_kat():
    path = __import__("os").path.join(__import__("os").path.dirname(__file__), "golden", "philox4x32_10_kat.txt")
    rows = []
    for line in open(path):
        if line.strip() and not line.startswith("#"):
            w = [int(t, 16) for t in line.split()]
            rows.append((w[0:4], w[4:6], w[6:10]))
    return rows


def test_philox_known_answers():
    # the published known-answer vectors: a wrong multiplier, key increment,
    # word order or round count changes every output word
    rows = _philox_kat()
    assert len(rows) == 3
    for ctr, key, out in rows:
        assert O.philox4x32_10(ctr, key) == out


def test_philox_mask_word_mapping():
    # element e takes word e mod 4 of block e // 4, the block's counter is
    # (e // 4, 0, offset lo, offset hi) and the key (seed lo, seed hi)
    seed, offset, p = 0x0123456789ABCDEF, 0x0000000500000007, 0.25
    thr = O.dropout_threshold(p)
    assert thr == 1 << 30
    keep = O.dropout_mask_philox(24, p, seed, offset)
    for e in range(24):
        w = O.philox4x32_10((e // 4, 0, 7, 5), (0x89ABCDEF, 0x01234567))[e % 4]
        assert keep[e] == (w >= thr)


def test_philox_mask_vectorised_equals_loop():
    for n, p, seed, off in ((40, 0.1, 3407, 0), (1000, 0.5, 2**40 + 9, 2**33 + 1), (8, 0.0, 1, 2)):
        assert np.array_equal(O.dropout_mask_philox(n, p, seed, off), O.dropout_mask_philox_np(n, p, seed, off))


def test_philox_mask_rate_and_limits():
    # p = 0 keeps everything (every word >= 0); the kept share of 2^18 draws
    # lies within 5 standard deviations of 1 - p; another seed or offset
    # gives another mask
    assert O.dropout_mask_philox_np(4096, 0.0, 5, 0).all()
    n = 1 << 18
    for p in (0.05, 0.1, 0.5):
        k = O.dropout_mask_philox_np(n, p, 3407, 0)
        sd = math.sqrt(n * p * (1 - p))
        assert abs(int(k.sum()) - n * (1 - p)) < 5 * sd
    a = O.dropout_mask_philox_np(4096, 0.5, 1, 0)
    assert not np.array_equal(a, O.dropout_mask_philox_np(4096, 0.5, 2, 0))
    assert not np.array_equal(a, O.dropout_mask_philox_np(4096, 0.5, 1, 1))


def test_dropout_pack_matches_bit_order():
    keep = O.dropout_mask_philox_np(64, 0.5, 77, 3)
    assert np.array_equal(O.dropout_keep(O.dropout_pack(keep), 1, 64)[0], keep)
