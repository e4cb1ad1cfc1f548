"""GPU parity of the grouped entry points (projections that share X) against
the float64 oracle, member by member: each member's Y, dX, dA and dB must
meet the single-projection bar, whatever the other members are.  The group
panel, the shared recomputation of X A^T and the single dA contraction over
X are what differ from the single-projection path."""
import numpy as np
import pytest
import torch

import oracle as O
from synth import gen
from tests.helpers import TOL, cpu64, draw, int_inputs, rel

pytestmark = pytest.mark.gpu


def _member_inputs(seed, M, d_in, d_out, r, dtype):
    W = draw(seed + 1, (d_out, d_in), "normal", 1.0 / np.sqrt(d_in), dtype)
    A = draw(seed + 2, (r, d_in), "uniform", 1.0 / np.sqrt(d_in), dtype)
    B = draw(seed + 3, (d_out, r), "normal", np.sqrt(0.02), dtype)
    dY = draw(seed + 4, (M, d_out), "normal", 1.0, dtype)
    return W, A, B, dY


def _oracle(X, m, dY, p):
    if m.get("rope"):
        return O.qk_rope_forward(X, m["W"], m["A"], m["B"], m["scale"], p), \
            O.qk_rope_backward(X, m["W"], m["A"], m["B"], m["scale"], p, dY)
    return O.lora_forward(X, m["W"], m["A"], m["B"], m["scale"]), \
        O.lora_backward(X, m["W"], m["A"], m["B"], m["scale"], dY)


# (M, d_in, [(d_out, r, rope), ...]): q/k/v-like groups with RoPE on q and k,
# ragged ranks, and sizes that reach the whole-tile kernel.
GROUPS = [
    (300, 264, [(256, 16, True), (128, 5, True), (136, 3, False)]),
    (2100, 1024, [(4096, 64, True), (1024, 64, True), (1024, 64, False)]),
    (4096, 1024, [(4096, 24, False), (1024, 100, True), (2048, 1, False), (512, 8, False)]),
    (129, 520, [(392, 16, False)]),
    # a member wider than 128 rank rows between two narrow ones: each alone
    # in its pass over X (the wide one on the generic panel and dA kernels)
    (600, 512, [(256, 8, False), (512, 200, True), (256, 16, False)]),
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("case", GROUPS, ids=[f"M{g[0]}_k{g[1]}_n{len(g[2])}" for g in GROUPS])
def test_group_parity(lib, dtype, case):
    M, d_in, spec = case
    seq = 2048
    X = draw(500 + M, (M, d_in), "normal", 1.0, dtype)
    pos = torch.from_numpy(gen.positions_mod(M, seq)).cuda()
    cos, sin = lib.rope_cache(seq, 128, 500000.0)
    members, dYs = [], []
    for g, (d_out, r, rope) in enumerate(spec):
        W, A, B, dY = _member_inputs(600 + 10 * g + M, M, d_in, d_out, r, dtype)
        members.append(dict(W=W, A=A, B=B, scale=(16.0 + 8 * g) / r, rope=rope))
        dYs.append(dY)
    Ys = lib.lora_group_fwd(X, members, pos, cos, sin)
    grads = lib.lora_group_bwd(X, members, dYs, pos, cos, sin)
    torch.cuda.synchronize()
    p = pos.cpu().numpy()
    for g, m in enumerate(members):
        Yr, (dXr, dAr, dBr) = _oracle(X, m, dYs[g], p)
        dX, dA, dB = grads[g]
        errs = dict(Y=rel(Ys[g], Yr), dX=rel(dX, dXr), dA=rel(dA, dAr), dB=rel(dB, dBr))
        print(dtype, case[:2], g, spec[g], errs)
        assert all(e <= TOL[dtype] for e in errs.values()), (g, errs)


def _group_kinds(fn):
    from lora_linear_layers_amd import _lib
    _lib.profile_begin(512)
    out = fn()
    torch.cuda.synchronize()
    _lib.profile_end()
    return out, set(_lib.profile_report())


# (M, d_in, [(d_out, r, rope), ...]): every member's tiles whole and r a
# multiple of 8, so the forward runs every member's GEMM in one launch: RoPE
# and store members mixed, members of one and of two column tiles.
GROUP_GEMM = [
    (512, 512, [(512, 16, True), (256, 8, True), (256, 24, False)]),
    (256, 320, [(256, 8, False), (768, 16, True)]),
]


@pytest.mark.parametrize("case", GROUP_GEMM, ids=[f"M{g[0]}_k{g[1]}_n{len(g[2])}" for g in GROUP_GEMM])
def test_group_gemm_parity(lib, case):
    M, d_in, spec = case
    seq = 128
    X = draw(900 + M, (M, d_in), "normal", 1.0, "bf16")
    pos = torch.from_numpy(gen.positions_mod(M, seq)).cuda()
    cos, sin = lib.rope_cache(seq, 128, 500000.0)
    members, dYs = [], []
    for g, (d_out, r, rope) in enumerate(spec):
        W, A, B, dY = _member_inputs(910 + 10 * g + M, M, d_in, d_out, r, "bf16")
        members.append(dict(W=W, A=A, B=B, scale=(16.0 + 8 * g) / r, rope=rope))
        dYs.append(dY)
    Ys, kinds = _group_kinds(lambda: lib.lora_group_fwd(X, members, pos, cos, sin))
    assert kinds & {k for k in kinds if k.startswith("gemm")} == {"gemm_bf16_256x256_nt_group"}, kinds
    p = pos.cpu().numpy()
    for g, m in enumerate(members):
        Yr = O.qk_rope_forward(X, m["W"], m["A"], m["B"], m["scale"], p) if m["rope"] else \
            O.lora_forward(X, m["W"], m["A"], m["B"], m["scale"])
        err = rel(Ys[g], Yr)
        print(case[:2], g, spec[g], err)
        assert err <= TOL["bf16"], (g, err)


def test_group_eight_members(lib):
    # the largest group: 8 members at a size where every dX runs on whole
    # tiles, so 16 batched transposes (B^T and A^T of each), 16 batched sums
    # (dA and dB of each), 8 entries of the group GEMM's member table and one
    # 64-row panel pass; RoPE on every other member.  Y and dX on sampled
    # rows, dA and dB in full.
    M, d_in, seq = 4096, 4096, 4096
    X = draw(1200, (M, d_in), "normal", 1.0, "bf16")
    pos = torch.from_numpy(gen.positions_mod(M, seq)).cuda()
    cos, sin = lib.rope_cache(seq, 128, 500000.0)
    members, dYs = [], []
    for g in range(8):
        W, A, B, dY = _member_inputs(1210 + 10 * g, M, d_in, 256, 8, "bf16")
        members.append(dict(W=W, A=A, B=B, scale=2.0 + g, rope=g % 2 == 0))
        dYs.append(dY)
    (Ys, grads), kinds = _group_kinds(lambda: (lib.lora_group_fwd(X, members, pos, cos, sin),
                                               lib.lora_group_bwd(X, members, dYs, pos, cos, sin)))
    assert {"gemm_bf16_256x256_nt_group", "gemm_bf16_256x256_nt_store", "reduce_splits", "transpose_ab"} <= kinds
    rng = np.random.default_rng(5)
    rows = np.sort(np.concatenate([[0, M - 1], rng.choice(np.arange(1, M - 1), 126, replace=False)]))
    tr = torch.from_numpy(rows).cuda()
    p = pos.cpu().numpy()
    for g, m in enumerate(members):
        W, A, B, s = m["W"], m["A"], m["B"], m["scale"]
        dX, dA, dB = grads[g]
        if m["rope"]:
            Yr = O.qk_rope_forward(X[tr], W, A, B, s, p[rows])
            G = O.rope_rotate(dYs[g], p, 128, 500000.0, inverse=True)
        else:
            Yr = O.lora_forward(X[tr], W, A, B, s)
            G = cpu64(dYs[g])
        dXr = O.lora_grad_x(W, A, B, s, G[rows])
        dAr, dBr = O.lora_grad_ab(X, A, B, s, G)
        errs = dict(Y=rel(Ys[g][tr], Yr), dX=rel(dX[tr], dXr), dA=rel(dA, dAr), dB=rel(dB, dBr))
        print(g, errs)
        assert all(e <= TOL["bf16"] for e in errs.values()), (g, errs)


def test_group_gemm_integer_exact(lib):
    # small integers: every product and sum exact on both sides, so each
    # member's Y from the one-launch group GEMM equals the oracle exactly
    M, d_in = 256, 64
    X, _, _, _, _ = int_inputs(41, M, d_in, 8, 1, "bf16")
    members = []
    for g, (d_out, r) in enumerate([(256, 8), (512, 16)]):
        _, W, A, B, _ = int_inputs(43 + g, M, d_in, d_out, r, "bf16")
        members.append(dict(W=W, A=A, B=B, scale=float(2 - g)))
    Ys, kinds = _group_kinds(lambda: lib.lora_group_fwd(X, members))
    assert "gemm_bf16_256x256_nt_group" in kinds, kinds
    for g, m in enumerate(members):
        Yr = O.lora_forward(X, m["W"], m["A"], m["B"], m["scale"])
        assert np.abs(Yr).max() <= 256
        assert np.array_equal(cpu64(Ys[g]), Yr), g


def test_group_whole_tile_parity(lib):
    # q, k, v of one attention block at full width: q (and dX of every member)
    # on the whole-tile kernel; Y and dX on sampled rows, dA and dB in full.
    M, d_in = 4096, 4096
    seq = 4096
    X = draw(71, (M, d_in), "normal", 1.0, "bf16")
    pos = torch.from_numpy(gen.positions_mod(M, seq)).cuda()
    cos, sin = lib.rope_cache(seq, 128, 500000.0)
    spec = [(4096, 64, True), (1024, 64, True), (1024, 64, False)]
    members, dYs = [], []
    for g, (d_out, r, rope) in enumerate(spec):
        W, A, B, dY = _member_inputs(80 + 10 * g, M, d_in, d_out, r, "bf16")
        members.append(dict(W=W, A=A, B=B, scale=16.0 / r, rope=rope))
        dYs.append(dY)
    Ys = lib.lora_group_fwd(X, members, pos, cos, sin)
    grads = lib.lora_group_bwd(X, members, dYs, pos, cos, sin)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    rows = np.sort(np.concatenate([[0, M - 1], rng.choice(np.arange(1, M - 1), 254, replace=False)]))
    tr = torch.from_numpy(rows).cuda()
    p = pos.cpu().numpy()
    for g, m in enumerate(members):
        W, A, B, s = m["W"], m["A"], m["B"], m["scale"]
        dX, dA, dB = grads[g]
        if m["rope"]:
            Yr = O.qk_rope_forward(X[tr], W, A, B, s, p[rows])
            G = O.rope_rotate(dYs[g], p, 128, 500000.0, inverse=True)
        else:
            Yr = O.lora_forward(X[tr], W, A, B, s)
            G = cpu64(dYs[g])
        dXr = O.lora_grad_x(W, A, B, s, G[rows])
        dAr, dBr = O.lora_grad_ab(X, A, B, s, G)
        errs = dict(Y=rel(Ys[g][tr], Yr), dX=rel(dX[tr], dXr), dA=rel(dA, dAr), dB=rel(dB, dBr))
        print("whole", g, errs)
        assert all(e <= TOL["bf16"] for e in errs.values()), (g, errs)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_group_integer_exact(lib, dtype):
    # Small integers keep every product and sum exact on both sides, so the
    # group must equal the oracle exactly, member by member.
    M, d_in = 1000, 40
    X, _, _, _, _ = int_inputs(5, M, d_in, 8, 1, dtype)
    members, dYs = [], []
    for g, (d_out, r) in enumerate([(40, 2), (48, 1), (32, 3)]):
        _, W, A, B, dY = int_inputs(11 + g, M, d_in, d_out, r, dtype)
        members.append(dict(W=W, A=A, B=B, scale=float(2 - g % 2)))
        dYs.append(dY)
    Ys = lib.lora_group_fwd(X, members)
    grads = lib.lora_group_bwd(X, members, dYs)
    torch.cuda.synchronize()
    for g, m in enumerate(members):
        Yr = O.lora_forward(X, m["W"], m["A"], m["B"], m["scale"])
        dXr, dAr, dBr = O.lora_backward(X, m["W"], m["A"], m["B"], m["scale"], dYs[g])
        if dtype == "bf16":
            assert np.abs(Yr).max() <= 256 and np.abs(dXr).max() <= 256
        assert np.array_equal(cpu64(Ys[g]), Yr), g
        for got, ref in zip(grads[g], (dXr, dAr, dBr)):
            assert np.array_equal(cpu64(got), ref), g


def test_group_nf4_members(lib):
    # gate and up with NF4 base weights next to a plain bf16 member
    tab = gen.nf4_table()
    M, d_in = 1500, 1024
    X = draw(91, (M, d_in), "normal", 1.0, "bf16")
    members, dYs, is_nf4 = [], [], []
    for g, (d_out, r, nf4) in enumerate([(2816, 16, True), (2816, 16, True), (1032, 8, False)]):
        W, A, B, dY = _member_inputs(95 + 10 * g, M, d_in, d_out, r, "bf16")
        m = dict(A=A, B=B, scale=16.0 / r)
        if nf4:
            codes = gen.nf4_random_codes(120 + g, d_out * d_in).cuda()
            absmax = gen.nf4_random_absmax(121 + g, d_out * d_in // 64, 1.0 / np.sqrt(d_in)).cuda()
            m.update(codes=codes, absmax=absmax)
        else:
            m.update(W=W)
        members.append(m)
        dYs.append(dY)
        is_nf4.append(nf4)
    Ys = lib.lora_group_fwd(X, members, table16=tab)
    grads = lib.lora_group_bwd(X, members, dYs, table16=tab)
    torch.cuda.synchronize()
    for g, m in enumerate(members):
        d_out = m["B"].shape[0]
        if is_nf4[g]:
            c, am = m["codes"].cpu().numpy(), m["absmax"].cpu().numpy()
            Yr = O.nf4_lora_forward(X, c, am, tab, m["A"], m["B"], m["scale"], d_out, d_in)
            ref = O.nf4_lora_backward(X, c, am, tab, m["A"], m["B"], m["scale"], dYs[g], d_out, d_in)
        else:
            Yr = O.lora_forward(X, m["W"], m["A"], m["B"], m["scale"])
            ref = O.lora_backward(X, m["W"], m["A"], m["B"], m["scale"], dYs[g])
        errs = dict(Y=rel(Ys[g], Yr), **{k: rel(v, rv) for k, v, rv in zip(("dX", "dA", "dB"), grads[g], ref)})
        print("nf4 group", g, errs)
        assert all(e <= TOL["bf16"] for e in errs.values()), (g, errs)


def test_group_matches_single_calls(lib):
    # Only the rank-r panels' split order differs from the single calls: a
    # group of one equals the single call exactly when its panel split is the
    # same, and any group stays within bf16 rounding of the single calls.
    M, d_in = 2100, 1024
    X = draw(31, (M, d_in), "normal", 1.0, "bf16")
    members, dYs = [], []
    for g, (d_out, r) in enumerate([(1024, 64), (1024, 16)]):
        W, A, B, dY = _member_inputs(33 + 10 * g, M, d_in, d_out, r, "bf16")
        members.append(dict(W=W, A=A, B=B, scale=2.0))
        dYs.append(dY)
    one = lib.lora_group_fwd(X, members[:1])[0]
    g1 = lib.lora_group_bwd(X, members[:1], dYs[:1])[0]
    Ys = lib.lora_group_fwd(X, members)
    grads = lib.lora_group_bwd(X, members, dYs)
    singles = [(lib.lora_linear_fwd(X, m["W"], m["A"], m["B"], 2.0),
                lib.lora_linear_bwd(X, m["W"], m["A"], m["B"], 2.0, dYs[g])) for g, m in enumerate(members)]
    torch.cuda.synchronize()
    assert torch.equal(one, singles[0][0])
    for a, b in zip(g1, singles[0][1]):
        assert torch.equal(a, b)
    for g in range(2):
        Ys1, (dX1, dA1, dB1) = singles[g]
        for got, ref in ((Ys[g], Ys1), (grads[g][0], dX1), (grads[g][1], dA1), (grads[g][2], dB1)):
            assert rel(got, cpu64(ref)) <= 1e-2


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_group_m_zero_and_no_dx(lib, dtype):
    d_in = 256
    X = torch.empty(0, d_in, dtype=gen_dtype(dtype), device="cuda")
    members, dYs = [], []
    for g, (d_out, r) in enumerate([(128, 8), (256, 3)]):
        W, A, B, _ = _member_inputs(3 + g, 1, d_in, d_out, r, dtype)
        members.append(dict(W=W, A=A, B=B, scale=1.0))
        dYs.append(torch.empty(0, d_out, dtype=X.dtype, device="cuda"))
    Ys = lib.lora_group_fwd(X, members)
    grads = lib.lora_group_bwd(X, members, dYs, need_dX=False)
    torch.cuda.synchronize()
    for g in range(2):
        assert Ys[g].shape == (0, members[g]["B"].shape[0])
        assert grads[g][0] is None
        assert torch.count_nonzero(grads[g][1]) == 0 and torch.count_nonzero(grads[g][2]) == 0
    # dX omitted at M > 0: dA and dB unchanged
    M = 300
    X = draw(8, (M, d_in), "normal", 1.0, dtype)
    dYs = [draw(9 + g, (M, m["B"].shape[0]), "normal", 1.0, dtype) for g, m in enumerate(members)]
    with_dx = lib.lora_group_bwd(X, members, dYs)
    no_dx = lib.lora_group_bwd(X, members, dYs, need_dX=False)
    torch.cuda.synchronize()
    for g in range(2):
        assert no_dx[g][0] is None
        assert torch.equal(with_dx[g][1], no_dx[g][1]) and torch.equal(with_dx[g][2], no_dx[g][2])


def gen_dtype(dtype):
    return torch.float32 if dtype == "f32" else torch.bfloat16


def test_transpose_exact(lib):
    W = draw(5, (1032, 520), "normal", 1.0, "bf16")
    Wt = lib.lora_transpose(W)
    torch.cuda.synchronize()
    assert torch.equal(Wt, W.t().contiguous())


def test_group_backward_with_caller_wt_is_bit_equal(lib):
    # whole tiles: dX reads W^T; a caller-held W^T gives the same bits as the
    # per-call transpose
    M, d_in = 4096, 4096
    X = draw(61, (M, d_in), "normal", 1.0, "bf16")
    members, with_t, dYs = [], [], []
    for g, (d_out, r) in enumerate([(1024, 16), (2048, 64)]):
        W, A, B, dY = _member_inputs(62 + 10 * g, M, d_in, d_out, r, "bf16")
        members.append(dict(W=W, A=A, B=B, scale=1.0))
        with_t.append(dict(W=W, A=A, B=B, scale=1.0, W_t=lib.lora_transpose(W)))
        dYs.append(dY)
    a = lib.lora_group_bwd(X, members, dYs)
    b = lib.lora_group_bwd(X, with_t, dYs)
    torch.cuda.synchronize()
    for ga, gb in zip(a, b):
        for x, y in zip(ga, gb):
            assert torch.equal(x, y)
