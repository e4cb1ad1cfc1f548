"""Python entry points with the C ABI's names (include/lora_linear.h).

Each call validates tensor placement/contiguity, allocates outputs (and the
workspace when none is passed) with torch, and calls the library on the
current HIP stream.  Row-major shapes:

    X [M, d_in]   W [d_out, d_in]   A [r, d_in]   B [d_out, r]   Y, dY [M, d_out]

scale is s = alpha / r.  dA and dB come back in fp32.
"""
from __future__ import annotations

import torch

from . import _lib as L


def _dims(X, W_rows, W_cols, A, B):
    M, d_in = X.shape
    r = A.shape[0]
    if A.shape != (r, d_in) or B.shape != (W_rows, r) or W_cols != d_in:
        raise ValueError("shape mismatch: X [M,d_in], W [d_out,d_in], A [r,d_in], B [d_out,r]")
    return M, d_in, W_rows, r


def lora_linear_fwd(X, W, A, B, scale: float, Y=None, ws=None):
    """Y = X W^T + scale (X A^T) B^T."""
    L._contig(X, W, A, B, Y)
    M, d_in, d_out, r = _dims(X, W.shape[0], W.shape[1], A, B)
    dt = L._dtype_code(X)
    if Y is None:
        Y = torch.empty(M, d_out, dtype=X.dtype, device=X.device)
    ws = L._workspace(L.OP_FWD, dt, M, d_in, d_out, r, X.device, ws)
    L._check("lora_linear_fwd", L.lib().lora_linear_fwd(
        dt, M, d_in, d_out, r, float(scale), L._ptr(X), L._ptr(W), L._ptr(A), L._ptr(B), L._ptr(Y),
        L._ptr(ws), ws.numel(), L._stream(X.device)))
    return Y


def lora_linear_fwd_noalloc(X, W, A, B, scale: float, Y=None):
    """lora_linear_fwd with the library's static scratch instead of a
    workspace (for callers that cannot allocate device memory; Y is allocated
    here only when the caller passes none)."""
    L._contig(X, W, A, B, Y)
    M, d_in, d_out, r = _dims(X, W.shape[0], W.shape[1], A, B)
    dt = L._dtype_code(X)
    if Y is None:
        Y = torch.empty(M, d_out, dtype=X.dtype, device=X.device)
    L._check("lora_linear_fwd_noalloc", L.lib().lora_linear_fwd_noalloc(
        dt, M, d_in, d_out, r, float(scale), L._ptr(X), L._ptr(W), L._ptr(A), L._ptr(B), L._ptr(Y),
        L._stream(X.device)))
    return Y


def lora_linear_bwd(X, W, A, B, scale: float, dY, need_dX: bool = True, ws=None, out=None):
    """(dX or None, dA fp32, dB fp32) for upstream gradient dY; X A^T is recomputed."""
    L._contig(X, W, A, B, dY)
    M, d_in, d_out, r = _dims(X, W.shape[0], W.shape[1], A, B)
    dt = L._dtype_code(X)
    if out is None:
        dX = torch.empty(M, d_in, dtype=X.dtype, device=X.device) if need_dX else None
        dA = torch.empty(r, d_in, dtype=torch.float32, device=X.device)
        dB = torch.empty(d_out, r, dtype=torch.float32, device=X.device)
    else:
        dX, dA, dB = out
    ws = L._workspace(L.OP_BWD, dt, M, d_in, d_out, r, X.device, ws)
    L._check("lora_linear_bwd", L.lib().lora_linear_bwd(
        dt, M, d_in, d_out, r, float(scale), L._ptr(X), L._ptr(W), L._ptr(A), L._ptr(B), L._ptr(dY), L._ptr(dX),
        L._ptr(dA), L._ptr(dB), L._ptr(ws), ws.numel(), L._stream(X.device)))
    return dX, dA, dB


def rope_cache(max_pos: int, head_dim: int = 128, theta: float = 500000.0, device="cuda"):
    """(cos, sin) fp32 [max_pos, head_dim/2], filled on the device in fp64."""
    cos = torch.empty(max_pos, head_dim // 2, dtype=torch.float32, device=device)
    sin = torch.empty_like(cos)
    L._check("lora_rope_cache", L.lib().lora_rope_cache(max_pos, head_dim, float(theta), L._ptr(cos), L._ptr(sin),
                                                        L._stream(cos.device)))
    return cos, sin


def lora_qk_rope_fwd(X, W, A, B, scale: float, positions, cos, sin, head_dim: int = 128, Y=None, ws=None):
    """RoPE(X W^T + scale (X A^T) B^T) with the rotation as the GEMM epilogue."""
    L._contig(X, W, A, B, positions, cos, sin, Y)
    M, d_in, d_out, r = _dims(X, W.shape[0], W.shape[1], A, B)
    dt = L._dtype_code(X)
    if positions.dtype != torch.int32 or positions.numel() != M:
        raise ValueError("positions must be int32 [M]")
    if Y is None:
        Y = torch.empty(M, d_out, dtype=X.dtype, device=X.device)
    ws = L._workspace(L.OP_ROPE_FWD, dt, M, d_in, d_out, r, X.device, ws)
    L._check("lora_qk_rope_fwd", L.lib().lora_qk_rope_fwd(
        dt, M, d_in, d_out, r, float(scale), L._ptr(X), L._ptr(W), L._ptr(A), L._ptr(B), head_dim,
        L._ptr(positions), L._ptr(cos), L._ptr(sin), cos.shape[0], L._ptr(Y), L._ptr(ws), ws.numel(),
        L._stream(X.device)))
    return Y


def lora_qk_rope_bwd(X, W, A, B, scale: float, positions, cos, sin, dY, head_dim: int = 128,
                     need_dX: bool = True, ws=None):
    """Backward of lora_qk_rope_fwd: inverse rotation of dY, then the LoRA backward."""
    L._contig(X, W, A, B, positions, cos, sin, dY)
    M, d_in, d_out, r = _dims(X, W.shape[0], W.shape[1], A, B)
    dt = L._dtype_code(X)
    dX = torch.empty(M, d_in, dtype=X.dtype, device=X.device) if need_dX else None
    dA = torch.empty(r, d_in, dtype=torch.float32, device=X.device)
    dB = torch.empty(d_out, r, dtype=torch.float32, device=X.device)
    ws = L._workspace(L.OP_ROPE_BWD, dt, M, d_in, d_out, r, X.device, ws)
    L._check("lora_qk_rope_bwd", L.lib().lora_qk_rope_bwd(
        dt, M, d_in, d_out, r, float(scale), L._ptr(X), L._ptr(W), L._ptr(A), L._ptr(B), head_dim,
        L._ptr(positions), L._ptr(cos), L._ptr(sin), cos.shape[0], L._ptr(dY), L._ptr(dX), L._ptr(dA), L._ptr(dB),
        L._ptr(ws), ws.numel(), L._stream(X.device)))
    return dX, dA, dB


def nf4_lora_linear_fwd(X, codes, absmax, table16, A, B, scale: float, d_out: int, blocksize: int = 64,
                        Y=None, ws=None):
    """Forward with the NF4 base weight dequantised inside the GEMM load stage."""
    L._contig(X, codes, absmax, A, B, Y)
    M, d_in = X.shape
    r = A.shape[0]
    if X.dtype != torch.bfloat16:
        raise TypeError("NF4 path takes bf16 activations")
    if Y is None:
        Y = torch.empty(M, d_out, dtype=X.dtype, device=X.device)
    ws = L._workspace(L.OP_NF4_FWD, L.LORA_BF16, M, d_in, d_out, r, X.device, ws)
    tab = L._table_ptr(table16)
    L._check("nf4_lora_linear_fwd", L.lib().nf4_lora_linear_fwd(
        M, d_in, d_out, r, float(scale), L._ptr(X), L._ptr(codes), L._ptr(absmax), blocksize, tab, L._ptr(A),
        L._ptr(B), L._ptr(Y), L._ptr(ws), ws.numel(), L._stream(X.device)))
    return Y


def nf4_lora_linear_bwd(X, codes, absmax, table16, A, B, scale: float, dY, blocksize: int = 64,
                        need_dX: bool = True, ws=None):
    """(dX or None, dA, dB) with the NF4 base weight; no dW."""
    L._contig(X, codes, absmax, A, B, dY)
    M, d_in = X.shape
    d_out = dY.shape[1]
    r = A.shape[0]
    dX = torch.empty(M, d_in, dtype=X.dtype, device=X.device) if need_dX else None
    dA = torch.empty(r, d_in, dtype=torch.float32, device=X.device)
    dB = torch.empty(d_out, r, dtype=torch.float32, device=X.device)
    ws = L._workspace(L.OP_NF4_BWD, L.LORA_BF16, M, d_in, d_out, r, X.device, ws)
    tab = L._table_ptr(table16)
    L._check("nf4_lora_linear_bwd", L.lib().nf4_lora_linear_bwd(
        M, d_in, d_out, r, float(scale), L._ptr(X), L._ptr(codes), L._ptr(absmax), blocksize, tab, L._ptr(A),
        L._ptr(B), L._ptr(dY), L._ptr(dX), L._ptr(dA), L._ptr(dB), L._ptr(ws), ws.numel(), L._stream(X.device)))
    return dX, dA, dB


def nf4_dequant(codes, absmax, table16, n: int, blocksize: int = 64):
    """bf16 [n] from NF4 codes with the GEMM load stage's own routine."""
    out = torch.empty(n, dtype=torch.bfloat16, device=codes.device)
    tab = L._table_ptr(table16)
    L._check("nf4_dequant", L.lib().nf4_dequant(L._ptr(codes), L._ptr(absmax), blocksize, n, tab, L._ptr(out),
                                                L._stream(codes.device)))
    return out


def lora_dropout_fwd(X, W, A, B, scale: float, p: float, keep, Y=None, ws=None):
    """Y = X W^T + scale (D A^T) B^T, D = X * keep / (1 - p); keep is the packed
    uint8 bit mask [M, d_in / 8] (bit b of byte (i, j) keeps element (i, 8 j + b))."""
    L._contig(X, W, A, B, keep, Y)
    M, d_in, d_out, r = _dims(X, W.shape[0], W.shape[1], A, B)
    _check_keep(keep, M, d_in)
    dt = L._dtype_code(X)
    if Y is None:
        Y = torch.empty(M, d_out, dtype=X.dtype, device=X.device)
    ws = L._workspace(L.OP_DROPOUT_FWD, dt, M, d_in, d_out, r, X.device, ws)
    L._check("lora_dropout_fwd", L.lib().lora_dropout_fwd(
        dt, M, d_in, d_out, r, float(scale), float(p), L._ptr(keep), L._ptr(X), L._ptr(W), L._ptr(A), L._ptr(B),
        L._ptr(Y), L._ptr(ws), ws.numel(), L._stream(X.device)))
    return Y


def lora_dropout_bwd(X, W, A, B, scale: float, p: float, keep, dY, need_dX: bool = True, ws=None):
    """(dX or None, dA fp32, dB fp32) of lora_dropout_fwd with the same keep mask."""
    L._contig(X, W, A, B, keep, dY)
    M, d_in, d_out, r = _dims(X, W.shape[0], W.shape[1], A, B)
    _check_keep(keep, M, d_in)
    dt = L._dtype_code(X)
    dX = torch.empty(M, d_in, dtype=X.dtype, device=X.device) if need_dX else None
    dA = torch.empty(r, d_in, dtype=torch.float32, device=X.device)
    dB = torch.empty(d_out, r, dtype=torch.float32, device=X.device)
    ws = L._workspace(L.OP_DROPOUT_BWD, dt, M, d_in, d_out, r, X.device, ws)
    L._check("lora_dropout_bwd", L.lib().lora_dropout_bwd(
        dt, M, d_in, d_out, r, float(scale), float(p), L._ptr(keep), L._ptr(X), L._ptr(W), L._ptr(A), L._ptr(B),
        L._ptr(dY), L._ptr(dX), L._ptr(dA), L._ptr(dB), L._ptr(ws), ws.numel(), L._stream(X.device)))
    return dX, dA, dB


def lora_dropout_mask(M: int, d_in: int, p: float, seed: int, offset: int = 0, device="cuda"):
    """The packed keep mask [M, d_in / 8] (uint8) that the Philox dropout entry
    points draw for (seed, offset), generated on the device."""
    keep = torch.empty(M, d_in // 8, dtype=torch.uint8, device=device)
    L._check("lora_dropout_mask", L.lib().lora_dropout_mask(M, d_in, float(p), int(seed), int(offset),
                                                            L._ptr(keep), L._stream(keep.device)))
    return keep


def lora_dropout_philox_fwd(X, W, A, B, scale: float, p: float, seed: int, offset: int = 0, Y=None, ws=None):
    """lora_dropout_fwd with the keep mask drawn on the device from Philox4x32-10
    (seed, offset), as lora_dropout_mask draws it."""
    L._contig(X, W, A, B, Y)
    M, d_in, d_out, r = _dims(X, W.shape[0], W.shape[1], A, B)
    dt = L._dtype_code(X)
    if Y is None:
        Y = torch.empty(M, d_out, dtype=X.dtype, device=X.device)
    ws = L._workspace(L.OP_DROPOUT_FWD, dt, M, d_in, d_out, r, X.device, ws)
    L._check("lora_dropout_philox_fwd", L.lib().lora_dropout_philox_fwd(
        dt, M, d_in, d_out, r, float(scale), float(p), int(seed), int(offset), L._ptr(X), L._ptr(W), L._ptr(A),
        L._ptr(B), L._ptr(Y), L._ptr(ws), ws.numel(), L._stream(X.device)))
    return Y


def lora_dropout_philox_bwd(X, W, A, B, scale: float, p: float, seed: int, dY, offset: int = 0,
                            need_dX: bool = True, ws=None):
    """(dX or None, dA fp32, dB fp32) of lora_dropout_philox_fwd with the same
    (seed, offset): the mask is drawn again, not stored."""
    L._contig(X, W, A, B, dY)
    M, d_in, d_out, r = _dims(X, W.shape[0], W.shape[1], A, B)
    dt = L._dtype_code(X)
    dX = torch.empty(M, d_in, dtype=X.dtype, device=X.device) if need_dX else None
    dA = torch.empty(r, d_in, dtype=torch.float32, device=X.device)
    dB = torch.empty(d_out, r, dtype=torch.float32, device=X.device)
    ws = L._workspace(L.OP_DROPOUT_BWD, dt, M, d_in, d_out, r, X.device, ws)
    L._check("lora_dropout_philox_bwd", L.lib().lora_dropout_philox_bwd(
        dt, M, d_in, d_out, r, float(scale), float(p), int(seed), int(offset), L._ptr(X), L._ptr(W), L._ptr(A),
        L._ptr(B), L._ptr(dY), L._ptr(dX), L._ptr(dA), L._ptr(dB), L._ptr(ws), ws.numel(), L._stream(X.device)))
    return dX, dA, dB


def _check_keep(keep, M, d_in):
    if keep.dtype != torch.uint8 or keep.numel() != M * d_in // 8:
        raise ValueError("keep must be a uint8 bit mask of M * d_in / 8 bytes")


def lora_transpose(W, out=None):
    """W^T (bf16) through the library's tiled transpose, e.g. the frozen
    weight's transpose that group members take as W_t."""
    L._contig(W, out)
    if W.dtype != torch.bfloat16 or W.dim() != 2:
        raise TypeError("bf16 matrix expected")
    rows, cols = W.shape
    if out is None:
        out = torch.empty(cols, rows, dtype=W.dtype, device=W.device)
    L._check("lora_transpose", L.lib().lora_transpose(L._ptr(W), rows, cols, L._ptr(out), L._stream(W.device)))
    return out


def lora_merge(W, A, B, scale: float, out=None, ws=None):
    """W + scale B A in W's dtype (out may be W itself); -scale unmerges."""
    L._contig(W, A, B, out)
    d_out, d_in = W.shape
    r = A.shape[0]
    if A.shape != (r, d_in) or B.shape != (d_out, r):
        raise ValueError("shape mismatch: W [d_out,d_in], A [r,d_in], B [d_out,r]")
    dt = L._dtype_code(W)
    if out is None:
        out = torch.empty_like(W)
    ws = L._workspace(L.OP_MERGE, dt, 0, d_in, d_out, r, W.device, ws)
    L._check("lora_merge", L.lib().lora_merge(dt, d_out, d_in, r, float(scale), L._ptr(W), L._ptr(A), L._ptr(B),
                                              L._ptr(out), L._ptr(ws), ws.numel(), L._stream(W.device)))
    return out


def _group_members(X, members):
    """ctypes array of lora_group_member from dicts with keys A, B, scale and
    either W or (codes, absmax), plus an optional rope flag."""
    n = len(members)
    if not 1 <= n <= L.GROUP_MAX:
        raise ValueError(f"a group holds 1..{L.GROUP_MAX} projections")
    arr = (L.GroupMember * n)()
    M, d_in = X.shape
    for g, m in enumerate(members):
        A, B = m["A"], m["B"]
        W, codes, absmax, Wt = m.get("W"), m.get("codes"), m.get("absmax"), m.get("W_t")
        L._contig(A, B, W, codes, absmax, Wt)
        r, d_out = A.shape[0], B.shape[0]
        if A.shape != (r, d_in) or B.shape != (d_out, r) or (W is not None and W.shape != (d_out, d_in)):
            raise ValueError("shape mismatch: X [M,d_in], W [d_out,d_in], A [r,d_in], B [d_out,r]")
        if (W is None) == (codes is None):
            raise ValueError("each member takes exactly one of W and NF4 codes")
        e = arr[g]
        e.d_out, e.r, e.scale, e.rope = d_out, r, float(m["scale"]), int(bool(m.get("rope", False)))
        if Wt is not None and (Wt.shape != (d_in, d_out) or Wt.dtype != torch.bfloat16):
            raise ValueError("W_t must be the bf16 [d_in, d_out] transpose of W")
        e.W, e.W_nf4, e.absmax, e.W_t = (L._ptr(t) for t in (W, codes, absmax, Wt))
        e.A, e.B = L._ptr(A), L._ptr(B)
    return arr


def _group_ws(backward, dt, M, d_in, arr, device, ws):
    if ws is not None:
        return ws  # the library checks its size
    n = int(L.lib().lora_group_workspace_bytes(int(backward), dt, M, d_in, len(arr), arr))
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device)


def _group_rope(positions, cos, sin, M):
    if positions is None:
        return None, None, None, 0
    L._contig(positions, cos, sin)
    if positions.dtype != torch.int32 or positions.numel() != M:
        raise ValueError("positions must be int32 [M]")
    return L._ptr(positions), L._ptr(cos), L._ptr(sin), cos.shape[0]


def lora_group_fwd(X, members, positions=None, cos=None, sin=None, table16=None, head_dim: int = 128, ws=None,
                   Ys=None):
    """[Y_1, .., Y_n] of projections sharing X, the rank-r panels in one pass over X."""
    L._contig(X)
    M, d_in = X.shape
    dt = L._dtype_code(X)
    arr = _group_members(X, members)
    if Ys is None:
        Ys = [torch.empty(M, arr[g].d_out, dtype=X.dtype, device=X.device) for g in range(len(arr))]
    for g, Y in enumerate(Ys):
        L._contig(Y)
        if Y.shape != (M, arr[g].d_out) or Y.dtype != X.dtype:
            raise ValueError("Y shape or dtype mismatch")
        arr[g].Y = L._ptr(Y)
    pos, c, s, max_pos = _group_rope(positions, cos, sin, M)
    tab = L._table_ptr(table16) if table16 is not None else None
    ws = _group_ws(False, dt, M, d_in, arr, X.device, ws)
    L._check("lora_group_fwd", L.lib().lora_group_fwd(
        dt, M, d_in, len(arr), arr, L._ptr(X), head_dim, pos, c, s, max_pos, tab, L._ptr(ws), ws.numel(),
        L._stream(X.device)))
    return Ys


def lora_group_bwd(X, members, dYs, positions=None, cos=None, sin=None, table16=None, head_dim: int = 128,
                   need_dX: bool = True, ws=None, outs=None):
    """[(dX_g or None, dA_g fp32, dB_g fp32)] per member; dX_g is the member's own
    input gradient (the caller sums them)."""
    L._contig(X, *dYs)
    M, d_in = X.shape
    dt = L._dtype_code(X)
    arr = _group_members(X, members)
    if len(dYs) != len(arr):
        raise ValueError("one dY per member")
    res = []
    for g in range(len(arr)):
        d_out, r = arr[g].d_out, arr[g].r
        if dYs[g].shape != (M, d_out):
            raise ValueError("dY shape mismatch")
        if outs is None:
            dX = torch.empty(M, d_in, dtype=X.dtype, device=X.device) if need_dX else None
            dA = torch.empty(r, d_in, dtype=torch.float32, device=X.device)
            dB = torch.empty(d_out, r, dtype=torch.float32, device=X.device)
        else:
            dX, dA, dB = outs[g]
            L._contig(dX, dA, dB)
            if (dX is not None and dX.shape != (M, d_in)) or dA.shape != (r, d_in) or dB.shape != (d_out, r) \
                    or dA.dtype != torch.float32 or dB.dtype != torch.float32:
                raise ValueError("output shape or dtype mismatch")
        arr[g].dY, arr[g].dX, arr[g].dA, arr[g].dB = L._ptr(dYs[g]), L._ptr(dX), L._ptr(dA), L._ptr(dB)
        res.append((dX, dA, dB))
    pos, c, s, max_pos = _group_rope(positions, cos, sin, M)
    tab = L._table_ptr(table16) if table16 is not None else None
    ws = _group_ws(True, dt, M, d_in, arr, X.device, ws)
    L._check("lora_group_bwd", L.lib().lora_group_bwd(
        dt, M, d_in, len(arr), arr, L._ptr(X), head_dim, pos, c, s, max_pos, tab, L._ptr(ws), ws.numel(),
        L._stream(X.device)))
    return res


def _swiglu_ws(backward, dt, M, d_in, arr, device, ws):
    if ws is not None:
        return ws  # the library checks its size
    n = int(L.lib().lora_swiglu_workspace_bytes(int(backward), dt, M, d_in, arr))
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device)


def lora_swiglu_fwd(X, members, table16=None, H=None, store_gu: bool = True, ws=None):
    """(H, G, U) for the gate (members[0]) and up (members[1]) projections of X:
    H = silu(G) * U; G and U come back (for the backward) when store_gu, else None."""
    L._contig(X, H)
    if len(members) != 2:
        raise ValueError("SwiGLU takes the gate and the up projection")
    M, d_in = X.shape
    dt = L._dtype_code(X)
    arr = _group_members(X, members)
    d = arr[0].d_out
    if H is None:
        H = torch.empty(M, d, dtype=X.dtype, device=X.device)
    G = U = None
    if store_gu:
        G = torch.empty(M, d, dtype=X.dtype, device=X.device)
        U = torch.empty(M, d, dtype=X.dtype, device=X.device)
        arr[0].Y, arr[1].Y = L._ptr(G), L._ptr(U)
    tab = L._table_ptr(table16) if table16 is not None else None
    ws = _swiglu_ws(False, dt, M, d_in, arr, X.device, ws)
    L._check("lora_swiglu_fwd", L.lib().lora_swiglu_fwd(dt, M, d_in, arr, L._ptr(X), tab, L._ptr(H), L._ptr(ws),
                                                        ws.numel(), L._stream(X.device)))
    return H, G, U


def lora_swiglu_bwd(X, members, dH, G, U, table16=None, need_dX: bool = True, ws=None):
    """(dX or None, [(dA_gate, dB_gate), (dA_up, dB_up)]); dX sums both input gradients."""
    L._contig(X, dH, G, U)
    if len(members) != 2:
        raise ValueError("SwiGLU takes the gate and the up projection")
    M, d_in = X.shape
    dt = L._dtype_code(X)
    arr = _group_members(X, members)
    d = arr[0].d_out
    for t in (dH, G, U):
        if t.shape != (M, d):
            raise ValueError("dH, G and U must be [M, d_out]")
    dX = torch.empty(M, d_in, dtype=X.dtype, device=X.device) if need_dX else None
    grads = []
    for g in range(2):
        dA = torch.empty(arr[g].r, d_in, dtype=torch.float32, device=X.device)
        dB = torch.empty(d, arr[g].r, dtype=torch.float32, device=X.device)
        arr[g].dA, arr[g].dB = L._ptr(dA), L._ptr(dB)
        grads.append((dA, dB))
    tab = L._table_ptr(table16) if table16 is not None else None
    ws = _swiglu_ws(True, dt, M, d_in, arr, X.device, ws)
    L._check("lora_swiglu_bwd", L.lib().lora_swiglu_bwd(
        dt, M, d_in, arr, L._ptr(X), tab, L._ptr(dH), L._ptr(G), L._ptr(U), L._ptr(dX), L._ptr(ws), ws.numel(),
        L._stream(X.device)))
    return dX, grads


class LoraLinearFunction(torch.autograd.Function):
    """Autograd wrapper: gradients for X, A and B (W frozen); A and B grads in fp32."""

    @staticmethod
    def forward(ctx, X, W, A, B, scale):
        ctx.save_for_backward(X, W, A, B)
        ctx.scale = scale
        return lora_linear_fwd(X, W, A, B, scale)

    @staticmethod
    def backward(ctx, dY):
        X, W, A, B = ctx.saved_tensors
        dX, dA, dB = lora_linear_bwd(X, W, A, B, ctx.scale, dY.contiguous(), need_dX=ctx.needs_input_grad[0])
        return dX, None, dA.to(A.dtype), dB.to(B.dtype), None
