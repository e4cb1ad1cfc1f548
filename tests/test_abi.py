"""C-ABI contract checks that need no GPU: the library loads, exports every
symbol the header declares, sizes workspaces, and rejects bad arguments
before any HIP call (so these run with fake, never-dereferenced pointers)."""
import ctypes
import os
import re
import subprocess

import pytest

import lora_linear_layers_amd as L
from lora_linear_layers_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lora_linear.h")

OK, ENULL, ESHAPE, EALIGN, EDTYPE, EWS, EDEV = 0, -1, -2, -3, -4, -5, -6
P = 0x100000  # fake 16-byte-aligned address; validation never dereferences it


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\**\s*([a-z_0-9]+)\s*\(", src, flags=re.M))


@pytest.fixture(scope="module")
def lib():
    return L.load()


def test_header_declares_the_abi():
    assert _declared() == set(_lib.EXPORTS)


def test_every_declared_symbol_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", L.LIB_PATH], capture_output=True, text=True).stdout
    syms = {ln.split()[-1] for ln in out.splitlines() if ln.strip()}
    for name in _declared():
        assert name in syms, name
        assert getattr(lib, name) is not None


def test_version_and_strerror(lib):
    assert lib.lora_abi_version() == 1
    for code in (OK, ENULL, ESHAPE, EALIGN, EDTYPE, EWS, EDEV):
        assert lib.lora_strerror(code)
    assert lib.lora_strerror(-99) == b"unknown error"


def test_workspace_sizes(lib):
    f = lib.lora_workspace_bytes
    # forward (bf16): the rank-r panel's split partials (64 row tiles of 128,
    # so 4 splits of the 4096 contraction for about one block per CU, fp32
    # [8192, 64] each) plus the [M, r8] bf16 panel
    assert f(_lib.OP_FWD, 1, 8192, 4096, 14336, 64) == 4 * 8192 * 64 * 4 + 8192 * 64 * 2
    # r not a multiple of 8 adds a padded copy of B
    assert f(_lib.OP_FWD, 1, 100, 64, 64, 3) > f(_lib.OP_FWD, 1, 100, 64, 64, 8) - 100 * 8 * 2
    bwd = f(_lib.OP_BWD, 1, 8192, 4096, 14336, 64)
    assert bwd >= 3 * 8192 * 64 * 2  # Pt, Qs, Qt
    assert f(_lib.OP_ROPE_BWD, 1, 8192, 4096, 4096, 64) >= f(_lib.OP_BWD, 1, 8192, 4096, 4096, 64) + 8192 * 4096 * 2
    assert f(_lib.OP_FWD, 0, 128, 256, 256, 8) == 128 * 8 * 4
    assert f(_lib.OP_FWD, 1, 0, 64, 64, 8) == 0
    # invalid arguments give 0
    assert f(9, 1, 8, 8, 8, 8) == 0
    assert f(_lib.OP_FWD, 7, 8, 8, 8, 8) == 0
    assert f(_lib.OP_FWD, 1, 8, 12, 8, 8) == 0


def _fwd(lib, dtype=1, M=16, d_in=64, d_out=64, r=8, X=P, W=P, A=P, B=P, Y=P, ws=P, wsb=1 << 30):
    return lib.lora_linear_fwd(dtype, M, d_in, d_out, r, 1.0, X, W, A, B, Y, ws, wsb, None)


def _bwd(lib, dtype=1, M=16, d_in=64, d_out=64, r=8, dY=P, dX=P, dA=P, dB=P, ws=P, wsb=1 << 30):
    return lib.lora_linear_bwd(dtype, M, d_in, d_out, r, 1.0, P, P, P, P, dY, dX, dA, dB, ws, wsb, None)


def test_fwd_validation(lib):
    assert _fwd(lib, dtype=2) == EDTYPE
    assert _fwd(lib, X=None) == ENULL
    assert _fwd(lib, W=None) == ENULL
    assert _fwd(lib, M=0, W=None) == ENULL
    assert _fwd(lib, Y=None) == ENULL
    assert _fwd(lib, d_in=12) == ESHAPE
    assert _fwd(lib, d_out=0) == ESHAPE
    assert _fwd(lib, r=0) == ESHAPE
    assert _fwd(lib, r=257) == ESHAPE
    assert _fwd(lib, M=-1) == ESHAPE
    assert _fwd(lib, W=P + 8) == EALIGN
    assert _fwd(lib, wsb=10) == EWS
    assert _fwd(lib, ws=None) == EWS
    assert _fwd(lib, ws=P + 4) == EALIGN


def test_bwd_validation(lib):
    assert _bwd(lib, dA=None) == ENULL
    assert _bwd(lib, dB=None) == ENULL
    assert _bwd(lib, dY=None) == ENULL
    assert _bwd(lib, dX=P + 2) == EALIGN
    assert _bwd(lib, wsb=1000) == EWS
    assert _bwd(lib, dtype=-1) == EDTYPE


def test_rope_validation(lib):
    def call(head_dim=128, d_out=256, pos=P, cs=P, max_pos=16):
        return lib.lora_qk_rope_fwd(1, 16, 64, d_out, 8, 1.0, P, P, P, P, head_dim, pos, cs, P, max_pos, P, P,
                                    1 << 30, None)
    assert call(head_dim=64) == ESHAPE
    assert call(d_out=192) == ESHAPE
    assert call(pos=None) == ENULL
    assert call(cs=P + 4) == EALIGN
    assert call(max_pos=0) == ESHAPE
    assert call(max_pos=1 << 23) == ESHAPE  # rows at 2^31 bytes and past
    assert call(max_pos=(1 << 23) - 1) != ESHAPE
    assert lib.lora_rope_cache(0, 128, 5e5, P, P, None) == ESHAPE
    assert lib.lora_rope_cache(16, 128, -1.0, P, P, None) == ESHAPE
    assert lib.lora_rope_cache(16, 128, 5e5, None, P, None) == ENULL


def test_nf4_validation(lib):
    tab = (ctypes.c_float * 16)(*range(16))

    def call(d_in=128, bs=64, codes=P, table=tab):
        return lib.nf4_lora_linear_fwd(16, d_in, 64, 8, 1.0, P, codes, P, bs, table, P, P, P, P, 1 << 30, None)
    assert call(bs=32) == ESHAPE
    assert call(d_in=96) == ESHAPE
    assert call(codes=None) == ENULL
    assert call(table=None) == ENULL
    assert lib.nf4_dequant(P, P, 64, 100, tab, P, None) == ESHAPE
    assert lib.nf4_dequant(P, P, 64, 128, None, P, None) == ENULL


@pytest.mark.skipif(__import__("torch").cuda.device_count() > 0, reason="checks the no-GPU path only")
def test_valid_call_without_gpu_reports_device_error(lib):
    # Arguments pass validation; with no device the library reports LORA_ERR_DEVICE
    # and launches nothing.
    assert _fwd(lib) == EDEV


def _members(n=2, **kw):
    arr = (_lib.GroupMember * n)()
    for g in range(n):
        e = arr[g]
        e.d_out, e.r, e.scale, e.rope = 64 * (g + 1), 8 + g, 1.0, 0
        e.W, e.A, e.B, e.Y, e.dY, e.dX, e.dA, e.dB = (P,) * 8
        for k, v in kw.items():
            setattr(e, k, v)
    return arr


def test_group_workspace_sizes(lib):
    f = lib.lora_group_workspace_bytes
    m = _members(3)
    fwd, bwd = f(0, 1, 4096, 1024, 3, m), f(1, 1, 4096, 1024, 3, m)
    rt = 8 + 16 + 16  # ranks 8, 9, 10 padded to multiples of 8
    assert fwd >= 4096 * rt * 2  # the group panel
    assert bwd >= 3 * 4096 * rt * 2  # Pt, Qs, Qt
    # fp32 groups run member by member: the largest member's own workspace
    single = max(lib.lora_workspace_bytes(_lib.OP_BWD, 0, 4096, 1024, 64 * (g + 1), 8 + g) for g in range(3))
    assert f(1, 0, 4096, 1024, 3, m) == single
    assert f(0, 1, 8, 8, 0, m) == 0
    assert f(0, 1, 8, 8, 9, _members(9)) == 0
    assert f(0, 5, 8, 64, 3, m) == 0
    assert f(0, 1, 8, 64, 3, None) == 0
    assert f(0, 1, 8, 64, 1, _members(1, r=0)) == 0


def _gfwd(lib, m, n=None, dtype=1, X=P, head_dim=128, pos=P, cs=P, max_pos=16, table=None, ws=P, wsb=1 << 30):
    n = len(m) if n is None else n
    return lib.lora_group_fwd(dtype, 16, 64, n, m, X, head_dim, pos, cs, cs, max_pos, table, ws, wsb, None)


def _gbwd(lib, m, dtype=1, ws=P, wsb=1 << 30):
    return lib.lora_group_bwd(dtype, 16, 64, len(m), m, P, 128, P, P, P, 16, None, ws, wsb, None)


def test_group_validation(lib):
    tab = (ctypes.c_float * 16)(*range(16))
    assert _gfwd(lib, _members(2), n=0) == ESHAPE
    assert _gfwd(lib, _members(9)) == ESHAPE
    assert _gfwd(lib, None, n=1) == ENULL
    assert _gfwd(lib, _members(2), dtype=3) == EDTYPE
    assert _gfwd(lib, _members(2), X=None) == ENULL
    assert _gfwd(lib, _members(2, Y=None)) == ENULL
    assert _gfwd(lib, _members(2, A=P + 2)) == EALIGN
    assert _gfwd(lib, _members(2, r=300)) == ESHAPE
    assert _gfwd(lib, _members(2, W=None)) == ENULL
    # RoPE members need head_dim 128 and d_out a multiple of it
    assert _gfwd(lib, _members(1, rope=1), head_dim=64) == ESHAPE
    assert _gfwd(lib, _members(2, rope=1)) == ESHAPE  # member 0 has d_out 64
    assert _gfwd(lib, _members(1, rope=1, d_out=128), pos=None) == ENULL
    # NF4 members: bf16 only, table required, no RoPE
    assert _gfwd(lib, _members(1, W=None, W_nf4=P, absmax=P), table=tab, dtype=0) == EDTYPE
    assert _gfwd(lib, _members(1, W=None, W_nf4=P, absmax=P)) == ENULL
    assert _gfwd(lib, _members(1, W=None, W_nf4=P, absmax=P, rope=1, d_out=128), table=tab) == ESHAPE
    assert _gfwd(lib, _members(2), wsb=100) == EWS
    assert _gbwd(lib, _members(2, dA=None)) == ENULL
    assert _gbwd(lib, _members(2, dY=None)) == ENULL
    assert _gbwd(lib, _members(2, dX=P + 8)) == EALIGN
    assert _gbwd(lib, _members(2), wsb=100) == EWS


def test_mfma_rate_validation(lib):
    assert lib.lora_mfma_rate(0, 4, P, None) == ESHAPE
    assert lib.lora_mfma_rate(4, 0, P, None) == ESHAPE
    assert lib.lora_mfma_rate(4, 4, None, None) == ENULL
    assert lib.lora_mfma_rate(4, 4, P + 4, None) == EALIGN


def test_profile_only_validation(lib):
    n = lib.lora_profile_kinds()
    assert lib.lora_profile_only(-2) == ESHAPE
    assert lib.lora_profile_only(n) == ESHAPE
    assert lib.lora_profile_only(n - 1) == 0
    assert lib.lora_profile_only(-1) == 0


def test_nf4_fwd_path_switch(lib):
    # the NF4 forward path switch: previous mode back, bad modes rejected, and
    # the workspace follows it (the load stage needs no dequantised W)
    f = lib.lora_workspace_bytes
    prev = lib.lora_set_nf4_fwd_path(1)
    try:
        assert lib.lora_set_nf4_fwd_path(3) == ESHAPE
        assert lib.lora_set_nf4_fwd_path(-1) == ESHAPE
        deq = f(_lib.OP_NF4_FWD, 1, 1024, 1024, 2048, 16)
        assert lib.lora_set_nf4_fwd_path(2) == 1
        whole = f(_lib.OP_NF4_FWD, 1, 1024, 1024, 2048, 16)
        assert deq - whole >= 2048 * 1024 * 2
        # below LORA_NF4_DEQUANT_MIN_TOKENS, or with tiles that are not whole,
        # nothing changes
        assert f(_lib.OP_NF4_FWD, 1, 256, 1024, 2048, 16) == f(_lib.OP_NF4_FWD, 1, 256, 1024, 2048, 16)
        lib.lora_set_nf4_fwd_path(1)
        ragged = f(_lib.OP_NF4_FWD, 1, 1000, 1024, 2048, 16)
        lib.lora_set_nf4_fwd_path(2)
        assert f(_lib.OP_NF4_FWD, 1, 1000, 1024, 2048, 16) == ragged
    finally:
        lib.lora_set_nf4_fwd_path(prev)


def test_merge_validation(lib):
    def call(dtype=1, d_out=64, d_in=64, r=8, W=P, A=P, B=P, out=P, ws=P, wsb=1 << 20):
        return lib.lora_merge(dtype, d_out, d_in, r, 1.0, W, A, B, out, ws, wsb, None)
    assert call(dtype=2) == EDTYPE
    assert call(d_in=12) == ESHAPE
    assert call(r=0) == ESHAPE
    assert call(r=300) == ESHAPE
    assert call(W=None) == ENULL
    assert call(out=None) == ENULL
    assert call(A=P + 8) == EALIGN
    assert call(r=3, wsb=10) == EWS
    assert call(r=3, ws=None) == EWS
    f = lib.lora_workspace_bytes
    assert f(_lib.OP_MERGE, 1, 0, 64, 64, 8) == 0
    assert f(_lib.OP_MERGE, 1, 0, 64, 96, 3) == 96 * 8 * 2
    assert f(_lib.OP_MERGE, 0, 0, 64, 96, 3) == 96 * 8 * 4


def test_swiglu_validation_and_workspace(lib):
    f = lib.lora_swiglu_workspace_bytes
    m = _members(2, d_out=1024, r=16)
    fused = f(0, 1, 4096, 4096, m)  # whole tiles: one GEMM, no G/U buffers
    ragged = f(0, 1, 4100, 4096, m)  # elementwise path: G and U in the workspace
    assert ragged >= 2 * 4100 * 1024 * 2 and fused < ragged
    assert f(1, 1, 4096, 4096, m) >= 2 * 4096 * 1024 * 2 + 4096 * 4096 * 2  # dG, dU, up's dX
    assert f(0, 1, 16, 64, _members(2)) == 0  # unequal d_out
    assert f(0, 5, 16, 64, m) == 0

    def fwd(mb, dtype=1, H=P, X=P, wsb=1 << 30):
        return lib.lora_swiglu_fwd(dtype, 16, 64, mb, X, None, H, P, wsb, None)
    assert fwd(_members(2)) == ESHAPE  # d_out 64 vs 128
    assert fwd(_members(2, d_out=64, rope=1)) == ESHAPE
    assert fwd(_members(2, d_out=64), H=None) == ENULL
    assert fwd(_members(2, d_out=64), X=None) == ENULL
    assert fwd(_members(2, d_out=64, Y=P + 2)) == EALIGN
    assert fwd(_members(2, d_out=64, W=None, W_nf4=P, absmax=P)) == ENULL  # NF4 without a table
    assert fwd(_members(2, d_out=64), wsb=10) == EWS
    assert fwd(None) == ENULL

    def bwd(mb, dH=P, dX=P):
        return lib.lora_swiglu_bwd(1, 16, 64, mb, P, None, dH, P, P, dX, P, 1 << 30, None)
    assert bwd(_members(2, d_out=64), dH=None) == ENULL
    assert bwd(_members(2, d_out=64, dA=None)) == ENULL
    assert bwd(_members(2, d_out=64), dX=P + 4) == EALIGN


def test_dropout_validation_and_workspace(lib):
    def fwd(p=0.1, keep=P, X=P, M=16, wsb=1 << 30):
        return lib.lora_dropout_fwd(1, M, 64, 64, 8, 1.0, p, keep, X, P, P, P, P, P, wsb, None)
    assert fwd(p=1.0) == ESHAPE
    assert fwd(p=-0.1) == ESHAPE
    assert fwd(p=float("nan")) == ESHAPE
    assert fwd(keep=None) == ENULL
    assert fwd(keep=P + 8) == EALIGN
    assert fwd(wsb=10) == EWS

    def bwd(dX=P, dA=P, keep=P):
        return lib.lora_dropout_bwd(1, 16, 64, 64, 8, 1.0, 0.1, keep, P, P, P, P, P, dX, dA, P, P, 1 << 30, None)
    assert bwd(keep=None) == ENULL
    assert bwd(dA=None) == ENULL
    assert bwd(dX=P + 2) == EALIGN
    f = lib.lora_workspace_bytes
    # the masked copy of X joins the plain layer's workspace
    assert f(_lib.OP_DROPOUT_FWD, 1, 4096, 4096, 4096, 16) >= f(_lib.OP_FWD, 1, 4096, 4096, 4096, 16) + 4096 * 4096 * 2
    assert f(_lib.OP_DROPOUT_BWD, 0, 4096, 4096, 4096, 16) >= f(_lib.OP_BWD, 0, 4096, 4096, 4096, 16) + 4096 * 4096 * 4


def test_transpose_and_wt_validation(lib):
    assert lib.lora_transpose(P, 12, 64, P, None) == ESHAPE
    assert lib.lora_transpose(P, 64, 0, P, None) == ESHAPE
    assert lib.lora_transpose(None, 64, 64, P, None) == ENULL
    assert lib.lora_transpose(P, 64, 64, P + 2, None) == EALIGN
    assert _gfwd(lib, _members(2, W_t=P + 8)) == EALIGN
    # a caller-held W^T removes the per-call transpose from the workspace
    m = _members(1, d_out=4096, r=16)
    mt = _members(1, d_out=4096, r=16, W_t=P)
    f = lib.lora_group_workspace_bytes
    assert f(1, 1, 8192, 4096, 1, m) - f(1, 1, 8192, 4096, 1, mt) >= 4096 * 4096 * 2 - 256


def test_dropout_mask_validation(lib):
    f = lib.lora_dropout_mask
    assert f(16, 12, 0.1, 1, 0, P, None) == ESHAPE  # d_in % 8
    assert f(16, 16, 1.0, 1, 0, P, None) == ESHAPE  # p outside [0, 1)
    assert f(16, 16, -0.1, 1, 0, P, None) == ESHAPE
    assert f(-1, 16, 0.1, 1, 0, P, None) == ESHAPE
    assert f(16, 16, 0.1, 1, 0, None, None) == ENULL
    assert f(0, 16, 0.1, 1, 0, None, None) == OK  # nothing to draw
    # the Philox layer entry points validate like the mask-taking ones
    fw = lib.lora_dropout_philox_fwd
    assert fw(1, 16, 64, 64, 8, 1.0, 1.0, 1, 0, P, P, P, P, P, P, 1 << 30, None) == ESHAPE
    assert fw(1, 16, 64, 64, 8, 1.0, 0.1, 1, 0, P, P, P, P, None, P, 1 << 30, None) == ENULL
    assert fw(1, 16, 64, 64, 8, 1.0, 0.1, 1, 0, P, P, P, P, P, P, 10, None) == EWS
    bw = lib.lora_dropout_philox_bwd
    assert bw(1, 16, 64, 64, 8, 1.0, 0.1, 1, 0, P, P, P, P, P, P, None, P, P, 1 << 30, None) == ENULL
    assert bw(1, 16, 64, 64, 8, 1.0, 0.1, 1, 0, P, P, P, P, P, P + 2, P, P, P, 1 << 30, None) == EALIGN
