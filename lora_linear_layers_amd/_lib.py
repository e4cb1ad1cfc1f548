"""ctypes binding of liblora_linear.so (the C ABI in include/lora_linear.h).

Argument marshalling only: torch tensors in, device pointers and the current
HIP stream out to the library, return codes turned into exceptions.  Every
step of the computation runs in the library's kernels; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liblora_linear.so")

LORA_F32, LORA_BF16 = 0, 1
STATIC_SCRATCH_BYTES = 32 << 20  # LORA_STATIC_SCRATCH_BYTES of the header
OP_FWD, OP_BWD, OP_ROPE_FWD, OP_ROPE_BWD, OP_NF4_FWD, OP_NF4_BWD, OP_MERGE, OP_DROPOUT_FWD, OP_DROPOUT_BWD = range(9)

_lib = None

_i64, _f32, _vp, _sz, _int, _dbl = (ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t,
                                    ctypes.c_int, ctypes.c_double)
_u64 = ctypes.c_uint64
_fp = ctypes.POINTER(ctypes.c_float)

GROUP_MAX = 8


class GroupMember(ctypes.Structure):
    """struct lora_group_member of the C ABI."""
    _fields_ = [("d_out", _i64), ("r", _i64), ("scale", _f32), ("rope", _int), ("W", _vp), ("W_nf4", _vp),
                ("absmax", _vp), ("A", _vp), ("B", _vp), ("Y", _vp), ("dY", _vp), ("dX", _vp), ("dA", _vp),
                ("dB", _vp), ("W_t", _vp)]


_mp = ctypes.POINTER(GroupMember)

_SIGS = {
    "lora_abi_version": ([], _int),
    "lora_strerror": ([_int], ctypes.c_char_p),
    "lora_workspace_bytes": ([_int, _int, _i64, _i64, _i64, _i64], _sz),
    "lora_linear_fwd": ([_int, _i64, _i64, _i64, _i64, _f32, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp], _int),
    "lora_linear_fwd_noalloc": ([_int, _i64, _i64, _i64, _i64, _f32, _vp, _vp, _vp, _vp, _vp, _vp], _int),
    "lora_linear_bwd": ([_int, _i64, _i64, _i64, _i64, _f32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz,
                         _vp], _int),
    "lora_rope_cache": ([_i64, _int, _dbl, _vp, _vp, _vp], _int),
    "lora_qk_rope_fwd": ([_int, _i64, _i64, _i64, _i64, _f32, _vp, _vp, _vp, _vp, _int, _vp, _vp, _vp, _i64, _vp,
                          _vp, _sz, _vp], _int),
    "lora_qk_rope_bwd": ([_int, _i64, _i64, _i64, _i64, _f32, _vp, _vp, _vp, _vp, _int, _vp, _vp, _vp, _i64, _vp,
                          _vp, _vp, _vp, _vp, _sz, _vp], _int),
    "nf4_lora_linear_fwd": ([_i64, _i64, _i64, _i64, _f32, _vp, _vp, _vp, _int, _fp, _vp, _vp, _vp, _vp, _sz, _vp],
                            _int),
    "nf4_lora_linear_bwd": ([_i64, _i64, _i64, _i64, _f32, _vp, _vp, _vp, _int, _fp, _vp, _vp, _vp, _vp, _vp, _vp,
                             _vp, _sz, _vp], _int),
    "nf4_dequant": ([_vp, _vp, _int, _i64, _fp, _vp, _vp], _int),
    "lora_group_workspace_bytes": ([_int, _int, _i64, _i64, _int, _mp], _sz),
    "lora_group_fwd": ([_int, _i64, _i64, _int, _mp, _vp, _int, _vp, _vp, _vp, _i64, _fp, _vp, _sz, _vp], _int),
    "lora_group_bwd": ([_int, _i64, _i64, _int, _mp, _vp, _int, _vp, _vp, _vp, _i64, _fp, _vp, _sz, _vp], _int),
    "lora_swiglu_fwd": ([_int, _i64, _i64, _mp, _vp, _fp, _vp, _vp, _sz, _vp], _int),
    "lora_swiglu_bwd": ([_int, _i64, _i64, _mp, _vp, _fp, _vp, _vp, _vp, _vp, _vp, _sz, _vp], _int),
    "lora_swiglu_workspace_bytes": ([_int, _int, _i64, _i64, _mp], _sz),
    "lora_merge": ([_int, _i64, _i64, _i64, _f32, _vp, _vp, _vp, _vp, _vp, _sz, _vp], _int),
    "lora_dropout_fwd": ([_int, _i64, _i64, _i64, _i64, _f32, _f32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp],
                         _int),
    "lora_dropout_bwd": ([_int, _i64, _i64, _i64, _i64, _f32, _f32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                          _vp, _sz, _vp], _int),
    "lora_dropout_mask": ([_i64, _i64, _f32, _u64, _u64, _vp, _vp], _int),
    "lora_dropout_philox_fwd": ([_int, _i64, _i64, _i64, _i64, _f32, _f32, _u64, _u64, _vp, _vp, _vp, _vp, _vp, _vp,
                                 _sz, _vp], _int),
    "lora_dropout_philox_bwd": ([_int, _i64, _i64, _i64, _i64, _f32, _f32, _u64, _u64, _vp, _vp, _vp, _vp, _vp, _vp,
                                 _vp, _vp, _vp, _sz, _vp], _int),
    "lora_mfma_rate": ([_int, _int, _vp, _vp], _int),
    "lora_transpose": ([_vp, _i64, _i64, _vp, _vp], _int),
    "lora_profile_begin": ([_int], _int),
    "lora_profile_end": ([], _int),
    "lora_profile_only": ([_int], _int),
    "lora_profile_kinds": ([], _int),
    "lora_set_nf4_fwd_path": ([_int], _int),
    "lora_profile_kind_name": ([_int], ctypes.c_char_p),
    "lora_profile_query": ([_int, ctypes.POINTER(_dbl), ctypes.POINTER(_int), ctypes.POINTER(_dbl),
                            ctypes.POINTER(_dbl)], _int),
}

EXPORTS = tuple(_SIGS)


class LoraError(RuntimeError):
    def __init__(self, fn, code):
        self.code = code
        msg = _lib.lora_strerror(code).decode() if _lib is not None else str(code)
        super().__init__(f"{fn} failed: {msg} ({code})")


def load(path: str = LIB_PATH):
    """Load the HIP library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m lora_linear_layers_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (args, res) in _SIGS.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = res
    _lib = lib
    return lib


def lib():
    return load()


def _check(fn, rc):
    if rc != 0:
        raise LoraError(fn, rc)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device=None):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return LORA_F32
    if t.dtype == torch.bfloat16:
        return LORA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _table_ptr(table16):
    tab = (ctypes.c_float * 16)(*[float(v) for v in table16])
    return tab


def workspace_bytes(op: int, dtype: int, M: int, d_in: int, d_out: int, r: int) -> int:
    return int(lib().lora_workspace_bytes(op, dtype, M, d_in, d_out, r))


def _workspace(op, dtype, M, d_in, d_out, r, device, ws=None):
    # a caller's workspace is passed through as it is: the library checks its
    # size against the layout itself (LORA_ERR_WORKSPACE)
    if ws is not None:
        return ws
    n = workspace_bytes(op, dtype, M, d_in, d_out, r)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device)


def _contig(*ts):
    for t in ts:
        if t is not None and not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def profile_begin(max_launches: int = 4096):
    _check("lora_profile_begin", lib().lora_profile_begin(max_launches))


def profile_end():
    _check("lora_profile_end", lib().lora_profile_end())


def profile_only(kind_name=None):
    """Record only launches of the named kind (None: every kind)."""
    k = -1
    if kind_name is not None:
        names = [lib().lora_profile_kind_name(i).decode() for i in range(lib().lora_profile_kinds())]
        k = names.index(kind_name)
    _check("lora_profile_only", lib().lora_profile_only(k))


NF4_PATH = {"auto": 0, "dequant": 1, "load_stage": 2}


def set_nf4_fwd_path(mode: str) -> str:
    """Pick the NF4 forward path for later calls ("auto", "dequant" or
    "load_stage", lora_set_nf4_fwd_path); returns the previous one."""
    prev = lib().lora_set_nf4_fwd_path(NF4_PATH[mode])
    if prev < 0:
        _check("lora_set_nf4_fwd_path", prev)
    return {v: k for k, v in NF4_PATH.items()}[prev]


def mfma_rate(iters: int = 4096, blocks: int = 1024, device=None) -> float:
    """Dense bf16 MFMA TFLOP/s the chip sustains right now (lora_mfma_rate)."""
    out = torch.empty(blocks * 256, dtype=torch.float32, device=device or "cuda")
    st = _stream(out.device)
    _check("lora_mfma_rate", lib().lora_mfma_rate(iters, blocks, _ptr(out), st))  # warm-up
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    _check("lora_mfma_rate", lib().lora_mfma_rate(iters, blocks, _ptr(out), st))
    e1.record()
    e1.synchronize()
    return blocks * 4.0 * iters * 8 * 32768 / (e0.elapsed_time(e1) * 1e-3) / 1e12


def profile_report():
    """{kind name: (total_ms, count, total_flop, total_bytes)} for kinds that ran."""
    out = {}
    ms, n, fl, by = ctypes.c_double(), ctypes.c_int(), ctypes.c_double(), ctypes.c_double()
    for k in range(lib().lora_profile_kinds()):
        _check("lora_profile_query", lib().lora_profile_query(k, ctypes.byref(ms), ctypes.byref(n),
                                                              ctypes.byref(fl), ctypes.byref(by)))
        if n.value:
            out[lib().lora_profile_kind_name(k).decode()] = (ms.value, n.value, fl.value, by.value)
    return out
