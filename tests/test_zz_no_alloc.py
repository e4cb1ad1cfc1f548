"""The allocation-free forward (lora_linear_fwd_noalloc): its scratch is the
library's static device array instead of a caller workspace.  Through the C
ABI it must give exactly what lora_linear_fwd gives (same kernels, so bit for
bit) and meet the oracle's bar, on calls in a row that reuse the array with
shrinking problems (a later call must not see an earlier call's data), over
every forward path: whole 256 x 256 tiles, generic tiles, the few-token split
and one-launch paths, the few-token W stream (its arrival counters and
partials live in the array), a ragged rank and fp32."""
import ctypes

import numpy as np
import pytest
import torch

import oracle as O
from tests.helpers import TOL, lora_inputs, rel, sample_rows

# (dtype, M, d_in, d_out, r): each sequence runs largest first
SEQUENCES = [
    [("bf16", 8192, 4096, 4096, 64), ("bf16", 300, 512, 768, 16)],
    [("bf16", 2100, 1024, 4096, 40), ("bf16", 100, 1024, 2048, 5), ("bf16", 16, 512, 512, 8)],
    [("f32", 1000, 520, 392, 24), ("f32", 128, 256, 256, 8)],
    [("bf16", 64, 2048, 4096, 32), ("bf16", 24, 1024, 1024, 8)],
]


def _check_call(lib, dtype, M, d_in, d_out, r, seed):
    s = 16.0 / r
    X, W, A, B, _ = lora_inputs(seed, M, d_in, d_out, r, dtype)
    Y = lib.lora_linear_fwd_noalloc(X, W, A, B, s)
    Yw = lib.lora_linear_fwd(X, W, A, B, s)
    torch.cuda.synchronize()
    assert torch.equal(Y, Yw), (dtype, M, d_in, d_out, r)
    rows = sample_rows(M, M, 1)
    tr = torch.from_numpy(rows).cuda()
    err = rel(Y[tr], O.lora_forward(X[tr], W, A, B, s))
    print(dtype, M, d_in, d_out, r, err, flush=True)
    assert err <= TOL[dtype]


@pytest.mark.gpu
@pytest.mark.parametrize("seq", SEQUENCES, ids=[f"seq{i}" for i in range(len(SEQUENCES))])
def test_noalloc_matches_workspace_forward(lib, seq):
    for i, (dtype, M, d_in, d_out, r) in enumerate(seq):
        _check_call(lib, dtype, M, d_in, d_out, r, 4100 + 17 * i + M)


@pytest.mark.gpu
def test_noalloc_rejects_what_does_not_fit(lib):
    from lora_linear_layers_amd import _lib

    X, W, A, B, _ = lora_inputs(5, 16, 256, 256, 8, "bf16")
    M = 1 << 20  # its panel partials alone exceed the static array
    need = _lib.workspace_bytes(_lib.OP_FWD, _lib.LORA_BF16, M, 4096, 4096, 64)
    assert need > _lib.STATIC_SCRATCH_BYTES
    p = ctypes.c_void_p(X.data_ptr())
    rc = _lib.lib().lora_linear_fwd_noalloc(_lib.LORA_BF16, M, 4096, 4096, 64, 1.0, p, p, p, p, p,
                                            _lib._stream(X.device))
    assert rc == -7, rc
    # nothing was launched: a following call still works
    _check_call(lib, "bf16", 300, 512, 768, 16, 77)
