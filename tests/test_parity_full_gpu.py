"""Full-size parity of every projection of the five workloads, each through
its single-projection entry point (lora_linear_*, lora_qk_rope_*,
nf4_lora_linear_*), against the float64 oracle.  The group calls with a
caller-held W^T that bench.py times are covered at the same sizes by
test_bench_workload_gpu.  All of dA and dB are compared; Y and dX on 256
seeded rows that include every sequence's first and last token (the oracle is
row-wise in them).  Bar: max|gpu - ref| / max|ref| <= 1e-5 (fp32 workload) or
2e-2 (bf16 inputs, fp32 accumulate)."""
import numpy as np
import pytest
import torch

import oracle as O
from synth import CONFIGS, gen
from synth.configs import Inputs
from tests.helpers import cpu64, rel, sample_rows

pytestmark = pytest.mark.gpu

CASES = [(c, p.name) for c, cfg in CONFIGS.items() for p in cfg.projections]


@pytest.mark.parametrize("cfg_id,pname", CASES, ids=[f"c{c}-{p}" for c, p in CASES])
def test_full_size_parity(lib, cfg_id, pname):
    cfg = CONFIGS[cfg_id]
    p = next(q for q in cfg.projections if q.name == pname)
    inp = Inputs(cfg, device="cuda")
    X, A, B, dY = inp.X(p), inp.A(p), inp.B(p), inp.dY(p)
    s = cfg.scale
    table = gen.nf4_table()
    pos = None
    if cfg.nf4:
        codes, absmax = inp.nf4(p)
        Y = lib.nf4_lora_linear_fwd(X, codes, absmax, table, A, B, s, p.d_out)
        dX, dA, dB = lib.nf4_lora_linear_bwd(X, codes, absmax, table, A, B, s, dY)
    elif p.rope:
        W = inp.W(p)
        pos = inp.positions()
        cos, sin = lib.rope_cache(cfg.seq_len, cfg.head_dim, cfg.rope_theta)
        Y = lib.lora_qk_rope_fwd(X, W, A, B, s, pos, cos, sin)
        dX, dA, dB = lib.lora_qk_rope_bwd(X, W, A, B, s, pos, cos, sin, dY)
    else:
        W = inp.W(p)
        Y = lib.lora_linear_fwd(X, W, A, B, s)
        dX, dA, dB = lib.lora_linear_bwd(X, W, A, B, s, dY)
    torch.cuda.synchronize()

    rows = sample_rows(cfg.M, cfg.seq_len, cfg.batch)
    tr = torch.from_numpy(rows).cuda()
    if cfg.nf4:
        W64 = O.nf4_dequant(codes.cpu().numpy(), absmax.cpu().numpy(), table, p.d_out, p.d_in)
    else:
        W64 = cpu64(W)
    if pos is not None:
        pnp = pos.cpu().numpy()
        G = O.rope_rotate(dY, pnp, cfg.head_dim, cfg.rope_theta, inverse=True)
        Yr = O.qk_rope_forward(X[tr], W64, A, B, s, pnp[rows], cfg.head_dim, cfg.rope_theta)
    else:
        G = cpu64(dY)
        Yr = O.lora_forward(X[tr], W64, A, B, s)
    dXr = O.lora_grad_x(W64, A, B, s, G[rows])
    dAr, dBr = O.lora_grad_ab(X, A, B, s, G)

    tol = 1e-5 if cfg.dtype == "f32" else 2e-2
    errs = dict(Y=rel(Y[tr], Yr), dX=rel(dX[tr], dXr), dA=rel(dA, dAr), dB=rel(dB, dBr))
    print(f"c{cfg_id} {pname}", {k: f"{v:.2e}" for k, v in errs.items()})
    assert all(e <= tol for e in errs.values()), errs
    # <dA, A> = <dB, B> (both equal s <G, (X A^T) B^T>), on the GPU outputs
    # themselves; the sums cancel heavily, so the bound scales with the sum of
    # the absolute terms
    ia = float((dA.double() * A.double()).sum())
    ib = float((dB.double() * B.double()).sum())
    mag = float(np.abs(dAr * cpu64(A)).sum() + np.abs(dBr * cpu64(B)).sum())
    assert abs(ia - ib) <= tol * mag
