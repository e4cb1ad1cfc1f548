"""Full-size parity of exactly what bench.py times.

bench.Workload builds each workload the way the benchmark runs it:
projections that read the same X as one group call (lora_group_fwd /
lora_group_bwd), and, for bf16 weights, the frozen W^T held by the caller
(lora_transpose, once) for the input-gradient GEMM.  One step (every forward,
then every backward in reverse order) is run and compared against the float64
oracle: every member's Y and dX on 256 seeded rows (each sequence's first and
last token among them; the oracle is row-wise in both), all of dA and dB.
Bar: max|gpu - ref| / max|ref| <= 2e-2 (bf16 inputs, fp32 accumulate).

The launch kinds of the step are recorded too, so the test fails if the
timed configuration stops reaching the kernels it is meant to cover (the
one-launch group GEMM of the forwards, the whole-tile input-gradient GEMM).
"""
import numpy as np
import pytest
import torch

import oracle as O
from synth import CONFIGS, gen
from tests.helpers import cpu64, rel, sample_rows

pytestmark = pytest.mark.gpu

# the bf16 and NF4 workloads; the fp32 one (c1) runs single calls and is
# covered in full by test_parity_full_gpu
WORKLOADS = [2, 3, 4, 5]


def _step_kinds(work):
    from lora_linear_layers_amd import _lib

    _lib.profile_only(None)
    _lib.profile_begin(16 * len(work.cfg.projections) + 64)
    work.step()
    torch.cuda.synchronize()
    _lib.profile_end()
    return set(_lib.profile_report())


@pytest.mark.parametrize("cfg_id", WORKLOADS, ids=[f"c{c}" for c in WORKLOADS])
def test_bench_workload_parity(lib, cfg_id):
    import bench

    cfg = CONFIGS[cfg_id]
    work = bench.Workload(cfg, device="cuda")
    kinds = _step_kinds(work)
    print(f"c{cfg_id} groups", [[it["p"].name for it in g] for g in work.groups], sorted(kinds))
    # the forwards of every group run as one whole-tile group launch; bf16
    # weights take the input gradient through the caller's W^T
    assert "gemm_bf16_256x256_nt_group" in kinds or cfg.nf4, kinds
    assert "gemm_bf16_256x256_nt_store" in kinds, kinds
    assert "transpose_w" not in kinds or cfg.nf4, kinds
    if cfg.nf4:
        assert "nf4_dequant" in kinds, kinds

    rows = sample_rows(cfg.M, cfg.seq_len, cfg.batch)
    tr = torch.from_numpy(rows).cuda()
    s = cfg.scale
    table = gen.nf4_table()
    pnp = work.pos.cpu().numpy() if hasattr(work, "pos") else None
    for it in work.items:
        p = it["p"]
        X, A, B, dY = it["X"], it["A"], it["B"], it["dY"]
        if cfg.nf4:
            W64 = O.nf4_dequant(it["codes"].cpu().numpy(), it["absmax"].cpu().numpy(), table, p.d_out, p.d_in)
        else:
            W64 = cpu64(it["W"])
        if p.rope:
            G = O.rope_rotate(dY, pnp, cfg.head_dim, cfg.rope_theta, inverse=True)
            Yr = O.qk_rope_forward(X[tr], W64, A, B, s, pnp[rows], cfg.head_dim, cfg.rope_theta)
        else:
            G = cpu64(dY)
            Yr = O.lora_forward(X[tr], W64, A, B, s)
        dXr = O.lora_grad_x(W64, A, B, s, G[rows])
        dAr, dBr = O.lora_grad_ab(X, A, B, s, G)
        errs = dict(Y=rel(it["Y"][tr], Yr), dX=rel(it["dX"][tr], dXr), dA=rel(it["dA"], dAr),
                    dB=rel(it["dB"], dBr))
        print(f"c{cfg_id} {p.name}", {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
        assert all(e <= 2e-2 for e in errs.values()), (p.name, errs)
        del G, W64
