#!/usr/bin/env python3
"""Throughput of the fused LoRA linear layer (forward + backward) on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config 3]

One step is one forward and one backward through every projection of the
workload (the whole hot path): Y = X W^T + s (X A^T) B^T with the optional RoPE
epilogue or NF4 base weight, then dX, dA, dB with X A^T recomputed.  Inputs
are seeded synthetic tensors drawn directly in HBM before timing.

Prints ONE JSON line: TFLOP/s of useful work (2M(2dk + 3r(d+k)) per
projection), tokens/s, the fraction of the bf16 dense MFMA peak, a roofline
entry for the dominant kernel (its launches timed with HIP events on the
library's stream during the timed steps), and the float64 oracle timed on a
bounded token sample on the host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused LoRA linear fwd+bwd TFLOP/s & tokens/s, % bf16 MFMA peak, 1 GPU"
PEAK = {"bf16": 2516.6, "f32": 157.3}  # TFLOP/s, dense MFMA (MI355X: 256 CU x 2.4 GHz)
HBM_PEAK = 8000.0  # GB/s
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = ["lora_linear_layers_amd/csrc/gemm.h", "lora_linear_layers_amd/csrc/gemm_w4.h",
                  "lora_linear_layers_amd/csrc/gemm_w4_nt.h",
                  "lora_linear_layers_amd/csrc/kernels.hip", "lora_linear_layers_amd/csrc/api.cpp"]


def kernel_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=3, help="workload: 1..5 (3 = Llama-3-8B MLP)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--call-reps", type=int, default=10,
                    help="HIP-event repetitions of each call for the per-call median/p10/p90 (0 = skip)")
    ap.add_argument("--no-small-token", action="store_true", help="skip the few-token HBM sweep")
    ap.add_argument("--no-wt", action="store_true",
                    help="do not keep W^T of the frozen weights (the backward then transposes W per call)")
    ap.add_argument("--no-group", action="store_true",
                    help="run projections that share X one by one instead of as one group")
    ap.add_argument("--no-configs", action="store_true",
                    help="measure only the chosen workload (not every other one as well)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target oracle time for the CPU sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one 1 GiB device copy (reference kernel for HBM counters)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic.json from two rocprofv3 --pmc counter_collection.csv files "
                         "(FETCH_SIZE run, WRITE_SIZE run of this script with --copy-calibration), then exit")
    return ap.parse_args()


# rocprofv3 kernel names -> the library profiler's kind names
KIND_OF = {
    "gemm_w4_nt_kernel<0>": "gemm_bf16_256x256_nt_store",
    "gemm_w4_nt_kernel<3>": "gemm_bf16_256x256_nt_rope",
    "gemm_w4_nt_kernel<6>": "gemm_bf16_256x256_swiglu",
    "gemm_w4_nt_kernel<8>": "gemm_bf16_256x256_nt_group",
    "gemm_w4_nn_kernel<2>": "gemm_bf16_256x256_nn_store",
    "gemm_w4_nf4_kernel": "gemm_nf4_256x256_nt_whole",
    "gemm_kernel<unsigned short, 256, 64, 4, 1, false, 4, 0>": "panel_bf16_split",
    "panel_dma_kernel": "panel_bf16_split",
    "splitnn_dma_kernel": "split_bf16_nn_partial",
    "skinny_fwd_kernel": "skinny_fwd",
    "panel_reduce_kernel": "panel_reduce",
    "gemm_kernel<unsigned short, 256, 256, 2, 4, false, 0, 0>": "gemm_bf16_256x256_nt_store",
    "gemm_kernel<unsigned short, 256, 256, 2, 4, true, 0, 0>": "gemm_bf16_256x256_nn_store",
    "gemm_kernel<unsigned short, 256, 256, 2, 2, false, 3, 0>": "gemm_bf16_256x256_nt_rope",
    "gemm_kernel<unsigned short, 128, 128, 4, 1, false, 0, 0>": "gemm_bf16_128x128_nt_store",
    "gemm_kernel<unsigned short, 128, 128, 4, 1, false, 3, 0>": "gemm_bf16_128x128_nt_rope",
    "gemm_kernel<unsigned short, 128, 128, 4, 1, true, 0, 0>": "gemm_bf16_128x128_nn_store",
    "gemm_kernel<unsigned short, 256, 256, 2, 4, false, 0, 1>": "gemm_nf4_256x256_nt_store",
    "gemm_kernel<unsigned short, 256, 256, 2, 4, true, 0, 1>": "gemm_nf4_256x256_nn_store",
    "gemm_kernel<unsigned short, 128, 128, 4, 1, false, 0, 1>": "gemm_nf4_128x128_nt_store",
    "gemm_kernel<unsigned short, 128, 128, 4, 1, true, 0, 1>": "gemm_nf4_128x128_nn_store",
    "gemm_kernel<unsigned short, 64, 256, 1, 4, true, 4, 0>": "split_bf16_nn_partial",
    "reduce_splits_kernel": "reduce_splits",
    "transpose_pad_kernel": "transpose_ab",
    "transpose_batch_kernel": "transpose_ab",
    "reduce_batch_kernel": "reduce_splits",
    "rope_inverse_kernel": "rope_inverse",
    "transpose_tile_kernel": "transpose_w",
    "split_finish_kernel": "split_finish",
    "few_panel_kernel": "few_panel",
    "few_reduce_kernel": "few_panel",
    "few_fwd_nf4_kernel": "few_fwd",
    "few_fwd_bf16_kernel": "few_fwd",
    "few_bwd_kernel": "few_bwd",
    "nf4_dequant_t_kernel": "nf4_dequant",
    "nf4_dequant_kernel": "nf4_dequant",
    "tiny_fwd_f32_kernel": "tiny_f32",
    "tiny_bwd_f32_kernel": "tiny_f32",
}


def _kind(name):
    for k, v in KIND_OF.items():
        if k in name:
            return v
    return None


def traffic_from(fetch_csv, write_csv, cfg_id):
    """HBM bytes per launch of each library kernel from FETCH_SIZE / WRITE_SIZE
    (KiB per dispatch), each scaled so that a 1 GiB device copy reads and
    writes exactly 1 GiB."""
    import csv

    def per_dispatch(path, counter):
        vals, grid = {}, {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            key = (r["Dispatch_Id"], r["Kernel_Name"])
            vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
            grid[key] = int(r["Grid_Size"])
        return vals, grid

    out = {}
    factors = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        vals, grid = per_dispatch(path, counter)
        # the 1 GiB device-to-device copy of --copy-calibration: the runtime's
        # copy kernel with the largest reading of this counter
        copies = [v for (d, n), v in vals.items() if "copyBuffer" in n]
        ref = max(copies) if copies else None
        factor = (float(1 << 30) / (ref * 1024.0)) if ref else 1.0
        factors[counter] = {"copy_kib": ref, "scale": factor}
        sums = {}
        for (d, n), v in vals.items():
            k = _kind(n)
            if k:
                s, c = sums.get(k, (0.0, 0))
                sums[k] = (s + v * 1024.0 * factor, c + 1)
        for k, (s, c) in sums.items():
            out.setdefault(k, {})[counter.lower() + "_bytes_per_launch"] = s / c
    for k, v in out.items():
        v["bytes_per_launch"] = v.get("fetch_size_bytes_per_launch", 0.0) + v.get("write_size_bytes_per_launch", 0.0)
    return {"config": cfg_id, "kernel_hash": kernel_hash(), "scale": factors, "kernels": out}


class Workload:
    """Device tensors and preallocated outputs for every projection of a config."""

    def __init__(self, cfg, device="cuda", group=True, keep_wt=True):
        import torch

        import lora_linear_layers_amd as L
        from synth import gen
        from synth.configs import Inputs

        self.cfg = cfg
        self.L = L
        inp = Inputs(cfg, device=device)
        self.items = []
        xs = {}
        M, r = cfg.M, cfg.r
        if any(p.rope for p in cfg.projections):
            self.pos = inp.positions()
            self.cos, self.sin = L.rope_cache(cfg.seq_len, cfg.head_dim, cfg.rope_theta, device=device)
        self.table = gen.nf4_table()
        wsmax = 0
        dt = L.LORA_F32 if cfg.dtype == "f32" else L.LORA_BF16
        for p in cfg.projections:
            if p.x_group not in xs:
                xs[p.x_group] = inp.X(p)
            it = {"p": p, "X": xs[p.x_group], "A": inp.A(p), "B": inp.B(p), "dY": inp.dY(p)}
            if cfg.nf4:
                it["codes"], it["absmax"] = inp.nf4(p)
                ops = (L.OP_NF4_FWD, L.OP_NF4_BWD)
            else:
                it["W"] = inp.W(p)
                ops = (L.OP_ROPE_FWD, L.OP_ROPE_BWD) if p.rope else (L.OP_FWD, L.OP_BWD)
            tdt = it["X"].dtype
            it["Y"] = torch.empty(M, p.d_out, dtype=tdt, device=device)
            it["dX"] = torch.empty(M, p.d_in, dtype=tdt, device=device)
            it["dA"] = torch.empty(r, p.d_in, dtype=torch.float32, device=device)
            it["dB"] = torch.empty(p.d_out, r, dtype=torch.float32, device=device)
            for op in ops:
                wsmax = max(wsmax, L.workspace_bytes(op, dt, M, p.d_in, p.d_out, r))
            self.items.append(it)
        # projections that read the same X run as one group (in config order)
        self.groups = []
        for it in self.items:
            if group and self.groups and self.groups[-1][0]["p"].x_group == it["p"].x_group:
                self.groups[-1].append(it)
            else:
                self.groups.append([it])
        self.members = []
        for grp in self.groups:
            ms = []
            for it in grp:
                m = {"A": it["A"], "B": it["B"], "scale": cfg.scale, "rope": it["p"].rope}
                if cfg.nf4:
                    m["codes"], m["absmax"] = it["codes"], it["absmax"]
                else:
                    m["W"] = it["W"]
                    if keep_wt and cfg.dtype == "bf16":
                        # the frozen weight's transpose, made once: the backward's
                        # input gradient reads it (outside the timed steps)
                        m["W_t"] = L.lora_transpose(it["W"])
                ms.append(m)
            self.members.append(ms)
            if len(grp) > 1 or any("W_t" in m for m in ms):
                arr = L.functional._group_members(grp[0]["X"], ms)
                for bwd in (0, 1):
                    wsmax = max(wsmax, int(L.lib().lora_group_workspace_bytes(bwd, dt, M, grp[0]["p"].d_in,
                                                                             len(arr), arr)))
        self.ws = torch.empty(max(wsmax, 256), dtype=torch.uint8, device=device)
        torch.cuda.synchronize()

    def _rope_args(self):
        return (self.pos, self.cos, self.sin) if hasattr(self, "pos") else (None, None, None)

    def call_name(self, gi):
        return "+".join(it["p"].name for it in self.groups[gi])

    def call_flop(self, gi, bwd):
        """Useful FLOP of one call: 2M(dk + r(d+k)) forward, 2M(dk + 2r(d+k)) backward."""
        M, r = self.cfg.M, self.cfg.r
        f = 0.0
        for it in self.groups[gi]:
            p = it["p"]
            f += 2.0 * M * (p.d_in * p.d_out + (2 if bwd else 1) * r * (p.d_in + p.d_out))
        return f

    def _as_group(self, gi):
        return len(self.groups[gi]) > 1 or any("W_t" in m for m in self.members[gi])

    def fwd(self, gi):
        L, cfg, ws, s = self.L, self.cfg, self.ws, self.cfg.scale
        grp, ms = self.groups[gi], self.members[gi]
        if self._as_group(gi):
            L.lora_group_fwd(grp[0]["X"], ms, *self._rope_args(), table16=self.table if cfg.nf4 else None, ws=ws,
                             Ys=[it["Y"] for it in grp])
            return
        it = grp[0]
        p = it["p"]
        if cfg.nf4:
            L.nf4_lora_linear_fwd(it["X"], it["codes"], it["absmax"], self.table, it["A"], it["B"], s,
                                  p.d_out, Y=it["Y"], ws=ws)
        elif p.rope:
            L.lora_qk_rope_fwd(it["X"], it["W"], it["A"], it["B"], s, self.pos, self.cos, self.sin,
                               Y=it["Y"], ws=ws)
        else:
            L.lora_linear_fwd(it["X"], it["W"], it["A"], it["B"], s, Y=it["Y"], ws=ws)

    def bwd(self, gi):
        L, cfg, ws, s = self.L, self.cfg, self.ws, self.cfg.scale
        grp, ms = self.groups[gi], self.members[gi]
        if self._as_group(gi):
            L.lora_group_bwd(grp[0]["X"], ms, [it["dY"] for it in grp], *self._rope_args(),
                             table16=self.table if cfg.nf4 else None, ws=ws,
                             outs=[(it["dX"], it["dA"], it["dB"]) for it in grp])
            return
        it = grp[0]
        p = it["p"]
        out = (it["dX"], it["dA"], it["dB"])
        if cfg.nf4:
            _nf4_bwd(L, it, self.table, s, ws, out)
        elif p.rope:
            _rope_bwd(L, it, self, s, ws, out)
        else:
            L.lora_linear_bwd(it["X"], it["W"], it["A"], it["B"], s, it["dY"], ws=ws, out=out)

    def step(self):
        """One pass of the layer over the batch: every projection's forward, then
        every backward in reverse order."""
        for gi in range(len(self.groups)):
            self.fwd(gi)
        for gi in reversed(range(len(self.groups))):
            self.bwd(gi)


def _pct(ts):
    ts = sorted(ts)
    pick = lambda q: ts[min(len(ts) - 1, int(round(q * (len(ts) - 1))))]  # noqa: E731
    return {"median": round(pick(0.5), 4), "p10": round(pick(0.1), 4), "p90": round(pick(0.9), 4)}


def per_call_times(work, reps):
    """HIP-event time of each call (forward and backward apart), median/p10/p90 in ms."""
    import torch

    out = {}
    for gi in range(len(work.groups)):
        res = {}
        for kind, fn in (("fwd", work.fwd), ("bwd", work.bwd)):
            ts = []
            for _ in range(reps):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                fn(gi)
                e1.record()
                e1.synchronize()
                ts.append(e0.elapsed_time(e1))
            res[kind + "_ms"] = _pct(ts)
        t = res["fwd_ms"]["median"] + res["bwd_ms"]["median"]
        res["tflops"] = round((work.call_flop(gi, False) + work.call_flop(gi, True)) / (t * 1e-3) / 1e12, 1)
        out[work.call_name(gi)] = res
    return out


def _time_ms(fn, reps):
    import torch

    fn()
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        e1.synchronize()
        ts.append(e0.elapsed_time(e1))
    return _pct(ts)


def _time_interleaved(fns, reps):
    """HIP-event times of the calls in fns (name -> callable), taken round-robin
    (one call of each per round) so that every variant meets the same clock and
    thermal state of the GPU; median / p10 / p90 in ms per name."""
    import torch

    for fn in fns.values():
        fn()
    ts = {name: [] for name in fns}
    for _ in range(reps):
        for name, fn in fns.items():
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            e1.synchronize()
            ts[name].append(e0.elapsed_time(e1))
    return {name: _pct(t) for name, t in ts.items()}


def next_rows(work, reps=10):
    """The rows beyond the layer itself, on this workload's gate / up pair:
    SwiGLU (fused epilogue vs. the pair's plain group forward) and the merge of
    the gate adapter into its weight (HBM-bound: W read and written once)."""
    import torch

    L, cfg = work.L, work.cfg
    pair = [it for it in work.items if it["p"].name in ("gate_proj", "up_proj")]
    if len(pair) != 2 or cfg.dtype == "f32":
        return None
    out = {}
    M, s = cfg.M, cfg.scale
    X = pair[0]["X"]
    k, d = pair[0]["p"].d_in, pair[0]["p"].d_out
    tab = work.table if cfg.nf4 else None
    ms = []
    for it in pair:
        m = {"A": it["A"], "B": it["B"], "scale": s}
        if cfg.nf4:
            m["codes"], m["absmax"] = it["codes"], it["absmax"]
        else:
            m["W"] = it["W"]
        ms.append(m)
    H = torch.empty(M, d, dtype=X.dtype, device=X.device)
    G, U = pair[0]["Y"], pair[1]["Y"]
    dH = pair[0]["dY"]
    fwd_flop = 2.0 * 2 * M * (d * k + cfg.r * (d + k))
    bwd_flop = 2.0 * 2 * M * (d * k + 2 * cfg.r * (d + k))
    arr = L.functional._group_members(X, ms)
    wsb = max([int(L.lib().lora_swiglu_workspace_bytes(b, L.LORA_BF16, M, k, arr)) for b in (0, 1)] +
              [int(L.lib().lora_group_workspace_bytes(b, L.LORA_BF16, M, k, 2, arr)) for b in (0, 1)])
    ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=X.device)
    Gs, Us = L.lora_swiglu_fwd(X, ms, table16=tab, ws=ws)[1:]
    dU = pair[1]["dY"]
    # (interleaved: the comparison meets one clock state)
    sw = _time_interleaved({
        "fwd_with_gu_ms": lambda: L.lora_swiglu_fwd(X, ms, table16=tab, H=H, ws=ws),
        "fwd_h_only_ms": lambda: L.lora_swiglu_fwd(X, ms, table16=tab, H=H, store_gu=False, ws=ws),
        "group_fwd_ms": lambda: L.lora_group_fwd(X, ms, table16=tab, Ys=[G, U], ws=ws),
        "bwd_ms": lambda: L.lora_swiglu_bwd(X, ms, dH, Gs, Us, table16=tab, ws=ws),
        "group_bwd_ms": lambda: L.lora_group_bwd(X, ms, [dH, dU], table16=tab, ws=ws)}, reps)
    for key, fl in (("fwd_with_gu_ms", fwd_flop), ("fwd_h_only_ms", fwd_flop), ("group_fwd_ms", fwd_flop),
                    ("bwd_ms", bwd_flop), ("group_bwd_ms", bwd_flop)):
        sw[key.replace("_ms", "_tflops")] = round(fl / (sw[key]["median"] * 1e-3) / 1e12, 1)
    sw["shape"] = f"gate/up {k}->{d}, M={M}, r={cfg.r}" + (", NF4 W" if cfg.nf4 else "")
    out["swiglu"] = sw
    del ws, Gs, Us
    if not cfg.nf4:
        it = pair[0]
        # LoRA dropout (p = 0.05) on the gate projection vs the plain layer
        p = 0.05
        g = torch.Generator(device=X.device).manual_seed(3407)
        keep = (torch.rand(M, k // 8, 8, generator=g, device=X.device) >= p).to(torch.uint8)
        keep = (keep << torch.arange(8, dtype=torch.uint8, device=X.device)).sum(-1).to(torch.uint8).contiguous()
        dws = torch.empty(max(L.workspace_bytes(op, L.LORA_BF16, M, k, d, cfg.r)
                              for op in (L.OP_DROPOUT_FWD, L.OP_DROPOUT_BWD)), dtype=torch.uint8, device=X.device)
        one_fwd = 2.0 * M * (d * k + cfg.r * (d + k))
        one_bwd = 2.0 * M * (d * k + 2 * cfg.r * (d + k))
        dr = {"shape": f"{it['p'].name} {k}->{d}, M={M}, r={cfg.r}, p={p}"}
        dr.update(_time_interleaved({
            "fwd_ms": lambda: L.lora_dropout_fwd(X, it["W"], it["A"], it["B"], s, p, keep, Y=it["Y"], ws=dws),
            "plain_fwd_ms": lambda: L.lora_linear_fwd(X, it["W"], it["A"], it["B"], s, Y=it["Y"], ws=dws),
            "bwd_ms": lambda: L.lora_dropout_bwd(X, it["W"], it["A"], it["B"], s, p, keep, it["dY"], ws=dws),
            "plain_bwd_ms": lambda: L.lora_linear_bwd(X, it["W"], it["A"], it["B"], s, it["dY"], ws=dws,
                                                      out=(it["dX"], it["dA"], it["dB"])),
            # the mask drawn on the device from Philox4x32-10 (seed 3407), again in the backward
            "philox_fwd_ms": lambda: L.lora_dropout_philox_fwd(X, it["W"], it["A"], it["B"], s, p, 3407, 0,
                                                               Y=it["Y"], ws=dws),
            "philox_bwd_ms": lambda: L.lora_dropout_philox_bwd(X, it["W"], it["A"], it["B"], s, p, 3407, it["dY"],
                                                               0, ws=dws)}, reps))
        for key, fl in (("fwd_ms", one_fwd), ("bwd_ms", one_bwd), ("plain_fwd_ms", one_fwd),
                        ("plain_bwd_ms", one_bwd), ("philox_fwd_ms", one_fwd), ("philox_bwd_ms", one_bwd)):
            dr[key.replace("_ms", "_tflops")] = round(fl / (dr[key]["median"] * 1e-3) / 1e12, 1)
        out["dropout"] = dr
        del dws, keep
        Wm = torch.empty_like(it["W"])
        mws = torch.empty(max(L.workspace_bytes(L.OP_MERGE, L.LORA_BF16, 0, k, d, cfg.r), 256),
                          dtype=torch.uint8, device=X.device)
        t = _time_ms(lambda: L.lora_merge(it["W"], it["A"], it["B"], s, out=Wm, ws=mws), reps)
        by = 2.0 * 2 * d * k + 2.0 * cfg.r * (d + k)
        out["merge"] = {"shape": f"W {d}x{k}, r={cfg.r}", "ms": t, "min_bytes": by,
                        "gbps": round(by / (t["median"] * 1e-3) / 1e9, 1),
                        "frac_hbm": round(by / (t["median"] * 1e-3) / 8e12, 3)}
    return out


def small_token_sweep(device, reps=10):
    """Few-token cases, where reading W bounds the layer: the Llama-3-8B q
    projection (4096->4096, r 16, RoPE, bf16) and the Qwen1.5-32B-shaped gate
    projection (5120->27392, r 64, NF4 W), M in {16, 64, 128}.  Each timed call
    follows a 1 GiB read that evicts the 256 MB MALL with clean lines, so W
    comes from HBM and no write-back of a flush's dirty lines competes with
    it.  GB/s = minimum HBM bytes of the call / its HIP-event time."""
    import math

    import torch

    import lora_linear_layers_amd as L
    from synth import gen

    flush = torch.ones(1 << 28, dtype=torch.float32, device=device)
    tab = gen.nf4_table()
    res = {}
    cases = [("q_proj 4096->4096 r16 rope bf16", 4096, 4096, 16, True, False),
             ("gate_proj 5120->27392 r64 nf4", 5120, 27392, 64, False, True)]
    for name, k, d, r, rope, nf4 in cases:
        seed = 9000 + d
        A = gen.to_storage(gen.uniform_sym(seed + 2, r * k, 1.0 / math.sqrt(k), device=device), (r, k), "bf16")
        B = gen.to_storage(gen.normal(seed + 3, d * r, math.sqrt(0.02), device=device), (d, r), "bf16")
        if nf4:
            codes = gen.nf4_random_codes(seed + 1, d * k, device=device)
            absmax = gen.nf4_random_absmax(seed + 4, d * k // 64, 1.0 / math.sqrt(k), device=device)
            wbytes = d * k / 2 + d * k / 64 * 4
        else:
            W = gen.to_storage(gen.normal(seed + 1, d * k, 1.0 / math.sqrt(k), device=device), (d, k), "bf16")
            wbytes = 2.0 * d * k
        cos, sin = L.rope_cache(2048, 128, 500000.0, device=device)
        for M in (16, 64, 128):
            X = gen.to_storage(gen.normal(seed + 5, M * k, 1.0, device=device), (M, k), "bf16")
            dY = gen.to_storage(gen.normal(seed + 6, M * d, 1.0, device=device), (M, d), "bf16")
            pos = torch.from_numpy(gen.positions_mod(M, 2048)).to(device)
            op_f, op_b = (L.OP_NF4_FWD, L.OP_NF4_BWD) if nf4 else \
                ((L.OP_ROPE_FWD, L.OP_ROPE_BWD) if rope else (L.OP_FWD, L.OP_BWD))
            wsb = max(L.workspace_bytes(op, L.LORA_BF16, M, k, d, r) for op in (op_f, op_b))
            ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=device)
            Y = torch.empty(M, d, dtype=torch.bfloat16, device=device)
            outs = (torch.empty(M, k, dtype=torch.bfloat16, device=device),
                    torch.empty(r, k, dtype=torch.float32, device=device),
                    torch.empty(d, r, dtype=torch.float32, device=device))
            if nf4:
                f = lambda: L.nf4_lora_linear_fwd(X, codes, absmax, tab, A, B, 0.25, d, Y=Y, ws=ws)  # noqa: E731
                it = {"X": X, "codes": codes, "absmax": absmax, "A": A, "B": B, "dY": dY}
                b = lambda: _nf4_bwd(L, it, tab, 0.25, ws, outs)  # noqa: E731
            else:
                f = lambda: L.lora_qk_rope_fwd(X, W, A, B, 1.0, pos, cos, sin, Y=Y, ws=ws)  # noqa: E731
                it = {"X": X, "W": W, "A": A, "B": B, "dY": dY}
                w = type("R", (), {"pos": pos, "cos": cos, "sin": sin})
                b = lambda: _rope_bwd(L, it, w, 1.0, ws, outs)  # noqa: E731
            fb = M * k * 2 + wbytes + r * k * 2 + d * r * 2 + M * d * 2
            bb = M * k * 2 + M * d * 2 + wbytes + r * k * 2 + d * r * 2 + M * k * 2 + 4.0 * r * (k + d)
            row = {}
            for kind, fn, by in (("fwd", f, fb), ("bwd", b, bb)):
                fn()
                ts = []
                for i in range(reps):
                    flush.sum()
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record()
                    fn()
                    e1.record()
                    e1.synchronize()
                    ts.append(e0.elapsed_time(e1))
                t = _pct(ts)
                row[kind] = {"ms": t, "min_bytes": by, "gbps": round(by / (t["median"] * 1e-3) / 1e9, 1),
                             "frac_hbm": round(by / (t["median"] * 1e-3) / 8e12, 3)}
            res[f"{name} M={M}"] = row
    del flush
    return res


def nf4_paths(device, reps=10):
    """The two NF4 forward paths on the Qwen1.5-32B MLP shapes (gate
    5120->27392, down 27392->5120, r 64): the whole-tile GEMM expanding the
    codes in its load stage against the one-pass dequantisation followed by
    the bf16 GEMM, timed round-robin, at 512, 2048 and 8192 tokens (the
    library's automatic choice takes the load stage only for 128-255 whole
    tiles)."""
    import math

    import torch

    import lora_linear_layers_amd as L
    from lora_linear_layers_amd import _lib
    from synth import gen

    tab = gen.nf4_table()
    res = {}
    r = 64
    prev = _lib.set_nf4_fwd_path("auto")
    try:
        for name, k, d in (("gate_proj", 5120, 27392), ("down_proj", 27392, 5120)):
            seed = 9500 + d
            codes = gen.nf4_random_codes(seed + 1, d * k, device=device)
            absmax = gen.nf4_random_absmax(seed + 4, d * k // 64, 1.0 / math.sqrt(k), device=device)
            A = gen.to_storage(gen.uniform_sym(seed + 2, r * k, 1.0 / math.sqrt(k), device=device), (r, k), "bf16")
            B = gen.to_storage(gen.normal(seed + 3, d * r, math.sqrt(0.02), device=device), (d, r), "bf16")
            for M in (512, 2048, 8192):
                X = gen.to_storage(gen.normal(seed + 5, M * k, 1.0, device=device), (M, k), "bf16")
                Y = torch.empty(M, d, dtype=torch.bfloat16, device=device)
                ws = {}
                for mode in ("load_stage", "dequant"):
                    _lib.set_nf4_fwd_path(mode)
                    ws[mode] = torch.empty(max(L.workspace_bytes(L.OP_NF4_FWD, L.LORA_BF16, M, k, d, r), 256),
                                           dtype=torch.uint8, device=device)

                def call(mode):
                    _lib.set_nf4_fwd_path(mode)
                    L.nf4_lora_linear_fwd(X, codes, absmax, tab, A, B, 0.25, d, Y=Y, ws=ws[mode])

                t = _time_interleaved({"load_stage_ms": lambda: call("load_stage"),
                                       "dequant_ms": lambda: call("dequant")}, reps)
                fl = 2.0 * M * d * (k + r)
                for key in ("load_stage_ms", "dequant_ms"):
                    t[key.replace("_ms", "_tflops")] = round(fl / (t[key]["median"] * 1e-3) / 1e12, 1)
                t["tiles_256"] = (M // 256) * (d // 256)
                res[f"{name} {k}->{d} M={M}"] = t
                del X, Y, ws
            del codes, absmax
    finally:
        _lib.set_nf4_fwd_path(prev)
    return res


def _rope_bwd(L, it, w, s, ws, out):
    from lora_linear_layers_amd import _lib

    X, W, A, B, dY = it["X"], it["W"], it["A"], it["B"], it["dY"]
    M, d_in = X.shape
    d_out, r = B.shape
    dt = _lib._dtype_code(X)
    dX, dA, dB = out
    _lib._check("lora_qk_rope_bwd", _lib.lib().lora_qk_rope_bwd(
        dt, M, d_in, d_out, r, float(s), _lib._ptr(X), _lib._ptr(W), _lib._ptr(A), _lib._ptr(B), 128,
        _lib._ptr(w.pos), _lib._ptr(w.cos), _lib._ptr(w.sin), w.cos.shape[0], _lib._ptr(dY), _lib._ptr(dX),
        _lib._ptr(dA), _lib._ptr(dB), _lib._ptr(ws), ws.numel(), _lib._stream(X.device)))


def _nf4_bwd(L, it, table, s, ws, out):
    from lora_linear_layers_amd import _lib

    X, A, B, dY = it["X"], it["A"], it["B"], it["dY"]
    M, d_in = X.shape
    d_out, r = B.shape
    dX, dA, dB = out
    tab = _lib._table_ptr(table)
    _lib._check("nf4_lora_linear_bwd", _lib.lib().nf4_lora_linear_bwd(
        M, d_in, d_out, r, float(s), _lib._ptr(X), _lib._ptr(it["codes"]), _lib._ptr(it["absmax"]), 64, tab,
        _lib._ptr(A), _lib._ptr(B), _lib._ptr(dY), _lib._ptr(dX), _lib._ptr(dA), _lib._ptr(dB), _lib._ptr(ws),
        ws.numel(), _lib._stream(X.device)))


def _rocm_version():
    try:
        return open("/opt/rocm/.info/version").read().strip()
    except OSError:
        return None


def _host_cpu():
    """The host's CPU model and how many logical CPUs this process may use."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = None
    return {"cpu_model": model, "nproc": os.cpu_count(), "usable_cpus": usable}


def cpu_baseline(cfg, work, target_s):
    """The float64 oracle, untuned, on the first S tokens of the same workload."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_info

    import oracle as O

    cpu = []
    for it in work.items:
        d = {"p": it["p"], "A": it["A"].cpu(), "B": it["B"].cpu()}
        if cfg.nf4:
            d["codes"], d["absmax"] = it["codes"].cpu().numpy(), it["absmax"].cpu().numpy()
        else:
            d["W"] = it["W"].cpu()
        d["Xf"], d["dYf"] = it["X"], it["dY"]
        cpu.append(d)
    pos_all = work.pos.cpu().numpy() if hasattr(work, "pos") else None

    def run(S):
        t0 = time.perf_counter()
        for d in cpu:
            p = d["p"]
            X, dY = d["Xf"][:S].cpu(), d["dYf"][:S].cpu()
            s = cfg.scale
            if cfg.nf4:
                O.nf4_lora_forward(X, d["codes"], d["absmax"], work.table, d["A"], d["B"], s, p.d_out, p.d_in)
                O.nf4_lora_backward(X, d["codes"], d["absmax"], work.table, d["A"], d["B"], s, dY, p.d_out, p.d_in)
            elif p.rope:
                O.qk_rope_forward(X, d["W"], d["A"], d["B"], s, pos_all[:S])
                O.qk_rope_backward(X, d["W"], d["A"], d["B"], s, pos_all[:S], dY)
            else:
                O.lora_forward(X, d["W"], d["A"], d["B"], s)
                O.lora_backward(X, d["W"], d["A"], d["B"], s, dY)
        return time.perf_counter() - t0

    # a first sample fixes the per-token cost (its fixed part, the weights'
    # widening to float64, makes the estimate conservative); then the largest
    # sample expected to fit the time target, up to the whole workload
    S0 = min(cfg.M, 512)
    t0 = run(S0)
    S = int(min(cfg.M, S0 * target_s / max(t0, 1e-3)))
    S = max(S0, (S // 64) * 64 if S < cfg.M else cfg.M)
    t = run(S) if S != S0 else t0
    # when that sample (or the whole workload) still takes well under the
    # target, repeat it so the measurement is about target_s of CPU work
    passes = 1
    while t < 0.7 * target_s:
        t += run(S)
        passes += 1
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [torch.get_num_threads()])
    flop = cfg.useful_flop(S) * passes
    what = f"the first {S} of {cfg.M} tokens" if S < cfg.M else f"all {cfg.M} tokens"
    what = f"{passes} passes of {what}" if passes > 1 else what
    return {"value": S * passes / t, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "host": _host_cpu(),
            "sample": f"{what} through all {len(cfg.projections)} projections, forward+backward, "
                      f"float64 numpy ({t:.1f} s; {flop / t / 1e9:.1f} GFLOP/s useful)",
            "seconds": round(t, 2), "tflops_equiv": flop / t / 1e12}


def timed_run(work, cfg, steps, warmup, detail=False):
    """W untimed steps, then K timed steps of the whole path.  HIP events (on
    the library's launch stream) bracket only the launches of the kind that
    dominates the step (found in an untimed pre-pass with every launch
    bracketed), so the other launches run without events.  Returns the
    seconds per step and the roofline entry of that kind; with detail, also a
    per-kind breakdown from a few fully bracketed steps after the timed
    region (their events slow them a little; shares are of their own time)."""
    import torch

    from lora_linear_layers_amd import _lib

    for _ in range(warmup):
        work.step()
    torch.cuda.synchronize()
    launches_per_step = 16 * len(cfg.projections)
    _lib.profile_only(None)
    _lib.profile_begin(launches_per_step + 64)
    work.step()
    torch.cuda.synchronize()
    _lib.profile_end()
    dname = max(_lib.profile_report().items(), key=lambda kv: kv[1][0])[0]

    _lib.profile_only(dname)
    _lib.profile_begin(launches_per_step * max(steps, 1) + 64)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        work.step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    _lib.profile_end()
    _lib.profile_only(None)
    dms, dn, dfl, dby = _lib.profile_report()[dname]
    sec = (t1 - t0) / max(steps, 1)

    kpeak = PEAK["f32" if "f32" in dname else "bf16"]
    achieved = dfl / (dms * 1e-3) / 1e12
    # below the ridge point (peak FLOP/s over HBM bytes/s) the kind is HBM-bound
    bound = "mfma" if dfl / max(dby, 1.0) >= kpeak * 1e12 / (HBM_PEAK * 1e9) else "hbm"
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        try:
            tr = json.load(open(TRAFFIC_FILE))
            ent = tr.get("kernels", {}).get(dname)
            if ent and tr.get("kernel_hash") == kernel_hash() and tr.get("config") == cfg.cfg_id:
                traffic = ent["bytes_per_launch"]
        except (ValueError, KeyError):
            traffic = None
    roofline = {"bound": bound, "kernel": dname, "achieved": round(achieved, 1), "peak": kpeak,
                "unit": "TFLOP/s", "frac": round(achieved / kpeak, 4), "traffic": traffic,
                "avg_launch_us": round(1e3 * dms / dn, 1), "flop_per_launch": dfl / dn,
                "algorithmic_bytes_per_launch": dby / dn,
                "achieved_gbps": round(dby / (dms * 1e-3) / 1e9, 1)}
    out = {"sec": sec, "roofline": roofline, "kernels": None, "nb": 0}
    if detail:
        nb = max(1, min(steps, 3))
        _lib.profile_begin(launches_per_step * nb + 64)
        torch.cuda.synchronize()
        tb0 = time.perf_counter()
        for _ in range(nb):
            work.step()
        torch.cuda.synchronize()
        tb1 = time.perf_counter()
        _lib.profile_end()
        kernels = {}
        for name, (ms, n, fl, by) in sorted(_lib.profile_report().items(), key=lambda kv: -kv[1][0]):
            kernels[name] = {"launches": n, "avg_us": round(1e3 * ms / n, 2),
                             "share": round(ms / ((tb1 - tb0) * 1e3), 4),
                             "tflops": round(fl / (ms * 1e-3) / 1e12, 2) if ms > 0 else None,
                             "gbps": round(by / (ms * 1e-3) / 1e9, 1) if ms > 0 else None}
        out["kernels"], out["nb"] = kernels, nb
    return out


def other_configs(args, dev, skip):
    """Every other workload at the same steps and warmup: TFLOP/s, tokens/s
    and the dominant kernel's roofline entry; the fp32 single-layer workload
    (launch-latency bound) also as forward and backward microseconds."""
    import torch

    from synth import CONFIGS

    out = {}
    for cid, cfg in CONFIGS.items():
        if cid == skip:
            continue
        work = Workload(cfg, device=dev)
        res = timed_run(work, cfg, args.steps, args.warmup)
        sec = res["sec"]
        flop = cfg.useful_flop()
        ent = {"workload": cfg.name, "tflops": round(flop / sec / 1e12, 3),
               "tokens_per_s": round(cfg.M / sec, 1), "ms_per_step": round(sec * 1e3, 4),
               "pct_bf16_peak": round(100.0 * flop / sec / 1e12 / PEAK["bf16"], 2),
               "dtype": "f32" if cfg.dtype == "f32" else ("nf4w-bf16" if cfg.nf4 else "bf16"),
               "x_groups": [[it["p"].name for it in grp] for grp in work.groups],
               "roofline": res["roofline"]}
        if cfg.dtype == "f32":
            reps = max(args.steps, 20)
            for kind, fn in (("fwd_us", work.fwd), ("bwd_us", work.bwd)):
                ent[kind] = {k: round(v * 1e3, 2) for k, v in _time_ms(lambda: fn(0), reps).items()}
        out[f"c{cid}"] = ent
        del work
        torch.cuda.empty_cache()
    return out


def without_wt(args, dev, cfg):
    """The workload with the backward transposing each frozen W per call
    instead of reading a caller-held W^T, and the bytes that W^T keeps
    resident."""
    import torch

    work = Workload(cfg, device=dev, keep_wt=False)
    res = timed_run(work, cfg, args.steps, args.warmup)
    sec = res["sec"]
    del work
    torch.cuda.empty_cache()
    wt_bytes = sum(2 * p.d_in * p.d_out for p in cfg.projections)
    return {"tflops": round(cfg.useful_flop() / sec / 1e12, 2), "ms_per_step": round(sec * 1e3, 3),
            "w_t_resident_bytes": wt_bytes}


def main():
    args = parse()
    if args.traffic_from:
        t = traffic_from(args.traffic_from[0], args.traffic_from[1], args.config)
        os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
        with open(TRAFFIC_FILE, "w") as f:
            json.dump(t, f, indent=1)
        print(json.dumps(t))
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}, WORLD_SIZE {world}); "
              "this build has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import torch

    import lora_linear_layers_amd as L
    from lora_linear_layers_amd import _lib
    from synth import CONFIGS

    L.load()
    cfg = CONFIGS[args.config]
    dev = "cuda:0"
    torch.cuda.set_device(0)
    work = Workload(cfg, device=dev, group=not args.no_group, keep_wt=not args.no_wt)

    if args.copy_calibration:
        a = torch.empty(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB
        b = torch.empty_like(a)
        a.fill_(1.0)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    res = timed_run(work, cfg, args.steps, args.warmup, detail=True)
    sec, roofline, kernels, nb = res["sec"], res["roofline"], res["kernels"], res["nb"]
    flop = cfg.useful_flop()
    tflops = flop / sec / 1e12
    tokens = cfg.M / sec
    if roofline["peak"] == PEAK["bf16"]:
        # the dense bf16 rate this chip sustains under its own power limit
        # (MFMA-only probe), as a second reference next to the published peak
        mr = _lib.mfma_rate(device=dev)
        roofline["peak_measured"] = round(mr, 1)
        roofline["frac_of_measured"] = round(roofline["achieved"] / mr, 4)
    calls = per_call_times(work, args.call_reps) if args.call_reps > 0 else None

    out = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "tokens_per_s": round(tokens, 1),
        "pct_bf16_peak": round(100.0 * tflops / PEAK["bf16"], 2),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(sec * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if cfg.dtype == "f32" else ("nf4w-bf16" if cfg.nf4 else "bf16"),
        "data": "synthetic (seeded splitmix64 draws: X,dY~N(0,1), W~N(0,1/d_in), A~U(+-1/sqrt(d_in)), "
                "B~N(0,0.02); NF4 codes uniform)",
        "config": {"workload": cfg.name, "tokens": cfg.M, "batch": cfg.batch, "seq_len": cfg.seq_len,
                   "r": cfg.r, "alpha": cfg.alpha, "nf4_base": cfg.nf4,
                   "projections": [f"{p.name} {p.d_in}->{p.d_out}{' +rope' if p.rope else ''}"
                                   for p in cfg.projections],
                   "x_groups": [[it["p"].name for it in grp] for grp in work.groups],
                   "frozen_w_transposed": (not args.no_wt) and cfg.dtype == "bf16" and not cfg.nf4,
                   "useful_tflop_per_step": round(flop / 1e12, 4), "parallelism": "none (1 GPU)"},
        "roofline": roofline,
        "kernels": kernels,
        "kernels_from": f"{nb} steps after the timed region with every launch bracketed by HIP events",
        "calls": calls,
        "device": torch.cuda.get_device_name(0),
        "rocm": _rocm_version(),
    }
    if not args.no_small_token:
        out["small_token"] = small_token_sweep(dev)
    if args.call_reps > 0:
        out["next_rows"] = next_rows(work, args.call_reps)
        out["nf4_paths"] = nf4_paths(dev, args.call_reps)
    if not args.no_configs:
        if cfg.dtype == "bf16" and not cfg.nf4 and not args.no_wt:
            out["config"]["without_w_t"] = without_wt(args, dev, cfg)
        out["configs"] = other_configs(args, dev, cfg.cfg_id)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, work, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
