#!/usr/bin/env python3
"""Benchmark of the batched Muon step on one MI355X.

One step = one muon_step call over the whole workload: momentum + Nesterov,
Frobenius normalisation, 5 quintic Newton-Schulz iterations and the update
apply, for every matrix. Inputs are seeded synthetic gradients already
resident in HBM when the timed region starts.

Default workload: the MoE expert bank, 256 experts each owning a 2048x1408
and a 1408x2048 bf16 matrix (512 matrices, grads N(0, 1e-3), 10% of
experts idle with zero gradients), momentum and params zero-initialised.

Prints one JSON line: metric, value (nominal NS TFLOP/s of the whole step),
matrices/s, the roofline of the dominant kernel measured with HIP events
around its launches, and the fp64 oracle timed on a bounded sample on the
host cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="moe_bank_2048x1408")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="oracle sample budget (0 = skip)")
    ap.add_argument("--profile-steps", type=int, default=2, help="steps timed per kernel with HIP events")
    ap.add_argument("--copy-calib", action="store_true",
                    help="also run one plain device copy of known size (for HBM counter scaling)")
    return ap.parse_args()


def make_inputs(w):
    """Device tensors, grouped as [E, rows, cols] banks per shape group."""
    import numpy as np
    import torch
    import workloads
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    banks = []
    for gi, g in enumerate(w.groups):
        G = torch.empty((g.count, g.rows, g.cols), dtype=dt, device="cuda")
        chunk = max(1, min(g.count, (1 << 28) // (g.rows * g.cols)))
        for s in range(0, g.count, chunk):
            idx = list(range(s, min(g.count, s + chunk)))
            sts = workloads.parallel_map(lambda j: workloads.grad(w, gi, j), idx)
            for j, st in zip(idx, sts):
                if w.dtype == "bf16":
                    G[j].copy_(torch.from_numpy(st.bits.view(np.int16)).view(torch.bfloat16))
                else:
                    G[j].copy_(torch.from_numpy(st.values))
        P = torch.zeros((g.count, g.rows, g.cols), dtype=dt, device="cuda")
        M = torch.zeros((g.count, g.rows, g.cols), dtype=torch.float32, device="cuda")
        banks.append((P, G, M))
    torch.cuda.synchronize()
    return banks


def cpu_baseline(w, budget_s):
    """fp64 oracle on a bounded sample of the workload's matrices."""
    import numpy as np
    import oracle
    import workloads
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas"] or [0])
    except Exception:  # pragma: no cover
        cores = 0
    if not cores:
        cores = len(os.sched_getaffinity(0))
    mats = w.matrices()
    # interleave the groups so the sample covers every shape
    order = []
    per = [[k for k, m in enumerate(mats) if m[0] == gi and not w.is_idle(gi, m[1])] for gi in range(len(w.groups))]
    while any(per):
        for lst in per:
            if lst:
                order.append(lst.pop(0))
    done, flops = 0, 0.0
    t0 = time.perf_counter()
    for k in order:
        gi, j, r, c = mats[k]
        g = workloads.grad(w, gi, j).as_f64()
        b = workloads.momentum(w, gi, j).astype(np.float64)
        p = workloads.params(w, gi, j).as_f64()
        oracle.muon_matrix_step(p, g, b, w.lr, w.beta, w.ns_steps)
        done += 1
        flops += oracle.nominal_ns_flops(r, c, w.ns_steps)
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    return {"value": flops / el / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "matrices_per_s": done / el,
            "sample": f"{done} of {len(mats)} matrices (idle experts skipped, groups interleaved), "
                      f"fp64 numpy, {el:.1f} s"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported (the library runs "
              f"on one device; see DESIGN.md for how the path would shard).", file=sys.stderr)
        sys.exit(2)
    import torch
    import newton_schulz_10_amd as nsa
    import oracle  # only for the nominal flop count and the CPU baseline leg
    import workloads

    nsa.load()
    w = workloads.WORKLOADS[args.workload]
    banks = make_inputs(w)
    mats_per_step = w.num_matrices
    flops_per_step = float(sum(oracle.nominal_ns_flops(r, c, w.ns_steps) for _, _, r, c in w.matrices()))

    def step():
        nsa.muon_step(banks, w.lr, w.beta, w.ns_steps)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    ms = e0.elapsed_time(e1) / args.steps

    # Per-kernel times with HIP events recorded on the library's stream.
    nsa.profile_enable(True)
    nsa.profile_read(reset=True)
    for _ in range(args.profile_steps):
        step()
    kinds = nsa.profile_read(reset=True)
    nsa.profile_enable(False)
    per_kernel = {k: {"launches": v["launches"], "avg_ms": v["total_ms"] / max(1, v["launches"]),
                      "total_ms_per_step": v["total_ms"] / args.profile_steps,
                      "tflops": (v["flops"] / (v["total_ms"] * 1e-3) / 1e12) if v["flops"] and v["total_ms"] else None,
                      "gbs": (v["bytes"] / (v["total_ms"] * 1e-3) / 1e9) if v["bytes"] and v["total_ms"] else None}
                  for k, v in kinds.items()}
    dom = max(kinds, key=lambda k: kinds[k]["total_ms"])
    dv = kinds[dom]
    if dv["flops"]:
        achieved = dv["flops"] / (dv["total_ms"] * 1e-3) / 1e12
        peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
        roof = {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s", "frac": achieved / peak,
                "traffic": None, "kernel": dom, "flops_per_launch": dv["flops"] / dv["launches"],
                "avg_launch_ms": dv["total_ms"] / dv["launches"]}
    else:
        achieved = dv["bytes"] / (dv["total_ms"] * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS, "traffic": None, "kernel": dom,
                "bytes_per_launch": dv["bytes"] / dv["launches"], "avg_launch_ms": dv["total_ms"] / dv["launches"]}
    gemm_ms = sum(v["total_ms"] for k, v in kinds.items() if k.startswith("ns_")) / args.profile_steps

    if args.copy_calib:
        a = torch.empty(1 << 28, dtype=torch.float32, device="cuda")  # 1 GiB
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()

    cpu = cpu_baseline(w, args.cpu_seconds) if args.cpu_seconds > 0 else None
    value = flops_per_step / (ms * 1e-3) / 1e12
    out = {
        "metric": "Batched Newton-Schulz TFLOP/s and Muon matrices/s (bf16, 1 MI355X)",
        "value": value,
        "unit": "TFLOP/s",
        "matrices_per_s": mats_per_step / (ms * 1e-3),
        "frac_of_peak": value / (PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS),
        "ns_gemm_tflops": flops_per_step / (gemm_ms * 1e-3) / 1e12 if gemm_ms else None,
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "wall_ms_per_step": wall_ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.key, "description": w.description, "matrices": mats_per_step,
                   "ns_steps": w.ns_steps, "nominal_ns_flops_per_step": flops_per_step,
                   "groups": [[g.rows, g.cols, g.count] for g in w.groups]},
        "roofline": roof,
        "kernels": per_kernel,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
