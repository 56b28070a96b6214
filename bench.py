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
matrices/s, the roofline of the dominant kernel (its algorithmic flops or
bytes per launch over its average launch time, both measured with HIP
events recorded around each launch on the library's stream during the
timed steps), its HBM traffic per launch from the committed rocprofv3
counter summary when that summary was taken on the current kernel sources,
and the fp64 oracle timed on a bounded sample on the host cores.

    python bench.py [--steps K --warmup W --workload NAME]
    python bench.py --summarize TRACE_DIR FETCH_DIR WRITE_DIR
        writes profiles/<kernel>_<workload>.md from the rocprofv3 outputs of
        a --kernel-trace --stats run and of --pmc FETCH_SIZE / WRITE_SIZE
        runs (all with --output-format csv), the counter runs made with
        --copy-calib so that each counter can be scaled by what it reads for
        a plain device copy of known size.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
COPY_CALIB_BYTES = 1 << 30  # device-to-device copy used to scale the HBM counters
METRIC = "Batched Newton-Schulz TFLOP/s and Muon matrices/s (bf16, 1 MI355X)"
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_NAMES = {  # rocprofv3 kernel name fragment -> library kernel kind
    "ns_gemm_bf16<0>": "ns_gram", "ns_gemm_bf16<1>": "ns_poly", "ns_gemm_bf16<2>": "ns_update",
    "ns_gemm_f32<0>": "ns_gram", "ns_gemm_f32<1>": "ns_poly", "ns_gemm_f32<2>": "ns_update",
    "momentum_kernel": "momentum", "finalize_kernel": "norm_finalize", "apply_kernel": "apply",
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="moe_bank_2048x1408")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="oracle sample budget (0 = skip)")
    ap.add_argument("--poly-form", default="square", choices=["square", "direct", "folded"],
                    help="bf16 form of the NS polynomial step (muon_options.poly_form)")
    ap.add_argument("--copy-calib", action="store_true",
                    help="also run one plain 1 GiB device copy (for HBM counter scaling)")
    ap.add_argument("--summarize", nargs=3, metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/ summaries from rocprofv3 csv outputs and exit")
    ap.add_argument("--mfma", metavar="MFMA_DIR",
                    help="with --summarize: a --pmc MfmaFlopsBF16 MfmaUtil run, for executed MFMA flops "
                         "and MFMA busy time per kernel")
    ap.add_argument("--f32-ns", metavar="COUNTxMxN",
                    help="side measurement instead of the step: muon_orthogonalize on COUNT float32 "
                         "M x N matrices (the float32 NS path), nominal and executed TFLOP/s")
    ap.add_argument("--clock", metavar="CLOCK_DIR",
                    help="with --summarize: a --pmc GRBM_GUI_ACTIVE --kernel-trace run, for each kernel's "
                         "effective shader clock (GPU-busy cycles over the dispatch's duration)")
    return ap.parse_args()


def source_hash() -> str:
    """Hash of the library's kernel and launch sources (a counter summary
    taken on other sources no longer describes the kernels)."""
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "newton_schulz_10_amd", "csrc", "*"))):
        with open(p, "rb") as f:
            h.update(os.path.basename(p).encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def nominal_ns_flops(rows: int, cols: int, ns_steps: int) -> int:
    """Nominal NS flops of one matrix: per iteration X X^T (2 m^2 n), A A
    (2 m^3) and B X (2 m^2 n), with m <= n after the transpose-first rule."""
    m, n = min(rows, cols), max(rows, cols)
    return ns_steps * (4 * m * m * n + 2 * m ** 3)


def executed_mfma_flops(rows: int, cols: int, ns_steps: int, poly_form: str = "square") -> dict:
    """bf16 MFMA flops the GEMM kernels execute for one matrix, per kernel
    kind, from their tile geometry: m padded to 128 and n to 256 (m <= n);
    256 x 256 tiles, plus 128 x 512 tiles over the half tile row when m_pad
    is an odd multiple of 128; Gram and Poly over the lower triangle of
    tiles, diagonal tiles multiplying 36 of their 64 blocks of 32 x 32 (in
    every form); Update over every tile of X'. The form does not change
    the MFMA work (poly_form is kept for callers)."""
    m, n = min(rows, cols), max(rows, cols)
    mp, np_ = -(-m // 128) * 128, -(-n // 256) * 256
    F, half = mp // 256, mp % 256 != 0
    full_tile, wide_tile = 2 * 256 * 256, 2 * 128 * 512   # flops per unit K
    ts = F + half
    wide_sym = (ts + 1) // 2 if half else 0
    tu = np_ // 256
    wide_upd = (tu + 1) // 2 if half else 0

    def sym(K, diag_frac):
        return (F * (F - 1) // 2 * full_tile + F * diag_frac * full_tile + wide_sym * wide_tile) * K

    gram = sym(np_, 36 / 64)
    poly = sym(mp, 36 / 64)
    upd = (F * tu * full_tile + wide_upd * wide_tile) * mp
    return {"ns_gram": ns_steps * gram, "ns_poly": ns_steps * poly, "ns_update": ns_steps * upd}


class ClockSampler:
    """Samples the GPU's GFX clock (MHz) and socket power (W) from the host
    with amdsmi in a background thread; summary() gives their means over the
    samples taken between start() and stop()."""

    def __init__(self, period_s: float = 0.01):
        self.period = period_s
        self.samples = []
        self.error = None
        self._stop = None
        self._thread = None
        self._h = None
        try:
            import amdsmi
            self._smi = amdsmi
            amdsmi.amdsmi_init()
            handles = amdsmi.amdsmi_get_processor_handles()
            self._h = handles[0] if handles else None
            try:
                import torch
                bus = torch.cuda.get_device_properties(0).pci_bus_id
                for h in handles:
                    if int(amdsmi.amdsmi_get_gpu_device_bdf(h).split(":")[1], 16) == bus:
                        self._h = h
            except Exception:  # pragma: no cover
                pass
        except Exception as e:  # pragma: no cover
            self.error = f"{type(e).__name__}: {e}"

    def _read(self):
        """(GFX clock MHz, socket power W) from the GPU metrics table: the
        mean of the per-XCD current gfx clocks (else the averaged gfx clock),
        and the current socket power (else the averaged one)."""
        smi = self._smi
        m = smi.amdsmi_get_gpu_metrics_info(self._h)

        def num(v):
            return float(v) if isinstance(v, (int, float)) and 0 < v < 65535 else None

        clks = [num(v) for v in (m.get("current_gfxclks") or []) if num(v)]
        clk = sum(clks) / len(clks) if clks else num(m.get("average_gfxclk_frequency"))
        w = num(m.get("current_socket_power")) or num(m.get("average_socket_power"))
        if clk is None:
            raise RuntimeError("no gfx clock in the GPU metrics table")
        return clk, w

    def start(self):
        import threading
        if self._h is None:
            return
        self._stop = threading.Event()

        def loop():
            while not self._stop.is_set():
                try:
                    self.samples.append(self._read())
                except Exception as e:  # pragma: no cover
                    self.error = f"{type(e).__name__}: {e}"
                    return
                self._stop.wait(self.period)

        self._thread = threading.Thread(target=loop, daemon=True)
        self._thread.start()

    def stop(self):
        if self._thread is not None:
            self._stop.set()
            self._thread.join()

    def summary(self):
        if not self.samples:
            return {"sclk_mhz": None, "samples": 0, "error": self.error}
        clk = [c for c, _ in self.samples]
        pw = [p for _, p in self.samples if p is not None]
        out = {"sclk_mhz_mean": sum(clk) / len(clk), "sclk_mhz_min": min(clk), "sclk_mhz_max": max(clk),
               "samples": len(clk),
               "source": "amdsmi GPU metrics (mean of the per-XCD current gfx clocks), sampled every 10 ms "
                         "during the timed steps; the kernels' own mean clock is in roofline.clock_mhz_profiled"}
        if pw:
            out["socket_power_w_mean"] = sum(pw) / len(pw)
        return out


def kernel_kind(name: str):
    for frag, kind in KERNEL_NAMES.items():
        if frag in name:
            return kind
    return None


# --------------------------------------------------------------------------
# rocprofv3 output -> profiles/ summary
# --------------------------------------------------------------------------

def _read_csvs(d: str, suffix: str):
    rows = []
    for p in sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True)):
        with open(p, newline="") as f:
            rows.extend(csv.DictReader(f))
    if not rows:
        raise SystemExit(f"no *{suffix} under {d}")
    return rows


def _counter_per_kind(rows, counter):
    """Mean counter value per dispatch for each library kernel kind, plus
    the value read for the calibration copy."""
    per_dispatch = {}
    for r in rows:
        if r["Counter_Name"] != counter:
            continue
        key = (r["Dispatch_Id"], r["Kernel_Name"])
        per_dispatch[key] = per_dispatch.get(key, 0.0) + float(r["Counter_Value"])
    kinds, copy = {}, None
    for (_, name), v in per_dispatch.items():
        k = kernel_kind(name)
        if k:
            kinds.setdefault(k, []).append(v)
        elif "copyBuffer" in name or "copy_kernel" in name:
            copy = v if copy is None else max(copy, v)
    return {k: sum(v) / len(v) for k, v in kinds.items()}, copy


def _clock_per_kind(d):
    """Effective shader clock (MHz) per kernel kind: GRBM_GUI_ACTIVE (GPU-busy
    cycles, summed by the tool over the XCDs) / XCD count / dispatch time."""
    rows = _read_csvs(d, "counter_collection.csv")
    trace = {r["Dispatch_Id"]: int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
             for r in _read_csvs(d, "kernel_trace.csv")}
    xcc = 1
    for r in _read_csvs(d, "agent_info.csv"):
        if r.get("Name", "").startswith("gfx") and int(r.get("Num_Xcc") or 0) > 0:
            xcc = int(r["Num_Xcc"])
    cyc, ns = {}, {}
    for r in rows:
        if r["Counter_Name"] != "GRBM_GUI_ACTIVE" or r["Dispatch_Id"] not in trace:
            continue
        k = kernel_kind(r["Kernel_Name"])
        if not k:
            continue
        cyc[k] = cyc.get(k, 0.0) + float(r["Counter_Value"]) / xcc
        ns[k] = ns.get(k, 0.0) + trace[r["Dispatch_Id"]]
    # Dispatches shorter than about 20 us are dominated by the counter's
    # start/stop granularity: no clock for those kinds.
    n = {}
    for r in rows:
        if r["Counter_Name"] == "GRBM_GUI_ACTIVE" and r["Dispatch_Id"] in trace and kernel_kind(r["Kernel_Name"]):
            k = kernel_kind(r["Kernel_Name"])
            n[k] = n.get(k, 0) + 1
    return {k: cyc[k] / ns[k] * 1e3 for k in cyc if ns.get(k) and ns[k] / n[k] >= 20e3}


def summarize(trace_dir, fetch_dir, write_dir, workload, mfma_dir=None, clock_dir=None):
    stats = _read_csvs(trace_dir, "kernel_stats.csv")
    clock = _clock_per_kind(clock_dir) if clock_dir else {}
    mflops, mutil = {}, {}
    if mfma_dir:
        rows = _read_csvs(mfma_dir, "counter_collection.csv")
        mflops, _ = _counter_per_kind(rows, "MfmaFlopsBF16")
        mutil, _ = _counter_per_kind(rows, "MfmaUtil")
    fetch, fcopy = _counter_per_kind(_read_csvs(fetch_dir, "counter_collection.csv"), "FETCH_SIZE")
    write, wcopy = _counter_per_kind(_read_csvs(write_dir, "counter_collection.csv"), "WRITE_SIZE")
    if not fcopy or not wcopy:
        raise SystemExit("calibration copy not found in the counter runs (run them with --copy-calib)")
    f_scale = COPY_CALIB_BYTES / (fcopy * 1024.0)
    w_scale = COPY_CALIB_BYTES / (wcopy * 1024.0)
    kinds = {}
    for r in stats:
        k = kernel_kind(r["Name"])
        if not k:
            continue
        e = kinds.setdefault(k, {"calls": 0, "total_ns": 0.0})
        e["calls"] += int(r["Calls"])
        e["total_ns"] += float(r["TotalDurationNs"])
    for k, e in kinds.items():
        e["avg_ms"] = e["total_ns"] / e["calls"] / 1e6
        e["hbm_read_bytes_per_launch"] = fetch.get(k, 0.0) * 1024.0 * f_scale if k in fetch else None
        e["hbm_write_bytes_per_launch"] = write.get(k, 0.0) * 1024.0 * w_scale if k in write else None
        if mfma_dir:
            e["mfma_bf16_flops_per_launch"] = mflops.get(k)
            e["mfma_busy_pct"] = mutil.get(k)
        if clock_dir:
            e["clock_mhz"] = clock.get(k)
    dom = max(kinds, key=lambda k: kinds[k]["total_ns"])
    data = {"workload": workload, "source_sha256": source_hash(),
            "calibration": {"copy_bytes": COPY_CALIB_BYTES, "fetch_kib_read": fcopy, "write_kib_read": wcopy,
                            "fetch_scale": f_scale, "write_scale": w_scale},
            "dominant": dom, "kernels": kinds}
    os.makedirs(PROFILES, exist_ok=True)
    out = os.path.join(PROFILES, f"{dom}_{workload}.md")
    with open(out, "w") as f:
        f.write(f"# rocprofv3 summary: {dom} on {workload}\n\n")
        f.write("Commands on the GPU host ($REPO = repository root):\n\n")
        f.write("```\ncd /tmp && export TMPDIR=/tmp\n")
        f.write(f"rocprofv3 --kernel-trace --stats --output-format csv -d <TRACE_DIR> -o trace -- "
                f"python3 $REPO/bench.py --workload {workload} --steps 3 --warmup 1 --cpu-seconds 0\n")
        for c, d in (("FETCH_SIZE", "<FETCH_DIR>"), ("WRITE_SIZE", "<WRITE_DIR>")):
            f.write(f"rocprofv3 --pmc {c} --output-format csv -d {d} -o pmc -- "
                    f"python3 $REPO/bench.py --workload {workload} --steps 1 --warmup 0 --cpu-seconds 0 --copy-calib\n")
        extra = ""
        if mfma_dir:
            f.write(f"rocprofv3 --pmc MfmaFlopsBF16 MfmaUtil --output-format csv -d <MFMA_DIR> -o pmc -- "
                    f"python3 $REPO/bench.py --workload {workload} --steps 1 --warmup 0 --cpu-seconds 0\n")
            extra += " --mfma <MFMA_DIR>"
        if clock_dir:
            f.write(f"rocprofv3 --pmc GRBM_GUI_ACTIVE --kernel-trace --output-format csv -d <CLOCK_DIR> -o pmc -- "
                    f"python3 $REPO/bench.py --workload {workload} --steps 1 --warmup 1 --cpu-seconds 0\n")
            extra += " --clock <CLOCK_DIR>"
        f.write(f"python3 $REPO/bench.py --summarize <TRACE_DIR> <FETCH_DIR> <WRITE_DIR>{extra} "
                f"--workload {workload}\n```\n\n")
        f.write(f"Counter scale: a {COPY_CALIB_BYTES >> 20} MiB device copy reads FETCH_SIZE {fcopy:.0f} KiB "
                f"(x{f_scale:.3f}) and WRITE_SIZE {wcopy:.0f} KiB (x{w_scale:.3f}).\n\n")
        if mfma_dir:
            f.write("MFMA columns: executed bf16 MFMA flops per launch (MfmaFlopsBF16, the MFMA op counter x 512), "
                    "the same over the launch's average duration, and MFMA busy time over GPU-active time "
                    "summed over all SIMDs (MfmaUtil).\n\n")
        if clock_dir:
            f.write("Clock column: GPU-busy cycles (GRBM_GUI_ACTIVE, summed over the XCDs by the tool, divided by "
                    "their number) over each dispatch's duration, i.e. the mean shader clock while the kernel "
                    "ran.\n\n")
        head = "| kernel | launches | avg ms | HBM read GB/launch | HBM write GB/launch |"
        rule = "|---|---|---|---|---|"
        if mfma_dir:
            head += " executed MFMA TFLOP/launch | executed TFLOP/s | MFMA busy % |"
            rule += "---|---|---|"
        if clock_dir:
            head += " clock MHz |"
            rule += "---|"
        f.write(head + "\n" + rule + "\n")
        for k, e in sorted(kinds.items(), key=lambda kv: -kv[1]["total_ns"]):
            rd = e["hbm_read_bytes_per_launch"]
            wr = e["hbm_write_bytes_per_launch"]
            line = (f"| {k} | {e['calls']} | {e['avg_ms']:.4f} | "
                    f"{'-' if rd is None else f'{rd / 1e9:.4f}'} | {'-' if wr is None else f'{wr / 1e9:.4f}'} |")
            if mfma_dir:
                fl, ut = e.get("mfma_bf16_flops_per_launch"), e.get("mfma_busy_pct")
                rate = fl / (e["avg_ms"] * 1e-3) / 1e12 if fl else None
                line += (f" {'-' if not fl else f'{fl / 1e12:.4f}'} |"
                         f" {'-' if rate is None else f'{rate:.1f}'} |"
                         f" {'-' if ut is None else f'{ut:.1f}'} |")
            if clock_dir:
                ck = e.get("clock_mhz")
                line += f" {'-' if ck is None else f'{ck:.0f}'} |"
            f.write(line + "\n")
        f.write("\nMachine-readable copy (bench.py reads it while `source_sha256` matches the sources):\n\n")
        f.write("```json\n" + json.dumps(data, indent=1) + "\n```\n")
    print(out)


def load_summary(workload, kind):
    """The committed rocprofv3 summary's entry for kernel `kind`, or None
    when there is none or it was taken on other kernel sources."""
    for p in glob.glob(os.path.join(PROFILES, f"*_{workload}.md")):
        with open(p) as f:
            m = re.search(r"```json\n(.*?)\n```", f.read(), re.S)
        if not m:
            continue
        data = json.loads(m.group(1))
        if data.get("source_sha256") != source_hash():
            continue
        e = data["kernels"].get(kind)
        if e:
            return e
    return None


def load_traffic(workload, kind):
    """HBM bytes per launch of `kind` from the committed summary, or None
    when there is none or it was taken on other kernel sources."""
    e = load_summary(workload, kind)
    if e and e.get("hbm_read_bytes_per_launch") is not None and e.get("hbm_write_bytes_per_launch") is not None:
        return e["hbm_read_bytes_per_launch"] + e["hbm_write_bytes_per_launch"]
    return None


def environment():
    """Versions and hardware the numbers were taken on."""
    import torch
    env = {"torch": torch.__version__, "hip": getattr(torch.version, "hip", None)}
    try:
        p = torch.cuda.get_device_properties(0)
        env["gpu"] = p.name
        env["gcn_arch"] = getattr(p, "gcnArchName", None)
        env["compute_units"] = p.multi_processor_count
    except Exception:  # pragma: no cover
        pass
    try:
        with open("/proc/cpuinfo") as f:
            info = {}
            for line in f:
                if ":" in line:
                    k, v = line.split(":", 1)
                    info.setdefault(k.strip(), v.strip())
        env["cpu"] = info.get("model name")
        env["cpu_family_model_stepping"] = "/".join(str(info.get(k)) for k in ("cpu family", "model", "stepping"))
        env["host_cores_visible"] = len(os.sched_getaffinity(0))
    except OSError:  # pragma: no cover
        pass
    try:
        from threadpoolctl import threadpool_info
        env["blas"] = [{k: i.get(k) for k in ("internal_api", "version", "num_threads", "architecture")}
                       for i in threadpool_info() if i.get("user_api") == "blas"]
    except Exception as e:  # pragma: no cover
        env["blas"] = f"unknown ({type(e).__name__})"
    return env


# --------------------------------------------------------------------------
# benchmark
# --------------------------------------------------------------------------

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
        flops += nominal_ns_flops(r, c, w.ns_steps)
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    return {"value": flops / el / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "matrices_per_s": done / el,
            "sample": f"{done} of {len(mats)} matrices (idle experts skipped, groups interleaved), "
                      f"fp64 numpy, {el:.1f} s"}


def f32_executed_flops(m: int, n: int, ns_steps: int) -> float:
    """MFMA flops the float32 kernels execute per matrix: 64 x 64 tiles over
    the padded shape, Gram and Poly on the upper tiles (diagonal tiles
    whole)."""
    mp, np_ = -(-m // 64) * 64, -(-n // 64) * 64
    t = mp // 64
    sym = t * (t + 1) // 2 * 64 * 64
    return ns_steps * (2.0 * sym * np_ + 2.0 * sym * mp + 2.0 * mp * mp * np_)


def f32_ns(args, torch, nsa) -> None:
    """The float32 NS path (muon_orthogonalize) on synthetic N(0, 1)
    matrices: one JSON line. A side figure, not the step's metric."""
    cnt, m, n = (int(v) for v in args.f32_ns.lower().split("x"))
    gen = torch.Generator(device="cuda").manual_seed(0)
    X = [torch.randn(m, n, device="cuda", generator=gen) for _ in range(cnt)]
    O = [torch.empty_like(x) for x in X]
    for _ in range(args.warmup):
        nsa.muon_orthogonalize(X, O)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        nsa.muon_orthogonalize(X, O)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    lo, hi = min(m, n), max(m, n)
    nominal = cnt * float(nominal_ns_flops(lo, hi, 5))
    executed = cnt * f32_executed_flops(lo, hi, 5)
    print(json.dumps({"metric": "float32 NS TFLOP/s (muon_orthogonalize)", "value": nominal / ms / 1e9,
                      "unit": "TFLOP/s", "executed_tflops": executed / ms / 1e9,
                      "frac_of_fp32_peak_executed": executed / ms / 1e9 / 157.3, "ms_per_call": ms,
                      "config": {"workload": f"{cnt} x {m}x{n} float32", "ns_steps": 5},
                      "steps": args.steps, "warmup": args.warmup, "dtype": "f32", "data": "synthetic"}))


def main():
    args = parse()
    if args.summarize:
        summarize(*args.summarize, args.workload, args.mfma, args.clock)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported (the library runs on "
              f"one device; sharding across GPUs is not built).", file=sys.stderr)
        sys.exit(2)
    import torch
    import newton_schulz_10_amd as nsa
    import workloads

    nsa.load()
    if args.f32_ns:
        f32_ns(args, torch, nsa)
        return
    w = workloads.WORKLOADS[args.workload]
    banks = make_inputs(w)
    mats_per_step = w.num_matrices
    flops_per_step = float(sum(nominal_ns_flops(r, c, w.ns_steps) for _, _, r, c in w.matrices()))
    # Idle experts (zero gradients) have an exactly-zero update: the library
    # finds them on the device and skips their GEMM tiles. The headline value
    # keeps the workload's nominal flops; the roofline and the *_live rate
    # count only the matrices that are computed (idle ones are spread evenly
    # over the batches, so every launch carries the same live share).
    idle = sum(1 for gi, j, _, _ in w.matrices() if w.is_idle(gi, j))
    live_flops_per_step = float(sum(nominal_ns_flops(r, c, w.ns_steps)
                                    for gi, j, r, c in w.matrices() if not w.is_idle(gi, j)))
    live_frac = live_flops_per_step / flops_per_step if flops_per_step else 1.0

    def step():
        nsa.muon_step(banks, w.lr, w.beta, w.ns_steps, poly_form=args.poly_form)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # Timed region (the headline): exactly K steps, uninstrumented.
    nsa.profile_enable(False)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    clock = ClockSampler()
    torch.cuda.synchronize()
    clock.start()
    t0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    clock.stop()
    ms = e0.elapsed_time(e1) / args.steps
    # Profiled region: K more steps in which the library records a HIP
    # event pair around each of its launches on its own stream, giving the
    # per-kernel times and the roofline's launch durations. The event
    # records cost about 1% of a step, so they stay out of the headline.
    nsa.profile_enable(True)
    nsa.profile_read(reset=True)
    p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    p0.record()
    for _ in range(args.steps):
        step()
    p1.record()
    torch.cuda.synchronize()
    profiled_ms = p0.elapsed_time(p1) / args.steps
    kinds = nsa.profile_read(reset=True)
    nsa.profile_enable(False)

    per_kernel = {k: {"launches": v["launches"], "avg_ms": v["total_ms"] / max(1, v["launches"]),
                      "total_ms_per_step": v["total_ms"] / args.steps,
                      "tflops": (v["flops"] / (v["total_ms"] * 1e-3) / 1e12) if v["flops"] and v["total_ms"] else None,
                      "gbs": (v["bytes"] / (v["total_ms"] * 1e-3) / 1e9) if v["bytes"] and v["total_ms"] else None}
                  for k, v in kinds.items()}
    dom = max(kinds, key=lambda k: kinds[k]["total_ms"])
    dv = kinds[dom]
    avg_launch_ms = dv["total_ms"] / dv["launches"]
    traffic = load_traffic(w.key, dom)
    if dv["flops"]:
        live_flops = dv["flops"] * live_frac
        achieved = live_flops / (dv["total_ms"] * 1e-3) / 1e12
        peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
        roof = {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s", "frac": achieved / peak,
                "traffic": traffic, "kernel": dom, "flops_per_launch": live_flops / dv["launches"],
                "flops_counted": "live matrices (idle experts excluded)",
                "avg_launch_ms": avg_launch_ms}
        summ = load_summary(w.key, dom)
        if summ and summ.get("mfma_bf16_flops_per_launch"):
            # From the committed counter run on the same sources: executed
            # MFMA flops per launch and MFMA busy time (rocprofv3).
            roof["executed_mfma_tflop_per_launch"] = summ["mfma_bf16_flops_per_launch"] / 1e12
            roof["mfma_busy_pct"] = summ.get("mfma_busy_pct")
        if summ and summ.get("clock_mhz"):
            # The kernel's mean shader clock in the committed counter run, and
            # the bf16 peak at that clock (the spec peak assumes 2.4 GHz).
            roof["clock_mhz_profiled"] = summ["clock_mhz"]
            roof["frac_of_peak_at_clock"] = achieved / (peak * summ["clock_mhz"] / 2400.0)
    else:
        achieved = dv["bytes"] / (dv["total_ms"] * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS, "traffic": traffic, "kernel": dom,
                "bytes_per_launch": dv["bytes"] / dv["launches"], "avg_launch_ms": avg_launch_ms}
    gemm_ms = sum(v["total_ms"] for k, v in kinds.items() if k.startswith("ns_")) / args.steps
    # Executed MFMA work of the GEMM kernels (live matrices only: idle ones
    # are not computed) beside the nominal rate.
    exe = {}
    if w.dtype == "bf16":
        for gi, j, r, c in w.matrices():
            if not w.is_idle(gi, j):
                for k, v in executed_mfma_flops(r, c, w.ns_steps, args.poly_form).items():
                    exe[k] = exe.get(k, 0.0) + v
    for k, v in exe.items():
        if k in per_kernel and per_kernel[k]["total_ms_per_step"]:
            rate = v / (per_kernel[k]["total_ms_per_step"] * 1e-3) / 1e12
            per_kernel[k]["executed_tflops"] = rate
            per_kernel[k]["executed_frac_of_peak"] = rate / PEAK_BF16_TFLOPS
    exe_total = sum(exe.values())

    if args.copy_calib:
        a = torch.empty(COPY_CALIB_BYTES // 4, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    cpu = cpu_baseline(w, args.cpu_seconds) if args.cpu_seconds > 0 else None
    value = flops_per_step / (ms * 1e-3) / 1e12
    peak_step = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "matrices_per_s": mats_per_step / (ms * 1e-3),
        "frac_of_peak": value / peak_step,
        "ns_gemm_tflops": flops_per_step / (gemm_ms * 1e-3) / 1e12 if gemm_ms else None,
        "ns_gemm_tflops_live": live_flops_per_step / (gemm_ms * 1e-3) / 1e12 if gemm_ms else None,
        "ns_gemm_executed_tflops": exe_total / (gemm_ms * 1e-3) / 1e12 if gemm_ms and exe_total else None,
        "ns_gemm_executed_frac_of_peak": (exe_total / (gemm_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS
                                          if gemm_ms and exe_total else None),
        "poly_form": args.poly_form,
        "idle_matrices": idle,
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "wall_ms_per_step": wall_ms, "profiled_ms_per_step": profiled_ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.key, "description": w.description, "matrices": mats_per_step,
                   "ns_steps": w.ns_steps, "nominal_ns_flops_per_step": flops_per_step,
                   "groups": [[g.rows, g.cols, g.count] for g in w.groups]},
        "roofline": roof,
        "kernels": per_kernel,
        "cpu_baseline": cpu,
        "env": dict(environment(), clock=clock.summary()),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
