"""CPU tests of bench.py's host logic: the flop count, the --gpus guard,
and the rocprofv3 summary (per-kernel durations, HBM bytes scaled by a
copy of known size, MFMA counters) read back only while the kernel
sources are unchanged."""
import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

UPD = "void muon::(anonymous namespace)::ns_gemm_bf16<2>(muon::GemmArgs)"
GRAM = "void muon::(anonymous namespace)::ns_gemm_bf16<0>(muon::GemmArgs)"
COPY = "__amd_rocclr_copyBuffer"


def _write(path, rows, fields):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        w.writerows(rows)


def _counters(d, name, per_kernel):
    rows = []
    for i, (kern, v) in enumerate(per_kernel):
        rows.append({"Dispatch_Id": i, "Kernel_Name": kern, "Counter_Name": name, "Counter_Value": v})
    _write(os.path.join(d, "pmc_counter_collection.csv"), rows,
           ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])


def test_nominal_flops():
    # per NS iteration 4 m^2 n + 2 m^3 with m <= n, either orientation
    assert bench.nominal_ns_flops(1408, 2048, 5) == 5 * (4 * 1408 ** 2 * 2048 + 2 * 1408 ** 3)
    assert bench.nominal_ns_flops(2048, 1408, 5) == bench.nominal_ns_flops(1408, 2048, 5)
    assert bench.nominal_ns_flops(3, 5, 0) == 0


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_summary_scales_counters_and_tracks_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))
    tr, fe, wr, mf = (str(tmp_path / d) for d in ("trace", "fetch", "write", "mfma"))
    _write(os.path.join(tr, "trace_kernel_stats.csv"),
           [{"Name": UPD, "Calls": 4, "TotalDurationNs": 4e6},
            {"Name": GRAM, "Calls": 4, "TotalDurationNs": 2e6},
            {"Name": "some_other_kernel", "Calls": 1, "TotalDurationNs": 9e9}],
           ["Name", "Calls", "TotalDurationNs"])
    # The copy of 1 GiB reads 0.5 GiB of FETCH_SIZE (scale 2) and 1 GiB of
    # WRITE_SIZE (scale 1); two Update dispatches average 1000 KiB fetched.
    _counters(fe, "FETCH_SIZE", [(UPD, 900.0), (UPD, 1100.0), (GRAM, 10.0), (COPY, 524288.0)])
    _counters(wr, "WRITE_SIZE", [(UPD, 300.0), (GRAM, 20.0), (COPY, 1048576.0)])
    _counters(mf, "MfmaFlopsBF16", [(UPD, 2e12), (GRAM, 1e12)])
    with open(os.path.join(mf, "pmc_counter_collection.csv"), "a", newline="") as f:
        csv.writer(f).writerows([[9, UPD, "MfmaUtil", 55.0], [10, GRAM, "MfmaUtil", 45.0]])
    bench.summarize(tr, fe, wr, "w_test", mf)
    out = tmp_path / "profiles" / "ns_update_w_test.md"
    text = out.read_text()
    assert "| ns_update | 4 | 1.0000 | 0.0020 | 0.0003 | 2.0000 | 2000.0 | 55.0 |" in text
    assert "some_other_kernel" not in text
    got = bench.load_traffic("w_test", "ns_update")
    assert got == pytest.approx(1000 * 1024 * 2 + 300 * 1024)
    # A summary taken on other kernel sources is not used.
    monkeypatch.setattr(bench, "source_hash", lambda: "0000000000000000")
    assert bench.load_traffic("w_test", "ns_update") is None


def test_summary_needs_the_calibration_copy(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))
    tr, fe, wr = (str(tmp_path / d) for d in ("trace", "fetch", "write"))
    _write(os.path.join(tr, "trace_kernel_stats.csv"), [{"Name": UPD, "Calls": 1, "TotalDurationNs": 1e6}],
           ["Name", "Calls", "TotalDurationNs"])
    _counters(fe, "FETCH_SIZE", [(UPD, 1.0)])
    _counters(wr, "WRITE_SIZE", [(UPD, 1.0)])
    with pytest.raises(SystemExit):
        bench.summarize(tr, fe, wr, "w_test")


def test_summary_clock_column(tmp_path, monkeypatch):
    # GRBM_GUI_ACTIVE comes summed over the XCDs: 8 XCDs x 1.8e6 busy cycles
    # in a 1 ms dispatch is a 1800 MHz clock; dispatches under 20 us get none.
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))
    tr, fe, wr, ck = (str(tmp_path / d) for d in ("trace", "fetch", "write", "clock"))
    _write(os.path.join(tr, "trace_kernel_stats.csv"),
           [{"Name": UPD, "Calls": 2, "TotalDurationNs": 2e6},
            {"Name": "muon::finalize_kernel(muon::FinalizeArgs)", "Calls": 1, "TotalDurationNs": 4e3}],
           ["Name", "Calls", "TotalDurationNs"])
    _counters(fe, "FETCH_SIZE", [(UPD, 1.0), (COPY, 524288.0)])
    _counters(wr, "WRITE_SIZE", [(UPD, 1.0), (COPY, 1048576.0)])
    fin = "muon::finalize_kernel(muon::FinalizeArgs)"
    _counters(ck, "GRBM_GUI_ACTIVE", [(UPD, 8 * 1.8e6), (UPD, 8 * 1.6e6), (fin, 8 * 50e3)])
    _write(os.path.join(ck, "pmc_kernel_trace.csv"),
           [{"Dispatch_Id": 0, "Start_Timestamp": 0, "End_Timestamp": 1000000},
            {"Dispatch_Id": 1, "Start_Timestamp": 0, "End_Timestamp": 1000000},
            {"Dispatch_Id": 2, "Start_Timestamp": 0, "End_Timestamp": 4000}],
           ["Dispatch_Id", "Start_Timestamp", "End_Timestamp"])
    _write(os.path.join(ck, "pmc_agent_info.csv"), [{"Name": "gfx950", "Num_Xcc": 8}], ["Name", "Num_Xcc"])
    bench.summarize(tr, fe, wr, "w_clk", None, ck)
    e = bench.load_summary("w_clk", "ns_update")
    assert e["clock_mhz"] == pytest.approx(1700.0)
    assert bench.load_summary("w_clk", "norm_finalize")["clock_mhz"] is None
    assert "| clock MHz |" in (tmp_path / "profiles" / "ns_update_w_clk.md").read_text()


def test_executed_mfma_flops_model():
    # 1408 x 2048: 5 full tile rows + a half row; Gram over the lower
    # triangle with 36/64 diagonal tiles, Update over every tile.
    e = bench.executed_mfma_flops(1408, 2048, 1, "square")
    full, wide = 2 * 256 * 256, 2 * 128 * 512
    assert e["ns_update"] == (5 * 8 * full + 4 * wide) * 1408
    assert e["ns_gram"] == pytest.approx((10 * full + 5 * 36 / 64 * full + 3 * wide) * 2048)
    assert bench.executed_mfma_flops(2048, 1408, 1) == e
    # Diagonal tiles take 36 of 64 blocks in every form (the operand tile
    # of the folded and direct forms is read in the diagonal tile too).
    assert bench.executed_mfma_flops(1408, 2048, 1, "direct")["ns_poly"] == pytest.approx(
        (10 * full + 5 * 36 / 64 * full + 3 * wide) * 1408)


def test_f32_executed_flops_model():
    # One 64 x 64 tile: Gram, Poly and Update each execute the nominal
    # 2 m^2 n, 2 m^3 and 2 m^2 n.
    assert bench.f32_executed_flops(64, 64, 5) == bench.nominal_ns_flops(64, 64, 5)
    # 100 x 300 pads to 128 x 320: 3 upper tiles of 64 x 64 for Gram and Poly.
    assert bench.f32_executed_flops(100, 300, 1) == 2 * 3 * 4096 * 320 + 2 * 3 * 4096 * 128 + 2 * 128 * 128 * 320
