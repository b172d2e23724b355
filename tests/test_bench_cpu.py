"""Host logic of bench.py: the one-GPU refusal, the traffic record from counter runs, and the
lookup that reports traffic only for the kernel source the counters were taken on."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

GU_BF16 = "void moe::expert_gemm_kernel<0, 8, 8, 45, 1, 1, 2, 0>(moe::GemmArgs)"
GU_ACT4 = "void moe::expert_gemm_kernel<0, 8, 8, 45, 1, 1, 2, 1>(moe::GemmArgs)"
DOWN = "void moe::expert_gemm_kernel<1, 8, 8, 45, 2, 1, 1, 0>(moe::GemmArgs)"
COPY = "__amd_rocclr_copyBuffer"


def _write_counters(d, counter, rows):
    """rows: (dispatch id, kernel, value); one dispatch may appear in several rows."""
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, n, v in rows:
            w.writerow(dict(Dispatch_Id=i, Kernel_Name=n, Counter_Name=counter, Counter_Value=v))
        w.writerow(dict(Dispatch_Id=99, Kernel_Name=GU_BF16, Counter_Name="OTHER", Counter_Value=1e9))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in json.loads(r.stdout.strip())["error"]


def test_traffic_record_scales_each_counter_by_the_copy_calibration(tmp_path):
    mib = 16
    kib = mib * 1024
    # FETCH_SIZE sees half of a copy's bytes (factor 2), WRITE_SIZE all of them (factor 1);
    # the gate/up dispatch 2 is split over two rows; the act4 dispatch and the down kernel
    # are not the bf16 gate/up kernel; only the last three copies calibrate
    _write_counters(tmp_path / "f", "FETCH_SIZE",
                    [(1, COPY, 123.0), (2, GU_BF16, 600.0), (2, GU_BF16, 400.0), (3, GU_ACT4, 5e6),
                     (4, DOWN, 7e6), (5, GU_BF16, 3000.0), (6, COPY, kib / 2), (7, COPY, kib / 2),
                     (8, COPY, kib / 2)])
    _write_counters(tmp_path / "w", "WRITE_SIZE",
                    [(2, GU_BF16, 10.0), (5, GU_BF16, 30.0), (6, COPY, kib), (7, COPY, kib), (8, COPY, kib)])
    rec = bench.traffic_record(str(tmp_path / "f"), str(tmp_path / "w"), mib, 1, "cmd")
    assert rec["fetch_gate_up_dispatches"] == 2 and rec["write_gate_up_dispatches"] == 2
    assert rec["fetch_copy_scale"] == 2.0 and rec["write_copy_scale"] == 1.0
    assert rec["fetch_bytes_per_launch"] == 2000 * 1024 * 2          # mean of 1000 and 3000 KiB, x 2
    assert rec["write_bytes_per_launch"] == 20 * 1024
    assert rec["hbm_bytes_per_launch"] == 2000 * 1024 * 2 + 20 * 1024
    assert rec["kernel_source_sha256_16"] == bench.gemm_source_hash()
    assert rec["workload"] == bench.workload_name(__import__("synth").CONFIGS[1])


def test_traffic_record_needs_three_calibration_copies(tmp_path):
    _write_counters(tmp_path / "f", "FETCH_SIZE", [(1, GU_BF16, 1.0), (2, COPY, 1.0), (3, COPY, 1.0)])
    _write_counters(tmp_path / "w", "WRITE_SIZE", [(1, GU_BF16, 1.0), (2, COPY, 1.0), (3, COPY, 1.0)])
    with pytest.raises(SystemExit):
        bench.traffic_record(str(tmp_path / "f"), str(tmp_path / "w"), 16, 1)


def test_traffic_is_reported_only_for_the_source_it_was_measured_on(monkeypatch):
    rec = json.load(open(os.path.join(ROOT, "profiles", "gate_up_gemm_traffic.json")))
    monkeypatch.setattr(bench, "gemm_source_hash", lambda: rec["kernel_source_sha256_16"])
    assert bench.traffic_for(rec["workload"]) == rec["hbm_bytes_per_launch"]
    assert bench.traffic_for(rec["workload"] + " (other)") is None
    monkeypatch.setattr(bench, "gemm_source_hash", lambda: "0" * 16)
    assert bench.traffic_for(rec["workload"]) is None


def test_pmc_summary_means_per_dispatch_and_derives_the_matrix_rate(tmp_path):
    d = tmp_path / "p"
    os.makedirs(d)
    with open(d / "run_counter_collection.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        # two dispatches of one kernel; dispatch 1's MOPS split over two rows
        for i, mops, busy in ((1, 1000.0, 2048.0), (2, 3000.0, 4096.0)):
            w.writerow(dict(Dispatch_Id=i, Kernel_Name=GU_BF16, Counter_Name="SQ_INSTS_VALU_MFMA_MOPS_F6F4",
                            Counter_Value=mops / 2))
            w.writerow(dict(Dispatch_Id=i, Kernel_Name=GU_BF16, Counter_Name="SQ_INSTS_VALU_MFMA_MOPS_F6F4",
                            Counter_Value=mops / 2))
            w.writerow(dict(Dispatch_Id=i, Kernel_Name=GU_BF16, Counter_Name="SQ_VALU_MFMA_BUSY_CYCLES",
                            Counter_Value=busy))
    with open(d / "run_kernel_trace.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        w.writerow(dict(Dispatch_Id=1, Kernel_Name=GU_BF16, Start_Timestamp=0, End_Timestamp=1000))
        w.writerow(dict(Dispatch_Id=2, Kernel_Name=GU_BF16, Start_Timestamp=5000, End_Timestamp=8000))
    (r,) = bench.pmc_summary(str(d))
    assert r["dispatches"] == 2
    assert r["counters"]["SQ_INSTS_VALU_MFMA_MOPS_F6F4"] == 2000.0
    assert abs(r["mean_us"] - 2.0) < 1e-9                                  # (1 + 3) us / 2
    assert abs(r["mfma_f6f4_TFLOP_per_s"] - 2000.0 * 512 / 2e-6 * 1e-12) < 1e-9
    assert r["mfma_busy_cycles_per_simd"] == 3072.0 / 1024
