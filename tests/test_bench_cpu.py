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
PF_BF16 = "void moe::expert_gemm_prefill_kernel<0, 45, 2, 4, 0>(moe::PrefillArgs)"
PF_ACT4 = "void moe::expert_gemm_prefill_kernel<0, 45, 2, 4, 1>(moe::PrefillArgs)"
PF_DOWN = "void moe::expert_gemm_prefill_kernel<1, 45, 2, 4, 0>(moe::PrefillArgs)"
PF_DOWN_ACT4 = "void moe::expert_gemm_prefill_kernel<1, 45, 2, 4, 1>(moe::PrefillArgs)"
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
    assert rec["kernel_source_sha256_16"] == bench.gemm_source_hash("decode")
    assert rec["workload"] == bench.workload_name(__import__("synth").CONFIGS[1])
    assert rec["kernel"].startswith("expert_gemm_kernel<0>")


def test_traffic_record_of_a_prefill_workload_counts_the_large_batch_kernel(tmp_path):
    mib = 16
    kib = mib * 1024
    _write_counters(tmp_path / "f", "FETCH_SIZE",
                    [(1, GU_BF16, 9e9), (2, PF_BF16, 500.0), (3, PF_ACT4, 7e9), (4, PF_BF16, 1500.0),
                     (6, COPY, kib / 2), (7, COPY, kib / 2), (8, COPY, kib / 2)])
    _write_counters(tmp_path / "w", "WRITE_SIZE",
                    [(2, PF_BF16, 10.0), (4, PF_BF16, 30.0), (6, COPY, kib), (7, COPY, kib), (8, COPY, kib)])
    rec = bench.traffic_record(str(tmp_path / "f"), str(tmp_path / "w"), mib, 4, "cmd")
    assert rec["fetch_gate_up_dispatches"] == 2
    assert rec["fetch_bytes_per_launch"] == 1000 * 1024 * 2
    assert rec["kernel_source_sha256_16"] == bench.gemm_source_hash("prefill")
    assert rec["kernel"].startswith("expert_gemm_prefill_kernel<0>")


def test_fractions_against_spec_and_measured_peaks():
    peaks = {"stream_read_nt_GB_per_s": 6000.0, "mfma_fp4xfp4_TFLOP_per_s": 7000.0,
             "mfma_fp6xfp4_TFLOP_per_s": 8000.0}
    # 1 TFLOP and 1 GB in 1 ms: 1 PF/s and 1 TB/s
    f = bench.fractions(1e12, 1e9, 1e-3, peaks, "default")
    assert f["spec"]["R_HBM"] == round(1000 / 8000, 4)
    assert f["spec"]["R_MXFP4"] == round(1000 / 10100, 4)
    # the default path issues two FP6 x FP4 instructions per tile: half the format's rate
    assert f["spec"]["R_roof"] == round(max(1e9 / 8e12, 1e12 / 5.05e15) / 1e-3, 4)
    assert f["spec"]["roof_bound"] == "mfma"
    assert f["measured"]["R_HBM"] == round(1000 / 6000, 4)
    assert f["measured"]["R_roof"] == round(max(1e9 / 6e12, 1e12 / 4e15) / 1e-3, 4)
    g = bench.fractions(1e12, 1e9, 1e-3, None, "act4")
    assert "measured" not in g and g["spec"]["R_roof"] == round(max(1e9 / 8e12, 1e12 / 10.1e15) / 1e-3, 4)


def test_the_headline_is_the_largest_workload():
    import synth
    sizes = {c: synth.CONFIGS[c]["T"] * synth.CONFIGS[c]["E"] for c in synth.CONFIGS}
    assert bench.HEADLINE == max(sizes, key=sizes.get)
    assert set(bench.SUB_RECORDS) | {bench.HEADLINE} == set(synth.CONFIGS) - {0}
    assert bench.gemm_kind(synth.CONFIGS[1]) == "decode" and bench.gemm_kind(synth.CONFIGS[4]) == "prefill"


def test_traffic_record_needs_three_calibration_copies(tmp_path):
    _write_counters(tmp_path / "f", "FETCH_SIZE", [(1, GU_BF16, 1.0), (2, COPY, 1.0), (3, COPY, 1.0)])
    _write_counters(tmp_path / "w", "WRITE_SIZE", [(1, GU_BF16, 1.0), (2, COPY, 1.0), (3, COPY, 1.0)])
    with pytest.raises(SystemExit):
        bench.traffic_record(str(tmp_path / "f"), str(tmp_path / "w"), 16, 1)


def test_traffic_is_reported_only_for_the_source_it_was_measured_on(monkeypatch, tmp_path):
    import synth
    cfg = dict(synth.CONFIGS[4])
    rec = {"workload": bench.workload_name(cfg), "kernel_source_sha256_16": "ab" * 8,
           "hbm_bytes_per_launch": 12345}
    path = tmp_path / "t.json"
    path.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "traffic_path", lambda c: str(path))
    monkeypatch.setattr(bench, "gemm_source_hash", lambda kind="decode": "ab" * 8)
    assert bench.traffic_for(cfg) == 12345
    assert bench.traffic_for(dict(cfg, T=4096)) is None                  # another workload
    monkeypatch.setattr(bench, "gemm_source_hash", lambda kind="decode": "0" * 16)
    assert bench.traffic_for(cfg) is None


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


def test_probe_crosscheck_divides_the_work_per_launch_by_the_trace_mean():
    rows = [dict(Name="void (anonymous namespace)::mfma_scaled_probe<2, 4>(int, float*)", AverageNs="2000000"),
            dict(Name="void (anonymous namespace)::stream_read_probe<1>(unsigned char const*)", AverageNs="500000")]
    rec = {"mfma_fp6xfp4_TFLOP_per_s": 6000.0, "stream_read_nt_GB_per_s": 4000.0,
           "work_per_launch": {"mfma_fp6xfp4_flop": 1.0e13, "stream_read_bytes": 2.0e9}}
    out = bench.probe_crosscheck(rows, rec)
    fp6 = next(l for l in out if l.startswith("fp6xfp4")).split()
    assert float(fp6[1]) == 6000.0 and float(fp6[2]) == 5000.0      # 1e13 flop / 2 ms = 5 PF
    nt = next(l for l in out if l.startswith("read_nt")).split()
    assert float(nt[1]) == 4000.0 and float(nt[2]) == 4000.0        # 2e9 B / 0.5 ms = 4 TB/s
    assert not any(l.startswith("bf16") for l in out)               # probes missing from the trace are left out


def test_traffic_record_carries_the_down_kernel_of_the_same_runs(tmp_path):
    mib = 16
    kib = mib * 1024
    _write_counters(tmp_path / "f", "FETCH_SIZE",
                    [(2, PF_BF16, 500.0), (3, PF_DOWN, 200.0), (4, PF_DOWN_ACT4, 9e9), (5, PF_DOWN, 400.0),
                     (6, COPY, kib / 2), (7, COPY, kib / 2), (8, COPY, kib / 2)])
    _write_counters(tmp_path / "w", "WRITE_SIZE",
                    [(2, PF_BF16, 10.0), (3, PF_DOWN, 50.0), (5, PF_DOWN, 70.0), (6, COPY, kib), (7, COPY, kib),
                     (8, COPY, kib)])
    rec = bench.traffic_record(str(tmp_path / "f"), str(tmp_path / "w"), mib, 2, "cmd")
    dn = rec["down"]
    assert dn["kernel"].startswith("expert_gemm_prefill_kernel<1>")
    assert dn["fetch_dispatches"] == 2 and dn["write_dispatches"] == 2       # the act4 down kernel is not it
    assert dn["fetch_bytes_per_launch"] == 300 * 1024 * 2                    # mean of 200 and 400 KiB, x 2
    assert dn["write_bytes_per_launch"] == 60 * 1024
    assert dn["hbm_bytes_per_launch"] == 300 * 1024 * 2 + 60 * 1024
    assert rec["hbm_bytes_per_launch"] == 500 * 1024 * 2 + 10 * 1024         # the gate/up record is unchanged
