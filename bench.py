#!/usr/bin/env python3
"""Benchmark of the MoE layer (MXFP4 experts) on one MI355X.

One step = one pass of the whole layer (route, permute, activation split,
gate/up GEMM + SwiGLU, down GEMM, combine) over one batch of synthetic tokens,
through ``moe_forward``, inputs resident in HBM.

The headline is the largest workload: the gpt-oss-120b MoE layer with skewed
routing, T=8192 tokens, d_model = d_ff = 2880, 128 experts, top-4 (a Zipf
router bias: 10% of the experts take about half of the assignments, 4 take
none).  The 20b decode (T=32), 20b prefill (T=4096) and 120b (T=4096)
workloads are measured first, each as a sub-record of the same line with its
own warm-up and step counts; the headline then runs exactly --warmup W untimed
and --steps K timed steps.  Steps rotate over L device copies of the layer's
weights (24 at decode, one decode step through every layer of the 20b model,
10.2 GB; 2 otherwise) so weights stream from HBM, not the 256 MB last-level
cache.

Every record carries tokens/s, TFLOP/s and GB/s of the algorithmic work and the
fractions R_HBM (of 8 TB/s), R_MXFP4 (of the 10.1 PFLOP/s dense FP4/FP6 matrix
peak) and R_roof (the time the roofline allows over the measured time, with the
matrix peak of the instruction mix the path issues: two FP6 x FP4 instructions
per weight tile), each against the published peaks and against the peaks the
probes of libmoe_peaks.so measure on the same GPU at the start of the run.

Prints one JSON line.  ``roofline`` is the headline's dominant kernel (the
gate/up expert GEMM) launched back to back on its stream between two HIP
events; ``cpu_baseline`` is the float64 oracle on the host on a bounded sample
of the headline workload, on all threads and on one.
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

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
FP4_PEAK_TFLOPS = 10100.0      # MI355X dense MXFP4 / MXFP6 matrix, published
EXPERT_BYTES_PER_PARAM = 17.0 / 32.0       # MXFP4: 4.25 bits
HEADLINE = 4                   # the largest workload: gpt-oss-120b, skewed routing, T=8192
SUB_RECORDS = (1, 2, 3)
# instruction mix of each path: matrix instructions per 32x32x64 weight tile and their format pair
MIX = {"default": dict(per_tile=2, fmt="fp6xfp4", what="two FP6 x FP4 instructions per weight tile "
                                                       "(bf16 activations as hi + lo FP6 terms)"),
       "act4": dict(per_tile=1, fmt="fp4xfp4", what="one FP4 x FP4 instruction per weight tile")}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=None,
                   help="timed steps of the headline (default: 200 at decode sizes, 30 otherwise)")
    p.add_argument("--warmup", type=int, default=None,
                   help="untimed steps before the headline's timed region (default: about 0.2 s of steps "
                        "for the workload, so the GPU clock has settled: 2000 decode steps, 300 prefill steps)")
    p.add_argument("--config", type=int, default=HEADLINE, help="headline workload index (4 = gpt-oss-120b skewed)")
    p.add_argument("--only", action="store_true", help="the headline workload only, no sub-records (profiling)")
    p.add_argument("--no-peaks", action="store_true", help="skip the ceiling probes (fractions against spec only)")
    p.add_argument("--layers", type=int, default=None, help="distinct weight copies to rotate over")
    p.add_argument("--kernel-steps", type=int, default=None, help="launches of the dominant kernel to time")
    p.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    p.add_argument("--cpu-tokens", type=int, default=None, help="tokens in the CPU-baseline sample")
    p.add_argument("--copy-mib", type=int, default=0,
                   help="after the measurements, run 3 plain device-to-device copies of this many MiB "
                        "(the calibration of the HBM byte counters)")
    p.add_argument("--traffic-report", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                   help="write the --config workload's gate/up kernel HBM traffic from two rocprofv3 --pmc "
                        "runs (FETCH_SIZE, WRITE_SIZE) of this script with --copy-mib, then exit")
    p.add_argument("--stats-report", nargs=2, metavar=("STATS_CSV", "OUT_TXT"),
                   help="summarise a rocprofv3 --stats kernel table as text, then exit")
    p.add_argument("--pmc-report", nargs=2, metavar=("PMC_DIR", "OUT_TXT"),
                   help="summarise a rocprofv3 --pmc --kernel-trace run (per-kernel counters, clock, MFMA rate)")
    p.add_argument("--command", default="", help="the command that made the profile (for the reports)")
    p.add_argument("--probe-json", default=None,
                   help="with --stats-report: the ceiling probes' JSON record of the same run, checked "
                        "against the trace")
    p.add_argument("--no-block", action="store_true", help="skip the timing of the pre-norm block forward")
    p.add_argument("--no-act4", action="store_true", help="skip the timing of the MXFP4-activation variant")
    return p.parse_args()


def workload_name(cfg: dict) -> str:
    return (f"gpt-oss MoE layer ({cfg['name']}): T={cfg['T']} tokens, d_model={cfg['D']}, d_ff={cfg['I']}, "
            f"{cfg['E']} experts, top-{cfg['k']}, MXFP4 experts, bf16 activations")


# the gate/up GEMM kernels and the sources whose device code they compile: the small-batch kernel
# (8-row tiles, decode) and the large-batch kernel (128-row tiles, prefill)
CSRC = os.path.join(ROOT, "mxfp4_expert_layer_moe_amd", "csrc")
GEMM_SRCS = {"decode": [os.path.join(CSRC, f) for f in ("gemm.hip", "mfma_ops.h", "moe_internal.h")],
             "prefill": [os.path.join(CSRC, f) for f in ("gemm_prefill.hip", "mfma_ops.h", "moe_internal.h")]}
GU_KERNEL = {"decode": ("void moe::expert_gemm_kernel<0,", ", 0>(moe::GemmArgs)"),
             "prefill": ("void moe::expert_gemm_prefill_kernel<0,", ", 0>(moe::PrefillArgs)")}
KERNEL_LABEL = {"decode": "expert_gemm_kernel<0> (gate/up + SwiGLU, 8-row tiles)",
                "prefill": "expert_gemm_prefill_kernel<0> (gate/up + SwiGLU, 128-row tiles)"}
DN_KERNEL = {"decode": ("void moe::expert_gemm_kernel<1,", ", 0>(moe::GemmArgs)"),
             "prefill": ("void moe::expert_gemm_prefill_kernel<1,", ", 0>(moe::PrefillArgs)")}
DN_LABEL = {"decode": "expert_gemm_kernel<1> (down, gate-scaled, 8-row tiles)",
            "prefill": "expert_gemm_prefill_kernel<1> (down, gate-scaled, 128-row tiles)"}


def gemm_kind(cfg: dict) -> str:
    """Which gate/up kernel the workload runs (the library's tile-height rule: 8-row tiles up to 6
    assignments per expert on average)."""
    return "decode" if cfg["T"] * cfg["k"] <= 6 * cfg["E"] else "prefill"


def gemm_source_hash(kind: str = "decode") -> str:
    h = hashlib.sha256()
    for f in GEMM_SRCS[kind]:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def traffic_path(cfg: dict) -> str:
    slug = cfg["name"].replace(" ", "_")
    return os.path.join(ROOT, "profiles", f"gate_up_gemm_traffic_{slug}_T{cfg['T']}.json")


COPY_KERNEL = "__amd_rocclr_copyBuffer"


def _counter_rows(d: str):
    import csv
    import glob
    files = sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True))
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    rows = []
    for f in files:
        rows += list(csv.DictReader(open(f)))
    return rows


def _per_dispatch(rows, counter: str):
    """{dispatch id: (kernel name, summed counter value)} in dispatch order."""
    out = {}
    for r in rows:
        if r["Counter_Name"] != counter:
            continue
        d = int(r["Dispatch_Id"])
        name, v = out.get(d, (r["Kernel_Name"], 0.0))
        out[d] = (name, v + float(r["Counter_Value"]))
    return dict(sorted(out.items()))


def traffic_record(fetch_dir: str, write_dir: str, copy_mib: int, config: int, command: str = "") -> dict:
    """Gate/up kernel HBM bytes per launch, each counter scaled by what it reads for a plain copy;
    the down kernel's from the same runs under "down".

    FETCH_SIZE and WRITE_SIZE are in KiB per dispatch (summed over the rows rocprofv3 writes for
    one dispatch).  The last three copyBuffer dispatches of each run are the --copy-mib
    calibration copies (read and write copy_mib MiB each).
    """
    cfg = dict(__import__("synth").CONFIGS[config])
    kind = gemm_kind(cfg)
    known = copy_mib * 2 ** 20
    if known <= 0:
        raise SystemExit("--traffic-report needs the --copy-mib the runs used")
    rec = {"workload": workload_name(cfg),
           "kernel": KERNEL_LABEL[kind],
           "kernel_source_sha256_16": gemm_source_hash(kind),
           "command": command}
    down = {"kernel": DN_LABEL[kind]}
    total = {"gu": 0.0, "dn": 0.0}
    for key, d, counter in (("fetch", fetch_dir, "FETCH_SIZE"), ("write", write_dir, "WRITE_SIZE")):
        per = _per_dispatch(_counter_rows(d), counter)
        cp = [v for n, v in per.values() if n.startswith(COPY_KERNEL)][-3:]
        sel = {tag: [v for n, v in per.values() if n.startswith(pre) and n.endswith(suf)]
               for tag, (pre, suf) in (("gu", GU_KERNEL[kind]), ("dn", DN_KERNEL[kind]))}
        if not sel["gu"] or len(cp) < 3:
            raise SystemExit(f"{d}: {len(sel['gu'])} gate/up dispatches, {len(cp)} calibration copies")
        factor = known / (sum(cp) / len(cp) * 1024.0)
        kib = sum(sel["gu"]) / len(sel["gu"])
        rec[f"{key}_kib_per_launch_raw"] = round(kib, 1)
        rec[f"{key}_gate_up_dispatches"] = len(sel["gu"])
        rec[f"{key}_copy_kib_raw"] = [round(v, 1) for v in cp]
        rec[f"{key}_copy_scale"] = round(factor, 5)
        rec[f"{key}_bytes_per_launch"] = int(kib * 1024.0 * factor)
        total["gu"] += kib * 1024.0 * factor
        if sel["dn"]:
            kd = sum(sel["dn"]) / len(sel["dn"])
            down[f"{key}_kib_per_launch_raw"] = round(kd, 1)
            down[f"{key}_dispatches"] = len(sel["dn"])
            down[f"{key}_bytes_per_launch"] = int(kd * 1024.0 * factor)
            total["dn"] += kd * 1024.0 * factor
    rec["copy_bytes_each_way"] = known
    rec["hbm_bytes_per_launch"] = int(total["gu"])
    if "fetch_bytes_per_launch" in down and "write_bytes_per_launch" in down:
        down["hbm_bytes_per_launch"] = int(total["dn"])
        rec["down"] = down
    return rec


def traffic_report(args):
    """Write the traffic record of two counter runs to profiles/gate_up_gemm_traffic_<workload>.json."""
    rec = traffic_record(args.traffic_report[0], args.traffic_report[1], args.copy_mib, args.config, args.command)
    path = traffic_path(__import__("synth").CONFIGS[args.config])
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec))


def stats_report(args):
    """Text table of a rocprofv3 kernel_stats.csv (per-kernel calls and durations)."""
    import csv
    rows = list(csv.DictReader(open(args.stats_report[0])))
    lines = [f"# rocprofv3 --kernel-trace --stats summary",
             f"# command: {args.command}" if args.command else "# command: (not given)",
             f"{'kernel':<72} {'calls':>7} {'avg_us':>9} {'min_us':>9} {'max_us':>9} {'pct':>6}"]
    for r in rows:
        lines.append(f"{r['Name'][:72]:<72} {int(r['Calls']):>7} {float(r['AverageNs']) / 1e3:>9.2f} "
                     f"{float(r['MinNs']) / 1e3:>9.2f} {float(r['MaxNs']) / 1e3:>9.2f} "
                     f"{float(r['Percentage']):>6.2f}")
    if args.probe_json:
        lines += probe_crosscheck(rows, json.load(open(args.probe_json)))
    with open(args.stats_report[1], "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def probe_crosscheck(rows: list, rec: dict) -> list:
    """The ceiling probes' own rates (HIP events around five back-to-back launches) beside the
    work per launch divided by the kernel trace's mean duration of the same run's probe kernels."""
    kern = {"fp6xfp4": "mfma_scaled_probe<2, 4>", "fp4xfp4": "mfma_scaled_probe<4, 4>",
            "fp8xfp4": "mfma_scaled_probe<0, 4>", "bf16": "mfma_bf16_probe",
            "read_nt": "stream_read_probe<1>", "read": "stream_read_probe<0>"}
    work = rec["work_per_launch"]
    out = ["", "# probe rates: events (the probe's own timing) vs work per launch / trace mean duration",
           f"{'probe':<10} {'events':>12} {'trace':>12} {'unit':>8}"]
    for name, k in kern.items():
        r = next((r for r in rows if k in r["Name"]), None)
        if r is None:
            continue
        secs = float(r["AverageNs"]) * 1e-9
        if name.startswith("read"):
            ev = rec["stream_read_nt_GB_per_s" if name == "read_nt" else "stream_read_GB_per_s"]
            tr = work["stream_read_bytes"] / secs / 1e9
            unit = "GB/s"
        else:
            ev = rec[f"mfma_{name}_TFLOP_per_s"]
            tr = work[f"mfma_{name}_flop"] / secs / 1e12
            unit = "TFLOP/s"
        out.append(f"{name:<10} {ev:>12.1f} {tr:>12.1f} {unit:>8}")
    out.append("# probe record: " + json.dumps(rec))
    return out


def pmc_summary(d: str) -> list:
    """Per kernel of a rocprofv3 --pmc --kernel-trace run: dispatches, mean duration, the mean of
    each counter per dispatch, and two derived figures when their counters are there:
    SQ_INSTS_VALU_MFMA_MOPS_F6F4 x 512 / duration (FP4/FP6 matrix FLOP/s executed, the counter
    being in units of 512 operations: 256 per 32x32x64 instruction) and
    SQ_VALU_MFMA_BUSY_CYCLES / 1024 (matrix-pipe busy cycles per SIMD: the counter sums all
    256 compute units x 4 SIMDs)."""
    import csv
    import glob
    rows = _counter_rows(d)
    traces = sorted(glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True))
    dur = {}
    for f in traces:
        for r in csv.DictReader(open(f)):
            dur[int(r["Dispatch_Id"])] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
    per = {}                                   # kernel -> dispatch -> counter -> summed value
    for r in rows:
        k = per.setdefault(r["Kernel_Name"], {}).setdefault(int(r["Dispatch_Id"]), {})
        k[r["Counter_Name"]] = k.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    out = []
    for name, ds in per.items():
        counters = sorted({c for v in ds.values() for c in v})
        mean = {c: sum(v.get(c, 0.0) for v in ds.values()) / len(ds) for c in counters}
        secs = [dur[i] for i in ds if i in dur]
        rec = dict(kernel=name, dispatches=len(ds), counters=mean)
        if "SQ_VALU_MFMA_BUSY_CYCLES" in mean:
            rec["mfma_busy_cycles_per_simd"] = mean["SQ_VALU_MFMA_BUSY_CYCLES"] / 1024
        if secs:
            t = sum(secs) / len(secs)
            rec["mean_us"] = t * 1e6
            if "SQ_INSTS_VALU_MFMA_MOPS_F6F4" in mean:
                rec["mfma_f6f4_TFLOP_per_s"] = mean["SQ_INSTS_VALU_MFMA_MOPS_F6F4"] * 512 / t * 1e-12
        out.append(rec)
    return sorted(out, key=lambda r: -r.get("mean_us", 0.0))


def pmc_report(args):
    recs = pmc_summary(args.pmc_report[0])
    lines = ["# rocprofv3 --pmc counter summary (mean per dispatch)",
             f"# command: {args.command}" if args.command else "# command: (not given)"]
    for r in recs:
        if not any(k in r["kernel"] for k in ("expert_gemm", "route", "combine", "permute", "rmsnorm", "pack")):
            continue
        head = f"{r['kernel']}  dispatches={r['dispatches']}"
        if "mean_us" in r:
            head += f"  mean={r['mean_us']:.2f} us"
        if r.get("mfma_f6f4_TFLOP_per_s"):
            head += f"  F6F4 MFMA executed={r['mfma_f6f4_TFLOP_per_s']:.1f} TFLOP/s"
        if r.get("mfma_busy_cycles_per_simd"):
            head += f"  MFMA busy={r['mfma_busy_cycles_per_simd']:.4g} cycles/SIMD"
        lines.append(head)
        for c, v in r["counters"].items():
            lines.append(f"    {c:<36} {v:.6g}")
    with open(args.pmc_report[1], "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def traffic_for(cfg: dict):
    """HBM bytes per launch of the workload's gate/up kernel from committed rocprofv3 counter runs,
    if they were taken on this kernel source."""
    path = traffic_path(cfg)
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_source_sha256_16") != gemm_source_hash(gemm_kind(cfg)) or \
            rec.get("workload") != workload_name(cfg):
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(inp, n_tokens):
    """The float64 oracle on the host on a bounded sample of the workload: routing of every token,
    experts and combine for the first n_tokens tokens.  Timed on all the threads numpy's BLAS uses
    and again on one."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        cores = max([d.get("num_threads", 1) for d in threadpool_info()] + [1])
    except Exception:                           # pragma: no cover - threadpoolctl is installed
        threadpool_limits = None
        cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    tokens = np.arange(min(n_tokens, inp.T))

    def timed():
        t0 = time.perf_counter()
        oracle.forward(inp, tokens=tokens)
        return time.perf_counter() - t0
    dt = timed()
    rec = dict(value=round(len(tokens) / dt, 3), unit="tokens/s", cores=cores, kind="oracle",
               sample=f"float64 oracle on the headline workload: routing of all {inp.T} tokens, experts and "
                      f"combine for {len(tokens)} tokens, one pass in {dt:.1f} s on {cores} threads",
               nproc=os.cpu_count(), cpu_model=cpu_model())
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            d1 = timed()
        rec["value_1_thread"] = round(len(tokens) / d1, 3)
        rec["seconds_1_thread"] = round(d1, 1)
    return rec


def fractions(flops: float, nbytes: float, secs: float, peaks: dict | None, mix: str) -> dict:
    """R_HBM, R_MXFP4 and R_roof of work (flops, bytes) done in secs, against the published peaks and
    the measured ones.  R_roof = max(bytes / BW, flops / P_mix) / secs, where P_mix is the matrix rate
    of the path's format pair divided by its instructions per weight tile."""
    m = MIX[mix]
    out = {"instruction_mix": m["what"]}
    sides = [("spec", HBM_PEAK_GBS, FP4_PEAK_TFLOPS, FP4_PEAK_TFLOPS)]
    if peaks:
        sides.append(("measured", peaks["stream_read_nt_GB_per_s"], peaks["mfma_fp4xfp4_TFLOP_per_s"],
                      peaks[f"mfma_{m['fmt']}_TFLOP_per_s"]))
    for side, bw, p4, pfmt in sides:
        bw_b, p4_f, pmix_f = bw * 1e9, p4 * 1e12, pfmt * 1e12 / m["per_tile"]
        t_roof = max(nbytes / bw_b, flops / pmix_f)
        out[side] = dict(R_HBM=round(nbytes / secs / bw_b, 4), R_MXFP4=round(flops / secs / p4_f, 4),
                         R_roof=round(t_roof / secs, 4),
                         roof_bound="hbm" if nbytes / bw_b >= flops / pmix_f else "mfma",
                         peaks=dict(hbm_GB_per_s=bw, mxfp4_TFLOP_per_s=p4,
                                    instruction_mix_TFLOP_per_s=round(pfmt / m["per_tile"], 1)))
    return out


def _time_steps(fn, copies, warmup: int, steps: int) -> float:
    """ms per call of fn(weights) over `steps` calls after `warmup` untimed ones, HIP events on the
    current stream (the calls run back to back on it), weight copies rotated."""
    import torch
    stream = torch.cuda.current_stream()
    L = len(copies)
    for s in range(warmup):
        fn(copies[s % L])
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for s in range(steps):
        fn(copies[s % L])
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def _time_alternating(fa, fb, copies, warmup: int, steps: int, rounds: int = 8) -> tuple:
    """Medians of ms per call of fa and of fb, timed in alternating stretches of steps // rounds calls
    (so a drift of the clock affects both alike), after `warmup` untimed calls of each."""
    import torch
    stream = torch.cuda.current_stream()
    L = len(copies)
    for s in range(warmup):
        fa(copies[s % L])
        fb(copies[s % L])
    n = max(1, steps // rounds)
    ta, tb = [], []
    for r in range(rounds):
        for fn, out in ((fa, ta), (fb, tb)):
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for s in range(n):
                fn(copies[s % L])
            b.record(stream)
            torch.cuda.synchronize()
            out.append(a.elapsed_time(b) / n)
    med = lambda v: sorted(v)[len(v) // 2]
    return med(ta), med(tb)


def default_counts(ci: int):
    """(warm-up, timed steps) of a workload: about 0.2 s of warm-up so the clock has settled."""
    decode = synth_configs()[ci]["T"] <= 64
    return (2000, 200) if decode else ((20, 20) if ci == 0 else (300, 30))


def synth_configs():
    import synth
    return synth.CONFIGS


class Workload:
    """A workload's inputs on the device, its weight copies and its algorithmic work."""

    def __init__(self, ci: int, layers: int | None):
        import synth
        from mxfp4_expert_layer_moe_amd.device import DeviceLayer
        self.ci = ci
        self.cfg = dict(synth.CONFIGS[ci])
        t0 = time.time()
        self.inp = synth.make_inputs(ci)
        self.layer = DeviceLayer(self.inp)
        self.L = layers or (24 if self.cfg["T"] <= 64 else 2)
        self.copies = [self.layer.weights] + [self.layer.weights.clone() for _ in range(self.L - 1)]
        print(f"[bench] workload {ci} ({self.cfg['name']}, T={self.cfg['T']}) ready in {time.time() - t0:.1f}s",
              file=sys.stderr, flush=True)

    def measure(self, warmup: int, steps: int, peaks: dict | None, block: bool = True, act4: bool = True,
                kernel_steps: int | None = None) -> dict:
        import torch
        inp, layer, copies = self.inp, self.layer, self.copies
        T, D, E, k, I = inp.T, inp.D, inp.E, inp.k, inp.I
        t0 = time.perf_counter()
        ms = _time_steps(lambda w: layer.forward(weights=w), copies, warmup, steps)
        wall = time.perf_counter() - t0
        layer.route(logits=False)
        layer.permute()
        layer.pack_x()
        torch.cuda.synchronize()
        touched = int((layer.counts.cpu().numpy() > 0).sum())
        flops = T * k * (2 * D * 2 * I + 2 * I * D) + 2 * T * D * E
        nbytes = touched * 3 * D * I * EXPERT_BYTES_PER_PARAM + T * D * 2 * 2 + E * D * 4
        secs = ms * 1e-3
        rec = {"workload": workload_name(self.cfg), "tokens_per_step": T, "experts_touched": touched,
               "weight_copies_rotated": self.L, "warmup": warmup, "steps": steps,
               "ms_per_step": round(ms, 5), "tokens_per_s": round(T / secs, 1),
               "TFLOP_per_s": round(flops / secs / 1e12, 2), "GB_per_s": round(nbytes / secs / 1e9, 1),
               "alg_flops": int(flops), "alg_bytes": int(nbytes), "wall_s_timed": round(wall, 3),
               "fractions": fractions(flops, nbytes, secs, peaks, "default")}
        # the dominant kernel alone: the gate/up expert GEMM, launched back to back
        kind = gemm_kind(self.cfg)
        k_ms = _time_steps(lambda w: layer.gate_up(weights=w), copies, warmup, kernel_steps or steps)
        gu_bytes = touched * 2 * I * D * EXPERT_BYTES_PER_PARAM + T * D * 2 + T * k * I * 2
        gu_flops = 2.0 * T * k * D * 2 * I
        ks = k_ms * 1e-3
        fr = fractions(gu_flops, gu_bytes, ks, peaks, "default")
        bound = fr["spec"]["roof_bound"]
        if bound == "hbm":
            achieved = gu_bytes / ks / 1e9
            roof = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                        frac=round(achieved / HBM_PEAK_GBS, 4))
        else:
            achieved = gu_flops / ks / 1e12
            roof = dict(bound="mfma", achieved=round(achieved, 1), peak=FP4_PEAK_TFLOPS, unit="TFLOP/s",
                        frac=round(achieved / FP4_PEAK_TFLOPS, 4))
        roof["traffic"] = traffic_for(self.cfg)
        roof.update(kernel=KERNEL_LABEL[kind], kernel_ms=round(k_ms, 5), alg_bytes_per_launch=int(gu_bytes),
                    alg_flops_per_launch=int(gu_flops), fractions=fr)
        rec["gate_up_kernel"] = roof
        if block:
            # the layer and the block timed in alternating stretches, medians of each
            l_ms, b_ms = _time_alternating(lambda w: layer.forward(weights=w),
                                           lambda w: layer.block_forward(weights=w), copies, warmup, 4 * steps)
            rec["block"] = {"what": "RMSNorm -> MoE layer -> residual add (moe_block_forward)",
                            "ms_per_step": round(b_ms, 5), "tokens_per_s": round(T / (b_ms * 1e-3), 1),
                            "layer_ms_per_step_alternating": round(l_ms, 5),
                            "extra_ms_over_layer": round(b_ms - l_ms, 5),
                            "timing": "layer and block in 8 alternating stretches of 4 * steps / 8 calls each, "
                                      "medians"}
        if act4:
            a_ms = _time_steps(lambda w: layer.forward_act4(weights=w), copies, warmup, steps)
            rec["act4"] = {"what": "MXFP4 activations into the expert GEMMs (moe_forward_act4; a lower-precision "
                                   "contract)", "ms_per_step": round(a_ms, 5),
                           "tokens_per_s": round(T / (a_ms * 1e-3), 1),
                           "fractions": fractions(flops, nbytes, a_ms * 1e-3, peaks, "act4")}
        return rec

    def free(self):
        import torch
        self.layer = self.copies = None
        torch.cuda.empty_cache()


def main():
    args = parse()
    if args.traffic_report:
        return traffic_report(args)
    if args.stats_report:
        return stats_report(args)
    if args.pmc_report:
        return pmc_report(args)
    if args.gpus != 1:
        print(json.dumps({"error": "the MoE layer here runs on one GPU only: --gpus must be 1 "
                          "(expert-parallel sharding over several GPUs is designed, not implemented)"}))
        sys.exit(2)
    import torch
    import mxfp4_expert_layer_moe_amd as M

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    M.lib()
    head_ci = args.config
    dw, ds = default_counts(head_ci)
    warmup = dw if args.warmup is None else args.warmup
    steps = ds if args.steps is None else args.steps
    subs = [] if args.only else [c for c in SUB_RECORDS if c != head_ci]
    # every workload is on the device before any timing, so the GPU does not idle between them
    work = {ci: Workload(ci, args.layers if ci == head_ci else None) for ci in subs + [head_ci]}
    peaks = None
    if not args.no_peaks:
        from mxfp4_expert_layer_moe_amd import peaks as P
        peaks = P.measure_all()
        print(f"[bench] measured ceilings {json.dumps(peaks)}", file=sys.stderr, flush=True)
    records = {}
    for ci in subs:
        sw, ss = default_counts(ci)
        records[ci] = work[ci].measure(sw, ss, peaks, block=not args.no_block, act4=not args.no_act4)
        print(f"[bench] workload {ci}: {records[ci]['ms_per_step']} ms/step", file=sys.stderr, flush=True)
    # ---- the headline: exactly `warmup` untimed and `steps` timed whole-layer steps -------------
    torch.cuda.synchronize()
    head = work[head_ci].measure(warmup, steps, peaks, block=not args.no_block, act4=not args.no_act4,
                                 kernel_steps=args.kernel_steps)
    cfg = work[head_ci].cfg
    roof = head.pop("gate_up_kernel")
    out = {
        "metric": "MoE-layer tokens/s (whole layer, one MI355X)",
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4 weights (e2m1, e8m0 per 32) x activations as hi+lo mxfp6 terms (e2m3, e8m0 per 32) "
                 "-> fp32 accumulate",
        "data": "synthetic",
        "config": {"workload": head["workload"], "tokens_per_step": cfg["T"],
                   "weight_copies_rotated": head["weight_copies_rotated"],
                   "experts_touched": head["experts_touched"]},
        "layer": {k: head[k] for k in ("alg_flops", "alg_bytes", "TFLOP_per_s", "GB_per_s", "wall_s_timed",
                                        "fractions")},
        "roofline": roof,
        "cpu_baseline": None,
        "peaks_measured": peaks,
        "workloads": {synth_configs()[ci]["name"]: rec for ci, rec in records.items()},
    }
    for key in ("block", "act4"):
        if key in head:
            out[key] = head[key]
    for w in work.values():
        w.free()
    if args.copy_mib > 0:                     # counter calibration: plain copies of known size, untimed
        n = args.copy_mib * 2 ** 20
        a = torch.empty(n, dtype=torch.uint8, device="cuda")
        b = torch.empty(n, dtype=torch.uint8, device="cuda")
        a.fill_(1)
        torch.cuda.synchronize()
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(work[head_ci].inp, args.cpu_tokens or (cfg["T"] if cfg["T"] <= 64 else 8))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
