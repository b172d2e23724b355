#!/usr/bin/env python3
"""Benchmark of the MoE layer (MXFP4 experts) on one MI355X.

One step = one pass of the whole layer (route, permute, activation split,
gate/up GEMM + SwiGLU, down GEMM, combine) over one batch of synthetic tokens,
through ``moe_forward``.  The default workload is the gpt-oss-20b MoE layer at
decode: T=32 tokens, d_model = d_ff = 2880, 32 experts, top-4.  Steps rotate
over L distinct device copies of the layer's weights (default 24, one decode
step through every layer of the 20b model: 10.2 GB) so each step streams its
weights from HBM rather than from the 256 MB last-level cache.

Prints one JSON line.  ``value`` is tokens/s of the layer; ``roofline`` is the
dominant kernel (the gate/up expert GEMM) launched back to back on its stream,
between two HIP events; ``cpu_baseline`` is the float64 oracle on the host on a bounded sample.
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
FP4_PEAK_TFLOPS = 10100.0      # MI355X dense MXFP4 matrix, published
EXPERT_BYTES_PER_PARAM = 17.0 / 32.0       # MXFP4: 4.25 bits


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=None,
                   help="untimed steps before each timed region (default: about 0.2 s of steps for the "
                        "workload, so the GPU clock has settled: 2000 decode steps, 300 prefill steps)")
    p.add_argument("--config", type=int, default=1, help="workload index (1 = gpt-oss-20b decode)")
    p.add_argument("--layers", type=int, default=None, help="distinct weight copies to rotate over")
    p.add_argument("--kernel-steps", type=int, default=None, help="launches of the dominant kernel to time")
    p.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    p.add_argument("--cpu-tokens", type=int, default=None, help="tokens in the CPU-baseline sample")
    p.add_argument("--copy-mib", type=int, default=0,
                   help="after the measurements, run 3 plain device-to-device copies of this many MiB "
                        "(the calibration of the HBM byte counters)")
    p.add_argument("--traffic-report", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                   help="write the gate/up kernel's HBM traffic from two rocprofv3 --pmc runs "
                        "(FETCH_SIZE, WRITE_SIZE) of this script with --copy-mib, then exit")
    p.add_argument("--stats-report", nargs=2, metavar=("STATS_CSV", "OUT_TXT"),
                   help="summarise a rocprofv3 --stats kernel table as text, then exit")
    p.add_argument("--pmc-report", nargs=2, metavar=("PMC_DIR", "OUT_TXT"),
                   help="summarise a rocprofv3 --pmc --kernel-trace run (per-kernel counters, clock, MFMA rate)")
    p.add_argument("--command", default="", help="the command that made the profile (for the reports)")
    p.add_argument("--no-block", action="store_true", help="skip the timing of the pre-norm block forward")
    p.add_argument("--no-act4", action="store_true", help="skip the timing of the MXFP4-activation variant")
    return p.parse_args()


def workload_name(cfg: dict) -> str:
    return (f"gpt-oss MoE layer ({cfg['name']}): T={cfg['T']} tokens, d_model={cfg['D']}, d_ff={cfg['I']}, "
            f"{cfg['E']} experts, top-{cfg['k']}, MXFP4 experts, bf16 activations")


# the decode GEMM kernel and the headers whose device code it compiles
GEMM_SRCS = [os.path.join(ROOT, "mxfp4_expert_layer_moe_amd", "csrc", f)
             for f in ("gemm.hip", "mfma_ops.h", "moe_internal.h")]


def gemm_source_hash() -> str:
    h = hashlib.sha256()
    for f in GEMM_SRCS:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]
GU_KERNEL_PREFIX = "void moe::expert_gemm_kernel<0,"
GU_KERNEL_BF16_SUFFIX = ", 0>(moe::GemmArgs)"     # last template argument: bf16 (split FP6) activations
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
    """Gate/up kernel HBM bytes per launch, each counter scaled by what it reads for a plain copy.

    FETCH_SIZE and WRITE_SIZE are in KiB per dispatch (summed over the rows rocprofv3 writes for
    one dispatch).  The last three copyBuffer dispatches of each run are the --copy-mib
    calibration copies (read and write copy_mib MiB each).
    """
    cfg = dict(__import__("synth").CONFIGS[config])
    known = copy_mib * 2 ** 20
    if known <= 0:
        raise SystemExit("--traffic-report needs the --copy-mib the runs used")
    rec = {"workload": workload_name(cfg),
           "kernel": "expert_gemm_kernel<0> (gate/up + SwiGLU)",
           "kernel_source_sha256_16": gemm_source_hash(),
           "command": command}
    total = 0.0
    for key, d, counter in (("fetch", fetch_dir, "FETCH_SIZE"), ("write", write_dir, "WRITE_SIZE")):
        per = _per_dispatch(_counter_rows(d), counter)
        gu = [v for n, v in per.values() if n.startswith(GU_KERNEL_PREFIX) and n.endswith(GU_KERNEL_BF16_SUFFIX)]
        cp = [v for n, v in per.values() if n.startswith(COPY_KERNEL)][-3:]
        if not gu or len(cp) < 3:
            raise SystemExit(f"{d}: {len(gu)} gate/up dispatches, {len(cp)} calibration copies")
        kib = sum(gu) / len(gu)
        factor = known / (sum(cp) / len(cp) * 1024.0)
        rec[f"{key}_kib_per_launch_raw"] = round(kib, 1)
        rec[f"{key}_gate_up_dispatches"] = len(gu)
        rec[f"{key}_copy_kib_raw"] = [round(v, 1) for v in cp]
        rec[f"{key}_copy_scale"] = round(factor, 5)
        rec[f"{key}_bytes_per_launch"] = int(kib * 1024.0 * factor)
        total += kib * 1024.0 * factor
    rec["copy_bytes_each_way"] = known
    rec["hbm_bytes_per_launch"] = int(total)
    return rec


def traffic_report(args):
    """Write the traffic record of two counter runs to profiles/gate_up_gemm_traffic.json."""
    rec = traffic_record(args.traffic_report[0], args.traffic_report[1], args.copy_mib, args.config, args.command)
    path = os.path.join(ROOT, "profiles", "gate_up_gemm_traffic.json")
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
    with open(args.stats_report[1], "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


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


def traffic_for(workload: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if taken on this kernel source."""
    path = os.path.join(ROOT, "profiles", "gate_up_gemm_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_source_sha256_16") != gemm_source_hash() or rec.get("workload") != workload:
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(inp, n_tokens):
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([d.get("num_threads", 1) for d in threadpool_info()] + [1])
    except Exception:
        cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    tokens = np.arange(min(n_tokens, inp.T))
    # whole passes over the sample until about 10 s of CPU work (at most 4 passes)
    passes, t0 = 0, time.perf_counter()
    while passes < 4 and (passes == 0 or time.perf_counter() - t0 < 10.0):
        oracle.forward(inp, tokens=tokens)
        passes += 1
    dt = time.perf_counter() - t0
    return dict(value=round(passes * len(tokens) / dt, 3), unit="tokens/s", cores=cores, kind="oracle",
                sample=f"float64 oracle, whole layer (routing of all {inp.T} tokens, experts and combine for "
                       f"{len(tokens)} tokens), {passes} pass(es) in {dt:.1f} s")


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
    import numpy as np
    import torch
    import synth
    import mxfp4_expert_layer_moe_amd as M
    from mxfp4_expert_layer_moe_amd.device import DeviceLayer

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    M.lib()
    cfg = synth.CONFIGS[args.config]
    decode = args.config == 1
    if args.warmup is None:
        # short warmups time the GPU partly before its clock has ramped up: measured 4-5% slower
        # prefill steps after 5 warmup steps than after 300
        args.warmup = 2000 if decode else (20 if args.config == 0 else 300)
    L = args.layers or (24 if decode else 2)
    t0 = time.time()
    inp = synth.make_inputs(args.config)
    print(f"[bench] inputs for config {args.config} in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    layer = DeviceLayer(inp)
    copies = [layer.weights] + [layer.weights.clone() for _ in range(L - 1)]
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    T, D, E, k, I = inp.T, inp.D, inp.E, inp.k, inp.I

    # ---- headline: K whole-layer steps ---------------------------------------
    for s in range(args.warmup):
        layer.forward(weights=copies[s % L])
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for s in range(args.steps):
        layer.forward(weights=copies[s % L])
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ms_total = ev0.elapsed_time(ev1)
    ms_step = ms_total / args.steps

    # ---- the pre-norm block around the layer, y = x + MoE(RMSNorm(x)), same steps -----
    block = None
    if not args.no_block:
        for s in range(args.warmup):
            layer.block_forward(weights=copies[s % L])
        torch.cuda.synchronize()
        eb0, eb1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        eb0.record(stream)
        for s in range(args.steps):
            layer.block_forward(weights=copies[s % L])
        eb1.record(stream)
        torch.cuda.synchronize()
        b_ms = eb0.elapsed_time(eb1) / args.steps
        block = {"what": "RMSNorm -> MoE layer -> residual add (moe_block_forward)",
                 "ms_per_step": round(b_ms, 5), "tokens_per_s": round(T / (b_ms * 1e-3), 1),
                 "extra_ms_over_layer": round(b_ms - ms_step, 5)}

    # ---- the activation-quantized variant (MXFP4 activations), same steps ---------
    act4 = None
    if not args.no_act4:
        for s in range(args.warmup):
            layer.forward_act4(weights=copies[s % L])
        torch.cuda.synchronize()
        e40, e41 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e40.record(stream)
        for s in range(args.steps):
            layer.forward_act4(weights=copies[s % L])
        e41.record(stream)
        torch.cuda.synchronize()
        a_ms = e40.elapsed_time(e41) / args.steps
        act4 = {"what": "MXFP4 activations into the expert GEMMs (moe_forward_act4; a lower-precision contract)",
                "ms_per_step": round(a_ms, 5), "tokens_per_s": round(T / (a_ms * 1e-3), 1)}

    # ---- dominant kernel alone: gate/up expert GEMM, per-launch HIP events -----
    layer.route(logits=False)
    layer.permute()
    layer.pack_x()
    torch.cuda.synchronize()
    counts = layer.counts.cpu().numpy()
    touched = int((counts > 0).sum())
    nk = args.kernel_steps or args.steps
    for s in range(args.warmup):
        layer.gate_up(weights=copies[s % L])
    ka, kb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ka.record(stream)                        # the launches run back to back on this stream
    for s in range(nk):
        layer.gate_up(weights=copies[s % L])
    kb.record(stream)
    torch.cuda.synchronize()
    k_ms = ka.elapsed_time(kb) / nk
    gu_weight_bytes = touched * 2 * I * D * EXPERT_BYTES_PER_PARAM
    gu_alg_bytes = gu_weight_bytes + T * D * 2 + T * k * I * 2            # weights + x in + h out (bf16)
    gu_flops = 2.0 * T * k * D * 2 * I
    workload = workload_name(cfg)
    if decode or gu_alg_bytes / HBM_PEAK_GBS > gu_flops / FP4_PEAK_TFLOPS / 1e3:
        achieved = gu_alg_bytes / (k_ms * 1e-3) / 1e9
        roof = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBS, 4))
    else:
        achieved = gu_flops / (k_ms * 1e-3) / 1e12
        roof = dict(bound="mfma", achieved=round(achieved, 1), peak=FP4_PEAK_TFLOPS, unit="TFLOP/s",
                    frac=round(achieved / FP4_PEAK_TFLOPS, 4))
    roof["traffic"] = traffic_for(workload)
    roof["kernel"] = "expert_gemm_kernel<0> (gate/up + SwiGLU)"
    roof["kernel_ms"] = round(k_ms, 5)
    roof["alg_bytes_per_launch"] = int(gu_alg_bytes)

    # whole-layer algorithmic bytes / flops (touched experts' weights, x and y in bf16, router weights)
    layer_bytes = touched * 3 * D * I * EXPERT_BYTES_PER_PARAM + T * D * 2 * 2 + E * D * 4
    layer_flops = T * k * (2 * D * 2 * I + 2 * I * D) + 2 * T * D * E

    out = {
        "metric": "MoE-layer tokens/s (whole layer, one MI355X)",
        "value": round(T / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4(e2m1,e8m0) x bf16 -> fp32",
        "data": "synthetic",
        "config": {"workload": workload, "tokens_per_step": T, "weight_copies_rotated": L,
                   "experts_touched": touched},
        "layer": {"alg_bytes": int(layer_bytes), "GB_per_s": round(layer_bytes / (ms_step * 1e-3) / 1e9, 1),
                  "hbm_frac": round(layer_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                  "TFLOP_per_s": round(layer_flops / (ms_step * 1e-3) / 1e12, 2),
                  "wall_s_timed": round(wall, 3)},
        "roofline": roof,
        "cpu_baseline": None,
    }
    if block is not None:
        out["block"] = block
    if act4 is not None:
        out["act4"] = act4
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
        out["cpu_baseline"] = cpu_baseline(inp, args.cpu_tokens or (T if decode else 8))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
