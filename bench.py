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
dominant kernel (the gate/up expert GEMM) timed alone with HIP events on its
stream; ``cpu_baseline`` is the float64 oracle on the host on a bounded sample.
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
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--config", type=int, default=1, help="workload index (1 = gpt-oss-20b decode)")
    p.add_argument("--layers", type=int, default=None, help="distinct weight copies to rotate over")
    p.add_argument("--kernel-steps", type=int, default=None, help="launches of the dominant kernel to time")
    p.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    p.add_argument("--cpu-tokens", type=int, default=None, help="tokens in the CPU-baseline sample")
    return p.parse_args()


def traffic_for(kernel_src: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if taken on this kernel source."""
    path = os.path.join(ROOT, "profiles", "gate_up_gemm_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    h = hashlib.sha256(open(kernel_src, "rb").read()).hexdigest()[:16]
    if rec.get("kernel_source_sha256_16") != h or rec.get("workload") != workload:
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
    t0 = time.perf_counter()
    oracle.forward(inp, tokens=tokens)
    dt = time.perf_counter() - t0
    return dict(value=round(len(tokens) / dt, 3), unit="tokens/s", cores=cores, kind="oracle",
                sample=f"float64 oracle, whole layer (routing of all {inp.T} tokens, experts and combine for "
                       f"{len(tokens)} tokens), {dt:.1f} s")


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only: --gpus must be 1 "
                          "(the multi-GPU sharding is described in the design notes, not built)"}))
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

    # ---- dominant kernel alone: gate/up expert GEMM, per-launch HIP events -----
    layer.route(logits=False)
    layer.permute()
    layer.pack_x()
    torch.cuda.synchronize()
    counts = layer.counts.cpu().numpy()
    touched = int((counts > 0).sum())
    nk = args.kernel_steps or args.steps
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(nk)]
    for s in range(args.warmup):
        layer.gate_up(weights=copies[s % L])
    for s in range(nk):
        evs[s][0].record(stream)
        layer.gate_up(weights=copies[s % L])
        evs[s][1].record(stream)
    torch.cuda.synchronize()
    k_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    gu_weight_bytes = touched * 2 * I * D * EXPERT_BYTES_PER_PARAM
    gu_alg_bytes = gu_weight_bytes + T * D * 2 + T * k * I * 2            # weights + x in + h out (bf16)
    gu_flops = 2.0 * T * k * D * 2 * I
    workload = (f"gpt-oss MoE layer ({cfg['name']}): T={T} tokens, d_model={D}, d_ff={I}, "
                f"{E} experts, top-{k}, MXFP4 experts, bf16 activations")
    src = os.path.join(ROOT, "mxfp4_expert_layer_moe_amd", "csrc", "gemm.hip")
    if decode or gu_alg_bytes / HBM_PEAK_GBS > gu_flops / FP4_PEAK_TFLOPS / 1e3:
        achieved = gu_alg_bytes / (k_ms * 1e-3) / 1e9
        roof = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBS, 4))
    else:
        achieved = gu_flops / (k_ms * 1e-3) / 1e12
        roof = dict(bound="mfma", achieved=round(achieved, 1), peak=FP4_PEAK_TFLOPS, unit="TFLOP/s",
                    frac=round(achieved / FP4_PEAK_TFLOPS, 4))
    roof["traffic"] = traffic_for(src, workload)
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
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(inp, args.cpu_tokens or (T if decode else 8))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
