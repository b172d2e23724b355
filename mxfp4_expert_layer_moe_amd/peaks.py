"""Python binding of libmoe_peaks.so: probes of the MI355X matrix-instruction rates and streaming
read bandwidth that the benchmark quotes the layer's roofline fractions against
(include/moe_peaks.h).  Argument marshalling and HIP-event timing only."""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_lib", "libmoe_peaks.so")
FP6_FP4, FP4_FP4, FP8_FP4, BF16 = range(4)
NAMES = {FP6_FP4: "fp6xfp4", FP4_FP4: "fp4xfp4", FP8_FP4: "fp8xfp4", BF16: "bf16"}
EXPORTS = ("moe_peak_mfma_flops", "moe_peak_mfma", "moe_peak_stream_read")

_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m mxfp4_expert_layer_moe_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.moe_peak_mfma_flops.restype = ctypes.c_double
        L.moe_peak_mfma_flops.argtypes = [ctypes.c_int, ctypes.c_int32, ctypes.c_int32]
        L.moe_peak_mfma.restype = ctypes.c_int
        L.moe_peak_mfma.argtypes = [ctypes.c_int, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
        L.moe_peak_stream_read.restype = ctypes.c_int
        L.moe_peak_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int32,
                                           ctypes.c_void_p, ctypes.c_void_p]
        _lib = L
    return _lib


def _timed(launch, reps: int) -> float:
    """Mean seconds per launch of `reps` back-to-back launches on torch's current stream."""
    import torch
    s = torch.cuda.current_stream()
    launch(s.cuda_stream)                      # warm
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(s)
    for _ in range(reps):
        launch(s.cuda_stream)
    b.record(s)
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e-3 / reps


def mfma_rate(fmt: int, workgroups: int = 2048, iters: int = 2000, reps: int = 5) -> float:
    """Sustained matrix FLOP/s of one operand-format pair, all compute units busy."""
    import torch
    sink = torch.empty(workgroups * 256, dtype=torch.float32, device="cuda")

    def go(st):
        if lib().moe_peak_mfma(fmt, workgroups, iters, sink.data_ptr(), st) != 0:
            raise RuntimeError("moe_peak_mfma failed")
    t = _timed(go, reps)
    return lib().moe_peak_mfma_flops(fmt, workgroups, iters) / t


def stream_read_rate(mib: int = 2048, nontemporal: bool = True, workgroups: int = 4096, reps: int = 5) -> float:
    """Sustained bytes/s of a streaming read of `mib` MiB (well past the 256 MB last-level cache)."""
    import torch
    n = mib << 20
    buf = torch.ones(n, dtype=torch.uint8, device="cuda")
    sink = torch.empty(workgroups * 256, dtype=torch.int32, device="cuda")

    def go(st):
        if lib().moe_peak_stream_read(buf.data_ptr(), n, int(nontemporal), workgroups, sink.data_ptr(), st) != 0:
            raise RuntimeError("moe_peak_stream_read failed")
    t = _timed(go, reps)
    del buf
    return n / t


def measure_all() -> dict:
    """Every probe once: matrix rates (TFLOP/s) per format and read bandwidth (GB/s)."""
    out = {f"mfma_{NAMES[f]}_TFLOP_per_s": round(mfma_rate(f) / 1e12, 1) for f in (FP6_FP4, FP4_FP4, FP8_FP4, BF16)}
    out["stream_read_nt_GB_per_s"] = round(stream_read_rate(nontemporal=True) / 1e9, 1)
    out["stream_read_GB_per_s"] = round(stream_read_rate(nontemporal=False) / 1e9, 1)
    return out


def main(argv: list | None = None) -> int:
    """`python -m mxfp4_expert_layer_moe_amd.peaks [OUT_JSON]`: every probe once, as one JSON object
    with the work per launch beside each rate, so a kernel trace of the same run (average launch
    duration x rate = work per launch) can be checked against it."""
    import json
    import sys
    argv = sys.argv[1:] if argv is None else argv
    rec = measure_all()
    rec["work_per_launch"] = {f"mfma_{NAMES[f]}_flop": lib().moe_peak_mfma_flops(f, 2048, 2000)
                              for f in (FP6_FP4, FP4_FP4, FP8_FP4, BF16)}
    rec["work_per_launch"]["stream_read_bytes"] = 2048 << 20
    rec["launches_per_probe"] = 6            # one warm launch, then five timed back to back
    line = json.dumps(rec)
    print(line, flush=True)
    if argv:
        with open(argv[0], "w") as f:
            f.write(line + "\n")
    return 0


if __name__ == "__main__":
    raise SystemExit(main())
