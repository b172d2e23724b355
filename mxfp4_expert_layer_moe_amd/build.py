"""Build libmoe_mxfp4.so (the layer) and libmoe_peaks.so (the ceiling probes), gfx950 only,
in-tree with hipcc.

    python -m mxfp4_expert_layer_moe_amd.build        # or build() from Python
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIBDIR = os.path.join(HERE, "_lib")
LIB = os.path.join(LIBDIR, "libmoe_mxfp4.so")
PEAKS_LIB = os.path.join(LIBDIR, "libmoe_peaks.so")
PEAKS_SOURCES = ["peaks.hip"]
ROOT = os.path.dirname(HERE)

SOURCES = ["api.cpp", "route.hip", "permute.hip", "pack.hip", "gemm.hip", "gemm_prefill.hip", "gemm_dense.hip", "combine.hip",
           "norm.hip"]
ARCH = "gfx950"
# packed-fp32 instructions are disabled: plain fp32 VALU only
HIPFLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-function"]
# per-source extras: the prefill GEMM's 45-step k-loop is unrolled whole (its ring slots and scale
# byte selectors must be compile-time constants), past LLVM's default pragma-unroll size limit
EXTRA = {"gemm_prefill.hip": ["-mllvm", "-pragma-unroll-threshold=100000"]}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the MI355X library needs ROCm's hipcc")


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950 and link both shared libraries; returns the layer's path."""
    os.makedirs(LIBDIR, exist_ok=True)
    cc = hipcc()
    objs, procs = [], []
    for src in SOURCES + PEAKS_SOURCES:
        path = os.path.join(CSRC, src)
        obj = os.path.join(LIBDIR, os.path.splitext(src)[0] + ".o")
        cmd = [cc, *HIPFLAGS, *EXTRA.get(src, []), "-x", "hip", "-c", path, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
        objs.append(obj)
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        msgs = "\n".join(l for l in out.splitlines() if "packed-fp32-ops" not in l)
        if p.returncode != 0:
            failed.append(src)
            print(msgs, file=sys.stderr)
        elif verbose and msgs.strip():
            print(msgs)
    if failed:
        raise RuntimeError(f"hipcc failed on {failed}")
    n = len(SOURCES)
    for lib, lib_objs in ((LIB, objs[:n]), (PEAKS_LIB, objs[n:])):
        tmp = lib + ".tmp"
        cmd = [cc, "-shared", f"--offload-arch={ARCH}", "-fPIC", *lib_objs, "-o", tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
