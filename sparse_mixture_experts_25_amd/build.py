"""Build libmoe.so (the HIP kernels and the C ABI) for gfx950 with hipcc, and
libmoe_peaks.so (the attainable-peak probe kernels of include/moe_peaks.h, a
measuring aid kept out of the layer library).

Usage: python -m sparse_mixture_experts_25_amd.build
Each translation unit is compiled to an object in _build/ (in parallel), then
linked into sparse_mixture_experts_25_amd/libmoe.so and libmoe_peaks.so.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libmoe.so")
PEAKS_LIB = os.path.join(HERE, "libmoe_peaks.so")
SOURCES = ["api.hip", "router.hip", "router_bwd.hip", "ec_route.hip", "balance.hip", "noisy.hip", "dispatch.hip",
           "gemm_bf16.hip", "gemm_f32.hip", "rows.hip"]
PEAKS_SOURCES = ["peaks.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 instructions are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
        if verbose and r.stderr.strip():
            print(r.stderr, file=sys.stderr)
        return obj

    with cf.ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(compile_one, SOURCES + PEAKS_SOURCES))
    for out, o in ((LIB, objs[:len(SOURCES)]), (PEAKS_LIB, objs[len(SOURCES):])):
        tmp = out + ".tmp"
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *o, "-o", tmp]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{r.stderr}")
        os.replace(tmp, out)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
