"""Build libwqd.so (HIP, gfx950) in-tree with hipcc.

Usage: python -m weight_quantized_decode_block_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libwqd.so")
# bench-only helper (a plain read of a buffer: the read ceiling bench.py reports)
BENCH_LIB = os.path.join(PKG, "libwqd_bench.so")
SOURCES = ["api.cpp", "pack.cpp", "q2_0_mfma.hip", "q2_0_valu.hip", "w8a16_gemm_m16.hip", "w8a16_gemv.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off",
    # packed fp32 VALU forms are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # kernel arguments preloaded into SGPRs at dispatch (no scalar load before the first instruction)
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    "-Wall", "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.sep not in cand or os.path.exists(cand)):
            return cand
    return "hipcc"


def build(verbose: bool = False) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), "-x", "hip", *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    tmp = BENCH_LIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-x", "hip", os.path.join(CSRC, "bench_read.hip"), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, BENCH_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
