"""Compile the HIP sources into weight_only_int4_group_amd/libq4.so for gfx950.

Usage: python -m weight_only_int4_group_amd.build   (or build() from Python).
Runs hipcc on the CPU; no GPU is needed to build.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libq4.so")
# Measurement helper for bench.py (a plain streaming read), kept out of the product library.
BENCH_LIB = os.path.join(PKG, "libq4_bench.so")
BENCH_SOURCES = [os.path.join("bench", "stream_read.hip")]

ARCH = "gfx950"
COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # hipcc fuses plain float code into packed-fp32 instructions by itself; keep them off.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-gpu-rdc", "-Wno-unused-result",
]
# The quantizer's bit-exact arithmetic must not be re-associated or contracted.
SOURCES = {
    "quantize.hip": ["-ffp-contract=off", "-fno-fast-math"],
    "gemv.hip": [],
    "gemm.hip": [],
    "prefill.hip": [],
    "decode.hip": [],
    "dequant.hip": [],
    "gemv8.hip": [],
    # the codes' IEEE quotient must not be contracted or re-associated
    "gptq.hip": ["-fno-fast-math"],
    # the activation scaling's IEEE division and product must not be contracted or re-associated
    "awq.hip": ["-ffp-contract=off", "-fno-fast-math"],
    "awq_static.hip": [],
    "q4_abi.cpp": [],
}


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the q4 library)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = [l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l]
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n" + "\n".join(errs))
    if verbose and errs:
        print("\n".join(errs), flush=True)


def build(verbose: bool = False, jobs: int = 4) -> str:
    """Compile every source, link libq4.so and the measurement helper libq4_bench.so; returns
    the path of libq4.so."""
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)

    def compile_one(item):
        name, extra = item
        obj = os.path.join(BUILD, name + ".o")
        _run([hipcc, *COMMON, *extra, "-c", os.path.join(CSRC, name), "-o", obj], verbose)
        return obj

    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(compile_one, SOURCES.items()))
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    bench_objs = []
    for src in BENCH_SOURCES:
        obj = os.path.join(BUILD, os.path.basename(src) + ".o")
        _run([hipcc, *COMMON, "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        bench_objs.append(obj)
    tmp = BENCH_LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *bench_objs], verbose)
    os.replace(tmp, BENCH_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
