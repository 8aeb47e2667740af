"""Build libmxq.so (all HIP sources under csrc/) for gfx950, in the package directory,
and the benchmark's streaming reference library libmxq_stream.so (csrc_bench/).

Usage: python -m mxfp4_microscaling_quantization_amd.build
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libmxq.so")
STREAM_LIB = os.path.join(PKG, "libmxq_stream.so")

HIP_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # exact rounding reasoning relies on IEEE fp32: no contraction, denormals kept,
    # correctly rounded division
    "-ffp-contract=off",
    "-fno-gpu-flush-denormals-to-zero",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Wall",
]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def _compile(srcs, out: str, verbose: bool) -> None:
    tmp = out + ".tmp"
    cmd = [hipcc(), *HIP_FLAGS, "-I", os.path.join(ROOT, "include"), *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)


def build(verbose: bool = True) -> str:
    _compile(sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip"))), LIB, verbose)
    _compile(sorted(glob.glob(os.path.join(PKG, "csrc_bench", "*.hip"))), STREAM_LIB, verbose)
    return LIB


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
