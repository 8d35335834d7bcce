"""Build libfp8kv.so (the gfx950 HIP kernels + the C ABI) in-tree with hipcc."""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfp8kv.so")
# measurement kernels of the benchmark (a contiguous and a gathered read floor), not part of the path
FLOOR_SRC = os.path.join(PKG, "floor", "read_floor.hip")
FLOOR_LIB = os.path.join(PKG, "libfp8kv_floor.so")
# measurement build of the same sources with per-wave stage-1 timestamps (the
# benchmark's --timeline leg), not part of the path
TIMELINE_LIB = os.path.join(PKG, "libfp8kv_timeline.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # exact fp32 division (the quantizer's s = amax/448 and x/s) and IEEE denormals
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-gpu-flush-denormals-to-zero",
    "-fno-fast-math",
    # inputs are finite by contract and masking uses -inf, so fmaxf/fminf need
    # no NaN canonicalization (one VALU instruction per operand otherwise)
    "-Xarch_device", "-fno-honor-nans",
    # no packed-fp32 VALU instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False, extra=None) -> str:
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, *(extra or []), "-I", INCLUDE, "-I", CSRC, *sources(), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    build_floor(verbose)
    build_timeline(verbose)
    return LIB


def build_timeline(verbose: bool = False) -> str:
    tmp = TIMELINE_LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, "-DFP8KV_WAVE_TIMELINE", "-I", INCLUDE, "-I", CSRC, *sources(), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, TIMELINE_LIB)
    return TIMELINE_LIB


def build_floor(verbose: bool = False) -> str:
    tmp = FLOOR_LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, FLOOR_SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, FLOOR_LIB)
    return FLOOR_LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
