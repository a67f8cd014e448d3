"""Builds libqjl.so (HIP kernels + C ABI) for gfx950 with hipcc.

    python -m jl_rotated_bit_amd.build          # or build() from Python

Every HIP source is compiled with packed-fp32 instructions disabled
(``-Xclang -target-feature -Xclang -packed-fp32-ops``); the host-side sketch
generator is compiled with ``-ffp-contract=off`` so that its fp64 arithmetic
rounds exactly as written.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libqjl.so")

HIP_SOURCES = ["qjl_abi.hip", "encode.hip", "decode.hip", "rotq.hip"]
# Per-source extras.  NaN inputs are outside the contract of both kernels, and
# without NaNs a min/max needs no operand canonicalization (which would
# otherwise cost an instruction per operand and block folding cross-lane
# moves into the max).
HIP_EXTRA = {"decode.hip": ["-fno-honor-nans"], "encode.hip": ["-fno-honor-nans"],
             # every operation that feeds a code decision rounds as written
             "rotq.hip": ["-ffp-contract=off"]}
HOST_SOURCES = ["sketch.cpp", "rotq_host.cpp"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]
HOST_FLAGS = ["-O2", "-fPIC", "-std=c++17", "-Wall", "-ffp-contract=off", "-I", INCLUDE, "-I", CSRC]


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature
    err = "\n".join(line for line in res.stderr.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in line)
    if res.returncode != 0:
        raise RuntimeError(f"build step failed ({res.returncode}): {' '.join(cmd)}\n{err}")
    return err


def build(verbose: bool = False) -> str:
    """Compiles every source and links libqjl.so; returns the library path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        jobs.append([HIPCC, "-x", "hip", *HIP_FLAGS, *HIP_EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj])
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        jobs.append(["g++", *HOST_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    with cf.ThreadPoolExecutor(max_workers=min(4, len(jobs))) as ex:
        for err in ex.map(_run, jobs):
            if verbose and err.strip():
                print(err, file=sys.stderr)
    objs = [j[-1] for j in jobs]
    tmp = LIB + ".tmp"
    err = _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
