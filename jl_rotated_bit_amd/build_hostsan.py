"""Host-sanitizer build of the C ABI layer, for CPU-only checks.

    python -m jl_rotated_bit_amd.build_hostsan      # or build() from Python

Builds ``_build/hostsan/libqjl_hostsan.so``: the ABI and validation layer
(``qjl_abi.hip``) with AddressSanitizer and UndefinedBehaviorSanitizer on its
host code only (the device code is compiled as usual), the host table
generators (``sketch.cpp``, ``rotq_host.cpp``) with the same sanitizers (ROCm's
clang, whose runtimes match hipcc's host pass), and
the kernels' objects of the regular build.  ``tests/native/hostsan_driver.cpp``
is linked against it: the driver calls every entry point with invalid
arguments and every host table generator, and exits non-zero on a wrong
status; the sanitizers abort it on any memory or undefined-behaviour error.
No GPU is needed (no call in the driver reaches the HIP runtime).
"""

from __future__ import annotations

import os
import sys

from . import build as base

OUT = os.path.join(base.BUILD_DIR, "hostsan")
LIB = os.path.join(OUT, "libqjl_hostsan.so")
DRIVER_SRC = os.path.join(base.ROOT, "tests", "native", "hostsan_driver.cpp")
DRIVER = os.path.join(OUT, "hostsan_driver")

# Host-side sanitizers for hipcc: each -fsanitize= goes to the host pass only.
HIP_HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]
CLANG_SAN = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=all"]
# hipcc's host pass is ROCm's clang, so the other objects, the library and the
# driver use the same clang and its sanitizer runtimes
CLANGXX = "/opt/rocm/llvm/bin/clang++"
ROCM_LIB = "/opt/rocm/lib"


def build(verbose: bool = False) -> str:
    """Builds the regular library's kernel objects if needed, the sanitized
    ABI layer and the driver; returns the driver's path."""
    kernel_objs = [os.path.join(base.BUILD_DIR, src + ".o") for src in base.HIP_SOURCES if src != "qjl_abi.hip"]
    if not all(os.path.exists(o) for o in kernel_objs):
        base.build(verbose)      # kernel objects in _build/ (and libqjl.so)
    os.makedirs(OUT, exist_ok=True)
    abi_obj = os.path.join(OUT, "qjl_abi.hip.o")
    base._run([base.HIPCC, "-x", "hip", *base.HIP_FLAGS, "-O1", *HIP_HOST_SAN, "-c",
               os.path.join(base.CSRC, "qjl_abi.hip"), "-o", abi_obj])
    objs = [abi_obj]
    for src in base.HOST_SOURCES:
        obj = os.path.join(OUT, src + ".o")
        base._run([CLANGXX, *base.HOST_FLAGS, *CLANG_SAN, "-c", os.path.join(base.CSRC, src), "-o", obj])
        objs.append(obj)
    objs += kernel_objs
    base._run([CLANGXX, "-shared", *CLANG_SAN, *objs, f"-L{ROCM_LIB}", "-lamdhip64",
               f"-Wl,-rpath,{ROCM_LIB}", "-o", LIB])
    base._run([CLANGXX, "-std=c++17", "-O1", *CLANG_SAN, "-I", base.INCLUDE, "-I", base.CSRC, DRIVER_SRC,
               f"-L{OUT}", "-lqjl_hostsan", f"-Wl,-rpath,{OUT}", "-o", DRIVER])
    return DRIVER


if __name__ == "__main__":
    print(build(verbose=True), file=sys.stderr)
