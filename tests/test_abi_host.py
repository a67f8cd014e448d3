"""C ABI checks that need no GPU: exports, host sketch, validation, plans.

Every error path exercised here returns before any HIP call, so these run on
a machine without a GPU.
"""

import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import oracle
from jl_rotated_bit_amd import qjl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qjl.h")

EINVAL, EUNSUP, EWS = 1, 2, 3


@pytest.fixture(scope="module")
def lib():
    return qjl.load()


def declared_functions():
    text = open(HEADER).read()
    return re.findall(r"QJL_API\s+[\w\s\*]+?\b(qjl_\w+)\s*\(", text)


def test_library_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) == 9, names
    for name in names:
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", qjl.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert set(names) <= exported
    # nothing else with the qjl_ prefix leaks out
    assert {n for n in exported if n.startswith("qjl_")} == set(names)


def test_encode_small_max_knob(lib):
    """The small-set encode limit: default 512, set and query without a GPU."""
    lib.qjl_set_encode_small_max.restype = ctypes.c_int32
    lib.qjl_set_encode_small_max.argtypes = [ctypes.c_int32]
    start = lib.qjl_set_encode_small_max(-1)
    try:
        assert start == 512
        assert lib.qjl_set_encode_small_max(0) == 512
        assert lib.qjl_set_encode_small_max(-5) == 0
        assert lib.qjl_set_encode_small_max(100000) == 0
        assert lib.qjl_set_encode_small_max(-1) == 100000
    finally:
        lib.qjl_set_encode_small_max(start)


def test_library_targets_gfx950_only():
    """The embedded offload bundle names the gfx950 target and no other GPU."""
    blob = open(qjl.LIB_PATH, "rb").read()
    targets = set(re.findall(rb"amdgcn-amd-amdhsa--(gfx[0-9a-f]+)", blob))
    assert targets == {b"gfx950"}, targets


def test_abi_version(lib):
    assert lib.qjl_abi_version() == qjl.ABI_VERSION


@pytest.mark.parametrize("seed,d,m", [(42, 128, 256), (42, 128, 512), (0, 1, 1), (3, 7, 9),
                                      (2 ** 64 - 1, 128, 256), (12345678901234567, 64, 96)])
def test_host_sketch_is_bit_identical_to_oracle(seed, d, m):
    assert np.array_equal(qjl.sketch_host(seed, d, m), oracle.sketch_bf16_bits(seed, d, m))


def test_host_sketch_errors(lib):
    assert lib.qjl_sketch_host(1, 0, 8, None) == EINVAL
    buf = np.zeros(8, np.uint16)
    assert lib.qjl_sketch_host(1, 0, 8, buf.ctypes.data) == EINVAL
    assert lib.qjl_sketch_host(1, 8, -1, buf.ctypes.data) == EINVAL
    assert lib.qjl_sketch_host(1, 1 << 14, 1 << 13, buf.ctypes.data) == EINVAL
    assert "too large" in qjl.last_error()


A16 = 1 << 20  # a fake, 16-byte aligned address; never dereferenced


def enc(lib, keys=A16, B=1, H=1, n=4, d=128, m=256, signs=A16, norms=A16, cap=8, pos=0):
    return lib.qjl_encode_keys(keys, B, H, n, d, m, 1, signs, norms, cap, pos, None)


def test_encode_validation(lib):
    assert enc(lib, d=64) == EUNSUP
    assert enc(lib, m=128) == EUNSUP
    assert enc(lib, m=384) == EUNSUP
    assert enc(lib, B=0) == EINVAL
    assert enc(lib, H=-1) == EINVAL
    assert enc(lib, n=-1) == EINVAL
    assert enc(lib, cap=0) == EINVAL
    assert enc(lib, pos=-1) == EINVAL
    assert enc(lib, n=5, pos=4, cap=8) == EINVAL
    assert "exceeds cap" in qjl.last_error()
    # more than 2^31 - 1 keys in one call (rejected before any pointer is used)
    assert enc(lib, B=2, H=2, n=1 << 29, cap=1 << 29) == EINVAL
    assert "2^31" in qjl.last_error()
    assert enc(lib, keys=None) == EINVAL
    assert enc(lib, signs=None) == EINVAL
    assert enc(lib, norms=None) == EINVAL
    assert enc(lib, keys=A16 + 8) == EINVAL
    assert enc(lib, signs=A16 + 4) == EINVAL
    assert enc(lib, norms=A16 + 2) == EINVAL
    assert "misaligned" in qjl.last_error()
    # n == 0 is a successful no-op, even with NULL buffers
    assert enc(lib, n=0, keys=None, signs=None, norms=None) == 0
    assert qjl.last_error() == ""


def dec(lib, q=A16, signs=A16, norms=A16, values=A16, B=1, Hq=4, Hkv=1, N=8, cap=8, d=128,
        m=256, scale=0.0, out=A16, ws=A16, ws_bytes=1 << 30):
    return lib.qjl_decode_attention(q, signs, norms, values, B, Hq, Hkv, N, cap, d, m, 1,
                                    ctypes.c_float(scale), out, ws, ws_bytes, None)


def test_decode_validation(lib):
    assert dec(lib, d=96) == EUNSUP
    assert dec(lib, m=1024) == EUNSUP
    assert dec(lib, Hq=6, Hkv=2) == EUNSUP          # G = 3
    assert dec(lib, Hq=32, Hkv=2) == EUNSUP         # G = 16
    assert dec(lib, Hq=6, Hkv=4) == EINVAL          # not a multiple
    assert dec(lib, N=0) == EINVAL
    assert dec(lib, N=9, cap=8) == EINVAL
    assert dec(lib, B=0) == EINVAL
    assert dec(lib, scale=-1.0) == EINVAL
    assert dec(lib, scale=float("inf")) == EINVAL
    assert dec(lib, scale=float("nan")) == EINVAL
    for name in ("q", "signs", "norms", "values", "out"):
        assert dec(lib, **{name: None}) == EINVAL
    assert dec(lib, q=A16 + 4) == EINVAL
    assert dec(lib, values=A16 + 2) == EINVAL
    assert dec(lib, out=A16 + 8) == EINVAL
    # a call that needs several splits checks its workspace
    big = dict(B=1, Hq=32, Hkv=8, N=32768, cap=32768)
    need = lib.qjl_decode_workspace_bytes(1, 32, 8, 32768, 128, 256)
    assert need > 0
    assert dec(lib, ws=None, **big) == EWS
    assert dec(lib, ws=A16 + 16, **big) == EWS
    assert dec(lib, ws_bytes=need - 1, **big) == EWS


def test_decode_plan_properties(lib):
    for B, Hq, Hkv, N, m in [(1, 8, 1, 4096, 256), (1, 32, 8, 32768, 256), (1, 32, 8, 65600, 512),
                             (8, 40, 40, 16384, 256), (1, 4, 4, 1, 256), (2, 16, 2, 777, 512),
                             (1, 8, 8, 10 ** 6, 256)]:
        ns = lib.qjl_decode_num_splits(B, Hq, Hkv, N, 128, m)
        assert 1 <= ns <= 1024
        assert ns <= max(1, -(-N // 256))
        ws = lib.qjl_decode_workspace_bytes(B, Hq, Hkv, N, 128, m)
        assert ws >= B * Hq * ns * 130 * 4
    assert lib.qjl_decode_num_splits(1, 8, 3, 100, 128, 256) == 0
    assert lib.qjl_decode_workspace_bytes(1, 8, 8, 0, 128, 256) == 0
