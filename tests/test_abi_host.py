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
TESTING_HEADER = os.path.join(ROOT, "jl_rotated_bit_amd", "csrc", "qjl_testing.h")

EINVAL, EUNSUP, EWS = 1, 2, 3


@pytest.fixture(scope="module")
def lib():
    return qjl.load()


def declared_functions(header=HEADER):
    text = open(header).read()
    return re.findall(r"QJL_API\s+[\w\s\*]+?\b(qjl_\w+)\s*\(", text)


def test_library_exports_every_declared_symbol(lib):
    names = declared_functions()
    testing = declared_functions(TESTING_HEADER)
    assert testing == ["qjl_testing_set_encode_small_max", "qjl_testing_set_rotq_margin"]
    for name in names + testing:
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", qjl.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert set(names) <= exported
    # nothing else with the qjl_ prefix leaks out: the public header's calls
    # and the test hooks of the internal header
    assert {n for n in exported if n.startswith("qjl_")} == set(names) | set(testing)
    # the public header holds no process-wide routing switch
    assert not any("small_max" in n for n in names)


def test_encode_small_max_hook_is_per_thread(lib):
    """The small-set encode limit (test hook): default 512, set and queried
    without a GPU, and a change on one thread leaves other threads at the
    default."""
    import threading
    f = lib.qjl_testing_set_encode_small_max
    start = f(-1)
    try:
        assert start == 512
        assert f(0) == 512
        assert f(-5) == 0
        assert f(100000) == 0
        seen = []
        t = threading.Thread(target=lambda: seen.append(f(-1)))
        t.start()
        t.join()
        assert seen == [512]
        assert f(-1) == 100000
    finally:
        f(start)


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


def dec_na(lib, q=A16, signs=A16, norms=A16, values=A16, B=1, Hq=4, Hkv=1, N=8, cap=8, d=128,
           m=256, scale=0.0, out=A16):
    return lib.qjl_decode_attention_noalloc(q, signs, norms, values, B, Hq, Hkv, N, cap, d, m, 1,
                                            ctypes.c_float(scale), out, None)


def test_decode_noalloc_validation(lib):
    """The allocation-free decode validates like qjl_decode_attention, and
    rejects plans whose split scratch exceeds the library's static array
    before any GPU call."""
    header = open(HEADER).read()
    assert "#define QJL_NOALLOC_SCRATCH_BYTES (4096u + (4u << 20))" in header
    assert qjl.NOALLOC_SCRATCH_BYTES == 4096 + (4 << 20)
    assert dec_na(lib, d=96) == EUNSUP
    assert dec_na(lib, Hq=6, Hkv=2) == EUNSUP
    assert dec_na(lib, N=9, cap=8) == EINVAL
    assert dec_na(lib, scale=-1.0) == EINVAL
    for name in ("q", "signs", "norms", "values", "out"):
        assert dec_na(lib, **{name: None}) == EINVAL
    assert dec_na(lib, out=A16 + 8) == EINVAL
    # 511 kv heads x 8 query heads each, two splits: 8176 partials of 130 floats
    big = dict(B=1, Hq=4088, Hkv=511, N=4096, cap=4096)
    need = lib.qjl_decode_workspace_bytes(1, 4088, 511, 4096, 128, 256)
    assert lib.qjl_decode_num_splits(1, 4088, 511, 4096, 128, 256) == 2
    assert need > qjl.NOALLOC_SCRATCH_BYTES
    assert dec_na(lib, **big) == EWS
    assert "more than the" in qjl.last_error()
    # the largest plans of the benchmark workloads fit
    for B, Hq, Hkv, N, m in [(1, 32, 8, 32768, 256), (1, 32, 8, 65600, 512), (8, 40, 40, 16384, 256),
                             (1, 2048, 256, 4096, 256)]:
        assert lib.qjl_decode_workspace_bytes(B, Hq, Hkv, N, 128, m) <= qjl.NOALLOC_SCRATCH_BYTES


def step(lib, q=A16, nk=A16, nv=A16, signs=A16, norms=A16, values=A16, B=1, Hq=4, Hkv=1, pos=7,
         cap=8, d=128, m=256, scale=0.0, out=A16, ws=A16, ws_bytes=1 << 30):
    return lib.qjl_decode_step(q, nk, nv, signs, norms, values, B, Hq, Hkv, pos, cap, d, m, 1,
                               ctypes.c_float(scale), out, ws, ws_bytes, None)


def test_decode_step_validation(lib):
    assert step(lib, pos=-1) == EINVAL
    assert step(lib, pos=8, cap=8) == EINVAL
    assert "outside" in qjl.last_error()
    assert step(lib, nk=None) == EINVAL
    assert step(lib, nv=None) == EINVAL
    assert step(lib, nk=A16 + 8) == EINVAL
    assert step(lib, nv=A16 + 2) == EINVAL
    assert step(lib, d=64) == EUNSUP
    assert step(lib, Hq=6, Hkv=2) == EUNSUP
    for name in ("q", "signs", "norms", "values", "out"):
        assert step(lib, **{name: None}) == EINVAL
    big = dict(B=1, Hq=32, Hkv=8, pos=32767, cap=32768)
    need = lib.qjl_decode_workspace_bytes(1, 32, 8, 32768, 128, 256)
    assert step(lib, ws=None, **big) == EWS
    assert step(lib, ws_bytes=need - 1, **big) == EWS


def base(lib, q=A16, k=A16, v=A16, B=1, Hq=4, Hkv=1, N=8, cap=8, d=128, scale=0.0, out=A16, ws=A16,
         ws_bytes=1 << 30):
    return lib.qjl_baseline_decode_attention_bf16(q, k, v, B, Hq, Hkv, N, cap, d, ctypes.c_float(scale),
                                                  out, ws, ws_bytes, None)


def test_baseline_validation(lib):
    assert base(lib, d=64) == EUNSUP
    assert base(lib, Hq=6, Hkv=2) == EUNSUP
    assert base(lib, Hq=6, Hkv=4) == EINVAL
    assert base(lib, N=9) == EINVAL
    assert base(lib, scale=-2.0) == EINVAL
    for name in ("q", "k", "v", "out"):
        assert base(lib, **{name: None}) == EINVAL
    assert base(lib, k=A16 + 2) == EINVAL
    big = dict(Hq=32, Hkv=8, N=32768, cap=32768)
    assert base(lib, ws=None, **big) == EWS


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


@pytest.mark.parametrize("seed", [42, 0, 7, 2 ** 64 - 5])
def test_host_rotation_is_bit_identical_to_oracle(seed):
    """The library's Householder QR and the oracle's numpy QR of the same
    seeded normals give the same fp32 rotation."""
    from oracle import turboquant as tq
    assert np.array_equal(qjl.rotation_host(seed, 128), tq.rotation(seed, 128))


@pytest.mark.parametrize("k", [1, 2, 3, 4])
def test_host_tq_codebook_is_bit_identical_to_oracle(k):
    """Two independent Lloyd-Max solvers (Gauss-Legendre quadrature here,
    the incomplete Beta function in the oracle) agree after rounding to the
    2^-20 grid."""
    from oracle import turboquant as tq
    assert np.array_equal(qjl.tq_codebook_host(128, k), tq.codebook(128, k)[0])


@pytest.mark.parametrize("level,bits", [(1, 4), (1, 3), (2, 2), (3, 2), (4, 2), (5, 2), (6, 2), (7, 2),
                                        (2, 3), (7, 1)])
def test_host_pq_codebook_matches_oracle(level, bits):
    """Tangent thresholds bit for bit; centroids exactly on the grid for
    levels >= 2, to fp32 rounding at level 1."""
    from oracle import polarquant as pq
    c, T = qjl.pq_codebook_host(level, bits)
    co, _, To = pq.level_codebook(level, bits)
    assert np.array_equal(T.astype(np.float64), To)
    if level == 1:
        assert np.allclose(c, co, rtol=2 ** -23, atol=0)
    else:
        assert np.array_equal(c.astype(np.float64), co)


def test_host_table_errors(lib):
    buf = np.zeros(64, np.float32)
    assert lib.qjl_rotation_host(1, 1, buf.ctypes.data) == EINVAL
    assert lib.qjl_rotation_host(1, 8, None) == EINVAL
    assert lib.qjl_tq_codebook_host(128, 0, buf.ctypes.data) == EINVAL
    assert lib.qjl_tq_codebook_host(128, 5, buf.ctypes.data) == EINVAL
    assert lib.qjl_pq_codebook_host(1, 1, buf.ctypes.data, buf.ctypes.data) == EINVAL
    assert lib.qjl_pq_codebook_host(0, 2, buf.ctypes.data, buf.ctypes.data) == EINVAL


def tqe(lib, keys=A16, B=1, H=1, n=4, d=128, k=2, codes=A16, bits=A16, norms=A16, gammas=A16, cap=8, pos=0):
    return lib.qjl_tq_encode_keys(keys, B, H, n, d, k, 7, codes, bits, norms, gammas, cap, pos, None)


def pqe(lib, keys=A16, B=1, H=1, n=4, d=128, codes=A16, radii=A16, cap=8, pos=0):
    return lib.qjl_pq_encode_keys(keys, B, H, n, d, 7, codes, radii, cap, pos, None)


def tqs(lib, q=A16, codes=A16, bits=A16, norms=A16, gammas=A16, B=1, Hq=4, Hkv=1, N=8, cap=8, d=128, k=2,
        out=A16, ws=A16, ws_bytes=1 << 20):
    return lib.qjl_tq_scores(q, codes, bits, norms, gammas, B, Hq, Hkv, N, cap, d, k, 7, out, ws, ws_bytes,
                             None)


def test_rotq_entry_point_validation(lib):
    """Argument errors of the rotate-then-quantize entry points are caught on
    the host, before any table upload or launch."""
    assert tqe(lib, d=64) == EUNSUP
    assert tqe(lib, k=0) == EUNSUP and tqe(lib, k=4) == EUNSUP
    assert tqe(lib, B=0) == EINVAL
    assert tqe(lib, n=5, pos=4, cap=8) == EINVAL
    assert "exceeds cap" in qjl.last_error()
    for name in ("keys", "codes", "bits", "norms", "gammas"):
        assert tqe(lib, **{name: None}) == EINVAL, name
    assert tqe(lib, keys=A16 + 4) == EINVAL            # keys need 16 B
    assert "misaligned" in qjl.last_error()
    assert tqe(lib, gammas=A16 + 2) == EINVAL
    assert tqe(lib, n=0, keys=None, codes=None, bits=None, norms=None, gammas=None) == 0
    assert pqe(lib, d=256) == EUNSUP
    assert pqe(lib, pos=-1) == EINVAL
    for name in ("keys", "codes", "radii"):
        assert pqe(lib, **{name: None}) == EINVAL, name
    assert pqe(lib, keys=A16 + 8) == EINVAL
    assert pqe(lib, radii=A16 + 1) == EINVAL
    assert pqe(lib, n=0, keys=None, codes=None, radii=None) == 0
    assert tqs(lib, k=5) == EUNSUP
    assert tqs(lib, Hq=6, Hkv=2) == EUNSUP             # G = 3
    assert tqs(lib, Hq=6, Hkv=4) == EINVAL             # not a multiple
    assert tqs(lib, N=0) == EINVAL and tqs(lib, N=9, cap=8) == EINVAL
    for name in ("q", "codes", "bits", "norms", "gammas", "out"):
        assert tqs(lib, **{name: None}) == EINVAL, name
    assert tqs(lib, out=A16 + 2) == EINVAL
    assert "misaligned" in qjl.last_error()
    assert tqs(lib, codes=A16 + 4) == EINVAL and tqs(lib, bits=A16 + 8) == EINVAL   # 16 B
    assert tqs(lib, B=70000, Hq=70000, Hkv=70000, N=1, cap=1) == EINVAL
    # the workspace holds 4096 bytes of prepared query per query head
    need = lib.qjl_tq_scores_workspace_bytes(2, 8, 128)
    assert need == 2 * 8 * 4096
    assert lib.qjl_tq_scores_workspace_bytes(0, 8, 128) == 0
    assert lib.qjl_tq_scores_workspace_bytes(2, 8, 64) == 0
    assert tqs(lib, B=2, Hq=8, Hkv=2, ws=None) == EWS
    assert tqs(lib, B=2, Hq=8, Hkv=2, ws=A16 + 16) == EWS
    assert tqs(lib, B=2, Hq=8, Hkv=2, ws_bytes=need - 4) == EWS
    assert "workspace" in qjl.last_error()
