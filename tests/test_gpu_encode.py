"""GPU parity of qjl_encode_keys against the oracle (bit-exact signs).

Sign words must match the oracle bit for bit (every bit is the sign of the
exact projection, sign(0) = +1); norms agree within 1e-5 relative (the fp32
sum of 128 exact squares carries at most ~128 * 2^-24 relative error).
"""

import numpy as np
import pytest

import oracle
from jl_rotated_bit_amd import workloads as wl

from .gpu_util import SENTINEL, cached_workload, gpu_encode, host_u32, oracle_encode, say

pytestmark = pytest.mark.gpu

SEED = 42
NORM_RTOL = 1e-5


def check_encode(qjl, keys, m, seed=SEED, cap=None, pos=0, label="", ref=None):
    """GPU encode of every key against the oracle: all sign words bit for
    bit, all norms within NORM_RTOL, rows outside [pos, pos + n) untouched.
    ``ref`` = (words [R][m/32], norms [R]) when the oracle's encode of these
    keys is already at hand."""
    B, H, n, d = keys.shape
    cap = n + pos if cap is None else cap
    say("encode", label, (B, H, n, d), "m", m, "cap", cap, "pos", pos)
    signs, norms = gpu_encode(qjl, keys, m, seed, cap=cap, pos=pos)
    got_w = host_u32(signs)
    got_n = norms.cpu().numpy()
    flat = keys.reshape(-1, d)
    rows = np.arange(flat.shape[0])
    if ref is None:
        ref = oracle_encode(flat, oracle.sketch(seed, d, m))
    ref_w, ref_n = ref
    bh, t = rows // n, rows % n
    gw = got_w[bh // H, bh % H, pos + t]
    gn = got_n[bh // H, bh % H, pos + t]
    bad = np.nonzero((gw != ref_w).any(axis=1))[0]
    assert bad.size == 0, f"{bad.size} keys with wrong bits, first row {rows[bad[0]]}"
    rel = np.abs(gn.astype(np.float64) - ref_n) / np.maximum(np.abs(ref_n.astype(np.float64)), 1e-300)
    zero = ref_n == 0
    assert np.all(gn[zero] == 0)
    assert rel[~zero].max(initial=0.0) <= NORM_RTOL
    # rows outside [pos, pos + n) are untouched
    mask = np.ones(cap, bool)
    mask[pos:pos + n] = False
    assert np.all(got_w[:, :, mask] == np.uint32(SENTINEL))
    assert np.all(np.isnan(got_n[:, :, mask]))
    return got_w, got_n


@pytest.fixture(params=["tile", "small"])
def enc_path(request, gpu_lib):
    """Runs a test through one encode kernel: the tile kernel (limit 0) or
    the small-set kernel (no limit), whatever the size."""
    prev = gpu_lib.testing_set_encode_small_max(0 if request.param == "tile" else 2 ** 31 - 1)
    yield request.param
    gpu_lib.testing_set_encode_small_max(prev)


def test_small_workload_keys(gpu_lib, enc_path):
    w = wl.small()
    check_encode(gpu_lib, w.keys, w.m, label="small")


@pytest.mark.parametrize("m", [256, 512])
@pytest.mark.parametrize("B,H,n,cap,pos", [(1, 1, 1, 1, 0), (1, 1, 1, 9, 7), (2, 3, 31, 40, 5),
                                            (1, 2, 33, 33, 0), (3, 1, 95, 200, 100),
                                            (1, 1, 1000, 1003, 3)])
def test_ragged_shapes_and_offsets(gpu_lib, enc_path, m, B, H, n, cap, pos):
    rng = np.random.default_rng(B * 1000 + H * 100 + n + m)
    keys = wl.gaussian_keys(rng, B * H * n).reshape(B, H, n, 128)
    check_encode(gpu_lib, keys, m, cap=cap, pos=pos, label="ragged")


def adversarial_keys(S, rng):
    """Keys whose projections are exactly zero or within float error of zero."""
    d, m = S.shape
    rows = []
    rows.append(np.zeros(d))
    negzero = np.zeros(d)
    rows.append(negzero)
    for j in rng.choice(d, 12, replace=False):
        k = np.zeros(d)
        k[j] = 2.0 ** int(rng.integers(-20, 20))
        rows.append(k)
        rows.append(-k)
    for _ in range(48):                        # exact cancellations at one coordinate
        a, b = rng.choice(d, 2, replace=False)
        i = int(rng.integers(m))
        k = np.zeros(d)
        k[a], k[b] = S[b, i], -S[a, i]
        rows.append(k)
    for n in range(48):                        # huge cancelling pair + tiny decider
        a, b, c = rng.choice(d, 3, replace=False)
        i = int(rng.integers(m))
        k = np.zeros(d)
        k[a], k[b] = S[b, i] * 2.0 ** 40, -S[a, i] * 2.0 ** 40
        k[c] = (1 if n % 2 else -1) * 2.0 ** -40
        rows.append(k)
    for _ in range(48):                        # dense cancellation: k and a tweak of -k
        g = rng.standard_normal(d)
        i = int(rng.integers(m))
        # make coordinate i's projection tiny: remove its component along S[:, i]
        s = S[:, i]
        k = g - (g @ s) / (s @ s) * s
        rows.append(k)
    for p in (-120, -100, -70, 30, 60, 100):   # very small and very large keys
        rows.append(rng.standard_normal(d) * 2.0 ** p)
    sub = np.zeros(d)                          # bf16 subnormal entries
    sub[rng.choice(d, 20, replace=False)] = rng.integers(1, 127, 20) * 2.0 ** -133
    rows.append(sub)
    mix = rng.standard_normal(d)
    mix[:10] = rng.integers(1, 127, 10) * 2.0 ** -133
    rows.append(mix)
    K = oracle.float64_to_bf16_bits(np.array(rows))
    K[1] = 0x8000                              # -0.0 everywhere
    return K


@pytest.mark.parametrize("m", [256, 512])
def test_adversarial_keys(gpu_lib, enc_path, m):
    S = oracle.sketch(SEED, 128, m)
    K = adversarial_keys(S, np.random.default_rng(m))
    got_w, _ = check_encode(gpu_lib, K.reshape(1, 1, -1, 128), m, label="adversarial")
    # the exact-zero rows really produced all-ones words
    assert np.all(got_w[0, 0, 0] == 0xFFFFFFFF) and np.all(got_w[0, 0, 1] == 0xFFFFFFFF)


@pytest.mark.parametrize("m", [256, 512])
def test_certification_queue_fills_and_overflows(gpu_lib, enc_path, m):
    """Keys scaled by 2^60 have every bit re-derived exactly (their fp32
    squared norm leaves the range the error bound is proved for), and each
    such key queues one word per wave and half.  Blocks 0 and 1 queue 96
    words per wave and block 2 pushes past the 112-entry queue, so the
    queued words are decided after the loop and the rest of the tile by
    the re-run path."""
    rng = np.random.default_rng(90 + m)
    n = 300
    scale = np.ones(n)
    scale[:16] = 2.0 ** 60            # block 0: 16 keys -> 32 queued words per wave
    scale[32:64] = 2.0 ** 60          # block 1: 64 more words
    scale[64::3] = 2.0 ** 60
    K = oracle.float64_to_bf16_bits(oracle.bf16_bits_to_float64(wl.gaussian_keys(rng, n)) * scale[:, None])
    check_encode(gpu_lib, K.reshape(1, 1, n, 128), m, label="queue overflow")


@pytest.mark.parametrize("m", [256, 512])
def test_zero_padding_rows(gpu_lib, enc_path, m):
    """All-(+/-)zero rows (padding) mixed with ordinary keys, in runs and
    one by one: every bit of a zero row is 1 and its norm is 0, and the
    ordinary rows around them are unaffected."""
    rng = np.random.default_rng(300 + m)
    B, H, n = 1, 1, 1500
    K = wl.gaussian_keys(rng, B * H * n).reshape(B, H, n, 128)
    K[:, :, ::3] = 0                  # every third row
    K[0, 0, 300:900] = 0              # a long run, spanning several 128-row tiles
    K[0, 0, 7] = 0x8000               # -0.0 everywhere
    got_w, got_n = check_encode(gpu_lib, K, m, label="zero padding")
    assert np.all(got_w[0, 0, 300:900] == 0xFFFFFFFF) and np.all(got_n[0, 0, 300:900] == 0)
    assert np.all(got_w[0, 0, 7] == 0xFFFFFFFF)


def test_matches_exact_rationals_on_cancellations(gpu_lib, enc_path):
    """Brute force with Fractions on rows built to cancel exactly or almost."""
    S = oracle.sketch(SEED, 128, 256)
    rng = np.random.default_rng(77)
    K = adversarial_keys(S, rng)[:40]
    signs, _ = gpu_encode(gpu_lib, K.reshape(1, 1, -1, 128), 256, SEED)
    bits = oracle.unpack_signs(host_u32(signs)[0, 0], 256)
    # exact rationals on a subset of coordinates (full rows are slow in Fractions)
    cols = rng.choice(256, 24, replace=False)
    brute = oracle.exact_sign_fraction(K, S[:, cols])
    assert np.array_equal(bits[:, cols], brute)


def test_prefill_workload_full(gpu_lib):
    w = wl.prefill()
    check_encode(gpu_lib, w.keys, w.m, label="prefill 16x8x8192")


def test_gqa32k_keys_full(gpu_lib):
    w = wl.gqa32k()
    check_encode(gpu_lib, w.keys, w.m, label="gqa32k keys")


def test_long64k_keys_m512(gpu_lib):
    w = wl.long64k()
    check_encode(gpu_lib, w.keys, w.m, label="long64k keys (m=512)")


def test_mha16k_keys_full(gpu_lib):
    """All 5 242 880 keys of the 40-head, batch-8, 16K cache (five launches)."""
    w, ref_w, ref_n = cached_workload("mha16k")
    check_encode(gpu_lib, w.keys, w.m, label="mha16k keys (all rows)",
                 ref=(ref_w.reshape(-1, w.m // 32), ref_n.reshape(-1)))


def test_large_ragged_uneven_split(gpu_lib):
    """Enough tiles that the first workgroup of each CU takes a larger share,
    with a tile count that is no multiple of the grid and a per-head row
    count that is no multiple of the 128-row tile (tiles cross heads);
    every row."""
    rng = np.random.default_rng(11)
    B, H, n = 1, 8, 32768 + 77
    keys = wl.gaussian_keys(rng, B * H * n).reshape(B, H, n, 128)
    check_encode(gpu_lib, keys, 256, cap=n + 5, pos=3, label="large ragged")


def launch_starts(R, m, cus=256):
    """First rows of the encode launches after the first one on a device
    with ``cus`` compute units: about 16 tiles of 128 keys per workgroup (two
    workgroups per unit at m = 256, one at m = 512), up to 1/8 more before a
    second launch is taken, and the tiles divided evenly among launches."""
    tiles = -(-R // 128)
    cap_tiles = 16 * cus * (2 if m == 256 else 1) * 9 // 8
    launches = -(-tiles // cap_tiles)
    chunk = -(-tiles // launches) * 128
    return list(range(chunk, R, chunk))


@pytest.mark.parametrize("m,H,n", [(256, 37, 32768 + 5), (512, 9, 65536 + 3), (512, 8, 65536 + 1)])
def test_across_launch_chunks(gpu_lib, m, H, n):
    """Key sets around the size one launch takes, with a per-head row count
    that is no multiple of the tile: two launches at m = 256 (1.2 M keys) and
    at m = 512 (590 K keys), and one launch in which a workgroup takes a
    seventeenth tile (65537 tokens of 8 heads at m = 512).  Every row."""
    rng = np.random.default_rng(13 + m + H)
    keys = wl.gaussian_keys(rng, H * n).reshape(1, H, n, 128)
    say("launch boundaries at rows", launch_starts(H * n, m))
    check_encode(gpu_lib, keys, m, label="across launch chunks")


def test_launch_starts_rule():
    """The launch-boundary rule the chunk test aims at (host arithmetic)."""
    assert launch_starts(8 * 65537, 512) == []
    assert launch_starts(9 * 65539, 512) == [2305 * 128]
    assert launch_starts(37 * 32773, 256) == [4737 * 128]
    assert launch_starts(40 * 8 * 16384, 256) == [k * 8192 * 128 for k in range(1, 5)]


def test_other_seed(gpu_lib, enc_path):
    rng = np.random.default_rng(3)
    keys = wl.gaussian_keys(rng, 4000).reshape(1, 4, 1000, 128)
    check_encode(gpu_lib, keys, 256, seed=2 ** 64 - 3, label="seed 2^64-3")
    check_encode(gpu_lib, keys, 512, seed=0, label="seed 0")


@pytest.mark.parametrize("m", [256, 512])
def test_default_limit_both_sides(gpu_lib, m):
    """With the default limit (512 keys), calls of 512 keys run the small-set
    kernel and calls of 513 the tile kernel; both match the oracle, and the
    one-token append of a decode step (one key per kv head) is exact."""
    assert gpu_lib.testing_set_encode_small_max(-1) == 512
    rng = np.random.default_rng(600 + m)
    for B, H, n in [(1, 4, 128), (1, 1, 513), (2, 8, 1)]:
        keys = wl.gaussian_keys(rng, B * H * n).reshape(B, H, n, 128)
        check_encode(gpu_lib, keys, m, cap=n + 9, pos=9, label=f"default limit {B * H * n} keys")

