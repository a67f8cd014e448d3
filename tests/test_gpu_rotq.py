"""GPU parity of the rotate-then-quantize encoders and TurboQuant's scores.

Codes, sign bits, norms, residual norms and radii are defined exactly (the
fp32 rounding of the exact rotation, then fixed-order IEEE operations), so
all of them must equal the oracle's bit for bit.  Scores are fp32 sums and
are compared per (batch, query head) row within 1e-5 of the row's scale (the
score arithmetic: fp32 rotation and sketch of q with ~1e-6 relative error,
fp32 sums of 128 terms).
"""

import numpy as np
import pytest

import oracle
from oracle import polarquant as opq
from oracle import turboquant as otq
from jl_rotated_bit_amd import workloads as wl

from .gpu_util import SENTINEL, dev_f32, dev_u16, dev_u32, host_u32, say

pytestmark = pytest.mark.gpu

SEED = 42
D = 128


def threaded(fn, keys, chunk=4096):
    """fn(keys) over row chunks on host threads, outputs joined in order."""
    import os
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    starts = list(range(0, keys.shape[0], chunk))
    if len(starts) == 1:
        return fn(keys)
    with threadpool_limits(1), ThreadPoolExecutor(max(1, min(16, len(os.sched_getaffinity(0))))) as ex:
        parts = list(ex.map(lambda c: fn(keys[c:c + chunk]), starts))
    return tuple(np.concatenate([p[i] for p in parts]) for i in range(len(parts[0])))


def special_keys(rng):
    rows = [np.zeros(D), np.zeros(D)]
    for j in (0, 5, 127):
        e = np.zeros(D)
        e[j] = 1.0
        rows += [e, -3.0 * e]
    for p in (-120, -60, 40, 100):
        rows.append(rng.standard_normal(D) * 2.0 ** p)
    sub = np.zeros(D)
    sub[rng.choice(D, 16, replace=False)] = rng.integers(1, 127, 16) * 2.0 ** -133
    rows.append(sub)
    ints = rng.integers(-3, 4, (8, D)).astype(np.float64)   # many exact ties and cancellations
    rows += list(ints)
    K = oracle.float64_to_bf16_bits(np.array(rows))
    K[1] = 0x8000
    return K


def gpu_tq(qjl, keys, k, cap=None, pos=0, seed=SEED):
    import torch
    B, H, n, d = keys.shape
    cap = n + pos if cap is None else cap
    codes = torch.full((B, H, cap, d * k // 32), SENTINEL, dtype=torch.int32, device="cuda")
    bits = torch.full((B, H, cap, d // 32), SENTINEL, dtype=torch.int32, device="cuda")
    norms = torch.full((B, H, cap), float("nan"), dtype=torch.float32, device="cuda")
    gammas = torch.full((B, H, cap), float("nan"), dtype=torch.float32, device="cuda")
    qjl.tq_encode_keys(dev_u16(keys), codes, bits, norms, gammas, pos, seed, k)
    torch.cuda.synchronize()
    return codes, bits, norms, gammas


def check_tq(qjl, keys, k, cap=None, pos=0, label=""):
    B, H, n, d = keys.shape
    cap = n + pos if cap is None else cap
    say("tq encode", label, (B, H, n), "k", k, "cap", cap, "pos", pos)
    codes, bits, norms, gammas = gpu_tq(qjl, keys, k, cap, pos)
    rc, rb, rn, rg = threaded(lambda x: otq.encode(x, k, SEED), keys.reshape(-1, d))
    sl = (slice(None), slice(None), slice(pos, pos + n))
    assert np.array_equal(host_u32(codes)[sl].reshape(-1, d * k // 32), rc), "codes differ"
    assert np.array_equal(host_u32(bits)[sl].reshape(-1, d // 32), rb), "sign bits differ"
    assert np.array_equal(norms.cpu().numpy()[sl].reshape(-1), rn), "norms differ"
    assert np.array_equal(gammas.cpu().numpy()[sl].reshape(-1), rg), "residual norms differ"
    mask = np.ones(cap, bool)
    mask[pos:pos + n] = False
    assert np.all(host_u32(codes)[:, :, mask] == np.uint32(SENTINEL))
    assert np.all(np.isnan(norms.cpu().numpy()[:, :, mask]))
    return codes, bits, norms, gammas


@pytest.mark.parametrize("k", [1, 2, 3])
def test_tq_encode_random_and_special(gpu_lib, k):
    rng = np.random.default_rng(20 + k)
    K = np.concatenate([wl.gaussian_keys(rng, 1000), special_keys(rng)])
    check_tq(gpu_lib, K.reshape(1, 1, -1, D), k, label="random + special")


@pytest.mark.parametrize("B,H,n,cap,pos", [(1, 1, 1, 1, 0), (2, 3, 31, 40, 5), (1, 2, 33, 100, 60),
                                            (3, 1, 95, 200, 100)])
def test_tq_encode_ragged(gpu_lib, B, H, n, cap, pos):
    rng = np.random.default_rng(B * 100 + n)
    keys = wl.gaussian_keys(rng, B * H * n, scale=3.0).reshape(B, H, n, D)
    check_tq(gpu_lib, keys, 2, cap=cap, pos=pos, label="ragged")


@pytest.mark.parametrize("k,margin", [(1, 40), (2, 40), (2, 12), (3, 12)])
def test_tq_encode_exact_paths(gpu_lib, k, margin):
    """Certificates widened by 2^margin: at 2^12 about a third of the
    rotated values (and every residual sign near zero) go to the wave's
    error-free butterfly sums, which decide them; at 2^40 those sums cannot
    decide either and every value takes the exact integer accumulator.
    Results are unchanged."""
    rng = np.random.default_rng(30 + k)
    K = np.concatenate([wl.gaussian_keys(rng, 200), special_keys(rng)])
    prev = gpu_lib.testing_set_rotq_margin(margin)
    try:
        check_tq(gpu_lib, K.reshape(1, 1, -1, D), k, label="exact paths")
    finally:
        gpu_lib.testing_set_rotq_margin(prev)


def test_tq_encode_workload_keys(gpu_lib):
    """All 262 144 keys of the 32K GQA workload (channel-scaled, outliers)."""
    w = wl.gqa32k()
    check_tq(gpu_lib, w.keys, 2, label="gqa32k keys")


@pytest.mark.parametrize("G", [1, 2, 4, 8])
@pytest.mark.parametrize("k", [1, 2, 3])
def test_tq_scores(gpu_lib, G, k):
    import torch
    rng = np.random.default_rng(40 + 10 * G + k)
    B, Hkv, N, cap = 2, 2, 700, 720
    keys = wl.gaussian_keys(rng, B * Hkv * cap, scale=2.0).reshape(B, Hkv, cap, D)
    q = rng.standard_normal((B, Hkv * G, D)).astype(np.float32)
    codes, bits, norms, gammas = gpu_tq(gpu_lib, keys, k)
    say("tq scores", "G", G, "k", k, "N", N)
    got = gpu_lib.tq_scores(dev_f32(q), codes, bits, norms, gammas, N, SEED, k)
    torch.cuda.synchronize()
    ref = otq.scores(q, host_u32(codes), host_u32(bits), norms.cpu().numpy(), gammas.cpu().numpy(), N, k, SEED)
    got = got.cpu().numpy().astype(np.float64)
    scale = np.sqrt(np.mean(ref ** 2, axis=-1, keepdims=True))
    assert np.max(np.abs(got - ref) / scale) <= 1e-5


@pytest.mark.parametrize("G,k", [(4, 2), (8, 1), (8, 2), (1, 1)])
def test_tq_scores_many_passes(gpu_lib, G, k):
    """Caches long enough that every wave of the matrix-core scores kernel
    takes several passes over several workgroups, from random bit patterns
    (every pattern is a valid cache), with a ragged end."""
    import torch
    rng = np.random.default_rng(60 + 10 * G + k)
    B, Hkv, N, cap = 1, 2, 300_001, 300_016
    codes = rng.integers(0, 2 ** 32, (B, Hkv, cap, D * k // 32), dtype=np.uint64).astype(np.uint32)
    bits = rng.integers(0, 2 ** 32, (B, Hkv, cap, D // 32), dtype=np.uint64).astype(np.uint32)
    norms = rng.uniform(0.5, 4.0, (B, Hkv, cap)).astype(np.float32)
    gammas = rng.uniform(0.0, 1.0, (B, Hkv, cap)).astype(np.float32)
    q = rng.standard_normal((B, Hkv * G, D)).astype(np.float32)
    say("tq scores many passes", "G", G, "k", k, "N", N)
    got = gpu_lib.tq_scores(dev_f32(q), dev_u32(codes), dev_u32(bits), dev_f32(norms), dev_f32(gammas), N, SEED, k)
    torch.cuda.synchronize()
    ref = otq.scores(q, codes, bits, norms, gammas, N, k, SEED)
    got = got.cpu().numpy().astype(np.float64)
    scale = np.sqrt(np.mean(ref ** 2, axis=-1, keepdims=True))
    assert np.max(np.abs(got - ref) / scale) <= 1e-5


@pytest.mark.parametrize("k", [1, 2])
@pytest.mark.parametrize("N", [24_000, 40_000])
def test_tq_scores_odd_passes(gpu_lib, k, N):
    """64 kv heads, so that each workgroup of the matrix-core scores kernel
    takes 768 or 1280 tokens and each wave an odd number of passes (3 or 5
    with 256 compute units): the pass loop alternates two row buffers, and
    these counts end it after a pass of the first one, once after going
    round (3) and once after going round twice (5); ragged last workgroup."""
    import torch
    rng = np.random.default_rng(80 + k + N % 97)
    B, Hkv, G = 1, 64, 1
    cap = N + 5
    codes = rng.integers(0, 2 ** 32, (B, Hkv, cap, D * k // 32), dtype=np.uint64).astype(np.uint32)
    bits = rng.integers(0, 2 ** 32, (B, Hkv, cap, D // 32), dtype=np.uint64).astype(np.uint32)
    norms = rng.uniform(0.5, 4.0, (B, Hkv, cap)).astype(np.float32)
    gammas = rng.uniform(0.0, 1.0, (B, Hkv, cap)).astype(np.float32)
    q = rng.standard_normal((B, Hkv * G, D)).astype(np.float32)
    say("tq scores odd passes", "k", k, "N", N, "Hkv", Hkv)
    got = gpu_lib.tq_scores(dev_f32(q), dev_u32(codes), dev_u32(bits), dev_f32(norms), dev_f32(gammas), N, SEED, k)
    torch.cuda.synchronize()
    got = got.cpu().numpy().astype(np.float64)
    # the oracle on three windows of 1536 tokens (each spans every pass of
    # the waves of the workgroups it touches): the start, the middle and the
    # ragged end
    L = 1536
    for t0 in (0, (N // 2) // 256 * 256, N - L):
        sl = slice(t0, t0 + L)
        ref = otq.scores(q, codes[:, :, sl], bits[:, :, sl], norms[:, :, sl], gammas[:, :, sl], L, k, SEED)
        scale = np.sqrt(np.mean(ref ** 2, axis=-1, keepdims=True))
        assert np.max(np.abs(got[:, :, sl] - ref) / scale) <= 1e-5, t0


@pytest.mark.parametrize("k", [1, 2, 3])
@pytest.mark.parametrize("N", [1, 17])
def test_tq_scores_edge_queries(gpu_lib, k, N):
    """Very short caches, and query heads that are zero, or scaled by 2^70
    or 2^-70 (the limbs' exponent follows each head's own largest value)."""
    import torch
    rng = np.random.default_rng(70 + 10 * k + N)
    G, B, Hkv, cap = 4, 1, 2, N + 3
    keys = wl.gaussian_keys(rng, B * Hkv * cap, scale=2.0).reshape(B, Hkv, cap, D)
    q = rng.standard_normal((B, Hkv * G, D)).astype(np.float32)
    q[0, 0] = 0.0
    q[0, 1] *= np.float32(2.0 ** 70)
    q[0, 2] *= np.float32(2.0 ** -70)
    q[0, 5] = 0.0
    codes, bits, norms, gammas = gpu_tq(gpu_lib, keys, k)
    say("tq scores edge queries", "k", k, "N", N)
    got = gpu_lib.tq_scores(dev_f32(q), codes, bits, norms, gammas, N, SEED, k)
    torch.cuda.synchronize()
    ref = otq.scores(q, host_u32(codes), host_u32(bits), norms.cpu().numpy(), gammas.cpu().numpy(), N, k, SEED)
    got = got.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got))
    for h in range(Hkv * G):
        if not np.any(q[0, h]):
            assert np.all(got[0, h] == 0.0), h
            continue
        scale = np.sqrt(np.mean(ref[0, h] ** 2))
        assert np.max(np.abs(got[0, h] - ref[0, h])) <= 1e-5 * scale, h


def test_tq_scores_track_exact_inner_products(gpu_lib):
    """Quality reading (not parity): over many keys the scores are unbiased
    estimates of <q, k> with the relative spread the oracle predicts."""
    import torch
    rng = np.random.default_rng(50)
    N = 4096
    keys = wl.gaussian_keys(rng, N).reshape(1, 1, N, D)
    q = rng.standard_normal((1, 4, D)).astype(np.float32)
    codes, bits, norms, gammas = gpu_tq(gpu_lib, keys, 2)
    got = gpu_lib.tq_scores(dev_f32(q), codes, bits, norms, gammas, N, SEED, 2)
    torch.cuda.synchronize()
    exact = q[0].astype(np.float64) @ oracle.bf16_bits_to_float64(keys[0, 0]).T
    err = got.cpu().numpy()[0] - exact
    rel = np.sqrt(np.mean(err ** 2) / np.mean(exact ** 2))
    assert rel < 0.6
    assert abs(err.mean()) < 4 * err.std() / np.sqrt(err.size) + 0.05


def gpu_pq(qjl, keys, cap=None, pos=0):
    import torch
    B, H, n, d = keys.shape
    cap = n + pos if cap is None else cap
    codes = torch.full((B, H, cap, 12), SENTINEL, dtype=torch.int32, device="cuda")
    radii = torch.full((B, H, cap), float("nan"), dtype=torch.float32, device="cuda")
    qjl.pq_encode_keys(dev_u16(keys), codes, radii, pos, SEED)
    torch.cuda.synchronize()
    return codes, radii


def check_pq(qjl, keys, cap=None, pos=0, label=""):
    B, H, n, d = keys.shape
    cap = n + pos if cap is None else cap
    say("pq encode", label, (B, H, n), "cap", cap, "pos", pos)
    codes, radii = gpu_pq(qjl, keys, cap, pos)
    rc, rr = threaded(lambda x: opq.encode(x, SEED), keys.reshape(-1, d))
    sl = (slice(None), slice(None), slice(pos, pos + n))
    assert np.array_equal(host_u32(codes)[sl].reshape(-1, 12), rc), "cells differ"
    assert np.array_equal(radii.cpu().numpy()[sl].reshape(-1), rr), "radii differ"
    mask = np.ones(cap, bool)
    mask[pos:pos + n] = False
    assert np.all(host_u32(codes)[:, :, mask] == np.uint32(SENTINEL))


def test_pq_encode_random_and_special(gpu_lib):
    rng = np.random.default_rng(60)
    K = np.concatenate([wl.gaussian_keys(rng, 1000), special_keys(rng)])
    check_pq(gpu_lib, K.reshape(1, 1, -1, D), label="random + special")


@pytest.mark.parametrize("B,H,n,cap,pos", [(1, 1, 1, 1, 0), (2, 3, 31, 40, 5), (3, 1, 95, 200, 100)])
def test_pq_encode_ragged(gpu_lib, B, H, n, cap, pos):
    rng = np.random.default_rng(B * 10 + n + 7)
    keys = wl.gaussian_keys(rng, B * H * n, scale=0.1).reshape(B, H, n, D)
    check_pq(gpu_lib, keys, cap=cap, pos=pos, label="ragged")


def test_pq_encode_exact_paths_and_workload(gpu_lib):
    rng = np.random.default_rng(61)
    K = np.concatenate([wl.gaussian_keys(rng, 200), special_keys(rng)])
    for margin in (12, 40):   # butterfly sums decide / the integer accumulator decides
        prev = gpu_lib.testing_set_rotq_margin(margin)
        try:
            check_pq(gpu_lib, K.reshape(1, 1, -1, D), label=f"exact paths, margin 2^{margin}")
        finally:
            gpu_lib.testing_set_rotq_margin(prev)
    w = wl.gqa32k()
    check_pq(gpu_lib, w.keys, label="gqa32k keys")
