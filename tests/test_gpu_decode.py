"""GPU parity of qjl_decode_attention against the oracle.

Gate: every (batch, query head) output row within 2e-2 relative L2 of the
fp64 oracle (the contract), and within 1e-4 (derived from the arithmetic: S^T q
and all sums in fp32 with relative error ~1e-6, exp2 to a few ulp; a wrong,
missing or extra token moves a row by far more than that in these tests).
"""

import math

import numpy as np
import pytest

import oracle
from jl_rotated_bit_amd import workloads as wl

from .gpu_util import (cached_workload, dev_f32, dev_u16, dev_u32, gpu_encode, host_u32,
                       oracle_encode, row_rel_l2, say)

pytestmark = pytest.mark.gpu

SEED = 42
CONTRACT_TOL = 2e-2
TIGHT_TOL = 1e-4


def oracle_cache(keys, m, seed=SEED):
    B, H, n, d = keys.shape
    words, norms = oracle_encode(keys.reshape(-1, d), oracle.sketch(seed, d, m))
    return words.reshape(B, H, n, m // 32), norms.reshape(B, H, n)


def run_decode(qjl, q, words, norms, values, N, m, seed=SEED, scale=None, workspace=None):
    import torch
    out = qjl.decode_attention(dev_f32(q), dev_u32(words), dev_f32(norms), dev_u16(values), N,
                               seed, m, scale=scale, workspace=workspace)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def check_decode(qjl, q, words, norms, values, N, m, seed=SEED, scale=None, label=""):
    B, Hq, d = q.shape
    say("decode", label, "B", B, "Hq", Hq, "Hkv", values.shape[1], "N", N, "cap", values.shape[2],
        "m", m, "splits", qjl.decode_num_splits(B, Hq, values.shape[1], N, d, m))
    got = run_decode(qjl, q, words, norms, values, N, m, seed, scale)
    ref = oracle.decode(q, words, norms, values, N, oracle.sketch(seed, d, m), scale=scale)
    err = row_rel_l2(got, ref)
    assert err <= CONTRACT_TOL, err
    assert err <= TIGHT_TOL, err
    return got, ref


def test_small_workload_end_to_end(gpu_lib):
    """GPU encode -> GPU decode, against oracle encode -> oracle decode."""
    w = wl.small()
    signs, norms = gpu_encode(gpu_lib, w.keys, w.m, SEED)
    ref_w, ref_n = oracle_cache(w.keys, w.m)
    assert np.array_equal(host_u32(signs), ref_w)
    import torch
    say("decode small end-to-end")
    out = gpu_lib.decode_attention(dev_f32(w.q), signs, norms, dev_u16(w.values), w.N, SEED, w.m)
    torch.cuda.synchronize()
    ref = oracle.decode(w.q, ref_w, ref_n, w.values, w.N, oracle.sketch(SEED, 128, w.m))
    err = row_rel_l2(out.cpu().numpy(), ref)
    assert err <= TIGHT_TOL, err
    # quality reading only (not gated): distance to exact softmax attention
    exact = oracle.exact_attention(w.q, w.keys, w.values, w.N)
    say("small: rel L2 to exact attention", row_rel_l2(out.cpu().numpy(), exact))


def test_gqa32k_full(gpu_lib):
    w = wl.gqa32k()
    words, norms = oracle_cache(w.keys, w.m)
    check_decode(gpu_lib, w.q, words, norms, w.values, w.N, w.m, label="gqa32k")


def test_gqa32k_tp8_share_end_to_end(gpu_lib):
    """One GPU's share of the 32K GQA workload under 8-way tensor parallelism
    (1 kv head, its 4 query heads, 32768 tokens): GPU encode (every word
    equal to the oracle's, norms within 1e-5), then GPU decode on those
    caches against the oracle decode on its own."""
    import torch
    w = wl.tp8()
    signs, norms = gpu_encode(gpu_lib, w.keys, w.m, SEED)
    ref_w, ref_n = oracle_cache(w.keys, w.m)
    assert np.array_equal(host_u32(signs), ref_w)
    gn = norms.cpu().numpy()
    assert np.max(np.abs(gn - ref_n) / ref_n) <= 1e-5
    say("decode gqa32k TP=8 share", "splits", gpu_lib.decode_num_splits(1, 4, 1, w.N, 128, w.m))
    out = gpu_lib.decode_attention(dev_f32(w.q), signs, norms, dev_u16(w.values), w.N, SEED, w.m)
    torch.cuda.synchronize()
    ref = oracle.decode(w.q, ref_w, ref_n, w.values, w.N, oracle.sketch(SEED, 128, w.m))
    err = row_rel_l2(out.cpu().numpy(), ref)
    assert err <= TIGHT_TOL, err


def test_mha16k_full(gpu_lib):
    """The whole 40-head, batch-8, 16K workload: the GPU encode of all
    5 242 880 keys equals the oracle's cache (every word, every norm within
    1e-5), then the decode runs on the oracle's own cache, so the two halves
    are checked independently."""
    w, ref_w, ref_n = cached_workload("mha16k")
    say("mha16k encode, all rows")
    signs, norms = gpu_encode(gpu_lib, w.keys, w.m, SEED)
    assert np.array_equal(host_u32(signs), ref_w)
    got_n = norms.cpu().numpy()
    assert np.all(np.abs(got_n.astype(np.float64) - ref_n) <= 1e-5 * ref_n)
    del signs, norms
    check_decode(gpu_lib, w.q, ref_w, ref_n, w.values, w.N, w.m, label="mha16k")


def test_long64k_append_steps(gpu_lib):
    """Prefill 65536 keys (m=512), then 64 steps of append-one-token + decode."""
    import torch
    w = wl.long64k()
    d, m, N0 = 128, w.m, w.N
    say("long64k prefill encode")
    signs, norms = gpu_encode(gpu_lib, w.keys[:, :, :N0], m, SEED, cap=w.cap)
    values = dev_u16(w.values)
    ws = torch.zeros(gpu_lib.decode_workspace_bytes(1, w.H_q, w.H_kv, w.cap, d, m),
                     dtype=torch.uint8, device="cuda")
    checked = {}
    for s in range(len(w.steps)):
        gpu_lib.encode_keys(dev_u16(w.keys[:, :, N0 + s:N0 + s + 1]), signs, norms, N0 + s, SEED, m)
        q = w.steps[s]
        out = gpu_lib.decode_attention(dev_f32(q), signs, norms, values, N0 + s + 1, SEED, m,
                                       workspace=ws)
        if s in (0, 31, 63):
            torch.cuda.synchronize()
            checked[s] = (q, out.cpu().numpy())
    torch.cuda.synchronize()
    words = host_u32(signs)
    ref_w, ref_n = oracle_cache(w.keys, m)
    assert np.array_equal(words, ref_w)
    S = oracle.sketch(SEED, d, m)
    for s, (q, got) in checked.items():
        say("long64k check step", s)
        ref = oracle.decode(q, ref_w, ref_n, w.values, N0 + s + 1, S)
        err = row_rel_l2(got, ref)
        assert err <= TIGHT_TOL, (s, err)


@pytest.mark.parametrize("m", [256, 512])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
@pytest.mark.parametrize("N,cap", [(1, 1), (2, 5), (63, 64), (64, 64), (65, 100), (255, 255),
                                    (257, 300), (1000, 1000), (4097, 5000)])
def test_shapes_ragged(gpu_lib, m, G, N, cap):
    rng = np.random.default_rng(N * 31 + G * 7 + m)
    B, Hkv, d = 2, 2, 128
    keys = wl.gaussian_keys(rng, B * Hkv * cap, scale=2.0).reshape(B, Hkv, cap, d)
    values = wl.gaussian_keys(rng, B * Hkv * cap).reshape(B, Hkv, cap, d)
    q = rng.standard_normal((B, Hkv * G, d)).astype(np.float32)
    words, norms = oracle_cache(keys, m)
    check_decode(gpu_lib, q, words, norms, values, N, m, label=f"ragged G={G}")


@pytest.mark.parametrize("m", [256, 512])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_eight_wave_workgroups(gpu_lib, m, G):
    """Few streams with a long context take the eight-wave workgroups (29
    splits here; four-wave workgroups would use 52), for every G and m."""
    rng = np.random.default_rng(500 + 10 * G + m)
    B, Hkv, d, N, cap = 1, 8, 128, 16421, 16432
    assert gpu_lib.decode_num_splits(B, Hkv * G, Hkv, N, d, m) == 29
    keys = wl.gaussian_keys(rng, B * Hkv * cap, scale=2.0).reshape(B, Hkv, cap, d)
    values = wl.gaussian_keys(rng, B * Hkv * cap).reshape(B, Hkv, cap, d)
    q = rng.standard_normal((B, Hkv * G, d)).astype(np.float32)
    words, norms = oracle_cache(keys, m)
    check_decode(gpu_lib, q, words, norms, values, N, m, label=f"eight waves G={G}")


def test_many_heads_one_round(gpu_lib):
    """40 kv heads at batch 1 (MHA): the split count is rounded down (6
    eight-wave splits, 240 workgroups), and every output row matches."""
    rng = np.random.default_rng(700)
    B, Hkv, G, d, N, cap, m = 1, 40, 1, 128, 5000, 5003, 256
    assert gpu_lib.decode_num_splits(B, Hkv * G, Hkv, N, d, m) == 6
    keys = wl.gaussian_keys(rng, B * Hkv * cap, scale=2.0).reshape(B, Hkv, cap, d)
    values = wl.gaussian_keys(rng, B * Hkv * cap).reshape(B, Hkv, cap, d)
    q = rng.standard_normal((B, Hkv * G, d)).astype(np.float32)
    words, norms = oracle_cache(keys, m)
    check_decode(gpu_lib, q, words, norms, values, N, m, label="40 heads, 6 splits")


def test_unused_cache_rows_are_not_read(gpu_lib):
    rng = np.random.default_rng(8)
    B, Hkv, G, cap, N, m = 1, 2, 4, 3000, 2049, 256
    keys = wl.gaussian_keys(rng, B * Hkv * cap).reshape(B, Hkv, cap, 128)
    values = wl.gaussian_keys(rng, B * Hkv * cap).reshape(B, Hkv, cap, 128)
    q = rng.standard_normal((B, Hkv * G, 128)).astype(np.float32)
    words, norms = oracle_cache(keys, m)
    got, _ = check_decode(gpu_lib, q, words, norms, values, N, m, label="N < cap")
    values2 = values.copy()
    values2[:, :, N:] = oracle.float64_to_bf16_bits(np.full((B, Hkv, cap - N, 128), 3e38))
    words2 = words.copy()
    words2[:, :, N:] = 0
    norms2 = norms.copy()
    norms2[:, :, N:] = 1e30
    got2 = run_decode(gpu_lib, q, words2, norms2, values2, N, m)
    assert np.array_equal(got, got2)


def test_every_token_counted_once(gpu_lib):
    """Identical keys give a uniform softmax; V_t = e_{t mod 128} then makes
    out[c] = #{t < N : t = c mod 128} / N, which a dropped or doubled token
    (at a tile or split boundary, say) changes by 1/N."""
    rng = np.random.default_rng(9)
    for N, G, m in [(32768, 4, 256), (65600, 4, 512), (16384, 1, 256), (5000, 8, 256)]:
        Hkv = 2
        words = np.broadcast_to(rng.integers(0, 2 ** 32, (1, 1, 1, m // 32), dtype=np.uint32),
                                (1, Hkv, N, m // 32)).copy()
        norms = np.full((1, Hkv, N), 3.0, np.float32)
        V = np.zeros((1, Hkv, N, 128))
        V[0, :, np.arange(N), np.arange(N) % 128] = 1.0
        values = oracle.float64_to_bf16_bits(V)
        q = rng.standard_normal((1, Hkv * G, 128)).astype(np.float32)
        say("token coverage", N, G, m)
        got = run_decode(gpu_lib, q, words, norms, values, N, m)
        counts = np.bincount(np.arange(N) % 128, minlength=128) / N
        assert np.allclose(got, counts[None, None, :], rtol=2e-5, atol=0), (N, G, m)


def test_special_inputs(gpu_lib):
    rng = np.random.default_rng(10)
    B, Hkv, G, N, m = 1, 2, 4, 3000, 256
    keys = wl.gaussian_keys(rng, B * Hkv * N).reshape(B, Hkv, N, 128)
    values = wl.gaussian_keys(rng, B * Hkv * N).reshape(B, Hkv, N, 128)
    words, norms = oracle_cache(keys, m)
    Vmean = oracle.bf16_bits_to_float64(values).mean(axis=2)          # [B][Hkv][d]
    # q = 0: uniform softmax
    got = run_decode(gpu_lib, np.zeros((B, Hkv * G, 128), np.float32), words, norms, values, N, m)
    assert row_rel_l2(got, np.repeat(Vmean, G, axis=1)) < TIGHT_TOL
    # explicit temperatures, including a very sharp one
    q = rng.standard_normal((B, Hkv * G, 128)).astype(np.float32)
    for scale in (0.01, 1.0, 25.0):
        check_decode(gpu_lib, q, words, norms, values, N, m, scale=scale, label=f"scale {scale}")
    # scale 0 means 1/sqrt(d)
    a = run_decode(gpu_lib, q, words, norms, values, N, m, scale=None)
    b = run_decode(gpu_lib, q, words, norms, values, N, m, scale=1 / math.sqrt(128))
    assert np.allclose(a, b, rtol=1e-6, atol=1e-7)


def test_workspace_reuse_across_calls(gpu_lib):
    """Arrival counters return to zero: back-to-back calls sharing one workspace
    (different sizes, different split counts, and counters 256 bytes apart
    for up to 16 kv heads, 128 bytes apart for 32) all stay correct."""
    import torch
    rng = np.random.default_rng(11)
    ws = torch.zeros(1 << 24, dtype=torch.uint8, device="cuda")
    cases = []
    for N, Hkv, G in [(20000, 8, 4), (777, 2, 2), (20000, 8, 4), (300, 1, 8), (9000, 4, 1), (3000, 32, 1)]:
        keys = wl.gaussian_keys(rng, Hkv * N).reshape(1, Hkv, N, 128)
        values = wl.gaussian_keys(rng, Hkv * N).reshape(1, Hkv, N, 128)
        q = rng.standard_normal((1, Hkv * G, 128)).astype(np.float32)
        words, norms = oracle_cache(keys, 256)
        cases.append((q, words, norms, values, N))
    outs = []
    say("workspace reuse")
    for q, words, norms, values, N in cases * 2:
        outs.append(run_decode(gpu_lib, q, words, norms, values, N, 256, workspace=ws))
    assert int(ws[:4096].cpu().numpy().view(np.uint32).max()) == 0
    S = oracle.sketch(SEED, 128, 256)
    for i, (q, words, norms, values, N) in enumerate(cases):
        ref = oracle.decode(q, words, norms, values, N, S)
        assert row_rel_l2(outs[i], ref) <= TIGHT_TOL
        assert np.array_equal(outs[i], outs[i + len(cases)])


def test_side_stream_with_fresh_workspace(gpu_lib):
    """A decode on a stream other than the current one, with the workspace
    and output made by the binding: they are allocated and zero-filled on
    that stream, so the result equals the oracle's and the default-stream
    result, bit for bit."""
    import torch
    rng = np.random.default_rng(12)
    B, Hkv, G, N, m = 1, 8, 4, 20000, 256
    keys = wl.gaussian_keys(rng, B * Hkv * N).reshape(B, Hkv, N, 128)
    values = wl.gaussian_keys(rng, B * Hkv * N).reshape(B, Hkv, N, 128)
    q = rng.standard_normal((B, Hkv * G, 128)).astype(np.float32)
    words, norms = oracle_cache(keys, m)
    say("decode on a side stream", "splits", gpu_lib.decode_num_splits(B, Hkv * G, Hkv, N, 128, m))
    qd, wd, nd, vd = dev_f32(q), dev_u32(words), dev_f32(norms), dev_u16(values)
    ref_dev = gpu_lib.decode_attention(qd, wd, nd, vd, N, SEED, m)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(3):
        gpu_lib._workspaces.clear()          # a fresh workspace for every call
        outs.append(gpu_lib.decode_attention(qd, wd, nd, vd, N, SEED, m, stream=side))
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ref = oracle.decode(q, words, norms, values, N, oracle.sketch(SEED, 128, m))
    for o in outs:
        assert row_rel_l2(o.cpu().numpy(), ref) <= TIGHT_TOL
        assert torch.equal(o, ref_dev)
