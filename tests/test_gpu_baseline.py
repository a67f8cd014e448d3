"""GPU parity of the uncompressed baseline (qjl_baseline_decode_attention_bf16)
against exact softmax attention over the same bf16 keys and values
(oracle.exact_attention, fp64).

Tolerance 1e-4 per (batch, query head) row, from the arithmetic: q enters as
three bf16 parts (their sum is fp32 q to 2^-24), each product of two bf16
values is exact in fp32 and the 128-term sums carry ~1e-6 relative error,
the probabilities enter P.V as bf16 hi + lo parts (2^-17 relative), and a
dropped or doubled token moves these rows by far more.
"""

import numpy as np
import pytest

import oracle
from jl_rotated_bit_amd import workloads as wl

from .gpu_util import dev_f32, dev_u16, row_rel_l2, say

pytestmark = pytest.mark.gpu

TOL = 1e-4


def run_baseline(qjl, q, keys, values, N, scale=None):
    import torch
    out = qjl.baseline_decode_attention_bf16(dev_f32(q), dev_u16(keys), dev_u16(values), N, scale=scale)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("G", [1, 2, 4, 8])
@pytest.mark.parametrize("N,cap", [(1, 1), (2, 5), (63, 64), (65, 100), (1000, 1000), (4097, 5000)])
def test_baseline_shapes(gpu_lib, G, N, cap):
    rng = np.random.default_rng(N * 13 + G)
    B, Hkv = 2, 2
    keys = wl.gaussian_keys(rng, B * Hkv * cap, scale=0.5).reshape(B, Hkv, cap, 128)
    values = wl.gaussian_keys(rng, B * Hkv * cap).reshape(B, Hkv, cap, 128)
    q = rng.standard_normal((B, Hkv * G, 128)).astype(np.float32)
    say("baseline bf16 decode", "G", G, "N", N, "cap", cap,
        "splits", gpu_lib.decode_num_splits(B, Hkv * G, Hkv, N, 128, 256))
    got = run_baseline(gpu_lib, q, keys, values, N)
    ref = oracle.exact_attention(q, keys, values, N)
    assert row_rel_l2(got, ref) <= TOL


@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_baseline_eight_wave_splits(gpu_lib, G):
    rng = np.random.default_rng(70 + G)
    B, Hkv, N, cap = 1, 8, 16421, 16432
    keys = wl.gaussian_keys(rng, B * Hkv * cap, scale=0.5).reshape(B, Hkv, cap, 128)
    values = wl.gaussian_keys(rng, B * Hkv * cap).reshape(B, Hkv, cap, 128)
    q = rng.standard_normal((B, Hkv * G, 128)).astype(np.float32)
    say("baseline bf16 decode, eight-wave splits, G", G)
    got = run_baseline(gpu_lib, q, keys, values, N)
    assert row_rel_l2(got, oracle.exact_attention(q, keys, values, N)) <= TOL


def test_baseline_workloads(gpu_lib):
    """The 32K GQA workload and the 40-head, batch-8, 16K MHA workload."""
    for name in ("gqa32k", "mha16k"):
        w = wl.WORKLOADS[name]()
        say("baseline bf16 decode", name)
        got = run_baseline(gpu_lib, w.q, w.keys, w.values, w.N)
        ref = oracle.exact_attention(w.q, w.keys, w.values, w.N)
        assert row_rel_l2(got, ref) <= TOL, name
        del w


def test_baseline_scale_and_unused_rows(gpu_lib):
    rng = np.random.default_rng(5)
    B, Hkv, G, N, cap = 1, 2, 4, 3000, 3500
    keys = wl.gaussian_keys(rng, B * Hkv * cap).reshape(B, Hkv, cap, 128)
    values = wl.gaussian_keys(rng, B * Hkv * cap).reshape(B, Hkv, cap, 128)
    q = rng.standard_normal((B, Hkv * G, 128)).astype(np.float32)
    for scale in (0.01, 0.3):
        got = run_baseline(gpu_lib, q, keys, values, N, scale=scale)
        assert row_rel_l2(got, oracle.exact_attention(q, keys, values, N, scale=scale)) <= TOL
    got = run_baseline(gpu_lib, q, keys, values, N)
    k2, v2 = keys.copy(), values.copy()
    k2[:, :, N:] = 0x7F7F       # huge keys and values past N must not be read
    v2[:, :, N:] = 0x7F7F
    assert np.array_equal(got, run_baseline(gpu_lib, q, k2, v2, N))
