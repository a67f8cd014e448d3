"""The allocation-free decode entry point (qjl_decode_attention_noalloc).

It runs the same kernels and split plan as qjl_decode_attention, with the
split scratch in the library's static per-GPU array instead of a caller's
workspace.  Checked through the C ABI against qjl_decode_attention on the
same inputs (bit for bit, and within the parity tolerance of the oracle), on
calls in a row whose sizes shrink, so the second call finds the first call's
contents in the shared scratch.
"""

import numpy as np
import pytest

import oracle
from jl_rotated_bit_amd import workloads as wl

from .gpu_util import dev_f32, dev_u16, dev_u32, row_rel_l2, say

pytestmark = pytest.mark.gpu

SEED = 42
TIGHT_TOL = 1e-4


def make_case(rng, B, Hkv, G, N, cap, m):
    keys = wl.gaussian_keys(rng, B * Hkv * cap, scale=2.0).reshape(B, Hkv, cap, 128)
    values = wl.gaussian_keys(rng, B * Hkv * cap).reshape(B, Hkv, cap, 128)
    q = rng.standard_normal((B, Hkv * G, 128)).astype(np.float32)
    words, norms = oracle.encode(keys.reshape(-1, 128), oracle.sketch(SEED, 128, m))
    return (q, words.reshape(B, Hkv, cap, m // 32), norms.reshape(B, Hkv, cap), values, N, m)


def test_noalloc_matches_workspace_entry(gpu_lib):
    import torch
    rng = np.random.default_rng(2024)
    cases = [make_case(rng, 1, 8, 4, 20000, 20011, 256),   # 32 eight-wave splits
             make_case(rng, 2, 2, 2, 3000, 3000, 256),     # fewer splits, other head count
             make_case(rng, 1, 4, 8, 9000, 9100, 512),     # m = 512
             make_case(rng, 1, 1, 1, 100, 100, 256)]       # one split (no scratch use)
    outs = []
    for q, words, norms, values, N, m in cases:
        B, Hq, d = q.shape
        Hkv = values.shape[1]
        say("noalloc decode", "B", B, "Hq", Hq, "Hkv", Hkv, "N", N, "m", m,
            "splits", gpu_lib.decode_num_splits(B, Hq, Hkv, N, d, m))
        qd, wd, nd, vd = dev_f32(q), dev_u32(words), dev_f32(norms), dev_u16(values)
        ref = gpu_lib.decode_attention(qd, wd, nd, vd, N, SEED, m)    # uploads S if needed
        torch.cuda.synchronize()
        got = []
        for _ in range(2):
            out = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device="cuda")
            gpu_lib.decode_attention_noalloc(qd, wd, nd, vd, N, SEED, m, out)
            torch.cuda.synchronize()
            got.append(out)
        outs.append((ref, got, q, words, norms, values, N, m))
    for ref, got, q, words, norms, values, N, m in outs:
        for g in got:
            assert torch.equal(g, ref)
        want = oracle.decode(q, words, norms, values, N, oracle.sketch(SEED, 128, m))
        assert row_rel_l2(got[-1].cpu().numpy(), want) <= TIGHT_TOL


def test_noalloc_needs_resident_sketch(gpu_lib):
    """With a seed never used on this device, S is not resident and the call
    returns QJL_EINVAL instead of allocating."""
    import torch
    q = torch.zeros((1, 4, 128), dtype=torch.float32, device="cuda")
    signs = torch.zeros((1, 1, 64, 8), dtype=torch.int32, device="cuda")
    norms = torch.ones((1, 1, 64), dtype=torch.float32, device="cuda")
    values = torch.zeros((1, 1, 64, 128), dtype=torch.int16, device="cuda")
    out = torch.empty((1, 4, 128), dtype=torch.float32, device="cuda")
    with pytest.raises(gpu_lib.QJLError) as ei:
        gpu_lib.decode_attention_noalloc(q, signs, norms, values, 64, 987654321, 256, out)
    assert ei.value.status == 1
    assert "not resident" in str(ei.value)
