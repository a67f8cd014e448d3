"""GPU parity of qjl_decode_step (append one token, then decode, one launch).

The appended row must equal the oracle's encode of the new key (sign words
bit for bit, norm within 1e-5) and the new value row; rows past `pos` stay
untouched; the output is checked against the oracle's decode over tokens
[0, pos] with the same tolerances as qjl_decode_attention (2e-2 contract,
1e-4 derived).
"""

import numpy as np
import pytest

import oracle
from jl_rotated_bit_amd import workloads as wl

from .gpu_util import (SENTINEL, dev_f32, dev_u16, dev_u32, host_u32, oracle_encode, row_rel_l2,
                       say)
from .test_gpu_encode import adversarial_keys

pytestmark = pytest.mark.gpu

SEED = 42
TIGHT_TOL = 1e-4
NORM_RTOL = 1e-5


def split_rule(B, Hkv, N, m):
    """Tokens per split of the decode plan (the host arithmetic of the
    library's split rule, checked against qjl_decode_num_splits)."""
    streams = B * Hkv
    target8 = 240 if m == 512 else 256

    def plan(nw):
        target = target8 * 8 // nw
        want = target // streams
        if nw == 4 and want < 2:
            want = -(-target // streams)
        if streams > 1024:
            want = 1
        want = max(1, min(want, -(-N // (nw * 64)), 256))
        t = -(-N // want)
        t = -(-t // 64) * 64
        return -(-N // t), t
    ns, tps = plan(8)
    if not (ns > 1 and streams * ns >= 64):
        ns, tps = plan(4)
        return ns, tps, 4
    return ns, tps, 8


def step_rule(ns, tps, nw, N):
    """Splits of the fused step (the library's host arithmetic): where a
    split gives each wave at least two tiles, fewer splits (at most an eighth
    fewer) until the last split, which appends the new token, is at least one
    tile per wave shorter than the others."""
    shorter = nw * 64
    if ns < 2 or tps < 2 * shorter:
        return ns, tps
    want = ns
    while want >= 2 and want >= ns - ns // 8:
        t = -(-(-(-N // want)) // 64) * 64
        n = -(-N // t)
        if n > 1 and N - (n - 1) * t <= t - shorter:
            return n, t
        want -= 1
    return ns, tps


def run_step_case(qjl, rng, B, Hkv, G, pos, cap, m, new_rows=None, label=""):
    import torch
    d = 128
    keys = wl.gaussian_keys(rng, B * Hkv * cap, scale=2.0).reshape(B, Hkv, cap, d)
    values = wl.gaussian_keys(rng, B * Hkv * cap).reshape(B, Hkv, cap, d)
    if new_rows is not None:
        keys[:, :, pos] = new_rows
    q = rng.standard_normal((B, Hkv * G, d)).astype(np.float32)
    S = oracle.sketch(SEED, d, m)
    ref_w, ref_n = oracle_encode(keys.reshape(-1, d), S)
    ref_w = ref_w.reshape(B, Hkv, cap, m // 32)
    ref_n = ref_n.reshape(B, Hkv, cap)
    # caches: the oracle's rows before pos, a sentinel at pos and after
    w0 = ref_w.copy()
    w0[:, :, pos:] = SENTINEL
    n0 = ref_n.copy()
    n0[:, :, pos:] = np.nan
    v0 = values.copy()
    v0[:, :, pos:] = 0x7FC0                   # bf16 NaN in the rows not yet appended
    signs, norms, vals = dev_u32(w0), dev_f32(n0), dev_u16(v0)
    ns, tps, nw = split_rule(B, Hkv, pos + 1, m)
    assert qjl.decode_num_splits(B, Hkv * G, Hkv, pos + 1, d, m) == ns
    ns, tps = step_rule(ns, tps, nw, pos + 1)
    first_tile_of_wave = (pos - (ns - 1) * tps) < nw * 64   # the new token is in a wave's first tile
    say("decode step", label, "B", B, "Hkv", Hkv, "G", G, "pos", pos, "cap", cap, "m", m,
        "splits", ns, "waves", nw, "deferred first tile", first_tile_of_wave)
    out = qjl.decode_step(dev_f32(q), dev_u16(keys[:, :, pos].copy()), dev_u16(values[:, :, pos].copy()),
                          signs, norms, vals, pos, SEED, m)
    torch.cuda.synchronize()
    got_w, got_n = host_u32(signs), norms.cpu().numpy()
    got_v = vals.cpu().numpy().view(np.uint16)
    assert np.array_equal(got_w[:, :, :pos + 1], ref_w[:, :, :pos + 1]), "sign words differ"
    assert np.all(got_w[:, :, pos + 1:] == np.uint32(SENTINEL)), "rows past pos were written"
    ref_np = ref_n[:, :, pos].astype(np.float64)
    rel = np.abs(got_n[:, :, pos].astype(np.float64) - ref_np) / np.maximum(ref_np, 1e-300)
    zero = ref_n[:, :, pos] == 0
    assert np.all(got_n[:, :, pos][zero] == 0)
    assert rel[~zero].max(initial=0.0) <= NORM_RTOL
    assert np.all(np.isnan(got_n[:, :, pos + 1:]))
    assert np.array_equal(got_v[:, :, :pos + 1], values[:, :, :pos + 1])
    assert np.all(got_v[:, :, pos + 1:] == 0x7FC0)
    ref = oracle.decode(q, ref_w, ref_n, values, pos + 1, S)
    err = row_rel_l2(out.cpu().numpy(), ref)
    assert err <= TIGHT_TOL, err
    return first_tile_of_wave


@pytest.mark.parametrize("m", [256, 512])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
@pytest.mark.parametrize("pos,cap", [(0, 3), (63, 64), (64, 70), (200, 300), (4096, 4100)])
def test_step_shapes(gpu_lib, m, G, pos, cap):
    rng = np.random.default_rng(pos * 7 + G * 3 + m)
    run_step_case(gpu_lib, rng, 2, 2, G, pos, cap, m, label="shapes")


@pytest.mark.parametrize("m", [256, 512])
def test_step_eight_wave_splits(gpu_lib, m):
    """Long contexts of 8 kv heads (eight-wave workgroups, many splits): the
    new token in the middle of the last split, and as the only token of a
    wave's first tile (its load waits for the append)."""
    for N in (16421, 16385, 20000 + 1):
        rng = np.random.default_rng(N + m)
        ns, tps, nw = split_rule(1, 8, N, m)
        assert nw == 8 and ns > 16
        run_step_case(gpu_lib, rng, 1, 8, 4, N - 1, N + 3, m, label=f"8 kv heads, N={N}")
    # a case whose last split holds a single token: the deferred-load path
    hit = False
    for N in range(16385, 16385 + 64 * 40, 64):
        ns, tps, _ = split_rule(1, 8, N, m)
        if N - (ns - 1) * tps == 1:
            hit = run_step_case(gpu_lib, np.random.default_rng(N), 1, 8, 2, N - 1, N, m,
                                label=f"last split of one token, N={N}")
            break
    assert hit


@pytest.mark.parametrize("m,N", [(256, 32768), (512, 61440)])
def test_step_shortened_last_split(gpu_lib, m, N):
    """Contexts whose plain plan ends with a full split (32K tokens of 8 kv
    heads at m = 256, 30 x 2048 tokens at m = 512): the step takes fewer,
    longer splits so that the appending workgroup's split is short."""
    ns, tps, nw = split_rule(1, 8, N, m)
    assert nw == 8 and N - (ns - 1) * tps == tps
    sns, stps = step_rule(ns, tps, nw, N)
    assert sns < ns and N - (sns - 1) * stps <= stps - nw * 64
    run_step_case(gpu_lib, np.random.default_rng(N + m), 1, 8, 4, N - 1, N, m, label=f"short last split, N={N}")


@pytest.mark.parametrize("m", [256, 512])
def test_step_adversarial_new_keys(gpu_lib, m):
    """New keys whose projections are exactly zero or within rounding of
    zero (the certified path and the exact integer fallback), zero and -0
    keys, and keys near the ends of the bf16 range, one per (batch, kv head)."""
    S = oracle.sketch(SEED, 128, m)
    K = adversarial_keys(S, np.random.default_rng(40 + m))
    rows = K.shape[0]
    per_call = 8
    for c0 in range(0, rows, per_call):
        new = K[c0:c0 + per_call]
        if new.shape[0] < per_call:
            new = np.concatenate([new, K[:per_call - new.shape[0]]])
        rng = np.random.default_rng(c0)
        run_step_case(gpu_lib, rng, 2, 4, 2, 130, 131, m, new_rows=new.reshape(2, 4, 128),
                      label=f"adversarial rows {c0}..")


def test_step_matches_two_calls(gpu_lib):
    """The fused step gives the same sign words as qjl_encode_keys of the one
    new key per kv head followed by qjl_decode_attention, and outputs that
    agree to fp32 rounding (norms may differ in the last bit)."""
    import torch
    rng = np.random.default_rng(99)
    B, Hkv, G, cap, m = 1, 8, 4, 9000, 256
    pos = 8191
    keys = wl.gaussian_keys(rng, B * Hkv * cap).reshape(B, Hkv, cap, 128)
    values = wl.gaussian_keys(rng, B * Hkv * cap).reshape(B, Hkv, cap, 128)
    q = dev_f32(rng.standard_normal((B, Hkv * G, 128)).astype(np.float32))
    S = oracle.sketch(SEED, 128, m)
    ref_w, ref_n = oracle_encode(keys.reshape(-1, 128), S)
    w0 = ref_w.reshape(B, Hkv, cap, m // 32).copy()
    n0 = ref_n.reshape(B, Hkv, cap).copy()
    a_s, a_n, a_v = dev_u32(w0), dev_f32(n0), dev_u16(values)
    b_s, b_n, b_v = dev_u32(w0), dev_f32(n0), dev_u16(values)
    nk, nv = dev_u16(keys[:, :, pos].copy()), dev_u16(values[:, :, pos].copy())
    say("fused step vs encode + decode")
    out_a = gpu_lib.decode_step(q, nk, nv, a_s, a_n, a_v, pos, SEED, m)
    gpu_lib.encode_keys(nk.reshape(B, Hkv, 1, 128), b_s, b_n, pos, SEED, m)
    out_b = gpu_lib.decode_attention(q, b_s, b_n, b_v, pos + 1, SEED, m)
    torch.cuda.synchronize()
    assert torch.equal(a_s, b_s)
    assert torch.allclose(a_n, b_n, rtol=2 ** -22, atol=0)
    assert row_rel_l2(out_a.cpu().numpy(), out_b.cpu().numpy()) <= 1e-6


def test_long64k_fused_steps(gpu_lib):
    """The long-context workload with the fused step: prefill 65536 keys
    (m = 512), then 64 steps that each append a token and decode; outputs
    at steps 0, 31 and 63 against the oracle, and the whole cache (signs,
    norms, values) after the last step."""
    import torch
    w = wl.long64k()
    d, m, N0 = 128, w.m, w.N
    say("long64k fused: prefill encode")
    signs = torch.full((1, w.H_kv, w.cap, m // 32), SENTINEL, dtype=torch.int32, device="cuda")
    norms = torch.full((1, w.H_kv, w.cap), float("nan"), dtype=torch.float32, device="cuda")
    gpu_lib.encode_keys(dev_u16(w.keys[:, :, :N0]), signs, norms, 0, SEED, m)
    vals_h = w.values.copy()
    vals_h[:, :, N0:] = 0
    values = dev_u16(vals_h)
    ws = torch.zeros(gpu_lib.decode_workspace_bytes(1, w.H_q, w.H_kv, w.cap, d, m),
                     dtype=torch.uint8, device="cuda")
    nk = [dev_u16(w.keys[:, :, N0 + s].copy()) for s in range(len(w.steps))]
    nv = [dev_u16(w.values[:, :, N0 + s].copy()) for s in range(len(w.steps))]
    checked = {}
    for s in range(len(w.steps)):
        q = w.steps[s]
        out = gpu_lib.decode_step(dev_f32(q), nk[s], nv[s], signs, norms, values, N0 + s, SEED, m,
                                  workspace=ws)
        if s in (0, 31, 63):
            torch.cuda.synchronize()
            checked[s] = (q, out.cpu().numpy())
    torch.cuda.synchronize()
    ref_w, ref_n = oracle_encode(w.keys.reshape(-1, d), oracle.sketch(SEED, d, m))
    ref_w = ref_w.reshape(1, w.H_kv, w.cap, m // 32)
    ref_n = ref_n.reshape(1, w.H_kv, w.cap)
    assert np.array_equal(host_u32(signs), ref_w)
    got_n = norms.cpu().numpy()
    assert np.all(np.abs(got_n.astype(np.float64) - ref_n) <= NORM_RTOL * ref_n)
    assert np.array_equal(values.cpu().numpy().view(np.uint16), w.values)
    S = oracle.sketch(SEED, d, m)
    for s, (q, got) in checked.items():
        say("long64k fused: check step", s)
        ref = oracle.decode(q, ref_w, ref_n, w.values, N0 + s + 1, S)
        err = row_rel_l2(got, ref)
        assert err <= TIGHT_TOL, (s, err)
