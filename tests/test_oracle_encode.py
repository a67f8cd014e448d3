"""Pins for the oracle's encode: exact sign bits, packing order, norms.

Bit i of key k is 1 iff the exact sum_j k_j S[j, i] >= 0 (sign(0) = +1),
packed LSB-first 32 per word ("The Geometry of Forgetting", QJL section:
Q(x) = sign(Sx); "QJL: 1-Bit Quantized JL Transform ...", Abstract).
"""

import math

import numpy as np
import pytest

import oracle

SEED = 42


def pack_reference(bits_row):
    """Independent packing: Python ints, bit i -> word i // 32, position i % 32."""
    m = len(bits_row)
    words = []
    for w in range(m // 32):
        v = 0
        for b in range(32):
            if bits_row[32 * w + b]:
                v |= 1 << b
        words.append(v)
    return words


def bf16(x):
    return oracle.float64_to_bf16_bits(np.asarray(x, dtype=np.float64))


@pytest.mark.parametrize("d,m", [(128, 256), (128, 512), (16, 64)])
def test_one_hot_keys_read_back_rows_of_S(d, m):
    S = oracle.sketch(SEED, d, m)
    keys = np.zeros((2 * d, d))
    for j in range(d):
        keys[j, j] = 2.0 ** (j % 7 - 3)      # positive scale: bits = [S[j, i] >= 0]
        keys[d + j, j] = -1.0                # negative: bits = [S[j, i] <= 0]
    words, norms = oracle.encode(bf16(keys), S)
    for j in range(d):
        assert words[j].tolist() == pack_reference(S[j] >= 0)
        assert words[d + j].tolist() == pack_reference(S[j] <= 0)
    assert np.array_equal(norms[:d], np.array([2.0 ** (j % 7 - 3) for j in range(d)], np.float32))
    assert np.all(norms[d:] == 1.0)


def test_zero_key_is_all_plus_one():
    d, m = 128, 256
    S = oracle.sketch(SEED, d, m)
    words, norms = oracle.encode(np.zeros((3, d), dtype=np.uint16), S)
    assert np.all(words == 0xFFFFFFFF)
    assert np.all(norms == 0.0)
    # -0.0 entries are zeros too
    words2, _ = oracle.encode(np.full((1, d), 0x8000, dtype=np.uint16), S)
    assert np.all(words2 == 0xFFFFFFFF)


def test_exact_cancellation_gives_plus_one():
    d, m = 128, 256
    S = oracle.sketch(SEED, d, m)
    rng = np.random.default_rng(5)
    rows = []
    targets = []
    for _ in range(40):
        a, b = rng.choice(d, size=2, replace=False)
        i = int(rng.integers(m))
        k = np.zeros(d)
        k[a] = S[b, i]
        k[b] = -S[a, i]           # k_a S[a,i] + k_b S[b,i] = 0 exactly
        rows.append(k)
        targets.append(i)
    words, _ = oracle.encode(bf16(np.array(rows)), S)
    bits = oracle.unpack_signs(words, m)
    for r, i in enumerate(targets):
        assert bits[r, i] == 1


def test_near_cancellation_needs_exact_sum():
    """Two huge products cancel; a tiny third term decides the sign.

    In float64 the tiny term is lost whenever it is added to a huge partial
    sum, so only an exact evaluation gets these bits right.
    """
    d, m = 128, 256
    S = oracle.sketch(SEED, d, m)
    rng = np.random.default_rng(9)
    rows, want = [], []
    for n in range(60):
        a, b, c = rng.choice(d, size=3, replace=False)
        i = int(rng.integers(m))
        k = np.zeros(d)
        k[a] = S[b, i] * 2.0 ** 60
        k[b] = -S[a, i] * 2.0 ** 60
        sgn = 1.0 if n % 2 else -1.0
        k[c] = sgn * 2.0 ** -60 * np.sign(S[c, i])   # term = sgn * 2^-60 |S[c,i]|
        rows.append(k)
        want.append((i, 1 if sgn > 0 else 0))
    words, _ = oracle.encode(bf16(np.array(rows)), S)
    bits = oracle.unpack_signs(words, m)
    for r, (i, w) in enumerate(want):
        assert bits[r, i] == w


def test_matches_exact_rational_brute_force():
    d, m = 8, 32
    S = oracle.sketch(SEED, d, m)
    rng = np.random.default_rng(11)
    K = rng.standard_normal((24, d)) * np.exp(rng.standard_normal((24, d)) * 3)
    # plant exact cancellations and zero keys
    K[0] = 0.0
    K[1, :] = 0.0
    K[1, 0], K[1, 1] = S[1, 3], -S[0, 3]
    K[2, :] = 0.0
    K[2, 2], K[2, 5] = S[5, 7] * 2.0 ** 40, -S[2, 7] * 2.0 ** 40
    K[2, 6] = 2.0 ** -40
    keys = bf16(K)
    words, _ = oracle.encode(keys, S)
    brute = oracle.exact_sign_fraction(keys, S)
    assert np.array_equal(oracle.unpack_signs(words, m), brute)


def test_scaling_by_powers_of_two_keeps_bits():
    d, m = 128, 256
    S = oracle.sketch(SEED, d, m)
    rng = np.random.default_rng(3)
    K = bf16(rng.standard_normal((32, d)))
    Kf = oracle.bf16_bits_to_float64(K)
    w0, n0 = oracle.encode(K, S)
    for p in (-100, -20, 7, 90):
        w, n = oracle.encode(bf16(Kf * 2.0 ** p), S)
        assert np.array_equal(w, w0)
        assert np.array_equal(n, (n0.astype(np.float64) * 2.0 ** p).astype(np.float32))


def test_negation_complements_nonzero_projections():
    d, m = 128, 256
    S = oracle.sketch(SEED, d, m)
    rng = np.random.default_rng(4)
    K = bf16(rng.standard_normal((16, d)))
    Kneg = K ^ np.uint16(0x8000)
    w, _ = oracle.encode(K, S)
    wn, _ = oracle.encode(Kneg, S)
    P = oracle.bf16_bits_to_float64(K) @ S
    nonzero = oracle.unpack_signs(np.full((1, m // 32), 0xFFFFFFFF, np.uint32), m)[0] * (np.abs(P) > 0)
    b, bn = oracle.unpack_signs(w, m), oracle.unpack_signs(wn, m)
    assert np.all((b ^ bn)[nonzero.astype(bool)] == 1)


def test_norm_closed_forms():
    d, m = 128, 256
    S = oracle.sketch(SEED, d, m)
    K = np.zeros((3, d))
    K[0] = 1.0
    K[1, 0], K[1, 1] = 3.0, 4.0
    K[2, 5] = -2.0 ** -126            # smallest normal: its square is exact in fp64
    _, n = oracle.encode(bf16(K), S)
    assert n[0] == np.float32(math.sqrt(128.0))
    assert n[1] == 5.0
    assert n[2] == np.float32(2.0 ** -126)


def test_projection_orientation_against_explicit_sum():
    """bit i uses column i of S (sum over the key channel j), not row i."""
    d, m = 32, 64
    S = oracle.sketch(SEED, d, m)
    rng = np.random.default_rng(8)
    K = bf16(rng.standard_normal((8, d)))
    Kf = oracle.bf16_bits_to_float64(K)
    words, _ = oracle.encode(K, S)
    bits = oracle.unpack_signs(words, m)
    for t in range(8):
        for i in range(m):
            s = sum(Kf[t, j] * S[j, i] for j in range(d))
            assert bits[t, i] == (1 if s >= 0 else 0)
