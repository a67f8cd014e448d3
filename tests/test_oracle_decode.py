"""Pins for the oracle's decode step: closed forms and special cases.

Decode = softmax over scale * (estimated <q, k_t>) followed by the weighted
sum of bf16 values; query head h reads kv head h // (H_q / H_kv).
"""

import math

import numpy as np

import oracle

SEED = 42


def bf16(x):
    return oracle.float64_to_bf16_bits(np.asarray(x, dtype=np.float64))


def encode_cache(K_bits, S):
    B, H, N, d = K_bits.shape
    words, norms = oracle.encode(K_bits.reshape(-1, d), S)
    return words.reshape(B, H, N, -1), norms.reshape(B, H, N)


def test_single_token_returns_its_value():
    d, m = 128, 256
    S = oracle.sketch(SEED, d, m)
    rng = np.random.default_rng(1)
    K = bf16(rng.standard_normal((2, 2, 1, d)))
    V = bf16(rng.standard_normal((2, 2, 1, d)))
    q = rng.standard_normal((2, 6, d))
    w, n = encode_cache(K, S)
    out = oracle.decode(q, w, n, V, 1, S)
    Vf = oracle.bf16_bits_to_float64(V)
    for b in range(2):
        for h in range(6):
            assert np.array_equal(out[b, h], Vf[b, h // 3, 0])


def test_zero_query_and_identical_keys_give_mean_value():
    d, m, N = 128, 256, 37
    S = oracle.sketch(SEED, d, m)
    rng = np.random.default_rng(2)
    V = bf16(rng.standard_normal((1, 1, N, d)))
    Vmean = oracle.bf16_bits_to_float64(V)[0, 0].mean(axis=0)
    K = bf16(rng.standard_normal((1, 1, N, d)))
    w, n = encode_cache(K, S)
    out = oracle.decode(np.zeros((1, 2, d)), w, n, V, N, S)
    assert np.allclose(out[0], Vmean[None, :], rtol=0, atol=1e-12)
    Ksame = np.repeat(K[:, :, :1], N, axis=2)
    w, n = encode_cache(Ksame, S)
    out = oracle.decode(rng.standard_normal((1, 2, d)), w, n, V, N, S)
    assert np.allclose(out[0], Vmean[None, :], rtol=0, atol=1e-12)


def test_two_tokens_hand_computed():
    """Keys a*e_j0 and b*e_j1, query alpha*e_j0, estimate worked out from S.

    est_0 = c * a * alpha * sum_i |S[j0,i]|,
    est_1 = c * b * alpha * sum_i S[j0,i] * sgn(S[j1,i]),  c = sqrt(pi/2)/m,
    with sgn(0) = +1; the output is sigma(scale (est_0 - est_1)) V_0 + (1 - sigma) V_1.
    """
    d, m = 128, 256
    S = oracle.sketch(SEED, d, m)
    rng = np.random.default_rng(3)
    j0, j1, a, b, alpha = 5, 77, 1.5, 3.0, 2.0
    K = np.zeros((1, 1, 2, d))
    K[0, 0, 0, j0] = a
    K[0, 0, 1, j1] = b
    V = bf16(rng.standard_normal((1, 1, 2, d)))
    q = np.zeros((1, 1, d))
    q[0, 0, j0] = alpha
    w, n = encode_cache(bf16(K), S)
    for scale in (None, 0.37):
        out = oracle.decode(q, w, n, V, 2, S, scale=scale)
        c = math.sqrt(math.pi / 2) / m
        sgn1 = np.where(S[j1] >= 0, 1.0, -1.0)
        est0 = c * a * alpha * np.abs(S[j0]).sum()
        est1 = c * b * alpha * (S[j0] * sgn1).sum()
        sc = 1 / math.sqrt(d) if scale is None else scale
        p0 = 1.0 / (1.0 + math.exp(-sc * (est0 - est1)))
        Vf = oracle.bf16_bits_to_float64(V)[0, 0]
        want = p0 * Vf[0] + (1 - p0) * Vf[1]
        assert np.allclose(out[0, 0], want, rtol=1e-12, atol=1e-12)


def test_gqa_head_mapping():
    d, m, N, Hkv, G = 64, 128, 20, 3, 4
    S = oracle.sketch(SEED, d, m)
    rng = np.random.default_rng(4)
    K = bf16(rng.standard_normal((1, Hkv, N, d)))
    V = bf16(np.broadcast_to(np.arange(1, Hkv + 1, dtype=np.float64)[None, :, None, None],
                             (1, Hkv, N, d)))
    q = rng.standard_normal((1, Hkv * G, d))
    w, n = encode_cache(K, S)
    out = oracle.decode(q, w, n, V, N, S)
    for h in range(Hkv * G):
        assert np.allclose(out[0, h], h // G + 1, rtol=0, atol=1e-12)


def test_only_first_N_tokens_are_read():
    d, m, cap, N = 64, 128, 50, 31
    S = oracle.sketch(SEED, d, m)
    rng = np.random.default_rng(6)
    K = bf16(rng.standard_normal((1, 1, cap, d)))
    V = bf16(rng.standard_normal((1, 1, cap, d)))
    q = rng.standard_normal((1, 1, d))
    w, n = encode_cache(K, S)
    ref = oracle.decode(q, w, n, V, N, S)
    V2 = V.copy()
    V2[:, :, N:] = bf16(np.full((1, 1, cap - N, d), 1e30))
    w2 = w.copy()
    w2[:, :, N:] = 0
    assert np.array_equal(oracle.decode(q, w2, n, V2, N, S), ref)
