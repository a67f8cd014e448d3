"""Pins for the oracle's estimator: unbiasedness, variance, constant, identities.

"The Geometry of Forgetting", QJL section: with Gaussian S the estimator of
<y, x> from sign(Sx) and the plain JL transform of y is unbiased, its variance
is at most pi/(2d) ||y||^2 (unit x, d sketch rows), and sqrt(pi/2) inverts
E[<s,y> sign<s,x>] = sqrt(2/pi) <y,x>/||x||.  "QJL: 1-Bit Quantized JL
Transform ...", Abstract: asymmetric, unbiased estimator.

With m sketch rows and the stored norm the estimator reads
sqrt(pi/2)/m * ||k|| * <S^T q, sign(S^T k)>, whose exact variance is
((pi/2) ||q||^2 ||k||^2 - <q,k>^2) / m (each of the m rows contributes an
independent term with second moment (pi/2) ||k||^2 E<s,q>^2).
"""

import math

import numpy as np
import pytest

import oracle


def mc_estimates(q, k, m, trials, rng):
    """Estimator values over independent fp64 Gaussian S draws (oracle calls)."""
    d = q.size
    kb = oracle.float64_to_bf16_bits(k[None, :])
    out = np.empty(trials)
    for t in range(trials):
        S = rng.standard_normal((d, m))
        words, norms = oracle.encode(kb, S)
        out[t] = oracle.estimate_scores(oracle.query_sketch(q, S), words, norms)[0, 0]
    return out


def exact_variance(q, k, m):
    return ((math.pi / 2) * (q @ q) * (k @ k) - (q @ k) ** 2) / m


@pytest.mark.parametrize("case", ["correlated", "anti", "orthogonalish"])
def test_unbiased_and_variance_closed_form(case):
    rng = np.random.default_rng({"correlated": 1, "anti": 2, "orthogonalish": 3}[case])
    d, m, trials = 24, 64, 6000
    k = oracle.bf16_bits_to_float64(oracle.float64_to_bf16_bits(rng.standard_normal(d) * 3.0))
    if case == "correlated":
        q = 0.8 * k / np.linalg.norm(k) * 2.0 + 0.3 * rng.standard_normal(d)
    elif case == "anti":
        q = -0.6 * k + 0.2 * rng.standard_normal(d)
    else:
        q = rng.standard_normal(d)
    est = mc_estimates(q, k, m, trials, rng)
    var = exact_variance(q, k, m)
    se = math.sqrt(var / trials)
    assert abs(est.mean() - q @ k) < 4.5 * se, (est.mean(), q @ k, se)
    assert abs(est.var() / var - 1.0) < 0.12
    # the stated bound (m rows, general norms)
    assert var <= math.pi / (2 * m) * (q @ q) * (k @ k)


def test_half_space_identity_constant():
    rng = np.random.default_rng(21)
    d, n = 16, 400000
    x = rng.standard_normal(d)
    y = rng.standard_normal(d)
    s = rng.standard_normal((n, d))
    sample = (s @ y) * np.where(s @ x >= 0, 1.0, -1.0)
    target = math.sqrt(2 / math.pi) * (y @ x) / np.linalg.norm(x)
    assert abs(sample.mean() - target) < 4.5 * sample.std() / math.sqrt(n)
    assert abs(oracle.ESTIMATOR_CONST * math.sqrt(2 / math.pi) - 1.0) < 1e-15


def test_dequantizer_form_equals_estimator():
    d, m = 128, 256
    S = oracle.sketch(42, d, m)
    rng = np.random.default_rng(4)
    K = oracle.float64_to_bf16_bits(rng.standard_normal((50, d)) * 2)
    q = rng.standard_normal((3, d))
    words, norms = oracle.encode(K, S)
    est = oracle.estimate_scores(oracle.query_sketch(q, S), words, norms)
    via_dequant = q @ oracle.dequantize(words, norms, S).T
    assert np.allclose(est, via_dequant, rtol=1e-12, atol=1e-12)


def test_one_hot_closed_form():
    """q = e_j, k = e_j: estimate = sqrt(pi/2)/m * sum_i |S[j, i]| (hand-derived)."""
    d, m = 128, 256
    S = oracle.sketch(42, d, m)
    for j in (0, 17, 127):
        k = np.zeros((1, d))
        k[0, j] = 1.0
        q = k[0].copy()
        words, norms = oracle.encode(oracle.float64_to_bf16_bits(k), S)
        est = oracle.estimate_scores(oracle.query_sketch(q, S), words, norms)[0, 0]
        want = math.sqrt(math.pi / 2) / m * np.abs(S[j]).sum()
        assert abs(est - want) < 1e-12
        # the estimate of ||e_j||^2 = 1 is within a few standard deviations
        assert abs(est - 1.0) < 4 * math.sqrt((math.pi / 2 - 1) / m)


def test_attention_converges_to_exact_as_m_grows():
    """The score variance falls like 1/m, so QJL attention approaches exact attention."""
    rng = np.random.default_rng(12)
    d, N, H = 64, 256, 4
    K = oracle.float64_to_bf16_bits(rng.standard_normal((1, 1, N, d)))
    V = oracle.float64_to_bf16_bits(rng.standard_normal((1, 1, N, d)))
    q = rng.standard_normal((1, H, d)) * 2.0
    ref = oracle.exact_attention(q, K, V, N)
    errs = []
    for m in (64, 256, 1024, 4096):
        S = oracle.sketch(1234, d, m)
        words, norms = oracle.encode(K.reshape(N, d), S)
        out = oracle.decode(q, words.reshape(1, 1, N, -1), norms.reshape(1, 1, N), V, N, S)
        errs.append(np.linalg.norm(out - ref) / np.linalg.norm(ref))
    assert errs[-1] < errs[0] / 4.0, errs
    assert all(b < a * 1.2 for a, b in zip(errs, errs[1:])), errs
