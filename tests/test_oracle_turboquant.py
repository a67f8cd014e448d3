"""Pins for the TurboQuant_prod oracle (oracle/turboquant.py), CPU only.

"The Geometry of Forgetting: How Three Papers Cracked KV Cache
Quantization", section "TurboQuant: bridging MSE and inner product, in two
stages": a Lloyd-Max codebook for the rotated-coordinate density (cell
boundaries at the midpoints of adjacent centroids), D_mse <= (sqrt(3) pi / 2)
4^-b, the Shannon floor 4^-b, QJL on the residual making the inner-product
estimate unbiased, and D_prod <= sqrt(3) pi^2 ||y||^2 / d 4^-b.
"""

import math
from fractions import Fraction

import numpy as np
import pytest
from scipy import integrate

import oracle
from oracle import turboquant as tq
from jl_rotated_bit_amd import workloads as wl

D = 128
# Lloyd-Max quantizer for the unit Gaussian (J. Max, "Quantizing for minimum
# distortion", IRE Trans. Inf. Theory, 1960): positive centroids and the
# mean squared error for 1, 2 and 3 bits.
MAX_1960 = {1: ([0.7979], 0.3634), 2: ([0.4528, 1.510], 0.1175),
            3: ([0.2451, 0.7560, 1.344, 2.152], 0.03454)}


def density(x, d):
    return float(oracle.rotated_coordinate_density(np.array([x]), d)[0])


@pytest.mark.parametrize("k", [1, 2, 3])
def test_lloyd_max_conditions_by_quadrature(k):
    """Each centroid is the mean of f_X over its cell (quadrature of the
    page's density, independent of the closed forms the solver uses), the
    cells split at midpoints, and the codebook is symmetric and ascending."""
    c = tq.lloyd_max_exact(D, k)
    assert np.all(np.diff(c) > 0)
    assert np.allclose(c, -c[::-1], atol=1e-14)
    edges = np.concatenate([[-1.0], 0.5 * (c[:-1] + c[1:]), [1.0]])
    for v in range(len(c)):
        a, b = edges[v], edges[v + 1]
        mass = integrate.quad(lambda x: density(x, D), a, b, epsabs=1e-14, epsrel=1e-12, limit=200)[0]
        mom = integrate.quad(lambda x: x * density(x, D), a, b, epsabs=1e-14, epsrel=1e-12, limit=200)[0]
        assert abs(mom / mass - c[v]) < 1e-9 * max(1.0, abs(c[v])) + 1e-12
    cq, beta = tq.codebook(D, k)
    assert np.all(np.abs(cq.astype(np.float64) - c) <= tq.CENTROID_GRID / 2)
    assert np.all(cq.astype(np.float64) / tq.CENTROID_GRID == np.round(cq.astype(np.float64) / tq.CENTROID_GRID))
    assert np.array_equal(beta.astype(np.float64), 0.5 * (cq[:-1].astype(np.float64) + cq[1:]))
    assert np.array_equal(cq, -cq[::-1])


@pytest.mark.parametrize("k", [1, 2, 3, 4])
def test_mse_bound_and_shannon_floor(k):
    """d times the per-coordinate distortion (the D_mse of a unit vector) lies
    between the Shannon floor 4^-k and the page's (sqrt(3) pi / 2) 4^-k; the
    closed-form distortion equals quadrature."""
    cq, beta = tq.codebook(D, k)
    dist = tq.coordinate_distortion(cq, D)
    edges = np.concatenate([[-1.0], beta.astype(np.float64), [1.0]])
    quad = sum(integrate.quad(lambda x: (x - float(cq[v])) ** 2 * density(x, D), edges[v], edges[v + 1],
                              epsabs=1e-15, epsrel=1e-11, limit=200)[0] for v in range(len(cq)))
    assert abs(dist - quad) < 1e-9 * quad
    assert 4.0 ** -k <= D * dist <= math.sqrt(3) * math.pi / 2 * 4.0 ** -k


@pytest.mark.parametrize("k", [1, 2, 3])
def test_codebook_tends_to_the_gaussian_lloyd_max(k):
    """For large d the density tends to N(0, 1/d), so sqrt(d) times the
    codebook tends to the published Gaussian Lloyd-Max quantizer."""
    d = 1 << 14
    c = tq.lloyd_max_exact(d, k)
    cents, dist = MAX_1960[k]
    assert np.allclose(np.sqrt(d) * c[len(c) // 2:], cents, atol=2e-3)
    assert abs(d * tq.coordinate_distortion(c, d) - dist) < 1e-3


def test_rotation_is_orthogonal_to_fp32_precision():
    for seed in (42, 7):
        R = tq.rotation(seed, D).astype(np.float64)
        assert np.abs(R @ R.T - np.eye(D)).max() < 1e-6
        Rf = tq.rotation_f64(seed, D)
        assert np.abs(Rf @ Rf.T - np.eye(D)).max() < 1e-13
        # Gram-Schmidt of the seeded Gaussian with positive R diagonal: the
        # first row of Pi^T (first column of Q) is the first Gaussian column
        # normalized
        A = oracle.qjl._sketch_f64(seed, D, D)
        assert np.allclose(Rf[:, 0], A[:, 0] / np.linalg.norm(A[:, 0]), atol=1e-13)


def test_rotated_rounding_is_exact_by_brute_force():
    """y = fp32 rounding of the exact rotation, checked against exact
    rationals with an independent round-to-nearest-even on a few keys,
    including ones built to land on fp32 rounding midpoints."""
    rng = np.random.default_rng(3)
    rot = tq.rotation(42, D).astype(np.float64)
    K = wl.gaussian_keys(rng, 6)
    # keys that make y_0 exactly a midpoint-ish value: k = e_j scaled picks
    # one rotation entry (exact), combinations of two entries give sums with
    # more bits than fp32 keeps
    extra = np.zeros((4, D))
    extra[0, 5] = 1.0
    extra[1, [3, 9]] = [1.0, 2.0 ** -24]
    extra[2, [3, 9]] = [3.0, -2.0 ** -20]
    extra[3, [1, 2, 4]] = [1.0, 1.0, 2.0 ** -30]
    Kb = np.concatenate([K, oracle.float64_to_bf16_bits(extra)])
    Kf = oracle.bf16_bits_to_float64(Kb)
    y = tq.rotate_rn32(Kf, rot)

    def rne32(x: Fraction) -> np.float32:
        f = np.float32(float(x))
        best = None
        for cand in (np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))):
            dist = abs(Fraction(float(cand)) - x)
            even = (int(np.float32(cand).view(np.uint32)) & 1) == 0
            key = (dist, not even)
            if best is None or key < best[0]:
                best = (key, cand)
        return best[1]
    for t in range(Kf.shape[0]):
        for i in range(0, D, 7):
            exact = sum((Fraction(float(Kf[t, j])) * Fraction(float(rot[i, j])) for j in range(D)), Fraction(0))
            assert y[t, i] == rne32(exact), (t, i)


def test_residual_signs_are_exact():
    """Bits are the signs of the exact S^T r (exact rationals on a subset)."""
    rng = np.random.default_rng(4)
    K = wl.gaussian_keys(rng, 5)
    rot = tq.rotation(42, D).astype(np.float64)
    S = oracle.sketch(43, D, D)
    idx, bits, n, g = tq.encode_with(K, 2, rot, S)
    cents, _ = tq.codebook(D, 2)
    Kf = oracle.bf16_bits_to_float64(K)
    y = tq.rotate_rn32(Kf, rot)
    for t in range(5):
        u = (y[t] / n[t]).astype(np.float32)
        r = (u - cents[idx[t]]).astype(np.float32)
        for l in range(0, D, 5):
            z = sum((Fraction(float(r[i])) * Fraction(float(S[i, l])) for i in range(D)), Fraction(0))
            assert bits[t, l] == (z >= 0)


def test_scale_invariance_and_zero_key():
    """Keys scaled by 2^p keep codes, bits and residual norm (u = y/n is
    invariant under exact scaling); n scales by 2^p.  A zero key takes
    u = 0 (the upper middle cell) and n = 0."""
    rng = np.random.default_rng(5)
    K = wl.gaussian_keys(rng, 64)
    Kf = oracle.bf16_bits_to_float64(K)
    c0, b0, n0, g0 = tq.encode(K, 2, 42)
    for p in (-30, 17):
        c1, b1, n1, g1 = tq.encode(oracle.float64_to_bf16_bits(Kf * 2.0 ** p), 2, 42)
        assert np.array_equal(c0, c1) and np.array_equal(b0, b1) and np.array_equal(g0, g1)
        assert np.array_equal(n1, (n0.astype(np.float64) * 2.0 ** p).astype(np.float32))
    z = np.zeros((1, D), np.uint16)
    cz, bz, nz, gz = tq.encode(z, 2, 42)
    assert nz[0] == 0
    assert np.all(tq.unpack_codes(cz, D, 2) == 2)


def test_code_packing_round_trip():
    rng = np.random.default_rng(6)
    for k in (1, 2, 3):
        idx = rng.integers(0, 2 ** k, (7, D)).astype(np.uint32)
        w = tq._pack_codes(idx, k)
        assert w.shape == (7, D * k // 32)
        assert np.array_equal(tq.unpack_codes(w, D, k), idx)
    # coordinate 0 in the lowest bits of word 0, coordinate 16 in word 1 (k = 2)
    idx = np.zeros((1, D), np.uint32)
    idx[0, 0], idx[0, 16] = 3, 1
    w = tq._pack_codes(idx, 2)
    assert w[0, 0] == 3 and w[0, 1] == 1


def test_mse_stage_monte_carlo():
    """Random unit keys: E ||u - c[idx]||^2 over keys matches d times the
    per-coordinate distortion (within 5%) and stays below the page's bound."""
    rng = np.random.default_rng(7)
    for k in (1, 2, 3):
        x = rng.standard_normal((4000, D))
        x /= np.linalg.norm(x, axis=1, keepdims=True)
        K = oracle.float64_to_bf16_bits(x)
        rot = tq.rotation(42, D).astype(np.float64)
        S = oracle.sketch(43, D, D)
        idx, bits, n, g = tq.encode_with(K, k, rot, S)
        mse = float(np.mean(g.astype(np.float64) ** 2))
        cq, _ = tq.codebook(D, k)
        want = D * tq.coordinate_distortion(cq, D)
        assert abs(mse - want) < 0.05 * want, (k, mse, want)
        assert mse <= math.sqrt(3) * math.pi / 2 * 4.0 ** -k


def _mc_estimates(q, K, k, T, rng, m=D, new_rotation=False):
    """Estimates of <q, k> over T independent draws of the residual sketch S
    (fp64 Gaussian: the method's S) and, if asked, of the rotation."""
    rot = tq.rotation(42, D).astype(np.float64)
    out = np.empty((T, K.shape[0]))
    for t in range(T):
        if new_rotation:
            rot = oracle.haar_rotation(D, rng).astype(np.float32).astype(np.float64)
        S = rng.standard_normal((D, m))
        idx, bits, n, g = tq.encode_with(K, k, rot, S)
        out[t] = tq.estimate_with(q, idx, bits, n, g, k, rot, S)[0]
    return out


def test_unbiased_inner_products():
    """Mean over independent residual sketches equals <q, k> within 4 sigma
    (the MSE stage alone is biased: its estimate is shown to be off)."""
    rng = np.random.default_rng(8)
    K = wl.gaussian_keys(rng, 3)
    Kf = oracle.bf16_bits_to_float64(K)
    q = rng.standard_normal((1, D))
    exact = (q @ Kf.T)[0]
    T = 3000
    est = _mc_estimates(q, K, 1, T, rng, m=64)
    mean, sd = est.mean(axis=0), est.std(axis=0, ddof=1)
    assert np.all(np.abs(mean - exact) < 4.0 * sd / math.sqrt(T) + 1e-4 * np.abs(exact)), (mean, exact)
    # the stage-one estimate n <Pi q, c[idx]> alone: biased by more than the noise
    rot = tq.rotation(42, D).astype(np.float64)
    idx, bits, n, g = tq.encode_with(K, 1, rot, np.zeros((D, 64)))
    mse_only = tq.estimate_with(q, idx, bits, n, np.zeros_like(g), 1, rot, np.zeros((D, 64)))[0]
    assert np.any(np.abs(mse_only - exact) > 8.0 * sd / math.sqrt(T))


@pytest.mark.parametrize("k", [1, 2])
def test_prod_distortion_bound(k):
    """E |<q, x> - estimate|^2 over rotations and sketches stays below the
    page's sqrt(3) pi^2 ||q||^2 / d 4^-b for unit x, b = k + 1 bits."""
    rng = np.random.default_rng(9 + k)
    x = rng.standard_normal((8, D))
    x /= np.linalg.norm(x, axis=1, keepdims=True)
    K = oracle.float64_to_bf16_bits(x)
    Kf = oracle.bf16_bits_to_float64(K)
    q = rng.standard_normal((1, D))
    est = _mc_estimates(q, K, k, 300, rng, new_rotation=True)
    exact = (q @ Kf.T)[0]
    dprod = float(np.mean((est - exact[None, :]) ** 2))
    bound = math.sqrt(3) * math.pi ** 2 * float((q @ q.T)[0, 0]) / D * 4.0 ** -(k + 1)
    assert dprod <= bound, (dprod, bound)
    # and the bound is not vacuous: the error is within a factor 8 of it
    assert dprod >= bound / 8.0


def test_rotation_makes_structured_keys_look_random():
    """After the rotation, coordinates of any fixed unit vector follow the
    same law (the page's load-bearing fact), so keys with outlier channels,
    and even one-hot keys, see the same mean squared residual as random keys
    (within 10%, averaged over many keys)."""
    rng = np.random.default_rng(12)
    k = 2
    cq, _ = tq.codebook(D, k)
    want = D * tq.coordinate_distortion(cq, D)
    scales = np.exp(rng.standard_normal(D))
    scales[rng.choice(D, 4, replace=False)] *= 20.0
    structured = rng.standard_normal((3000, D)) * scales[None, :]
    onehot = np.zeros((2 * D, D))
    onehot[np.arange(2 * D), np.arange(2 * D) % D] = np.where(np.arange(2 * D) < D, 1.0, -3.0)
    rot = tq.rotation(42, D).astype(np.float64)
    S = oracle.sketch(43, D, D)
    for X in (structured, onehot):
        idx, bits, n, g = tq.encode_with(oracle.float64_to_bf16_bits(X), k, rot, S)
        mse = float(np.mean(g.astype(np.float64) ** 2))
        assert abs(mse - want) < 0.1 * want, (mse, want)
