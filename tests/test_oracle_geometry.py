"""Pins for the rotation facts and the rotated-coordinate density.

"The Geometry of Forgetting", section "Random rotation, and what high
dimensions do to your intuitions": rotations keep lengths and inner products;
a coordinate of a randomly rotated unit vector has the scaled-Beta density
Gamma(d/2)/(sqrt(pi) Gamma((d-1)/2)) (1-x^2)^((d-3)/2), close to N(0, 1/d)
for large d.
"""

import math

import numpy as np
import pytest
from scipy import integrate, stats

import oracle


def test_rotation_preserves_norms_and_inner_products():
    rng = np.random.default_rng(1)
    for d in (3, 16, 128):
        P = oracle.haar_rotation(d, rng)
        assert np.allclose(P.T @ P, np.eye(d), atol=1e-12)
        x, y = rng.standard_normal(d), rng.standard_normal(d)
        assert abs(np.linalg.norm(P @ x) - np.linalg.norm(x)) < 1e-12 * np.linalg.norm(x)
        assert abs((P @ x) @ (P @ y) - x @ y) < 1e-12 * np.linalg.norm(x) * np.linalg.norm(y)


def test_rotation_is_haar_distributed():
    """Trace moments of a Haar orthogonal matrix: E[tr] = 0, E[tr^2] = 1 (d >= 2)."""
    rng = np.random.default_rng(2)
    d, T = 6, 4000
    tr = np.array([np.trace(oracle.haar_rotation(d, rng)) for _ in range(T)])
    assert abs(tr.mean()) < 4.5 / math.sqrt(T)
    assert abs((tr ** 2).mean() - 1.0) < 0.12


@pytest.mark.parametrize("d", [3, 8, 128])
def test_density_mass_and_second_moment(d):
    f = lambda x: float(oracle.rotated_coordinate_density(np.array([x]), d)[0])
    mass, _ = integrate.quad(f, -1, 1)
    m2, _ = integrate.quad(lambda x: x * x * f(x), -1, 1)
    assert abs(mass - 1.0) < 1e-8
    assert abs(m2 - 1.0 / d) < 1e-8


def test_density_special_cases():
    # d = 3: uniform on [-1, 1] (Archimedes' hat-box theorem)
    xs = np.linspace(-0.99, 0.99, 41)
    assert np.allclose(oracle.rotated_coordinate_density(xs, 3), 0.5, atol=1e-14)
    # large d: close to the N(0, 1/d) density
    d = 128
    xs = np.linspace(-0.2, 0.2, 21)
    normal = stats.norm(scale=1 / math.sqrt(d)).pdf(xs)
    assert np.allclose(oracle.rotated_coordinate_density(xs, d), normal, rtol=0.02)
    # CDF agrees with the integral of the density
    for d in (3, 8, 128):
        for x in (-0.5, -0.05, 0.0, 0.1, 0.7):
            val, _ = integrate.quad(
                lambda t: float(oracle.rotated_coordinate_density(np.array([t]), d)[0]), -1, x)
            assert abs(val - float(oracle.rotated_coordinate_cdf(np.array([x]), d)[0])) < 1e-8


@pytest.mark.parametrize("d", [3, 8, 128])
def test_rotated_unit_vector_coordinates_fit_density(d):
    rng = np.random.default_rng(100 + d)
    x = rng.standard_normal(d)
    x /= np.linalg.norm(x)
    T = 3000 if d < 128 else 600
    coords = np.concatenate([(oracle.haar_rotation(d, rng) @ x)[: min(d, 4)] for _ in range(T)])
    res = stats.kstest(coords, lambda v: oracle.rotated_coordinate_cdf(v, d))
    assert res.pvalue > 1e-3
    if d == 128:
        assert stats.kstest(coords, stats.norm(scale=1 / math.sqrt(d)).cdf).pvalue > 1e-3
