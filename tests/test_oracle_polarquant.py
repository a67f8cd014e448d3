"""Pins for the PolarQuant oracle (oracle/polarquant.py), CPU only.

"The Geometry of Forgetting: How Three Papers Cracked KV Cache
Quantization", section "PolarQuant: skipping Cartesian altogether": the
recursive polar transform; for a Gaussian vector the radius and all angles
are independent, level-1 angles uniform on [0, 2 pi), level-l angles with
density proportional to sin^(2^(l-1) - 1)(2 psi); per-level codebooks; more
than 4.2x compression.
"""

import math

import numpy as np
import pytest
from scipy import integrate, stats

import oracle
from oracle import polarquant as pq
from jl_rotated_bit_amd import workloads as wl

D = 128


def test_transform_inverts_exactly():
    rng = np.random.default_rng(1)
    y = rng.standard_normal((50, D))
    angles, radius = pq.polar_transform(y)
    assert [a.shape[1] for a in angles] == [64, 32, 16, 8, 4, 2, 1]
    assert np.allclose(radius, np.linalg.norm(y, axis=1), rtol=1e-14)
    assert np.allclose(pq.polar_inverse(angles, radius), y, atol=1e-12)
    # level-l angle = atan(norm of the slice's second half / first half)
    s = y[3, 8:16]
    assert math.isclose(angles[2][3, 1], math.atan2(np.linalg.norm(s[4:]), np.linalg.norm(s[:4])),
                        rel_tol=1e-13)


def test_level_laws_and_independence_on_gaussian_vectors():
    """The page's joint law: uniform level-1 angles, sin^(2^(l-1)-1)(2 psi)
    at level l, radius and angles independent (Kolmogorov-Smirnov against
    the level CDFs; correlations near zero)."""
    rng = np.random.default_rng(2)
    y = rng.standard_normal((6000, D))
    angles, radius = pq.polar_transform(y)
    a1 = angles[0][:, :4].ravel()
    assert stats.kstest(a1, stats.uniform(loc=0, scale=2 * math.pi).cdf).pvalue > 1e-3
    for lev in range(2, 8):
        a = angles[lev - 1][:, 0]
        assert stats.kstest(a, lambda x: pq.level_cdf(x, lev)).pvalue > 1e-3, lev
        assert abs(np.corrcoef(a, radius)[0, 1]) < 0.06
    # and the laws are normalized densities
    for lev in range(2, 8):
        mass = integrate.quad(lambda x: float(pq.level_density(x, lev)), 0, math.pi / 2, limit=200)[0]
        assert abs(mass - 1.0) < 1e-9


@pytest.mark.parametrize("lev", [2, 3, 5, 7])
def test_level_codebook_lloyd_conditions(lev):
    """Centroids are conditional means of their cells (independent
    trapezoid integration of the density), symmetric about pi/4."""
    c = pq.lloyd_max_level(lev, 2)
    edges = np.concatenate([[0.0], 0.5 * (c[:-1] + c[1:]), [math.pi / 2]])
    for v in range(len(c)):
        x = np.linspace(edges[v], edges[v + 1], 200001)
        f = pq.level_density(x, lev)
        assert abs(np.trapezoid(x * f, x) / np.trapezoid(f, x) - c[v]) < 1e-8
    assert np.allclose(c + c[::-1], math.pi / 2, atol=1e-12)
    cq, bounds, T = pq.level_codebook(lev, 2)
    assert np.all(np.abs(cq - c) <= 2.0 ** -21)
    assert np.allclose(T, np.tan(bounds), atol=2.0 ** -21)


def test_cells_agree_with_angles():
    """Cells from the comparison rules equal the cells of the atan2 angles
    (away from boundaries, where both are unambiguous)."""
    rng = np.random.default_rng(3)
    y = rng.standard_normal((3000, D)).astype(np.float32).astype(np.float64)
    angles, _ = pq.polar_transform(y)
    c1 = pq.level1_cells(y, 4)
    cents, bounds, _ = pq.level_codebook(1, 4)
    ref1 = np.searchsorted(bounds, angles[0], side="right")
    far = np.min(np.abs(angles[0][..., None] - bounds[None, None, :]), axis=-1) > 1e-5
    assert np.array_equal(c1[far], ref1[far])
    ups, s = pq.upper_cells(y, pq.DEFAULT_BITS)
    for lev in range(2, 8):
        _, b2, _ = pq.level_codebook(lev, 2)
        a = angles[lev - 1]
        ref = np.searchsorted(b2, a, side="right")
        far = np.min(np.abs(a[..., None] - b2[None, None, :]), axis=-1) > 1e-5
        assert np.array_equal(ups[lev - 2][far], ref[far]), lev
    assert np.allclose(np.sqrt(s), np.linalg.norm(y, axis=1), rtol=1e-14)


def test_special_pairs():
    """Quadrant edges and the zero pair: (1, 0) -> 0, (0, 1) -> cell of pi/2,
    (-1, 0) -> cell of pi, (0, -1) -> cell of 3 pi/2, (0, 0) -> 0; a zero
    first half gives the top cell at the levels above."""
    y = np.zeros((5, D))
    y[0, :2] = [1, 0]
    y[1, :2] = [0, 1]
    y[2, :2] = [-1, 0]
    y[3, :2] = [0, -1]
    c1 = pq.level1_cells(y, 4)
    assert list(c1[:, 0]) == [0, 4, 8, 12, 0]
    ups, _ = pq.upper_cells(y, pq.DEFAULT_BITS)
    assert ups[0][4, 0] == 3          # s_a = s_b = 0
    assert ups[0][1, 0] == 0          # s_b = 0 < s_a


def test_compression_beats_the_pages_figure():
    """Stored bits per key against 16-bit keys: more than the page's 4.2x."""
    words = pq.code_words(D)
    assert words == 12
    bits = words * 32 + 32            # cells + fp32 radius
    assert 16 * D / bits > 4.2


def test_error_falls_with_bits_and_scale_invariance():
    rng = np.random.default_rng(4)
    K = wl.gaussian_keys(rng, 1500)
    Kf = oracle.bf16_bits_to_float64(K)
    errs = []
    for alloc in [(3, 1, 1, 1, 1, 1, 1), pq.DEFAULT_BITS, (5, 3, 3, 3, 3, 3, 3)]:
        codes, rad = pq.encode(K, 42, alloc)
        rec = pq.dequantize(codes, rad, 42, D, alloc)
        errs.append(float(np.mean(np.sum((rec - Kf) ** 2, 1) / np.sum(Kf ** 2, 1))))
    assert errs[0] > errs[1] > errs[2]
    assert errs[1] < 0.05
    codes, rad = pq.encode(K, 42)
    for p in (-40, 20):
        c2, r2 = pq.encode(oracle.float64_to_bf16_bits(Kf * 2.0 ** p), 42)
        assert np.array_equal(codes, c2)
        assert np.array_equal(r2, (rad.astype(np.float64) * 2.0 ** p).astype(np.float32))


def test_stream_packing():
    """Level 1 first, angle 0 in the lowest bits, then the levels above."""
    cells = [np.zeros((1, 64), np.int64)] + [np.zeros((1, 32 >> i), np.int64) for i in range(6)]
    cells[0][0, 0] = 5
    cells[0][0, 63] = 9
    cells[1][0, 0] = 3
    w = pq._pack_stream(cells, pq.DEFAULT_BITS, pq.code_words(D))
    assert w[0, 0] == 5 and (w[0, 7] >> 28) == 9 and (w[0, 8] & 3) == 3
    back = pq.unpack(w, D)
    for a, b in zip(back, cells):
        assert np.array_equal(a, b)
