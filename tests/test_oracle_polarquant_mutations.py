"""Planted mistakes in the PolarQuant oracle (CPU only) must be caught by its
pins (tests/test_oracle_polarquant.py)."""

import math

import numpy as np
import pytest
from scipy import special

from oracle import polarquant as pq

from . import test_oracle_polarquant as tpq


def _fails(fn, *args):
    with pytest.raises(AssertionError):
        fn(*args)


def test_wrong_level_exponent_is_caught(monkeypatch):
    """sin^(2^(l-1))(2 psi) instead of sin^(2^(l-1) - 1)(2 psi)."""
    def cdf_wrong(psi, level):
        a = 2 ** (level - 2) + 0.5
        psi = np.clip(np.asarray(psi, dtype=np.float64), 0.0, math.pi / 2)
        return special.betainc(a, a, np.sin(psi) ** 2)
    monkeypatch.setattr(pq, "level_cdf", cdf_wrong)
    _fails(tpq.test_level_laws_and_independence_on_gaussian_vectors)


def test_swapped_halves_are_caught(monkeypatch):
    """atan(first half / second half) instead of second / first."""
    def transform_swapped(y):
        y = np.asarray(y, dtype=np.float64)
        a, b = y[:, 0::2], y[:, 1::2]
        angles = [np.mod(np.arctan2(b, a), 2 * math.pi)]
        rho = np.hypot(a, b)
        while rho.shape[1] > 1:
            ra, rb = rho[:, 0::2], rho[:, 1::2]
            angles.append(np.arctan2(ra, rb))
            rho = np.hypot(ra, rb)
        return angles, rho[:, 0]
    monkeypatch.setattr(pq, "polar_transform", transform_swapped)
    _fails(tpq.test_transform_inverts_exactly)


def test_strict_threshold_is_caught(monkeypatch):
    """s_b > T^2 s_a instead of >= (the zero slices take the wrong cell)."""
    def upper_strict(y, bit_alloc):
        y = np.asarray(y, dtype=np.float64)
        s = y[:, 0::2] ** 2 + y[:, 1::2] ** 2
        out, lev = [], 2
        while s.shape[1] > 1:
            sa, sb = s[:, 0::2], s[:, 1::2]
            _, _, T = pq.level_codebook(lev, bit_alloc[lev - 1])
            cells = np.zeros(sa.shape, dtype=np.int64)
            for t in T:
                cells += (sb > (t * t) * sa)
            out.append(cells)
            s, lev = sa + sb, lev + 1
        return out, s[:, 0]
    monkeypatch.setattr(pq, "upper_cells", upper_strict)
    _fails(tpq.test_special_pairs)
