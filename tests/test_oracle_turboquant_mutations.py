"""Planted mistakes in the TurboQuant oracle (CPU only) must be caught by
its pins (tests/test_oracle_turboquant.py)."""

import numpy as np
import pytest

from oracle import turboquant as tq

from . import test_oracle_turboquant as ttq


def _fails(fn, *args):
    with pytest.raises(AssertionError):
        fn(*args)


def test_boundaries_at_centroids_are_caught(monkeypatch):
    real = tq.lloyd_max_exact

    def lm_wrong_cells(d, k, tol=1e-15, max_iter=100000):
        c = real(d, k)
        # one Lloyd step with cells split at the centroids' quarter points
        edges = np.concatenate([[-1.0], 0.75 * c[:-1] + 0.25 * c[1:], [1.0]])
        return np.diff(tq._first_moment(edges, d)) / np.diff(tq._cdf(edges, d))
    monkeypatch.setattr(tq, "lloyd_max_exact", lm_wrong_cells)
    _fails(ttq.test_lloyd_max_conditions_by_quadrature, 2)


def test_dropped_qjl_term_is_caught(monkeypatch):
    real = tq.estimate_with

    def est_mse_only(q, idx, bits, n, g, k, rot, S):
        return real(q, idx, bits, n, np.zeros_like(g), k, rot, S)
    monkeypatch.setattr(tq, "estimate_with", est_mse_only)
    _fails(ttq.test_unbiased_inner_products)


def test_constant_over_d_instead_of_m_is_caught(monkeypatch):
    real = tq.estimate_with

    def est_over_d(q, idx, bits, n, g, k, rot, S):
        d, m = S.shape
        return real(q, idx, bits, n, np.asarray(g, np.float64) * m / d, k, rot, S)
    monkeypatch.setattr(tq, "estimate_with", est_over_d)
    _fails(ttq.test_unbiased_inner_products)


def test_flipped_residual_sign_is_caught(monkeypatch):
    real = tq.encode_with

    def enc_flip(keys, k, rot, S):
        idx, b, n, g = real(keys, k, rot, S)
        return idx, ~b, n, g
    monkeypatch.setattr(tq, "encode_with", enc_flip)
    _fails(ttq.test_unbiased_inner_products)


def test_rotation_without_sign_fix_is_caught(monkeypatch):
    def rot_nofix(seed, d):
        Q, _ = np.linalg.qr(tq._sketch_f64(seed, d, d))
        return Q
    tq.rotation_f64.cache_clear()
    monkeypatch.setattr(tq, "rotation_f64", rot_nofix)
    try:
        _fails(ttq.test_rotation_is_orthogonal_to_fp32_precision)
    finally:
        monkeypatch.undo()
        tq.rotation_f64.cache_clear()


def test_unrotated_codes_are_caught(monkeypatch):
    """Quantizing the key's own coordinates (no rotation): the Beta law no
    longer holds for keys with outlier channels, so the Monte-Carlo MSE pin
    fails on such keys."""
    real = tq.rotate_rn32

    def no_rotation(K, rot):
        return real(K, np.eye(K.shape[1]))
    monkeypatch.setattr(tq, "rotate_rn32", no_rotation)
    _fails(ttq.test_rotation_makes_structured_keys_look_random)
