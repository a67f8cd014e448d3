"""Planted mistakes in the oracle (CPU only) must be caught by the pins.

Each case swaps one oracle function for a plausibly wrong variant (a dropped
term, a wrong sign rule, a reversed bit order, a wrong head mapping, a missing
temperature, a wrong constant) and checks that at least one pin test fails.
"""

import math

import numpy as np
import pytest

import oracle
from oracle import qjl as oq

from . import test_oracle_decode as tdec
from . import test_oracle_encode as tenc
from . import test_oracle_estimator as test_est


def _patch(monkeypatch, name, fn):
    monkeypatch.setattr(oq, name, fn)
    monkeypatch.setattr(oracle, name, fn)


def _fails(fn, *args):
    with pytest.raises(AssertionError):
        fn(*args)


def test_strict_sign_rule_is_caught(monkeypatch):
    real = oq._pack_bits

    def encode_strict(keys, S, chunk=1 << 16):
        K = oq.bf16_bits_to_float64(keys)
        words = real((K @ S) > 0.0)             # sign(0) -> -1: wrong
        norms = np.sqrt((K * K).sum(axis=1)).astype(np.float32)
        return words, norms
    _patch(monkeypatch, "encode", encode_strict)
    _fails(tenc.test_zero_key_is_all_plus_one)
    _fails(tenc.test_exact_cancellation_gives_plus_one)


def test_float_only_sign_is_caught(monkeypatch):
    real = oq._pack_bits

    def encode_float(keys, S, chunk=1 << 16):
        K = oq.bf16_bits_to_float64(keys)
        # sequential float64 sum in channel order, no exact re-evaluation
        P = np.zeros((K.shape[0], S.shape[1]))
        for j in range(K.shape[1]):
            P = P + K[:, j:j + 1] * S[j][None, :]
        return real(P >= 0.0), np.sqrt((K * K).sum(axis=1)).astype(np.float32)
    _patch(monkeypatch, "encode", encode_float)
    _fails(tenc.test_near_cancellation_needs_exact_sum)


def test_msb_first_packing_is_caught(monkeypatch):
    def pack_msb(bits):
        m = bits.shape[-1]
        b = bits.astype(np.uint64).reshape(bits.shape[:-1] + (m // 32, 32))
        weights = np.uint64(1) << np.arange(31, -1, -1, dtype=np.uint64)
        return (b * weights).sum(axis=-1).astype(np.uint32)
    monkeypatch.setattr(oq, "_pack_bits", pack_msb)
    _fails(tenc.test_one_hot_keys_read_back_rows_of_S, 16, 64)


def test_dropped_norm_is_caught(monkeypatch):
    real = oq.estimate_scores

    def est_no_norm(Sq, words, norms):
        return real(Sq, words, np.ones_like(np.asarray(norms)))
    _patch(monkeypatch, "estimate_scores", est_no_norm)
    _fails(test_est.test_unbiased_and_variance_closed_form, "correlated")


def test_wrong_constant_is_caught(monkeypatch):
    real = oq.estimate_scores

    def est_d_not_m(Sq, words, norms):
        m = np.atleast_2d(Sq).shape[1]
        return real(Sq, words, norms) * m / 128.0      # constant over d, not m
    _patch(monkeypatch, "estimate_scores", est_d_not_m)
    _fails(test_est.test_one_hot_closed_form)
    monkeypatch.setattr(oq, "ESTIMATOR_CONST", 1.0)
    _patch(monkeypatch, "estimate_scores", real)
    _fails(test_est.test_one_hot_closed_form)


def test_wrong_sign_of_estimate_is_caught(monkeypatch):
    real = oq.estimate_scores
    _patch(monkeypatch, "estimate_scores", lambda Sq, w, n: -real(Sq, w, n))
    _fails(tdec.test_two_tokens_hand_computed)


def test_wrong_head_mapping_is_caught(monkeypatch):
    real = oq.decode

    def decode_modulo(q, words, norms, values, N, S, scale=None, token_chunk=16384):
        B, Hq, d = q.shape
        Hkv = words.shape[1]
        out = np.zeros((B, Hq, d))
        for h in range(Hq):                   # h % H_kv instead of h // G
            c = h % Hkv
            out[:, h:h + 1] = real(q[:, h:h + 1], words[:, c:c + 1], norms[:, c:c + 1],
                                   values[:, c:c + 1], N, S, scale)
        return out
    _patch(monkeypatch, "decode", decode_modulo)
    _fails(tdec.test_gqa_head_mapping)


def test_missing_temperature_is_caught(monkeypatch):
    real = oq.decode
    _patch(monkeypatch, "decode",
           lambda q, w, n, v, N, S, scale=None, token_chunk=16384: real(q, w, n, v, N, S, 1.0))
    _fails(tdec.test_two_tokens_hand_computed)


def test_transposed_query_sketch_is_caught(monkeypatch):
    # square S makes the transposed product shape-compatible
    def qs_transposed(q, S):
        return np.asarray(q, dtype=np.float64) @ S.T
    _patch(monkeypatch, "query_sketch", qs_transposed)
    d = m = 64
    S = oracle.sketch(42, d, m)
    k = np.zeros((1, d))
    k[0, 3] = 1.0
    words, norms = oracle.encode(oracle.float64_to_bf16_bits(k), S)
    est = oracle.estimate_scores(oracle.query_sketch(k[0], S), words, norms)[0, 0]
    want = math.sqrt(math.pi / 2) / m * np.abs(S[3]).sum()
    assert abs(est - want) > 1e-6
