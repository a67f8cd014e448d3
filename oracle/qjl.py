"""Plain fp64 CPU oracle of the QJL encode/decode path (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  It shares no code, tables or constants
with the HIP library; the one thing both sides have in common is the published
definition of the random-number generator that draws S from a seed, which each
side implements on its own.

What is computed, and where it comes from:

* S, the JL matrix.  "The Geometry of Forgetting: How Three Papers Cracked KV
  Cache Quantization", section "QJL: one bit, zero parameters, unbiased inner
  products": S has i.i.d. standard normal entries, is shared by every vector
  and is regenerated from a seed instead of being stored.  The pages name no
  generator; this oracle reads the step as the SplitMix64 output stream
  (Steele, Lea and Flood, OOPSLA 2014) turned into normals by the Box-Muller
  transform (Box and Muller, 1958), rounded to fp32 and then to bf16 so that
  the encode can run as a bf16 matrix product.  The page draws S as d x d;
  here it has m sketch rows s_i of length d (each row is a random hyperplane,
  same section), stored as a d x m array so that a key block K (rows = keys)
  projects as K @ S.
* Encode.  Same section, and "QJL: 1-Bit Quantized JL Transform for KV Cache
  Quantization with Zero Overhead", Abstract: Q(k) = sign(S k), one bit per
  sketch coordinate, no zero point or scale.  The key norm is kept beside the
  bits because the page's formulas assume unit-norm input, which the random
  rotation section says can always be arranged by scaling.  Bit i of a key
  is 1 iff the exact real number sum_j k_j * S[j, i] is >= 0 (so a zero sum
  gives +1); bits are packed 32 per uint32 word, lowest coordinate in the
  least significant bit.
* Decode.  Abstract (asymmetric estimator: the query gets the plain JL
  transform, the key the quantized one; unbiased) and the QJL section (the
  dequantizer constant sqrt(pi/2) divided by the sketch size; the expectation
  identity behind it).  The estimate of <q, k> is
  sqrt(pi/2)/m * ||k|| * sum_i (S^T q)_i * (2 b_i - 1); attention then takes a
  softmax of scale * estimate over the cached tokens and the weighted sum of
  the (bf16) values.

Parity pins: every function here is pinned by tests in ``tests/`` against
closed forms, special cases, brute force with exact rationals, Monte-Carlo
checks of the unbiasedness and variance statements, or an independent C
implementation of the generator.  None is "parity unpinned".
"""

from __future__ import annotations

import math
from fractions import Fraction
from functools import lru_cache

import numpy as np

MASK64 = (1 << 64) - 1
# Weyl increment of the SplitMix64 generator (the golden-ratio constant
# 2^64 / phi, rounded to odd), as published with the generator.
GOLDEN_GAMMA = 0x9E3779B97F4A7C15

# sqrt(pi/2): inverts E[<s,y> sign<s,x>] = sqrt(2/pi) <y,x>/||x|| for a
# standard Gaussian s ("The Geometry of Forgetting", QJL section).
ESTIMATOR_CONST = math.sqrt(math.pi / 2.0)


# --------------------------------------------------------------------------
# bf16 helpers (plain definitions; bf16 = the top 16 bits of an IEEE fp32)
# --------------------------------------------------------------------------

def bf16_bits_to_float64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact float64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def _fp32_bits_to_bf16_bits_rne(u32: np.ndarray) -> np.ndarray:
    """Round fp32 bit patterns to bf16, nearest with ties to even.

    Keeping the upper 16 bits and adding half an ulp of the kept part
    (0x7FFF plus the parity of the lowest kept bit) rounds to nearest and
    sends exact halfway cases to the even neighbour.  Inputs must be finite.
    """
    u = np.asarray(u32, dtype=np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    return ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)


def float64_to_bf16_bits(x) -> np.ndarray:
    """float64 -> fp32 (round to nearest even) -> bf16 (round to nearest even)."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    if not np.all(np.isfinite(f)):
        raise ValueError("bf16 rounding is defined here for finite values only")
    return _fp32_bits_to_bf16_bits_rne(f.view(np.uint32))


# --------------------------------------------------------------------------
# S from a seed
# --------------------------------------------------------------------------

def splitmix64_mix(z: int) -> int:
    """The SplitMix64 output function (a 64-bit finalizer), on Python ints."""
    z &= MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
    return z ^ (z >> 31)


def _splitmix64_output(seed: int, n: int) -> int:
    """n-th output (n >= 1) of SplitMix64 started from state ``seed``."""
    return splitmix64_mix((seed + n * GOLDEN_GAMMA) & MASK64)


def _uniform_open0_closed1(r: int) -> float:
    """Top 53 bits of a 64-bit word mapped to (0, 1]: ((r >> 11) + 1) * 2^-53."""
    return ((r >> 11) + 1) * (2.0 ** -53)


@lru_cache(maxsize=16)
def _sketch_f64(seed: int, d: int, m: int) -> np.ndarray:
    """Box-Muller normals for S, one pair per two consecutive elements.

    Element e = j*m + i (row j = key channel, column i = sketch coordinate)
    takes z0 of pair e // 2 when e is even and z1 when e is odd, where pair c
    uses SplitMix64 outputs 2c+1 and 2c+2 as u0 and u1.
    """
    if d <= 0 or m <= 0:
        raise ValueError("d and m must be positive")
    seed &= MASK64
    n = d * m
    out = np.empty(n, dtype=np.float64)
    for c in range((n + 1) // 2):
        u0 = _uniform_open0_closed1(_splitmix64_output(seed, 2 * c + 1))
        u1 = _uniform_open0_closed1(_splitmix64_output(seed, 2 * c + 2))
        radius = math.sqrt(-2.0 * math.log(u0))
        angle = 2.0 * math.pi * u1
        out[2 * c] = radius * math.cos(angle)
        if 2 * c + 1 < n:
            out[2 * c + 1] = radius * math.sin(angle)
    return out.reshape(d, m)


def sketch_bf16_bits(seed: int, d: int, m: int) -> np.ndarray:
    """bf16 bit patterns of S, shape [d][m] (row j = key channel)."""
    return float64_to_bf16_bits(_sketch_f64(seed, d, m))


def sketch(seed: int, d: int, m: int) -> np.ndarray:
    """S as exact float64 values of its bf16 entries, shape [d][m]."""
    return bf16_bits_to_float64(sketch_bf16_bits(seed, d, m))


# --------------------------------------------------------------------------
# Encode: sign bits of the exact projection, packed, plus the key norm
# --------------------------------------------------------------------------

def _pack_bits(bits: np.ndarray) -> np.ndarray:
    """[..., m] array of 0/1 -> [..., m/32] uint32, coordinate 32w+j at bit j."""
    m = bits.shape[-1]
    if m % 32:
        raise ValueError("sketch size must be a multiple of 32")
    b = bits.astype(np.uint64).reshape(bits.shape[:-1] + (m // 32, 32))
    weights = np.uint64(1) << np.arange(32, dtype=np.uint64)
    return (b * weights).sum(axis=-1).astype(np.uint32)


def encode(keys_bf16, S: np.ndarray, chunk: int = 1 << 16):
    """Encode keys: (packed sign words, fp32 norms).

    keys_bf16: [R][d] uint16 bf16 bit patterns.  S: [d][m] float64 whose
    entries are exactly representable in bf16 (``sketch``).

    Each product k_j * S[j, i] of two bf16 values is exact in float64, so the
    float64 matrix product differs from the exact sum by at most
    d * 2^-53 * sum_j |k_j S[j, i]| (any summation order).  Entries within
    twice that of zero are recomputed with ``math.fsum``, which returns the
    correctly rounded exact sum and hence its exact sign.
    """
    keys = np.asarray(keys_bf16, dtype=np.uint16)
    R, d = keys.shape
    if S.shape[0] != d:
        raise ValueError("S must have d rows")
    m = S.shape[1]
    words = np.empty((R, m // 32), dtype=np.uint32)
    norms = np.empty(R, dtype=np.float32)
    absS = np.abs(S)
    for r0 in range(0, R, chunk):
        K = bf16_bits_to_float64(keys[r0:r0 + chunk])
        P = K @ S
        bound = np.abs(K) @ absS
        risky = np.abs(P) <= 2.0 * d * (2.0 ** -53) * bound
        bits = P >= 0.0
        for t, i in zip(*np.nonzero(risky)):
            exact = math.fsum(float(K[t, j]) * float(S[j, i]) for j in range(d))
            bits[t, i] = exact >= 0.0
        words[r0:r0 + chunk] = _pack_bits(bits)
        # Squares of bf16 values are exact in float64; the norm is rounded
        # once to fp32 at the end.
        norms[r0:r0 + chunk] = np.sqrt((K * K).sum(axis=1)).astype(np.float32)
    return words, norms


def exact_sign_fraction(keys_bf16, S: np.ndarray) -> np.ndarray:
    """Brute-force sign bits with exact rational arithmetic (tiny shapes only).

    Returns the [R][m] 0/1 array with bit = 1 iff sum_j k_j S[j, i] >= 0,
    every term held as a ``fractions.Fraction``.
    """
    K = bf16_bits_to_float64(keys_bf16)
    R, d = K.shape
    m = S.shape[1]
    out = np.zeros((R, m), dtype=np.uint8)
    for t in range(R):
        kf = [Fraction(float(v)) for v in K[t]]
        for i in range(m):
            total = sum((kf[j] * Fraction(float(S[j, i])) for j in range(d)),
                        Fraction(0))
            out[t, i] = 1 if total >= 0 else 0
    return out


def unpack_signs(words: np.ndarray, m: int) -> np.ndarray:
    """[..., m/32] uint32 -> [..., m] array of 0/1 (inverse of the packing)."""
    w = np.asarray(words, dtype=np.uint32)
    idx = np.arange(m)
    return ((w[..., idx // 32] >> (idx % 32).astype(np.uint32)) & 1).astype(np.uint8)


# --------------------------------------------------------------------------
# Decode: asymmetric estimator, softmax, weighted sum of values
# --------------------------------------------------------------------------

def query_sketch(q, S: np.ndarray) -> np.ndarray:
    """Plain (unquantized) JL transform of queries: (S^T q), shape [..., m]."""
    return np.asarray(q, dtype=np.float64) @ S


def estimate_scores(Sq: np.ndarray, words: np.ndarray, norms) -> np.ndarray:
    """Estimated <q, k_t> for every query row of Sq and every encoded key t.

    Sq: [Q][m] query sketches.  words: [T][m/32].  norms: [T].
    Returns [Q][T] = sqrt(pi/2)/m * ||k_t|| * sum_i Sq_i (2 b_ti - 1).
    """
    Sq = np.atleast_2d(np.asarray(Sq, dtype=np.float64))
    m = Sq.shape[1]
    pm1 = 2.0 * unpack_signs(words, m).astype(np.float64) - 1.0      # [T][m]
    n = np.asarray(norms, dtype=np.float64)
    return (ESTIMATOR_CONST / m) * (Sq @ pm1.T) * n[None, :]


def dequantize(words: np.ndarray, norms, S: np.ndarray) -> np.ndarray:
    """Key reconstruction ||k|| * sqrt(pi/2)/m * S z with z in {-1,+1}^m.

    The QJL section's dequantizer (written there for unit vectors and a
    square S), scaled by the stored norm.  Decode never calls it; it pins the
    estimator: <q, dequantize(k)> equals estimate_scores.
    """
    m = S.shape[1]
    pm1 = 2.0 * unpack_signs(words, m).astype(np.float64) - 1.0      # [T][m]
    n = np.asarray(norms, dtype=np.float64)
    return (ESTIMATOR_CONST / m) * (pm1 @ S.T) * n[:, None]


def decode(q, words, norms, values_bf16, N: int, S: np.ndarray,
           scale: float | None = None, token_chunk: int = 16384) -> np.ndarray:
    """One decode step of QJL attention, fp64.

    q:           [B][H_q][d] float queries.
    words:       [B][H_kv][cap][m/32] uint32 packed sign bits.
    norms:       [B][H_kv][cap] key norms.
    values_bf16: [B][H_kv][cap][d] uint16 bf16 bit patterns.
    N:           number of cached tokens attended to (rows [0, N)).
    scale:       softmax temperature applied to the estimate; None -> 1/sqrt(d).

    Query head h reads kv head h // (H_q / H_kv).  Returns [B][H_q][d] fp64.
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, d = q.shape
    Hkv = words.shape[1]
    m = S.shape[1]
    if Hq % Hkv:
        raise ValueError("H_q must be a multiple of H_kv")
    if N <= 0:
        raise ValueError("N must be positive")
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = np.zeros((B, Hq, d), dtype=np.float64)
    for b in range(B):
        for c in range(Hkv):
            Sq = query_sketch(q[b, c * G:(c + 1) * G], S)              # [G][m]
            logits = np.empty((G, N), dtype=np.float64)
            for t0 in range(0, N, token_chunk):
                t1 = min(N, t0 + token_chunk)
                logits[:, t0:t1] = scale * estimate_scores(
                    Sq, words[b, c, t0:t1], norms[b, c, t0:t1])
            logits -= logits.max(axis=1, keepdims=True)
            p = np.exp(logits)
            p /= p.sum(axis=1, keepdims=True)
            acc = np.zeros((G, d), dtype=np.float64)
            for t0 in range(0, N, token_chunk):
                t1 = min(N, t0 + token_chunk)
                acc += p[:, t0:t1] @ bf16_bits_to_float64(values_bf16[b, c, t0:t1])
            out[b, c * G:(c + 1) * G] = acc
    return out


def exact_attention(q, keys_bf16, values_bf16, N: int, scale: float | None = None):
    """Unquantized softmax attention over bf16 keys (a quality reading only).

    Same shapes as ``decode`` with keys [B][H_kv][cap][d] in bf16 bits.
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, d = q.shape
    Hkv = keys_bf16.shape[1]
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = np.zeros((B, Hq, d), dtype=np.float64)
    for b in range(B):
        for c in range(Hkv):
            K = bf16_bits_to_float64(keys_bf16[b, c, :N])
            V = bf16_bits_to_float64(values_bf16[b, c, :N])
            logits = scale * (q[b, c * G:(c + 1) * G] @ K.T)
            logits -= logits.max(axis=1, keepdims=True)
            p = np.exp(logits)
            p /= p.sum(axis=1, keepdims=True)
            out[b, c * G:(c + 1) * G] = p @ V
    return out
