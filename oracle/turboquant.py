"""Plain fp64 CPU oracle of TurboQuant_prod on keys (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module; the product path never calls it and
shares no code, table or constant generator with it.

Source: "The Geometry of Forgetting: How Three Papers Cracked KV Cache
Quantization", section "TurboQuant: bridging MSE and inner product, in two
stages", and the section "Random rotation, and what high dimensions do to
your intuitions" before it.  What the page fixes:

* Stage one (b - 1 bits per coordinate): rotate the unit vector by a random
  rotation Pi (orthogonalized Gaussian matrix); quantize every coordinate on
  its own with the optimal scalar quantizer for the rotated-coordinate
  density f_X (a Lloyd-Max codebook of 2^(b-1) centroids on [-1, 1], cell
  boundaries at the midpoints between adjacent centroids), computed once.
* Stage two (1 bit per coordinate): QJL on the residual x - x_hat, which
  debiases the inner product: the estimate of <y, x> is <y, x_hat> plus the
  QJL estimate of <y, x - x_hat>.
* Guarantees used as pins: D_mse <= (sqrt(3) pi / 2) 4^-b for the MSE stage
  at b bits, the Shannon floor 4^-b, unbiasedness of the two-stage
  estimator, and D_prod <= sqrt(3) pi^2 ||y||^2 / d * 4^-b.

Readings where the page is silent (the kernels implement the same ones):

* tq1 Keys are not unit vectors: the oracle stores n = ||k|| (fp32) and
  quantizes k / n, as the page's "we can always arrange by scaling".
* tq2 Pi comes from the same seeded Gaussian stream as the QJL sketch (the
  d x d fp64 normals of ``seed``), orthogonalized by QR with the column signs
  fixed so that R has a positive diagonal (Haar; Mezzadri 2007), then
  rounded to fp32.  The residual's QJL sketch is the QJL sketch of
  ``seed + 1`` with m = d sketch rows (one bit per coordinate).
* tq3 Centroids: the Lloyd-Max fixed point for f_X, rounded to the nearest
  multiple of 2^-20, so that two accurate solvers agree exactly; boundaries
  are the exact midpoints of the rounded centroids.
* tq4 Every value that feeds a decision is defined exactly, so that codes
  and bits are unique:
    n   = fp32(sqrt(s)), s the fp64 sum of k_j^2 taken in channel order;
    y_i = the fp32 rounding (nearest, ties to even) of the exact real
          sum_j Pi[i, j] k_j;
    u_i = fp32(y_i / n) (u = 0 for a zero key);
    idx_i = the number of boundaries <= u_i (fp32 comparisons);
    r_i = fp32(u_i - c[idx_i]);
    g   = fp32(sqrt(fp64 sum of r_i^2 in coordinate order));
    bit_l = [the exact real sum_i S[i, l] r_i >= 0] (sign(0) = +1).
* tq5 Storage per key: idx packed (b - 1) bits per coordinate, least
  significant bit first across uint32 words (coordinate i at bits
  (b-1) i .. (b-1) i + b - 2 of the stream); bits packed like QJL words; n
  and g as fp32.
* tq6 Estimate: <q, k> ~ n (<Pi q, c[idx]> + sqrt(pi/2)/m g <S^T Pi q, 2 bit - 1>).

Parity pins (tests/test_oracle_turboquant.py): the Lloyd-Max conditions by
independent quadrature, symmetry, the D_mse bound and the Shannon floor, the
Gaussian limit of the codebook, Monte-Carlo D_mse of rotated unit vectors,
unbiasedness and the D_prod bound of the two-stage estimator by Monte Carlo,
exactness of the rounded rotation by brute force with exact rationals,
power-of-two scale invariance of the codes, and planted mistakes.
"""

from __future__ import annotations

import math
from fractions import Fraction
from functools import lru_cache

import numpy as np
from scipy import special

from .qjl import ESTIMATOR_CONST, _pack_bits, _sketch_f64, bf16_bits_to_float64, sketch

CENTROID_GRID = 2.0 ** -20


# --------------------------------------------------------------------------
# The rotated-coordinate density and its Lloyd-Max codebook
# --------------------------------------------------------------------------

def _density_const(d: int) -> float:
    return math.exp(math.lgamma(d / 2.0) - 0.5 * math.log(math.pi) - math.lgamma((d - 1) / 2.0))


def _cdf(x, d: int):
    """F(x) of the rotated-coordinate density: x^2 ~ Beta(1/2, (d-1)/2)."""
    x = np.clip(np.asarray(x, dtype=np.float64), -1.0, 1.0)
    return 0.5 + 0.5 * np.sign(x) * special.betainc(0.5, 0.5 * (d - 1), x * x)


def _first_moment(x, d: int):
    """int_{-1}^{x} t f(t) dt = -C (1 - x^2)^((d-1)/2) / (d - 1) (antiderivative
    of t (1 - t^2)^((d-3)/2); zero at both ends)."""
    x = np.clip(np.asarray(x, dtype=np.float64), -1.0, 1.0)
    return -_density_const(d) * np.power(1.0 - x * x, 0.5 * (d - 1)) / (d - 1)


def lloyd_max_exact(d: int, k: int, tol: float = 1e-15, max_iter: int = 100000) -> np.ndarray:
    """The Lloyd-Max fixed point for f_X with 2^k levels, fp64, ascending.

    Alternates the two optimality conditions of the page's 1-D k-means: each
    boundary is the midpoint of its neighbours, each centroid the mean of f_X
    over its cell (first moment / mass, both in closed form).  Starts from the
    quantiles of f_X.
    """
    L = 2 ** k
    # quantile start: centroid v at the (v + 1/2)/L quantile (bisection on F)
    c = np.empty(L)
    for v in range(L):
        target = (v + 0.5) / L
        lo, hi = -1.0, 1.0
        for _ in range(200):
            mid = 0.5 * (lo + hi)
            if _cdf(mid, d) < target:
                lo = mid
            else:
                hi = mid
        c[v] = 0.5 * (lo + hi)
    for _ in range(max_iter):
        edges = np.concatenate([[-1.0], 0.5 * (c[:-1] + c[1:]), [1.0]])
        mass = np.diff(_cdf(edges, d))
        mom = np.diff(_first_moment(edges, d))
        new = mom / mass
        if np.max(np.abs(new - c)) < tol:
            c = new
            break
        c = new
    return c


@lru_cache(maxsize=32)
def codebook(d: int, k: int):
    """(centroids, boundaries) as fp32, reading tq3: the fixed point rounded to
    multiples of 2^-20; boundaries are the midpoints (exact in fp32)."""
    c = lloyd_max_exact(d, k)
    cq = np.round(c / CENTROID_GRID) * CENTROID_GRID
    beta = 0.5 * (cq[:-1] + cq[1:])
    return cq.astype(np.float32), beta.astype(np.float32)


def coordinate_distortion(centroids, d: int) -> float:
    """E[(x - Q(x))^2] for one coordinate x ~ f_X under the nearest-centroid
    quantizer of the given centroids (closed-form cell integrals)."""
    c = np.sort(np.asarray(centroids, dtype=np.float64))
    edges = np.concatenate([[-1.0], 0.5 * (c[:-1] + c[1:]), [1.0]])
    # int (x - c)^2 f = E2 - 2 c E1 + c^2 E0 per cell; E2 from the variance
    # identity: int x^2 f over a cell = F-weighted second moment, taken by
    # the Beta law of x^2: int_0^a x^2 f(x) dx = (1/d) * I_{a^2}(3/2, (d-1)/2) / 2
    def second(x):
        x = np.clip(x, -1.0, 1.0)
        return 0.5 / d + 0.5 / d * np.sign(x) * special.betainc(1.5, 0.5 * (d - 1), x * x)
    E0 = np.diff(_cdf(edges, d))
    E1 = np.diff(_first_moment(edges, d))
    E2 = np.diff(second(edges))
    return float(np.sum(E2 - 2.0 * c * E1 + c * c * E0))


# --------------------------------------------------------------------------
# The rotation
# --------------------------------------------------------------------------

@lru_cache(maxsize=8)
def rotation_f64(seed: int, d: int) -> np.ndarray:
    """Haar rotation from the seeded Gaussian stream (reading tq2), fp64."""
    A = _sketch_f64(seed, d, d)
    Q, R = np.linalg.qr(A)
    return Q * np.sign(np.diag(R))[None, :]


def rotation(seed: int, d: int) -> np.ndarray:
    """The rotation as used: fp32 entries (returned as float32)."""
    return rotation_f64(seed, d).astype(np.float32)


# --------------------------------------------------------------------------
# Exactly rounded sums
# --------------------------------------------------------------------------

def _rn32_of_exact(terms) -> np.float32:
    """fp32 rounding (nearest, ties to even) of the exact sum of fp64 terms."""
    exact = Fraction(0)
    for t in terms:
        exact += Fraction(float(t))
    v = float(exact)                       # nearest fp64 (exact rational -> float)
    f = np.float32(v)
    # v is the fp64 nearest to the exact value; fp32(v) can only differ from
    # fp32(exact) when v sits exactly on an fp32 rounding midpoint
    lo = np.nextafter(f, np.float32(-np.inf))
    hi = np.nextafter(f, np.float32(np.inf))
    for a, b in ((lo, f), (f, hi)):
        mid = (Fraction(float(a)) + Fraction(float(b))) / 2
        if Fraction(v) == mid and exact != mid:
            return b if exact > mid else a
    return f


def _sequential_sum_sq(X: np.ndarray) -> np.ndarray:
    """fp64 sum of squares over the last axis, added in index order."""
    s = np.zeros(X.shape[:-1], dtype=np.float64)
    for j in range(X.shape[-1]):
        s = s + X[..., j] * X[..., j]
    return s


# --------------------------------------------------------------------------
# Encode
# --------------------------------------------------------------------------

def _pack_codes(idx: np.ndarray, k: int) -> np.ndarray:
    """[R][d] codes of k bits -> [R][d*k/32] uint32, LSB first across words."""
    R, d = idx.shape
    if (d * k) % 32:
        raise ValueError("d * k must be a multiple of 32")
    bits = ((idx[..., None].astype(np.uint32) >> np.arange(k, dtype=np.uint32)) & 1).reshape(R, d * k)
    return _pack_bits(bits)


def unpack_codes(words: np.ndarray, d: int, k: int) -> np.ndarray:
    """Inverse of the code packing: [..., d*k/32] uint32 -> [..., d] codes."""
    w = np.asarray(words, dtype=np.uint32)
    pos = np.arange(d * k)
    bits = (w[..., pos // 32] >> (pos % 32).astype(np.uint32)) & 1
    bits = bits.reshape(w.shape[:-1] + (d, k)).astype(np.uint32)
    return (bits << np.arange(k, dtype=np.uint32)).sum(axis=-1).astype(np.uint32)


def rotate_rn32(K: np.ndarray, rot: np.ndarray) -> np.ndarray:
    """y = fp32 rounding (nearest, ties to even) of the exact K @ rot^T.

    K [R][d] holds bf16 values and rot fp32 values (both as fp64), so every
    product is exact in fp64 and the fp64 sum is within E = 2 d 2^-53
    sum_j |K_j rot_ij| of the exact value; when both ends of that interval
    round to the same fp32 number, so does the exact sum, and otherwise the
    sum is taken exactly.
    """
    P = K @ rot.T
    E = 2.0 * K.shape[1] * 2.0 ** -53 * (np.abs(K) @ np.abs(rot).T)
    lo = (P - E).astype(np.float32)
    y = (P + E).astype(np.float32)
    for t, i in zip(*np.nonzero(lo != y)):
        y[t, i] = _rn32_of_exact(K[t] * rot[i])
    return y


def encode_with(keys_bf16, k: int, rot: np.ndarray, S: np.ndarray):
    """The encode steps of reading tq4 for explicit matrices: rot [d][d]
    (fp32 values, as fp64) and S [d][m] (as fp64; any real values).
    Returns (idx [R][d], bits 0/1 [R][m], n fp32 [R], g fp32 [R])."""
    K = bf16_bits_to_float64(np.asarray(keys_bf16, dtype=np.uint16))
    d = K.shape[1]
    cents, bounds = codebook(d, k)
    n = np.sqrt(_sequential_sum_sq(K)).astype(np.float32)
    y = rotate_rn32(K, rot)
    u = np.zeros_like(y)
    nz = n > 0
    u[nz] = y[nz] / n[nz, None]                # fp32 division
    idx = (u[..., None] >= bounds[None, None, :]).sum(axis=-1)
    resid = (u - cents[idx]).astype(np.float32)
    g = np.sqrt(_sequential_sum_sq(resid.astype(np.float64))).astype(np.float32)
    # exact signs of S^T r: the fp64 products r_i S[i, l] are exact when S
    # holds bf16 values; the sum is re-taken with fsum near zero
    r64 = resid.astype(np.float64)
    Z = r64 @ S
    risky = np.abs(Z) <= 2.0 * d * 2.0 ** -53 * (np.abs(r64) @ np.abs(S))
    b = Z >= 0.0
    for t, l in zip(*np.nonzero(risky)):
        b[t, l] = math.fsum(float(r64[t, i]) * float(S[i, l]) for i in range(d)) >= 0.0
    return idx, b, n, g


def encode(keys_bf16, k: int, seed: int, m: int | None = None, chunk: int = 8192):
    """TurboQuant_prod encode of bf16 keys [R][d] (readings tq1-tq5).

    k = b - 1 bits per coordinate for the MSE stage; m sketch rows for the
    residual's QJL stage (default d: one bit per coordinate).
    Returns (codes uint32 [R][d k/32], bits uint32 [R][m/32], n fp32 [R],
    g fp32 [R]).
    """
    keys = np.asarray(keys_bf16, dtype=np.uint16)
    R, d = keys.shape
    m = d if m is None else m
    rot = rotation(seed, d).astype(np.float64)
    S = sketch(seed + 1, d, m)                 # exact fp64 values of the bf16 sketch
    codes = np.empty((R, d * k // 32), dtype=np.uint32)
    bits_out = np.empty((R, m // 32), dtype=np.uint32)
    n_out = np.empty(R, dtype=np.float32)
    g_out = np.empty(R, dtype=np.float32)
    for r0 in range(0, R, chunk):
        idx, b, n, g = encode_with(keys[r0:r0 + chunk], k, rot, S)
        codes[r0:r0 + chunk] = _pack_codes(idx, k)
        bits_out[r0:r0 + chunk] = _pack_bits(b)
        n_out[r0:r0 + chunk] = n
        g_out[r0:r0 + chunk] = g
    return codes, bits_out, n_out, g_out


def estimate_with(q, idx, bits, n, g, k: int, rot: np.ndarray, S: np.ndarray) -> np.ndarray:
    """Reading tq6 for explicit matrices: q [Q][d] against keys given as
    (idx [T][d], bits 0/1 [T][m], n [T], g [T]); returns [Q][T]."""
    q = np.atleast_2d(np.asarray(q, dtype=np.float64))
    d = q.shape[1]
    m = S.shape[1]
    cents, _ = codebook(d, k)
    qr = q @ rot.T                                       # Pi q
    mse = qr @ cents.astype(np.float64)[np.asarray(idx)].T
    pm1 = 2.0 * np.asarray(bits, dtype=np.float64) - 1.0
    qjl = (ESTIMATOR_CONST / m) * ((qr @ S) @ pm1.T) * np.asarray(g, np.float64)[None, :]
    return np.asarray(n, np.float64)[None, :] * (mse + qjl)


# --------------------------------------------------------------------------
# Decode side: inner-product estimates
# --------------------------------------------------------------------------

def scores(q, codes, bits, n, g, N: int, k: int, seed: int, m: int | None = None) -> np.ndarray:
    """Estimated <q, k_t> for every query head and cached token t < N.

    q [B][H_q][d] fp32; codes [B][H_kv][cap][d k/32]; bits [B][H_kv][cap][m/32];
    n, g [B][H_kv][cap].  Query head h reads kv head h // (H_q / H_kv).
    Returns [B][H_q][N] fp64 (reading tq6).
    """
    from .qjl import unpack_signs
    q = np.asarray(q, dtype=np.float64)
    B, Hq, d = q.shape
    Hkv = codes.shape[1]
    G = Hq // Hkv
    m = d if m is None else m
    rot = rotation(seed, d).astype(np.float64)
    S = sketch(seed + 1, d, m)
    out = np.empty((B, Hq, N), dtype=np.float64)
    for b in range(B):
        for c in range(Hkv):
            idx = unpack_codes(codes[b, c, :N], d, k)
            bt = unpack_signs(bits[b, c, :N], m)
            out[b, c * G:(c + 1) * G] = estimate_with(q[b, c * G:(c + 1) * G], idx, bt, n[b, c, :N],
                                                      g[b, c, :N], k, rot, S)
    return out
