"""Plain CPU oracle of the PolarQuant key encode (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module; the product path never calls it and
shares no code, table or constant generator with it.

Source: "The Geometry of Forgetting: How Three Papers Cracked KV Cache
Quantization", section "PolarQuant: skipping Cartesian altogether".  What the
page fixes:

* Precondition the vector with a random rotation (its distribution becomes
  known), then convert it to polar form recursively: pair the coordinates and
  write each pair as a radius and an angle; pair the radii and do the same;
  after log2 d levels one radius is left, with levels of 1, 2, ..., d/2
  angles.  Level-1 angles are atan(x_2j / x_2j-1) over the full circle;
  level-l angles are atan(||second half of a slice|| / ||first half||).
* For a Gaussian input the radius and every angle are independent; level-1
  angles are uniform on [0, 2 pi); level-l angles (l >= 2) have density
  proportional to sin^(2^(l-1) - 1)(2 psi) on [0, pi/2].
* A codebook is precomputed for each level's law; encode stores each angle's
  bucket index and keeps the radius in floating point.  The page reports
  more than 4.2x compression of the KV cache.

Readings where the page is silent (the kernels implement the same ones):

* pq1 The rotation is TurboQuant's (oracle.turboquant, reading tq2), and the
  rotated key is y_i = the fp32 rounding of the exact sum_j Pi[i, j] k_j
  (reading tq4), so every later step starts from exactly defined numbers.
* pq2 Bits per level: 4 at level 1, 2 at every level above (d = 128: 7
  levels, 64 * 4 + 63 * 2 = 382 bits, padded to 12 words).
* pq3 Level 1 (uniform law): 2^b cells of equal width, centroid at each
  cell's middle.  Levels l >= 2: the Lloyd-Max fixed point for
  sin^(2^(l-1) - 1)(2 psi), rounded to multiples of 2^-20; cell boundaries are
  the midpoints of the rounded centroids.
* pq4 Decisions without angles: a boundary angle theta enters only through
  T = tan(theta) rounded to a multiple of 2^-20.  Level 1: the pair
  (a, b) = (y_2j, y_2j+1) picks its quadrant by signs (the angle of (a, b)
  lies in [q pi/2, (q+1) pi/2)), is turned into the first quadrant exactly
  ((a, b), (b, -a), (-a, -b), (-b, a)), and its cell within the quadrant is
  the number of in-quadrant thresholds T with b' >= T a' (fp64, T a'
  rounded once).  (0, 0) takes angle 0.  Levels l >= 2: with the slice sums
  of squares s_a, s_b (fp64, level-1 sums y_2j^2 + y_2j+1^2, then pairwise
  sums up the tree), the cell is the number of thresholds with
  s_b >= T^2 s_a (T^2 exact, the product rounded once); s_a = 0 therefore
  gives the top cell (angle pi/2), also when s_b = 0.
* pq5 Radius: fp32(sqrt(s)) with s the tree sum of the whole vector.
* pq6 Storage: the cells of level 1 (angle 0 first), then of level 2, ...,
  each in its level's bit width, least significant bit first across uint32
  words; the radius as fp32.
* pq7 Reconstruction (for the pins and for a decode): the top radius is
  split down the tree by cos and sin of each level's centroid, then the
  rotation is undone (Pi^T y).

Parity pins (tests/test_oracle_polarquant.py): the page's level laws and
their independence on Gaussian vectors (Kolmogorov-Smirnov), the exact
inverse of the unquantized transform, Lloyd-Max conditions by quadrature and
symmetry about pi/4, the decisions against atan2 on random vectors, the
compression ratio against the page's 4.2x, error falling with the bits, and
power-of-two scale invariance.
"""

from __future__ import annotations

import math
from functools import lru_cache

import numpy as np
from scipy import integrate, special

from .qjl import _pack_bits, bf16_bits_to_float64
from .turboquant import CENTROID_GRID, rotate_rn32, rotation

DEFAULT_BITS = (4, 2, 2, 2, 2, 2, 2)
TAN_GRID = 2.0 ** -20


def levels(d: int) -> int:
    L = int(round(math.log2(d)))
    if 2 ** L != d:
        raise ValueError("d must be a power of two")
    return L


# --------------------------------------------------------------------------
# Level laws and codebooks
# --------------------------------------------------------------------------

def level_density(psi, level: int) -> np.ndarray:
    """Normalized density of a level-l angle (l >= 2) on [0, pi/2]:
    proportional to sin^(2^(l-1) - 1)(2 psi).  With t = sin^2 psi the law is
    Beta(2^(l-2), 2^(l-2)), which gives the normalization."""
    psi = np.asarray(psi, dtype=np.float64)
    a = 2 ** (level - 2)
    # f(psi) = sin^(2a - 1)(2 psi) * 2^(2 - 2a) / B(a, a)  (dt = sin(2 psi) dpsi)
    logc = (2 - 2 * a) * math.log(2.0) - special.betaln(a, a)
    s = np.sin(2.0 * np.clip(psi, 0.0, math.pi / 2))
    out = np.exp(logc + (2 * a - 1) * np.log(np.maximum(s, 1e-300)))
    return np.where((psi >= 0) & (psi <= math.pi / 2), out, 0.0)


def level_cdf(psi, level: int):
    a = 2 ** (level - 2)
    psi = np.clip(np.asarray(psi, dtype=np.float64), 0.0, math.pi / 2)
    return special.betainc(a, a, np.sin(psi) ** 2)


def lloyd_max_level(level: int, bits: int, tol: float = 1e-14, max_iter: int = 20000) -> np.ndarray:
    """Lloyd-Max fixed point (fp64, ascending) for a level-l angle, l >= 2:
    boundaries at midpoints, centroids at the conditional means (first
    moments by adaptive quadrature, masses by the Beta CDF)."""
    L = 2 ** bits
    c = np.empty(L)
    for v in range(L):              # quantile start
        target = (v + 0.5) / L
        lo, hi = 0.0, math.pi / 2
        for _ in range(200):
            mid = 0.5 * (lo + hi)
            if level_cdf(mid, level) < target:
                lo = mid
            else:
                hi = mid
        c[v] = 0.5 * (lo + hi)
    for _ in range(max_iter):
        edges = np.concatenate([[0.0], 0.5 * (c[:-1] + c[1:]), [math.pi / 2]])
        new = np.empty(L)
        for v in range(L):
            mass = float(level_cdf(edges[v + 1], level) - level_cdf(edges[v], level))
            mom = integrate.quad(lambda x: x * float(level_density(x, level)), edges[v], edges[v + 1],
                                 epsabs=1e-16, epsrel=1e-13, limit=200)[0]
            new[v] = mom / mass
        done = np.max(np.abs(new - c)) < tol
        c = new
        if done:
            break
    return c


@lru_cache(maxsize=64)
def level_codebook(level: int, bits: int):
    """(centroids, boundaries, tangent thresholds), readings pq3/pq4.

    Level 1: uniform cells on [0, 2 pi); thresholds are those inside one
    quadrant (tan of the cell edges pi/2 q + w, ..., strictly inside).
    Levels >= 2: rounded Lloyd-Max centroids, midpoint boundaries, thresholds
    tan(boundary) rounded to multiples of 2^-20.
    """
    L = 2 ** bits
    if level == 1:
        w = 2.0 * math.pi / L
        cents = (np.arange(L) + 0.5) * w
        bounds = np.arange(1, L) * w
        per_q = L // 4
        T = np.array([round(math.tan(t * w) / TAN_GRID) * TAN_GRID for t in range(1, per_q)])
        return cents, bounds, T
    c = lloyd_max_level(level, bits)
    cq = np.round(c / CENTROID_GRID) * CENTROID_GRID
    bounds = 0.5 * (cq[:-1] + cq[1:])
    T = np.round(np.tan(bounds) / TAN_GRID) * TAN_GRID
    return cq, bounds, T


# --------------------------------------------------------------------------
# The recursive polar transform
# --------------------------------------------------------------------------

def polar_transform(y: np.ndarray):
    """Unquantized transform of [R][d] vectors: (angles per level, radius).

    angles[0] [R][d/2] in [0, 2 pi) (atan2 of each pair), angles[l-1]
    [R][d/2^l] in [0, pi/2] for l >= 2; radius [R].  (fp64, for the pins.)
    """
    y = np.asarray(y, dtype=np.float64)
    a, b = y[:, 0::2], y[:, 1::2]
    angles = [np.mod(np.arctan2(b, a), 2 * math.pi)]
    rho = np.hypot(a, b)
    while rho.shape[1] > 1:
        ra, rb = rho[:, 0::2], rho[:, 1::2]
        angles.append(np.arctan2(rb, ra))
        rho = np.hypot(ra, rb)
    return angles, rho[:, 0]


def polar_inverse(angles, radius) -> np.ndarray:
    """Rebuild [R][d] from per-level angles and the radius (reading pq7)."""
    rho = np.asarray(radius, dtype=np.float64)[:, None]
    for psi in reversed(angles[1:]):
        out = np.empty((rho.shape[0], 2 * rho.shape[1]))
        out[:, 0::2] = rho * np.cos(psi)
        out[:, 1::2] = rho * np.sin(psi)
        rho = out
    psi = angles[0]
    y = np.empty((rho.shape[0], 2 * rho.shape[1]))
    y[:, 0::2] = rho * np.cos(psi)
    y[:, 1::2] = rho * np.sin(psi)
    return y


# --------------------------------------------------------------------------
# Encode: cells by exact-order comparisons (reading pq4)
# --------------------------------------------------------------------------

def level1_cells(y: np.ndarray, bits: int) -> np.ndarray:
    """Cell of each pair's full-circle angle, [R][d/2]."""
    _, _, T = level_codebook(1, bits)
    per_q = 2 ** bits // 4
    a = np.asarray(y[:, 0::2], dtype=np.float64)
    b = np.asarray(y[:, 1::2], dtype=np.float64)
    # quadrant q: angle in [q pi/2, (q+1) pi/2); (0, 0) has angle 0
    q = np.where(b > 0, np.where(a > 0, 0, 1), np.where(b < 0, np.where(a < 0, 2, 3),
                                                        np.where(a < 0, 2, 0)))
    # b == 0: angle 0 for a >= 0 (quadrant 0), pi for a < 0 (quadrant 2)
    ap = np.select([q == 0, q == 1, q == 2, q == 3], [a, b, -a, -b])
    bp = np.select([q == 0, q == 1, q == 2, q == 3], [b, -a, -b, a])
    within = np.zeros(a.shape, dtype=np.int64)
    for t in T:
        within += (bp >= t * ap)
    within[(ap == 0) & (bp == 0)] = 0          # (0, 0): angle 0
    return q * per_q + within


def upper_cells(y: np.ndarray, bit_alloc) -> list:
    """Cells of the level >= 2 angles from tree sums of squares."""
    y = np.asarray(y, dtype=np.float64)
    s = y[:, 0::2] * y[:, 0::2] + y[:, 1::2] * y[:, 1::2]
    out = []
    lev = 2
    while s.shape[1] > 1:
        sa, sb = s[:, 0::2], s[:, 1::2]
        _, _, T = level_codebook(lev, bit_alloc[lev - 1])
        cells = np.zeros(sa.shape, dtype=np.int64)
        for t in T:
            cells += (sb >= (t * t) * sa)
        out.append(cells)
        s = sa + sb
        lev += 1
    return out, s[:, 0]


def _pack_stream(cells_per_level, bit_alloc, words: int) -> np.ndarray:
    R = cells_per_level[0].shape[0]
    cols = []
    for cells, b in zip(cells_per_level, bit_alloc):
        c = np.asarray(cells, dtype=np.uint64)
        cols.append(((c[..., None] >> np.arange(b, dtype=np.uint64)) & 1).reshape(R, -1))
    bits = np.concatenate(cols, axis=1)
    pad = words * 32 - bits.shape[1]
    bits = np.concatenate([bits, np.zeros((R, pad), dtype=np.uint64)], axis=1)
    return _pack_bits(bits)


def code_words(d: int, bit_alloc=DEFAULT_BITS) -> int:
    L = levels(d)
    total = sum((d >> (lev + 1)) * bit_alloc[lev] for lev in range(L))
    return -(-total // 32)


def encode(keys_bf16, seed: int, bit_alloc=DEFAULT_BITS):
    """PolarQuant encode of bf16 keys [R][d]: (codes uint32 [R][words], radius fp32 [R])."""
    K = bf16_bits_to_float64(np.asarray(keys_bf16, dtype=np.uint16))
    R, d = K.shape
    if len(bit_alloc) != levels(d):
        raise ValueError("one bit width per level")
    y = rotate_rn32(K, rotation(seed, d).astype(np.float64))
    c1 = level1_cells(y, bit_alloc[0])
    ups, s = upper_cells(y, bit_alloc)
    radius = np.sqrt(s).astype(np.float32)
    return _pack_stream([c1] + ups, bit_alloc, code_words(d, bit_alloc)), radius


def unpack(codes, d: int, bit_alloc=DEFAULT_BITS) -> list:
    """Codes -> list of per-level cell arrays."""
    w = np.asarray(codes, dtype=np.uint32)
    R = w.shape[0]
    pos = 0
    out = []
    for lev in range(levels(d)):
        n, b = d >> (lev + 1), bit_alloc[lev]
        idx = pos + np.arange(n * b)
        bits = ((w[:, idx // 32] >> (idx % 32).astype(np.uint32)) & 1).reshape(R, n, b)
        out.append((bits.astype(np.int64) << np.arange(b)).sum(axis=-1))
        pos += n * b
    return out


def dequantize(codes, radius, seed: int, d: int, bit_alloc=DEFAULT_BITS) -> np.ndarray:
    """Reconstructed keys [R][d] (reading pq7), fp64."""
    cells = unpack(codes, d, bit_alloc)
    angles = [level_codebook(lev + 1, bit_alloc[lev])[0][cells[lev]] for lev in range(levels(d))]
    y = polar_inverse(angles, radius)
    return y @ rotation(seed, d).astype(np.float64)
