"""Random rotations and the rotated-coordinate density (test infrastructure).

"The Geometry of Forgetting: How Three Papers Cracked KV Cache Quantization",
section "Random rotation, and what high dimensions do to your intuitions":

* A random rotation is obtained by orthogonalizing a Gaussian matrix; it keeps
  lengths and inner products of the vectors it rotates.
* For a unit vector in d dimensions, each coordinate after a random rotation
  has the density Gamma(d/2) / (sqrt(pi) Gamma((d-1)/2)) * (1-x^2)^((d-3)/2)
  on [-1, 1], a scaled Beta law that tends to N(0, 1/d) as d grows.

QJL's own S is a Gaussian (not orthogonal) matrix; these functions are not on
the hot path.  They back the tests that pin the pages' geometric facts.
Parity pinned: closed forms (d = 3 gives the uniform law on [-1, 1]), unit
total mass, second moment 1/d, and agreement of sampled coordinates with the
CDF (Kolmogorov-Smirnov).
"""

from __future__ import annotations

import math

import numpy as np
from scipy import special


def haar_rotation(d: int, rng: np.random.Generator) -> np.ndarray:
    """Uniformly random orthogonal d x d matrix.

    QR-factorize a matrix of i.i.d. N(0,1) entries and flip the columns of Q
    so that R has a positive diagonal (Mezzadri, "How to generate random
    matrices from the classical compact groups", 2007); without the flip the
    distribution is not uniform.
    """
    A = rng.standard_normal((d, d))
    Q, R = np.linalg.qr(A)
    return Q * np.sign(np.diag(R))[None, :]


def rotated_coordinate_density(x, d: int) -> np.ndarray:
    """Density of one coordinate of a randomly rotated unit vector, d >= 2."""
    x = np.asarray(x, dtype=np.float64)
    logc = math.lgamma(d / 2.0) - 0.5 * math.log(math.pi) - math.lgamma((d - 1) / 2.0)
    inside = np.abs(x) < 1.0
    out = np.zeros_like(x)
    out[inside] = np.exp(logc + 0.5 * (d - 3) * np.log1p(-x[inside] ** 2))
    return out


def rotated_coordinate_cdf(x, d: int) -> np.ndarray:
    """CDF of the density above.

    x^2 follows Beta(1/2, (d-1)/2) (the density in x^2 after the change of
    variables), and the law is symmetric about 0, so
    F(x) = 1/2 + sign(x)/2 * I_{x^2}(1/2, (d-1)/2) with I the regularized
    incomplete Beta function.
    """
    x = np.clip(np.asarray(x, dtype=np.float64), -1.0, 1.0)
    return 0.5 + 0.5 * np.sign(x) * special.betainc(0.5, 0.5 * (d - 1), x * x)
