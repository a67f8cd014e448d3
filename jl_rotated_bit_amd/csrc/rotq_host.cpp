// Host-side tables of the rotate-then-quantize encoders (TurboQuant_prod and
// PolarQuant): the seeded Haar rotation and the Lloyd-Max codebooks.
//
// "The Geometry of Forgetting: How Three Papers Cracked KV Cache
// Quantization":
// * section "Random rotation, and what high dimensions do to your
//   intuitions": a random rotation is an orthogonalized Gaussian matrix; a
//   coordinate of a rotated unit vector has density
//   Gamma(d/2) / (sqrt(pi) Gamma((d-1)/2)) (1 - x^2)^((d-3)/2) on [-1, 1];
// * section "TurboQuant: bridging MSE and inner product, in two stages": the
//   codebook is the optimal scalar (Lloyd-Max) quantizer of that density,
//   cell boundaries at the midpoints of adjacent centroids, computed once;
// * section "PolarQuant: skipping Cartesian altogether": level-1 angles are
//   uniform on [0, 2 pi), level-l angles have density proportional to
//   sin^(2^(l-1) - 1)(2 psi) on [0, pi/2]; each level has its own codebook.
//
// The rotation is the Q of a Householder QR of the seed's d x d normals with
// R's diagonal made positive (the Haar measure; Mezzadri 2007), rounded to
// fp32.  Centroids are Lloyd-Max fixed points rounded to multiples of 2^-20
// (so that any two accurate solvers agree exactly); cell masses and first
// moments come from composite Gauss-Legendre quadrature (plus the closed-form
// first moment of the rotated-coordinate density).  PolarQuant cells are
// decided through tan(boundary), rounded to multiples of 2^-20.  Compiled with
// -ffp-contract=off.

#include <algorithm>
#include <cmath>
#include <vector>

#include "internal.h"

namespace qjl {
namespace {

constexpr double kGrid = 0x1.0p-20;

double round_to_grid(double x) { return std::nearbyint(x / kGrid) * kGrid; }

// Gauss-Legendre nodes and weights on [-1, 1] (Newton on P_n).
struct GaussLegendre {
  std::vector<double> x, w;
  explicit GaussLegendre(int n) : x(n), w(n) {
    for (int i = 0; i < n; ++i) {
      double z = std::cos(M_PI * (i + 0.75) / (n + 0.5));
      for (int it = 0; it < 100; ++it) {
        double p0 = 1.0, p1 = z;
        for (int k = 2; k <= n; ++k) {
          const double p2 = ((2.0 * k - 1.0) * z * p1 - (k - 1.0) * p0) / k;
          p0 = p1;
          p1 = p2;
        }
        const double dp = n * (z * p1 - p0) / (z * z - 1.0);
        const double dz = p1 / dp;
        z -= dz;
        if (std::fabs(dz) < 1e-16) {
          // weight from the derivative at the converged node
          double q0 = 1.0, q1 = z;
          for (int k = 2; k <= n; ++k) {
            const double q2 = ((2.0 * k - 1.0) * z * q1 - (k - 1.0) * q0) / k;
            q0 = q1;
            q1 = q2;
          }
          const double dq = n * (z * q1 - q0) / (z * z - 1.0);
          x[i] = z;
          w[i] = 2.0 / ((1.0 - z * z) * dq * dq);
          break;
        }
      }
    }
  }
};

// int_a^b f over `pieces` equal subintervals of 32-point Gauss-Legendre.
template <class F>
double integrate(const F& f, double a, double b, int pieces = 64) {
  static const GaussLegendre gl(32);
  const double h = (b - a) / pieces;
  double total = 0.0;
  for (int p = 0; p < pieces; ++p) {
    const double lo = a + p * h, mid = lo + 0.5 * h;
    double s = 0.0;
    for (size_t i = 0; i < gl.x.size(); ++i) s += gl.w[i] * f(mid + 0.5 * h * gl.x[i]);
    total += 0.5 * h * s;
  }
  return total;
}

// Lloyd-Max for a density on [lo, hi]: mass(a, b) and moment(a, b) give the
// cell integrals; quantile start; returns the fp64 fixed point, ascending.
template <class Mass, class Moment>
std::vector<double> lloyd_max(int levels, double lo, double hi, const Mass& mass, const Moment& moment,
                              double tol) {
  const double total = mass(lo, hi);
  std::vector<double> c(levels);
  for (int v = 0; v < levels; ++v) {
    const double target = (v + 0.5) / levels * total;
    double a = lo, b = hi;
    for (int it = 0; it < 200; ++it) {
      const double m = 0.5 * (a + b);
      if (mass(lo, m) < target) a = m;
      else b = m;
    }
    c[v] = 0.5 * (a + b);
  }
  std::vector<double> nc(levels), edges(levels + 1);
  for (int it = 0; it < 100000; ++it) {
    edges[0] = lo;
    edges[levels] = hi;
    for (int v = 1; v < levels; ++v) edges[v] = 0.5 * (c[v - 1] + c[v]);
    double delta = 0.0;
    for (int v = 0; v < levels; ++v) {
      nc[v] = moment(edges[v], edges[v + 1]) / mass(edges[v], edges[v + 1]);
      delta = std::max(delta, std::fabs(nc[v] - c[v]));
    }
    c.swap(nc);
    if (delta < tol) break;
  }
  return c;
}

}  // namespace

void make_rotation_f32(uint64_t seed, int d, float* out) {
  const size_t n = static_cast<size_t>(d) * d;
  std::vector<double> A(n);
  generate_normals_f64(seed, d, d, A.data());   // A[j][i], row j, column i
  // Householder QR, column by column; the reflectors are kept in A's lower
  // part and R's diagonal in rdiag.
  std::vector<double> rdiag(d), v(d);
  std::vector<std::vector<double>> refl(d);
  for (int k = 0; k < d; ++k) {
    double norm = 0.0;
    for (int r = k; r < d; ++r) norm += A[r * d + k] * A[r * d + k];
    norm = std::sqrt(norm);
    const double x0 = A[k * d + k];
    const double alpha = x0 >= 0.0 ? -norm : norm;
    std::vector<double>& u = refl[k];
    u.assign(d - k, 0.0);
    for (int r = k; r < d; ++r) u[r - k] = A[r * d + k];
    u[0] -= alpha;
    double un = 0.0;
    for (double e : u) un += e * e;
    un = std::sqrt(un);
    if (un > 0.0)
      for (double& e : u) e /= un;
    // A[k:, k:] -= 2 u (u^T A[k:, k:])
    for (int c = k; c < d; ++c) {
      double dot = 0.0;
      for (int r = k; r < d; ++r) dot += u[r - k] * A[r * d + c];
      for (int r = k; r < d; ++r) A[r * d + c] -= 2.0 * u[r - k] * dot;
    }
    rdiag[k] = A[k * d + k];
  }
  // Q = H_0 H_1 ... H_{d-1} applied to the identity (right to left)
  std::vector<double> Q(n, 0.0);
  for (int i = 0; i < d; ++i) Q[i * d + i] = 1.0;
  for (int k = d - 1; k >= 0; --k) {
    const std::vector<double>& u = refl[k];
    for (int c = 0; c < d; ++c) {
      double dot = 0.0;
      for (int r = k; r < d; ++r) dot += u[r - k] * Q[r * d + c];
      for (int r = k; r < d; ++r) Q[r * d + c] -= 2.0 * u[r - k] * dot;
    }
  }
  // columns whose R diagonal is negative flip sign
  for (int c = 0; c < d; ++c)
    if (rdiag[c] < 0.0)
      for (int r = 0; r < d; ++r) Q[r * d + c] = -Q[r * d + c];
  for (size_t e = 0; e < n; ++e) out[e] = static_cast<float>(Q[e]);
}

void make_tq_codebook(int d, int k, float* centroids) {
  const double logc = std::lgamma(d / 2.0) - 0.5 * std::log(M_PI) - std::lgamma((d - 1) / 2.0);
  const double C = std::exp(logc);
  auto f = [&](double x) { return C * std::pow(std::max(0.0, 1.0 - x * x), 0.5 * (d - 3)); };
  auto mass = [&](double a, double b) { return integrate(f, a, b); };
  // int t (1 - t^2)^((d-3)/2) = -(1 - t^2)^((d-1)/2) / (d - 1)
  auto prim = [&](double x) { return -C * std::pow(std::max(0.0, 1.0 - x * x), 0.5 * (d - 1)) / (d - 1); };
  auto moment = [&](double a, double b) { return prim(b) - prim(a); };
  const std::vector<double> c = lloyd_max(1 << k, -1.0, 1.0, mass, moment, 1e-15);
  for (int v = 0; v < (1 << k); ++v) centroids[v] = static_cast<float>(round_to_grid(c[v]));
}

void make_pq_codebook(int level, int bits, float* centroids, float* thresholds) {
  const int L = 1 << bits;
  if (level == 1) {
    const double w = 2.0 * M_PI / L;
    for (int v = 0; v < L; ++v) centroids[v] = static_cast<float>((v + 0.5) * w);
    for (int t = 1; t < L / 4; ++t) thresholds[t - 1] = static_cast<float>(round_to_grid(std::tan(t * w)));
    return;
  }
  const double a = std::ldexp(1.0, level - 2);
  auto f = [&](double psi) { return std::pow(std::max(0.0, std::sin(2.0 * psi)), 2.0 * a - 1.0); };
  auto mass = [&](double x, double y) { return integrate(f, x, y); };
  auto moment = [&](double x, double y) { return integrate([&](double p) { return p * f(p); }, x, y); };
  const std::vector<double> c = lloyd_max(L, 0.0, M_PI / 2, mass, moment, 1e-14);
  std::vector<double> cq(L);
  for (int v = 0; v < L; ++v) {
    cq[v] = round_to_grid(c[v]);
    centroids[v] = static_cast<float>(cq[v]);
  }
  for (int t = 1; t < L; ++t) thresholds[t - 1] = static_cast<float>(round_to_grid(std::tan(0.5 * (cq[t - 1] + cq[t]))));
}

}  // namespace qjl
