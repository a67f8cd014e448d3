// Host-side generator of the JL matrix S (bf16 values) from a 64-bit seed.
//
// "The Geometry of Forgetting: How Three Papers Cracked KV Cache
// Quantization", section "QJL: one bit, zero parameters, unbiased inner
// products": S has i.i.d. standard normal entries and is regenerated from a
// seed.  The generator is SplitMix64 (Steele, Lea and Flood, "Fast splittable
// pseudorandom number generators", OOPSLA 2014) feeding the Box-Muller
// transform (Box and Muller, 1958).  Generation happens on the host only, so
// no device math library is involved; this file is compiled with
// -ffp-contract=off so every fp64 operation rounds exactly as written.

#include "internal.h"

#include <cmath>
#include <cstring>
#include <vector>

namespace qjl {

namespace {

constexpr uint64_t kWeyl = 0x9E3779B97F4A7C15ull;

inline uint64_t splitmix64_finalize(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// Output number k (k >= 1) of the SplitMix64 stream whose state starts at seed.
inline uint64_t stream_output(uint64_t seed, uint64_t k) {
  return splitmix64_finalize(seed + k * kWeyl);
}

// 53 high bits -> (0, 1]; never 0, so log() below is finite.
inline double to_unit_interval(uint64_t r) {
  return static_cast<double>((r >> 11) + 1) * 0x1.0p-53;
}

inline uint16_t fp32_to_bf16_rne(float f) {
  uint32_t u;
  std::memcpy(&u, &f, sizeof(u));
  const uint32_t lsb = (u >> 16) & 1u;
  return static_cast<uint16_t>((static_cast<uint64_t>(u) + 0x7FFFu + lsb) >> 16);
}

}  // namespace

void generate_normals_f64(uint64_t seed, int d, int m, double* out) {
  const int64_t n = static_cast<int64_t>(d) * m;
  const double two_pi = 2.0 * M_PI;
  for (int64_t pair = 0; 2 * pair < n; ++pair) {
    const double u0 = to_unit_interval(stream_output(seed, 2 * pair + 1));
    const double u1 = to_unit_interval(stream_output(seed, 2 * pair + 2));
    const double r = std::sqrt(-2.0 * std::log(u0));
    const double a = two_pi * u1;
    out[2 * pair] = r * std::cos(a);
    if (2 * pair + 1 < n) out[2 * pair + 1] = r * std::sin(a);
  }
}

void generate_sketch_bf16(uint64_t seed, int d, int m, uint16_t* out) {
  const int64_t n = static_cast<int64_t>(d) * m;
  std::vector<double> z(static_cast<size_t>(n));
  generate_normals_f64(seed, d, m, z.data());
  for (int64_t e = 0; e < n; ++e) out[e] = fp32_to_bf16_rne(static_cast<float>(z[e]));
}

}  // namespace qjl
