// Exact-sign helpers shared by the encode kernels and the decode step's
// append: bf16 -> fp64 conversion, fp64 sums over a quad of lanes, and the
// exact sign of a 128-term bf16 dot product through a long integer
// accumulator.  The sign of the exact real sum decides a sign bit
// ("The Geometry of Forgetting: How Three Papers Cracked KV Cache
// Quantization", section "QJL: one bit, zero parameters, unbiased inner
// products": Q(x) = sign(Sx)), with sign(0) = +1.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "internal.h"

namespace qjl {
namespace {

constexpr int ACC_WORDS = 18;        // long accumulator: 576 bits

// Adds v (< 2^48) << (32 * w) into a little-endian multiword integer in LDS.
__device__ void long_add(uint32_t* acc, int w, uint64_t v) {
  uint64_t carry = v;
  for (int i = w; i < ACC_WORDS && carry != 0; ++i) {
    const uint64_t t = static_cast<uint64_t>(acc[i]) + (carry & 0xFFFFFFFFull);
    acc[i] = static_cast<uint32_t>(t);
    carry = (carry >> 32) + (t >> 32);
  }
}

// Exact sign of sum_c key[c] * s[c] over the 128 channels, from bf16 bits.
// Serial (one lane); only reached when a tree sum in fp64 cannot decide.
// Every bf16 value is sig * 2^(E - 134) with sig < 2^8 and 1 <= E <= 254, so
// each product is an integer sig_k*sig_s < 2^16 times 2^(Ek + Es - 268):
// it is added, shifted by Ek + Es - 2 bits, into one of two 576-bit
// magnitudes (positive / negative terms), which are compared at the end.
__device__ __forceinline__ bool exact_sign_long_inl(const uint16_t* key, const uint16_t* s_row,
                                                   uint32_t* scratch) {
  uint32_t* pos = scratch;
  uint32_t* neg = scratch + ACC_WORDS;
  for (int i = 0; i < 2 * ACC_WORDS; ++i) scratch[i] = 0;
  for (int c = 0; c < kHeadDim; ++c) {
    const uint32_t uk = key[c];
    const uint32_t us = s_row[c];
    uint32_t ek = (uk >> 7) & 0xFF, es = (us >> 7) & 0xFF;
    const uint32_t sk = ek ? ((uk & 0x7F) | 0x80) : (uk & 0x7F);
    const uint32_t ss = es ? ((us & 0x7F) | 0x80) : (us & 0x7F);
    if (sk == 0 || ss == 0) continue;
    ek = ek ? (ek > 254 ? 254 : ek) : 1;  // Inf/NaN inputs: undefined but in bounds
    es = es ? (es > 254 ? 254 : es) : 1;
    const uint32_t shift = ek + es - 2;   // 0 .. 506
    const uint64_t v = static_cast<uint64_t>(sk * ss) << (shift & 31);
    long_add(((uk ^ us) & 0x8000) ? neg : pos, static_cast<int>(shift >> 5), v);
  }
  for (int i = ACC_WORDS - 1; i >= 0; --i) {
    if (pos[i] != neg[i]) return pos[i] > neg[i];
  }
  return true;  // exact zero: sign(0) = +1
}
// The same as a call (kept out of line where its registers would crowd a
// kernel's main loop).
__device__ __attribute__((noinline)) bool exact_sign_long(const uint16_t* key, const uint16_t* s_row,
                                                          uint32_t* scratch) {
  return exact_sign_long_inl(key, s_row, scratch);
}

// Exact bf16 -> fp64 via fp32: a bf16 value is an fp32 value whose low 16
// bits are zero (normal or subnormal), and fp32 -> fp64 is exact.
__device__ __forceinline__ double bf16_lo_f64(uint32_t pair) {
  return static_cast<double>(__uint_as_float(pair << 16));
}
__device__ __forceinline__ double bf16_hi_f64(uint32_t pair) {
  return static_cast<double>(__uint_as_float(pair & 0xFFFF0000u));
}

// fp64 move within a quad of lanes through DPP (each half separately)
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double x) {
  const uint64_t u = __double_as_longlong(x);
  const uint32_t lo = __builtin_amdgcn_update_dpp(0u, static_cast<uint32_t>(u), CTRL, 0xF, 0xF, true);
  const uint32_t hi = __builtin_amdgcn_update_dpp(0u, static_cast<uint32_t>(u >> 32), CTRL, 0xF, 0xF, true);
  return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(hi) << 32) | lo));
}
constexpr int kQuadXor1 = 0xB1;   // quad_perm [1, 0, 3, 2]
constexpr int kQuadXor2 = 0x4E;   // quad_perm [2, 3, 0, 1]
// Sum over a quad of lanes: each step adds a lane's value to its partner's
// and the partner adds the same two numbers, so all four lanes end with
// bit-identical totals.
__device__ __forceinline__ double quad_sum_f64(double x) {
  x += dpp_f64<kQuadXor1>(x);
  x += dpp_f64<kQuadXor2>(x);
  return x;
}
__device__ __forceinline__ uint32_t quad_or(uint32_t x) {
  x |= __builtin_amdgcn_update_dpp(0u, x, kQuadXor1, 0xF, 0xF, true);
  x |= __builtin_amdgcn_update_dpp(0u, x, kQuadXor2, 0xF, 0xF, true);
  return x;
}

}  // namespace
}  // namespace qjl
