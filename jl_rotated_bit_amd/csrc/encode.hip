// QJL key encode for gfx950: sign bits of S^T k and ||k|| for every key.
//
// Method: "QJL: 1-Bit Quantized JL Transform for KV Cache Quantization with
// Zero Overhead", Abstract (JL transform, then one sign bit per coordinate,
// no quantization constants) and "The Geometry of Forgetting: How Three
// Papers Cracked KV Cache Quantization", section "QJL: one bit, zero
// parameters, unbiased inner products" (Q(x) = sign(Sx)).  The norm is kept
// because that section's formulas are written for unit vectors, which the
// random-rotation section reaches by scaling.
//
// Kernel design (one launch per call):
// * The projection P^T = S^T K^T runs on the matrix cores
//   (v_mfma_f32_32x32x16_bf16, fp32 accumulate).  A workgroup has m/64
//   waves; wave w owns sketch coordinates [64w, 64w+64) and keeps its slice
//   of S^T (64 x 128 bf16, 64 VGPRs) resident for the whole kernel.
// * Keys stream through LDS in tiles of 32 (one MFMA column block), loaded
//   with coalesced 16-byte reads and double-buffered; the next tile's loads
//   are in flight while the current tile is multiplied.
// * The A-operand rows are permuted so that lane (key j, half h) ends up
//   holding coordinates 64w + 32h + 0..31 of key j in its 32 accumulators:
//   one word of packed bits per lane, assembled with v_alignbit (one
//   instruction per bit-lane), no cross-lane traffic.
// * ||k||^2 comes from the same B fragments (bf16 dot2, fp32 accumulate).
// * Certification: an accumulator with |acc| <= tau, where tau bounds the
//   accumulation error of a d-term fp32 dot product of exact bf16 products
//   (with margin), is re-evaluated exactly: the wave sums the 128 fp64
//   products (exact) in a tree with a rigorous error bound, and falls back to
//   an exact integer long accumulator when even that is inconclusive.  The
//   resulting bit is the sign of the exact real sum, with sign(0) = +1.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "internal.h"

namespace qjl {
namespace {

typedef __bf16 bf16x8_t __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef __bf16 bf16x2_t __attribute__((__vector_size__(2 * sizeof(__bf16))));
typedef float f32x16_t __attribute__((__vector_size__(16 * sizeof(float))));

constexpr int D = kHeadDim;          // 128 key channels
constexpr int KB = 32;               // keys per MFMA column block
constexpr int NBLK = 4;              // column blocks per tile
constexpr int KT = KB * NBLK;        // keys per tile (128)
constexpr int CW = 64;               // sketch coordinates per wave
constexpr int ROW_B = D * 2;         // 256 bytes per key
constexpr int LDS_ROW = ROW_B + 16;  // padded LDS row: spreads lanes over banks
constexpr int TILE_LDS = KT * LDS_ROW;
constexpr int CHUNKS = KT * ROW_B / 16;  // 16-byte chunks per key tile (2048)
constexpr int ACC_WORDS = 18;        // long accumulator: 576 bits
constexpr int QCAP = 64;             // deferred-fix queue entries per wave
constexpr int FIXB = 16;             // (word, bit) fixes per batch of loads

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }
__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t v) { return __builtin_bit_cast(bf16x2_t, v); }

// Exact bf16 -> fp64 built from the bit fields (no fp32 step, so bf16
// subnormals are never flushed).
__device__ __forceinline__ double bf16_to_f64(uint32_t bits16) {
  const uint32_t e = (bits16 >> 7) & 0xFF;
  const uint32_t f = bits16 & 0x7F;
  const double v = e ? __longlong_as_double((static_cast<long long>(e + 896) << 52) |
                                            (static_cast<long long>(f) << 45))
                     : static_cast<double>(f) * 0x1.0p-133;
  return (bits16 & 0x8000) ? -v : v;
}

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
__device__ __attribute__((noinline)) bool exact_sign_long(const uint16_t* key_lds, const uint16_t* s_row,
                                                          uint32_t* scratch) {
  uint32_t* pos = scratch;
  uint32_t* neg = scratch + ACC_WORDS;
  for (int i = 0; i < 2 * ACC_WORDS; ++i) scratch[i] = 0;
  for (int c = 0; c < D; ++c) {
    const uint32_t uk = key_lds[c];
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

// DPP move of a float with every lane enabled and no old value (the
// compiler folds it into the consuming add)
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}

// lane src's pointer, as a wave-uniform value
__device__ __forceinline__ const uint16_t* readlane_ptr(const uint16_t* p, int src) {
  const uint64_t u = reinterpret_cast<uintptr_t>(p);
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(u), src));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(u >> 32), src));
  return reinterpret_cast<const uint16_t*>((static_cast<uint64_t>(hi) << 32) | lo);
}

// The same pairwise tree over the 64 lanes, through DPP row rotations and
// 16-/32-lane row swaps (VALU only, no LDS round trips): every lane ends
// with the sum of all 64 inputs, formed with 6 levels of additions.
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double x) {
  const uint64_t u = __double_as_longlong(x);
  const uint32_t lo = __builtin_amdgcn_update_dpp(0u, static_cast<uint32_t>(u), CTRL, 0xF, 0xF, true);
  const uint32_t hi = __builtin_amdgcn_update_dpp(0u, static_cast<uint32_t>(u >> 32), CTRL, 0xF, 0xF, true);
  return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(hi) << 32) | lo));
}
// x + (x of the lane 16 (WIDE: 32) lanes away): with both operands equal, a
// row swap returns [x g0, x g0, x g2, x g2] and [x g1, x g1, x g3, x g3]
// (16-lane groups g); their sum is the butterfly step in every lane.
template <bool WIDE>
__device__ __forceinline__ double swap_add_f64(double x) {
  const uint64_t u = __double_as_longlong(x);
  const uint32_t lo = static_cast<uint32_t>(u), hi = static_cast<uint32_t>(u >> 32);
  uint32_t l0, l1, h0, h1;
  if constexpr (WIDE) {
    const auto a = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
    const auto c = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
    l0 = a[0]; l1 = a[1]; h0 = c[0]; h1 = c[1];
  } else {
    const auto a = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
    const auto c = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
    l0 = a[0]; l1 = a[1]; h0 = c[0]; h1 = c[1];
  }
  return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(h0) << 32) | l0)) +
         __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(h1) << 32) | l1));
}
__device__ __forceinline__ double wave_sum_f64_dpp(double x) {
  x += dpp_f64<0x128>(x);   // row_ror:8
  x += dpp_f64<0x124>(x);   // row_ror:4
  x += dpp_f64<0x122>(x);   // row_ror:2
  x += dpp_f64<0x121>(x);   // row_ror:1
  x = swap_add_f64<false>(x);
  return swap_add_f64<true>(x);
}

// Exact bf16 -> fp64 via fp32: a bf16 value is an fp32 value whose low 16
// bits are zero (normal or subnormal), and fp32 -> fp64 is exact.
__device__ __forceinline__ double bf16_lo_f64(uint32_t pair) {
  return static_cast<double>(__uint_as_float(pair << 16));
}
__device__ __forceinline__ double bf16_hi_f64(uint32_t pair) {
  return static_cast<double>(__uint_as_float(pair & 0xFFFF0000u));
}

// lane 0's value as a wave-uniform double
__device__ __forceinline__ double uniform_f64(double x) {
  const uint64_t u = __double_as_longlong(x);
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(u)));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(u >> 32)));
  return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(hi) << 32) | lo));
}

// Exact sign bit of sum_c key[c] * s[c] for one (key, coordinate): lane l
// holds channels 2l and 2l+1 of both as bf16 pairs.  The 128 products are
// exact in fp64; pair_sum adds them in a 7-level tree, so
// |sum - exact| <= 7 * 2^-53 * sum|p| < 2^-50 * bnd for any bnd >= sum|p|,
// such as ||k|| max_i ||s_i|| (Cauchy-Schwarz).  decide() takes the bit when
// |sum| > 2^-49 * bnd and otherwise asks the exact integer accumulator.
__device__ __forceinline__ double pair_sum(uint32_t kpair, uint32_t spair) {
  const double p = bf16_lo_f64(kpair) * bf16_lo_f64(spair) + bf16_hi_f64(kpair) * bf16_hi_f64(spair);
  return wave_sum_f64_dpp(p);
}
__device__ bool decide(double sum, double bnd, uint32_t kpair, uint32_t spair, const uint16_t* key_row,
                       const uint16_t* s_row, uint32_t* scratch, int lane) {
  if (!(bnd < INFINITY)) {
    // the key norm left the fp32 range: bound from the magnitudes instead
    const double m = __builtin_fabs(bf16_lo_f64(kpair) * bf16_lo_f64(spair)) +
                     __builtin_fabs(bf16_hi_f64(kpair) * bf16_hi_f64(spair));
    bnd = uniform_f64(wave_sum_f64_dpp(m)) * (1.0 + 0x1.0p-40);
  }
  if (__builtin_fabs(sum) > 0x1.0p-49 * bnd) return sum > 0.0;
  bool b = false;
  if (lane == 0) b = exact_sign_long(key_row, s_row, scratch);
  return __builtin_amdgcn_readfirstlane(static_cast<int>(b)) != 0;
}

// Norm of a key whose fp32 sum of squares under- or overflowed: scale by a
// power of two first (exact), then undo it.
__device__ float scaled_norm(const uint16_t* key_lds) {
  uint32_t emax = 0;
  for (int c = 0; c < D; ++c) {
    const uint32_t e = (key_lds[c] >> 7) & 0xFF;
    emax = e > emax ? e : emax;
  }
  if (emax == 0) {
    // all zeros or bf16 subnormals: scale up by 2^64 (exact)
    float s = 0.f;
    for (int c = 0; c < D; ++c) {
      const float v = __uint_as_float(static_cast<uint32_t>(key_lds[c]) << 16) * 0x1.0p64f;
      s = __builtin_fmaf(v, v, s);
    }
    return __builtin_sqrtf(s) * 0x1.0p-64f;
  }
  const int e = static_cast<int>(emax) - 127;
  float s = 0.f;
  for (int c = 0; c < D; ++c) {
    const float v = __builtin_ldexpf(__uint_as_float(static_cast<uint32_t>(key_lds[c]) << 16), -e);
    s = __builtin_fmaf(v, v, s);
  }
  return __builtin_ldexpf(__builtin_sqrtf(s), e);
}

// Sign of sum_c key[c] * s[c] for one (key, coordinate) in one lane: kr
// holds the key's 128 bf16 values, s_row points at the sketch row.  Every
// product of two bf16 values is exact in fp64; four running sums of 32
// products each and their total form a summation tree of height 34, so the
// result is off by at most 34 * 2^-53 * sum|p| < 2^-47 * bnd for any
// bnd >= sum|p| (such as ||k|| max_i ||s_i||, by Cauchy-Schwarz).  Returns
// the bit (1 for a positive sum) when |sum| > 2^-46 * bnd, else -1.
// (Each 8-product group's conversions stay next to its products; hoisted,
// the 256 doubles would not fit in registers.)
__device__ __forceinline__ int serial_sign(const uint4 (&kr)[D / 8], const uint4* s_row, double bnd) {
  uint4 sv[D / 8];
#pragma unroll
  for (int i = 0; i < D / 8; ++i) sv[i] = s_row[i];
  double acc[4] = {0.0, 0.0, 0.0, 0.0};
  double mag = 0.0;
  const bool need_mag = !(bnd < INFINITY);   // the key norm left the fp32 range
#pragma unroll
  for (int i = 0; i < D / 8; ++i) {
    __builtin_amdgcn_sched_barrier(0);
    uint32_t kw[4] = {kr[i].x, kr[i].y, kr[i].z, kr[i].w};
    // opaque to the optimizer: the caller loops over bits with kr fixed, and
    // hoisting these conversions out of that loop would need 256 doubles
    asm volatile("" : "+v"(kw[0]), "+v"(kw[1]), "+v"(kw[2]), "+v"(kw[3]));
    const uint32_t sw[4] = {sv[i].x, sv[i].y, sv[i].z, sv[i].w};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const double p0 = bf16_lo_f64(kw[u]) * bf16_lo_f64(sw[u]);
      const double p1 = bf16_hi_f64(kw[u]) * bf16_hi_f64(sw[u]);
      acc[u] += p0;
      acc[u] += p1;
      if (need_mag) mag += __builtin_fabs(p0) + __builtin_fabs(p1);
    }
  }
  const double sum = (acc[0] + acc[1]) + (acc[2] + acc[3]);
  // magnitude bound: sum|p| computed with relative error below 2^-46
  if (need_mag) bnd = mag * (1.0 + 0x1.0p-40);
  if (__builtin_fabs(sum) > 0x1.0p-46 * bnd) return sum > 0.0 ? 1 : 0;
  return -1;
}

template <int M>
__global__ __launch_bounds__(64 * (M / CW)) __attribute__((amdgpu_waves_per_eu(2))) void encode_kernel(
    const uint16_t* __restrict__ keys, const uint16_t* __restrict__ s_md,
    const float* __restrict__ col_norm_max, uint32_t* __restrict__ signs,
    float* __restrict__ norms, int R, int n, int cap, int pos, int ntiles, float c1,
    float c2) {
  constexpr int W = M / CW;
  constexpr int NT = 64 * W;
  constexpr int LOADS = CHUNKS / NT;  // 16-byte loads per thread per tile
  constexpr int WPR = M / 32;         // words per key row
  static_assert(NT % 16 == 0, "the 16 chunks of a key row must sit in one 16-lane row");

  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * TILE_LDS];
  __shared__ float n2buf[2][KT];   // squared key norms of the tile
  __shared__ uint32_t long_scratch[W][2 * ACC_WORDS];
  // Sign words with bits to certify, queued per wave for an exact fix after
  // the last tile: {key row | half << 31, word, flags, 0}.  The fix then
  // gives one entry to each lane, all loads in flight together.
  __shared__ uint4 fixq[W][QCAP];
  __shared__ float fixn[W][QCAP];   // upper bound of ||k|| of the entry's key
  int qn = 0;   // queued entries of this wave (uniform)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int j = lane & 31;
  const int cb = wave * CW;
  const uint32_t un = static_cast<uint32_t>(n);
  const uint32_t uR = static_cast<uint32_t>(R);

  // Resident A operand: S^T rows for this wave's coordinates.  Block b, row i
  // holds coordinate cb + 32*((i >> 2) & 1) + 16*b + 4*(i >> 3) + (i & 3), so
  // the 32x32 result places coordinate cb + 32*half + 16*b + r in register r
  // of lane (j, half).
  bf16x8_t a[2][8];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int coord = cb + 32 * ((j >> 2) & 1) + 16 * b + 4 * (j >> 3) + (j & 3);
    const uint4* row = reinterpret_cast<const uint4*>(s_md + static_cast<int64_t>(coord) * D);
#pragma unroll
    for (int s = 0; s < 8; ++s) a[b][s] = as_bf16x8(row[2 * s + half]);
  }
  const float smax = col_norm_max[wave];

  // chunk c of a tile: key row c / 16, 16-byte column c % 16; the 16 chunks
  // of a row belong to 16 consecutive threads (one DPP row)
  uint4 pf[LOADS];
  auto load_tile = [&](int tile) {
#pragma unroll
    for (int k = 0; k < LOADS; ++k) {
      const int c = tid + k * NT;
      const uint32_t r = static_cast<uint32_t>(tile) * KT + (c >> 4);
      pf[k] = r < uR ? reinterpret_cast<const uint4*>(keys + static_cast<int64_t>(r) * D)[c & 15]
                     : make_uint4(0, 0, 0, 0);
    }
  };

  if (blockIdx.x < ntiles) load_tile(blockIdx.x);
  int buf = 0;
  for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    uint8_t* tl = lds + buf * TILE_LDS;
    // squared norms of the tile's keys, once per tile: each thread squares its
    // chunks (bf16 dot2, fp32), a DPP row sum adds the 16 chunks of a key
#pragma unroll
    for (int k = 0; k < LOADS; ++k) {
      const uint4 v = pf[k];
      float q = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(v.x), as_bf16x2(v.x), 0.f, false);
      q = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(v.y), as_bf16x2(v.y), q, false);
      q = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(v.z), as_bf16x2(v.z), q, false);
      q = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(v.w), as_bf16x2(v.w), q, false);
      q += dpp_f32<0x128>(q);   // row_ror:8
      q += dpp_f32<0x124>(q);   // row_ror:4
      q += dpp_f32<0x122>(q);   // row_ror:2
      q += dpp_f32<0x121>(q);   // row_ror:1
      if ((tid & 15) == 0) n2buf[buf][(tid >> 4) + k * (NT / 16)] = q;
    }
#pragma unroll
    for (int k = 0; k < LOADS; ++k) {
      const int c = tid + k * NT;
      *reinterpret_cast<uint4*>(tl + (c >> 4) * LDS_ROW + (c & 15) * 16) = pf[k];
    }
    __syncthreads();
    if (tile + static_cast<int>(gridDim.x) < ntiles) load_tile(tile + gridDim.x);
    // (batch * head, position) of the tile's first key, once per tile (the
    // host keeps the key count below 2^31)
    const uint32_t tb = static_cast<uint32_t>(tile) * KT;
    const uint32_t tbh = tb / un;
    const uint32_t toff = tb - tbh * un;

    // ---- projection on the matrix cores ----
    auto project = [&](int nb, f32x16_t& acc0, f32x16_t& acc1) {
      acc0 = f32x16_t{};
      acc1 = f32x16_t{};
      const uint8_t* krow = tl + (nb * KB + j) * LDS_ROW + 16 * half;
  #pragma unroll
      for (int s = 0; s < 8; ++s) {
        const bf16x8_t bf = as_bf16x8(*reinterpret_cast<const uint4*>(krow + 32 * s));
        acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0][s], bf, acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1][s], bf, acc1, 0, 0, 0);
      }
    };

    // ---- bits of one block: signs, certification, stores ----
    auto process = [&](int nb, const f32x16_t& acc0, const f32x16_t& acc1) {
      const float n2 = n2buf[buf][nb * KB + j];
      // ---- certification threshold for this lane's key ----
      // ||k|| <= sqrt(n2 (1 + 2^-14) + 2^-119): fp32 rounding of 128 exact
      // squares plus squares lost below the fp32 normal range (with margin).
      const float knorm_up = __builtin_sqrtf(__builtin_fmaf(n2, 1.0f + 0x1.0p-14f, 0x1.0p-118f));
      const float tau = __builtin_fmaf(c1 * knorm_up, smax, c2);

      // ---- sign word, highest coordinate shifted in first ----
      uint32_t sw = 0;
      float amin = __builtin_fabsf(acc0[0]);
  #pragma unroll
      for (int r = 15; r >= 0; --r) {
        sw = __builtin_amdgcn_alignbit(sw, __float_as_uint(acc1[r]), 31);
        amin = fminf(amin, __builtin_fabsf(acc1[r]));
      }
  #pragma unroll
      for (int r = 15; r >= 0; --r) {
        sw = __builtin_amdgcn_alignbit(sw, __float_as_uint(acc0[r]), 31);
        amin = fminf(amin, __builtin_fabsf(acc0[r]));
      }
      uint32_t word = ~sw;
      // ---- flag word (|acc| <= tau), only when some lane of the wave has one ----
      uint32_t flags = 0;
      if (__ballot(amin <= tau) != 0) {
        uint32_t fw = 0;
  #pragma unroll
        for (int r = 15; r >= 0; --r) fw = __builtin_amdgcn_alignbit(fw, __float_as_uint(tau - __builtin_fabsf(acc1[r])), 31);
  #pragma unroll
        for (int r = 15; r >= 0; --r) fw = __builtin_amdgcn_alignbit(fw, __float_as_uint(tau - __builtin_fabsf(acc0[r])), 31);
        flags = ~fw;
      }
      // keys so large that products can overflow fp32: certify every bit
      if (!(n2 < 0x1.0p100f)) flags = 0xFFFFFFFFu;
      const uint32_t r = tb + nb * KB + j;
      const bool valid = r < uR;
      if (!valid) flags = 0;  // zero padding of a ragged last tile
      // destination row: (batch * head) = tbh + wraps, position = offset
      uint32_t off = toff + nb * KB + j, bhl = tbh;
      if (un > static_cast<uint32_t>(KT)) {   // at most one wrap within a tile
        if (off >= un) {
          off -= un;
          ++bhl;
        }
      } else {
        const uint32_t w = off / un;
        bhl += w;
        off -= w * un;
      }
      const int64_t dst = static_cast<int64_t>(bhl) * cap + pos + off;

      // ---- flagged words: queued for the exact fix after the last tile, or
      // (queue full) fixed here, one (key, coordinate) pair at a time ----
      const uint64_t need = __ballot(flags != 0);
      bool deferred = false;
      if (need) {
        const int cnt = __popcll(need);
        if (qn + cnt <= QCAP) {
          if (flags != 0) {
            const int slot = qn + static_cast<int>(__builtin_amdgcn_mbcnt_hi(
                                      static_cast<uint32_t>(need >> 32),
                                      __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(need), 0u)));
            fixq[wave][slot] = make_uint4(r | (static_cast<uint32_t>(half) << 31), word, flags, 0u);
            fixn[wave][slot] = knorm_up;
            deferred = true;
          }
          qn += cnt;
        } else {
          uint64_t todo = need;
          while (todo) {
            const int src = __builtin_ctzll(todo);
            todo &= todo - 1;
            uint32_t fsrc = __shfl(flags, src);
            const int jsrc = src & 31;
            const int hsrc = src >> 5;
            const uint16_t* key_lds = reinterpret_cast<const uint16_t*>(tl + (nb * KB + jsrc) * LDS_ROW);
            const uint32_t kpair = reinterpret_cast<const uint32_t*>(key_lds)[lane];
            if (__ballot((kpair & 0x7FFF7FFFu) != 0) == 0) {
              // the key is all (+/-) zeros: every projection is exactly 0 -> bit 1
              if (lane == src) word |= fsrc;
              continue;
            }
            while (fsrc) {
              const int p = __builtin_ctz(fsrc);
              fsrc &= fsrc - 1;
              const uint16_t* s_row = s_md + static_cast<int64_t>(cb + 32 * hsrc + p) * D;
              const uint32_t spair = reinterpret_cast<const uint32_t*>(s_row)[lane];
              const double bnd = static_cast<double>(__shfl(knorm_up, src)) * smax;
              const bool bit = decide(uniform_f64(pair_sum(kpair, spair)), bnd, kpair, spair, key_lds, s_row,
                                      long_scratch[wave], lane);
              if (lane == src) word = bit ? (word | (1u << p)) : (word & ~(1u << p));
            }
          }
        }
      }

      // ---- stores ----
      if (valid) {
        if (!deferred) signs[dst * WPR + (cb >> 5) + half] = word;
        if (wave == 0 && half == 0) {
          float nrm = __builtin_sqrtf(n2);
          if (!(n2 >= 0x1.0p-100f && n2 <= 0x1.0p100f)) {
            nrm = scaled_norm(reinterpret_cast<const uint16_t*>(tl + (nb * KB + j) * LDS_ROW));
          }
          norms[dst] = nrm;
        }
      }
    };

    // Software pipeline over the blocks of the tile: the next block's matrix
    // products are issued before this block's bit extraction, so they run
    // while it executes.
    f32x16_t c0, c1, d0, d1;
    project(0, c0, c1);
  #pragma unroll
    for (int nb = 0; nb < NBLK; ++nb) {
      if (nb + 1 < NBLK) project(nb + 1, d0, d1);
      process(nb, c0, c1);
      c0 = d0;
      c1 = d1;
    }
    buf ^= 1;
  }

  // ---- deferred exact fixes: lane e takes queue entry e (QCAP <= 64) and
  // decides its flagged bits one per pass, lowest first, from its own loads
  // of the key row and of the sketch row; the rare sums too close to zero
  // for the fp64 bound go, one at a time, to the exact integer accumulator ----
  if (qn > 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const bool act = lane < qn;
    const uint4 ent = act ? fixq[wave][lane] : make_uint4(0, 0, 0, 0);
    const float knu = act ? fixn[wave][lane] : 0.f;
    const uint32_t r = ent.x & 0x7FFFFFFFu;
    const int hf = static_cast<int>(ent.x >> 31);
    uint32_t word = ent.y;
    uint32_t fl = ent.z;
    const uint16_t* krow = keys + static_cast<int64_t>(r) * D;
    uint4 kr[D / 8];
#pragma unroll
    for (int i = 0; i < D / 8; ++i) kr[i] = act ? reinterpret_cast<const uint4*>(krow)[i] : make_uint4(0, 0, 0, 0);
    uint32_t nz = 0;
#pragma unroll
    for (int i = 0; i < D / 8; ++i) nz |= (kr[i].x | kr[i].y | kr[i].z | kr[i].w) & 0x7FFF7FFFu;
    if (nz == 0) {   // an all (+/-) zero key projects to exactly 0: bit 1
      word |= fl;
      fl = 0;
    }
    const double bnd = static_cast<double>(knu) * smax;
    uint32_t slow = 0;   // bits the fp64 sum could not decide
    while (__ballot(fl != 0)) {
      if (fl) {
        const int p = __builtin_ctz(fl);
        const uint16_t* srow = s_md + static_cast<int64_t>(cb + 32 * hf + p) * D;
        const int bit = serial_sign(kr, reinterpret_cast<const uint4*>(srow), bnd);
        if (bit < 0) slow |= 1u << p;
        else word = bit ? (word | (1u << p)) : (word & ~(1u << p));
        fl &= fl - 1;
      }
    }
    // exact integer sums, one (key, coordinate) at a time on lane 0
    for (uint64_t lanes = __ballot(slow != 0); lanes; lanes &= lanes - 1) {
      const int src = __builtin_ctzll(lanes);
      uint32_t bits = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(slow), src));
      const uint16_t* kp = readlane_ptr(krow, src);
      const int hsrc = __builtin_amdgcn_readlane(hf, src);
      while (bits) {
        const int p = __builtin_ctz(bits);
        bits &= bits - 1;
        bool b = false;
        if (lane == 0) b = exact_sign_long(kp, s_md + static_cast<int64_t>(cb + 32 * hsrc + p) * D, long_scratch[wave]);
        b = __builtin_amdgcn_readfirstlane(static_cast<int>(b)) != 0;
        if (lane == src) word = b ? (word | (1u << p)) : (word & ~(1u << p));
      }
    }
    if (act) {
      const uint32_t bh = r / un;
      const int64_t dst = static_cast<int64_t>(bh) * cap + pos + (r - bh * un);
      signs[dst * WPR + (cb >> 5) + hf] = word;
    }
  }
}

template <int M>
int launch_encode_m(const DeviceSketch& s, const void* keys, int R, int n, uint32_t* signs,
                    float* norms, int cap, int pos, hipStream_t stream) {
  constexpr int NT = 64 * (M / CW);
  const int ntiles = static_cast<int>((static_cast<int64_t>(R) + KT - 1) / KT);
  static int max_grid = 0;  // resident workgroups on this device (fixed per template)
  if (max_grid == 0) {
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return hipErrorInvalidDevice;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return hipErrorInvalidDevice;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, encode_kernel<M>, NT, 0) !=
        hipSuccess)
      return hipErrorInvalidDeviceFunction;
    max_grid = cus * (per_cu > 0 ? per_cu : 1);
  }
  const int grid = ntiles < max_grid ? ntiles : max_grid;
  // Error bound of an fp32 sum of D exact products, with a factor 4 margin
  // over round-to-nearest (covers truncating or blocked accumulation).
  const float c1 = static_cast<float>(4.0 * D * 0x1.0p-24 * (1.0 + 0x1.0p-10));
  const float c2 = 0x1.0p-110f;  // absolute floor: subnormal flushes
  hipLaunchKernelGGL(encode_kernel<M>, dim3(grid), dim3(NT), 0, stream,
                     static_cast<const uint16_t*>(keys), s.s_md, s.col_norm_max, signs, norms, R,
                     n, cap, pos, ntiles, c1, c2);
  return hipGetLastError();
}

}  // namespace

int launch_encode(const DeviceSketch& s, const void* keys, int B, int H_kv, int n, uint32_t* signs,
                  float* norms, int cap, int pos, void* stream) {
  const int64_t R = static_cast<int64_t>(B) * H_kv * n;
  if (R == 0) return hipSuccess;
  if (R > INT32_MAX) return hipErrorInvalidValue;   // the kernel indexes keys in 32 bits
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (s.m == 256) return launch_encode_m<256>(s, keys, static_cast<int>(R), n, signs, norms, cap, pos, st);
  return launch_encode_m<512>(s, keys, static_cast<int>(R), n, signs, norms, cap, pos, st);
}

}  // namespace qjl
