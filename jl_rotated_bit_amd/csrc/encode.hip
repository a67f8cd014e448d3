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
#include <type_traits>

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

// Exact bf16 -> fp64 via fp32: a bf16 value is an fp32 value whose low 16
// bits are zero (normal or subnormal), and fp32 -> fp64 is exact.
__device__ __forceinline__ double bf16_lo_f64(uint32_t pair) {
  return static_cast<double>(__uint_as_float(pair << 16));
}
__device__ __forceinline__ double bf16_hi_f64(uint32_t pair) {
  return static_cast<double>(__uint_as_float(pair & 0xFFFF0000u));
}

// Norm of a key whose fp32 sum of squares under- or overflowed: scale by a
// power of two first (exact), then undo it.
__device__ float scaled_norm(const uint16_t* key) {
  uint32_t emax = 0;
  for (int c = 0; c < D; ++c) {
    const uint32_t e = (key[c] >> 7) & 0xFF;
    emax = e > emax ? e : emax;
  }
  if (emax == 0) {
    // all zeros or bf16 subnormals: scale up by 2^64 (exact)
    float s = 0.f;
    for (int c = 0; c < D; ++c) {
      const float v = __uint_as_float(static_cast<uint32_t>(key[c]) << 16) * 0x1.0p64f;
      s = __builtin_fmaf(v, v, s);
    }
    return __builtin_sqrtf(s) * 0x1.0p-64f;
  }
  const int e = static_cast<int>(emax) - 127;
  float s = 0.f;
  for (int c = 0; c < D; ++c) {
    const float v = __builtin_ldexpf(__uint_as_float(static_cast<uint32_t>(key[c]) << 16), -e);
    s = __builtin_fmaf(v, v, s);
  }
  return __builtin_ldexpf(__builtin_sqrtf(s), e);
}

// fp64 move across a 16-lane row through DPP (each half separately)
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double x) {
  const uint64_t u = __double_as_longlong(x);
  const uint32_t lo = __builtin_amdgcn_update_dpp(0u, static_cast<uint32_t>(u), CTRL, 0xF, 0xF, true);
  const uint32_t hi = __builtin_amdgcn_update_dpp(0u, static_cast<uint32_t>(u >> 32), CTRL, 0xF, 0xF, true);
  return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(hi) << 32) | lo));
}
constexpr int kRowMirror = 0x140;      // lane i <-> 15 - i
constexpr int kRowHalfMirror = 0x141;  // lane i <-> 7 - i within each half row
constexpr int kQuadXor2 = 0x4E;        // quad_perm [2, 3, 0, 1]
constexpr int kQuadXor1 = 0xB1;        // quad_perm [1, 0, 3, 2]
// Sum over a 16-lane row: mirror, half-mirror, then quad swaps.  Every step
// adds a lane's value to its partner's and the partner adds the same two
// numbers, so all 16 lanes end with bit-identical totals (tree height 4).
__device__ __forceinline__ double row_sum_f64(double x) {
  x += dpp_f64<kRowMirror>(x);
  x += dpp_f64<kRowHalfMirror>(x);
  x += dpp_f64<kQuadXor2>(x);
  x += dpp_f64<kQuadXor1>(x);
  return x;
}
__device__ __forceinline__ uint32_t row_or(uint32_t x) {
  x |= __builtin_amdgcn_update_dpp(0u, x, kRowMirror, 0xF, 0xF, true);
  x |= __builtin_amdgcn_update_dpp(0u, x, kRowHalfMirror, 0xF, 0xF, true);
  x |= __builtin_amdgcn_update_dpp(0u, x, kQuadXor2, 0xF, 0xF, true);
  x |= __builtin_amdgcn_update_dpp(0u, x, kQuadXor1, 0xF, 0xF, true);
  return x;
}

// Exact-sign evaluation of queued sign words (the words whose flagged bits
// the fp32 projection could not certify).  Sixteen lanes serve one entry:
// lane (group g, sub c) loads 16 bytes (channels 8c .. 8c+7) of the key row
// and of the sketch row, so every load instruction reads four whole rows.
// The eight products of a lane are exact in fp64 and are added in order,
// then row_sum_f64 adds the 16 lanes: a summation tree of height 11, off by
// at most 11 * 2^-53 * sum|p| < 2^-49 * bnd for any bnd >= sum|p| (such as
// ||k|| max_i ||s_i||, Cauchy-Schwarz).  The bit is the sign of the sum when
// |sum| > 2^-46 * bnd; the rare sums below that go, one at a time, to the
// exact integer accumulator.  RU rounds of four entries have their loads in
// flight together; flagged bits of an entry are taken one pass each, lowest
// first.  fq/fk: the queue ({key row | half << 31, word, flags, -}, norm
// bound); the decided words are stored to their rows.
template <int RU>
__device__ __forceinline__ void fix_queue(const uint4* fq, const float* fk, int qn, const uint16_t* keys,
                                          const uint16_t* s_md, int cb, float smax, uint32_t* signs,
                                          uint32_t un, int cap, int pos, int wpr, uint32_t* scratch,
                                          int lane) {
  const int g = lane >> 4, sub = lane & 15;
  for (int base = 0; base < qn; base += 4 * RU) {
    uint4 kc[RU], sc[RU];
    uint32_t word[RU], fl[RU], row[RU], slow[RU];
    int hf[RU], p[RU];
    double bnd[RU];
#pragma unroll
    for (int t = 0; t < RU; ++t) {
      const int e = base + 4 * t + g;
      const bool act = e < qn;
      const uint4 ent = act ? fq[e] : make_uint4(0, 0, 0, 0);
      row[t] = ent.x & 0x7FFFFFFFu;
      hf[t] = static_cast<int>(ent.x >> 31);
      word[t] = ent.y;
      fl[t] = ent.z;   // zero for inactive entries
      bnd[t] = act ? static_cast<double>(fk[e]) * smax : 0.0;
      p[t] = fl[t] ? __builtin_ctz(fl[t]) : 0;
      slow[t] = 0;
      kc[t] = act ? reinterpret_cast<const uint4*>(keys + static_cast<int64_t>(row[t]) * D)[sub]
                  : make_uint4(0, 0, 0, 0);
      sc[t] = fl[t] ? reinterpret_cast<const uint4*>(s_md + static_cast<int64_t>(cb + 32 * hf[t] + p[t]) * D)[sub]
                    : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int t = 0; t < RU; ++t) {   // an all (+/-) zero key projects to exactly 0: bit 1
      if (row_or((kc[t].x | kc[t].y | kc[t].z | kc[t].w) & 0x7FFF7FFFu) == 0) {
        word[t] |= fl[t];
        fl[t] = 0;
      }
    }
    for (;;) {
      uint32_t any = 0;
#pragma unroll
      for (int t = 0; t < RU; ++t) any |= fl[t];
      if (__ballot(any != 0) == 0) break;
#pragma unroll
      for (int t = 0; t < RU; ++t) {
        if (fl[t] == 0) continue;   // uniform over the entry's 16 lanes
        const uint32_t kw[4] = {kc[t].x, kc[t].y, kc[t].z, kc[t].w};
        const uint32_t sw[4] = {sc[t].x, sc[t].y, sc[t].z, sc[t].w};
        double acc = 0.0, mag = 0.0;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const double p0 = bf16_lo_f64(kw[u]) * bf16_lo_f64(sw[u]);
          const double p1 = bf16_hi_f64(kw[u]) * bf16_hi_f64(sw[u]);
          acc += p0;
          acc += p1;
          mag += __builtin_fabs(p0);
          mag += __builtin_fabs(p1);
        }
        const double sum = row_sum_f64(acc);
        double b = bnd[t];
        if (!(b < INFINITY)) b = row_sum_f64(mag) * (1.0 + 0x1.0p-40);   // the key norm left fp32
        const uint32_t m = 1u << p[t];
        if (__builtin_fabs(sum) > 0x1.0p-46 * b) word[t] = sum > 0.0 ? (word[t] | m) : (word[t] & ~m);
        else slow[t] |= m;
        fl[t] &= fl[t] - 1;
        if (fl[t]) {   // next flagged coordinate of this entry
          p[t] = __builtin_ctz(fl[t]);
          sc[t] = reinterpret_cast<const uint4*>(s_md + static_cast<int64_t>(cb + 32 * hf[t] + p[t]) * D)[sub];
        }
      }
    }
    // exact integer sums, one (key, coordinate) at a time on lane 0
#pragma unroll
    for (int t = 0; t < RU; ++t) {
      for (uint64_t heads = __ballot(sub == 0 && slow[t] != 0); heads; heads &= heads - 1) {
        const int src = __builtin_ctzll(heads);
        uint32_t bits = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(slow[t]), src));
        const uint32_t rsrc = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(row[t]), src));
        const int hsrc = __builtin_amdgcn_readlane(hf[t], src);
        while (bits) {
          const int q = __builtin_ctz(bits);
          bits &= bits - 1;
          bool bit = false;
          if (lane == 0)
            bit = exact_sign_long(keys + static_cast<int64_t>(rsrc) * D,
                                  s_md + static_cast<int64_t>(cb + 32 * hsrc + q) * D, scratch);
          bit = __builtin_amdgcn_readfirstlane(static_cast<int>(bit)) != 0;
          if ((lane >> 4) == (src >> 4)) word[t] = bit ? (word[t] | (1u << q)) : (word[t] & ~(1u << q));
        }
      }
    }
#pragma unroll
    for (int t = 0; t < RU; ++t) {
      if (sub == 0 && base + 4 * t + g < qn) {
        const uint32_t bh = row[t] / un;
        const int64_t dst = static_cast<int64_t>(bh) * cap + pos + (row[t] - bh * un);
        signs[dst * wpr + (cb >> 5) + hf[t]] = word[t];
      }
    }
  }
}

template <int M>
__global__ __launch_bounds__(64 * (M / CW)) __attribute__((amdgpu_waves_per_eu(2))) void encode_kernel(
    const uint16_t* __restrict__ keys, const uint16_t* __restrict__ s_md,
    const uint16_t* __restrict__ s_efrag, const float* __restrict__ col_norm_max, uint32_t* __restrict__ signs,
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
  // (s_efrag holds these fragments in lane order: one 1 KB load each)
  bf16x8_t a[2][8];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const uint4* fr = reinterpret_cast<const uint4*>(s_efrag) + (static_cast<int64_t>(wave) * 2 + b) * 8 * 64 + lane;
#pragma unroll
    for (int s = 0; s < 8; ++s) a[b][s] = as_bf16x8(fr[s * 64]);
  }
  const float smax = col_norm_max[wave];
  // decides and stores the queued words of this wave (uniform call): RU
  // rounds of four entries at a time (fewer registers inside the tile loop)
  auto flush = [&](auto ru) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    fix_queue<decltype(ru)::value>(fixq[wave], fixn[wave], qn, keys, s_md, cb, smax, signs, un, cap, pos, WPR,
                                   long_scratch[wave], lane);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

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

  // staged tile -> LDS tile bb, and its keys' squared norms -> n2buf[bb]:
  // each thread squares its chunks (bf16 dot2, fp32), a DPP row sum adds the
  // 16 chunks of a key
  auto stage = [&](int bb) {
    uint8_t* t = lds + bb * TILE_LDS;
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
      if ((tid & 15) == 0) n2buf[bb][(tid >> 4) + k * (NT / 16)] = q;
    }
#pragma unroll
    for (int k = 0; k < LOADS; ++k) {
      const int c = tid + k * NT;
      *reinterpret_cast<uint4*>(t + (c >> 4) * LDS_ROW + (c & 15) * 16) = pf[k];
    }
  };

  // ---- projection on the matrix cores (block nb of LDS tile bb) ----
  auto project = [&](int bb, int nb, f32x16_t& acc0, f32x16_t& acc1) {
    acc0 = f32x16_t{};
    acc1 = f32x16_t{};
    const uint8_t* krow = lds + bb * TILE_LDS + (nb * KB + j) * LDS_ROW + 16 * half;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const bf16x8_t bf = as_bf16x8(*reinterpret_cast<const uint4*>(krow + 32 * s));
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0][s], bf, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1][s], bf, acc1, 0, 0, 0);
    }
  };

  // Software pipeline: the next block's matrix products (across tile
  // boundaries too) are issued before this block's bit extraction, so they
  // run while it executes.  Tiles alternate between two LDS buffers; the
  // barrier that publishes tile t+1 sits inside the last block of tile t.
  // An LDS tile is read only by project(), and its last reads (tile t-1)
  // come before the barrier that precedes its next write (tile t+1); the
  // norms are copied to registers right after the barrier that publishes them.
  int buf = 0;
  f32x16_t cur0, cur1, nxt0, nxt1;   // accumulators of this block and the next
  float n2r[NBLK];
  if (blockIdx.x < ntiles) {
    load_tile(blockIdx.x);
    stage(0);
    __syncthreads();
    if (static_cast<int>(blockIdx.x + gridDim.x) < ntiles) load_tile(blockIdx.x + gridDim.x);
#pragma unroll
    for (int k = 0; k < NBLK; ++k) n2r[k] = n2buf[0][k * KB + j];
    project(0, 0, cur0, cur1);
  }
  for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const bool more = tile + static_cast<int>(gridDim.x) < ntiles;   // uniform
    // (batch * head, position) of the tile's first key, once per tile (the
    // host keeps the key count below 2^31)
    const uint32_t tb = static_cast<uint32_t>(tile) * KT;
    const uint32_t tbh = tb / un;
    const uint32_t toff = tb - tbh * un;
    const int64_t dst0 = static_cast<int64_t>(tbh) * cap + pos + toff;   // row tb's destination
    const uint32_t wrap_at = un - toff;                                  // first row of the next (b, h)
    const uint32_t wrap_add = static_cast<uint32_t>(cap) - un;
    float n2n[NBLK];

    // ---- bits of one block: signs, certification, stores ----
    auto process = [&](int nb, const f32x16_t& acc0, const f32x16_t& acc1, float n2) {
      // ---- certification threshold for this lane's key ----
      // ||k|| <= sqrt(n2 (1 + 2^-14) + 2^-119): fp32 rounding of 128 exact
      // squares plus squares lost below the fp32 normal range (with margin).
      // (v_sqrt_f32 is within 1 ulp; the factor 1 + 2^-20 keeps the bound)
      const float knorm_up =
          __builtin_amdgcn_sqrtf(__builtin_fmaf(n2, 1.0f + 0x1.0p-14f, 0x1.0p-118f)) * (1.0f + 0x1.0p-20f);
      const float tau = __builtin_fmaf(c1 * knorm_up, smax, c2);

      // ---- sign word, highest coordinate shifted in first: acc1 gives bits
      // 16..31, acc0 bits 0..15 ----
      uint32_t sw = 0;
      float amin1 = __builtin_fabsf(acc1[0]);
      float amin0 = __builtin_fabsf(acc0[0]);
  #pragma unroll
      for (int r = 15; r >= 0; --r) {
        sw = __builtin_amdgcn_alignbit(sw, __float_as_uint(acc1[r]), 31);
        amin1 = fminf(amin1, __builtin_fabsf(acc1[r]));
      }
  #pragma unroll
      for (int r = 15; r >= 0; --r) {
        sw = __builtin_amdgcn_alignbit(sw, __float_as_uint(acc0[r]), 31);
        amin0 = fminf(amin0, __builtin_fabsf(acc0[r]));
      }
      uint32_t word = ~sw;
      // ---- flag bits (|acc| <= tau), each half only when some lane of the
      // wave has one there ----
      uint32_t fw1 = 0xFFFFu, fw0 = 0xFFFFu;   // set bit: not flagged
      if (__ballot(amin1 <= tau) != 0) {
        fw1 = 0;
  #pragma unroll
        for (int r = 15; r >= 0; --r) fw1 = __builtin_amdgcn_alignbit(fw1, __float_as_uint(tau - __builtin_fabsf(acc1[r])), 31);
      }
      if (__ballot(amin0 <= tau) != 0) {
        fw0 = 0;
  #pragma unroll
        for (int r = 15; r >= 0; --r) fw0 = __builtin_amdgcn_alignbit(fw0, __float_as_uint(tau - __builtin_fabsf(acc0[r])), 31);
      }
      uint32_t flags = ~((fw1 << 16) | fw0);
      // keys so large that products can overflow fp32: certify every bit
      if (!(n2 < 0x1.0p100f)) flags = 0xFFFFFFFFu;
      const uint32_t r = tb + nb * KB + j;
      const bool valid = r < uR;
      if (!valid) flags = 0;  // zero padding of a ragged last tile
      // destination row: the tile's first row plus this row's offset, plus
      // cap - n past a (batch, head) boundary
      int64_t dst;
      if (un > static_cast<uint32_t>(KT)) {   // at most one boundary within a tile
        const uint32_t rel = nb * KB + j;
        dst = dst0 + (rel + (rel >= wrap_at ? wrap_add : 0u));
      } else {
        const uint32_t off0 = toff + nb * KB + j;
        const uint32_t w = off0 / un;
        dst = static_cast<int64_t>(tbh + w) * cap + pos + (off0 - w * un);
      }

      // ---- flagged words: queued for the exact fix after the last tile, or
      // (queue full) fixed here, one (key, coordinate) pair at a time ----
      const uint64_t need = __ballot(flags != 0);
      bool deferred = false;
      if (need) {
        const int cnt = __popcll(need);
        if (qn + cnt > QCAP) {   // full: decide the queued words now
          flush(std::integral_constant<int, 1>{});
          qn = 0;
        }
        if (flags != 0) {
          const int slot = qn + static_cast<int>(__builtin_amdgcn_mbcnt_hi(
                                    static_cast<uint32_t>(need >> 32),
                                    __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(need), 0u)));
          fixq[wave][slot] = make_uint4(r | (static_cast<uint32_t>(half) << 31), word, flags, 0u);
          fixn[wave][slot] = knorm_up;
          deferred = true;
        }
        qn += cnt;
      }

      // ---- stores ----
      if (valid) {
        if (!deferred) signs[dst * WPR + (cb >> 5) + half] = word;
        // the norm of block nb's keys is stored by wave nb (spreads the work)
        if (wave == nb && half == 0) {
          // v_sqrt_f32: within 1 ulp of the square root
          float nrm = __builtin_amdgcn_sqrtf(n2);
          if (!(n2 >= 0x1.0p-100f && n2 <= 0x1.0p100f)) {
            nrm = scaled_norm(keys + static_cast<int64_t>(r) * D);
          }
          norms[dst] = nrm;
        }
      }
    };

#pragma unroll
    for (int nb = 0; nb < NBLK; ++nb) {
      if (nb + 1 < NBLK) {
        project(buf, nb + 1, nxt0, nxt1);
      } else if (more) {   // publish the next tile, start its first block
        stage(buf ^ 1);
        __syncthreads();
        if (tile + 2 * static_cast<int>(gridDim.x) < ntiles) load_tile(tile + 2 * gridDim.x);
#pragma unroll
        for (int k = 0; k < NBLK; ++k) n2n[k] = n2buf[buf ^ 1][k * KB + j];
        project(buf ^ 1, 0, nxt0, nxt1);
      }
      process(nb, cur0, cur1, n2r[nb]);
      cur0 = nxt0;
      cur1 = nxt1;
    }
#pragma unroll
    for (int k = 0; k < NBLK; ++k) n2r[k] = n2n[k];
    buf ^= 1;
  }

  if (qn > 0) flush(std::integral_constant<int, 4>{});
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
                     static_cast<const uint16_t*>(keys), s.s_md, s.s_efrag, s.col_norm_max, signs, norms, R,
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
