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
// Two kernels: a tile kernel for key sets of any size (one launch, or
// several for sets beyond about 16 tiles per workgroup), and a small-set
// kernel for calls of a few hundred keys at most (see encode_small_kernel).
//
// Tile kernel design:
// * The projection P^T = S^T K^T runs on the matrix cores
//   (v_mfma_f32_32x32x16_bf16, fp32 accumulate).  A workgroup has m/64
//   waves; wave w owns sketch coordinates [64w, 64w+64) and keeps its slice
//   of -S^T (64 x 128 bf16, 64 VGPRs) resident for the whole kernel.  The
//   slice is negated so that the sign bit of an accumulator is already the
//   stored bit (1 for a non-negative projection).
// * Keys stream through LDS in tiles of 128 rows, loaded with coalesced
//   16-byte buffer loads (rows past the end read as zero) and
//   double-buffered; the next tile's loads are in flight while the current
//   tile is multiplied.
// * The A-operand rows are permuted so that lane (key j, half h) ends up
//   holding coordinates 64w + 32h + 0..31 of key j in its 32 accumulators:
//   one word of packed bits per lane, assembled with v_alignbit (one
//   instruction per bit-lane), no cross-lane traffic.
// * ||k||^2 is summed (bf16 dot2, fp32) while a tile is staged into LDS.
// * Certification: an accumulator with |acc| <= tau, where tau bounds the
//   accumulation error of a d-term fp32 dot product of exact bf16 products
//   (with margin), is re-evaluated exactly: its word is queued and, after the
//   last tile, the wave sums the 128 fp64 products (exact) with a rigorous
//   error bound, falling back to an exact integer long accumulator when even
//   that is inconclusive.  The resulting bit is the sign of the exact real
//   sum, with sign(0) = +1.  A wave whose queue fills keeps going (later
//   words are stored as computed) and afterwards re-runs its tiles from the
//   first one it could not queue, deciding every flagged word there; keys
//   whose squared norm left the accurate fp32 range get their norms
//   recomputed the same way.  Neither path adds code to the tile loop.

#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>
#include <type_traits>

#include "exact_sign.h"
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
constexpr int QCAP = 112;            // deferred-fix queue entries per wave

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }
__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t v) { return __builtin_bit_cast(bf16x2_t, v); }

// DPP move of a float with every lane enabled and no old value (the
// compiler folds it into the consuming add)
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
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

// Buffer descriptor over [base, base + bytes): loads past the end return
// zero.  base and bytes must be wave-uniform.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;   // 32-bit data format, no swizzle
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           __builtin_amdgcn_readfirstlane(bytes), kRsrcWord3);
}

// Destination row of global key row r: (batch, head) = r / n, position
// pos + r % n in a cache of cap rows per (batch, head).
__device__ __forceinline__ int64_t dest_row(uint32_t r, uint32_t un, int cap, int pos) {
  const uint32_t bh = r / un;
  return static_cast<int64_t>(bh) * cap + pos + (r - bh * un);
}

// Exact-sign evaluation of queued sign words (the words whose flagged bits
// the fp32 projection could not certify).  Four lanes serve one entry: lane
// (group g, sub c) loads 16-byte chunks c, 4 + c, 8 + c, 12 + c (32
// channels) of the key row and of the sketch row of the entry's lowest
// flagged coordinate, so one pass decides one flagged bit of sixteen entries
// and each load instruction reads 64 contiguous bytes per quad.  The 32
// products of a lane are exact in fp64 and accumulated by fma (one rounding
// each), then quad_sum_f64 adds the four lanes: at most 34 roundings, each
// within 2^-53 of sum|p|, so the error is below 2^-47 * bnd for any
// bnd >= sum|p| (such as ||k|| max_i ||s_i||, Cauchy-Schwarz).  The bit is
// the sign of the sum when |sum| > 2^-46 * bnd; the rare sums below that
// go, one at a time, to the exact integer accumulator.  fq/fk: the queue
// ({key row | half << 31, word, flags, -}, norm bound); the decided words
// are stored to their rows.
__device__ __forceinline__ void fix_queue(const uint4* fq, const float* fk, int qn, const uint16_t* keys,
                                          const uint16_t* s_md, int cb, float smax, uint32_t* signs,
                                          uint32_t un, int cap, int pos, int wpr, uint32_t* scratch,
                                          int lane, uint32_t r0) {
  const int g = lane >> 2, sub = lane & 3;
  const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
  for (int base = 0; base < qn; base += 16) {
    const int e = base + g;
    const bool act = e < qn;
    const uint4 ent = act ? fq[e] : zero;
    const uint32_t row = ent.x & 0x7FFFFFFFu;
    const int hf = static_cast<int>(ent.x >> 31);
    uint32_t word = ent.y, fl = ent.z, slow = 0;   // fl is zero for inactive entries
    const double bnd = act ? static_cast<double>(fk[e]) * smax : 0.0;
    int p = fl ? __builtin_ctz(fl) : 0;
    // unconditional 16-byte loads (an inactive entry reads key row 0 and
    // sketch row cb, both in bounds, and decides nothing)
    const uint4* krow = reinterpret_cast<const uint4*>(keys + static_cast<int64_t>(row) * D);
    uint4 kc[4], sc[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) kc[u] = krow[4 * u + sub];
    auto load_s = [&]() {
      const uint4* srow = reinterpret_cast<const uint4*>(s_md + static_cast<int64_t>(cb + 32 * hf + p) * D);
#pragma unroll
      for (int u = 0; u < 4; ++u) sc[u] = srow[4 * u + sub];
    };
    load_s();
    // an all (+/-) zero key projects to exactly 0: bit 1
    uint32_t nz = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) nz |= kc[u].x | kc[u].y | kc[u].z | kc[u].w;
    if (quad_or(nz & 0x7FFF7FFFu) == 0) {
      word |= fl;
      fl = 0;
    }
    for (;;) {
      if (__ballot(fl != 0) == 0) break;
      if (fl != 0) {   // uniform over the entry's four lanes
        double acc = 0.0;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint32_t kw[4] = {kc[u].x, kc[u].y, kc[u].z, kc[u].w};
          const uint32_t sw[4] = {sc[u].x, sc[u].y, sc[u].z, sc[u].w};
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            acc = __builtin_fma(bf16_lo_f64(kw[t]), bf16_lo_f64(sw[t]), acc);
            acc = __builtin_fma(bf16_hi_f64(kw[t]), bf16_hi_f64(sw[t]), acc);
          }
        }
        const double sum = quad_sum_f64(acc);
        double b = bnd;
        if (!(b < INFINITY)) {   // the key norm left fp32: bound by sum|p| itself
          double mag = 0.0;
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const uint32_t kw[4] = {kc[u].x, kc[u].y, kc[u].z, kc[u].w};
            const uint32_t sw[4] = {sc[u].x, sc[u].y, sc[u].z, sc[u].w};
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              mag += __builtin_fabs(bf16_lo_f64(kw[t]) * bf16_lo_f64(sw[t]));
              mag += __builtin_fabs(bf16_hi_f64(kw[t]) * bf16_hi_f64(sw[t]));
            }
          }
          b = quad_sum_f64(mag) * (1.0 + 0x1.0p-40);
        }
        const uint32_t mbit = 1u << p;
        if (__builtin_fabs(sum) > 0x1.0p-46 * b) word = sum > 0.0 ? (word | mbit) : (word & ~mbit);
        else slow |= mbit;
        fl &= fl - 1;
        if (fl) {   // next flagged coordinate of this entry
          p = __builtin_ctz(fl);
          load_s();
        }
      }
    }
    // exact integer sums, one (key, coordinate) at a time on lane 0
    for (uint64_t heads = __ballot(sub == 0 && slow != 0); heads; heads &= heads - 1) {
      const int src = __builtin_ctzll(heads);
      uint32_t bits = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(slow), src));
      const uint32_t rsrc = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(row), src));
      const int hsrc = __builtin_amdgcn_readlane(hf, src);
      while (bits) {
        const int q = __builtin_ctz(bits);
        bits &= bits - 1;
        bool bit = false;
        if (lane == 0)
          bit = exact_sign_long(keys + static_cast<int64_t>(rsrc) * D,
                                s_md + static_cast<int64_t>(cb + 32 * hsrc + q) * D, scratch);
        bit = __builtin_amdgcn_readfirstlane(static_cast<int>(bit)) != 0;
        if ((lane >> 2) == (src >> 2)) word = bit ? (word | (1u << q)) : (word & ~(1u << q));
      }
    }
    if (sub == 0 && act) signs[dest_row(r0 + row, un, cap, pos) * wpr + (cb >> 5) + hf] = word;
  }
}

// ALIGNED: n is a multiple of the 128-key tile, so every tile is full and
// lies within one (batch, head).
template <int M, bool ALIGNED>
__global__ __launch_bounds__(64 * (M / CW)) __attribute__((amdgpu_waves_per_eu(2))) void encode_kernel(
    const uint16_t* __restrict__ keys, const uint16_t* __restrict__ s_md,
    const uint16_t* __restrict__ s_efrag, const float* __restrict__ col_norm_max, uint32_t* __restrict__ signs,
    float* __restrict__ norms, int R, int n, int cap, int pos, int ntiles, int ga, int ta, float c1,
    float c2, int r0_) {
  constexpr int W = M / CW;
  constexpr int NT = 64 * W;
  constexpr int LOADS = CHUNKS / NT;  // 16-byte loads per thread per tile
  constexpr int WPR = M / 32;         // words per key row
  static_assert(NT % 16 == 0, "the 16 chunks of a key row must sit in one 16-lane row");

  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * TILE_LDS];
  __shared__ float n2buf[2][KT];   // squared key norms of the tile
  __shared__ float n2sink[W][64];  // written by lanes that own no norm (no branch)
  __shared__ uint32_t long_scratch[W][2 * ACC_WORDS];
  // Sign words with bits to certify, queued per wave for an exact fix after
  // the last tile: {key row | half << 31, word, flags, 0}.
  __shared__ uint4 fixq[W][QCAP];
  __shared__ float fixn[W][QCAP];   // upper bound of ||k|| of the entry's key
  int qn = 0;              // queued entries of this wave (uniform)
  int ovf = INT_MAX;       // first tile with a flagged word the queue had no room for (uniform)
  bool odd_norm = false;   // some key of this wave's norm blocks left the accurate range (uniform)

  // Tiles of this workgroup: workgroups [0, ga) share tiles [0, ta) and the
  // rest share [ta, ntiles), each group round-robin.  (The host gives the
  // first workgroup of each CU, whose waves are older and win issue, a
  // larger share.)
  const int grp_a = static_cast<int>(blockIdx.x) < ga;
  const int t_first = grp_a ? static_cast<int>(blockIdx.x) : ta + static_cast<int>(blockIdx.x) - ga;
  const int t_step = grp_a ? ga : static_cast<int>(gridDim.x) - ga;
  const int t_end = grp_a ? ta : ntiles;
  if (t_first >= t_end) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int j = lane & 31;
  const int cb = wave * CW;
  const uint32_t un = static_cast<uint32_t>(n);
  const uint32_t uR = static_cast<uint32_t>(R);
  // keys and rows are local to this launch; r0 is the global row of local
  // row 0 (destination rows are computed from global rows)
  const uint32_t r0 = static_cast<uint32_t>(r0_);

  bf16x8_t a[2][8];   // loaded after the first tile's requests (see below)
  const float smax = col_norm_max[wave];
  const float c1s = c1 * smax;   // tau = c1s * ||k||_up + c2

  uint4 pf[LOADS];   // 16-byte key chunks in flight (rows past the end read as zero)
  // Part p of a tile is block p (rows 32p .. 32p+31, 512 chunks of 16
  // bytes).  A thread holds CPT chunks of one row: L = 16 / CPT consecutive
  // lanes cover a row, lane i its chunks i, i + L, ...  Each group of L lanes
  // reads whole 128-byte lines, and a key's squared norm needs a sum over L
  // lanes only.
  constexpr int LPB = LOADS / NBLK;   // chunks staged (and reloaded) per block
  constexpr int CPT = LPB;            // chunks per thread per row
  constexpr int L = 16 / CPT;         // lanes per row
  static_assert(LOADS % NBLK == 0 && (L == 8 || L == 16), "unsupported chunk split");
  const int prow = tid / L;           // row within the block
  const int pcol = tid % L;           // first chunk
  // (a tile past the end gets an empty descriptor: its loads return zeros
  // and touch no memory, so every load in the loop is unconditional and the
  // compiler's wait counts stay exact)
  auto load_part = [&](int tile, int part) {
    const uint32_t tb = static_cast<uint32_t>(tile) * KT;
    const uint32_t rows = tile < t_end ? (ALIGNED ? static_cast<uint32_t>(KT) : min(uR - tb, static_cast<uint32_t>(KT))) : 0u;
    const rsrc_t rs = make_rsrc(keys + static_cast<int64_t>(tb) * D, static_cast<int>(rows) * ROW_B);
#pragma unroll
    for (int i = 0; i < CPT; ++i)
      pf[part * CPT + i] = __builtin_bit_cast(
          uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, (part * KB + prow) * ROW_B + (pcol + L * i) * 16, 0, 0));
  };

  // staged chunks -> LDS tile bb, and their keys' squared norms ->
  // n2buf[bb]: each thread squares its chunks (bf16 dot2, fp32), then a DPP
  // all-reduce over the row's L lanes (pairs xor 1, xor 2, then the mirror
  // within 8 lanes, then within 16)
  auto stage_part = [&](int bb, int part) {
    uint8_t* t = lds + bb * TILE_LDS + (part * KB + prow) * LDS_ROW;
    float q = 0.f;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const uint4 v = pf[part * CPT + i];
      q = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(v.x), as_bf16x2(v.x), q, false);
      q = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(v.y), as_bf16x2(v.y), q, false);
      q = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(v.z), as_bf16x2(v.z), q, false);
      q = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(v.w), as_bf16x2(v.w), q, false);
      *reinterpret_cast<uint4*>(t + (pcol + L * i) * 16) = v;
    }
    q += dpp_f32<0xB1>(q);    // quad_perm [1, 0, 3, 2]
    q += dpp_f32<0x4E>(q);    // quad_perm [2, 3, 0, 1]
    q += dpp_f32<0x141>(q);   // row_half_mirror
    if constexpr (L == 16) q += dpp_f32<0x140>(q);   // row_mirror
    *(pcol == 0 ? &n2buf[bb][part * KB + prow] : &n2sink[wave][lane]) = q;
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

  // certification threshold of a key from its fp32 squared norm:
  // ||k|| <= sqrt(n2 (1 + 2^-14) + 2^-119) covers the fp32 rounding of 128
  // exact squares and squares lost below the fp32 normal range (with
  // margin); v_sqrt_f32 is within 1 ulp, which the factor 1 + 2^-20 keeps.
  auto norm_bound = [&](float n2) {
    return __builtin_amdgcn_sqrtf(__builtin_fmaf(n2, 1.0f + 0x1.0p-14f, 0x1.0p-118f)) * (1.0f + 0x1.0p-20f);
  };
  // sign word of a lane, highest coordinate shifted in first (acc1 gives
  // bits 16..31, acc0 bits 0..15); with -S the sign bit is the stored bit
  auto sign_word = [](const f32x16_t& acc0, const f32x16_t& acc1) {
    uint32_t sw = 0;
#pragma unroll
    for (int r = 15; r >= 0; --r) sw = __builtin_amdgcn_alignbit(sw, __float_as_uint(acc1[r]), 31);
#pragma unroll
    for (int r = 15; r >= 0; --r) sw = __builtin_amdgcn_alignbit(sw, __float_as_uint(acc0[r]), 31);
    return sw;
  };

  // Software pipeline: the next block's matrix products (across tile
  // boundaries too) are issued before this block's bit extraction, so they
  // run while it executes.  Tiles alternate between two LDS buffers: while
  // tile t is multiplied, block nb stages a quarter of tile t+1 (loaded
  // during tile t-1) into the other buffer and reloads those registers with
  // the same quarter of tile t+2; the barrier in block 3 publishes tile t+1.
  // That buffer's previous tile (t-1) was last read before the barrier that
  // published tile t, and so were its norms.
  int buf = 0;
  f32x16_t cur0, cur1, nxt0, nxt1;   // accumulators of this block and the next
  float n2r[NBLK];
#pragma unroll
  for (int p = 0; p < NBLK; ++p) load_part(t_first, p);
  // (the first tile's memory requests go out before the L2-resident
  // sketch fragments)
  // Resident A operand: -S^T rows for this wave's coordinates.  Block b, row
  // i holds coordinate cb + 32*((i >> 2) & 1) + 16*b + 4*(i >> 3) + (i & 3),
  // so the 32x32 result places coordinate cb + 32*half + 16*b + r in
  // register r of lane (j, half).
  // (s_efrag holds these fragments in lane order: one 1 KB load each)
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const uint4* fr = reinterpret_cast<const uint4*>(s_efrag) + (static_cast<int64_t>(wave) * 2 + b) * 8 * 64 + lane;
#pragma unroll
    for (int s = 0; s < 8; ++s) a[b][s] = as_bf16x8(fr[s * 64]);
  }
#pragma unroll
  for (int p = 0; p < NBLK; ++p) stage_part(0, p);
  __syncthreads();
#pragma unroll
  for (int p = 0; p < NBLK; ++p) load_part(t_first + t_step, p);
#pragma unroll
  for (int k = 0; k < NBLK; ++k) n2r[k] = n2buf[0][k * KB + j];
  project(0, 0, cur0, cur1);
  // Every value loaded before the loop is consumed here, so no wait for
  // them lands inside the loop (where it would also wait for the prefetched
  // tile and the stores).
  asm volatile("" ::"s"(c1s));
  // One tile; the last one (LAST) stages and prefetches nothing.
  auto tile_step = [&](int tile, auto last_c) {
    constexpr bool LAST = decltype(last_c)::value;
    // per-tile geometry (uniform; the host keeps the key count below 2^31)
    const uint32_t tb = static_cast<uint32_t>(tile) * KT;
    const uint32_t rows = ALIGNED ? static_cast<uint32_t>(KT) : min(uR - tb, static_cast<uint32_t>(KT));
    const uint32_t tbh = (r0 + tb) / un;
    const uint32_t toff = r0 + tb - tbh * un;
    const bool straddle = !ALIGNED && toff + rows > un;   // rows of more than one (batch, head)
    const int64_t dst0 = static_cast<int64_t>(tbh) * cap + pos + toff;   // row tb's destination
    uint32_t* const sg_tile = signs + dst0 * WPR + (cb >> 5);
    float* const nm_tile = norms + dst0;
    float n2n[NBLK];
    // Words of blocks 0..2 wait in registers and are stored right after the
    // barrier in block 3: no store then sits between the prefetched tile's
    // loads and the wait for them (the memory counter retires in order).
    uint32_t wbuf[NBLK - 1];
    uint32_t okbits = 0;   // bit nb: store block nb's word; bit NBLK: store nbuf
    float nbuf = 0.f;      // norm of this lane's key in block `wave`
    // destination row of tile row rel when the tile straddles a (batch, head)
    // boundary: the tile's first row plus rel, plus cap - n past each boundary
    auto dst_straddle = [&](uint32_t rel) -> int64_t {
      if (un > static_cast<uint32_t>(KT))   // at most one boundary within a tile
        return dst0 + (rel + (rel >= un - toff ? static_cast<uint32_t>(cap) - un : 0u));
      return dest_row(r0 + tb + rel, un, cap, pos);
    };
    auto store_word = [&](uint32_t rel, uint32_t word) {
      if (!straddle) sg_tile[rel * WPR + half] = word;
      else signs[dst_straddle(rel) * WPR + (cb >> 5) + half] = word;
    };
    auto store_norm = [&](uint32_t rel, float nrm) {
      if (!straddle) nm_tile[rel] = nrm;
      else norms[dst_straddle(rel)] = nrm;
    };
    auto flush_stores = [&]() {
#pragma unroll
      for (int nb = 0; nb < NBLK - 1; ++nb)
        if (okbits & (1u << nb)) store_word(nb * KB + j, wbuf[nb]);
      if (okbits & (1u << NBLK)) store_norm(wave * KB + j, nbuf);
    };

    // ---- bits of one block: signs, certification, stores ----
    auto process = [&](int nb, const f32x16_t& acc0, const f32x16_t& acc1, float n2) {
      const float knorm_up = norm_bound(n2);
      const float tau = __builtin_fmaf(c1s, knorm_up, c2);
      uint32_t word = sign_word(acc0, acc1);
      // An all-(+/-)zero key projects to exactly 0, every bit 1: found through
      // n2 == 0 and a look at its row in LDS (rare), so padding rows never
      // reach the exact fix.
      bool zero_key = false;
      if (__ballot(n2 == 0.f) != 0) {
        const uint4* zr = reinterpret_cast<const uint4*>(lds + buf * TILE_LDS + (nb * KB + j) * LDS_ROW + 128 * half);
        uint32_t o = 0;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const uint4 v = zr[c];
          o |= v.x | v.y | v.z | v.w;
        }
        o &= 0x7FFF7FFFu;
        o |= __shfl_xor(o, 32);   // the other half of the row
        zero_key = n2 == 0.f && o == 0;
        if (zero_key) word = 0xFFFFFFFFu;
      }
      float amin1 = __builtin_fabsf(acc1[0]);
      float amin0 = __builtin_fabsf(acc0[0]);
#pragma unroll
      for (int r = 1; r < 16; ++r) {
        amin1 = fminf(amin1, __builtin_fabsf(acc1[r]));
        amin0 = fminf(amin0, __builtin_fabsf(acc0[r]));
      }
      // ---- a word with some |acc| <= tau (or a key whose fp32 norm left
      // the range the bound is proved for) is queued for the exact fix after
      // the last tile, which finds its flagged bits; with the queue full it
      // is stored as computed and the tile is re-run afterwards ----
      const uint32_t rel = nb * KB + j;   // row within the tile
      const bool valid = ALIGNED || rel < rows;   // (zero padding of a ragged last tile)
      const bool huge = !(n2 < 0x1.0p100f);
      const uint64_t need = __ballot(valid && !zero_key && (fminf(amin1, amin0) <= tau || huge));
      bool deferred = false;
      if (need) {
        const int cnt = __popcll(need);
        if ((need >> lane) & 1) {
          const int slot = qn + static_cast<int>(__builtin_amdgcn_mbcnt_hi(
                                    static_cast<uint32_t>(need >> 32),
                                    __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(need), 0u)));
          if (slot < QCAP) {
            // flags: all bits for a huge key, else found after the loop
            fixq[wave][slot] = make_uint4((tb + rel) | (static_cast<uint32_t>(half) << 31), word,
                                          huge ? 0xFFFFFFFFu : 0u, 0u);
            fixn[wave][slot] = knorm_up;
            deferred = true;
          }
        }
        if (qn + cnt > QCAP) {
          if (ovf == INT_MAX) ovf = tile;
          qn = QCAP;
        } else {
          qn += cnt;
        }
      }

      // ---- stores; the norms of block nb's keys are stored by wave nb ----
      const bool norm_lane = wave == nb && half == 0;
      // v_sqrt_f32: within 1 ulp of the square root where n2 is accurate;
      // keys outside that range are redone after the tile loop
      const float nrm = __builtin_amdgcn_sqrtf(n2);
      if (wave == nb) {
        if (__ballot(half == 0 && valid && !zero_key && !(n2 >= 0x1.0p-100f && n2 <= 0x1.0p100f)) != 0)
          odd_norm = true;
      }
      if (nb < NBLK - 1) {
        wbuf[nb] = word;
        if (valid && !deferred) okbits |= 1u << nb;
        if (norm_lane && valid) {
          nbuf = nrm;
          okbits |= 1u << NBLK;
        }
      } else if (valid) {
        if (!deferred) store_word(rel, word);
        if (norm_lane) store_norm(rel, nrm);
      }
    };

    constexpr bool more = !LAST;
#pragma unroll
    for (int nb = 0; nb < NBLK; ++nb) {
      if (nb + 1 < NBLK) project(buf, nb + 1, nxt0, nxt1);
      if constexpr (more) {
        stage_part(buf ^ 1, nb);
        load_part(tile + 2 * t_step, nb);   // (past the range: an empty descriptor)
      }
      if (nb + 1 == NBLK) {
        if constexpr (more) {   // publish the next tile, start its first block
          __syncthreads();
          flush_stores();
#pragma unroll
          for (int k = 0; k < NBLK; ++k) n2n[k] = n2buf[buf ^ 1][k * KB + j];
          project(buf ^ 1, 0, nxt0, nxt1);
        } else {
          flush_stores();
        }
      }
      process(nb, cur0, cur1, n2r[nb]);
      cur0 = nxt0;
      cur1 = nxt1;
    }
    if constexpr (more) {
#pragma unroll
      for (int k = 0; k < NBLK; ++k) n2r[k] = n2n[k];
      buf ^= 1;
    }
  };
  int tile = t_first;
  for (; tile + t_step < t_end; tile += t_step) tile_step(tile, std::false_type{});
  // The last tile needs no staging, so its registers carry the re-
  // multiplication's first 32 keys (queued so far): their loads run while
  // the tile is multiplied.  Keys queued during the last tile are read from
  // its LDS buffer afterwards.
  const int qn_pre = qn;
  const uint32_t tb_last = static_cast<uint32_t>(tile) * KT;
  uint4 fb[8];
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");   // queue entries of other lanes
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  {
    const uint4 ent = fixq[wave][j < qn_pre ? j : 0];
    const uint32_t row = j < qn_pre ? (ent.x & 0x7FFFFFFFu) : 0u;   // row 0: in bounds, unused
    const uint4* krow = reinterpret_cast<const uint4*>(keys + static_cast<int64_t>(row) * D);
#pragma unroll
    for (int s = 0; s < 8; ++s) fb[s] = krow[2 * s + half];
  }
  tile_step(tile, std::true_type{});

  // ---- after the tile loop: queued words, overflowed tiles, odd norms ----
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  if (qn > 0) {
    // Flagged bits of the queued words: the queued keys are multiplied again
    // (entry e in column e % 32), and the word and its flags are taken from
    // these products, so nothing depends on the loop's column order.
    for (int e0 = 0; e0 < qn; e0 += 32) {
      const int e = e0 + j;
      const bool act = e < qn;
      const uint4 ent = fixq[wave][act ? e : 0];
      const uint32_t row = ent.x & 0x7FFFFFFFu;
      f32x16_t acc0 = f32x16_t{}, acc1 = f32x16_t{};
      if (e0 == 0) {   // prefetched keys, or the last tile's rows in LDS
        const bool in_lds = e >= qn_pre;
        const uint32_t rel = in_lds && act ? row - tb_last : 0u;
        const uint8_t* lrow = lds + buf * TILE_LDS + rel * LDS_ROW + 16 * half;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const uint4 l = *reinterpret_cast<const uint4*>(lrow + 32 * s);
          const bf16x8_t v = as_bf16x8(in_lds ? l : fb[s]);
          acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0][s], v, acc0, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1][s], v, acc1, 0, 0, 0);
        }
      } else {
        const uint4* krow = reinterpret_cast<const uint4*>(keys + static_cast<int64_t>(row) * D);
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const bf16x8_t v = as_bf16x8(krow[2 * s + half]);
          acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0][s], v, acc0, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1][s], v, acc1, 0, 0, 0);
        }
      }
      if (act && static_cast<int>(ent.x >> 31) == half) {
        const float tau = __builtin_fmaf(c1s, fixn[wave][e], c2);
        uint32_t nf = 0;   // set bit: |acc| > tau (certified)
#pragma unroll
        for (int r = 15; r >= 0; --r) nf = __builtin_amdgcn_alignbit(nf, __float_as_uint(tau - __builtin_fabsf(acc1[r])), 31);
#pragma unroll
        for (int r = 15; r >= 0; --r) nf = __builtin_amdgcn_alignbit(nf, __float_as_uint(tau - __builtin_fabsf(acc0[r])), 31);
        fixq[wave][e].y = sign_word(acc0, acc1);
        fixq[wave][e].z |= ~nf;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    fix_queue(fixq[wave], fixn[wave], qn, keys, s_md, cb, smax, signs, un, cap, pos, WPR, long_scratch[wave], lane, r0);
  }
  if (ovf != INT_MAX) {
    // Re-run of this wave's tiles from the first one whose flagged words did
    // not all fit: the same products from B fragments read straight from
    // memory, every word stored again (certified as computed, or queued and
    // decided exactly batch by batch).
    qn = 0;
    for (int tile = ovf; tile < t_end; tile += t_step) {
      const uint32_t tb = static_cast<uint32_t>(tile) * KT;
      const uint32_t rows = min(uR - tb, static_cast<uint32_t>(KT));
      for (int nb = 0; nb < NBLK; ++nb) {
        const uint32_t rel = nb * KB + j;
        const bool valid = rel < rows;
        // rows past the end read row tb (in bounds) and are never stored
        const uint4* krow = reinterpret_cast<const uint4*>(keys + static_cast<int64_t>(valid ? tb + rel : tb) * D);
        float n2 = 0.f;
        f32x16_t acc0 = f32x16_t{}, acc1 = f32x16_t{};
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const uint4 v = krow[2 * s + half];
          n2 = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(v.x), as_bf16x2(v.x), n2, false);
          n2 = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(v.y), as_bf16x2(v.y), n2, false);
          n2 = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(v.z), as_bf16x2(v.z), n2, false);
          n2 = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(v.w), as_bf16x2(v.w), n2, false);
          acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0][s], as_bf16x8(v), acc0, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1][s], as_bf16x8(v), acc1, 0, 0, 0);
        }
        n2 += __shfl_xor(n2, 32);   // the other half of the key's channels
        const float knorm_up = norm_bound(n2);
        const float tau = __builtin_fmaf(c1s, knorm_up, c2);
        const uint32_t word = sign_word(acc0, acc1);
        uint32_t nf = 0;   // set bit: |acc| > tau (certified)
#pragma unroll
        for (int r = 15; r >= 0; --r) nf = __builtin_amdgcn_alignbit(nf, __float_as_uint(tau - __builtin_fabsf(acc1[r])), 31);
#pragma unroll
        for (int r = 15; r >= 0; --r) nf = __builtin_amdgcn_alignbit(nf, __float_as_uint(tau - __builtin_fabsf(acc0[r])), 31);
        uint32_t fl = ~nf;
        if (!(n2 < 0x1.0p100f)) fl = 0xFFFFFFFFu;
        if (!valid) fl = 0;
        if (valid && fl == 0) signs[dest_row(r0 + tb + rel, un, cap, pos) * WPR + (cb >> 5) + half] = word;
        const uint64_t need = __ballot(fl != 0);
        if (need) {
          if (fl != 0) {
            const int slot = qn + static_cast<int>(__builtin_amdgcn_mbcnt_hi(
                                      static_cast<uint32_t>(need >> 32),
                                      __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(need), 0u)));
            fixq[wave][slot] = make_uint4((tb + rel) | (static_cast<uint32_t>(half) << 31), word, fl, 0u);
            fixn[wave][slot] = knorm_up;
          }
          qn += __popcll(need);
          if (qn > QCAP - 64) {   // no room for another block's words: decide these now
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            fix_queue(fixq[wave], fixn[wave], qn, keys, s_md, cb, smax, signs, un, cap, pos, WPR,
                      long_scratch[wave], lane, r0);
            qn = 0;
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
          }
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (qn > 0) fix_queue(fixq[wave], fixn[wave], qn, keys, s_md, cb, smax, signs, un, cap, pos, WPR,
                          long_scratch[wave], lane, r0);
  }
  if (odd_norm) {
    // norms of this wave's blocks (nb == wave), one lane per key, with the
    // scaled evaluation where the fp32 sum of squares is inaccurate
    for (int tile = t_first; tile < t_end; tile += t_step) {
      const uint32_t tb = static_cast<uint32_t>(tile) * KT;
      const uint32_t rows = min(uR - tb, static_cast<uint32_t>(KT));
      const uint32_t rel = wave * KB + j;
      if (half == 0 && rel < rows) {
        const uint16_t* key = keys + static_cast<int64_t>(tb + rel) * D;
        const uint4* kr = reinterpret_cast<const uint4*>(key);
        float n2 = 0.f;
        for (int c = 0; c < 16; ++c) {
          const uint4 v = kr[c];
          n2 = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(v.x), as_bf16x2(v.x), n2, false);
          n2 = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(v.y), as_bf16x2(v.y), n2, false);
          n2 = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(v.z), as_bf16x2(v.z), n2, false);
          n2 = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(v.w), as_bf16x2(v.w), n2, false);
        }
        float nrm = __builtin_amdgcn_sqrtf(n2);
        if (!(n2 >= 0x1.0p-100f && n2 <= 0x1.0p100f)) nrm = scaled_norm(key);
        norms[dest_row(r0 + tb + rel, un, cap, pos)] = nrm;
      }
    }
  }
}

// Resident workgroups of encode_kernel<M, ALIGNED> per CU and on the device
// (fixed per template and device model; queried once).
template <int M, bool ALIGNED>
int encode_occupancy(int* max_grid_out, int* wg_per_cu_out) {
  constexpr int NT = 64 * (M / CW);
  static int max_grid = 0;
  static int wg_per_cu = 0;
  if (max_grid == 0) {
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return hipErrorInvalidDevice;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return hipErrorInvalidDevice;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, encode_kernel<M, ALIGNED>, NT, 0) !=
        hipSuccess)
      return hipErrorInvalidDeviceFunction;
    wg_per_cu = per_cu > 0 ? per_cu : 1;
    max_grid = cus * wg_per_cu;
  }
  *max_grid_out = max_grid;
  *wg_per_cu_out = wg_per_cu;
  return hipSuccess;
}

// One launch over local rows [0, R) of keys, whose global row 0 is r0.
template <int M, bool ALIGNED>
int launch_encode_mt(const void* keys, int R, int r0, const DeviceSketch& s, int n, uint32_t* signs,
                     float* norms, int cap, int pos, int max_grid, int wg_per_cu, hipStream_t stream) {
  constexpr int NT = 64 * (M / CW);
  const int ntiles = static_cast<int>((static_cast<int64_t>(R) + KT - 1) / KT);
  const int grid = ntiles < max_grid ? ntiles : max_grid;
  // Two workgroups per CU: the one dispatched first (index below grid/2)
  // keeps the older waves, which win instruction issue; its first tile
  // arrives ~3 us earlier and it runs a tile 10-15% faster (measured with
  // in-kernel timestamps).  With 8 or more tiles per pair of workgroups it
  // takes one tile more than half, which measured best at 8, 16 and 32
  // tiles per pair (an even split stays best at 4).
  int ga = grid, ta = ntiles;
  if (wg_per_cu == 2 && grid == max_grid && ntiles >= 8 * (grid / 2)) {
    ga = grid / 2;
    const int n_pair = ntiles / ga;   // whole tiles per pair of workgroups
    ta = (n_pair / 2 + 1) * ga;
    if (ta > ntiles - (grid - ga)) ta = ntiles - (grid - ga);
  }
  // Error bound of an fp32 sum of D exact products, with a factor 4 margin
  // over round-to-nearest (covers truncating or blocked accumulation).
  const float c1 = static_cast<float>(4.0 * D * 0x1.0p-24 * (1.0 + 0x1.0p-10));
  const float c2 = 0x1.0p-110f;  // absolute floor: subnormal flushes
  hipLaunchKernelGGL((encode_kernel<M, ALIGNED>), dim3(grid), dim3(NT), 0, stream,
                     static_cast<const uint16_t*>(keys), s.s_md, s.s_efrag, s.col_norm_max, signs, norms, R,
                     n, cap, pos, ntiles, ga, ta, c1, c2, r0);
  return hipGetLastError();
}

// Keys are encoded in launches of about kMaxTilesPerWg tiles per workgroup:
// a wave then queues ~43 words on average (one in ~100 words needs the exact
// fix), far below its QCAP-entry queue, whose overflow path (re-running the
// wave's tiles) is slow.  A launch may take up to 1/8 more, so that a small
// remainder (65537 tokens per head, say) does not need a launch of its own,
// which would cost a whole prologue and end phase for a few keys; larger key
// sets are divided evenly, in whole tiles, among the fewest launches.  At
// m = 256 on 256 compute units one launch covers up to 9 * 2^17 keys.
constexpr int kMaxTilesPerWg = 16;

template <int M, bool ALIGNED>
int launch_encode_chunks(const DeviceSketch& s, const void* keys, int R, int n, uint32_t* signs,
                         float* norms, int cap, int pos, hipStream_t stream) {
  int max_grid = 0, wg_per_cu = 0;
  const int e = encode_occupancy<M, ALIGNED>(&max_grid, &wg_per_cu);
  if (e != hipSuccess) return e;
  const int64_t tiles = (static_cast<int64_t>(R) + KT - 1) / KT;
  const int64_t cap_tiles = static_cast<int64_t>(kMaxTilesPerWg) * max_grid * 9 / 8;
  const int64_t launches = (tiles + cap_tiles - 1) / cap_tiles;
  const int64_t chunk = (tiles + launches - 1) / launches * KT;   // a multiple of KT
  for (int64_t r0 = 0; r0 < R; r0 += chunk) {
    const int rows = static_cast<int>(R - r0 < chunk ? R - r0 : chunk);
    const int err = launch_encode_mt<M, ALIGNED>(static_cast<const uint16_t*>(keys) + r0 * D, rows,
                                                 static_cast<int>(r0), s, n, signs, norms, cap, pos,
                                                 max_grid, wg_per_cu, stream);
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

// ---- small key sets: four lanes per (key, sketch coordinate) ----
// For a handful of keys (a decode step appends one per kv head) the tile
// kernel's fixed costs (a workgroup's resident S^T operand, a whole tile, the
// deferred-fix phase) dominate.  Here a 256-thread workgroup takes one key
// and 64 coordinates; the four lanes of a quad share a coordinate, each
// multiplying 32 of the 128 channels (16-byte chunks sub, sub + 4, sub + 8,
// sub + 12 of the key row, staged once in LDS as fp64, and of the S^T row)
// in fp64, and a quad sum joins them (the same value in all four lanes).
// Every bf16 x bf16 product is exact in fp64 and a sum takes at most 34
// roundings on any path, so it lies within 2^-47 ||k|| max_i ||s_i|| of the
// exact value: a projection beyond 2^-45 ||k|| max_i ||s_i|| decides its
// sign, and the rest (none in practice) go to the exact integer evaluation,
// one at a time.  All-zero keys take all-ones words.  The norm is fp32 of the
// fp64 square root of the fp64 sum of squares.
template <int M>
__global__ __launch_bounds__(256) void encode_small_kernel(
    const uint16_t* __restrict__ keys, const uint16_t* __restrict__ s_md, float cnmax,
    uint32_t* __restrict__ signs, float* __restrict__ norms, int n, int cap, int pos) {
  constexpr int WPR = M / 32;
  constexpr int BPK = M / 64;              // workgroups per key
  __shared__ double kf[D];
  __shared__ double ksq_part[2];
  __shared__ uint32_t long_scratch[4][2 * ACC_WORDS];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int sub = lane & 3;
  const uint32_t r = blockIdx.x / BPK;                                  // key
  const int cbase = static_cast<int>(blockIdx.x % BPK) * 64;            // first coordinate
  const int i = cbase + (tid >> 2);                                     // this quad's coordinate
  const uint16_t* krow = keys + static_cast<int64_t>(r) * D;
  if (tid < D) {
    const double v = static_cast<double>(__uint_as_float(static_cast<uint32_t>(krow[tid]) << 16));
    kf[tid] = v;
    // squares of bf16 values are exact in fp64; two waves reduce 64 each
    double q = v * v;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) q += __shfl_xor(q, o);
    if (lane == 0) ksq_part[wave] = q;
  }
  // chunks sub, sub + 4, sub + 8, sub + 12 of the S^T row, requested while
  // the key is staged
  const uint4* srow = reinterpret_cast<const uint4*>(s_md + static_cast<int64_t>(i) * D);
  uint4 sv[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) sv[u] = srow[4 * u + sub];
  __syncthreads();
  const double ksq = ksq_part[0] + ksq_part[1];
  double part[2] = {0.0, 0.0};
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int c0 = 8 * (4 * u + sub);
    const uint32_t w[4] = {sv[u].x, sv[u].y, sv[u].z, sv[u].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      part[e & 1] = __builtin_fma(kf[c0 + 2 * e], bf16_lo_f64(w[e]), part[e & 1]);
      part[e & 1] = __builtin_fma(kf[c0 + 2 * e + 1], bf16_hi_f64(w[e]), part[e & 1]);
    }
  }
  const double acc = quad_sum_f64(part[0] + part[1]);
  const double knorm = __builtin_sqrt(ksq);
  const double thr = 0x1.0p-45 * knorm * static_cast<double>(cnmax);
  bool bit = acc >= 0.0;
  const bool decided = ksq == 0.0 || __builtin_fabs(acc) > thr;
  if (ksq == 0.0) bit = true;   // all-(+/-)zero key: every projection is exactly 0
  uint64_t open = __ballot(!decided && sub == 0);
  while (open != 0) {   // wave-uniform
    const int l = __builtin_ctzll(open);
    if (lane == l) bit = exact_sign_long(krow, s_md + static_cast<int64_t>(i) * D, long_scratch[wave]);
    open &= open - 1;
  }
  // lane 4q (q = 0..15) holds the bit of coordinate cbase + 16 wave + q
  const uint64_t mask = __ballot(bit && sub == 0);
  uint32_t half = 0;
#pragma unroll
  for (int q = 0; q < 16; ++q) half |= static_cast<uint32_t>((mask >> (4 * q)) & 1u) << q;
  const int64_t row = dest_row(r, static_cast<uint32_t>(n), cap, pos);
  if (lane == 0) {
    // coordinates cbase + 16 wave .. +15: half (wave & 1) of word (cbase + 16 wave) / 32
    const int c = cbase + 16 * wave;
    reinterpret_cast<uint16_t*>(signs + row * WPR + c / 32)[(c / 16) & 1] = static_cast<uint16_t>(half);
    if (cbase == 0 && wave == 0) norms[row] = static_cast<float>(knorm);
  }
}

template <int M>
int launch_encode_small(const DeviceSketch& s, const void* keys, int R, int n, uint32_t* signs,
                        float* norms, int cap, int pos, hipStream_t stream) {
  const int64_t blocks = static_cast<int64_t>(R) * (M / 64);
  hipLaunchKernelGGL(encode_small_kernel<M>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(keys), s.s_md, s.col_norm_all, signs, norms, n, cap, pos);
  return hipGetLastError();
}

template <int M>
int launch_encode_m(const DeviceSketch& s, const void* keys, int R, int n, uint32_t* signs,
                    float* norms, int cap, int pos, hipStream_t stream) {
  // (chunks start at multiples of the tile, so alignment carries over)
  if (n % KT == 0) return launch_encode_chunks<M, true>(s, keys, R, n, signs, norms, cap, pos, stream);
  return launch_encode_chunks<M, false>(s, keys, R, n, signs, norms, cap, pos, stream);
}

}  // namespace

// Key sets of at most this many keys go to the small-set kernel.  The limit
// is per thread (a test hook may move it for its own calls only).
thread_local int encode_small_max = kEncodeSmallMaxDefault;

int launch_encode(const DeviceSketch& s, const void* keys, int B, int H_kv, int n, uint32_t* signs,
                  float* norms, int cap, int pos, void* stream) {
  const int64_t R = static_cast<int64_t>(B) * H_kv * n;
  if (R == 0) return hipSuccess;
  if (R > INT32_MAX) return hipErrorInvalidValue;   // the kernel indexes keys in 32 bits
  hipStream_t st = static_cast<hipStream_t>(stream);
  // (the small-set grid, R * m / 64 workgroups of 256 threads, stays below
  // 2^31 threads whatever the limit is set to)
  if (R <= encode_small_max && R * (s.m / 64) <= (int64_t{1} << 23)) {
    if (s.m == 256) return launch_encode_small<256>(s, keys, static_cast<int>(R), n, signs, norms, cap, pos, st);
    return launch_encode_small<512>(s, keys, static_cast<int>(R), n, signs, norms, cap, pos, st);
  }
  if (s.m == 256) return launch_encode_m<256>(s, keys, static_cast<int>(R), n, signs, norms, cap, pos, st);
  return launch_encode_m<512>(s, keys, static_cast<int>(R), n, signs, norms, cap, pos, st);
}

int set_encode_small_max(int keys) {
  const int prev = encode_small_max;
  if (keys >= 0) encode_small_max = keys;
  return prev;
}

}  // namespace qjl
