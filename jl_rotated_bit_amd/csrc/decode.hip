// QJL decode attention for gfx950: one kernel per decode step.
//
// Method: "QJL: 1-Bit Quantized JL Transform for KV Cache Quantization with
// Zero Overhead", Abstract (asymmetric estimator: the query takes the plain
// JL transform, the key its sign bits; unbiased) and "The Geometry of
// Forgetting: How Three Papers Cracked KV Cache Quantization", section "QJL:
// one bit, zero parameters, unbiased inner products" (the sqrt(pi/2) constant
// over the sketch size; attention scores are inner products).  For query head
// h and cached token t:
//   est_t = sqrt(pi/2)/m * ||k_t|| * sum_i (S^T q)_i (2 b_ti - 1),
//   out   = sum_t softmax_t(scale * est) v_t.
//
// Kernel design.  The step is bound by HBM: per (token, kv head) it reads m/8
// bytes of sign words, 4 bytes of norm and 2d bytes of bf16 values.
// * Grid = (context split, kv head, batch).  A workgroup (4 waves) serves the
//   G query heads of one kv head over one token range.
// * Prologue: q is split once per workgroup into three bf16 parts; S^T q for
//   the G heads then runs on the matrix cores (fp32 accumulation), and feeds
//   an LDS table of the 16 signed sums of every group of 4 consecutive sketch
//   coordinates, per head.  A token's bit dot product then costs m/4 table
//   reads and adds per head instead of m masked adds.  The first token tile's
//   loads are in flight during the whole prologue.
// * Main loop, per wave and 64-token tile: lane t scores token t (its sign
//   words and norm arrive with 16-byte loads) and does the online-softmax
//   update; the probabilities, split into bf16 hi + lo parts, go to LDS.  The
//   value rows (16-byte loads, 16 lanes per row) go to a wave-private,
//   padded, row-permuted LDS tile, are read back transposed (ds_read_b64_tr_b16) as
//   the B operand of v_mfma_f32_16x16x32_bf16, and P (rows = head x part) V
//   accumulates on the matrix cores.  The next tile's loads are issued
//   before the current tile is used.
// * Epilogue: waves merge in LDS; the workgroup stores its partial
//   (max, sum, acc) per head with coherent stores; the last workgroup of a
//   (batch, kv head) to arrive (atomic counter) merges all splits by
//   log-sum-exp and writes out, then returns the counter to zero.

#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "internal.h"

namespace qjl {
namespace {

constexpr int D = kHeadDim;
constexpr int NW = 4;            // waves per workgroup
constexpr int NT = 64 * NW;
constexpr int TILE = 64;         // tokens per wave per step
constexpr int HALF = 32;         // tokens per P.V matrix step (MFMA K)
constexpr int VCH = TILE * D * 2 / 16 / 64;  // 16-byte value chunks per lane per tile (16)
constexpr int NDB = D / 16;      // 16-column blocks of the output (8)
constexpr int VROW = D * 2 + 32; // bytes per value row in LDS (256 + 32 padding)
constexpr int VBUF = HALF * VROW;            // wave-private value tile (9 KB)
constexpr int MAX_SPLITS = 256;

typedef __bf16 bf16x8_t __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x16_t __attribute__((__vector_size__(16 * sizeof(float))));
typedef float f32x4_t __attribute__((__vector_size__(4 * sizeof(float))));
typedef short i16x4_t __attribute__((ext_vector_type(4)));

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

// 16-byte global load as a native vector (a struct copy would become a
// memcpy that keeps the destination array out of registers)
__device__ __forceinline__ uint4 ld16(const void* p) {
  const u32x4_t v = *reinterpret_cast<const u32x4_t*>(p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Cross-lane moves through DPP (VALU, no LDS round trip).
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), CTRL, ROW_MASK, 0xF, false));
}
constexpr int kQuadSwap1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kQuadSwap2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;
constexpr int kRowBcast15 = 0x142;    // lane 15 of each row -> next row
constexpr int kRowBcast31 = 0x143;    // lane 31 -> rows 2 and 3
constexpr int kRowShl = 0x100;        // + n: lane l reads lane l + n of its row

// Reductions over the 64 lanes: quad, half-row, row, then two row
// broadcasts leave the total in lane 63, which is read back as a uniform.
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp<kQuadSwap1>(x));
  x = fmaxf(x, dpp<kQuadSwap2>(x));
  x = fmaxf(x, dpp<kRowHalfMirror>(x));
  x = fmaxf(x, dpp<kRowMirror>(x));
  x = fmaxf(x, dpp<kRowBcast15, 0xA>(x));
  x = fmaxf(x, dpp<kRowBcast31, 0xC>(x));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}
__device__ __forceinline__ float wave_sum(float x) {
  x += dpp<kQuadSwap1>(x);
  x += dpp<kQuadSwap2>(x);
  x += dpp<kRowHalfMirror>(x);
  x += dpp<kRowMirror>(x);
  x += dpp<kRowBcast15, 0xA>(x);
  x += dpp<kRowBcast31, 0xC>(x);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}

// LDS row of token t (0..31) of a half tile.  A transposed read by 32 lanes
// touches tokens {0..3, 8..11} (+4, +16 variants); with 288-byte rows, row r
// starts on bank 8*(r mod 8), so swapping rows 8..11 with 12..15 (and 24..27
// with 28..31) puts those 8 tokens on 8 distinct bank groups.  Every column
// offset stays an immediate.
__device__ __forceinline__ constexpr int vrow(int t) { return t ^ ((t & 8) >> 1); }

// G floats read or written as one LDS access (b32 / b64 / b128; two b128 for G = 8).
template <int G>
struct alignas(G >= 4 ? 16 : 4 * G) VecG {
  float v[G];
};

template <int M, int G>
struct DecodeLds {
  static constexpr int NPOS = M / 4;                 // nibble positions
  static constexpr int LUT_FLOATS = NPOS * 16 * G;
  static constexpr int LUT_BYTES = LUT_FLOATS * 4;
  static constexpr int PB_BYTES = NW * 2 * G * TILE * 2;   // bf16 P parts
  static constexpr int VB_BYTES = NW * VBUF;               // value tiles
  // prologue scratch (aliases the value tiles)
  static constexpr int QS_BYTES = G * D * 4;
  static constexpr int QF_BYTES = 8 * 2 * 32 * 16;         // q parts as MFMA operand
  static constexpr int SQ_BYTES = G * M * 4;
  static_assert(QS_BYTES + QF_BYTES + SQ_BYTES <= VB_BYTES, "prologue scratch exceeds the value tiles");
  static_assert(G * D * 4 <= VBUF, "wave partial exceeds its value tile");
  static constexpr int TOTAL = LUT_BYTES + PB_BYTES + VB_BYTES;
};

template <int M, int G>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2))) void decode_kernel(
    const float* __restrict__ q, const uint32_t* __restrict__ signs,
    const float* __restrict__ norms, const uint16_t* __restrict__ values,
    const uint16_t* __restrict__ s_frag, int H_kv, int N, int cap, int n_split, int tps,
    float coef, float* __restrict__ out, uint32_t* __restrict__ counters,
    float* __restrict__ part_acc, float* __restrict__ part_ml) {
  using L = DecodeLds<M, G>;
  constexpr int WPR = M / 32;        // sign words per token
  constexpr int SV = WPR / 4;        // 16-byte sign loads per token
  constexpr int NPOS = L::NPOS;
  static_assert(2 * G <= 16, "P rows (head x part) must fit one 16-row MFMA block");

  __shared__ __attribute__((aligned(16))) uint8_t smem[L::TOTAL];
  __shared__ float red_ml[NW][G][2];
  __shared__ int is_last;
  float* lut = reinterpret_cast<float*>(smem);
  uint8_t* pb_all = smem + L::LUT_BYTES;
  uint8_t* vb_all = smem + L::LUT_BYTES + L::PB_BYTES;
  float* qs = reinterpret_cast<float*>(vb_all);                                  // [G][D]
  uint4* qfrag = reinterpret_cast<uint4*>(vb_all + L::QS_BYTES);                 // [8][2][32]
  float* sq = reinterpret_cast<float*>(vb_all + L::QS_BYTES + L::QF_BYTES);      // [G][M]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int split = blockIdx.x;
  const int kvh = blockIdx.y;
  const int b = blockIdx.z;
  const int64_t bh = static_cast<int64_t>(b) * H_kv + kvh;
  const int t_begin = split * tps;
  const int t_end = min(N, t_begin + tps);

  const uint32_t* sg_base = signs + bh * cap * WPR;
  const float* nm_base = norms + bh * cap;
  const uint16_t* v_base = values + bh * cap * D;
  uint16_t* pbh = reinterpret_cast<uint16_t*>(pb_all) + wave * 2 * G * TILE;  // [2][G][TILE]
  uint8_t* vbuf = vb_all + wave * VBUF;

  uint4 vc[VCH];
  uint4 sc[SV];
  float nc = 0.f;
  // Tile loads are branch-free: rows past the end of the split are clamped to
  // its last row (masked later: logit -inf, probability 0).  Branches around
  // loads would make the compiler's memory-counter waits conservative (a full
  // drain), which would serialize the prologue behind the tile prefetch.
  auto load_signs = [&](int t0, uint4* ss, float& nn) {
    const int ts = min(t0 + lane, t_end - 1);
    const uint4* p = reinterpret_cast<const uint4*>(sg_base + static_cast<int64_t>(ts) * WPR);
#pragma unroll
    for (int k = 0; k < SV; ++k) ss[k] = ld16(p + k);
    nn = nm_base[ts];
  };
  // value chunk c of a tile: token t0 + 4c + lane/16, channels 8*(lane%16) .. +7
  auto load_values = [&](int t0, auto half_const) {
    constexpr int c_begin = decltype(half_const)::value * (VCH / 2);
#pragma unroll
    for (int u = 0; u < VCH / 2; ++u) {
      const int tv = min(t0 + 4 * (c_begin + u) + (lane >> 4), t_end - 1);
      vc[c_begin + u] = ld16(reinterpret_cast<const uint4*>(v_base + static_cast<int64_t>(tv) * D) + (lane & 15));
    }
  };
  int t0 = t_begin + wave * TILE;

  // ---- prologue ----
  // q and the S^T fragments are requested first; memory counters drain in
  // order, so waiting for them leaves the later tile loads in flight.
  constexpr int NBLK = M / 32;            // blocks of 32 sketch coordinates
  constexpr int BPW = NBLK / NW;          // blocks per wave (2 or 4)
  constexpr int BATCH = BPW;             // all fragments go out before the tile loads
  static_assert(BPW % BATCH == 0, "blocks per wave must be a multiple of the batch");
  const int col = lane & 31;
  const int half = lane >> 5;
  // S^T comes in fragment order (see DeviceSketch::s_frag): the operand of
  // (block, k-step) is 64 lanes x 16 contiguous bytes, one 1 KB load.
  uint4 af[BATCH][8];
  auto load_frags = [&](int batch) {
#pragma unroll
    for (int bb = 0; bb < BATCH; ++bb) {
      const int blk = wave + NW * (batch * BATCH + bb);
      const uint4* fr = reinterpret_cast<const uint4*>(s_frag) + static_cast<int64_t>(blk) * 8 * 64 + lane;
#pragma unroll
      for (int st = 0; st < 8; ++st) af[bb][st] = fr[st * 64];
    }
  };
  const float* qb = q + bh * G * D;
  constexpr int QPT = (G * D + NT - 1) / NT;
  float qv[QPT];
#pragma unroll
  for (int k = 0; k < QPT; ++k) qv[k] = (tid + k * NT < G * D) ? qb[tid + k * NT] : 0.f;
  // every wave has requested q before any wave requests S^T or its tile, so
  // q is at the head of this compute unit's memory queue
  __syncthreads();
  load_frags(0);
  load_signs(t0, sc, nc);
  load_values(t0, std::integral_constant<int, 0>{});
  load_values(t0, std::integral_constant<int, 1>{});
#pragma unroll
  for (int k = 0; k < QPT; ++k) {
    const int i = tid + k * NT;
    if (i < G * D) qs[i] = qv[k];
  }
  __syncthreads();
  // q -> three bf16 parts (hi + mid + lo equals fp32 q to within 2^-24
  // relative), laid out as the MFMA B operand: column c = part * G + head.
  for (int e = tid; e < 8 * 2 * 32; e += NT) {
    const int st = e >> 6, hf = (e >> 5) & 1, c = e & 31;
    const int part = c / G, g = c % G;
    uint32_t pk[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      uint32_t h2[2];
#pragma unroll
      for (int v = 0; v < 2; ++v) {
        const float x = part < 3 ? qs[g * D + 16 * st + 8 * hf + 2 * u + v] : 0.f;
        const uint32_t hi = f32_to_bf16_rne(x);
        const float r1 = x - __uint_as_float(hi << 16);
        const uint32_t mid = f32_to_bf16_rne(r1);
        const float r2 = r1 - __uint_as_float(mid << 16);
        const uint32_t lo = f32_to_bf16_rne(r2);
        h2[v] = part == 0 ? hi : (part == 1 ? mid : lo);
      }
      pk[u] = h2[0] | (h2[1] << 16);
    }
    qfrag[e] = make_uint4(pk[0], pk[1], pk[2], pk[3]);
  }
  __syncthreads();
  {
#pragma unroll
    for (int batch = 0; batch < BPW / BATCH; ++batch) {
      if (batch > 0) load_frags(batch);
#pragma unroll
      for (int bb = 0; bb < BATCH; ++bb) {
        const int blk = wave + NW * (batch * BATCH + bb);
        f32x16_t acc = {};
#pragma unroll
        for (int st = 0; st < 8; ++st)
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, af[bb][st]),
                                                        __builtin_bit_cast(bf16x8_t, qfrag[(st * 2 + half) * 32 + col]),
                                                        acc, 0, 0, 0);
        // lane (col, half), register r -> coordinate 32*blk + 8*(r/4) + 4*half + r%4
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float v;
          if (G < 8) {   // columns col + G and col + 2G lie in the same 16-lane row
            v = acc[r] + dpp<kRowShl + G>(acc[r]) + dpp<kRowShl + 2 * G>(acc[r]);
          } else {
            v = acc[r] + __shfl(acc[r], lane + G) + __shfl(acc[r], lane + 2 * G);
          }
          if (col < G) sq[col * M + 32 * blk + 8 * (r >> 2) + 4 * half + (r & 3)] = v;
        }
      }
    }
  }
  __syncthreads();
  // entry v of group p: sum_k (bit k of v ? +1 : -1) * sq[4p + k]
  //   = base + 2 * sum_{k in v} sq[4p + k],  base = -sum_k sq[4p + k]
  for (int e = tid; e < NPOS * G; e += NT) {
    const int p = e / G, g = e % G;
    const float4 x = *reinterpret_cast<const float4*>(&sq[g * M + 4 * p]);
    float t[16];
    t[0] = -(x.x + x.y + x.z + x.w);
    t[1] = t[0] + 2.f * x.x;
    t[2] = t[0] + 2.f * x.y;
    t[3] = t[1] + 2.f * x.y;
#pragma unroll
    for (int v = 4; v < 8; ++v) t[v] = t[v - 4] + 2.f * x.z;
#pragma unroll
    for (int v = 8; v < 16; ++v) t[v] = t[v - 8] + 2.f * x.w;
#pragma unroll
    for (int v = 0; v < 16; ++v) lut[(p * 16 + v) * G + g] = t[v];
  }
  __syncthreads();

  // ---- main loop ----
  float m_run[G], l_run[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m_run[g] = -INFINITY;
    l_run[g] = 0.f;
  }
  f32x4_t acc[NDB];
#pragma unroll
  for (int nb = 0; nb < NDB; ++nb) acc[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // P operand rows: row = part * G + head for row < 2G (lane & 15 = row)
  const int prow = lane & 15;
  const int ppart = prow / G, phead = prow % G;
  const bool prow_live = prow < 2 * G;
  const int kgrp = lane >> 4;       // MFMA k group: tokens 8*kgrp .. +7 of the step
  int row_head[4];                  // head of accumulator row 4*kgrp + r, or -1
#pragma unroll
  for (int r = 0; r < 4; ++r) row_head[r] = (4 * kgrp + r < 2 * G) ? (4 * kgrp + r) % G : -1;
  // transposed-read source: lane s of a 16-lane group addresses token
  // 8*kgrp + s/4 (+4 for the second read), columns 4*(s%4) .. +3 of the block
  const int tr_tok = 8 * kgrp + ((lane & 15) >> 2);
  const uint8_t* tr_base0 = vbuf + vrow(tr_tok) * VROW + 8 * (lane & 3);
  const uint8_t* tr_base1 = vbuf + vrow(tr_tok + 4) * VROW + 8 * (lane & 3);

  // Only one tile of values lives in registers: each half is reloaded with
  // the next tile's rows as soon as it has been copied into LDS.  Sign words
  // and norms of the next tile are requested first, so waiting for them does
  // not wait for the values.
  while (t0 < t_end) {
    const int t_next = t0 + NW * TILE;
    uint4 sn[SV];
    float nn;
    load_signs(t_next, sn, nn);

    // scores: lane <-> token t0 + lane
    float sc_g[G];
#pragma unroll
    for (int g = 0; g < G; ++g) sc_g[g] = 0.f;
#pragma unroll
    for (int k = 0; k < SV; ++k) {
      const uint32_t wv[4] = {sc[k].x, sc[k].y, sc[k].z, sc[k].w};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t w = wv[u];
#pragma unroll
        for (int nib = 0; nib < 8; ++nib) {
          const int pos = (4 * k + u) * 8 + nib;
          const uint32_t idx = (w >> (4 * nib)) & 15u;
          const VecG<G> t = *reinterpret_cast<const VecG<G>*>(&lut[(pos * 16 + idx) * G]);
#pragma unroll
          for (int g = 0; g < G; ++g) sc_g[g] += t.v[g];
        }
        // keep at most one word's table reads in flight (register pressure)
        __asm__ __volatile__("" ::: "memory");
      }
    }
    const bool valid = (t0 + lane) < t_end;
    float alpha_g[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float logit = valid ? sc_g[g] * (coef * nc) : -INFINITY;
      const float tmax = wave_max(logit);
      const float m_new = fmaxf(m_run[g], tmax);
      const float alpha = exp2f(m_run[g] - m_new);
      const float p = valid ? exp2f(logit - m_new) : 0.f;
      l_run[g] = l_run[g] * alpha + p;
      m_run[g] = m_new;
      // P as bf16 hi + lo (about 16 significant bits)
      const uint32_t hi = f32_to_bf16_rne(p);
      const uint32_t lo = f32_to_bf16_rne(p - __uint_as_float(hi << 16));
      pbh[g * TILE + lane] = static_cast<uint16_t>(hi);
      pbh[(G + g) * TILE + lane] = static_cast<uint16_t>(lo);
      alpha_g[g] = alpha;
    }
    // rescale the running output: register r of this lane holds row
    // 4*kgrp + r, i.e. head row_head[r] (rows >= 2G are unused)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float a = 1.f;
#pragma unroll
      for (int g = 0; g < G; ++g) a = (row_head[r] == g) ? alpha_g[g] : a;
#pragma unroll
      for (int nb = 0; nb < NDB; ++nb) acc[nb][r] *= a;
    }

    // P.V for rows 32*HS .. +31 of the tile (HS = 0, 1 as constants, so the
    // value registers are addressed statically)
    auto pv_half = [&](auto hs_const) {
      constexpr int hstep = decltype(hs_const)::value;
      // value rows 32*hstep .. +31 of the tile -> wave-private LDS tile
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        // token 4u + lane/16 of the half tile; vrow() only permutes the
        // groups of 4 rows, so the lane part stays a per-lane base
        const int row = vrow(4 * u) + (lane >> 4);
        *reinterpret_cast<uint4*>(vbuf + row * VROW + (lane & 15) * 16) = vc[8 * hstep + u];
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      load_values(t_next, hs_const);
      // A operand: P rows, tokens 32*hstep + 8*kgrp .. +7
      uint4 pa = make_uint4(0, 0, 0, 0);
      if (prow_live)
        pa = *reinterpret_cast<const uint4*>(pbh + (ppart * G + phead) * TILE + HALF * hstep + 8 * kgrp);
      const bf16x8_t a_op = __builtin_bit_cast(bf16x8_t, pa);
#pragma unroll
      for (int nb = 0; nb < NDB; ++nb) {
        const uint8_t* p0 = tr_base0 + 32 * nb;
        const uint8_t* p1 = tr_base1 + 32 * nb;
        const i16x4_t lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4_t*)(p0));
        const i16x4_t hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4_t*)(p1));
        const uint2 l2 = __builtin_bit_cast(uint2, lo4);
        const uint2 h2 = __builtin_bit_cast(uint2, hi4);
        const uint4 bv = make_uint4(l2.x, l2.y, h2.x, h2.y);
        acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_op, __builtin_bit_cast(bf16x8_t, bv), acc[nb], 0, 0, 0);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };
    pv_half(std::integral_constant<int, 0>{});
    pv_half(std::integral_constant<int, 1>{});

    t0 = t_next;
#pragma unroll
    for (int k = 0; k < SV; ++k) sc[k] = sn[k];
    nc = nn;
  }

  // ---- wave result: out row = hi row + lo row, into this wave's LDS tile ----
  // Accumulator block nb: lane l holds row 4*(l/16) + r, column l%16.  Row g
  // (hi part of head g) pairs with row G + g (lo part): for G >= 4 the lo row
  // sits G/4 lane groups later in the same register; for G < 4 both rows are
  // registers of lanes 0..15.
  float* wacc = reinterpret_cast<float*>(vbuf);   // [G][D]
#pragma unroll
  for (int g = 0; g < G; ++g) l_run[g] = wave_sum(l_run[g]);
#pragma unroll
  for (int nb = 0; nb < NDB; ++nb) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (G >= 4) {
        const float v = acc[nb][r] + __shfl(acc[nb][r], (lane + 16 * (G / 4)) & 63);
        const int row = 4 * kgrp + r;
        if (row < G) wacc[row * D + 16 * nb + (lane & 15)] = v;
      } else if (r < G) {
        if (kgrp == 0) wacc[r * D + 16 * nb + (lane & 15)] = acc[nb][r] + acc[nb][(r + G) & 3];
      }
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      red_ml[wave][g][0] = m_run[g];
      red_ml[wave][g][1] = l_run[g];
    }
  }
  __syncthreads();

  const int64_t slot0 = bh * n_split + split;   // partial index base
  for (int i = tid; i < G * D; i += NT) {
    const int g = i / D, dd = i % D;
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) mx = fmaxf(mx, red_ml[w][g][0]);
    float Ls = 0.f, A = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float mw = red_ml[w][g][0];
      const float f = mw == -INFINITY ? 0.f : exp2f(mw - mx);
      Ls += red_ml[w][g][1] * f;
      A += reinterpret_cast<const float*>(vb_all + w * VBUF)[g * D + dd] * f;
    }
    if (n_split == 1) {
      out[(bh * G + g) * D + dd] = A / Ls;
    } else {
      // coherent (sc1) stores: visible to every XCD once complete, with no
      // L2-wide write-back (an agent-scope fence would flush the whole L2)
      __hip_atomic_store(&part_acc[(slot0 * G + g) * D + dd], A, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
      if (dd == 0) {
        __hip_atomic_store(&part_ml[(slot0 * G + g) * 2 + 0], mx, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&part_ml[(slot0 * G + g) * 2 + 1], Ls, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  if (n_split == 1) return;

  // ---- last workgroup of this (batch, kv head) merges the splits ----
  // Release: wait until this thread's coherent partial stores are complete,
  // then (after the barrier) count this workgroup in.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) {
    const uint32_t prev =
        __hip_atomic_fetch_add(&counters[bh], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    is_last = (prev == static_cast<uint32_t>(n_split - 1));
  }
  __syncthreads();
  if (!is_last) return;

  // Acquire for this workgroup only: drop stale cache lines, after which
  // plain (vector) loads see the partials the other workgroups stored
  // coherently.  Only the last workgroup of each (batch, kv head) pays it.
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  // Threads own (head, 4 channels) pairs; with fewer pairs than threads the
  // splits are divided among REP replicas whose sums meet in LDS.  The
  // (max, sum) pairs and the first MCH partial accumulators of every thread
  // are requested together, so the merge costs one round trip to memory.
  constexpr int PAIRS = G * D / 4;
  constexpr int REP = PAIRS >= NT ? 1 : NT / PAIRS;
  constexpr int MCH = 32;                 // float4 loads in flight per thread
  static_assert(REP == 1 || REP * PAIRS * 16 <= L::VB_BYTES, "merge replicas exceed the LDS buffer");
  float* ml_l = lut;                      // 2 * n_split * G floats
  float* wts = lut + 2 * MAX_SPLITS * G;  // n_split * G floats
  static_assert(3 * MAX_SPLITS * G <= L::LUT_FLOATS, "merge scratch exceeds the table");
  const float2* ml_src = reinterpret_cast<const float2*>(part_ml + bh * n_split * G * 2);
  const float4* pa = reinterpret_cast<const float4*>(part_acc);
  constexpr int ML_PT = (MAX_SPLITS * G + NT - 1) / NT;
  float2 mlv[ML_PT];
#pragma unroll
  for (int k = 0; k < ML_PT; ++k) {
    const int i = tid + k * NT;
    if (i < n_split * G) mlv[k] = ml_src[i];
  }
  const int pr = tid % PAIRS, rep = tid / PAIRS;       // valid when tid < PAIRS * REP
  const int mg = pr / (D / 4), c4 = pr % (D / 4);
  float4 av[MCH];
#pragma unroll
  for (int u = 0; u < MCH; ++u) {
    const int s = rep + u * REP;
    if (tid < PAIRS * REP && s < n_split) av[u] = pa[((bh * n_split + s) * G + mg) * (D / 4) + c4];
  }
#pragma unroll
  for (int k = 0; k < ML_PT; ++k) {
    const int i = tid + k * NT;
    if (i < n_split * G) reinterpret_cast<float2*>(ml_l)[i] = mlv[k];
  }
  __syncthreads();
  // per head: global max and normalizer, then per-split weights
  __shared__ float gmax[G], gsum[G];
  for (int g = wave; g < G; g += NW) {
    float mx = -INFINITY;
    for (int s = lane; s < n_split; s += 64) mx = fmaxf(mx, ml_l[(s * G + g) * 2]);
    mx = wave_max(mx);
    float Ls = 0.f;
    for (int s = lane; s < n_split; s += 64) Ls += ml_l[(s * G + g) * 2 + 1] * exp2f(ml_l[(s * G + g) * 2] - mx);
    Ls = wave_sum(Ls);
    if (lane == 0) {
      gmax[g] = mx;
      gsum[g] = Ls;
    }
  }
  __syncthreads();
  for (int i = tid; i < n_split * G; i += NT) wts[i] = exp2f(ml_l[2 * i] - gmax[i % G]) / gsum[i % G];
  __syncthreads();
  if (tid < PAIRS * REP) {
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int u = 0; u < MCH; ++u) {
      const int s = rep + u * REP;
      if (s < n_split) {
        const float wgt = wts[s * G + mg];
        o.x = __builtin_fmaf(wgt, av[u].x, o.x);
        o.y = __builtin_fmaf(wgt, av[u].y, o.y);
        o.z = __builtin_fmaf(wgt, av[u].z, o.z);
        o.w = __builtin_fmaf(wgt, av[u].w, o.w);
      }
    }
    for (int s = rep + MCH * REP; s < n_split; s += REP) {   // splits beyond the first batch
      const float4 v = pa[((bh * n_split + s) * G + mg) * (D / 4) + c4];
      const float wgt = wts[s * G + mg];
      o.x = __builtin_fmaf(wgt, v.x, o.x);
      o.y = __builtin_fmaf(wgt, v.y, o.y);
      o.z = __builtin_fmaf(wgt, v.z, o.z);
      o.w = __builtin_fmaf(wgt, v.w, o.w);
    }
    if (REP == 1) {
      reinterpret_cast<float4*>(out)[(bh * G + mg) * (D / 4) + c4] = o;
    } else {
      reinterpret_cast<float4*>(vb_all)[rep * PAIRS + pr] = o;
    }
  }
  if (REP > 1) {
    __syncthreads();
    for (int p2 = tid; p2 < PAIRS; p2 += NT) {
      float4 o = reinterpret_cast<const float4*>(vb_all)[p2];
      for (int r2 = 1; r2 < REP; ++r2) {
        const float4 v = reinterpret_cast<const float4*>(vb_all)[r2 * PAIRS + p2];
        o.x += v.x;
        o.y += v.y;
        o.z += v.z;
        o.w += v.w;
      }
      const int g = p2 / (D / 4), cc = p2 % (D / 4);
      reinterpret_cast<float4*>(out)[(bh * G + g) * (D / 4) + cc] = o;
    }
  }
  if (tid == 0) __hip_atomic_store(&counters[bh], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int M, int G>
int launch_decode_mg(const DeviceSketch& s, const DecodePlan& plan, const float* q,
                     const uint32_t* signs, const float* norms, const void* values, int B,
                     int H_kv, int N, int cap, float coef, float* out, void* workspace,
                     hipStream_t stream) {
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  uint32_t* counters = reinterpret_cast<uint32_t*>(ws);
  float* part_acc = reinterpret_cast<float*>(ws + plan.counter_bytes);
  float* part_ml = part_acc + static_cast<size_t>(B) * H_kv * G * plan.n_split * D;
  dim3 grid(plan.n_split, H_kv, B);
  hipLaunchKernelGGL((decode_kernel<M, G>), grid, dim3(NT), 0, stream, q, signs, norms,
                     static_cast<const uint16_t*>(values), s.s_frag, H_kv, N, cap, plan.n_split,
                     plan.tokens_per_split, coef, out, counters, part_acc, part_ml);
  return hipGetLastError();
}

template <int M>
int launch_decode_m(int G, const DeviceSketch& s, const DecodePlan& plan, const float* q,
                    const uint32_t* signs, const float* norms, const void* values, int B,
                    int H_kv, int N, int cap, float coef, float* out, void* workspace,
                    hipStream_t st) {
  switch (G) {
    case 1: return launch_decode_mg<M, 1>(s, plan, q, signs, norms, values, B, H_kv, N, cap, coef, out, workspace, st);
    case 2: return launch_decode_mg<M, 2>(s, plan, q, signs, norms, values, B, H_kv, N, cap, coef, out, workspace, st);
    case 4: return launch_decode_mg<M, 4>(s, plan, q, signs, norms, values, B, H_kv, N, cap, coef, out, workspace, st);
    case 8: return launch_decode_mg<M, 8>(s, plan, q, signs, norms, values, B, H_kv, N, cap, coef, out, workspace, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool make_decode_plan(int B, int H_q, int H_kv, int N, int d, int m, DecodePlan* plan) {
  if (B <= 0 || H_q <= 0 || H_kv <= 0 || N <= 0 || d != D || (m != 256 && m != 512)) return false;
  if (H_q % H_kv) return false;
  const int64_t streams = static_cast<int64_t>(B) * H_kv;
  // Aim for about two workgroups per compute unit (256 CUs) while keeping at
  // least one full step (4 waves x 64 tokens) per split.
  constexpr int64_t kTargetWorkgroups = 512;
  constexpr int kMinTokens = NW * TILE;
  int64_t want = (kTargetWorkgroups + streams - 1) / streams;
  if (streams > kMaxCounters) want = 1;   // splits (and counters) only for few streams
  const int64_t most = (N + kMinTokens - 1) / kMinTokens;
  if (want > most) want = most;
  if (want > MAX_SPLITS) want = MAX_SPLITS;
  if (want < 1) want = 1;
  int64_t tps = (N + want - 1) / want;
  tps = (tps + TILE - 1) / TILE * TILE;
  const int64_t n_split = (N + tps - 1) / tps;
  plan->n_split = static_cast<int>(n_split);
  plan->tokens_per_split = static_cast<int>(tps);
  // A fixed-size counter region keeps the counters of every plan clear of the
  // partials of any other plan, so one zero-filled workspace serves calls of
  // all sizes.
  plan->counter_bytes = kCounterRegionBytes;
  const size_t parts = static_cast<size_t>(B) * H_q * n_split;
  plan->partial_bytes = parts * (D + 2) * sizeof(float);
  plan->total_bytes = plan->counter_bytes + plan->partial_bytes;
  return true;
}

int launch_decode(const DeviceSketch& s, const DecodePlan& plan, const float* q,
                  const uint32_t* signs, const float* norms, const void* values, int B, int H_q,
                  int H_kv, int N, int cap, float scale, float* out, void* workspace,
                  void* stream) {
  const int G = H_q / H_kv;
  // logits are kept in base 2: coef = sqrt(pi/2)/m * scale * log2(e)
  const double c = 1.2533141373155002512 / s.m * static_cast<double>(scale) * 1.4426950408889634074;
  const float coef = static_cast<float>(c);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (s.m == 256)
    return launch_decode_m<256>(G, s, plan, q, signs, norms, values, B, H_kv, N, cap, coef, out, workspace, st);
  return launch_decode_m<512>(G, s, plan, q, signs, norms, values, B, H_kv, N, cap, coef, out, workspace, st);
}

}  // namespace qjl
