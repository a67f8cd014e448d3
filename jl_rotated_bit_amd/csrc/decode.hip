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
// * Grid = (context split, kv head, batch).  A workgroup (4 waves, or 8
//   when the context is split and the grid still fills the chip) serves the
//   G query heads of one kv head over one token range.
// * Prologue: q is split once per workgroup into three bf16 parts; S^T q for
//   the G heads runs on the matrix cores (fp32 accumulation).  Each head's
//   S^T q is then written as integers Q_i = round(Sq_i / 2^E) with |Q_i| <=
//   2^21, where 2^(E+21) bounds ||s_i|| ||q|| (Cauchy-Schwarz), as three signed
//   byte limbs (Q = a 2^16 + b 2^8 + c) in LDS.  The first token tile is
//   requested once q is split (in the S^T q waves of eight-wave workgroups at
//   m = 256, once S^T q is done), so its loads are in flight meanwhile.
// * Scores on the int8 matrix cores: per 16-token block, A = the tokens' sign
//   bits spread to 0/1 bytes (rows = tokens), B = the limbs (columns = limb x
//   head), so sum_i b_ti Q_i is exact in int32.  Limb rows are weighted by
//   shifts and summed with 16- and 32-lane row swaps, a reduce-scatter that
//   leaves lane t with token t for all G heads, and est = (2 sum_i b_ti Q_i -
//   sum_i Q_i) 2^E.
// * Online softmax per head in registers; the probabilities, split into bf16
//   hi + lo parts, are already laid out as the A operand (rows = part x head,
//   k = tokens) of v_mfma_f32_16x16x32_bf16.  The value rows (16-byte loads,
//   16 lanes per row) go to a wave-private padded LDS tile and are read back
//   transposed (ds_read_b64_tr_b16) as its B operand.  The next tile's loads
//   are issued before the current tile is used; token tiles are read with
//   the non-temporal cache policy (each byte is read once per call).
// * Epilogue: waves merge in LDS; the workgroup stores its partial
//   (max, sum, acc) per head with coherent stores; the last workgroup of a
//   (batch, kv head) to arrive (atomic counter) merges all splits by
//   log-sum-exp (reading the partials with coherent loads, no cache
//   invalidation) and writes out, then returns the counter to zero.

#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "exact_sign.h"
#include "internal.h"

namespace qjl {
namespace {

constexpr int D = kHeadDim;
constexpr int TILE = 64;         // tokens per wave per step (4 blocks of 16)
constexpr int HALF = 32;         // tokens per P.V matrix step (MFMA K)
constexpr int VCH = TILE * D * 2 / 16 / 64;  // 16-byte value chunks per lane per tile (16)
constexpr int NDB = D / 16;      // 16-column blocks of the output (8)
constexpr int VROW = D * 2 + 32; // bytes per value row in LDS (256 + 32 padding)
constexpr int VBUF = HALF * VROW;            // wave-private value tile (9 KB)
constexpr int MAX_SPLITS = 256;

// Words between the arrival counters of consecutive (batch, kv head) streams
// in the fixed counter region: 64 (a 256-byte line each) when at most 16
// streams split, so that the arrivals of different kv heads do not queue at
// one line's atomic unit; otherwise as far apart as the region allows.
int counter_stride(int B, int H_kv) {
  const int64_t streams = static_cast<int64_t>(B) * H_kv;
  int cs = 64;
  while (cs > 1 && streams * cs > kMaxCounters) cs >>= 1;
  return cs;
}
constexpr int QBITS = 21;        // |Q_i| <= 2^21
constexpr int PROW = 32;         // bytes per token of probability rows (16 bf16: head x part)

typedef __bf16 bf16x8_t __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x16_t __attribute__((__vector_size__(16 * sizeof(float))));
typedef float f32x4_t __attribute__((__vector_size__(4 * sizeof(float))));
typedef int i32x4_t __attribute__((__vector_size__(4 * sizeof(int))));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// 16- and 8-byte global loads as native vectors (a struct copy would become
// a memcpy that keeps the destination array out of registers)
__device__ __forceinline__ uint4 ld16(const void* p) {
  const u32x4_t v = *reinterpret_cast<const u32x4_t*>(p);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 ld8(const void* p) {
  const u32x2_t v = *reinterpret_cast<const u32x2_t*>(p);
  return make_uint2(v.x, v.y);
}

// Buffer descriptor over [base, base + bytes): loads at offsets past the end
// return zero, so the rows past a split's end need no clamping.  base and
// bytes must be wave-uniform.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;   // 32-bit data format, no swizzle
// Cache policy of the token-tile loads: non-temporal (each byte of the cache
// is read once per call).  A plain read stream over 1.5 GB measured 6.0 TB/s
// with the default policy and 6.8 TB/s with this one.
constexpr int kStream = 2;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int bytes) {
  // readfirstlane keeps the (uniform) size in a scalar register; a vector
  // register there would make the compiler loop over lanes around each load
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           __builtin_amdgcn_readfirstlane(bytes), kRsrcWord3);
}

// two floats -> two bf16 (round to nearest even) in one register, low first
__device__ __forceinline__ uint32_t cvt2_bf16(float a, float b) {
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Cross-lane moves through DPP (VALU, no LDS round trip).
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), CTRL, ROW_MASK, 0xF, false));
}
constexpr int kRowShl = 0x100;        // + n: lane l reads lane l + n of its row
constexpr int kRowRor = 0x120;        // + n: rotate within the row by n lanes

// DPP move with every lane enabled and no old value, so the compiler can fold
// it into the consuming VALU instruction.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}

// wave-uniform value kept in a scalar register
__device__ __forceinline__ float uniform(float x) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x)));
}

// Reductions over the 64 lanes: rotations within each 16-lane row, then a
// 16-lane and a 32-lane row swap; the result is read back as a uniform.
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp_f<kRowRor + 8>(x));
  x = fmaxf(x, dpp_f<kRowRor + 4>(x));
  x = fmaxf(x, dpp_f<kRowRor + 2>(x));
  x = fmaxf(x, dpp_f<kRowRor + 1>(x));
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
  return uniform(x);
}
__device__ __forceinline__ float wave_sum(float x) {
  x += dpp_f<kRowRor + 8>(x);
  x += dpp_f<kRowRor + 4>(x);
  x += dpp_f<kRowRor + 2>(x);
  x += dpp_f<kRowRor + 1>(x);
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(c[0]) + __uint_as_float(c[1]);
  return uniform(x);
}

// Sum over the four 16-lane groups of x_j, leaving the total of x_g in
// group g: two 16-lane and one 32-lane row swaps (VALU, no LDS).
// max over each 16-lane row (result in every lane of the row)
__device__ __forceinline__ float row_max(float x) {
  x = fmaxf(x, dpp_f<kRowRor + 8>(x));
  x = fmaxf(x, dpp_f<kRowRor + 4>(x));
  x = fmaxf(x, dpp_f<kRowRor + 2>(x));
  return fmaxf(x, dpp_f<kRowRor + 1>(x));
}
__device__ __forceinline__ float fmax_swap16(float a, float b) {   // [a g0|g1, b g0|g1, a g2|g3, b g2|g3]
  const auto t = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return fmaxf(__uint_as_float(t[0]), __uint_as_float(t[1]));
}
__device__ __forceinline__ float fmax_swap32(float a, float b) {   // [a g0|g2, a g1|g3, b g0|g2, b g1|g3]
  const auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return fmaxf(__uint_as_float(t[0]), __uint_as_float(t[1]));
}
// Maxima over the 64 lanes of G per-lane values (G = 2, 4, 8), as uniforms.
template <int G>
__device__ __forceinline__ void wave_max_heads(const float (&x)[G], float (&m)[G]) {
  float y[G];
#pragma unroll
  for (int h = 0; h < G; ++h) y[h] = row_max(x[h]);
  if constexpr (G == 2) {
    const float z = fmax_swap16(y[0], y[1]);       // groups: h0 (01), h1 (01), h0 (23), h1 (23)
    const float w = fmax_swap32(z, z);             // groups 0, 2: h0; groups 1, 3: h1
    m[0] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), 0));
    m[1] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), 16));
  } else {
#pragma unroll
    for (int q = 0; q < G / 4; ++q) {
      // group g ends with head 4q + g
      const float w = fmax_swap32(fmax_swap16(y[4 * q], y[4 * q + 1]), fmax_swap16(y[4 * q + 2], y[4 * q + 3]));
#pragma unroll
      for (int g = 0; g < 4; ++g) m[4 * q + g] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), 16 * g));
    }
  }
}

__device__ __forceinline__ int reduce_scatter4(int x0, int x1, int x2, int x3) {
  const auto a = __builtin_amdgcn_permlane16_swap(x0, x1, false, false);   // [x0 g0, x1 g0, x0 g2, x1 g2], [.. g1 .. g3]
  const auto b = __builtin_amdgcn_permlane16_swap(x2, x3, false, false);
  const auto c = __builtin_amdgcn_permlane32_swap(a[0] + a[1], b[0] + b[1], false, false);
  return static_cast<int>(c[0] + c[1]);
}

// ---- the decode step's append (one new token per (batch, kv head)) ----
// Four waves (256 threads) of the workgroup whose token range ends with the
// new token encode its key exactly as the encode kernels do: the sign of
// every coordinate of S^T k, certified (four lanes per coordinate multiply
// 32 channels each in fp64, a quad sum joins them: at most 34 roundings, so
// the sum lies within 2^-47 ||k|| max_i ||s_i|| of the exact value and a sum
// beyond 2^-45 ||k|| max_i ||s_i|| fixes the sign; others go to the exact
// integer accumulator), sign(0) = +1, an all-zero key gives all ones.  The
// norm is fp32 of the fp64 root of the fp64 sum of squares.  The bits, the
// norm and the value row are stored to row `pos` of the caches and the
// stores are waited for, so that the workgroup's barrier that follows makes
// them visible to its own tile loads.
template <int M>
__device__ void append_token(const AppendArgs& a, int64_t bh, int cap, int atid, float cnmax,
                             uint32_t* scratch) {
  constexpr int WPR = M / 32;
  const int lane = atid & 63;
  const int aw = atid >> 6;
  const int sub = lane & 3;
  const int quad = atid >> 2;
  const uint16_t* krow = a.key + bh * D;
  const uint4* kr4 = reinterpret_cast<const uint4*>(krow);
  uint4 kc[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) kc[u] = kr4[4 * u + sub];
  double sq = 0.0;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const uint32_t kw[4] = {kc[u].x, kc[u].y, kc[u].z, kc[u].w};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const double lo = bf16_lo_f64(kw[t]), hi = bf16_hi_f64(kw[t]);
      sq += lo * lo;   // squares of bf16 values are exact in fp64
      sq += hi * hi;
    }
  }
  const double ksq = quad_sum_f64(sq);
  const double knorm = __builtin_sqrt(ksq);
  const double thr = 0x1.0p-45 * knorm * static_cast<double>(cnmax);
  const int64_t row = bh * cap + a.pos;
  uint16_t* srow_out = reinterpret_cast<uint16_t*>(a.signs + row * WPR);
#pragma unroll 1
  for (int r = 0; r < M / 64; ++r) {
    const int i = 64 * r + quad;   // this quad's coordinate
    const uint4* srow = reinterpret_cast<const uint4*>(a.s_md + static_cast<int64_t>(i) * D);
    double acc = 0.0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint4 sv = srow[4 * u + sub];
      const uint32_t kw[4] = {kc[u].x, kc[u].y, kc[u].z, kc[u].w};
      const uint32_t sw[4] = {sv.x, sv.y, sv.z, sv.w};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        acc = __builtin_fma(bf16_lo_f64(kw[t]), bf16_lo_f64(sw[t]), acc);
        acc = __builtin_fma(bf16_hi_f64(kw[t]), bf16_hi_f64(sw[t]), acc);
      }
    }
    const double sum = quad_sum_f64(acc);
    bool bit = ksq == 0.0 || sum >= 0.0;   // all-(+/-)zero key: every projection is exactly 0
    const bool decided = ksq == 0.0 || __builtin_fabs(sum) > thr;
    for (uint64_t open = __ballot(!decided && sub == 0); open != 0; open &= open - 1) {
      const int l = __builtin_ctzll(open);   // wave-uniform
      if (lane == l) bit = exact_sign_long_inl(krow, a.s_md + static_cast<int64_t>(i) * D, scratch + aw * 2 * ACC_WORDS);
    }
    // lane 4q holds the bit of coordinate 64 r + 16 aw + q
    const uint64_t mask = __ballot(bit && sub == 0);
    uint32_t half = 0;
#pragma unroll
    for (int q = 0; q < 16; ++q) half |= static_cast<uint32_t>((mask >> (4 * q)) & 1u) << q;
    if (lane == 0) srow_out[4 * r + aw] = static_cast<uint16_t>(half);
  }
  if (atid == 0) a.norms[row] = static_cast<float>(knorm);
  if (atid < 16)
    reinterpret_cast<uint4*>(a.values + row * D)[atid] = reinterpret_cast<const uint4*>(a.val + bh * D)[atid];
  __builtin_amdgcn_s_waitcnt(0);   // the stores are complete before the barrier
}

__device__ __forceinline__ float reduce_scatter4f(float x0, float x1, float x2, float x3) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x0), __float_as_uint(x1), false, false);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x2), __float_as_uint(x3), false, false);
  const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(__uint_as_float(a[0]) + __uint_as_float(a[1])),
                                                  __float_as_uint(__uint_as_float(b[0]) + __uint_as_float(b[1])),
                                                  false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

template <int M, int G, int NW>
struct DecodeLds {
  static constexpr int NT = 64 * NW;
  static constexpr int NSQ = (3 * G + 15) / 16;      // 16-column sets of limb columns
  static constexpr int LROW = M + 16;                // bytes per limb row (padded)
  static constexpr int LIMB_BYTES = 16 * NSQ * LROW; // rows = limb * G + head; others zero
  static constexpr int P_BYTES = NW * TILE * PROW;   // per-wave probability rows
  static constexpr int VB_BYTES = NW * VBUF;         // value tiles
  // prologue scratch (aliases the value tiles)
  static constexpr int QF_BYTES = 8 * 2 * 32 * 16;   // q parts as MFMA operand
  static constexpr int QSS_BYTES = G * 16 * 4;       // partial sums of q^2
  static_assert(QF_BYTES + QSS_BYTES <= VB_BYTES, "prologue scratch exceeds the value tiles");
  static_assert(G * D * 4 <= VBUF, "wave partial exceeds its value tile");
  // split-merge scratch (aliases the value tiles once the wave partials are merged)
  static constexpr int PAIRS = G * D / 4;
  static constexpr int REP = PAIRS >= NT ? 1 : NT / PAIRS;
  static constexpr int ML_FLOATS = 2 * MAX_SPLITS * G;
  static constexpr int WT_FLOATS = MAX_SPLITS * G;
  static_assert((ML_FLOATS + WT_FLOATS) * 4 + (REP > 1 ? REP * PAIRS * 16 : 0) <= VB_BYTES,
                "merge scratch exceeds the value tiles");
  static constexpr int TOTAL = VB_BYTES + LIMB_BYTES + P_BYTES;
};

// APPEND: the step first appends token N - 1 (see append_token); the caches
// are then written and read in one launch, so their pointers carry no
// __restrict__.
// BF16K: the uncompressed baseline.  Scores are the exact q . k over bf16
// keys `kbf` ([B][H_kv][cap][d]) on the bf16 matrix cores (q split into three
// bf16 parts, the A operand; the key rows, loaded straight into registers in
// operand order, the B operand), logit = scale * q . k; the sign words, norms
// and S^T q are not used.  Softmax, P.V and the split merge are shared.
template <int M, int G, int NW, bool APPEND, bool BF16K = false>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2))) void decode_kernel(
    const float* __restrict__ q, const uint32_t* signs, const float* norms, const uint16_t* values,
    const uint16_t* __restrict__ s_frag, float cnmax, int H_kv, int N, int cap, int n_split,
    int tps, float coef, float* __restrict__ out, uint32_t* __restrict__ counters, int cstride,
    float* __restrict__ part_acc, float* __restrict__ part_ml, AppendArgs app,
    const uint16_t* kbf) {
  static_assert(!(APPEND && BF16K), "the baseline kernel has no append");
  static_assert(!BF16K || M == 256, "the baseline kernel reuses the m = 256 LDS layout (256-byte q rows)");
  using L = DecodeLds<M, G, NW>;
  constexpr int NT = 64 * NW;
  constexpr int WPR = M / 32;        // sign words per token
  constexpr int CW = M / 128;        // sign words per lane per 16-token block
  constexpr int KS = M / 64;         // score k-steps of 64 coordinates
  constexpr int NSQ = L::NSQ;
  static_assert(2 * G <= 16, "P rows (head x part) must fit one 16-row MFMA block");

  __shared__ __attribute__((aligned(16))) uint8_t smem[L::TOTAL];
  __shared__ float red_ml[NW][G][2];
  __shared__ int sumq[G];
  __shared__ int is_last;
  __shared__ uint32_t app_scratch[APPEND ? 4 * 2 * ACC_WORDS : 1];
  uint8_t* vb_all = smem;
  uint8_t* limbs = smem + L::VB_BYTES;
  uint8_t* p_all = smem + L::VB_BYTES + L::LIMB_BYTES;
  uint4* qfrag = reinterpret_cast<uint4*>(vb_all);                            // [8][2][32]
  float* qss = reinterpret_cast<float*>(vb_all + L::QF_BYTES);                // [G][16]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15;
  const int grp = lane >> 4;
  const int split = blockIdx.x;
  const int kvh = blockIdx.y;
  const int b = blockIdx.z;
  const int64_t bh = static_cast<int64_t>(b) * H_kv + kvh;
  const int t_begin = split * tps;
  const int t_end = min(N, t_begin + tps);

  const uint32_t* sg_base = signs + bh * cap * WPR;
  const float* nm_base = norms + bh * cap;
  const uint16_t* v_base = values + bh * cap * D;
  uint8_t* vbuf = vb_all + wave * VBUF;
  uint8_t* pbuf = p_all + wave * TILE * PROW;

  uint4 vc[VCH];
  uint32_t sw[4][CW];
  float nv = 0.f;
  uint4 kc[BF16K ? 16 : 1];   // BF16K: key chunks of the current tile
  const uint16_t* k_base = BF16K ? kbf + bh * cap * D : nullptr;
  // Tile loads go through buffer descriptors that start at the tile and end
  // at the split's end: rows past the end read as zero (their logits are
  // masked to -inf), with no per-lane clamping or 64-bit address arithmetic,
  // and no branches (which would make the compiler's memory-counter waits
  // conservative and serialize the prologue behind the tile prefetch).
  // Sign words of block j: lane (row l16, group grp) takes token 16j + l16,
  // coordinates (M/4) grp .. (M/4)(grp + 1) - 1 (CW words); lane t takes the
  // norm of token t0 + t.
  auto tile_rows = [&](int t0_) { return max(0, min(TILE, t_end - t0_)); };
  const int so_lane = l16 * WPR * 4 + CW * 4 * grp;
  auto load_signs = [&](int t0_, uint32_t (&s)[4][CW], float& n) {
    const int rows = tile_rows(t0_);
    const rsrc_t rs = make_rsrc(sg_base + static_cast<int64_t>(t0_) * WPR, rows * WPR * 4);
    const rsrc_t rn = make_rsrc(nm_base + t0_, rows * 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int off = so_lane + 16 * j * WPR * 4;
      if constexpr (CW == 2) {
        const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, kStream);
        s[j][0] = v.x;
        s[j][1] = v.y;
      } else {
        const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, kStream);
        s[j][0] = v.x;
        s[j][1] = v.y;
        s[j][2] = v.z;
        s[j][3] = v.w;
      }
    }
    n = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rn, lane * 4, 0, kStream));
  };
  // BF16K key chunk 4 j + ks: token 16 j + l16 of the tile, channels
  // 32 ks + 8 grp .. +7 (the B operand of v_mfma_f32_16x16x32_bf16 for
  // token block j and channel step ks)
  auto load_keys = [&](int t0_) {
    const rsrc_t rk = make_rsrc(k_base + static_cast<int64_t>(t0_) * D, tile_rows(t0_) * D * 2);
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rk, (16 * j + l16) * D * 2 + 64 * ks + 16 * grp, 0, kStream);
        kc[4 * j + ks] = make_uint4(v.x, v.y, v.z, v.w);
      }
  };
  // value chunk c of a tile: token t0 + 4c + lane/16, channels 8*(lane%16) .. +7
  const int vo_lane = grp * D * 2 + l16 * 16;
  auto load_values = [&](int t0_, auto half_const) {
    constexpr int c_begin = decltype(half_const)::value * (VCH / 2);
    const rsrc_t rv = make_rsrc(v_base + static_cast<int64_t>(t0_) * D, tile_rows(t0_) * D * 2);
#pragma unroll
    for (int u = 0; u < VCH / 2; ++u) {
      const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rv, vo_lane + 4 * (c_begin + u) * D * 2, 0, kStream);
      vc[c_begin + u] = make_uint4(v.x, v.y, v.z, v.w);
    }
  };
  // With eight waves the tiles go to the waves in reverse order: when a
  // split's tiles do not divide evenly, the extra ones go to the last
  // waves, which do not compute S^T q and start streaming first.
  int t0 = t_begin + (NW == 8 ? NW - 1 - wave : wave) * TILE;
  // With APPEND, the workgroup whose range ends with the new token appends
  // it during the prologue; a wave whose first tile holds that token loads
  // the tile only after the append (behind the prologue's last barrier).
  const bool app_wg = APPEND && app.pos >= t_begin && app.pos < t_end;
  const bool defer_first = app_wg && app.pos >= t0 && app.pos < t0 + TILE;

  int e_all[G] = {};
  if constexpr (BF16K) {
    // ---- prologue (baseline) ----
    // rows >= 3G of the q operand and the probability rows stay zero
    constexpr int ZERO_U4 = (16 * L::NSQ - 3 * G) * L::LROW / 16;
    for (int i = tid; i < ZERO_U4; i += NT)
      reinterpret_cast<uint4*>(limbs + 3 * G * L::LROW)[i] = make_uint4(0, 0, 0, 0);
    for (int i = tid; i < L::P_BYTES / 16; i += NT) reinterpret_cast<uint4*>(p_all)[i] = make_uint4(0, 0, 0, 0);
    load_keys(t0);
    load_values(t0, std::integral_constant<int, 0>{});
    load_values(t0, std::integral_constant<int, 1>{});
    // q -> three bf16 parts (hi + mid + lo equals fp32 q to within 2^-24
    // relative): row part * G + head, 256 bytes per row
    const float* qb = q + bh * G * D;
    for (int e = tid; e < G * (D / 8); e += NT) {
      const int h = e / (D / 8), c8 = e % (D / 8);
      const float4* src = reinterpret_cast<const float4*>(qb + h * D + 8 * c8);
      const float4 a0 = src[0], a1 = src[1];
      const float x[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
      uint32_t hi[4], mid[4], lo[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float x0 = x[2 * u], x1 = x[2 * u + 1];
        hi[u] = cvt2_bf16(x0, x1);
        const float r0 = x0 - __uint_as_float(hi[u] << 16), r1 = x1 - __uint_as_float(hi[u] & 0xFFFF0000u);
        mid[u] = cvt2_bf16(r0, r1);
        lo[u] = cvt2_bf16(r0 - __uint_as_float(mid[u] << 16), r1 - __uint_as_float(mid[u] & 0xFFFF0000u));
      }
      *reinterpret_cast<uint4*>(limbs + h * L::LROW + 16 * c8) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
      *reinterpret_cast<uint4*>(limbs + (G + h) * L::LROW + 16 * c8) = make_uint4(mid[0], mid[1], mid[2], mid[3]);
      *reinterpret_cast<uint4*>(limbs + (2 * G + h) * L::LROW + 16 * c8) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
    }
    __syncthreads();
  } else {
  // ---- prologue ----
  // q (straight into the split entries) and the S^T fragments are requested
  // first; the first tile is requested once q is split (or, in the S^T q
  // waves of eight-wave workgroups at m = 256, once S^T q is done), so that q
  // does not queue behind the whole chip's tile traffic.
  // S^T q runs on the first SQW waves only: with eight waves, the younger
  // four would reach it only after their (lower-priority) tile requests,
  // holding up the whole workgroup.
  constexpr int SQW = NW < 4 ? NW : 4;
  constexpr int NBLK = M / 32;            // blocks of 32 sketch coordinates
  constexpr int BPW = NBLK / SQW;         // blocks per S^T q wave
  static_assert(NBLK % SQW == 0, "sketch blocks must divide among the waves");
  static_assert(8 * 2 * 32 % NT == 0, "q entries must divide among the threads");
  const int col = lane & 31;
  const int half = lane >> 5;
  // q entry e = (k-step st, half hf, column c): q[head][16 st + 8 hf .. +7],
  // column c = part * G + head (columns >= 3G are zero); every entry loads
  // (the head index is valid for any c), so the loads need no branch.
  constexpr int QE = 8 * 2 * 32;
  constexpr int QEPT = QE / NT;
  const float* qb = q + bh * G * D;
  float4 qa[QEPT][2];
#pragma unroll
  for (int k = 0; k < QEPT; ++k) {
    const int e = tid + k * NT;
    const int c = e & 31, st = e >> 6, hf = (e >> 5) & 1;
    const float4* src = reinterpret_cast<const float4*>(qb + (c % G) * D + 16 * st + 8 * hf);
    qa[k][0] = src[0];
    qa[k][1] = src[1];
  }
  // S^T comes in fragment order (see DeviceSketch::s_frag): the operand of
  // (block, k-step) is 64 lanes x 16 contiguous bytes, one 1 KB load.
  uint4 af[BPW][8];
  if (wave < SQW)
#pragma unroll
  for (int bb = 0; bb < BPW; ++bb) {
    const int blk = wave + SQW * bb;
    const uint4* fr = reinterpret_cast<const uint4*>(s_frag) + static_cast<int64_t>(blk) * 8 * 64 + lane;
#pragma unroll
    for (int st = 0; st < 8; ++st) af[bb][st] = fr[st * 64];
  }

  // limb rows >= 3G and probability rows >= 2G stay zero; the sums of Q
  // start at zero
  constexpr int ZERO_U4 = (16 * NSQ - 3 * G) * L::LROW / 16;
  for (int i = tid; i < ZERO_U4; i += NT)
    reinterpret_cast<uint4*>(limbs + 3 * G * L::LROW)[i] = make_uint4(0, 0, 0, 0);
  for (int i = tid; i < L::P_BYTES / 16; i += NT) reinterpret_cast<uint4*>(p_all)[i] = make_uint4(0, 0, 0, 0);
  if (tid < G) sumq[tid] = 0;

  // q -> three bf16 parts (hi + mid + lo equals fp32 q to within 2^-24
  // relative), laid out as the MFMA B operand: column c = part * G + head.
#pragma unroll
  for (int k = 0; k < QEPT; ++k) {
    const int e = tid + k * NT;
    const int c = e & 31;
    const int part = c / G;
    const float x[8] = {qa[k][0].x, qa[k][0].y, qa[k][0].z, qa[k][0].w,
                        qa[k][1].x, qa[k][1].y, qa[k][1].z, qa[k][1].w};
    uint32_t pk[4];
    float ss = 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float x0 = x[2 * u], x1 = x[2 * u + 1];
      ss = __builtin_fmaf(x0, x0, ss);
      ss = __builtin_fmaf(x1, x1, ss);
      const uint32_t hi = cvt2_bf16(x0, x1);
      const float r0 = x0 - __uint_as_float(hi << 16), r1 = x1 - __uint_as_float(hi & 0xFFFF0000u);
      const uint32_t mid = cvt2_bf16(r0, r1);
      const uint32_t lo = cvt2_bf16(r0 - __uint_as_float(mid << 16), r1 - __uint_as_float(mid & 0xFFFF0000u));
      pk[u] = part == 0 ? hi : (part == 1 ? mid : (part == 2 ? lo : 0u));
    }
    qfrag[e] = make_uint4(pk[0], pk[1], pk[2], pk[3]);
    if (c < G) qss[c * 16 + (e >> 5)] = ss;   // e >> 5 = 2 st + hf
  }
  __syncthreads();
  // The first tile.  With eight waves at m = 256 the S^T q waves request
  // theirs after S^T q, so that a tile request held up by the chip-wide
  // start-up traffic does not hold up S^T q (and with it every wave's first
  // tile), while the other four waves keep the memory busy (measured: 32K
  // 20.65 -> 20.1 us; at m = 512, and with four waves, requesting before S^T q
  // measured faster).  With m = 512 the S^T fragments fill half the
  // registers: the second half of the first tile's values is requested
  // after S^T q in every wave.
  constexpr bool kLateTile = M == 256 && NW > SQW;
  auto first_tile = [&]() {
    load_signs(t0, sw, nv);
    load_values(t0, std::integral_constant<int, 0>{});
    if constexpr (M == 256) load_values(t0, std::integral_constant<int, 1>{});
  };
  if ((!kLateTile || wave >= SQW) && !defer_first) first_tile();

  // quantization step 2^E of head h: 2^(E + 21) exceeds ||q_h|| max_i ||s_i||
  // (with margin for the rounding of S^T q and of the norm itself)
  auto head_exp = [&](int h) -> int {
    const float4* p = reinterpret_cast<const float4*>(qss + h * 16);
    const float4 a0 = p[0], a1 = p[1], a2 = p[2], a3 = p[3];
    const float s = ((a0.x + a0.y) + (a0.z + a0.w)) + ((a1.x + a1.y) + (a1.z + a1.w)) +
                    ((a2.x + a2.y) + (a2.z + a2.w)) + ((a3.x + a3.y) + (a3.z + a3.w));
    const float bound = __builtin_sqrtf(s) * cnmax * (1.0f + 0x1p-10f) + 0x1p-100f;
    int e = __builtin_amdgcn_frexp_expf(bound);   // bound < 2^e
    e -= QBITS;
    return min(100, max(-100, e));
  };

  // Exponents of all heads, and of the head of this lane's S^T q columns
  // (col % G); taken here because the q^2 sums share LDS with the value tiles.
#pragma unroll
  for (int h = 0; h < G; ++h) e_all[h] = __builtin_amdgcn_readfirstlane(head_exp(h));
  const int e_h = head_exp(col % G);

  // S^T q on the matrix cores, then its limbs.  Lane (col, half), register r
  // of block blk holds coordinate 32 blk + 8 (r/4) + 4 half + r%4.
  if (wave < SQW) {
    const float inv_s = __builtin_ldexpf(1.0f, -e_h);
    int qsum = 0;
#pragma unroll
    for (int bb = 0; bb < BPW; ++bb) {
      const int blk = wave + SQW * bb;
      f32x16_t acc = {};
#pragma unroll
      for (int st = 0; st < 8; ++st)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, af[bb][st]),
                                                      __builtin_bit_cast(bf16x8_t, qfrag[(st * 2 + half) * 32 + col]),
                                                      acc, 0, 0, 0);
      // limb p of coordinate 32 blk + 8 a4 + 4 half + i goes to byte
      // 32 blk + 16 half + 4 i + a4 of its row (the order in which the score
      // loop spreads a sign word: byte b of register q takes bit 8 b + q)
      uint32_t pk[3][4] = {};
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 4 * a4 + i;
          float v;
          if (G < 8) {   // columns col + G and col + 2G lie in the same 16-lane row
            v = acc[r] + dpp<kRowShl + G>(acc[r]) + dpp<kRowShl + 2 * G>(acc[r]);
          } else {
            v = acc[r] + __shfl(acc[r], lane + G) + __shfl(acc[r], lane + 2 * G);
          }
          int Q = static_cast<int>(__builtin_rintf(v * inv_s));
          Q = min(1 << QBITS, max(-(1 << QBITS), Q));
          qsum += Q;
          const int c0 = ((Q + 128) & 255) - 128;
          const int q1 = (Q - c0) >> 8;
          const int c1 = ((q1 + 128) & 255) - 128;
          const int c2 = (q1 - c1) >> 8;
          pk[0][i] |= (static_cast<uint32_t>(c2) & 255u) << (8 * a4);
          pk[1][i] |= (static_cast<uint32_t>(c1) & 255u) << (8 * a4);
          pk[2][i] |= (static_cast<uint32_t>(c0) & 255u) << (8 * a4);
        }
      }
      if (col < G) {
#pragma unroll
        for (int p = 0; p < 3; ++p)
          *reinterpret_cast<uint4*>(limbs + (p * G + col) * L::LROW + 32 * blk + 16 * half) =
              make_uint4(pk[p][0], pk[p][1], pk[p][2], pk[p][3]);
      }
    }
    if (col < G) atomicAdd(&sumq[col], qsum);
    if constexpr (kLateTile) {
      if (!defer_first) first_tile();
    }
  }
  if constexpr (M != 256) {
    if (!defer_first) load_values(t0, std::integral_constant<int, 1>{});
  }
  if constexpr (APPEND) {
    // the last four waves (idle during S^T q in eight-wave workgroups)
    if (app_wg && wave >= NW - 4) append_token<M>(app, bh, cap, tid - (NW - 4) * 64, cnmax, app_scratch);
  }
  __syncthreads();
  if constexpr (APPEND) {
    if (defer_first) {
      load_signs(t0, sw, nv);
      load_values(t0, std::integral_constant<int, 0>{});
      load_values(t0, std::integral_constant<int, 1>{});
    }
  }

  }

  // ---- main loop setup ----
  // Per head: logit (base 2) = (kap[h] * sum_i b_i Q_i + bet[h]) * ||k||,
  // kap = 2 coef 2^E, bet = -coef 2^E sum_i Q_i.
  float kap[G], bet[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float s_h = __builtin_ldexpf(1.0f, e_all[h]);
    kap[h] = uniform(2.0f * coef * s_h);
    bet[h] = uniform(-coef * s_h * static_cast<float>(__builtin_amdgcn_readfirstlane(sumq[h])));
  }
  // A operand of the score product: limb row 16 cb + l16, coordinates
  // (M/4) grp + 16 ks .. +15
  const uint8_t* brow[NSQ];
#pragma unroll
  for (int cb = 0; cb < NSQ; ++cb)
    brow[cb] = limbs + (16 * cb + l16) * L::LROW + (BF16K ? 16 * grp : (M / 4) * grp);
  // Score accumulator of block j: lane (grp, l16), register r holds limb row
  // 16 cb + 4 grp + r (limb p = row / G, head row % G) for token 16 j + l16.
  // Rows are weighted 2^16, 2^8, 1 by limb, then summed over the lane
  // groups so that group g keeps block g: each lane ends with its token
  // t0 + lane and all G heads.
  const uint32_t sh_grp = grp == 0 ? 16u : (grp == 1 ? 8u : 0u);    // G = 4: limb = grp
  const uint32_t sh_g2 = grp == 0 ? 16u : 0u;                         // G = 2: rows h, 4 + h
  const uint32_t sh_g8 = grp < 2 ? 16u : 8u;                          // G = 8: limb 0 or 1
  const int odd_mask = -(grp & 1);                                    // G = 8: heads 4..7 rows

  float m_run[G], l_run[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m_run[h] = -INFINITY;
    l_run[h] = 0.f;
  }
  f32x4_t acc[NDB];
#pragma unroll
  for (int nb = 0; nb < NDB; ++nb) acc[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // transposed-read sources: lane s of group grp addresses token 4 grp + s/4
  // of the half tile (first read) and 16 + 4 grp + s/4 (second read), at
  // columns 4 (s%4) .. +3 of a 16-column block (values) or rows 4 (s%4) .. +3
  // of the probability rows.  With 288-byte value rows (32-byte probability
  // rows) the 8 rows touched by each 32 lanes fall on distinct banks.
  const uint8_t* tr_base0 = vbuf + (4 * grp + (l16 >> 2)) * VROW + 8 * (lane & 3);
  const uint8_t* tr_base1 = tr_base0 + 16 * VROW;
  const uint8_t* pr_base0 = pbuf + (4 * grp + (l16 >> 2)) * PROW + 8 * (lane & 3);
  const uint8_t* pr_base1 = pr_base0 + 16 * PROW;

  auto body = [&](auto prefetch_const) {
    constexpr bool PF = decltype(prefetch_const)::value;
    const int t_next = t0 + NW * TILE;
    uint32_t swn[4][CW];
    float nvn = 0.f;
    if constexpr (PF && !BF16K) load_signs(t_next, swn, nvn);
    float logit[G];
    if constexpr (BF16K) {
      // scores: block j, q-row set cb (A = q parts, B = key rows)
      f32x4_t fsacc[NSQ][4];
#pragma unroll
      for (int cb = 0; cb < NSQ; ++cb)
#pragma unroll
        for (int j = 0; j < 4; ++j) fsacc[cb][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        bf16x8_t lop[NSQ];
#pragma unroll
        for (int cb = 0; cb < NSQ; ++cb) lop[cb] = *reinterpret_cast<const bf16x8_t*>(brow[cb] + 64 * ks);
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int cb = 0; cb < NSQ; ++cb)
            fsacc[cb][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                lop[cb], __builtin_bit_cast(bf16x8_t, kc[4 * j + ks]), fsacc[cb][j], 0, 0, 0);
      }
      if constexpr (PF) load_keys(t_next);   // the next tile's keys reuse kc
      // q . k of token t0 + lane per head: the three part rows summed, with
      // the same reduce-scatter as the integer scores (weights 1)
      if constexpr (G == 1) {
        float x[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = fsacc[0][j][0] + fsacc[0][j][1] + fsacc[0][j][2];
        logit[0] = reduce_scatter4f(x[0], x[1], x[2], x[3]);
      } else if constexpr (G == 2) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          float x[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) x[j] = fsacc[0][j][h] + fsacc[0][j][2 + h];
          logit[h] = reduce_scatter4f(x[0], x[1], x[2], x[3]);
        }
      } else if constexpr (G == 4) {
#pragma unroll
        for (int h = 0; h < 4; ++h)
          logit[h] = reduce_scatter4f(fsacc[0][0][h], fsacc[0][1][h], fsacc[0][2][h], fsacc[0][3][h]);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          uint32_t z[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) z[j] = __float_as_uint(fsacc[0][j][r] + fsacc[1][j][r]);
          const auto a01 = __builtin_amdgcn_permlane32_swap(z[0], z[1], false, false);
          const auto a23 = __builtin_amdgcn_permlane32_swap(z[2], z[3], false, false);
          const auto c = __builtin_amdgcn_permlane32_swap(
              __float_as_uint(__uint_as_float(a01[0]) + __uint_as_float(a01[1])),
              __float_as_uint(__uint_as_float(a23[0]) + __uint_as_float(a23[1])), false, false);
          const auto dd = __builtin_amdgcn_permlane16_swap(c[0], c[1], false, false);
          logit[r] = __uint_as_float(dd[0]);
          logit[4 + r] = __uint_as_float(dd[1]);
        }
      }
#pragma unroll
      for (int h = 0; h < G; ++h) logit[h] *= coef;
    } else {
      // scores: block j, limb-row set cb (A = limbs, B = token bits)
      i32x4_t sacc[NSQ][4];
#pragma unroll
      for (int cb = 0; cb < NSQ; ++cb)
#pragma unroll
        for (int j = 0; j < 4; ++j) sacc[cb][j] = i32x4_t{0, 0, 0, 0};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        i32x4_t lop[NSQ];
#pragma unroll
        for (int cb = 0; cb < NSQ; ++cb) lop[cb] = *reinterpret_cast<const i32x4_t*>(brow[cb] + 16 * ks);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t w = sw[j][ks >> 1];
          // register qd, byte b: bit 8 b + 4 (ks % 2) + qd of the word (the
          // limbs were stored in this order)
          i32x4_t bits;
#pragma unroll
          for (int qd = 0; qd < 4; ++qd) bits[qd] = static_cast<int>((w >> (4 * (ks & 1) + qd)) & 0x01010101u);
#pragma unroll
          for (int cb = 0; cb < NSQ; ++cb)
            sacc[cb][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(lop[cb], bits, sacc[cb][j], 0, 0, 0);
        }
      }
      // sum_i b_i Q_i of token t0 + lane, per head
      int tot[G];
      auto u = [](int x) { return static_cast<uint32_t>(x); };
      if constexpr (G == 1) {
        int x[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          x[j] = static_cast<int>((u(sacc[0][j][0]) << 16) + (u(sacc[0][j][1]) << 8) + u(sacc[0][j][2]));
        tot[0] = reduce_scatter4(x[0], x[1], x[2], x[3]);
      } else if constexpr (G == 2) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          int x[4];
#pragma unroll
          for (int j = 0; j < 4; ++j)
            x[j] = static_cast<int>((u(sacc[0][j][h]) << sh_g2) + (u(sacc[0][j][2 + h]) << 8));
          tot[h] = reduce_scatter4(x[0], x[1], x[2], x[3]);
        }
      } else if constexpr (G == 4) {
#pragma unroll
        for (int h = 0; h < 4; ++h)
          tot[h] = reduce_scatter4(static_cast<int>(u(sacc[0][0][h]) << sh_grp), static_cast<int>(u(sacc[0][1][h]) << sh_grp),
                                   static_cast<int>(u(sacc[0][2][h]) << sh_grp), static_cast<int>(u(sacc[0][3][h]) << sh_grp));
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          int z[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) z[j] = static_cast<int>((u(sacc[0][j][r]) << sh_g8) + u(sacc[1][j][r]));
          const auto a01 = __builtin_amdgcn_permlane32_swap(z[0], z[1], false, false);
          const auto a23 = __builtin_amdgcn_permlane32_swap(z[2], z[3], false, false);
          const auto c = __builtin_amdgcn_permlane32_swap(a01[0] + a01[1], a23[0] + a23[1], false, false);
          const auto d = __builtin_amdgcn_permlane16_swap(c[0], c[1], false, false);
          tot[r] = static_cast<int>(d[0]);
          tot[4 + r] = static_cast<int>(d[1]);
        }
      }
#pragma unroll
      for (int h = 0; h < G; ++h) logit[h] = __builtin_fmaf(static_cast<float>(tot[h]), kap[h], bet[h]) * nv;
    }
    // online softmax per head (maxima and rescale factors are wave-uniform)
    const bool live = PF || (t0 + lane < t_end);
    float p[G], al[G], tmax[G];
#pragma unroll
    for (int h = 0; h < G; ++h) p[h] = live ? logit[h] : -INFINITY;
    if constexpr (G == 1) {
      tmax[0] = wave_max(p[0]);
    } else {
      wave_max_heads<G>(p, tmax);
    }
    bool rescale = false;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float m_new = fmaxf(m_run[h], tmax[h]);
      rescale |= m_new > m_run[h];
      al[h] = uniform(__builtin_amdgcn_exp2f(m_run[h] - m_new));
      m_run[h] = m_new;
      p[h] = __builtin_amdgcn_exp2f(p[h] - m_new);
      l_run[h] = __builtin_fmaf(l_run[h], al[h], p[h]);
    }
    // probabilities of this token as bf16 hi (rows 0..G-1) and lo (rows
    // G..2G-1) parts; rows 2G..15 stay zero
    {
      uint32_t hi[(G + 1) / 2], lo[(G + 1) / 2];
#pragma unroll
      for (int i = 0; i < (G + 1) / 2; ++i) {
        const float p0 = p[2 * i], p1 = 2 * i + 1 < G ? p[2 * i + 1] : 0.f;
        hi[i] = cvt2_bf16(p0, p1);
        lo[i] = cvt2_bf16(p0 - __uint_as_float(hi[i] << 16), p1 - __uint_as_float(hi[i] & 0xFFFF0000u));
      }
      uint8_t* prow = pbuf + lane * PROW;
      if constexpr (G == 1) {
        *reinterpret_cast<uint32_t*>(prow) = (hi[0] & 0xFFFFu) | (lo[0] << 16);
      } else if constexpr (G == 2) {
        *reinterpret_cast<uint2*>(prow) = make_uint2(hi[0], lo[0]);
      } else if constexpr (G == 4) {
        *reinterpret_cast<uint4*>(prow) = make_uint4(hi[0], hi[1], lo[0], lo[1]);
      } else {
        *reinterpret_cast<uint4*>(prow) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
        *reinterpret_cast<uint4*>(prow + 16) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
      }
    }
    // rescale the running output (only when some head's maximum rose):
    // accumulator row 4 grp + r belongs to head (4 grp + r) % G
    if (rescale)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float a;
      if constexpr (G <= 4) {
        a = al[r % G];
      } else {   // bitwise select (a conditional here becomes an indexed private array)
        a = __int_as_float((__float_as_int(al[4 + r]) & odd_mask) | (__float_as_int(al[r]) & ~odd_mask));
      }
#pragma unroll
      for (int nb = 0; nb < NDB; ++nb) acc[nb][r] *= a;
    }

    // P.V for tokens 32*HS .. +31 of the tile (HS = 0, 1 as constants, so the
    // value registers are addressed statically)
    auto pv_half = [&](auto hs_const) {
      constexpr int hstep = decltype(hs_const)::value;
      // value rows 32*hstep .. +31 of the tile -> wave-private LDS tile
#pragma unroll
      for (int u8 = 0; u8 < 8; ++u8)
        *reinterpret_cast<uint4*>(vbuf + (4 * u8 + grp) * VROW + l16 * 16) = vc[8 * hstep + u8];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      if constexpr (PF) load_values(t_next, hs_const);
      // A operand: probability rows, tokens as for the value reads
      const i16x4_t pa0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4_t*)(pr_base0 + 32 * PROW * hstep));
      const i16x4_t pa1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4_t*)(pr_base1 + 32 * PROW * hstep));
      const uint2 pl = __builtin_bit_cast(uint2, pa0);
      const uint2 ph = __builtin_bit_cast(uint2, pa1);
      const bf16x8_t a_op = __builtin_bit_cast(bf16x8_t, make_uint4(pl.x, pl.y, ph.x, ph.y));
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

    if constexpr (PF) {
      t0 = t_next;
      if constexpr (!BF16K) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int w = 0; w < CW; ++w) sw[j][w] = swn[j][w];
        nv = nvn;
      }
    }
  };
  if (t0 < t_end) {
    while (t0 + NW * TILE < t_end) body(std::true_type{});
    body(std::false_type{});
  }

  // ---- wave result: out row = hi row + lo row, into this wave's LDS tile ----
#pragma unroll
  for (int h = 0; h < G; ++h) l_run[h] = wave_sum(l_run[h]);
  // Accumulator block nb: lane l holds row 4*(l/16) + r, column l%16.  Row g
  // (hi part of head g) pairs with row G + g (lo part): for G >= 4 the lo row
  // sits G/4 lane groups later in the same register; for G < 4 both rows are
  // registers of lanes 0..15.
  float* wacc = reinterpret_cast<float*>(vbuf);   // [G][D]
  if constexpr (G >= 4) {
    // a 16-lane (G = 4) or 32-lane (G = 8) row swap brings each lo row next
    // to its hi row (VALU, no LDS round trip)
    float v[NDB][4];
#pragma unroll
    for (int nb = 0; nb < NDB; ++nb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t x = __float_as_uint(acc[nb][r]);
        const auto t = G == 4 ? __builtin_amdgcn_permlane16_swap(x, x, false, false)
                              : __builtin_amdgcn_permlane32_swap(x, x, false, false);
        v[nb][r] = __uint_as_float(t[0]) + __uint_as_float(t[1]);
      }
    if (grp < G / 4)
#pragma unroll
      for (int nb = 0; nb < NDB; ++nb)
#pragma unroll
        for (int r = 0; r < 4; ++r) wacc[(4 * grp + r) * D + 16 * nb + l16] = v[nb][r];
  } else if (grp == 0) {
#pragma unroll
    for (int nb = 0; nb < NDB; ++nb)
#pragma unroll
      for (int r = 0; r < G; ++r) wacc[r * D + 16 * nb + l16] = acc[nb][r] + acc[nb][r + G];
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      red_ml[wave][h][0] = m_run[h];
      red_ml[wave][h][1] = l_run[h];
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
        __hip_atomic_fetch_add(&counters[bh * cstride], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    is_last = (prev == static_cast<uint32_t>(n_split - 1));
  }
  __syncthreads();
  if (!is_last) return;

  // The partials are read with device-coherent (sc1) loads, the load side of
  // the coherent stores above: each reads the value at the device's
  // coherence point, and every store it must see completed before its
  // workgroup counted in, which happened before this workgroup's count
  // returned.  No cache invalidation is needed (an acquire fence would drop
  // the whole L2 of this XCD).
  // Threads own (head, 4 channels) pairs; with fewer pairs than threads the
  // splits are divided among REP replicas whose sums meet in LDS.  The
  // (max, sum) pairs and the first MCH partial accumulators of every thread
  // are requested together, so the merge costs one round trip to memory.
  constexpr int PAIRS = L::PAIRS;
  constexpr int REP = L::REP;
  constexpr int MCH = 32;                 // float4 loads in flight per thread
  float* ml_l = reinterpret_cast<float*>(vb_all);   // 2 * n_split * G floats
  float* wts = ml_l + L::ML_FLOATS;                 // n_split * G floats
  float4* rep_sum = reinterpret_cast<float4*>(wts + L::WT_FLOATS);
  constexpr int kCoherent = 16;   // sc1: device-scope coherent access
  const rsrc_t ml_rs = make_rsrc(part_ml + bh * n_split * G * 2, n_split * G * 8);
  const rsrc_t pa_rs = make_rsrc(part_acc + bh * n_split * G * D, n_split * G * D * 4);
  constexpr int ML_PT = (MAX_SPLITS * G + NT - 1) / NT;
  float2 mlv[ML_PT];
#pragma unroll
  for (int k = 0; k < ML_PT; ++k) {
    const int i = tid + k * NT;
    if (i < n_split * G) {
      const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(ml_rs, i * 8, 0, kCoherent);
      mlv[k] = make_float2(__uint_as_float(v.x), __uint_as_float(v.y));
    }
  }
  const int pr = tid % PAIRS, rep = tid / PAIRS;       // valid when tid < PAIRS * REP
  const int mg = pr / (D / 4), c4 = pr % (D / 4);
  auto load_partial = [&](int s_) {   // float4 c4 of head mg of split s_
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(pa_rs, ((s_ * G + mg) * (D / 4) + c4) * 16, 0, kCoherent);
    return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w));
  };
  float4 av[MCH];
#pragma unroll
  for (int u = 0; u < MCH; ++u) {
    const int s = rep + u * REP;
    if (tid < PAIRS * REP && s < n_split) av[u] = load_partial(s);
  }
#pragma unroll
  for (int k = 0; k < ML_PT; ++k) {
    const int i = tid + k * NT;
    if (i < n_split * G) reinterpret_cast<float2*>(ml_l)[i] = mlv[k];
  }
  __syncthreads();
  // per head (one wave each): global max and normalizer, then the weight of
  // every split
  for (int g = wave; g < G; g += NW) {
    float mx = -INFINITY;
    for (int s = lane; s < n_split; s += 64) mx = fmaxf(mx, ml_l[(s * G + g) * 2]);
    mx = wave_max(mx);
    float Ls = 0.f;
    for (int s = lane; s < n_split; s += 64) Ls += ml_l[(s * G + g) * 2 + 1] * exp2f(ml_l[(s * G + g) * 2] - mx);
    Ls = wave_sum(Ls);
    for (int s = lane; s < n_split; s += 64) wts[s * G + g] = exp2f(ml_l[(s * G + g) * 2] - mx) / Ls;
  }
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
      const float4 v = load_partial(s);
      const float wgt = wts[s * G + mg];
      o.x = __builtin_fmaf(wgt, v.x, o.x);
      o.y = __builtin_fmaf(wgt, v.y, o.y);
      o.z = __builtin_fmaf(wgt, v.z, o.z);
      o.w = __builtin_fmaf(wgt, v.w, o.w);
    }
    if (REP == 1) {
      reinterpret_cast<float4*>(out)[(bh * G + mg) * (D / 4) + c4] = o;
    } else {
      rep_sum[rep * PAIRS + pr] = o;
    }
  }
  if (REP > 1) {
    __syncthreads();
    for (int p2 = tid; p2 < PAIRS; p2 += NT) {
      float4 o = rep_sum[p2];
      for (int r2 = 1; r2 < REP; ++r2) {
        const float4 v = rep_sum[r2 * PAIRS + p2];
        o.x += v.x;
        o.y += v.y;
        o.z += v.z;
        o.w += v.w;
      }
      const int g = p2 / (D / 4), cc = p2 % (D / 4);
      reinterpret_cast<float4*>(out)[(bh * G + g) * (D / 4) + cc] = o;
    }
  }
  if (tid == 0) __hip_atomic_store(&counters[bh * cstride], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int G, int NW>
int launch_decode_bf16_gw(const DecodePlan& plan, const float* q, const void* keys, const void* values,
                          int B, int H_kv, int N, int cap, float coef, float* out, void* workspace,
                          hipStream_t stream) {
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  uint32_t* counters = reinterpret_cast<uint32_t*>(ws);
  float* part_acc = reinterpret_cast<float*>(ws + plan.counter_bytes);
  float* part_ml = part_acc + static_cast<size_t>(B) * H_kv * G * plan.n_split * D;
  dim3 grid(plan.n_split, H_kv, B);
  hipLaunchKernelGGL((decode_kernel<256, G, NW, false, true>), grid, dim3(64 * NW), 0, stream, q,
                     nullptr, nullptr, static_cast<const uint16_t*>(values), nullptr, 0.f, H_kv, N, cap,
                     plan.n_split, plan.tokens_per_split, coef, out, counters, counter_stride(B, H_kv), part_acc, part_ml,
                     AppendArgs{}, static_cast<const uint16_t*>(keys));
  return hipGetLastError();
}

template <int G>
int launch_decode_bf16_g(const DecodePlan& plan, const float* q, const void* keys, const void* values,
                         int B, int H_kv, int N, int cap, float coef, float* out, void* workspace,
                         hipStream_t stream) {
  if (plan.waves == 8)
    return launch_decode_bf16_gw<G, 8>(plan, q, keys, values, B, H_kv, N, cap, coef, out, workspace, stream);
  return launch_decode_bf16_gw<G, 4>(plan, q, keys, values, B, H_kv, N, cap, coef, out, workspace, stream);
}

template <int M, int G, int NW>
int launch_decode_mgw(const DeviceSketch& s, const DecodePlan& plan, const float* q,
                      const uint32_t* signs, const float* norms, const void* values, int B,
                      int H_kv, int N, int cap, float coef, float* out, void* workspace,
                      const AppendArgs* app, hipStream_t stream) {
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  uint32_t* counters = reinterpret_cast<uint32_t*>(ws);
  float* part_acc = reinterpret_cast<float*>(ws + plan.counter_bytes);
  float* part_ml = part_acc + static_cast<size_t>(B) * H_kv * G * plan.n_split * D;
  dim3 grid(plan.n_split, H_kv, B);
  const uint16_t* v = static_cast<const uint16_t*>(values);
  if (app != nullptr) {
    hipLaunchKernelGGL((decode_kernel<M, G, NW, true>), grid, dim3(64 * NW), 0, stream, q, signs, norms,
                       v, s.s_frag, s.col_norm_all, H_kv, N, cap, plan.n_split, plan.tokens_per_split,
                       coef, out, counters, counter_stride(B, H_kv), part_acc, part_ml, *app, nullptr);
  } else {
    hipLaunchKernelGGL((decode_kernel<M, G, NW, false>), grid, dim3(64 * NW), 0, stream, q, signs, norms,
                       v, s.s_frag, s.col_norm_all, H_kv, N, cap, plan.n_split, plan.tokens_per_split,
                       coef, out, counters, counter_stride(B, H_kv), part_acc, part_ml, AppendArgs{}, nullptr);
  }
  return hipGetLastError();
}

template <int M, int G>
int launch_decode_mg(const DeviceSketch& s, const DecodePlan& plan, const float* q,
                     const uint32_t* signs, const float* norms, const void* values, int B,
                     int H_kv, int N, int cap, float coef, float* out, void* workspace,
                     const AppendArgs* app, hipStream_t stream) {
  if (plan.waves == 8)
    return launch_decode_mgw<M, G, 8>(s, plan, q, signs, norms, values, B, H_kv, N, cap, coef, out, workspace, app, stream);
  return launch_decode_mgw<M, G, 4>(s, plan, q, signs, norms, values, B, H_kv, N, cap, coef, out, workspace, app, stream);
}

template <int M>
int launch_decode_m(int G, const DeviceSketch& s, const DecodePlan& plan, const float* q,
                    const uint32_t* signs, const float* norms, const void* values, int B,
                    int H_kv, int N, int cap, float coef, float* out, void* workspace,
                    const AppendArgs* app, hipStream_t st) {
  switch (G) {
    case 1: return launch_decode_mg<M, 1>(s, plan, q, signs, norms, values, B, H_kv, N, cap, coef, out, workspace, app, st);
    case 2: return launch_decode_mg<M, 2>(s, plan, q, signs, norms, values, B, H_kv, N, cap, coef, out, workspace, app, st);
    case 4: return launch_decode_mg<M, 4>(s, plan, q, signs, norms, values, B, H_kv, N, cap, coef, out, workspace, app, st);
    case 8: return launch_decode_mg<M, 8>(s, plan, q, signs, norms, values, B, H_kv, N, cap, coef, out, workspace, app, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

namespace {
// Context splits for workgroups of nw waves: at most about 2048 / nw
// workgroups (every compute unit busy, none left for a second round: with 40
// streams, 7 splits made 280 eight-wave workgroups for 256 compute units and
// took 48.2 us at 16K, 6 splits 35.3 us), at least one full step (nw x 64
// tokens) per split, splits only for few streams.  With four waves a stream
// count just above the target still gets two splits (320 streams at 16K:
// 237 us with two, 265 us with one).
// target: workgroups wanted at eight waves each (twice as many at four)
void split_plan(int64_t streams, int N, int nw, int64_t target8, int64_t* n_split, int64_t* tps) {
  const int64_t target = target8 * 8 / nw;
  const int min_tokens = nw * TILE;
  int64_t want = target / streams;
  if (nw == 4 && want < 2) want = (target + streams - 1) / streams;
  if (streams > kMaxCounters) want = 1;   // splits (and counters) only for few streams
  const int64_t most = (N + min_tokens - 1) / min_tokens;
  if (want > most) want = most;
  if (want > MAX_SPLITS) want = MAX_SPLITS;
  if (want < 1) want = 1;
  int64_t t = (N + want - 1) / want;
  t = (t + TILE - 1) / TILE * TILE;
  *tps = t;
  *n_split = (N + t - 1) / t;
}
}  // namespace

bool make_decode_plan(int B, int H_q, int H_kv, int N, int d, int m, DecodePlan* plan) {
  if (B <= 0 || H_q <= 0 || H_kv <= 0 || N <= 0 || d != D || (m != 256 && m != 512)) return false;
  if (H_q % H_kv) return false;
  const int64_t streams = static_cast<int64_t>(B) * H_kv;
  // Eight-wave workgroups (one per compute unit) when the context must be
  // split into at least 64 workgroups: half the S^T fragment traffic per
  // compute unit and half the partials to merge (and half the arrivals on
  // each counter, which serialize when every workgroup has a single tile:
  // 8K tokens of 8 kv heads took 15.2 us with 256 four-wave workgroups and
  // 13.8 us with 128 eight-wave ones).  Otherwise four waves.
  // At m = 512 each workgroup also reads twice the S^T fragments: slightly
  // fewer, longer splits (240 rather than 256 workgroups) measured faster.
  const int64_t target8 = m == 512 ? 240 : 256;
  int64_t n_split = 0, tps = 0;
  split_plan(streams, N, 8, target8, &n_split, &tps);
  int waves = 8;
  if (!(n_split > 1 && streams * n_split >= 64)) {
    waves = 4;
    split_plan(streams, N, 4, target8, &n_split, &tps);
  }
  plan->waves = waves;
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

namespace {
// Plan of a decode step that appends a token.  The workgroup whose range
// holds the new token (always the last split) appends it in its prologue,
// about 1.6 us of work the other workgroups do not have; with a full last
// split it ends that much later and holds up the merge (32K: 21.8 us against
// 19.9 us for the plain decode).  Where a split gives each wave at least two
// tiles, fewer splits are taken, one at a time and at most an eighth fewer,
// until the last split is at least one tile per wave shorter than the
// others.  The plan never gains splits, so the plain plan's workspace fits.
DecodePlan append_plan(const DecodePlan& plan, int N) {
  DecodePlan p = plan;
  const int shorter = plan.waves * TILE;
  if (plan.n_split < 2 || plan.tokens_per_split < 2 * shorter) return p;
  for (int64_t want = plan.n_split; want >= 2 && want >= plan.n_split - plan.n_split / 8; --want) {
    const int64_t t = ((N + want - 1) / want + TILE - 1) / TILE * TILE;
    const int64_t n = (N + t - 1) / t;
    if (n > 1 && N - (n - 1) * t <= t - shorter) {
      p.n_split = static_cast<int>(n);
      p.tokens_per_split = static_cast<int>(t);
      break;
    }
  }
  return p;
}
}  // namespace

int launch_decode(const DeviceSketch& s, const DecodePlan& plan_in, const float* q,
                  const uint32_t* signs, const float* norms, const void* values, int B, int H_q,
                  int H_kv, int N, int cap, float scale, float* out, void* workspace,
                  const AppendArgs* app, void* stream) {
  const int G = H_q / H_kv;
  const DecodePlan plan = app != nullptr ? append_plan(plan_in, N) : plan_in;
  // logits are kept in base 2: coef = sqrt(pi/2)/m * scale * log2(e)
  const double c = 1.2533141373155002512 / s.m * static_cast<double>(scale) * 1.4426950408889634074;
  const float coef = static_cast<float>(c);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (s.m == 256)
    return launch_decode_m<256>(G, s, plan, q, signs, norms, values, B, H_kv, N, cap, coef, out, workspace, app, st);
  return launch_decode_m<512>(G, s, plan, q, signs, norms, values, B, H_kv, N, cap, coef, out, workspace, app, st);
}

int launch_decode_bf16(const DecodePlan& plan, const float* q, const void* keys, const void* values,
                       int B, int H_q, int H_kv, int N, int cap, float scale, float* out,
                       void* workspace, void* stream) {
  const int G = H_q / H_kv;
  // logits in base 2: scale * log2(e) * q . k
  const float coef = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634074);
  hipStream_t st = static_cast<hipStream_t>(stream);
  switch (G) {
    case 1: return launch_decode_bf16_g<1>(plan, q, keys, values, B, H_kv, N, cap, coef, out, workspace, st);
    case 2: return launch_decode_bf16_g<2>(plan, q, keys, values, B, H_kv, N, cap, coef, out, workspace, st);
    case 4: return launch_decode_bf16_g<4>(plan, q, keys, values, B, H_kv, N, cap, coef, out, workspace, st);
    case 8: return launch_decode_bf16_g<8>(plan, q, keys, values, B, H_kv, N, cap, coef, out, workspace, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qjl
