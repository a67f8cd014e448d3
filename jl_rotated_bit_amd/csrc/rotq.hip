// Rotate-then-quantize key encoders for gfx950: TurboQuant_prod and
// PolarQuant, plus TurboQuant's inner-product scores.
//
// "The Geometry of Forgetting: How Three Papers Cracked KV Cache
// Quantization":
// * section "TurboQuant: bridging MSE and inner product, in two stages":
//   rotate the (unit) key by a random rotation, quantize every coordinate
//   with the Lloyd-Max codebook of the rotated-coordinate density (b - 1
//   bits), then spend one bit per coordinate on QJL of the residual; the
//   estimate of <q, k> adds the QJL estimate of <q, residual> to
//   <q, reconstruction> and is unbiased;
// * section "PolarQuant: skipping Cartesian altogether": rotate, transform
//   recursively to polar form (pairs of coordinates, then pairs of radii),
//   store each angle's cell in its level's codebook and the radius.
//
// Every value that decides a code is defined exactly, so codes and bits
// are unique (the same definitions as the CPU oracle):
//   n   = fp32(sqrt(fp64 sum of k_j^2 in channel order));
//   y_i = the fp32 rounding (nearest even) of the exact sum_j Pi[i][j] k_j;
// TurboQuant: u = fp32(y / n) (0 for a zero key), idx = #{boundaries <= u},
//   r = fp32(u - c[idx]), g = fp32(sqrt(fp64 sum of r_i^2 in order)),
//   bit_l = [exact sum_i S[i][l] r_i >= 0];
// PolarQuant: level-1 pair cells by quadrant and fp64 comparisons
//   b' >= T a'; level-l cells by s_b >= T^2 s_a on fp64 tree sums of
//   squares; radius = fp32(sqrt(total)).
//
// Kernel design.  A workgroup (eight waves, one per CU: the tables fill most
// of the LDS) keeps Pi^T (fp32, 64 KB) and, for TurboQuant, S (bf16, 32 KB)
// in LDS for the whole launch and walks over tiles of 32 keys; the next
// tile's keys (one 16-byte chunk per thread) load into registers while the
// current tile is encoded.  The rotation y = K Pi^T, and TurboQuant's
// residual sketch S^T r, are fp64 products on the matrix cores
// (v_mfma_f64_16x16x4f64): every product of a bf16 key value or an fp32
// residual with an fp32 rotation entry or a bf16 sketch entry is exact in
// fp64, so a sum carries at most d roundings in whatever order the unit adds.
// Wave w computes keys 16 (w & 1) .. +15 against the 32 columns
// 32 (w >> 1) .. +31.  The fp32 rounding is certified: with
// E = 2 d 2^-53 ||k|| max_i ||Pi_i|| bounding the fp64 error, y = fp32(v + E)
// when that equals fp32(v - E); otherwise (about one value in 10^5) the lanes
// of the wave take turns recomputing their open sums exactly in a 576-bit
// integer accumulator and rounding from there.  The residual's QJL signs are
// certified the same way (the sign of the fp64 sum when it exceeds its error
// bound, else the exact integer sum).
// This file is compiled with -ffp-contract=off: every fp64/fp32 operation
// that feeds a decision rounds exactly as written.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "exact_sign.h"
#include "internal.h"

namespace qjl {
namespace {

constexpr int D = kHeadDim;      // 128
constexpr int TK = 32;           // keys per tile
constexpr int TKP = TK + 1;      // LDS row stride of the [channel][key] tile (odd: spreads banks)
constexpr int NT = 512;          // threads per workgroup (two waves per SIMD)
constexpr int NW = NT / 64;      // waves
constexpr int CB = D / 16 / (NW / 2);  // 16-column result blocks per wave (2)
constexpr int PQ_LEVELS = 7;     // log2(128)
constexpr int PQ_WORDS = 12;     // 64 * 4 + 63 * 2 = 382 bits
constexpr int PQ_MAXT = 8;       // thresholds per level (<= 2^3 - 1 or 2^bits/4 - 1)

// ---- exact fallbacks: 576-bit signed sums of fp32 x bf16 products ----
// A bf16 value is sk 2^(ek - 134) (sk < 2^8, ek >= 1) and an fp32 value
// sp 2^(ep - 150) (sp < 2^24); each product is the integer sk sp < 2^32
// times 2^(ek + ep - 284), added shifted by ek + ep - 2 bits, so the sum is
// N 2^-282 with N held as two 576-bit magnitudes (positive / negative terms).
__device__ __forceinline__ void add_product(uint32_t* pos, uint32_t* neg, uint32_t kb, float p) {
  const uint32_t up = __float_as_uint(p);
  uint32_t ek = (kb >> 7) & 0xFF, ep = (up >> 23) & 0xFF;
  const uint32_t sk = ek ? ((kb & 0x7F) | 0x80) : (kb & 0x7F);
  const uint32_t sp = ep ? ((up & 0x7FFFFF) | 0x800000) : (up & 0x7FFFFF);
  if (sk == 0 || sp == 0) return;
  ek = ek ? (ek > 254 ? 254 : ek) : 1;   // Inf/NaN inputs: undefined but in bounds
  ep = ep ? (ep > 254 ? 254 : ep) : 1;
  const uint32_t shift = ek + ep - 2;
  const uint64_t v = (static_cast<uint64_t>(sk) * sp) << (shift & 31);
  long_add(((kb >> 15) ^ (up >> 31)) & 1 ? neg : pos, static_cast<int>(shift >> 5), v);
}

// Sign of pos - neg (true for >= 0).
__device__ bool long_sign(const uint32_t* pos, const uint32_t* neg) {
  for (int i = ACC_WORDS - 1; i >= 0; --i)
    if (pos[i] != neg[i]) return pos[i] > neg[i];
  return true;
}

// fp32 rounding (nearest, ties to even) of (pos - neg) 2^-282.
__device__ float long_to_f32(uint32_t* pos, uint32_t* neg) {
  const bool nonneg = long_sign(pos, neg);
  uint32_t* a = nonneg ? pos : neg;
  const uint32_t* b = nonneg ? neg : pos;
  // a -= b (a >= b)
  uint64_t borrow = 0;
  for (int i = 0; i < ACC_WORDS; ++i) {
    const uint64_t t = static_cast<uint64_t>(a[i]) - b[i] - borrow;
    a[i] = static_cast<uint32_t>(t);
    borrow = (t >> 63) & 1;
  }
  int top = -1;
  for (int i = ACC_WORDS - 1; i >= 0 && top < 0; --i)
    if (a[i]) top = 32 * i + 31 - __builtin_clz(a[i]);
  if (top < 0) return 0.0f;
  // quantum of the result: 24 significant bits, or 2^-149 for subnormals
  // (bit 133 of N is 2^-149)
  const int q = max(top - 23, 133);
  auto bit = [&](int p) -> uint32_t { return p < 0 ? 0u : (a[p >> 5] >> (p & 31)) & 1u; };
  uint32_t mant = 0;
  for (int p = top; p >= q; --p) mant = (mant << 1) | bit(p);
  const uint32_t rbit = bit(q - 1);
  bool sticky = false;
  for (int p = q - 2; p >= 0 && !sticky; --p) sticky = bit(p) != 0;
  if (rbit && (sticky || (mant & 1u))) ++mant;
  const float r = __builtin_ldexpf(static_cast<float>(mant), q - 282);
  return nonneg ? r : -r;
}

__device__ __forceinline__ void long_clear(uint32_t* s) {
  for (int i = 0; i < 2 * ACC_WORDS; ++i) s[i] = 0;
}

// Tables of one launch (device pointers; see RotqTables in internal.h).
struct RotqArgs {
  const uint16_t* keys;     // bf16 [R][d] (this launch's rows)
  int R;                    // keys in this launch
  int n;                    // keys per (batch, kv head) of the call
  int cap, pos;
  uint32_t r0;              // global row of keys[0]
  const float* rotT;        // Pi^T [j][i] fp32
  const float* rot;         // Pi [i][j] fp32 (exact fallback rows)
  float rot_row_max;        // max_i ||Pi_i||, rounded up
  // TurboQuant
  const uint16_t* s_il;     // S [i][l] bf16 (i = coordinate, l = sketch row), m = d
  float s_col_max;          // max_l ||S[:, l]||, rounded up
  const float* cents;       // 2^k
  int k;
  uint32_t* codes;          // [rows][d k / 32]
  uint32_t* bits;           // [rows][d / 32]
  float* norms;
  float* gammas;
  // PolarQuant
  const float* pq_thr;      // [PQ_LEVELS][PQ_MAXT] tangent thresholds
  uint32_t* pq_codes;       // [rows][PQ_WORDS]
  float* radii;
  int margin_log2;          // test hook: widens both certificates by 2^margin_log2
};

__device__ __forceinline__ int64_t dest_row(uint32_t r, uint32_t un, int cap, int pos) {
  const uint32_t bh = r / un;
  return static_cast<int64_t>(bh) * cap + pos + (r - bh * un);
}

struct RotqLds {
  float rotT[D * D];               // 64 KB
  uint16_t s_il[D * D];            // 32 KB (TurboQuant)
  double kt[D * TKP];              // keys (then residuals), [j][t]: 33 KB
  float y[TK][D + 1];              // rotated keys
  double nsq[TK];                  // fp64 sums of squares
  float nrm[TK];
  uint8_t cell[TK][D];             // codes / level cells
  uint32_t qwords[TK][4];          // TurboQuant sign words
  uint32_t scratch[NT / 64][2 * ACC_WORDS];
  float thr[PQ_LEVELS * PQ_MAXT];  // PolarQuant thresholds
};

typedef double f64x4_t __attribute__((ext_vector_type(4)));

// The tile's fp64 product on the matrix cores (v_mfma_f64_16x16x4_f64):
// out[key][col] = sum_k x[k][key] col(k, col) over the d channels, for 32
// keys x 128 columns.  Wave w takes keys 16 (w & 1) .. +15 and columns
// 32 (w >> 1) .. +31 as two 16 x 16 blocks.  Operand lanes: A (16 keys x 4
// channels) lane l = key l % 16, channel l / 16; B (4 channels x 16 columns)
// lane l = channel l / 16, column l % 16.  Result: acc[c][r] of lane l is
// key 16 (w & 1) + l / 16 + 4 r, column 16 (2 (w >> 1) + c) + l % 16 (the
// result rows of this instruction are interleaved by register; the operand
// and result layouts were checked on the GPU with a one-hot probe).
// Each product of two values exact in fp64 (a bf16 key or an fp32 residual
// times an fp32 rotation entry or a bf16 sketch entry) is exact; the sums
// carry at most d roundings, whatever order the unit adds in.
// Even and odd k-steps accumulate into separate registers (four independent
// product chains per wave) that are added at the end: d products still take
// d - 1 additions, so the bound above holds.
template <class Col>
__device__ __forceinline__ void mfma_tile(const Col& col, const double* x, int wave, int lane,
                                          f64x4_t (&acc)[CB]) {
  const int kb = wave & 1, cg = wave >> 1;
  const int lr = lane & 15, lk = lane >> 4;
  f64x4_t acc2[CB];
#pragma unroll
  for (int c = 0; c < CB; ++c) acc[c] = acc2[c] = f64x4_t{0.0, 0.0, 0.0, 0.0};
#pragma unroll 4
  for (int s = 0; s < D / 4; s += 2) {
    const int kk = 4 * s + lk, kk2 = 4 * (s + 1) + lk;
    const double av = x[kk * TKP + 16 * kb + lr];
    const double av2 = x[kk2 * TKP + 16 * kb + lr];
#pragma unroll
    for (int c = 0; c < CB; ++c) {
      acc[c] = __builtin_amdgcn_mfma_f64_16x16x4f64(av, col(kk, 16 * (CB * cg + c) + lr), acc[c], 0, 0, 0);
      acc2[c] = __builtin_amdgcn_mfma_f64_16x16x4f64(av2, col(kk2, 16 * (CB * cg + c) + lr), acc2[c], 0, 0, 0);
    }
  }
#pragma unroll
  for (int c = 0; c < CB; ++c) acc[c] += acc2[c];
}

// A power of two at least sqrt(s) (s >= 0, finite), from the exponent field
// alone: s < 2^(e + 1) with e = floor(log2 s), so sqrt(s) < 2^(e / 2 + 1).
// Used for the certificate bounds, which need an upper bound of a norm, not
// the norm (an fp64 square root is a long instruction sequence).
__device__ __forceinline__ double sqrt_upper_pow2(double s) {
  const int e = static_cast<int>((__double_as_longlong(s) >> 52) & 0x7FF) - 1023;   // s >= 0
  return __builtin_ldexp(1.0, (e >> 1) + 1);
}

// Wave-cooperative evaluation of a 128-term sum of exact fp64 products
// (lane l holds the products of channels 2 l and 2 l + 1): an error-free
// butterfly in which each level adds the two partial sums with TwoSum
// (Knuth; the rounding error is recovered exactly) and accumulates the
// errors, so every lane ends with the same sum s, error sum e and magnitude
// sum a.  Level h adds at most (2 h + 1) 2^-106 a of error, 48 2^-106 a over
// the six levels; returns V = fl(s + e) and B = 2^-90 a + 2^-50 |V| with
// |exact - V| <= B, both wave-uniform.  `exact` (wave-uniform) is set when no
// addition of the errors, nor the final one, rounded (each checked with
// TwoSum): V is then the exact sum.  That is the common case, and the one
// that matters: after heavy cancellation the exact sum has few significant
// bits and can sit exactly on an fp32 tie, which no error bound decides.
// Needs -ffp-contract=off (no fused operations inside TwoSum).
__device__ __forceinline__ double two_sum_err(double x, double y, double s) {
  const double b = s - x;
  return (x - (s - b)) + (y - b);
}
__device__ __forceinline__ void wave_exact_sum(double p0, double p1, double& V, double& B, bool& exact) {
  double s = p0 + p1;
  double e = two_sum_err(p0, p1, s);
  double a = __builtin_fabs(p0) + __builtin_fabs(p1);
  bool inexact = false;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    const double s2 = __shfl_xor(s, m), e2 = __shfl_xor(e, m), a2 = __shfl_xor(a, m);
    const double sn = s + s2;
    const double t = two_sum_err(s, s2, sn);
    const double es = e + e2;
    const double en = es + t;
    inexact = inexact || two_sum_err(e, e2, es) != 0.0 || two_sum_err(es, t, en) != 0.0;
    e = en;
    s = sn;
    a = a + a2;
  }
  V = s + e;
  inexact = inexact || two_sum_err(s, e, V) != 0.0;
  exact = __ballot(inexact) == 0;
  B = a * 0x1.0p-90 + __builtin_fabs(V) * 0x1.0p-50;
}

// fp64 sum of squares of x[j][t] over j in order (the exact definition the
// codes use), loads batched 16 at a time
__device__ __forceinline__ double ordered_sumsq(const double* x, int t) {
  double s = 0.0;
  for (int j0 = 0; j0 < D; j0 += 16) {
    double v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) v[u] = x[(j0 + u) * TKP + t];
#pragma unroll
    for (int u = 0; u < 16; ++u) s = s + v[u] * v[u];
  }
  return s;
}

// A tile's keys: thread tid holds 16-byte chunks tid + NT r of the tile (row
// = chunk / 16, channels 8 (chunk % 16) .. +7); rows past nk are 0.
constexpr int KCH = TK * D / 8 / NT;   // chunks per thread (1)
struct KeyRegs {
  uint4 c[KCH];
};
__device__ __forceinline__ void load_key_regs(KeyRegs& kr, const RotqArgs& a, int row0, int nk) {
#pragma unroll
  for (int r = 0; r < KCH; ++r) {
    const int e = threadIdx.x + NT * r;
    const int t = e >> 4;
    kr.c[r] = t < nk ? reinterpret_cast<const uint4*>(a.keys + static_cast<int64_t>(row0 + t) * D)[e & 15]
                     : make_uint4(0u, 0u, 0u, 0u);
  }
}

// Stage A: y = RN32(exact Pi k) for the tile's keys (rows t < nk valid), from
// the keys already in kr.
__device__ void rotate_tile(RotqLds& L, const RotqArgs& a, int row0, int nk, const KeyRegs& kr) {
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  // keys -> LDS as fp64, transposed ([j][t])
#pragma unroll
  for (int r = 0; r < KCH; ++r) {
    const int e = tid + NT * r;
    const int t = e >> 4, j0 = 8 * (e & 15);
    const uint32_t w[4] = {kr.c[r].x, kr.c[r].y, kr.c[r].z, kr.c[r].w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      L.kt[(j0 + 2 * q) * TKP + t] = static_cast<double>(__uint_as_float(w[q] << 16));
      L.kt[(j0 + 2 * q + 1) * TKP + t] = static_cast<double>(__uint_as_float(w[q] & 0xFFFF0000u));
    }
  }
  __syncthreads();
  // ||k||^2 in channel order (one thread per key)
  if (tid < TK) {
    const double s = ordered_sumsq(L.kt, tid);
    L.nsq[tid] = s;
    L.nrm[tid] = static_cast<float>(__builtin_sqrt(s));
  }
  // the fp64 product y = K Pi^T on the matrix cores
  f64x4_t acc[CB];
  mfma_tile([&](int j, int col) { return static_cast<double>(L.rotT[j * D + col]); }, L.kt, wave, lane, acc);
  __syncthreads();   // nsq ready
  // certify the fp32 rounding: |v - exact| <= 2 d 2^-53 ||k|| ||Pi_i||
  const double wide = __builtin_ldexp(1.0, a.margin_log2);
  const int t_base = 16 * (wave & 1) + (lane >> 4);
  const int i_base = 16 * CB * (wave >> 1) + (lane & 15);
  uint32_t open = 0;
  double Er[4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
    Er[r] = 2.0 * D * 0x1.0p-53 * sqrt_upper_pow2(L.nsq[t_base + 4 * r]) *
                static_cast<double>(a.rot_row_max) * wide + 0x1.0p-1060;
#pragma unroll
  for (int c = 0; c < CB; ++c)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = t_base + 4 * r, i = i_base + 16 * c;
      const double E = Er[r];
      const float lo = static_cast<float>(acc[c][r] - E);
      const float hi = static_cast<float>(acc[c][r] + E);
      L.y[t][i] = hi;
      if (lo != hi && t < nk) open |= 1u << (4 * c + r);
    }
  // The uncertified values (about one in 10^4): the whole wave sums each
  // one's 128 exact products (keys and rotation from LDS) with the
  // error-free butterfly and rounds once the bound decides the fp32 value;
  // otherwise (with the bound, about one in 10^8) one lane takes the exact
  // integer accumulator.
  for (uint64_t any = __ballot(open != 0); any != 0; any = __ballot(open != 0)) {
    const int l = __builtin_ctzll(any);   // wave-uniform
    const uint32_t ol = __builtin_amdgcn_readlane(open, l);
    const int u = __builtin_ctz(ol);
    const int t = 16 * (wave & 1) + (l >> 4) + 4 * (u & 3);
    const int i = 16 * CB * (wave >> 1) + (l & 15) + 16 * (u >> 2);
    const double p0 = L.kt[(2 * lane) * TKP + t] * static_cast<double>(L.rotT[(2 * lane) * D + i]);
    const double p1 = L.kt[(2 * lane + 1) * TKP + t] * static_cast<double>(L.rotT[(2 * lane + 1) * D + i]);
    double V, B;
    bool exact;
    wave_exact_sum(p0, p1, V, B, exact);
    B *= wide;
    // an exact V rounds directly (ties to even); the test hook's widest
    // margins skip that, so that the integer path below is exercised
    const bool direct = exact && wide < 0x1.0p32;
    const float lo = static_cast<float>(direct ? V : V - B);
    float yv = static_cast<float>(direct ? V : V + B);
    if (__float_as_uint(lo) != __float_as_uint(yv)) {   // wave-uniform
      float ex = 0.f;
      if (lane == 0) {
        uint32_t* pos = L.scratch[wave];
        uint32_t* neg = pos + ACC_WORDS;
        long_clear(pos);
        const uint16_t* krow = a.keys + static_cast<int64_t>(row0 + t) * D;
        for (int j = 0; j < D; ++j) add_product(pos, neg, krow[j], a.rot[i * D + j]);
        ex = long_to_f32(pos, neg);
      }
      yv = __shfl(ex, 0);
    }
    if (lane == l) {
      L.y[t][i] = yv;
      open &= open - 1;   // value u done
    }
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// TurboQuant_prod encode
// ---------------------------------------------------------------------------
template <int K>
__global__ __launch_bounds__(NT) void tq_encode_kernel(RotqArgs a, int tiles) {
  __shared__ __attribute__((aligned(16))) RotqLds L;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  for (int e = tid; e < D * D / 4; e += NT)
    reinterpret_cast<float4*>(L.rotT)[e] = reinterpret_cast<const float4*>(a.rotT)[e];
  for (int e = tid; e < D * D / 8; e += NT)
    reinterpret_cast<uint4*>(L.s_il)[e] = reinterpret_cast<const uint4*>(a.s_il)[e];
  constexpr int L2 = 1 << K;
  float cents[L2], bnds[L2 - 1];
#pragma unroll
  for (int v = 0; v < L2; ++v) cents[v] = a.cents[v];
#pragma unroll
  for (int v = 0; v < L2 - 1; ++v) bnds[v] = 0.5f * (cents[v] + cents[v + 1]);
  const double wide = __builtin_ldexp(1.0, a.margin_log2);
  __syncthreads();

  KeyRegs kr;
  if (blockIdx.x < tiles) load_key_regs(kr, a, blockIdx.x * TK, min(TK, a.R - static_cast<int>(blockIdx.x) * TK));
  for (int tile = blockIdx.x; tile < tiles; tile += gridDim.x) {
    const int row0 = tile * TK;
    const int nk = min(TK, a.R - row0);
    rotate_tile(L, a, row0, nk, kr);
    // the next tile's keys load while this one is encoded
    const int next = tile + gridDim.x;
    if (next < tiles) load_key_regs(kr, a, next * TK, min(TK, a.R - next * TK));
    // u, codes, residual (thread per (coordinate, quarter of the keys); the
    // reads are issued together)
    {
      constexpr int PT = TK * D / NT;   // keys per thread
      const int i = tid & (D - 1), h = tid >> 7;
      float yv[PT], nv[PT];
#pragma unroll
      for (int u8 = 0; u8 < PT; ++u8) {
        nv[u8] = L.nrm[PT * h + u8];
        yv[u8] = L.y[PT * h + u8][i];
      }
#pragma unroll
      for (int u8 = 0; u8 < PT; ++u8) {
        const int t = PT * h + u8;
        const float u = nv[u8] > 0.f ? yv[u8] / nv[u8] : 0.f;
        int idx = 0;
#pragma unroll
        for (int v = 0; v < L2 - 1; ++v) idx += u >= bnds[v] ? 1 : 0;
        float c = cents[0];
#pragma unroll
        for (int v = 1; v < L2; ++v) c = idx == v ? cents[v] : c;
        const float r = u - c;
        L.cell[t][i] = static_cast<uint8_t>(idx);
        L.y[t][i] = r;                                   // the residual replaces y
        L.kt[i * TKP + t] = static_cast<double>(r);     // and the keys, as fp64 [i][t]
      }
    }
    __syncthreads();
    if (tid < TK) L.nsq[tid] = ordered_sumsq(L.kt, tid);
    // z = S^T r on the matrix cores (columns = sketch coordinates)
    f64x4_t acc[CB];
    mfma_tile([&](int ii, int col) {
      return static_cast<double>(__uint_as_float(static_cast<uint32_t>(L.s_il[ii * D + col]) << 16));
    }, L.kt, wave, lane, acc);
    __syncthreads();   // nsq (residual) ready
    const int t_base = 16 * (wave & 1) + (lane >> 4);
    uint32_t open = 0;
    double Er[4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
      Er[r] = 2.0 * D * 0x1.0p-53 * sqrt_upper_pow2(L.nsq[t_base + 4 * r]) *
                  static_cast<double>(a.s_col_max) * wide + 0x1.0p-1060;
#pragma unroll
    for (int c = 0; c < CB; ++c)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (!(__builtin_fabs(acc[c][r]) > Er[r]) && t_base + 4 * r < nk) open |= 1u << (4 * c + r);
    // exact signs for the uncertified sums (rare): the wave's error-free
    // butterfly over the 128 exact products, then, if the bound cannot
    // decide, one lane's integer accumulator
    for (uint64_t any = __ballot(open != 0); any != 0; any = __ballot(open != 0)) {
      const int ln = __builtin_ctzll(any);   // wave-uniform
      const uint32_t ol = __builtin_amdgcn_readlane(open, ln);
      const int u = __builtin_ctz(ol);
      const int t = 16 * (wave & 1) + (ln >> 4) + 4 * (u & 3);
      const int lc = 16 * CB * (wave >> 1) + (ln & 15) + 16 * (u >> 2);
      const double p0 = static_cast<double>(L.y[t][2 * lane]) *
                        static_cast<double>(__uint_as_float(static_cast<uint32_t>(L.s_il[(2 * lane) * D + lc]) << 16));
      const double p1 = static_cast<double>(L.y[t][2 * lane + 1]) *
                        static_cast<double>(__uint_as_float(static_cast<uint32_t>(L.s_il[(2 * lane + 1) * D + lc]) << 16));
      double V, B;
      bool exact;
      wave_exact_sum(p0, p1, V, B, exact);
      B *= wide;
      if (exact && wide < 0x1.0p32) B = 0.0;   // V is the exact sum
      int positive;
      if (V > B) {
        positive = 1;
      } else if (V < -B) {
        positive = 0;
      } else if (B == 0.0) {
        positive = V >= 0.0 ? 1 : 0;   // exact: sign(0) = +1
      } else {
        int sg = 0;
        if (lane == 0) {
          uint32_t* pos = L.scratch[wave];
          uint32_t* neg = pos + ACC_WORDS;
          long_clear(pos);
          for (int ii = 0; ii < D; ++ii) add_product(pos, neg, L.s_il[ii * D + lc], L.y[t][ii]);
          sg = long_sign(pos, neg) ? 1 : 0;
        }
        positive = __shfl(sg, 0);
      }
      if (lane == ln) {
        acc[u >> 2][u & 3] = positive ? 1.0 : -1.0;
        open &= open - 1;   // value u done
      }
    }
    // sign words: ballot bit l of register (c, r) is key 16 (wave & 1) +
    // l / 16 + 4 r, coordinate 16 (CB (wave >> 1) + c) + l % 16; each 16-lane
    // group fills one half-word of its key's row
    uint16_t* qh = reinterpret_cast<uint16_t*>(&L.qwords[0][0]);
#pragma unroll
    for (int c = 0; c < CB; ++c)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint64_t m = __ballot(acc[c][r] >= 0.0);
        if (lane < 4) {
          const int t = 16 * (wave & 1) + lane + 4 * r;
          qh[t * 8 + CB * (wave >> 1) + c] = static_cast<uint16_t>(m >> (16 * lane));
        }
      }
    __syncthreads();
    // stores: codes (bit stream, k bits per coordinate), sign words, n, g
    const int cw = D * K / 32;
    for (int e = tid; e < TK * (cw + 4); e += NT) {
      const int t = e / (cw + 4), w = e % (cw + 4);
      if (t >= nk) continue;
      const int64_t row = dest_row(a.r0 + row0 + t, static_cast<uint32_t>(a.n), a.cap, a.pos);
      if (w < cw) {
        uint32_t word = 0;
        if (K == 2) {   // coordinates 16 w .. 16 w + 15, two bits each
          const uint4 c4 = *reinterpret_cast<const uint4*>(&L.cell[t][16 * w]);
          const uint32_t cb[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int bb = 0; bb < 4; ++bb) word |= ((cb[q] >> (8 * bb)) & 3u) << (2 * (4 * q + bb));
        } else {
          for (int p = 0; p < 32; ++p) {
            const int b = 32 * w + p;
            word |= ((static_cast<uint32_t>(L.cell[t][b / K]) >> (b % K)) & 1u) << p;
          }
        }
        a.codes[row * cw + w] = word;
      } else {
        a.bits[row * 4 + (w - cw)] = L.qwords[t][w - cw];
      }
    }
    if (tid < nk) {
      const int64_t row = dest_row(a.r0 + row0 + tid, static_cast<uint32_t>(a.n), a.cap, a.pos);
      a.norms[row] = L.nrm[tid];
      a.gammas[row] = static_cast<float>(__builtin_sqrt(L.nsq[tid]));
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// PolarQuant encode
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(NT) void pq_encode_kernel(RotqArgs a, int tiles) {
  __shared__ __attribute__((aligned(16))) RotqLds L;
  double* sq = L.kt;   // tree sums of squares (two buffers in the key tile's LDS)
  const int tid = threadIdx.x;
  for (int e = tid; e < D * D / 4; e += NT)
    reinterpret_cast<float4*>(L.rotT)[e] = reinterpret_cast<const float4*>(a.rotT)[e];
  if (tid < PQ_LEVELS * PQ_MAXT) L.thr[tid] = a.pq_thr[tid];
  __syncthreads();
  // bits per level: 4, then 2; thresholds per level: 3 (level 1), 3
  constexpr int kBits[PQ_LEVELS] = {4, 2, 2, 2, 2, 2, 2};

  KeyRegs kr;
  if (blockIdx.x < tiles) load_key_regs(kr, a, blockIdx.x * TK, min(TK, a.R - static_cast<int>(blockIdx.x) * TK));
  for (int tile = blockIdx.x; tile < tiles; tile += gridDim.x) {
    const int row0 = tile * TK;
    const int nk = min(TK, a.R - row0);
    rotate_tile(L, a, row0, nk, kr);
    const int next = tile + gridDim.x;
    if (next < tiles) load_key_regs(kr, a, next * TK, min(TK, a.R - next * TK));
    // Each wave takes the levels of its own KPW keys, so the levels need no
    // workgroup barrier (a wave's LDS accesses complete in order; the fences
    // keep the compiler from moving them).  A key keeps the same D / 2 slots
    // of each sum buffer at every level, so no wave touches another's keys.
    // level 1: pair cells and the pairs' sums of squares
    constexpr int KPW = TK / (NT / 64);
    const int wave = tid >> 6, lane = tid & 63;
    for (int r = 0; r < KPW; ++r) {
      const int t = KPW * wave + r, j = lane;
      const double av = static_cast<double>(L.y[t][2 * j]);
      const double bv = static_cast<double>(L.y[t][2 * j + 1]);
      int q;
      double ap, bp;
      if (bv > 0.0) {
        q = av > 0.0 ? 0 : 1;
      } else if (bv < 0.0) {
        q = av < 0.0 ? 2 : 3;
      } else {
        q = av < 0.0 ? 2 : 0;
      }
      ap = q == 0 ? av : (q == 1 ? bv : (q == 2 ? -av : -bv));
      bp = q == 0 ? bv : (q == 1 ? -av : (q == 2 ? -bv : av));
      int within = 0;
      for (int u = 0; u < (1 << kBits[0]) / 4 - 1; ++u) {
        const double T = static_cast<double>(L.thr[u]);
        within += bp >= T * ap ? 1 : 0;
      }
      if (ap == 0.0 && bp == 0.0) within = 0;
      L.cell[t][j] = static_cast<uint8_t>(q * ((1 << kBits[0]) / 4) + within);
      sq[t * (D / 2) + j] = av * av + bv * bv;   // [t][pair]
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    // levels 2 .. 7: cells from the slice sums, then the pairwise sums
    // (ping-pong between two halves of the key tile's LDS)
    double* cur = sq;
    double* nxt = sq + TK * (D / 2);
    int width = D / 2;       // sums at the level below
    int cell_off = D / 2;    // cells of level l follow those of lower levels
    for (int lev = 2; lev <= PQ_LEVELS; ++lev) {
      const int half = width / 2;
      const int nthr = (1 << kBits[lev - 1]) - 1;
      for (int e = lane; e < KPW * half; e += 64) {
        const int t = KPW * wave + e / half, j = e % half;
        const double sa = cur[t * (D / 2) + 2 * j], sb = cur[t * (D / 2) + 2 * j + 1];
        int c = 0;
        for (int u = 0; u < nthr; ++u) {
          const double T = static_cast<double>(L.thr[(lev - 1) * PQ_MAXT + u]);
          c += sb >= (T * T) * sa ? 1 : 0;
        }
        L.cell[t][cell_off + j] = static_cast<uint8_t>(c);
        nxt[t * (D / 2) + j] = sa + sb;
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
      double* tmp = cur;
      cur = nxt;
      nxt = tmp;
      cell_off += half;
      width = half;
    }
    if (lane < KPW) L.nsq[KPW * wave + lane] = cur[(KPW * wave + lane) * (D / 2)];   // the top-level sums
    __syncthreads();   // every key's cells and sums
    // stream: level 1 cells (4 bits each), then 2-bit cells of levels 2..7
    for (int e = tid; e < TK * PQ_WORDS; e += NT) {
      const int t = e / PQ_WORDS, w = e % PQ_WORDS;
      if (t >= nk) continue;
      // words 0..7: eight 4-bit level-1 cells each; words 8..11: sixteen
      // 2-bit cells of levels 2..7 each (cell 127 does not exist: its bits,
      // the top two of word 11, stay zero)
      uint32_t word = 0;
      if (w < 8) {
        const uint2 c8 = *reinterpret_cast<const uint2*>(&L.cell[t][8 * w]);
        const uint32_t cb[2] = {c8.x, c8.y};
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
          for (int bb = 0; bb < 4; ++bb) word |= ((cb[q] >> (8 * bb)) & 15u) << (4 * (4 * q + bb));
      } else {
        const uint4 c16 = *reinterpret_cast<const uint4*>(&L.cell[t][D / 2 + 16 * (w - 8)]);
        const uint32_t cb[4] = {c16.x, c16.y, c16.z, c16.w};
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int bb = 0; bb < 4; ++bb) word |= ((cb[q] >> (8 * bb)) & 3u) << (2 * (4 * q + bb));
        if (w == PQ_WORDS - 1) word &= 0x3FFFFFFFu;
      }
      const int64_t row = dest_row(a.r0 + row0 + t, static_cast<uint32_t>(a.n), a.cap, a.pos);
      a.pq_codes[row * PQ_WORDS + w] = word;
    }
    if (tid < nk) {
      const int64_t row = dest_row(a.r0 + row0 + tid, static_cast<uint32_t>(a.n), a.cap, a.pos);
      a.radii[row] = static_cast<float>(__builtin_sqrt(L.nsq[tid]));
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// TurboQuant_prod scores: est_t = n_t (<Pi q, c[idx_t]> + sqrt(pi/2)/m g_t
// <S^T Pi q, 2 bit_t - 1>) for every token t < N and query head
// ---------------------------------------------------------------------------
// Two kernels.  tq_query_kernel prepares each query head once into the
// workspace: Pi q and S^T Pi q (fp32 FMAs over one table [Pi; M], M =
// S^T Pi) and, for k = 1, 2, their integer operands below.
//
// Scores for k = 1, 2 (tq_scores_mfma_kernel) are dot products of 0/1
// bit-planes on the int8 matrix cores.  With idx = b0 + 2 b1, c[idx] = c0 +
// (c1 - c0) b0 + (c2 - c0) b1 + (c3 - c2 - c1 + c0) b0 b1 (k = 1: c0 +
// (c1 - c0) b0), where the last coefficient is 0 for the symmetric
// codebooks used here, so
//   <Pi q, c[idx]> = c0 sum_i (Pi q)_i + sum over planes P of sum_i v_P,i P_i,
// v_P = alpha_P Pi q, and <S^T Pi q, 2 bit - 1> = 2 sum_l s_l bit_l - sum_l s_l.
// The prep quantizes every v_P (one exponent per head, from the largest
// |v_P,i|) and s (likewise) to integers Q = round(v / 2^E), |Q| <= 2^30
// (error at most 2^-31 of the largest |v| per term), written as four signed
// byte limbs: the A operand of
// v_mfma_i32_16x16x64_i8, rows = head x limb for four heads, held in
// registers for the whole kernel.  The tokens' bit-planes, spread to 0/1
// bytes with one shift and one mask per register, are the B operand
// (columns = 16 tokens); the int32 sums are exact, and a lane of the result
// holds the four limb rows of one head for one token, combined in registers.
// Scores for k = 3 (tq_scores_kernel; 3-bit codes do not fall on byte lanes):
// a workgroup takes a range of tokens of one (batch, kv head); its prologue
// builds nibble tables in LDS from the prepared queries of the kv head's G
// query heads, the G heads' values of one table entry side by side (so one
// 16-byte LDS read serves four heads): for the sign words, the sum of
// S^T Pi q over the set bits of every 4-bit group; for the codes, <Pi q,
// c[idx]> of every coordinate's 8 codes.  A thread scores its tokens with one
// table read per sign nibble and per coordinate (per four heads).

// rows of the query table: [Pi; M]
constexpr int kQRows = 2 * D;
// prepared query of head hq, kQPrepBytes apart: floats Pi q at [0, 512) and
// S^T Pi q at [512, 1024); limb operands at [1024, 3072): 16 bytes per
// (plane p, k-step ks, limb j, k-group g), p = 0, 1 code planes (b0, b1;
// k = 1 uses b0 only; slot 2 is unused), p = 3 the sign plane; scalars at
// 3072: 2^E of the code planes, 2^E of the sign plane, c0 sum_i (Pi q)_i,
// sum_l s_l.
constexpr int kQPrepBytes = 4096;
constexpr int kQPrepFloats = kQPrepBytes / 4;
constexpr int kLimbOffset = 1024;
constexpr int kScalarOffset = 3072;

// Workgroup (query head, half s) computes rows 128 s .. 128 s + 127 of
// [Pi; M] q: half 0 Pi q, half 1 S^T Pi q = M q, so neither waits for the
// other.  Thread (jp, i4) sums the products of 16 inputs j (part jp of 8)
// for rows 4 i4 .. 4 i4 + 3 (one 16-byte read of the transposed table per
// input); the 8 partial sums of a row are added in part order.  For k = 1,
// 2 each half then writes the byte limbs of its planes (half 0 the code
// planes, half 1 the sign plane) with the exponent of its own largest value,
// and its sum.
constexpr int kQueryThreads = 256;
__global__ __launch_bounds__(kQueryThreads) void tq_query_kernel(const float* __restrict__ q,
                                                                 const float* __restrict__ qtab,
                                                                 const float* __restrict__ cents, int K,
                                                                 uint8_t* __restrict__ prep_bytes) {
  constexpr int PARTS = kQueryThreads / (D / 4);   // 8 parts of 16 inputs
  constexpr int JP = D / PARTS;                    // 16
  __shared__ float qs[D], vals[D];
  __shared__ __attribute__((aligned(16))) float part[PARTS][D];
  __shared__ float red[2][2];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int i4 = tid % (D / 4), jp = tid / (D / 4);
  const int s = blockIdx.y;
  const int64_t hq = blockIdx.x;
  // the table reads do not depend on q: issued first
  float4 r[JP];
#pragma unroll
  for (int u = 0; u < JP; ++u)
    r[u] = *reinterpret_cast<const float4*>(qtab + (jp * JP + u) * kQRows + D * s + 4 * i4);
  if (tid < D) qs[tid] = q[hq * D + tid];
  __syncthreads();
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int u = 0; u < JP; ++u) {
    const float qj = qs[jp * JP + u];
    acc.x = __builtin_fmaf(r[u].x, qj, acc.x);
    acc.y = __builtin_fmaf(r[u].y, qj, acc.y);
    acc.z = __builtin_fmaf(r[u].z, qj, acc.z);
    acc.w = __builtin_fmaf(r[u].w, qj, acc.w);
  }
  reinterpret_cast<float4*>(part[jp])[i4] = acc;
  __syncthreads();
  float* prep = reinterpret_cast<float*>(prep_bytes + hq * kQPrepBytes);
  float v = 0.f;
  if (tid < D) {
#pragma unroll
    for (int p2 = 0; p2 < PARTS; ++p2) v += part[p2][tid];
    vals[tid] = v;
    prep[D * s + tid] = v;   // Pi q at [0, D), S^T Pi q at [D, 2 D)
  }
  if (K == 3) return;   // the table kernel reads Pi q and S^T Pi q only
  // the half's largest |value| and its sum (waves 0 and 1 hold the D values)
  if (tid < D) {
    float mx = __builtin_fabsf(v), sm = v;
    for (int m = 32; m >= 1; m >>= 1) {
      mx = fmaxf(mx, __shfl_xor(mx, m));
      sm += __shfl_xor(sm, m);
    }
    if (lane == 0) {
      red[wv][0] = mx;
      red[wv][1] = sm;
    }
  }
  __syncthreads();
  // plane coefficients (k = 1: b0; k = 2: b0, b1).  The codebooks are
  // symmetric (c[v] = -c[2^k - 1 - v], checked when the tables are built), so
  // the b0 b1 coefficient c3 - c2 - c1 + c0 is exactly 0 in fp32 (c3 - c2 and
  // c1 - c0 are the same fp32 difference) and that plane is left out.
  const float c0 = cents[0];
  const float alpha[2] = {cents[1] - c0, K == 2 ? cents[2] - c0 : 0.f};
  const bool code = s == 0;
  const float amax = fmaxf(__builtin_fabsf(alpha[0]), __builtin_fabsf(alpha[1]));
  // every |fl(alpha_P x)| <= fl(amax max|x|) (rounding is monotonic), so
  // with that < 2^(E + 30), |Q| <= 2^30 and the top limb fits a byte
  const float top = (code ? amax : 1.f) * fmaxf(red[0][0], red[1][0]);
  const int e = top > 0.f ? __builtin_amdgcn_frexp_expf(top) - 30 : 0;
  // limb dword (((p 2 + ks) 4 + j) 4 + g) 4 + qq holds bytes b = 0..3 (byte
  // x = 4 qq + b of the operand) of limb j of coordinate coord(p, g, ks, x)
  uint32_t* limbs = reinterpret_cast<uint32_t*>(prep_bytes + hq * kQPrepBytes + kLimbOffset);
  const int nd = code ? (K == 2 ? 2 : 1) * 128 : 128;
  for (int t = tid; t < nd; t += kQueryThreads) {
    const int qq = t & 3, g = (t >> 2) & 3, j = (t >> 4) & 3, ks = (t >> 6) & 1;
    const int pl = code ? t >> 7 : 3;
    const float al = pl == 0 ? alpha[0] : alpha[1];
    uint32_t word = 0;
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) {
      int coord;
      if (code && K == 2) coord = 16 * (2 * g + ks) + 4 * bb + qq;   // code word 2 g + ks, 2 bits a coordinate
      else coord = 32 * g + 8 * bb + 4 * ks + qq;                    // one bit a coordinate
      const float x = code ? al * vals[coord] : vals[coord];
      const int Q = static_cast<int>(__builtin_rintf(__builtin_ldexpf(x, -e)));
      // balanced base-256 digits: Q = l0 + 256 l1 + 65536 l2 + 2^24 l3
      int rest = Q, lj = 0;
#pragma unroll
      for (int k2 = 0; k2 <= 3; ++k2) {
        const int l = ((rest + 128) & 255) - 128;
        if (k2 == j) lj = l;
        rest = (rest - l) >> 8;
      }
      word |= (static_cast<uint32_t>(lj) & 255u) << (8 * bb);
    }
    limbs[(((pl * 2 + ks) * 4 + j) * 4 + g) * 4 + qq] = word;
  }
  if (tid == 0) {
    float* sc = reinterpret_cast<float*>(prep_bytes + hq * kQPrepBytes + kScalarOffset);
    const float sum = red[0][1] + red[1][1];
    sc[code ? 0 : 1] = __builtin_ldexpf(1.0f, e);
    sc[code ? 2 : 3] = code ? c0 * sum : sum;
  }
}

// acc[h] += entry[h] for GH (<= 4) heads of one table entry, one LDS read
template <int GH>
__device__ __forceinline__ void add_entry(const float* e, float (&acc)[GH]) {
  if constexpr (GH == 4) {
    const float4 v = *reinterpret_cast<const float4*>(e);
    acc[0] += v.x;
    acc[1] += v.y;
    acc[2] += v.z;
    acc[3] += v.w;
  } else if constexpr (GH == 2) {
    const float2 v = *reinterpret_cast<const float2*>(e);
    acc[0] += v.x;
    acc[1] += v.y;
  } else {
    acc[0] += e[0];
  }
}

// one token's cache row at k = 3: code words, sign words, norm and gamma
constexpr int kTq3Words = D * 3 / 32;   // 12: whole 16-byte chunks
struct TqRow {
  uint32_t cw[kTq3Words];
  uint32_t bw[4];
  float n, g;
};
__device__ __forceinline__ void load_tq_row(TqRow& r, const uint32_t* __restrict__ codes,
                                            const uint32_t* __restrict__ bits, const float* __restrict__ norms,
                                            const float* __restrict__ gammas, int64_t row) {
  constexpr int CW = kTq3Words;
#pragma unroll
  for (int w4 = 0; w4 < CW / 4; ++w4) {
    const uint4 v = reinterpret_cast<const uint4*>(codes + row * CW)[w4];
    r.cw[4 * w4] = v.x;
    r.cw[4 * w4 + 1] = v.y;
    r.cw[4 * w4 + 2] = v.z;
    r.cw[4 * w4 + 3] = v.w;
  }
  const uint4 v = reinterpret_cast<const uint4*>(bits + row * 4)[0];
  r.bw[0] = v.x;
  r.bw[1] = v.y;
  r.bw[2] = v.z;
  r.bw[3] = v.w;
  r.n = norms[row];
  r.g = gammas[row];
}

template <int G>
__global__ __launch_bounds__(256) void tq_scores_kernel(
    const float* __restrict__ prep, const uint32_t* __restrict__ codes, const uint32_t* __restrict__ bits,
    const float* __restrict__ norms, const float* __restrict__ gammas, const float* __restrict__ cents, int H_kv,
    int N, int cap, int tpw, float coef, float* __restrict__ out) {
  constexpr int CW = kTq3Words;                        // code words per token
  constexpr int CROWS = D;                             // code-table rows (coordinates)
  constexpr int CCOLS = 8;                             // codes
  __shared__ float qr[G][D];                           // Pi q
  __shared__ float qs[G][D];                           // S^T Pi q
  __shared__ __attribute__((aligned(16))) float lb[D / 4][16][G];   // sign-word nibbles
  __shared__ __attribute__((aligned(16))) float lc[CROWS][CCOLS][G];  // code nibbles
  __shared__ float ssum[G];
  const int tid = threadIdx.x;
  const int kvh = blockIdx.y, b = blockIdx.z;
  const int64_t bh = static_cast<int64_t>(b) * H_kv + kvh;
  const int t_end = min(N, (static_cast<int>(blockIdx.x) + 1) * tpw);
  // the first token's row is in flight while the tables are built
  int t = blockIdx.x * tpw + tid;
  TqRow cur;
  if (t < t_end) load_tq_row(cur, codes, bits, norms, gammas, bh * cap + t);
  float c[8];
#pragma unroll
  for (int v = 0; v < 8; ++v) c[v] = cents[v];
  for (int e = tid; e < G * D; e += 256) {
    const int h = e / D, i = e % D;
    const float* p = prep + (bh * G + h) * kQPrepFloats;
    qr[h][i] = p[i];
    qs[h][i] = p[D + i];
  }
  __syncthreads();
  for (int e = tid; e < (D / 4) * 16 * G; e += 256) {
    const int h = e % G, nib = (e / G) % 16, g4 = e / (16 * G);
    float v = 0.f;
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) v += (nib >> bb) & 1 ? qs[h][4 * g4 + bb] : 0.f;
    lb[g4][nib][h] = v;
  }
  for (int e = tid; e < CROWS * CCOLS * G; e += 256) {
    const int h = e % G, col = (e / G) % CCOLS, row = e / (G * CCOLS);
    lc[row][col][h] = qr[h][row] * c[col];
  }
  if (tid < G) {
    float s2 = 0.f;
    for (int l = 0; l < D; ++l) s2 += qs[tid][l];
    ssum[tid] = s2;
  }
  __syncthreads();
#pragma unroll 1
  for (; t < t_end; t += 256) {
    // the next token's row loads while this one is scored
    TqRow nxt = cur;
    if (t + 256 < t_end) load_tq_row(nxt, codes, bits, norms, gammas, bh * cap + t + 256);
    const uint32_t* cwd = cur.cw;
    const uint32_t* bw = cur.bw;
    const float n = cur.n, g = cur.g;
    // heads in groups of up to four (one 16-byte table read per nibble)
    constexpr int GH = G < 4 ? G : 4;
#pragma unroll 1
    for (int h0 = 0; h0 < G; h0 += GH) {
      // the words pass through an empty asm per group, so the table
      // addresses derived from them are recomputed in the loop, not held
      // live across it (96 to 160 registers otherwise)
      uint32_t cw2[CW], bw2[4];
#pragma unroll
      for (int w = 0; w < CW; ++w) {
        cw2[w] = cwd[w];
        asm volatile("" : "+v"(cw2[w]));
      }
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        bw2[w] = bw[w];
        asm volatile("" : "+v"(bw2[w]));
      }
      float mse[GH], pos[GH];
#pragma unroll
      for (int h = 0; h < GH; ++h) {
        mse[h] = 0.f;
        pos[h] = 0.f;
      }
#pragma unroll
      for (int i = 0; i < D; ++i) {
        const int bpos = 3 * i;
        uint32_t idx = cw2[bpos >> 5] >> (bpos & 31);
        if ((bpos & 31) > 29) idx |= cw2[(bpos >> 5) + 1] << (32 - (bpos & 31));
        add_entry<GH>(&lc[i][idx & 7][h0], mse);
      }
#pragma unroll
      for (int r = 0; r < D / 4; ++r) add_entry<GH>(&lb[r][(bw2[r >> 3] >> (4 * (r & 7))) & 15][h0], pos);
#pragma unroll
      for (int h = 0; h < GH; ++h)
        out[((bh * G + h0 + h) * static_cast<int64_t>(N)) + t] =
            n * (mse[h] + coef * g * (2.f * pos[h] - ssum[h0 + h]));
    }
    cur = nxt;
  }
}


typedef int i32x4_t __attribute__((__vector_size__(4 * sizeof(int))));

// 0/1 bytes of one token's bit-plane for one k-step: register q, byte b =
// bit 8 b + sh + step q of word w (the limb operand was laid out to match)
template <int STEP>
__device__ __forceinline__ i32x4_t plane_bytes(uint32_t w, int sh) {
  i32x4_t v;
#pragma unroll
  for (int q = 0; q < 4; ++q) v[q] = static_cast<int>((w >> (sh + STEP * q)) & 0x01010101u);
  return v;
}

// Buffer descriptor over [base, base + bytes): loads past the end return
// zero (base and bytes wave-uniform).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t rows_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           __builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

// the tokens' rows of one 64-token chunk of a wave: lane (row, grp) holds
// token t0 + 16 u + row's code words (k = 2: words 2 grp, 2 grp + 1; k = 1:
// word grp), its sign word grp, norm and gamma.  Loaded through descriptors
// over the chunk's nrows valid rows (row0 = the first one's cache row), so
// the lane offsets are the same every pass and rows past N read as zero.
template <int K>
struct TqChunk {
  uint32_t c0[4], c1[4], sw[4];
  float n[4], g[4];
};
template <int K>
__device__ __forceinline__ void load_tq_chunk(TqChunk<K>& c, const uint32_t* __restrict__ codes,
                                              const uint32_t* __restrict__ bits, const float* __restrict__ norms,
                                              const float* __restrict__ gammas, int64_t row0, int nrows, int row,
                                              int grp) {
  constexpr int CW = D * K / 32;   // code words per token
  const rsrc_t rc = rows_rsrc(codes + row0 * CW, nrows * CW * 4);
  const rsrc_t rs = rows_rsrc(bits + row0 * 4, nrows * 16);
  const rsrc_t rn = rows_rsrc(norms + row0, nrows * 4);
  const rsrc_t rg = rows_rsrc(gammas + row0, nrows * 4);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int r = 16 * u + row;
    if constexpr (K == 2) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b64(rc, (r * CW + 2 * grp) * 4, 0, 0);
      c.c0[u] = v[0];
      c.c1[u] = v[1];
    } else {
      c.c0[u] = __builtin_amdgcn_raw_buffer_load_b32(rc, (r * CW + grp) * 4, 0, 0);
      c.c1[u] = 0;
    }
    c.sw[u] = __builtin_amdgcn_raw_buffer_load_b32(rs, (r * 4 + grp) * 4, 0, 0);
    c.n[u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rn, r * 4, 0, 0));
    c.g[u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rg, r * 4, 0, 0));
  }
}

// k = 1, 2: a workgroup of four waves takes 256-token chunks of one (batch,
// kv head); a wave scores 64 tokens a pass as four 16-token tiles.  The
// limb operands of the kv head's G query heads stay in registers (rows 4 h'
// + j of row block rb: head 4 rb + h', limb j; zero rows past G); the result
// lane (row, grp) of row block rb holds head 4 rb + grp's four limb sums for
// token row of the tile.
template <int G, int K>
__global__ __launch_bounds__(256) void tq_scores_mfma_kernel(
    const uint8_t* __restrict__ prep, const uint32_t* __restrict__ codes, const uint32_t* __restrict__ bits,
    const float* __restrict__ norms, const float* __restrict__ gammas, int H_kv, int N, int cap, int tpw,
    float coef, float* __restrict__ out) {
  constexpr int NRB = (G + 3) / 4;
  constexpr int NP = K == 2 ? 2 : 1;   // code planes (b0, b1)
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform passes
  const int row = lane & 15, grp = lane >> 4;
  const int kvh = blockIdx.y, b = blockIdx.z;
  const int64_t bh = static_cast<int64_t>(b) * H_kv + kvh;
  const int64_t base = bh * cap;
  const int t_end = min(N, (static_cast<int>(blockIdx.x) + 1) * tpw);
  int t0 = blockIdx.x * tpw + 64 * wave;
  auto valid_rows = [&](int t) { return max(0, min(64, N - t)); };
  // the first chunk's rows are in flight while the operands load
  TqChunk<K> cur;
  if (t0 < t_end) load_tq_chunk<K>(cur, codes, bits, norms, gammas, base + t0, valid_rows(t0), row, grp);
  i32x4_t ac[NRB][NP][2], as[NRB][2];
  float4 sc[NRB];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    const int h = 4 * rb + (row >> 2), j = row & 3;
    const uint8_t* lp = prep + (bh * G + h) * kQPrepBytes + kLimbOffset + (j * 4 + grp) * 16;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int p = 0; p < NP; ++p)
        ac[rb][p][ks] = h < G ? *reinterpret_cast<const i32x4_t*>(lp + (p * 2 + ks) * 256) : i32x4_t{0, 0, 0, 0};
      as[rb][ks] = h < G ? *reinterpret_cast<const i32x4_t*>(lp + (3 * 2 + ks) * 256) : i32x4_t{0, 0, 0, 0};
    }
    const int ho = 4 * rb + grp;
    sc[rb] = ho < G ? *reinterpret_cast<const float4*>(prep + (bh * G + ho) * kQPrepBytes + kScalarOffset)
                    : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  // two row buffers used in turn (a pass scores one while the next pass's
  // rows load into the other), so no registers are copied between passes
  auto score = [&](const TqChunk<K>& c, int tp) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      i32x4_t bc[NP][2], bs[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        if constexpr (K == 2) {
          // word 2 grp + ks: coordinate 16 (2 grp + ks) + 4 b + q at bits
          // 8 b + 2 q (b0) and 8 b + 2 q + 1 (b1)
          const uint32_t w = ks ? c.c1[u] : c.c0[u];
          bc[0][ks] = plane_bytes<2>(w, 0);
          bc[1][ks] = plane_bytes<2>(w, 1);
        } else {
          // word grp: coordinate 32 grp + 8 b + 4 ks + q at bit 8 b + 4 ks + q
          bc[0][ks] = plane_bytes<1>(c.c0[u], 4 * ks);
        }
        bs[ks] = plane_bytes<1>(c.sw[u], 4 * ks);
      }
      const int t = tp + 16 * u + row;
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        i32x4_t accc = {0, 0, 0, 0}, accs = {0, 0, 0, 0};
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
          for (int p = 0; p < NP; ++p)
            accc = __builtin_amdgcn_mfma_i32_16x16x64_i8(ac[rb][p][ks], bc[p][ks], accc, 0, 0, 0);
          accs = __builtin_amdgcn_mfma_i32_16x16x64_i8(as[rb][ks], bs[ks], accs, 0, 0, 0);
        }
        // sum_j 256^j acc[j] = hi 2^16 + lo with lo = acc0 + 256 acc1 and hi =
        // acc2 + 256 acc3 (|acc_j| <= 2 128 128, the top limb <= 64 in
        // magnitude: both below 2^24, exact in int32 and fp32), one rounding
        const int loc = accc[0] + 256 * accc[1], hic = accc[2] + 256 * accc[3];
        const int los = accs[0] + 256 * accs[1], his = accs[2] + 256 * accs[3];
        const float vc = __builtin_fmaf(static_cast<float>(hic), 65536.f, static_cast<float>(loc));
        const float vs = __builtin_fmaf(static_cast<float>(his), 65536.f, static_cast<float>(los));
        const float mse = __builtin_fmaf(sc[rb].x, vc, sc[rb].z);
        const float qjl = __builtin_fmaf(2.f * sc[rb].y, vs, -sc[rb].w);   // <s, 2 bit - 1>
        const int ho = 4 * rb + grp;
        if (ho < G && t < t_end)
          out[(bh * G + ho) * static_cast<int64_t>(N) + t] = c.n[u] * __builtin_fmaf(coef * c.g[u], qjl, mse);
      }
    }
  };
  TqChunk<K> alt;
#pragma unroll 1
  while (t0 < t_end) {
    if (t0 + 256 < t_end)
      load_tq_chunk<K>(alt, codes, bits, norms, gammas, base + t0 + 256, valid_rows(t0 + 256), row, grp);
    score(cur, t0);
    t0 += 256;
    if (t0 >= t_end) break;
    if (t0 + 256 < t_end)
      load_tq_chunk<K>(cur, codes, bits, norms, gammas, base + t0 + 256, valid_rows(t0 + 256), row, grp);
    score(alt, t0);
    t0 += 256;
  }
}
}  // namespace

int launch_rotq_encode(const RotqTables& tb, int method, int k, const void* keys, int B, int H_kv, int n,
                       uint32_t* codes, uint32_t* bits, float* norms, float* gammas, int cap, int pos,
                       int margin_log2, void* stream) {
  const int64_t R = static_cast<int64_t>(B) * H_kv * n;
  if (R == 0) return hipSuccess;
  RotqArgs a{};
  a.keys = static_cast<const uint16_t*>(keys);
  a.R = static_cast<int>(R);
  a.n = n;
  a.cap = cap;
  a.pos = pos;
  a.r0 = 0;
  a.rotT = tb.rotT;
  a.rot = tb.rot;
  a.rot_row_max = tb.rot_row_max;
  a.s_il = tb.s_il;
  a.s_col_max = tb.s_col_max;
  a.k = k;
  a.cents = method == 0 ? tb.tq_cents + 8 * (k - 1) : nullptr;
  a.pq_thr = tb.pq_thr;
  a.margin_log2 = margin_log2;
  if (method == 0) {
    a.codes = codes;
    a.bits = bits;
    a.norms = norms;
    a.gammas = gammas;
  } else {
    a.pq_codes = codes;
    a.radii = norms;
  }
  const int tiles = static_cast<int>((R + TK - 1) / TK);
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess) (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  const int grid = tiles < cus ? tiles : cus;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (method == 0) {
    switch (k) {
      case 1: hipLaunchKernelGGL(tq_encode_kernel<1>, dim3(grid), dim3(NT), 0, st, a, tiles); break;
      case 2: hipLaunchKernelGGL(tq_encode_kernel<2>, dim3(grid), dim3(NT), 0, st, a, tiles); break;
      case 3: hipLaunchKernelGGL(tq_encode_kernel<3>, dim3(grid), dim3(NT), 0, st, a, tiles); break;
      default: return hipErrorInvalidValue;
    }
  }
  else hipLaunchKernelGGL(pq_encode_kernel, dim3(grid), dim3(NT), 0, st, a, tiles);
  return hipGetLastError();
}

size_t tq_scores_workspace_bytes(int B, int H_q) {
  return static_cast<size_t>(B) * H_q * kQPrepBytes;
}

int launch_tq_scores(const RotqTables& tb, int k, const float* q, const uint32_t* codes,
                     const uint32_t* bits, const float* norms, const float* gammas, int B, int H_q,
                     int H_kv, int N, int cap, float* out, void* workspace, void* stream) {
  const int G = H_q / H_kv;
  // sqrt(pi/2) / m with m = d
  const float coef = static_cast<float>(1.2533141373155002512 / D);
  hipStream_t st = static_cast<hipStream_t>(stream);
  uint8_t* prep_bytes = static_cast<uint8_t*>(workspace);
  const float* prep = static_cast<const float*>(workspace);
  const float* cents = tb.tq_cents + 8 * (k - 1);
  hipLaunchKernelGGL(tq_query_kernel, dim3(B * H_q, 2), dim3(kQueryThreads), 0, st, q, tb.qtab, cents, k,
                     prep_bytes);
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess) (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  const int64_t heads = static_cast<int64_t>(B) * H_kv;
  if (k != 3) {
    // up to eight workgroups per compute unit, each a multiple of 256 tokens
    const int64_t chunks = (N + 255) / 256;
    const int64_t want8 = 8 * static_cast<int64_t>(cus) / heads, want = want8 > 1 ? want8 : 1;
    const int tpw = static_cast<int>((chunks + want - 1) / want * 256);
    dim3 grid((N + tpw - 1) / tpw, H_kv, B);
#define QJL_TQ_MFMA(GG)                                                                                       \
  if (k == 1) hipLaunchKernelGGL((tq_scores_mfma_kernel<GG, 1>), grid, dim3(256), 0, st, prep_bytes, codes, bits, \
                                 norms, gammas, H_kv, N, cap, tpw, coef, out);                                  \
  else hipLaunchKernelGGL((tq_scores_mfma_kernel<GG, 2>), grid, dim3(256), 0, st, prep_bytes, codes, bits, norms, \
                          gammas, H_kv, N, cap, tpw, coef, out)
    switch (G) {
      case 1: QJL_TQ_MFMA(1); break;
      case 2: QJL_TQ_MFMA(2); break;
      case 4: QJL_TQ_MFMA(4); break;
      case 8: QJL_TQ_MFMA(8); break;
      default: return hipErrorInvalidValue;
    }
#undef QJL_TQ_MFMA
    return hipGetLastError();
  }
  // k = 3: about two workgroups per compute unit, each a multiple of 256 tokens
  const int64_t want = (2 * static_cast<int64_t>(cus) + heads - 1) / heads;
  const int64_t per = (N + want - 1) / want;
  const int tpw = static_cast<int>((per + 255) / 256 * 256);
  dim3 grid((N + tpw - 1) / tpw, H_kv, B);
#define QJL_TQ_SCORES(GG)                                                                              \
  hipLaunchKernelGGL((tq_scores_kernel<GG>), grid, dim3(256), 0, st, prep, codes, bits, norms, gammas, cents, \
                     H_kv, N, cap, tpw, coef, out)
  switch (G) {
    case 1: QJL_TQ_SCORES(1); break;
    case 2: QJL_TQ_SCORES(2); break;
    case 4: QJL_TQ_SCORES(4); break;
    case 8: QJL_TQ_SCORES(8); break;
    default: return hipErrorInvalidValue;
  }
#undef QJL_TQ_SCORES
  return hipGetLastError();
}

}  // namespace qjl
