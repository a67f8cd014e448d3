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
// * Prologue: S^T q for the G heads (fp32) and, from it, a table in LDS of the
//   16 possible signed sums of every group of 4 consecutive sketch
//   coordinates (per head).  The bit dot product of a token then costs m/4
//   table reads and adds per head instead of m masked adds.
// * Main loop: a wave takes 64 tokens at a time.  Lane t of the wave scores
//   token t (its m/32 sign words and norm arrive with 16-byte loads); the
//   wave does the online-softmax update; then lanes regroup to 16 per token
//   row and accumulate p * v over 16-byte value chunks.  The next tile's loads
//   are issued before the current tile is used.
// * Epilogue: waves merge in LDS; the workgroup writes its partial
//   (max, sum, acc) per head; the last workgroup of a (batch, kv head) to
//   arrive (atomic counter) merges all splits by log-sum-exp and writes out,
//   then returns the counter to zero.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "internal.h"

namespace qjl {
namespace {

constexpr int D = kHeadDim;
constexpr int NW = 4;            // waves per workgroup
constexpr int NT = 64 * NW;
constexpr int TILE = 64;         // tokens per wave per step
constexpr int VCH = TILE * D * 2 / 16 / 64;  // 16-byte value chunks per lane per tile (16)
constexpr int MAX_SPLITS = 256;

typedef __bf16 bf16x8_t __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x16_t __attribute__((__vector_size__(16 * sizeof(float))));

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float bf16lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

// G floats read or written as one LDS access (b32 / b64 / b128; two b128 for G = 8).
template <int G>
struct alignas(G >= 4 ? 16 : 4 * G) VecG {
  float v[G];
};

template <int M, int G>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(G <= 4 ? 2 : 1))) void decode_kernel(
    const float* __restrict__ q, const uint32_t* __restrict__ signs,
    const float* __restrict__ norms, const uint16_t* __restrict__ values,
    const uint16_t* __restrict__ s_md, int H_kv, int N, int cap, int n_split, int tps,
    float coef, float* __restrict__ out, uint32_t* __restrict__ counters,
    float* __restrict__ part_acc, float* __restrict__ part_ml) {
  constexpr int WPR = M / 32;        // sign words per token
  constexpr int SV = WPR / 4;        // 16-byte sign loads per token
  constexpr int NPOS = M / 4;        // nibble positions
  constexpr int LUT_FLOATS = NPOS * 16 * G;

  __shared__ __attribute__((aligned(16))) float lut[LUT_FLOATS];
  __shared__ __attribute__((aligned(16))) float qs[G][D];
  __shared__ __attribute__((aligned(16))) float sq[G][M];
  __shared__ __attribute__((aligned(16))) float pbuf[NW][TILE][G];
  // wave partials [NW][G][D] after the loop; merge replicas [REP][G*D/4] float4 later
  constexpr int RED_FLOATS = (NW * G * D > 4 * NT) ? NW * G * D : 4 * NT;
  __shared__ __attribute__((aligned(16))) float red_buf[RED_FLOATS];
  __shared__ float red_ml[NW][G][2];
  __shared__ int is_last;

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

  // ---- first tile's loads go out before the prologue ----
  uint4 vc[VCH];
  uint4 sc[SV];
  float nc;
  auto load_tile = [&](int t0, uint4* vv, uint4* ss, float& nn) {
    const int ts = t0 + lane;
    if (ts < t_end) {
      const uint4* p = reinterpret_cast<const uint4*>(sg_base + static_cast<int64_t>(ts) * WPR);
#pragma unroll
      for (int k = 0; k < SV; ++k) ss[k] = p[k];
      nn = nm_base[ts];
    } else {
#pragma unroll
      for (int k = 0; k < SV; ++k) ss[k] = make_uint4(0, 0, 0, 0);
      nn = 0.f;
    }
#pragma unroll
    for (int c = 0; c < VCH; ++c) {
      const int tv = t0 + 4 * c + (lane >> 4);
      vv[c] = tv < t_end
                  ? reinterpret_cast<const uint4*>(v_base + static_cast<int64_t>(tv) * D)[lane & 15]
                  : make_uint4(0, 0, 0, 0);
    }
  };
  int t0 = t_begin + wave * TILE;

  // ---- prologue: q -> LDS, S^T q on the matrix cores, nibble table ----
  // q is split into three bf16 parts (hi + mid + lo reproduces fp32 q to
  // within 2^-24 relative); column 3*... of the B operand holds part p of head
  // g at column p*G + g, so one 32x32x16 MFMA chain per block of 32 sketch
  // coordinates yields all parts of all heads, with fp32 accumulation.
  constexpr int NBLK = M / 32;            // blocks of 32 sketch coordinates
  constexpr int BPW = NBLK / NW;          // blocks per wave (2 or 4)
  constexpr int BATCH = 2;                // blocks whose S^T fragments are in flight together
  static_assert(BPW % BATCH == 0, "blocks per wave must be a multiple of the batch");
  const int col = lane & 31;
  const int half = lane >> 5;
  uint4 af[BATCH][8];
  auto load_frags = [&](int batch) {
#pragma unroll
    for (int bb = 0; bb < BATCH; ++bb) {
      const int blk = wave + NW * (batch * BATCH + bb);
      const uint4* arow = reinterpret_cast<const uint4*>(s_md + static_cast<int64_t>(32 * blk + col) * D);
#pragma unroll
      for (int st = 0; st < 8; ++st) af[bb][st] = arow[2 * st + half];
    }
  };
  load_frags(0);

  // Issue order matters: the S^T fragments and q are loaded before the first
  // tile, so waiting for q (memory counters drain in order) does not also
  // wait for the tile, which stays in flight through the whole prologue.
  const float* qb = q + (static_cast<int64_t>(b) * H_kv + kvh) * G * D;
  constexpr int QPT = (G * D + NT - 1) / NT;
  float qv[QPT];
#pragma unroll
  for (int k = 0; k < QPT; ++k) qv[k] = (tid + k * NT < G * D) ? qb[tid + k * NT] : 0.f;
  if (t0 < t_end) load_tile(t0, vc, sc, nc);
#pragma unroll
  for (int k = 0; k < QPT; ++k) {
    const int i = tid + k * NT;
    if (i < G * D) qs[i / D][i % D] = qv[k];
  }
  __syncthreads();
  {
    const int part = col / G;
    const int g = col % G;
    bf16x8_t bq[8];
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      uint32_t pk[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        uint32_t h2[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const float x = part < 3 ? qs[g][16 * st + 8 * half + e + u] : 0.f;
          const uint32_t hi = f32_to_bf16_rne(x);
          const float r1 = x - __uint_as_float(hi << 16);
          const uint32_t mid = f32_to_bf16_rne(r1);
          const float r2 = r1 - __uint_as_float(mid << 16);
          const uint32_t lo = f32_to_bf16_rne(r2);
          h2[u] = part == 0 ? hi : (part == 1 ? mid : lo);
        }
        pk[e / 2] = h2[0] | (h2[1] << 16);
      }
      bq[st] = __builtin_bit_cast(bf16x8_t, make_uint4(pk[0], pk[1], pk[2], pk[3]));
    }
#pragma unroll
    for (int batch = 0; batch < BPW / BATCH; ++batch) {
      if (batch > 0) load_frags(batch);
#pragma unroll
      for (int bb = 0; bb < BATCH; ++bb) {
        const int blk = wave + NW * (batch * BATCH + bb);
        f32x16_t acc = {};
#pragma unroll
        for (int st = 0; st < 8; ++st)
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, af[bb][st]), bq[st], acc, 0, 0, 0);
        // lane (col, half), register r -> coordinate 32*blk + 8*(r/4) + 4*half + r%4
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float v = acc[r] + __shfl(acc[r], lane + G) + __shfl(acc[r], lane + 2 * G);
          if (col < G) sq[col][32 * blk + 8 * (r >> 2) + 4 * half + (r & 3)] = v;
        }
      }
    }
  }
  __syncthreads();
  for (int e = tid; e < NPOS * 16; e += NT) {
    const int p = e >> 4, v = e & 15;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float sacc = 0.f;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float x = sq[g][4 * p + k];
        sacc += ((v >> k) & 1) ? x : -x;
      }
      lut[e * G + g] = sacc;
    }
  }
  __syncthreads();

  // ---- main loop ----
  float m_run[G], l_run[G], acc[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m_run[g] = -INFINITY;
    l_run[g] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[g][e] = 0.f;
  }

  while (t0 < t_end) {
    const int t_next = t0 + NW * TILE;
    uint4 vn[VCH];
    uint4 sn[SV];
    float nn = 0.f;
    if (t_next < t_end) load_tile(t_next, vn, sn, nn);

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
      }
    }
    const bool valid = (t0 + lane) < t_end;
    VecG<G> pw;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float logit = valid ? sc_g[g] * (coef * nc) : -INFINITY;
      const float tmax = wave_max(logit);
      const float m_new = fmaxf(m_run[g], tmax);
      const float alpha = exp2f(m_run[g] - m_new);
      const float p = valid ? exp2f(logit - m_new) : 0.f;
      l_run[g] = l_run[g] * alpha + p;
      m_run[g] = m_new;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[g][e] *= alpha;
      pw.v[g] = p;
    }
    *reinterpret_cast<VecG<G>*>(&pbuf[wave][lane][0]) = pw;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // p * v: lane <-> (token 4c + lane/16, channels 8*(lane%16) .. +7)
#pragma unroll
    for (int c = 0; c < VCH; ++c) {
      const VecG<G> pt = *reinterpret_cast<const VecG<G>*>(&pbuf[wave][4 * c + (lane >> 4)][0]);
      const float v8[8] = {bf16lo(vc[c].x), bf16hi(vc[c].x), bf16lo(vc[c].y), bf16hi(vc[c].y),
                           bf16lo(vc[c].z), bf16hi(vc[c].z), bf16lo(vc[c].w), bf16hi(vc[c].w)};
#pragma unroll
      for (int g = 0; g < G; ++g) {
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[g][e] = __builtin_fmaf(pt.v[g], v8[e], acc[g][e]);
      }
    }
    __builtin_amdgcn_wave_barrier();

    t0 = t_next;
#pragma unroll
    for (int c = 0; c < VCH; ++c) vc[c] = vn[c];
#pragma unroll
    for (int k = 0; k < SV; ++k) sc[k] = sn[k];
    nc = nn;
  }

  // ---- merge within the wave, then across waves ----
#pragma unroll
  for (int g = 0; g < G; ++g) {
    l_run[g] = wave_sum(l_run[g]);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float x = acc[g][e];
      x += __shfl_xor(x, 16);
      x += __shfl_xor(x, 32);
      acc[g][e] = x;
    }
  }
  if (lane < 16) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int e = 0; e < 8; ++e) red_buf[(wave * G + g) * D + 8 * lane + e] = acc[g][e];
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
    float L = 0.f, A = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float mw = red_ml[w][g][0];
      const float f = mw == -INFINITY ? 0.f : exp2f(mw - mx);
      L += red_ml[w][g][1] * f;
      A += red_buf[(w * G + g) * D + dd] * f;
    }
    if (n_split == 1) {
      out[(bh * G + g) * D + dd] = A / L;
    } else {
      // coherent (sc1) stores: visible to every XCD once complete, with no
      // L2-wide write-back (an agent-scope fence would flush the whole L2)
      __hip_atomic_store(&part_acc[(slot0 * G + g) * D + dd], A, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
      if (dd == 0) {
        __hip_atomic_store(&part_ml[(slot0 * G + g) * 2 + 0], mx, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&part_ml[(slot0 * G + g) * 2 + 1], L, __ATOMIC_RELAXED,
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
  // (1) all (max, sum) pairs into LDS in one round of loads
  float* ml_l = lut;                      // 2 * n_split * G floats
  float* wts = lut + 2 * MAX_SPLITS * G;  // n_split * G floats
  static_assert(3 * MAX_SPLITS * G <= LUT_FLOATS, "merge scratch exceeds the table");
  {
    const float2* src = reinterpret_cast<const float2*>(part_ml + bh * n_split * G * 2);
    for (int i = tid; i < n_split * G; i += NT) reinterpret_cast<float2*>(ml_l)[i] = src[i];
  }
  __syncthreads();
  // (2) per head: global max and normalizer, then per-split weights
  __shared__ float gmax[G], gsum[G];
  for (int g = wave; g < G; g += NW) {
    float mx = -INFINITY;
    for (int s = lane; s < n_split; s += 64) mx = fmaxf(mx, ml_l[(s * G + g) * 2]);
    mx = wave_max(mx);
    float L = 0.f;
    for (int s = lane; s < n_split; s += 64) L += ml_l[(s * G + g) * 2 + 1] * exp2f(ml_l[(s * G + g) * 2] - mx);
    L = wave_sum(L);
    if (lane == 0) {
      gmax[g] = mx;
      gsum[g] = L;
    }
  }
  __syncthreads();
  for (int i = tid; i < n_split * G; i += NT) wts[i] = exp2f(ml_l[2 * i] - gmax[i % G]) / gsum[i % G];
  __syncthreads();
  // (3) weighted sum of the partial accumulators.  Threads own (head, 4
  // channels) pairs; with fewer pairs than threads the splits are divided
  // among REP replicas whose sums meet in LDS.  Loads go out 8 at a time.
  {
    constexpr int PAIRS = G * D / 4;
    constexpr int REP = PAIRS >= NT ? 1 : NT / PAIRS;
    static_assert(REP == 1 || REP * PAIRS * 4 <= RED_FLOATS, "merge replicas exceed the LDS buffer");
    float4* rbuf = reinterpret_cast<float4*>(red_buf);
    const float4* pa = reinterpret_cast<const float4*>(part_acc);
    for (int i = tid; i < PAIRS * REP; i += NT) {
      const int pr = i % PAIRS, rep = i / PAIRS;
      const int g = pr / (D / 4), c4 = pr % (D / 4);
      float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
      int s = rep;
      for (; s + 7 * REP < n_split; s += 8 * REP) {
        float4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = pa[((bh * n_split + s + u * REP) * G + g) * (D / 4) + c4];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const float wgt = wts[(s + u * REP) * G + g];
          o.x = __builtin_fmaf(wgt, v[u].x, o.x);
          o.y = __builtin_fmaf(wgt, v[u].y, o.y);
          o.z = __builtin_fmaf(wgt, v[u].z, o.z);
          o.w = __builtin_fmaf(wgt, v[u].w, o.w);
        }
      }
      for (; s < n_split; s += REP) {
        const float4 v = pa[((bh * n_split + s) * G + g) * (D / 4) + c4];
        const float wgt = wts[s * G + g];
        o.x = __builtin_fmaf(wgt, v.x, o.x);
        o.y = __builtin_fmaf(wgt, v.y, o.y);
        o.z = __builtin_fmaf(wgt, v.z, o.z);
        o.w = __builtin_fmaf(wgt, v.w, o.w);
      }
      if (REP == 1) {
        reinterpret_cast<float4*>(out)[(bh * G + g) * (D / 4) + c4] = o;
      } else {
        rbuf[rep * PAIRS + pr] = o;
      }
    }
    if (REP > 1) {
      __syncthreads();
      for (int pr = tid; pr < PAIRS; pr += NT) {
        float4 o = rbuf[pr];
        for (int rep = 1; rep < REP; ++rep) {
          const float4 v = rbuf[rep * PAIRS + pr];
          o.x += v.x;
          o.y += v.y;
          o.z += v.z;
          o.w += v.w;
        }
        const int g = pr / (D / 4), c4 = pr % (D / 4);
        reinterpret_cast<float4*>(out)[(bh * G + g) * (D / 4) + c4] = o;
      }
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
                     static_cast<const uint16_t*>(values), s.s_md, H_kv, N, cap, plan.n_split,
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
