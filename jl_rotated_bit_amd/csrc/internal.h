// Internal interfaces between the C ABI layer (qjl_abi.hip), the host sketch
// generator (sketch.cpp) and the kernel launchers (encode.hip, decode.hip).
#pragma once

#include <cstddef>
#include <cstdint>

namespace qjl {

constexpr int kHeadDim = 128;

// bf16 bit patterns of S ([d][m] row-major) for a seed; see sketch.cpp.
void generate_sketch_bf16(uint64_t seed, int d, int m, uint16_t* out);
// The fp64 normals behind it (element e = j*m + i), before any rounding.
void generate_normals_f64(uint64_t seed, int d, int m, double* out);

// ---- rotate-then-quantize tables (rotq_host.cpp) ----
// The Haar rotation of a seed: QR of the d x d normals of generate_normals_f64
// with R's diagonal made positive, Q rounded to fp32, row-major Pi[i][j].
void make_rotation_f32(uint64_t seed, int d, float* out);
// TurboQuant: the Lloyd-Max codebook (2^k centroids, ascending) of one
// coordinate of a randomly rotated unit vector in d dimensions, rounded to
// multiples of 2^-20.
void make_tq_codebook(int d, int k, float* centroids);
// PolarQuant: centroids (2^bits angles) and tangent thresholds of a level's
// codebook (level 1: the 2^bits / 4 - 1 thresholds inside one quadrant;
// level >= 2: the 2^bits - 1 thresholds), multiples of 2^-20.
void make_pq_codebook(int level, int bits, float* centroids, float* thresholds);

// Device-resident copies of one S, kept by the cache in qjl_abi.hip.
struct DeviceSketch {
  const uint16_t* s_dm = nullptr;   // [d][m]  bf16 bits (decode: S^T q)
  const uint16_t* s_md = nullptr;   // [m][d]  bf16 bits (encode: matrix-core A operand)
  // S^T in the lane order of the A operand of v_mfma_f32_32x32x16_bf16:
  // [m/32 blocks][8 k-steps][64 lanes][8 bf16], lane l holding
  // S^T[32*block + l%32][16*kstep + 8*(l/32) .. +7] (decode: S^T q)
  const uint16_t* s_frag = nullptr;
  // -S^T (sign bits flipped) in the lane order of the encode's resident A
  // operand (v_mfma_f32_32x32x16_bf16): [m/64 waves][2 blocks][8 k-steps][64
  // lanes][8 bf16], lane (j, h) of (wave w, block b, k-step s) holding
  // -S^T[64w + 32((j >> 2) & 1) + 16b + 4(j >> 3) + (j & 3)][16s + 8h .. +7]
  // (j = lane % 32, h = lane / 32), so each (w, b, s) is one contiguous 1 KB load.
  const uint16_t* s_efrag = nullptr;
  const float* col_norm_max = nullptr;  // [m/64] max_{i in group} ||S[:, i]||_2, rounded up
  float col_norm_all = 0.f;             // max over all m columns of ||S[:, i]||_2, rounded up
  int d = 0;
  int m = 0;
};

// The decode workspace starts with a fixed region of arrival counters (one
// uint32 per (batch, kv head)); calls with more streams than that never split.
constexpr size_t kCounterRegionBytes = 4096;
constexpr int64_t kMaxCounters = kCounterRegionBytes / 4;

// Decode split geometry, shared by the workspace query and the launch.
struct DecodePlan {
  int waves = 4;            // waves per workgroup (4 or 8)
  int n_split = 0;          // context splits per (batch, kv head)
  int tokens_per_split = 0; // multiple of the token tile
  size_t counter_bytes = 0; // kCounterRegionBytes
  size_t partial_bytes = 0; // B*H_q*n_split*(d + 2) floats
  size_t total_bytes = 0;
};

bool make_decode_plan(int B, int H_q, int H_kv, int N, int d, int m, DecodePlan* plan);

// Kernel launchers; return the HIP error code (0 == hipSuccess).
int launch_encode(const DeviceSketch& s, const void* keys, int B, int H_kv, int n, uint32_t* signs,
                  float* norms, int cap, int pos, void* stream);

// Encode calls with at most this many keys (B * H_kv * n) use the small-set
// kernel; set_encode_small_max changes the calling thread's limit (negative:
// query only) and returns the previous one.
constexpr int kEncodeSmallMaxDefault = 512;
int set_encode_small_max(int keys);

// The decode step's append: token `pos` (= N - 1) of every (batch, kv head)
// is encoded from `key` and its value copied from `val` (both bf16
// [B][H_kv][d]) into row `pos` of the caches, inside the decode launch.
struct AppendArgs {
  const uint16_t* key = nullptr;
  const uint16_t* val = nullptr;
  const uint16_t* s_md = nullptr;   // S^T [m][d] bf16 bits
  uint32_t* signs = nullptr;
  float* norms = nullptr;
  uint16_t* values = nullptr;
  int pos = 0;
};

// app == nullptr: a plain decode step; otherwise the step appends first.
int launch_decode(const DeviceSketch& s, const DecodePlan& plan, const float* q,
                  const uint32_t* signs, const float* norms, const void* values, int B, int H_q,
                  int H_kv, int N, int cap, float scale, float* out, void* workspace,
                  const AppendArgs* app, void* stream);

// The uncompressed baseline: exact softmax attention over bf16 keys and
// values with the same split plan, softmax, P.V and merge as the decode.
int launch_decode_bf16(const DecodePlan& plan, const float* q, const void* keys, const void* values,
                       int B, int H_q, int H_kv, int N, int cap, float scale, float* out,
                       void* workspace, void* stream);

// Device copies of the rotate-then-quantize tables of one seed.
struct RotqTables {
  const float* rot = nullptr;     // Pi [i][j] fp32
  const float* rotT = nullptr;    // Pi^T [j][i] fp32
  const uint16_t* s_il = nullptr; // QJL sketch of seed + 1 with m = d, bf16 [i][l]
  const float* tq_cents = nullptr;  // TurboQuant centroids, k = 1..3 at 8 * (k - 1)
  const float* pq_thr = nullptr;    // PolarQuant thresholds [7 levels][8]
  const float* qtab = nullptr;     // [j][r]: rows r of [Pi; S^T Pi] (2d of them), fp32
  float rot_row_max = 0.f;        // max_i ||Pi_i|| rounded up
  float s_col_max = 0.f;          // max_l ||S[:, l]|| rounded up
};
constexpr int kPqBits[7] = {4, 2, 2, 2, 2, 2, 2};   // PolarQuant bits per level (d = 128)

// method 0: TurboQuant_prod with k MSE bits (codes, bits, norms, gammas);
// method 1: PolarQuant (codes -> cells, norms -> radii).  margin_log2 > 0
// widens the certificates (test hook: routes values to the exact paths).
int launch_rotq_encode(const RotqTables& tb, int method, int k, const void* keys, int B, int H_kv, int n,
                       uint32_t* codes, uint32_t* bits, float* norms, float* gammas, int cap, int pos,
                       int margin_log2, void* stream);
// the scores' workspace: the prepared queries, 4096 bytes a query head
size_t tq_scores_workspace_bytes(int B, int H_q);
int launch_tq_scores(const RotqTables& tb, int k, const float* q, const uint32_t* codes,
                     const uint32_t* bits, const float* norms, const float* gammas, int B, int H_q,
                     int H_kv, int N, int cap, float* out, void* workspace, void* stream);

}  // namespace qjl
