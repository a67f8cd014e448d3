// Internal interfaces between the C ABI layer (qjl_abi.hip), the host sketch
// generator (sketch.cpp) and the kernel launchers (encode.hip, decode.hip).
#pragma once

#include <cstddef>
#include <cstdint>

namespace qjl {

constexpr int kHeadDim = 128;

// bf16 bit patterns of S ([d][m] row-major) for a seed; see sketch.cpp.
void generate_sketch_bf16(uint64_t seed, int d, int m, uint16_t* out);

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
// kernel; set_encode_small_max changes the limit (negative: query only) and
// returns the previous one.
constexpr int kEncodeSmallMaxDefault = 512;
int set_encode_small_max(int keys);

int launch_decode(const DeviceSketch& s, const DecodePlan& plan, const float* q,
                  const uint32_t* signs, const float* norms, const void* values, int B, int H_q,
                  int H_kv, int N, int cap, float scale, float* out, void* workspace,
                  void* stream);

}  // namespace qjl
