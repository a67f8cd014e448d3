// Host-only exercise of the C ABI under AddressSanitizer and
// UndefinedBehaviorSanitizer (built by jl_rotated_bit_amd/build_hostsan.py,
// run by tests/test_host_sanitizers.py).  Every call here either runs on the
// host only (the table generators, the size queries) or is rejected by
// argument validation before any HIP call, so no GPU is needed.  Pointers
// passed to rejected calls are fake addresses that are never dereferenced.
// Exits 0 when every status and table check holds; prints the first failure
// otherwise.

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "qjl.h"

namespace {

int failures = 0;

#define CHECK(cond)                                                              \
  do {                                                                           \
    if (!(cond)) {                                                               \
      std::fprintf(stderr, "check failed at line %d: %s (last error: %s)\n",      \
                   __LINE__, #cond, qjl_last_error());                           \
      ++failures;                                                                \
    }                                                                            \
  } while (0)

constexpr qjl_status OK = 0, EINVAL = 1, EUNSUP = 2, EWS = 3;

void* fake(uintptr_t offset = 0) { return reinterpret_cast<void*>((uintptr_t{1} << 20) + offset); }

void host_tables() {
  // S: finite bf16 values, both sketch sizes, deterministic
  for (int m : {256, 512}) {
    std::vector<uint16_t> s(128 * m), s2(128 * m);
    CHECK(qjl_sketch_host(42, 128, m, s.data()) == OK);
    CHECK(qjl_sketch_host(42, 128, m, s2.data()) == OK);
    CHECK(s == s2);
    size_t nonzero = 0;
    for (uint16_t v : s) {
      CHECK(((v >> 7) & 0xFF) != 0xFF);
      nonzero += (v & 0x7FFF) != 0;
    }
    CHECK(nonzero > s.size() * 99 / 100);
  }
  std::vector<uint16_t> s(128 * 256);
  CHECK(qjl_sketch_host(42, 0, 256, s.data()) == EINVAL);
  CHECK(std::strlen(qjl_last_error()) > 0);
  CHECK(qjl_sketch_host(42, 1 << 14, 1 << 13, s.data()) == EINVAL);   // d*m beyond 2^26
  CHECK(qjl_sketch_host(42, 128, 256, nullptr) == EINVAL);

  // rotation: orthogonal to fp32 precision
  std::vector<float> rot(128 * 128);
  CHECK(qjl_rotation_host(42, 128, rot.data()) == OK);
  double worst = 0.0;
  for (int a = 0; a < 128; ++a)
    for (int b = a; b < 128; ++b) {
      double dot = 0.0;
      for (int j = 0; j < 128; ++j) dot += double(rot[a * 128 + j]) * rot[b * 128 + j];
      worst = std::fmax(worst, std::fabs(dot - (a == b ? 1.0 : 0.0)));
    }
  CHECK(worst < 1e-5);
  CHECK(qjl_rotation_host(42, 1, rot.data()) == EINVAL);
  CHECK(qjl_rotation_host(42, 128, nullptr) == EINVAL);

  // codebooks: ascending, symmetric, inside the support
  for (int k = 1; k <= 3; ++k) {
    std::vector<float> c(1 << k);
    CHECK(qjl_tq_codebook_host(128, k, c.data()) == OK);
    for (int v = 0; v + 1 < (1 << k); ++v) CHECK(c[v] < c[v + 1]);
    for (int v = 0; v < (1 << k); ++v) {
      CHECK(c[v] == -c[(1 << k) - 1 - v]);
      CHECK(std::fabs(c[v]) < 1.0f);
    }
  }
  std::vector<float> c(16), t(16);
  CHECK(qjl_tq_codebook_host(128, 0, c.data()) == EINVAL);
  CHECK(qjl_tq_codebook_host(128, 5, c.data()) == EINVAL);
  CHECK(qjl_pq_codebook_host(1, 4, c.data(), t.data()) == OK);
  for (int v = 0; v + 1 < 16; ++v) CHECK(c[v] < c[v + 1]);
  for (int level = 2; level <= 7; ++level) {
    CHECK(qjl_pq_codebook_host(level, 2, c.data(), t.data()) == OK);
    for (int v = 0; v + 1 < 4; ++v) CHECK(c[v] < c[v + 1] && c[v] > 0.0f && c[v + 1] < 1.5708f);
    for (int v = 0; v + 1 < 3; ++v) CHECK(t[v] < t[v + 1]);
  }
  CHECK(qjl_pq_codebook_host(1, 1, c.data(), t.data()) == EINVAL);
  CHECK(qjl_pq_codebook_host(0, 2, c.data(), t.data()) == EINVAL);
}

void sizes() {
  CHECK(qjl_abi_version() == 3);
  CHECK(qjl_decode_workspace_bytes(1, 32, 8, 32768, 128, 256) > 0);
  CHECK(qjl_decode_num_splits(1, 32, 8, 32768, 128, 256) > 1);
  CHECK(qjl_decode_workspace_bytes(1, 32, 8, 32768, 128, 384) == 0);
  CHECK(qjl_decode_num_splits(0, 32, 8, 32768, 128, 256) <= 0);
  CHECK(qjl_tq_scores_workspace_bytes(2, 8, 128) == 2 * 8 * 4096);
  CHECK(qjl_tq_scores_workspace_bytes(0, 8, 128) == 0);
  CHECK(qjl_tq_scores_workspace_bytes(2, 8, 64) == 0);
}

void rejected_calls() {
  auto* keys = static_cast<const void*>(fake());
  auto* u32 = static_cast<uint32_t*>(fake());
  auto* f32 = static_cast<float*>(fake());
  // encode
  CHECK(qjl_encode_keys(keys, 1, 1, 4, 64, 256, 1, u32, f32, 8, 0, nullptr) == EUNSUP);
  CHECK(qjl_encode_keys(keys, 1, 1, 4, 128, 384, 1, u32, f32, 8, 0, nullptr) == EUNSUP);
  CHECK(qjl_encode_keys(keys, 0, 1, 4, 128, 256, 1, u32, f32, 8, 0, nullptr) == EINVAL);
  CHECK(qjl_encode_keys(keys, 1, 1, 5, 128, 256, 1, u32, f32, 8, 4, nullptr) == EINVAL);
  CHECK(qjl_encode_keys(keys, 2, 2, 1 << 29, 128, 256, 1, u32, f32, 1 << 29, 0, nullptr) == EINVAL);
  CHECK(qjl_encode_keys(nullptr, 1, 1, 4, 128, 256, 1, u32, f32, 8, 0, nullptr) == EINVAL);
  CHECK(qjl_encode_keys(fake(8), 1, 1, 4, 128, 256, 1, u32, f32, 8, 0, nullptr) == EINVAL);
  CHECK(qjl_encode_keys(keys, 1, 1, 4, 128, 256, 1, u32, static_cast<float*>(fake(2)), 8, 0, nullptr) == EINVAL);
  CHECK(qjl_encode_keys(nullptr, 1, 1, 0, 128, 256, 1, nullptr, nullptr, 8, 0, nullptr) == OK);
  CHECK(std::strlen(qjl_last_error()) == 0);
  // decode
  auto* q = static_cast<const float*>(fake());
  const uint32_t* sg = u32;
  const float* nm = f32;
  const void* val = fake();
  float* out = f32;
  void* ws = fake();
  const size_t wsb = size_t{1} << 30;
  CHECK(qjl_decode_attention(q, sg, nm, val, 1, 4, 1, 8, 8, 96, 256, 1, 0.f, out, ws, wsb, nullptr) == EUNSUP);
  CHECK(qjl_decode_attention(q, sg, nm, val, 1, 6, 2, 8, 8, 128, 256, 1, 0.f, out, ws, wsb, nullptr) == EUNSUP);
  CHECK(qjl_decode_attention(q, sg, nm, val, 1, 6, 4, 8, 8, 128, 256, 1, 0.f, out, ws, wsb, nullptr) == EINVAL);
  CHECK(qjl_decode_attention(q, sg, nm, val, 1, 4, 1, 9, 8, 128, 256, 1, 0.f, out, ws, wsb, nullptr) == EINVAL);
  CHECK(qjl_decode_attention(q, sg, nm, val, 1, 4, 1, 8, 8, 128, 256, 1, -1.f, out, ws, wsb, nullptr) == EINVAL);
  CHECK(qjl_decode_attention(q, sg, nm, val, 1, 4, 1, 8, 8, 128, 256, 1, NAN, out, ws, wsb, nullptr) == EINVAL);
  CHECK(qjl_decode_attention(nullptr, sg, nm, val, 1, 4, 1, 8, 8, 128, 256, 1, 0.f, out, ws, wsb, nullptr) == EINVAL);
  CHECK(qjl_decode_attention(static_cast<const float*>(fake(4)), sg, nm, val, 1, 4, 1, 8, 8, 128, 256, 1, 0.f,
                             out, ws, wsb, nullptr) == EINVAL);
  CHECK(qjl_decode_attention(q, sg, nm, val, 1, 32, 8, 32768, 32768, 128, 256, 1, 0.f, out, nullptr, wsb,
                             nullptr) == EWS);
  CHECK(qjl_decode_attention(q, sg, nm, val, 1, 32, 8, 32768, 32768, 128, 256, 1, 0.f, out, ws, 16,
                             nullptr) == EWS);
  // fused step
  CHECK(qjl_decode_step(q, keys, val, u32, f32, fake(), 1, 4, 1, 8, 8, 128, 256, 1, 0.f, out, ws, wsb,
                        nullptr) == EINVAL);   // pos == cap
  CHECK(qjl_decode_step(q, keys, fake(2), u32, f32, fake(), 1, 4, 1, 3, 8, 128, 256, 1, 0.f, out, ws, wsb,
                        nullptr) == EINVAL);   // misaligned new value row
  // baseline
  CHECK(qjl_baseline_decode_attention_bf16(q, keys, val, 1, 4, 1, 8, 8, 64, 0.f, out, ws, wsb, nullptr) == EUNSUP);
  CHECK(qjl_baseline_decode_attention_bf16(q, fake(2), val, 1, 4, 1, 8, 8, 128, 0.f, out, ws, wsb, nullptr) ==
        EINVAL);
  // allocation-free decode: plans beyond the static scratch are refused
  CHECK(qjl_decode_attention_noalloc(q, sg, nm, val, 1, 4088, 511, 4096, 4096, 128, 256, 1, 0.f, out,
                                     nullptr) == EWS);
  // rotate-then-quantize
  CHECK(qjl_tq_encode_keys(keys, 1, 1, 4, 128, 0, 7, u32, u32, f32, f32, 8, 0, nullptr) == EUNSUP);
  CHECK(qjl_tq_encode_keys(fake(4), 1, 1, 4, 128, 2, 7, u32, u32, f32, f32, 8, 0, nullptr) == EINVAL);
  CHECK(qjl_pq_encode_keys(keys, 1, 1, 4, 256, 7, u32, f32, 8, 0, nullptr) == EUNSUP);
  CHECK(qjl_pq_encode_keys(keys, 1, 1, 4, 128, 7, u32, f32, 8, -1, nullptr) == EINVAL);
  CHECK(qjl_tq_scores(q, u32, u32, f32, f32, 1, 6, 2, 8, 8, 128, 2, 7, out, ws, wsb, nullptr) == EUNSUP);
  CHECK(qjl_tq_scores(q, u32, u32, f32, f32, 2, 8, 2, 8, 8, 128, 2, 7, out, nullptr, wsb, nullptr) == EWS);
  CHECK(qjl_tq_scores(q, u32, u32, f32, f32, 2, 8, 2, 8, 8, 128, 2, 7, out, ws, 64, nullptr) == EWS);
}

}  // namespace

int main() {
  host_tables();
  sizes();
  rejected_calls();
  if (failures != 0) {
    std::fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  std::printf("hostsan driver: all checks passed\n");
  return 0;
}
