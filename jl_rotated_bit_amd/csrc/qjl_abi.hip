// C ABI of the QJL library: argument validation, the per-device cache of S,
// and dispatch to the encode / decode kernels.  Declarations and the full
// contract of every entry point are in include/qjl.h.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <tuple>
#include <vector>

#include "internal.h"
#include "qjl.h"

namespace {

constexpr int32_t kAbiVersion = 1;

thread_local std::string g_last_error;

qjl_status fail(qjl_status code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool supported_dm(int d, int m) { return d == qjl::kHeadDim && (m == 256 || m == 512); }

// ---- device cache of S, keyed by (device, seed, d, m) ----
struct CacheEntry {
  qjl::DeviceSketch view;
  void* mem = nullptr;  // one allocation holding every device copy of S
};

std::mutex g_cache_mu;
std::map<std::tuple<int, uint64_t, int, int>, CacheEntry> g_cache;

qjl_status get_sketch(uint64_t seed, int d, int m, qjl::DeviceSketch* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(QJL_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  std::lock_guard<std::mutex> lock(g_cache_mu);
  const auto key = std::make_tuple(dev, seed, d, m);
  auto it = g_cache.find(key);
  if (it != g_cache.end()) {
    *out = it->second.view;
    return QJL_OK;
  }
  const size_t n = static_cast<size_t>(d) * m;
  std::vector<uint16_t> s_dm(n), s_md(n);
  qjl::generate_sketch_bf16(seed, d, m, s_dm.data());
  for (int j = 0; j < d; ++j)
    for (int i = 0; i < m; ++i) s_md[static_cast<size_t>(i) * d + j] = s_dm[static_cast<size_t>(j) * m + i];
  // max column norm per group of 64 sketch coordinates, rounded up to fp32
  std::vector<float> cmax(m / 64);
  for (int g = 0; g < m / 64; ++g) {
    double best = 0.0;
    for (int i = 64 * g; i < 64 * g + 64; ++i) {
      double ss = 0.0;
      for (int j = 0; j < d; ++j) {
        uint32_t u = static_cast<uint32_t>(s_dm[static_cast<size_t>(j) * m + i]) << 16;
        float f;
        std::memcpy(&f, &u, sizeof(f));
        ss += static_cast<double>(f) * f;
      }
      best = std::max(best, std::sqrt(ss));
    }
    cmax[g] = std::nextafter(static_cast<float>(best), INFINITY);
  }
  std::vector<uint16_t> s_frag(n);
  for (int blk = 0; blk < m / 32; ++blk)
    for (int st = 0; st < d / 16; ++st)
      for (int l = 0; l < 64; ++l)
        for (int e = 0; e < 8; ++e)
          s_frag[((static_cast<size_t>(blk) * (d / 16) + st) * 64 + l) * 8 + e] =
              s_md[static_cast<size_t>(32 * blk + l % 32) * d + 16 * st + 8 * (l / 32) + e];
  std::vector<uint16_t> s_efrag(n);
  for (int w = 0; w < m / 64; ++w)
    for (int b = 0; b < 2; ++b)
      for (int st = 0; st < d / 16; ++st)
        for (int l = 0; l < 64; ++l) {
          const int jj = l % 32, hh = l / 32;
          const int coord = 64 * w + 32 * ((jj >> 2) & 1) + 16 * b + 4 * (jj >> 3) + (jj & 3);
          for (int e = 0; e < 8; ++e)
            s_efrag[(((static_cast<size_t>(w) * 2 + b) * (d / 16) + st) * 64 + l) * 8 + e] =
                static_cast<uint16_t>(s_md[static_cast<size_t>(coord) * d + 16 * st + 8 * hh + e] ^ 0x8000u);
        }
  const size_t bytes_s = n * sizeof(uint16_t);
  const size_t padded = (bytes_s + 255) / 256 * 256;
  const size_t off_md = padded;
  const size_t off_fr = off_md + padded;
  const size_t off_ef = off_fr + padded;
  const size_t off_cm = off_ef + padded;
  const size_t total = off_cm + cmax.size() * sizeof(float);
  void* mem = nullptr;
  e = hipMalloc(&mem, total);
  if (e != hipSuccess) return fail(QJL_ENOMEM, "hipMalloc(%zu) for S: %s", total, hipGetErrorString(e));
  auto* base = static_cast<uint8_t*>(mem);
  e = hipMemcpy(base, s_dm.data(), bytes_s, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(base + off_md, s_md.data(), bytes_s, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(base + off_fr, s_frag.data(), bytes_s, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(base + off_ef, s_efrag.data(), bytes_s, hipMemcpyHostToDevice);
  if (e == hipSuccess)
    e = hipMemcpy(base + off_cm, cmax.data(), cmax.size() * sizeof(float), hipMemcpyHostToDevice);
  if (e != hipSuccess) {
    (void)hipFree(mem);
    return fail(QJL_EHIP, "uploading S: %s", hipGetErrorString(e));
  }
  CacheEntry ce;
  ce.mem = mem;
  ce.view.s_dm = reinterpret_cast<const uint16_t*>(base);
  ce.view.s_md = reinterpret_cast<const uint16_t*>(base + off_md);
  ce.view.s_frag = reinterpret_cast<const uint16_t*>(base + off_fr);
  ce.view.s_efrag = reinterpret_cast<const uint16_t*>(base + off_ef);
  ce.view.col_norm_max = reinterpret_cast<const float*>(base + off_cm);
  for (float c : cmax) ce.view.col_norm_all = std::max(ce.view.col_norm_all, c);
  ce.view.d = d;
  ce.view.m = m;
  g_cache.emplace(key, ce);
  *out = ce.view;
  return QJL_OK;
}

}  // namespace

extern "C" {

QJL_API int32_t qjl_abi_version(void) { return kAbiVersion; }

QJL_API const char* qjl_last_error(void) { return g_last_error.c_str(); }

QJL_API qjl_status qjl_sketch_host(uint64_t seed, int32_t d, int32_t m, uint16_t* out) {
  g_last_error.clear();
  if (out == nullptr) return fail(QJL_EINVAL, "qjl_sketch_host: out is NULL");
  if (d <= 0 || m <= 0) return fail(QJL_EINVAL, "qjl_sketch_host: d=%d m=%d must be positive", d, m);
  if (static_cast<int64_t>(d) * m > (int64_t{1} << 26))
    return fail(QJL_EINVAL, "qjl_sketch_host: d*m too large");
  qjl::generate_sketch_bf16(seed, d, m, out);
  return QJL_OK;
}

QJL_API qjl_status qjl_encode_keys(const void* keys_bf16, int32_t B, int32_t H_kv, int32_t n,
                                   int32_t d, int32_t m, uint64_t seed, uint32_t* signs,
                                   float* norms, int32_t cap, int32_t pos, void* stream) {
  g_last_error.clear();
  if (!supported_dm(d, m))
    return fail(QJL_EUNSUPPORTED, "qjl_encode_keys: d=%d m=%d unsupported (d=128, m in {256,512})", d, m);
  if (B <= 0 || H_kv <= 0 || n < 0 || cap <= 0 || pos < 0)
    return fail(QJL_EINVAL, "qjl_encode_keys: bad sizes B=%d H_kv=%d n=%d cap=%d pos=%d", B, H_kv, n, cap, pos);
  if (static_cast<int64_t>(pos) + n > cap)
    return fail(QJL_EINVAL, "qjl_encode_keys: pos+n=%lld exceeds cap=%d",
                static_cast<long long>(pos) + n, cap);
  if (static_cast<int64_t>(B) * H_kv * cap > (int64_t{1} << 40))
    return fail(QJL_EINVAL, "qjl_encode_keys: cache too large");
  if (static_cast<int64_t>(B) * H_kv * n > INT32_MAX)
    return fail(QJL_EINVAL, "qjl_encode_keys: B*H_kv*n=%lld keys in one call (at most 2^31 - 1)",
                static_cast<long long>(B) * H_kv * n);
  if (n == 0) return QJL_OK;
  if (keys_bf16 == nullptr || signs == nullptr || norms == nullptr)
    return fail(QJL_EINVAL, "qjl_encode_keys: NULL pointer");
  if (!aligned(keys_bf16, 16) || !aligned(signs, 16) || !aligned(norms, 4))
    return fail(QJL_EINVAL, "qjl_encode_keys: misaligned pointer (keys/signs need 16 B, norms 4 B)");
  qjl::DeviceSketch s;
  qjl_status st = get_sketch(seed, d, m, &s);
  if (st != QJL_OK) return st;
  const int e = qjl::launch_encode(s, keys_bf16, B, H_kv, n, signs, norms, cap, pos, stream);
  if (e != hipSuccess)
    return fail(QJL_EHIP, "qjl_encode_keys: launch failed: %s", hipGetErrorString(static_cast<hipError_t>(e)));
  return QJL_OK;
}

QJL_API int32_t qjl_set_encode_small_max(int32_t keys) { return qjl::set_encode_small_max(keys); }

QJL_API int32_t qjl_decode_num_splits(int32_t B, int32_t H_q, int32_t H_kv, int32_t N, int32_t d,
                                      int32_t m) {
  qjl::DecodePlan p;
  if (!qjl::make_decode_plan(B, H_q, H_kv, N, d, m, &p)) return 0;
  return p.n_split;
}

QJL_API size_t qjl_decode_workspace_bytes(int32_t B, int32_t H_q, int32_t H_kv, int32_t N,
                                          int32_t d, int32_t m) {
  qjl::DecodePlan p;
  if (!qjl::make_decode_plan(B, H_q, H_kv, N, d, m, &p)) return 0;
  return p.total_bytes;
}

QJL_API qjl_status qjl_decode_attention(const float* q, const uint32_t* signs, const float* norms,
                                        const void* values_bf16, int32_t B, int32_t H_q,
                                        int32_t H_kv, int32_t N, int32_t cap, int32_t d,
                                        int32_t m, uint64_t seed, float scale, float* out,
                                        void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  if (!supported_dm(d, m))
    return fail(QJL_EUNSUPPORTED, "qjl_decode_attention: d=%d m=%d unsupported (d=128, m in {256,512})", d, m);
  if (B <= 0 || H_q <= 0 || H_kv <= 0 || cap <= 0 || N <= 0 || N > cap)
    return fail(QJL_EINVAL, "qjl_decode_attention: bad sizes B=%d H_q=%d H_kv=%d N=%d cap=%d", B, H_q, H_kv, N, cap);
  if (H_q % H_kv != 0)
    return fail(QJL_EINVAL, "qjl_decode_attention: H_q=%d is not a multiple of H_kv=%d", H_q, H_kv);
  const int G = H_q / H_kv;
  if (G != 1 && G != 2 && G != 4 && G != 8)
    return fail(QJL_EUNSUPPORTED, "qjl_decode_attention: G=H_q/H_kv=%d unsupported (1, 2, 4, 8)", G);
  if (static_cast<int64_t>(B) * H_kv * cap > (int64_t{1} << 40))
    return fail(QJL_EINVAL, "qjl_decode_attention: cache too large");
  if (!(scale >= 0.0f) || std::isinf(scale))
    return fail(QJL_EINVAL, "qjl_decode_attention: scale must be finite and >= 0");
  if (q == nullptr || signs == nullptr || norms == nullptr || values_bf16 == nullptr || out == nullptr)
    return fail(QJL_EINVAL, "qjl_decode_attention: NULL pointer");
  if (!aligned(q, 16) || !aligned(signs, 16) || !aligned(norms, 4) || !aligned(values_bf16, 16) ||
      !aligned(out, 16))
    return fail(QJL_EINVAL, "qjl_decode_attention: misaligned pointer");
  qjl::DecodePlan plan;
  if (!qjl::make_decode_plan(B, H_q, H_kv, N, d, m, &plan))
    return fail(QJL_EINVAL, "qjl_decode_attention: no plan for these sizes");
  if (plan.n_split > 1) {
    if (workspace == nullptr || !aligned(workspace, 256))
      return fail(QJL_EWORKSPACE, "qjl_decode_attention: workspace NULL or not 256-byte aligned");
    if (workspace_bytes < plan.total_bytes)
      return fail(QJL_EWORKSPACE, "qjl_decode_attention: workspace %zu bytes < %zu needed",
                  workspace_bytes, plan.total_bytes);
  }
  qjl::DeviceSketch s;
  qjl_status st = get_sketch(seed, d, m, &s);
  if (st != QJL_OK) return st;
  const float sc = scale == 0.0f ? static_cast<float>(1.0 / std::sqrt(static_cast<double>(d))) : scale;
  const int e = qjl::launch_decode(s, plan, q, signs, norms, values_bf16, B, H_q, H_kv, N, cap, sc,
                                   out, workspace, stream);
  if (e != hipSuccess)
    return fail(QJL_EHIP, "qjl_decode_attention: launch failed: %s", hipGetErrorString(static_cast<hipError_t>(e)));
  return QJL_OK;
}

QJL_API qjl_status qjl_release_cache(void) {
  g_last_error.clear();
  std::lock_guard<std::mutex> lock(g_cache_mu);
  int cur = 0;
  const bool have_dev = hipGetDevice(&cur) == hipSuccess;
  qjl_status rc = QJL_OK;
  for (auto& kv : g_cache) {
    const int dev = std::get<0>(kv.first);
    if (hipSetDevice(dev) == hipSuccess) {
      (void)hipDeviceSynchronize();
      if (hipFree(kv.second.mem) != hipSuccess) rc = fail(QJL_EHIP, "qjl_release_cache: hipFree failed");
    }
  }
  g_cache.clear();
  if (have_dev) (void)hipSetDevice(cur);
  return rc;
}

}  // extern "C"
