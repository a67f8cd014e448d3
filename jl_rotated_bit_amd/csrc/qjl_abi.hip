// C ABI of the QJL library: argument validation, the per-device cache of S,
// and dispatch to the encode / decode kernels.  Declarations and the full
// contract of every entry point are in include/qjl.h.

#include <hip/hip_runtime.h>

#include <dlfcn.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <algorithm>
#include <climits>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <tuple>
#include <vector>

#include "internal.h"
#include "qjl.h"
#include "qjl_testing.h"

// ---- library-held scratch of the allocation-free decode ----
// Arrival counters (the same fixed region a caller's workspace starts with)
// and the split partials, in one static device array; every GPU the library
// runs on holds its own copy until the process ends.  Host code never uses
// this name as an address: the per-device address comes from
// hipGetSymbolAddress (scratch_for_device below).
static constexpr size_t kScratchBytes = QJL_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes > qjl::kCounterRegionBytes, "scratch must hold the counter region");
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

constexpr int32_t kAbiVersion = 3;

thread_local std::string g_last_error;

// ---- logging and trace ranges (environment, read once) ----
// QJL_LOG=1: every failed call prints its error to stderr; QJL_LOG=2: every
// entry into a compute entry point prints its name too.  QJL_TRACE=1: each
// entry point is a roctx range (the ROCm tracer's marker API, loaded with
// dlopen on first use; the ranges show in rocprofv3 --marker-trace).
int log_level() {
  static const int level = [] {
    const char* v = std::getenv("QJL_LOG");
    return v == nullptr ? 0 : std::atoi(v);
  }();
  return level;
}

struct Roctx {
  int (*push)(const char*) = nullptr;
  int (*pop)() = nullptr;
};
const Roctx& roctx() {
  static const Roctx r = [] {
    Roctx t;
    const char* v = std::getenv("QJL_TRACE");
    if (v == nullptr || std::atoi(v) == 0) return t;
    for (const char* lib : {"librocprofiler-sdk-roctx.so.1", "libroctx64.so.4"}) {
      void* h = dlopen(lib, RTLD_NOW | RTLD_LOCAL);
      if (h == nullptr) continue;
      auto push = reinterpret_cast<int (*)(const char*)>(dlsym(h, "roctxRangePushA"));
      auto pop = reinterpret_cast<int (*)()>(dlsym(h, "roctxRangePop"));
      if (push != nullptr && pop != nullptr) {
        t.push = push;
        t.pop = pop;
        return t;
      }
    }
    if (log_level() > 0) std::fprintf(stderr, "[qjl] QJL_TRACE: no roctx library found\n");
    return t;
  }();
  return r;
}

// Entry of a public call: clears the thread's last error, logs and traces.
class CallScope {
 public:
  explicit CallScope(const char* name) : traced_(roctx().push != nullptr) {
    g_last_error.clear();
    if (log_level() >= 2) std::fprintf(stderr, "[qjl] %s\n", name);
    if (traced_) roctx().push(name);
  }
  ~CallScope() {
    if (traced_) roctx().pop();
  }
  CallScope(const CallScope&) = delete;
  CallScope& operator=(const CallScope&) = delete;

 private:
  bool traced_;
};

qjl_status fail(qjl_status code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  if (log_level() >= 1) std::fprintf(stderr, "[qjl] error %d: %s\n", static_cast<int>(code), buf);
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

// ---- device cache of the rotate-then-quantize tables, keyed by (device, seed) ----
struct RotqEntry {
  qjl::RotqTables view;
  void* mem = nullptr;
};
std::map<std::tuple<int, uint64_t>, RotqEntry> g_rotq;   // guarded by g_cache_mu
thread_local int g_rotq_margin = 0;                       // test hook

float round_up_f32(double x) { return std::nextafter(static_cast<float>(x), INFINITY); }

qjl_status get_rotq(uint64_t seed, qjl::RotqTables* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(QJL_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  std::lock_guard<std::mutex> lock(g_cache_mu);
  const auto key = std::make_tuple(dev, seed);
  auto it = g_rotq.find(key);
  if (it != g_rotq.end()) {
    *out = it->second.view;
    return QJL_OK;
  }
  constexpr int d = qjl::kHeadDim;
  std::vector<float> rot(d * d), rotT(d * d);
  qjl::make_rotation_f32(seed, d, rot.data());
  double rmax = 0.0;
  for (int i = 0; i < d; ++i) {
    double ss = 0.0;
    for (int j = 0; j < d; ++j) {
      rotT[j * d + i] = rot[i * d + j];
      ss += static_cast<double>(rot[i * d + j]) * rot[i * d + j];
    }
    rmax = std::max(rmax, std::sqrt(ss));
  }
  std::vector<uint16_t> s_il(d * d);
  qjl::generate_sketch_bf16(seed + 1, d, d, s_il.data());
  double smax = 0.0;
  for (int l = 0; l < d; ++l) {
    double ss = 0.0;
    for (int i = 0; i < d; ++i) {
      uint32_t u = static_cast<uint32_t>(s_il[i * d + l]) << 16;
      float f;
      std::memcpy(&f, &u, sizeof(f));
      ss += static_cast<double>(f) * f;
    }
    smax = std::max(smax, std::sqrt(ss));
  }
  // query table of the scores: [j][r] = row r of [Pi; M] at input j, M =
  // S^T Pi (so S^T Pi q = M q in one pass); M from fp64 sums of the stored
  // bf16 and fp32 entries, rounded to fp32
  std::vector<float> qtab(static_cast<size_t>(2 * d) * d);
  std::vector<double> m64(static_cast<size_t>(d) * d, 0.0);
  for (int i = 0; i < d; ++i)
    for (int l = 0; l < d; ++l) {
      uint32_t u = static_cast<uint32_t>(s_il[i * d + l]) << 16;
      float sf;
      std::memcpy(&sf, &u, sizeof(sf));
      for (int j = 0; j < d; ++j) m64[l * d + j] += static_cast<double>(sf) * rot[i * d + j];
    }
  for (int r = 0; r < d; ++r)
    for (int j = 0; j < d; ++j) {
      qtab[j * 2 * d + r] = rot[r * d + j];
      qtab[j * 2 * d + d + r] = static_cast<float>(m64[r * d + j]);
    }
  std::vector<float> cents(24, 0.f), thr(7 * 8, 0.f), pc(32);
  for (int k = 1; k <= 3; ++k) {
    float* c = cents.data() + 8 * (k - 1);
    qjl::make_tq_codebook(d, k, c);
    // the scores kernel for k = 1, 2 relies on c[v] = -c[2^k - 1 - v]
    for (int v = 0; v < (1 << k); ++v)
      if (c[v] != -c[(1 << k) - 1 - v]) return fail(QJL_EHIP, "TurboQuant codebook (k=%d) is not symmetric", k);
  }
  for (int lev = 1; lev <= 7; ++lev) qjl::make_pq_codebook(lev, qjl::kPqBits[lev - 1], pc.data(), thr.data() + 8 * (lev - 1));
  const size_t b_rot = d * d * 4, b_s = d * d * 2, b_c = 24 * 4, b_t = 56 * 4, b_q = qtab.size() * 4;
  const size_t o_rotT = b_rot, o_s = 2 * b_rot, o_c = o_s + b_s, o_t = o_c + 256, o_q = o_t + 256,
               total = o_q + b_q;
  void* mem = nullptr;
  e = hipMalloc(&mem, total);
  if (e != hipSuccess) return fail(QJL_ENOMEM, "hipMalloc(%zu) for the rotation tables: %s", total, hipGetErrorString(e));
  auto* base = static_cast<uint8_t*>(mem);
  e = hipMemcpy(base, rot.data(), b_rot, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(base + o_rotT, rotT.data(), b_rot, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(base + o_s, s_il.data(), b_s, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(base + o_c, cents.data(), b_c, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(base + o_t, thr.data(), b_t, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(base + o_q, qtab.data(), b_q, hipMemcpyHostToDevice);
  if (e != hipSuccess) {
    (void)hipFree(mem);
    return fail(QJL_EHIP, "uploading the rotation tables: %s", hipGetErrorString(e));
  }
  RotqEntry ent;
  ent.mem = mem;
  ent.view.rot = reinterpret_cast<const float*>(base);
  ent.view.rotT = reinterpret_cast<const float*>(base + o_rotT);
  ent.view.s_il = reinterpret_cast<const uint16_t*>(base + o_s);
  ent.view.tq_cents = reinterpret_cast<const float*>(base + o_c);
  ent.view.pq_thr = reinterpret_cast<const float*>(base + o_t);
  ent.view.rot_row_max = round_up_f32(rmax);
  ent.view.s_col_max = round_up_f32(smax);
  ent.view.qtab = reinterpret_cast<const float*>(base + o_q);
  g_rotq.emplace(key, ent);
  *out = ent.view;
  return QJL_OK;
}

qjl_status check_rows(const char* fn, int32_t B, int32_t H_kv, int32_t n, int32_t cap, int32_t pos) {
  if (B <= 0 || H_kv <= 0 || n < 0 || cap <= 0 || pos < 0)
    return fail(QJL_EINVAL, "%s: bad sizes B=%d H_kv=%d n=%d cap=%d pos=%d", fn, B, H_kv, n, cap, pos);
  if (static_cast<int64_t>(pos) + n > cap)
    return fail(QJL_EINVAL, "%s: pos+n=%lld exceeds cap=%d", fn, static_cast<long long>(pos) + n, cap);
  if (static_cast<int64_t>(B) * H_kv * cap > (int64_t{1} << 40)) return fail(QJL_EINVAL, "%s: cache too large", fn);
  if (static_cast<int64_t>(B) * H_kv * n > INT32_MAX)
    return fail(QJL_EINVAL, "%s: B*H_kv*n=%lld keys in one call (at most 2^31 - 1)", fn,
                static_cast<long long>(B) * H_kv * n);
  return QJL_OK;
}

// The cached S for (current device, seed, d, m), or QJL_EINVAL when it is
// not resident yet.  Never allocates.
qjl_status find_sketch(uint64_t seed, int d, int m, qjl::DeviceSketch* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(QJL_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  std::lock_guard<std::mutex> lock(g_cache_mu);
  auto it = g_cache.find(std::make_tuple(dev, seed, d, m));
  if (it == g_cache.end())
    return fail(QJL_EINVAL,
                "S for seed %llu, d=%d, m=%d is not resident on device %d: a qjl_encode_keys or "
                "qjl_decode_attention call with this seed on this device uploads it",
                static_cast<unsigned long long>(seed), d, m, dev);
  *out = it->second.view;
  return QJL_OK;
}

__global__ void zero_words_kernel(uint32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

std::mutex g_scratch_mu;
std::map<int, void*> g_scratch;   // device -> address of that device's `scratch`

// Address of `scratch` on the current device.  The first call on a device
// looks it up (hipGetSymbolAddress; the array's name in host code is only a
// stand-in) and queues a fill kernel that clears the counter region on
// `stream`.  Allocates nothing.
qjl_status scratch_for_device(hipStream_t stream, void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(QJL_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  auto it = g_scratch.find(dev);
  if (it != g_scratch.end()) {
    *out = it->second;
    return QJL_OK;
  }
  void* ptr = nullptr;
  e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess || ptr == nullptr)
    return fail(QJL_EHIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
  constexpr int kWords = static_cast<int>(qjl::kCounterRegionBytes / 4);
  hipLaunchKernelGGL(zero_words_kernel, dim3((kWords + 255) / 256), dim3(256), 0, stream,
                     static_cast<uint32_t*>(ptr), kWords);
  e = hipGetLastError();
  if (e != hipSuccess) return fail(QJL_EHIP, "clearing the scratch counters: %s", hipGetErrorString(e));
  g_scratch.emplace(dev, ptr);
  *out = ptr;
  return QJL_OK;
}

// Shared by qjl_decode_attention and its allocation-free variant: validation,
// plan, sketch and launch.  With `noalloc`, the workspace is the library's
// static scratch and S must already be resident.
qjl_status decode_common(const char* fn, const float* q, const uint32_t* signs, const float* norms,
                         const void* values_bf16, int32_t B, int32_t H_q, int32_t H_kv, int32_t N,
                         int32_t cap, int32_t d, int32_t m, uint64_t seed, float scale, float* out,
                         void* workspace, size_t workspace_bytes, void* stream, bool noalloc,
                         const qjl::AppendArgs* append = nullptr) {
  const CallScope scope(fn);
  if (!supported_dm(d, m))
    return fail(QJL_EUNSUPPORTED, "%s: d=%d m=%d unsupported (d=128, m in {256,512})", fn, d, m);
  if (B <= 0 || H_q <= 0 || H_kv <= 0 || cap <= 0 || N <= 0 || N > cap)
    return fail(QJL_EINVAL, "%s: bad sizes B=%d H_q=%d H_kv=%d N=%d cap=%d", fn, B, H_q, H_kv, N, cap);
  if (H_q % H_kv != 0)
    return fail(QJL_EINVAL, "%s: H_q=%d is not a multiple of H_kv=%d", fn, H_q, H_kv);
  const int G = H_q / H_kv;
  if (G != 1 && G != 2 && G != 4 && G != 8)
    return fail(QJL_EUNSUPPORTED, "%s: G=H_q/H_kv=%d unsupported (1, 2, 4, 8)", fn, G);
  if (static_cast<int64_t>(B) * H_kv * cap > (int64_t{1} << 40))
    return fail(QJL_EINVAL, "%s: cache too large", fn);
  if (!(scale >= 0.0f) || std::isinf(scale))
    return fail(QJL_EINVAL, "%s: scale must be finite and >= 0", fn);
  if (q == nullptr || signs == nullptr || norms == nullptr || values_bf16 == nullptr || out == nullptr)
    return fail(QJL_EINVAL, "%s: NULL pointer", fn);
  if (!aligned(q, 16) || !aligned(signs, 16) || !aligned(norms, 4) || !aligned(values_bf16, 16) ||
      !aligned(out, 16))
    return fail(QJL_EINVAL, "%s: misaligned pointer", fn);
  qjl::DecodePlan plan;
  if (!qjl::make_decode_plan(B, H_q, H_kv, N, d, m, &plan))
    return fail(QJL_EINVAL, "%s: no plan for these sizes", fn);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (noalloc) {
    if (plan.n_split > 1 && plan.total_bytes > kScratchBytes)
      return fail(QJL_EWORKSPACE,
                  "%s: these sizes need %zu bytes of split scratch, more than the %zu the "
                  "library holds; use qjl_decode_attention with a workspace",
                  fn, plan.total_bytes, kScratchBytes);
    qjl::DeviceSketch s;
    qjl_status rc = find_sketch(seed, d, m, &s);
    if (rc != QJL_OK) return rc;
    rc = scratch_for_device(st, &workspace);
    if (rc != QJL_OK) return rc;
    workspace_bytes = kScratchBytes;
    const float sc = scale == 0.0f ? static_cast<float>(1.0 / std::sqrt(static_cast<double>(d))) : scale;
    const int e = qjl::launch_decode(s, plan, q, signs, norms, values_bf16, B, H_q, H_kv, N, cap, sc,
                                     out, workspace, nullptr, stream);
    if (e != hipSuccess)
      return fail(QJL_EHIP, "%s: launch failed: %s", fn, hipGetErrorString(static_cast<hipError_t>(e)));
    return QJL_OK;
  }
  if (plan.n_split > 1) {
    if (workspace == nullptr || !aligned(workspace, 256))
      return fail(QJL_EWORKSPACE, "%s: workspace NULL or not 256-byte aligned", fn);
    if (workspace_bytes < plan.total_bytes)
      return fail(QJL_EWORKSPACE, "%s: workspace %zu bytes < %zu needed", fn, workspace_bytes,
                  plan.total_bytes);
  }
  qjl::DeviceSketch s;
  qjl_status rc = get_sketch(seed, d, m, &s);
  if (rc != QJL_OK) return rc;
  const float sc = scale == 0.0f ? static_cast<float>(1.0 / std::sqrt(static_cast<double>(d))) : scale;
  qjl::AppendArgs app;
  if (append != nullptr) {
    app = *append;
    app.s_md = s.s_md;
  }
  const int e = qjl::launch_decode(s, plan, q, signs, norms, values_bf16, B, H_q, H_kv, N, cap, sc,
                                   out, workspace, append != nullptr ? &app : nullptr, stream);
  if (e != hipSuccess)
    return fail(QJL_EHIP, "%s: launch failed: %s", fn, hipGetErrorString(static_cast<hipError_t>(e)));
  return QJL_OK;
}

}  // namespace

extern "C" {

QJL_API int32_t qjl_abi_version(void) { return kAbiVersion; }

QJL_API const char* qjl_last_error(void) { return g_last_error.c_str(); }

QJL_API qjl_status qjl_sketch_host(uint64_t seed, int32_t d, int32_t m, uint16_t* out) {
  const CallScope scope("qjl_sketch_host");
  if (out == nullptr) return fail(QJL_EINVAL, "qjl_sketch_host: out is NULL");
  if (d <= 0 || m <= 0) return fail(QJL_EINVAL, "qjl_sketch_host: d=%d m=%d must be positive", d, m);
  if (static_cast<int64_t>(d) * m > (int64_t{1} << 26))
    return fail(QJL_EINVAL, "qjl_sketch_host: d*m too large");
  qjl::generate_sketch_bf16(seed, d, m, out);
  return QJL_OK;
}

QJL_API qjl_status qjl_rotation_host(uint64_t seed, int32_t d, float* out) {
  const CallScope scope("qjl_rotation_host");
  if (out == nullptr) return fail(QJL_EINVAL, "qjl_rotation_host: out is NULL");
  if (d < 2 || d > 1024) return fail(QJL_EINVAL, "qjl_rotation_host: d=%d outside [2, 1024]", d);
  qjl::make_rotation_f32(seed, d, out);
  return QJL_OK;
}

QJL_API qjl_status qjl_tq_codebook_host(int32_t d, int32_t k, float* centroids) {
  const CallScope scope("qjl_tq_codebook_host");
  if (centroids == nullptr) return fail(QJL_EINVAL, "qjl_tq_codebook_host: centroids is NULL");
  if (d < 4 || d > 65536 || k < 1 || k > 4)
    return fail(QJL_EINVAL, "qjl_tq_codebook_host: d=%d k=%d outside d in [4, 65536], k in [1, 4]", d, k);
  qjl::make_tq_codebook(d, k, centroids);
  return QJL_OK;
}

QJL_API qjl_status qjl_pq_codebook_host(int32_t level, int32_t bits, float* centroids, float* thresholds) {
  const CallScope scope("qjl_pq_codebook_host");
  if (centroids == nullptr || thresholds == nullptr) return fail(QJL_EINVAL, "qjl_pq_codebook_host: NULL pointer");
  if (level < 1 || level > 10 || bits < 1 || bits > 5 || (level == 1 && bits < 2))
    return fail(QJL_EINVAL, "qjl_pq_codebook_host: level=%d bits=%d unsupported", level, bits);
  qjl::make_pq_codebook(level, bits, centroids, thresholds);
  return QJL_OK;
}

QJL_API qjl_status qjl_encode_keys(const void* keys_bf16, int32_t B, int32_t H_kv, int32_t n,
                                   int32_t d, int32_t m, uint64_t seed, uint32_t* signs,
                                   float* norms, int32_t cap, int32_t pos, void* stream) {
  const CallScope scope("qjl_encode_keys");
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

QJL_API int32_t qjl_testing_set_encode_small_max(int32_t keys) { return qjl::set_encode_small_max(keys); }

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
  return decode_common("qjl_decode_attention", q, signs, norms, values_bf16, B, H_q, H_kv, N, cap,
                       d, m, seed, scale, out, workspace, workspace_bytes, stream, false);
}

QJL_API qjl_status qjl_decode_attention_noalloc(const float* q, const uint32_t* signs,
                                                const float* norms, const void* values_bf16,
                                                int32_t B, int32_t H_q, int32_t H_kv, int32_t N,
                                                int32_t cap, int32_t d, int32_t m, uint64_t seed,
                                                float scale, float* out, void* stream) {
  return decode_common("qjl_decode_attention_noalloc", q, signs, norms, values_bf16, B, H_q, H_kv,
                       N, cap, d, m, seed, scale, out, nullptr, 0, stream, true);
}

QJL_API qjl_status qjl_decode_step(const float* q, const void* new_keys_bf16,
                                   const void* new_values_bf16, uint32_t* signs, float* norms,
                                   void* values_bf16, int32_t B, int32_t H_q, int32_t H_kv,
                                   int32_t pos, int32_t cap, int32_t d, int32_t m, uint64_t seed,
                                   float scale, float* out, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  g_last_error.clear();
  if (pos < 0 || cap <= 0 || pos >= cap)
    return fail(QJL_EINVAL, "qjl_decode_step: pos=%d outside [0, cap=%d)", pos, cap);
  if (new_keys_bf16 == nullptr || new_values_bf16 == nullptr)
    return fail(QJL_EINVAL, "qjl_decode_step: NULL pointer");
  if (!aligned(new_keys_bf16, 16) || !aligned(new_values_bf16, 16))
    return fail(QJL_EINVAL, "qjl_decode_step: misaligned pointer (new keys/values need 16 B)");
  qjl::AppendArgs app;
  app.key = static_cast<const uint16_t*>(new_keys_bf16);
  app.val = static_cast<const uint16_t*>(new_values_bf16);
  app.signs = signs;
  app.norms = norms;
  app.values = static_cast<uint16_t*>(values_bf16);
  app.pos = pos;
  return decode_common("qjl_decode_step", q, signs, norms, values_bf16, B, H_q, H_kv, pos + 1, cap,
                       d, m, seed, scale, out, workspace, workspace_bytes, stream, false, &app);
}

QJL_API qjl_status qjl_baseline_decode_attention_bf16(const float* q, const void* keys_bf16,
                                                      const void* values_bf16, int32_t B, int32_t H_q,
                                                      int32_t H_kv, int32_t N, int32_t cap, int32_t d,
                                                      float scale, float* out, void* workspace,
                                                      size_t workspace_bytes, void* stream) {
  const char* fn = "qjl_baseline_decode_attention_bf16";
  const CallScope scope(fn);
  if (d != qjl::kHeadDim) return fail(QJL_EUNSUPPORTED, "%s: d=%d unsupported (d=128)", fn, d);
  if (B <= 0 || H_q <= 0 || H_kv <= 0 || cap <= 0 || N <= 0 || N > cap)
    return fail(QJL_EINVAL, "%s: bad sizes B=%d H_q=%d H_kv=%d N=%d cap=%d", fn, B, H_q, H_kv, N, cap);
  if (H_q % H_kv != 0)
    return fail(QJL_EINVAL, "%s: H_q=%d is not a multiple of H_kv=%d", fn, H_q, H_kv);
  const int G = H_q / H_kv;
  if (G != 1 && G != 2 && G != 4 && G != 8)
    return fail(QJL_EUNSUPPORTED, "%s: G=H_q/H_kv=%d unsupported (1, 2, 4, 8)", fn, G);
  if (static_cast<int64_t>(B) * H_kv * cap > (int64_t{1} << 40)) return fail(QJL_EINVAL, "%s: cache too large", fn);
  if (!(scale >= 0.0f) || std::isinf(scale)) return fail(QJL_EINVAL, "%s: scale must be finite and >= 0", fn);
  if (q == nullptr || keys_bf16 == nullptr || values_bf16 == nullptr || out == nullptr)
    return fail(QJL_EINVAL, "%s: NULL pointer", fn);
  if (!aligned(q, 16) || !aligned(keys_bf16, 16) || !aligned(values_bf16, 16) || !aligned(out, 16))
    return fail(QJL_EINVAL, "%s: misaligned pointer", fn);
  qjl::DecodePlan plan;
  if (!qjl::make_decode_plan(B, H_q, H_kv, N, d, 256, &plan)) return fail(QJL_EINVAL, "%s: no plan", fn);
  if (plan.n_split > 1) {
    if (workspace == nullptr || !aligned(workspace, 256))
      return fail(QJL_EWORKSPACE, "%s: workspace NULL or not 256-byte aligned", fn);
    if (workspace_bytes < plan.total_bytes)
      return fail(QJL_EWORKSPACE, "%s: workspace %zu bytes < %zu needed", fn, workspace_bytes, plan.total_bytes);
  }
  const float sc = scale == 0.0f ? static_cast<float>(1.0 / std::sqrt(static_cast<double>(d))) : scale;
  const int e = qjl::launch_decode_bf16(plan, q, keys_bf16, values_bf16, B, H_q, H_kv, N, cap, sc, out,
                                        workspace, stream);
  if (e != hipSuccess)
    return fail(QJL_EHIP, "%s: launch failed: %s", fn, hipGetErrorString(static_cast<hipError_t>(e)));
  return QJL_OK;
}

QJL_API qjl_status qjl_tq_encode_keys(const void* keys_bf16, int32_t B, int32_t H_kv, int32_t n,
                                      int32_t d, int32_t k, uint64_t seed, uint32_t* codes,
                                      uint32_t* bits, float* norms, float* gammas, int32_t cap,
                                      int32_t pos, void* stream) {
  const char* fn = "qjl_tq_encode_keys";
  const CallScope scope(fn);
  if (d != qjl::kHeadDim || k < 1 || k > 3)
    return fail(QJL_EUNSUPPORTED, "%s: d=%d k=%d unsupported (d=128, k in {1,2,3})", fn, d, k);
  qjl_status st = check_rows(fn, B, H_kv, n, cap, pos);
  if (st != QJL_OK || n == 0) return st;
  if (keys_bf16 == nullptr || codes == nullptr || bits == nullptr || norms == nullptr || gammas == nullptr)
    return fail(QJL_EINVAL, "%s: NULL pointer", fn);
  if (!aligned(keys_bf16, 16) || !aligned(codes, 4) || !aligned(bits, 4) || !aligned(norms, 4) || !aligned(gammas, 4))
    return fail(QJL_EINVAL, "%s: misaligned pointer (keys need 16 B, the rest 4 B)", fn);
  qjl::RotqTables tb;
  st = get_rotq(seed, &tb);
  if (st != QJL_OK) return st;
  const int e = qjl::launch_rotq_encode(tb, 0, k, keys_bf16, B, H_kv, n, codes, bits, norms, gammas, cap, pos,
                                        g_rotq_margin, stream);
  if (e != hipSuccess) return fail(QJL_EHIP, "%s: launch failed: %s", fn, hipGetErrorString(static_cast<hipError_t>(e)));
  return QJL_OK;
}

QJL_API qjl_status qjl_pq_encode_keys(const void* keys_bf16, int32_t B, int32_t H_kv, int32_t n,
                                      int32_t d, uint64_t seed, uint32_t* codes, float* radii,
                                      int32_t cap, int32_t pos, void* stream) {
  const char* fn = "qjl_pq_encode_keys";
  const CallScope scope(fn);
  if (d != qjl::kHeadDim) return fail(QJL_EUNSUPPORTED, "%s: d=%d unsupported (d=128)", fn, d);
  qjl_status st = check_rows(fn, B, H_kv, n, cap, pos);
  if (st != QJL_OK || n == 0) return st;
  if (keys_bf16 == nullptr || codes == nullptr || radii == nullptr) return fail(QJL_EINVAL, "%s: NULL pointer", fn);
  if (!aligned(keys_bf16, 16) || !aligned(codes, 4) || !aligned(radii, 4))
    return fail(QJL_EINVAL, "%s: misaligned pointer (keys need 16 B, the rest 4 B)", fn);
  qjl::RotqTables tb;
  st = get_rotq(seed, &tb);
  if (st != QJL_OK) return st;
  const int e = qjl::launch_rotq_encode(tb, 1, 0, keys_bf16, B, H_kv, n, codes, nullptr, radii, nullptr, cap,
                                        pos, g_rotq_margin, stream);
  if (e != hipSuccess) return fail(QJL_EHIP, "%s: launch failed: %s", fn, hipGetErrorString(static_cast<hipError_t>(e)));
  return QJL_OK;
}

QJL_API size_t qjl_tq_scores_workspace_bytes(int32_t B, int32_t H_q, int32_t d) {
  if (B <= 0 || H_q <= 0 || d != qjl::kHeadDim) return 0;
  return qjl::tq_scores_workspace_bytes(B, H_q);
}

QJL_API qjl_status qjl_tq_scores(const float* q, const uint32_t* codes, const uint32_t* bits,
                                 const float* norms, const float* gammas, int32_t B, int32_t H_q,
                                 int32_t H_kv, int32_t N, int32_t cap, int32_t d, int32_t k,
                                 uint64_t seed, float* scores, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  const char* fn = "qjl_tq_scores";
  const CallScope scope(fn);
  if (d != qjl::kHeadDim || k < 1 || k > 3)
    return fail(QJL_EUNSUPPORTED, "%s: d=%d k=%d unsupported (d=128, k in {1,2,3})", fn, d, k);
  if (B <= 0 || H_q <= 0 || H_kv <= 0 || cap <= 0 || N <= 0 || N > cap)
    return fail(QJL_EINVAL, "%s: bad sizes B=%d H_q=%d H_kv=%d N=%d cap=%d", fn, B, H_q, H_kv, N, cap);
  if (H_q % H_kv != 0) return fail(QJL_EINVAL, "%s: H_q=%d is not a multiple of H_kv=%d", fn, H_q, H_kv);
  const int G = H_q / H_kv;
  if (G != 1 && G != 2 && G != 4 && G != 8)
    return fail(QJL_EUNSUPPORTED, "%s: G=H_q/H_kv=%d unsupported (1, 2, 4, 8)", fn, G);
  if (static_cast<int64_t>(B) * H_kv * cap > (int64_t{1} << 40)) return fail(QJL_EINVAL, "%s: cache too large", fn);
  if (static_cast<int64_t>(B) * H_q * N > (int64_t{1} << 40)) return fail(QJL_EINVAL, "%s: output too large", fn);
  if (B > 65535 || H_kv > 65535) return fail(QJL_EINVAL, "%s: B=%d or H_kv=%d above 65535", fn, B, H_kv);
  if (q == nullptr || codes == nullptr || bits == nullptr || norms == nullptr || gammas == nullptr || scores == nullptr)
    return fail(QJL_EINVAL, "%s: NULL pointer", fn);
  if (!aligned(q, 4) || !aligned(codes, 16) || !aligned(bits, 16) || !aligned(norms, 4) || !aligned(gammas, 4) ||
      !aligned(scores, 4))
    return fail(QJL_EINVAL, "%s: misaligned pointer (codes and bits need 16 B, the rest 4 B)", fn);
  if (workspace == nullptr || !aligned(workspace, 256))
    return fail(QJL_EWORKSPACE, "%s: workspace NULL or not 256-byte aligned", fn);
  const size_t need = qjl::tq_scores_workspace_bytes(B, H_q);
  if (workspace_bytes < need)
    return fail(QJL_EWORKSPACE, "%s: workspace %zu bytes < %zu needed", fn, workspace_bytes, need);
  qjl::RotqTables tb;
  qjl_status st = get_rotq(seed, &tb);
  if (st != QJL_OK) return st;
  const int e = qjl::launch_tq_scores(tb, k, q, codes, bits, norms, gammas, B, H_q, H_kv, N, cap, scores,
                                      workspace, stream);
  if (e != hipSuccess) return fail(QJL_EHIP, "%s: launch failed: %s", fn, hipGetErrorString(static_cast<hipError_t>(e)));
  return QJL_OK;
}

QJL_API int32_t qjl_testing_set_rotq_margin(int32_t log2_factor) {
  const int prev = g_rotq_margin;
  if (log2_factor >= 0 && log2_factor <= 60) g_rotq_margin = log2_factor;
  return prev;
}

QJL_API qjl_status qjl_release_cache(void) {
  const CallScope scope("qjl_release_cache");
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
  for (auto& kv : g_rotq) {
    if (hipSetDevice(std::get<0>(kv.first)) == hipSuccess) {
      (void)hipDeviceSynchronize();
      if (hipFree(kv.second.mem) != hipSuccess) rc = fail(QJL_EHIP, "qjl_release_cache: hipFree failed");
    }
  }
  g_rotq.clear();
  if (have_dev) (void)hipSetDevice(cur);
  return rc;
}

}  // extern "C"
