// The extern "C" entry points of libawq declared in include/awq.h: argument
// checks, workspace carving and kernel dispatch.  No entry point allocates
// memory, synchronises the device or lets a C++ exception escape.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <initializer_list>
#include <mutex>
#include <string>

#include "awq.h"
#include "awq_internal.h"

namespace awq {
namespace {
thread_local KernelPlan* g_plan = nullptr;
}  // namespace

KernelPlan* active_plan() { return g_plan; }
void install_plan(KernelPlan* p) { g_plan = p; }

hipError_t plan_record(KernelPlan* p, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(p->text, sizeof(p->text), fmt, ap);
  va_end(ap);
  return hipSuccess;
}
}  // namespace awq

namespace {

thread_local std::string g_last_error = "no error";

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  try {
    g_last_error = buf;
  } catch (...) {
  }
  return status;
}

int device_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return AWQ_OK;
  return fail(AWQ_ERROR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Every device pointer an entry point takes must be 16-byte aligned (the
// kernels move 16-byte pieces, several of them straight into LDS); the first
// misaligned one is named in the error.  NULL entries (optional arguments
// left out) are skipped.
struct DevPtr {
  const void* p;
  const char* name;
};
int check_aligned(std::initializer_list<DevPtr> ptrs) {
  for (const DevPtr& d : ptrs)
    if (d.p != nullptr && !aligned16(d.p)) return fail(AWQ_ERROR_MISALIGNED, "%s must be 16-byte aligned", d.name);
  return AWQ_OK;
}

#define AWQ_REQUIRE(cond, status, ...) \
  do {                                 \
    if (!(cond)) return fail(status, __VA_ARGS__); \
  } while (0)

#define AWQ_GUARD_BEGIN try {
#define AWQ_GUARD_END                                            \
  }                                                              \
  catch (...) {                                                  \
    return fail(AWQ_ERROR_DEVICE, "unexpected C++ exception"); \
  }

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

int check_bits(int32_t bits) {
  AWQ_REQUIRE(bits == 4 || bits == 3, AWQ_ERROR_INVALID_VALUE, "bits must be 4 or 3 (got %d)", bits);
  return AWQ_OK;
}

int check_layer(int64_t N, int64_t K, int32_t group) {
  AWQ_REQUIRE(N >= 1 && K >= 1, AWQ_ERROR_INVALID_VALUE, "N and K must be >= 1 (got N=%lld K=%lld)", (long long)N,
              (long long)K);
  AWQ_REQUIRE(group == AWQ_GROUP, AWQ_ERROR_INVALID_VALUE, "group must be %d (got %d)", AWQ_GROUP, group);
  AWQ_REQUIRE(K % group == 0, AWQ_ERROR_INVALID_VALUE, "K=%lld is not a multiple of group %d", (long long)K, group);
  AWQ_REQUIRE(N < (int64_t(1) << 31) && K <= (int64_t(1) << 20), AWQ_ERROR_INVALID_VALUE,
              "N=%lld or K=%lld exceeds the supported range", (long long)N, (long long)K);
  return AWQ_OK;
}

// Workspace of awq_quantize, carved in this order (each piece 256-byte aligned).
// M < K uses the direct form of the loss (E in fp32); M >= K the Gram form
// (channel exponents, G as scaled fp16 hi/lo, X^T, G in fp32 and the fp64
// partial tiles of its split tiles, E' hi/lo).
// The statistics of X come first, at offsets that depend on K and M only.
struct QuantizeWorkspace {
  bool direct;
  size_t a, s_all, inv_all, xt, g, gp, gh, gl, ex, eh, el, e32, partial, loss, b, mask, total;
  int64_t mp, partials;
};

// The keep-fp16 ablation adds the weight magnitudes b [K] and a channel mask [K].
QuantizeWorkspace quantize_workspace(int64_t N, int64_t K, int64_t M, int32_t n_alpha, bool ablation = false) {
  QuantizeWorkspace w{};
  w.direct = M < K;
  w.mp = (M + 63) / 64 * 64;
  w.partials = w.direct ? awq::loss_direct_partial_count(M, N) : awq::loss_partial_count(N, K);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off = round_up(off + bytes, 256);
    return at;
  };
  // statistics of X first (they depend on K and M only), then what depends on N and n_alpha
  w.a = take(sizeof(double) * (size_t)K);
  if (!w.direct) {
    w.ex = take(sizeof(int32_t) * (size_t)K);
    w.gh = take(2 * (size_t)K * (size_t)K);
    w.gl = take(2 * (size_t)K * (size_t)K);
    w.xt = take(2 * (size_t)K * (size_t)w.mp);
    w.g = take(sizeof(float) * (size_t)K * (size_t)K);
    w.gp = take(awq::gram_partial_bytes(K, w.mp));
  }
  w.s_all = take(sizeof(float) * (size_t)n_alpha * (size_t)K);
  w.inv_all = take(sizeof(double) * (size_t)n_alpha * (size_t)K);
  if (w.direct) {
    w.e32 = take(sizeof(float) * (size_t)N * (size_t)K);
  } else {
    w.eh = take(2 * (size_t)N * (size_t)K);
    w.el = take(2 * (size_t)N * (size_t)K);
  }
  w.partial = take(sizeof(double) * (size_t)w.partials);
  w.loss = take(sizeof(double) * (size_t)n_alpha);
  if (ablation) {
    w.b = take(sizeof(double) * (size_t)K);
    w.mask = take((size_t)K);
  }
  w.total = off;
  return w;
}

// The device array behind awq_gemm_scaled_static: the scaled input of calls
// made by callers that cannot allocate.  Each GPU the library runs on holds
// its own copy until the process ends.  In host code `scratch` is only a
// stand-in for the symbol, never a device address: the address is looked up
// per device with hipGetSymbolAddress and kept in g_scratch_ptr.
static __device__ __align__(256) unsigned char scratch[AWQ_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch`, looked up on the first call made
// with that device current.
int device_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(AWQ_ERROR_DEVICE, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(AWQ_ERROR_DEVICE, "device %d outside [0, %d)", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(AWQ_ERROR_DEVICE, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return AWQ_OK;
}

}  // namespace

extern "C" {

int awq_version(void) { return 1 * 10000 + 0 * 100 + 0; }

const char* awq_status_string(int status) {
  switch (status) {
    case AWQ_OK: return "AWQ_OK";
    case AWQ_ERROR_INVALID_VALUE: return "AWQ_ERROR_INVALID_VALUE";
    case AWQ_ERROR_MISALIGNED: return "AWQ_ERROR_MISALIGNED";
    case AWQ_ERROR_WORKSPACE_TOO_SMALL: return "AWQ_ERROR_WORKSPACE_TOO_SMALL";
    case AWQ_ERROR_DEVICE: return "AWQ_ERROR_DEVICE";
    case AWQ_ERROR_NOT_IMPLEMENTED: return "AWQ_ERROR_NOT_IMPLEMENTED";
    default: return "AWQ_UNKNOWN_STATUS";
  }
}

const char* awq_last_error(void) { return g_last_error.c_str(); }

size_t awq_packed_bytes(int64_t N, int64_t K) { return awq_packed_bytes_bits(N, K, 4); }

size_t awq_packed_bytes_bits(int64_t N, int64_t K, int32_t bits) {
  if (N < 1 || K < 1) return 0;
  if (bits == 4) return K % 8 == 0 ? (size_t)N * (size_t)(K / 8) * 4 : 0;
  if (bits == 3) return K % 32 == 0 ? (size_t)N * (size_t)(K / 32) * 12 : 0;
  return 0;
}

size_t awq_scales_bytes(int64_t N, int64_t K, int32_t group) {
  if (N < 1 || K < 1 || group < 1 || K % group != 0) return 0;
  return (size_t)N * (size_t)(K / group) * 2;
}

size_t awq_zeros_bytes(int64_t N, int64_t K, int32_t group) {
  if (N < 1 || K < 1 || group < 1 || K % group != 0) return 0;
  return (size_t)N * (size_t)((K / group + 1) / 2);
}

size_t awq_quantize_workspace_bytes(int64_t N, int64_t K, int64_t M, int32_t group, int32_t n_alpha) {
  if (N < 1 || K < 1 || M < 1 || group != AWQ_GROUP || K % group != 0 || n_alpha < 1 || n_alpha > AWQ_MAX_ALPHAS)
    return 0;
  return quantize_workspace(N, K, M, n_alpha).total;
}

int awq_channel_mean_abs(const void* X, int64_t M, int64_t K, double* a, void* stream) {
  AWQ_GUARD_BEGIN
  AWQ_REQUIRE(X && a, AWQ_ERROR_INVALID_VALUE, "X and a must not be NULL");
  AWQ_REQUIRE(M >= 1 && M <= AWQ_MAX_CALIB_ROWS, AWQ_ERROR_INVALID_VALUE, "M=%lld outside [1, 2^23]", (long long)M);
  AWQ_REQUIRE(K >= 8 && K % 8 == 0 && K <= (int64_t(1) << 20), AWQ_ERROR_INVALID_VALUE,
              "K=%lld must be a positive multiple of 8", (long long)K);
  if (int st = check_aligned({{X, "X"}, {a, "a"}})) return st;
  return device_status(awq::launch_channel_mean_abs(X, M, K, a, as_stream(stream)), "awq_channel_mean_abs");
  AWQ_GUARD_END
}

int awq_pack(const void* W, const float* s, int64_t N, int64_t K, int32_t group, void* packed, void* scales,
             void* zeros, void* stream) {
  return awq_pack_bits(W, s, N, K, group, 4, packed, scales, zeros, stream);
}

int awq_pack_bits(const void* W, const float* s, int64_t N, int64_t K, int32_t group, int32_t bits, void* packed,
                  void* scales, void* zeros, void* stream) {
  AWQ_GUARD_BEGIN
  AWQ_REQUIRE(W && packed && scales && zeros, AWQ_ERROR_INVALID_VALUE, "W, packed, scales, zeros must not be NULL");
  int st = check_layer(N, K, group);
  if (st == AWQ_OK) st = check_bits(bits);
  if (st != AWQ_OK) return st;
  if (int st2 = check_aligned({{W, "W"}, {s, "s"}, {packed, "packed"}, {scales, "scales"}, {zeros, "zeros"}}))
    return st2;
  return device_status(awq::launch_pack(W, s, N, K, bits, packed, scales, zeros, as_stream(stream)), "awq_pack");
  AWQ_GUARD_END
}

int awq_quantize(const void* W, const void* X, int64_t N, int64_t K, int64_t M, int32_t group, const float* alphas,
                 int32_t n_alpha, void* packed, void* scales, void* zeros, float* s, int32_t* best_alpha,
                 double* loss, void* workspace, size_t workspace_bytes, void* stream) {
  return awq_quantize_bits(W, X, N, K, M, group, 4, alphas, n_alpha, packed, scales, zeros, s, best_alpha, loss,
                           workspace, workspace_bytes, stream);
}

int awq_quantize_bits(const void* W, const void* X, int64_t N, int64_t K, int64_t M, int32_t group, int32_t bits,
                      const float* alphas, int32_t n_alpha, void* packed, void* scales, void* zeros, float* s,
                      int32_t* best_alpha, double* loss, void* workspace, size_t workspace_bytes, void* stream) {
  return awq_quantize_shared(W, X, N, K, M, group, bits, alphas, n_alpha, 0, packed, scales, zeros, s, best_alpha,
                             loss, workspace, workspace_bytes, stream);
}

int awq_quantize_shared(const void* W, const void* X, int64_t N, int64_t K, int64_t M, int32_t group, int32_t bits,
                        const float* alphas, int32_t n_alpha, int32_t reuse_statistics, void* packed, void* scales,
                        void* zeros, float* s, int32_t* best_alpha, double* loss, void* workspace,
                        size_t workspace_bytes, void* stream) {
  AWQ_GUARD_BEGIN
  AWQ_REQUIRE(reuse_statistics == 0 || reuse_statistics == 1, AWQ_ERROR_INVALID_VALUE,
              "reuse_statistics=%d must be 0 or 1", reuse_statistics);
  AWQ_REQUIRE(W && X && alphas && packed && scales && zeros && s && best_alpha && workspace, AWQ_ERROR_INVALID_VALUE,
              "W, X, alphas, packed, scales, zeros, s, best_alpha and workspace must not be NULL");
  int st = check_layer(N, K, group);
  if (st == AWQ_OK) st = check_bits(bits);
  if (st != AWQ_OK) return st;
  AWQ_REQUIRE(M >= 1 && M <= AWQ_MAX_CALIB_ROWS, AWQ_ERROR_INVALID_VALUE, "M=%lld outside [1, 2^23]", (long long)M);
  AWQ_REQUIRE(n_alpha >= 1 && n_alpha <= AWQ_MAX_ALPHAS, AWQ_ERROR_INVALID_VALUE, "n_alpha=%d outside [1, %d]",
              n_alpha, AWQ_MAX_ALPHAS);
  awq::AlphaGrid grid{};
  for (int i = 0; i < n_alpha; ++i) {
    AWQ_REQUIRE(std::isfinite(alphas[i]) && alphas[i] >= 0.0f, AWQ_ERROR_INVALID_VALUE,
                "alphas[%d]=%g must be finite and >= 0", i, (double)alphas[i]);
    grid.v[i] = alphas[i];
  }
  if (int st2 = check_aligned({{W, "W"}, {X, "X"}, {packed, "packed"}, {scales, "scales"}, {zeros, "zeros"},
                                {s, "s"}, {best_alpha, "best_alpha"}, {loss, "loss"}, {workspace, "workspace"}}))
    return st2;
  const QuantizeWorkspace w = quantize_workspace(N, K, M, n_alpha);
  AWQ_REQUIRE(workspace_bytes >= w.total, AWQ_ERROR_WORKSPACE_TOO_SMALL, "workspace %zu bytes, need %zu",
              workspace_bytes, w.total);

  char* base = static_cast<char*>(workspace);
  double* a = reinterpret_cast<double*>(base + w.a);
  float* s_all = reinterpret_cast<float*>(base + w.s_all);
  double* inv_all = reinterpret_cast<double*>(base + w.inv_all);
  double* partial = reinterpret_cast<double*>(base + w.partial);
  double* L = loss ? loss : reinterpret_cast<double*>(base + w.loss);
  hipStream_t hs = as_stream(stream);
  const double mn = (double)M * (double)N;

  // The statistics of X (a, and in the Gram form the exponents and the scaled
  // hi/lo split of G) sit in the workspace ahead of everything that depends on N,
  // so a call with the same X, M and K may take them from the previous call.
  hipError_t e = reuse_statistics ? hipSuccess : awq::launch_channel_mean_abs(X, M, K, a, hs);
  if (e == hipSuccess) e = awq::launch_scales(a, grid, n_alpha, K, s_all, inv_all, hs);
  if (w.direct) {
    float* E = reinterpret_cast<float*>(base + w.e32);
    for (int i = 0; i < n_alpha && e == hipSuccess; ++i) {
      e = awq::launch_quant_error32(W, s_all + (size_t)i * (size_t)K, inv_all + (size_t)i * (size_t)K, nullptr, N, K,
                                    bits, E, hs);
      if (e == hipSuccess) e = awq::launch_loss_direct(X, E, M, N, K, partial, hs);
      if (e == hipSuccess) e = awq::launch_loss_reduce(partial, w.partials, mn, L + i, hs);
    }
  } else {
    void* xt = base + w.xt;
    float* G = reinterpret_cast<float*>(base + w.g);
    void* Ghi = base + w.gh;
    void* Glo = base + w.gl;
    int32_t* ex = reinterpret_cast<int32_t*>(base + w.ex);
    void* Ehi = base + w.eh;
    void* Elo = base + w.el;
    if (!reuse_statistics) {
      if (e == hipSuccess) e = awq::launch_transpose(X, M, K, w.mp, xt, hs);
      if (e == hipSuccess) e = awq::launch_gram(xt, w.mp, K, G, reinterpret_cast<double*>(base + w.gp), hs);
      if (e == hipSuccess) e = awq::launch_gram_split(G, K, ex, Ghi, Glo, hs);
    }
    for (int i = 0; i < n_alpha && e == hipSuccess; ++i) {
      e = awq::launch_quant_error(W, s_all + (size_t)i * (size_t)K, inv_all + (size_t)i * (size_t)K, ex, nullptr, N,
                                  K, bits, Ehi, Elo, hs);
      if (e == hipSuccess) e = awq::launch_loss_partials(Ehi, Elo, Ghi, Glo, N, K, partial, hs);
      if (e == hipSuccess) e = awq::launch_loss_reduce(partial, w.partials, mn, L + i, hs);
    }
  }
  if (e == hipSuccess) e = awq::launch_argmin(L, n_alpha, best_alpha, hs);
  if (e == hipSuccess) e = awq::launch_select_scale(s_all, best_alpha, K, s, hs);
  if (e == hipSuccess) e = awq::launch_pack(W, s, N, K, bits, packed, scales, zeros, hs);
  return device_status(e, "awq_quantize");
  AWQ_GUARD_END
}

size_t awq_ablation_workspace_bytes(int64_t N, int64_t K, int64_t M, int32_t group) {
  if (N < 1 || K < 1 || M < 1 || group != AWQ_GROUP || K % group != 0) return 0;
  return quantize_workspace(N, K, M, 1, true).total;
}

int awq_keep_fp16_ablation(const void* W, const void* X, int64_t N, int64_t K, int64_t M, int32_t group, int32_t bits,
                           int32_t n_keep, const int32_t* random_keep, int32_t* keep_act, int32_t* keep_wt,
                           double* loss, void* workspace, size_t workspace_bytes, void* stream) {
  AWQ_GUARD_BEGIN
  AWQ_REQUIRE(W && X && loss && workspace && (n_keep == 0 || (random_keep && keep_act && keep_wt)),
              AWQ_ERROR_INVALID_VALUE, "W, X, loss, workspace (and the keep lists when n_keep > 0) must not be NULL");
  int st = check_layer(N, K, group);
  if (st == AWQ_OK) st = check_bits(bits);
  if (st != AWQ_OK) return st;
  AWQ_REQUIRE(M >= 1 && M <= AWQ_MAX_CALIB_ROWS && N <= AWQ_MAX_CALIB_ROWS, AWQ_ERROR_INVALID_VALUE,
              "M=%lld and N=%lld must be in [1, 2^23]", (long long)M, (long long)N);
  AWQ_REQUIRE(n_keep >= 0 && n_keep <= K, AWQ_ERROR_INVALID_VALUE, "n_keep=%d outside [0, K]", n_keep);
  if (int st2 = check_aligned({{W, "W"}, {X, "X"}, {random_keep, "random_keep"}, {keep_act, "keep_act"},
                                {keep_wt, "keep_wt"}, {loss, "loss"}, {workspace, "workspace"}}))
    return st2;
  const QuantizeWorkspace w = quantize_workspace(N, K, M, 1, true);
  AWQ_REQUIRE(workspace_bytes >= w.total, AWQ_ERROR_WORKSPACE_TOO_SMALL, "workspace %zu bytes, need %zu",
              workspace_bytes, w.total);
  char* base = static_cast<char*>(workspace);
  double* a = reinterpret_cast<double*>(base + w.a);
  double* b = reinterpret_cast<double*>(base + w.b);
  uint8_t* mask = reinterpret_cast<uint8_t*>(base + w.mask);
  double* partial = reinterpret_cast<double*>(base + w.partial);
  hipStream_t hs = as_stream(stream);
  const double mn = (double)M * (double)N;

  // activation magnitude of each input channel, and weight magnitude: the same
  // exact mean of |.| over the rows of W [N][K]
  hipError_t e = awq::launch_channel_mean_abs(X, M, K, a, hs);
  if (e == hipSuccess) e = awq::launch_channel_mean_abs(W, N, K, b, hs);
  if (e == hipSuccess && n_keep > 0) e = awq::launch_top_channels(a, K, n_keep, keep_act, hs);
  if (e == hipSuccess && n_keep > 0) e = awq::launch_top_channels(b, K, n_keep, keep_wt, hs);
  int32_t* ex = reinterpret_cast<int32_t*>(base + w.ex);
  if (!w.direct) {
    if (e == hipSuccess) e = awq::launch_transpose(X, M, K, w.mp, base + w.xt, hs);
    if (e == hipSuccess)
      e = awq::launch_gram(base + w.xt, w.mp, K, reinterpret_cast<float*>(base + w.g),
                           reinterpret_cast<double*>(base + w.gp), hs);
    if (e == hipSuccess)
      e = awq::launch_gram_split(reinterpret_cast<float*>(base + w.g), K, ex, base + w.gh, base + w.gl, hs);
  }
  const int32_t* sets[4] = {nullptr, keep_act, keep_wt, random_keep};
  for (int i = 0; i < 4 && e == hipSuccess; ++i) {
    e = awq::launch_keep_mask(sets[i], i == 0 ? 0 : n_keep, K, mask, hs);
    if (w.direct) {
      float* E = reinterpret_cast<float*>(base + w.e32);
      if (e == hipSuccess) e = awq::launch_quant_error32(W, nullptr, nullptr, mask, N, K, bits, E, hs);
      if (e == hipSuccess) e = awq::launch_loss_direct(X, E, M, N, K, partial, hs);
    } else {
      if (e == hipSuccess)
        e = awq::launch_quant_error(W, nullptr, nullptr, ex, mask, N, K, bits, base + w.eh, base + w.el, hs);
      if (e == hipSuccess) e = awq::launch_loss_partials(base + w.eh, base + w.el, base + w.gh, base + w.gl, N, K,
                                                         partial, hs);
    }
    if (e == hipSuccess) e = awq::launch_loss_reduce(partial, w.partials, mn, loss + i, hs);
  }
  return device_status(e, "awq_keep_fp16_ablation");
  AWQ_GUARD_END
}

// The product's dispatch on the code width and M (each launcher picks its own
// kernel and layout; see the launchers for the measured rules).
static hipError_t launch_product(const void* x, const void* packed, const void* scales, const void* zeros, void* y,
                                 int64_t M, int64_t N, int64_t K, int32_t bits, hipStream_t hs, void* ws = nullptr) {
  if (bits == 3) return awq::launch_gemm3(x, packed, scales, zeros, y, M, N, K, ws, hs);
  if (M <= 16) return awq::launch_gemv(x, packed, scales, zeros, y, M, N, K, hs);
  return awq::launch_gemm(x, packed, scales, zeros, y, M, N, K, ws, hs);
}

int awq_gemm(const void* x, const void* packed, const void* scales, const void* zeros, void* y, int64_t M, int64_t N,
             int64_t K, int32_t group, void* stream) {
  return awq_gemm_bits(x, packed, scales, zeros, y, M, N, K, group, 4, stream);
}

int awq_gemm_bits(const void* x, const void* packed, const void* scales, const void* zeros, void* y, int64_t M,
                  int64_t N, int64_t K, int32_t group, int32_t bits, void* stream) {
  AWQ_GUARD_BEGIN
  AWQ_REQUIRE(x && packed && scales && zeros && y, AWQ_ERROR_INVALID_VALUE,
              "x, packed, scales, zeros and y must not be NULL");
  int st = check_layer(N, K, group);
  if (st == AWQ_OK) st = check_bits(bits);
  if (st != AWQ_OK) return st;
  AWQ_REQUIRE(M >= 1 && M <= (int64_t(1) << 22), AWQ_ERROR_INVALID_VALUE, "M=%lld outside [1, 2^22]", (long long)M);
  if (int st2 = check_aligned({{x, "x"}, {packed, "packed"}, {scales, "scales"}, {zeros, "zeros"}, {y, "y"}}))
    return st2;
  return device_status(launch_product(x, packed, scales, zeros, y, M, N, K, bits, as_stream(stream)), "awq_gemm");
  AWQ_GUARD_END
}

size_t awq_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t bits) {
  if (M < 1 || N < 1 || K < 1 || K % AWQ_GROUP != 0 || (bits != 4 && bits != 3)) return 0;
  return awq::gemm_pipe_streamk(M, N, K, bits) ? awq::gemm_pipe_workspace_bytes(M, N) : 0;
}

int awq_gemm_ws(const void* x, const void* packed, const void* scales, const void* zeros, void* y, int64_t M,
                int64_t N, int64_t K, int32_t group, int32_t bits, void* workspace, size_t workspace_bytes,
                void* stream) {
  AWQ_GUARD_BEGIN
  AWQ_REQUIRE(x && packed && scales && zeros && y, AWQ_ERROR_INVALID_VALUE,
              "x, packed, scales, zeros and y must not be NULL");
  int st = check_layer(N, K, group);
  if (st == AWQ_OK) st = check_bits(bits);
  if (st != AWQ_OK) return st;
  AWQ_REQUIRE(M >= 1 && M <= (int64_t(1) << 22), AWQ_ERROR_INVALID_VALUE, "M=%lld outside [1, 2^22]", (long long)M);
  const size_t need = awq_gemm_workspace_bytes(M, N, K, bits);
  AWQ_REQUIRE(workspace || need == 0, AWQ_ERROR_INVALID_VALUE, "workspace must not be NULL (%zu bytes needed)", need);
  if (int st2 = check_aligned({{x, "x"}, {packed, "packed"}, {scales, "scales"}, {zeros, "zeros"}, {y, "y"},
                                {workspace, "workspace"}}))
    return st2;
  AWQ_REQUIRE(workspace_bytes >= need, AWQ_ERROR_WORKSPACE_TOO_SMALL, "workspace %zu bytes, need %zu", workspace_bytes,
              need);
  return device_status(launch_product(x, packed, scales, zeros, y, M, N, K, bits, as_stream(stream),
                                      need ? workspace : nullptr),
                       "awq_gemm_ws");
  AWQ_GUARD_END
}

static int gemm_kernel_query(int64_t M, int64_t N, int64_t K, int32_t group, int32_t bits, bool with_ws, char* out,
                             size_t out_bytes);

int awq_gemm_kernel(int64_t M, int64_t N, int64_t K, int32_t group, int32_t bits, char* out, size_t out_bytes) {
  return gemm_kernel_query(M, N, K, group, bits, false, out, out_bytes);
}

int awq_gemm_ws_kernel(int64_t M, int64_t N, int64_t K, int32_t group, int32_t bits, char* out, size_t out_bytes) {
  return gemm_kernel_query(M, N, K, group, bits, true, out, out_bytes);
}

static int gemm_kernel_query(int64_t M, int64_t N, int64_t K, int32_t group, int32_t bits, bool with_ws, char* out,
                             size_t out_bytes) {
  AWQ_GUARD_BEGIN
  AWQ_REQUIRE(out && out_bytes > 0, AWQ_ERROR_INVALID_VALUE, "out must not be NULL and out_bytes must be positive");
  out[0] = 0;
  int st = check_layer(N, K, group);
  if (st == AWQ_OK) st = check_bits(bits);
  if (st != AWQ_OK) return st;
  AWQ_REQUIRE(M >= 1 && M <= (int64_t(1) << 22), AWQ_ERROR_INVALID_VALUE, "M=%lld outside [1, 2^22]", (long long)M);
  struct Installed {  // the plan stays installed only for this call, also if something throws
    awq::KernelPlan plan;
    Installed() {
      plan.text[0] = 0;
      awq::install_plan(&plan);
    }
    ~Installed() { awq::install_plan(nullptr); }
  } dry;
  // a dry run computes the launch only: no pointer is dereferenced, nothing is enqueued
  // a dry run never dereferences the workspace: any non-null address stands for one
  void* ws = with_ws && awq_gemm_workspace_bytes(M, N, K, bits) ? reinterpret_cast<void*>(uintptr_t(256)) : nullptr;
  const hipError_t e = launch_product(nullptr, nullptr, nullptr, nullptr, nullptr, M, N, K, bits, nullptr, ws);
  AWQ_REQUIRE(e == hipSuccess && dry.plan.text[0] != 0, AWQ_ERROR_INVALID_VALUE,
              "no kernel launches for M=%lld N=%lld K=%lld bits=%d", (long long)M, (long long)N, (long long)K, bits);
  snprintf(out, out_bytes, "%s", dry.plan.text);
  return AWQ_OK;
  AWQ_GUARD_END
}

int awq_scale_input(const void* x, const float* s, int64_t M, int64_t K, void* xs, void* stream) {
  AWQ_GUARD_BEGIN
  AWQ_REQUIRE(x && s && xs, AWQ_ERROR_INVALID_VALUE, "x, s and xs must not be NULL");
  AWQ_REQUIRE(M >= 1 && M <= (int64_t(1) << 22), AWQ_ERROR_INVALID_VALUE, "M=%lld outside [1, 2^22]", (long long)M);
  AWQ_REQUIRE(K >= 8 && K % 8 == 0 && K <= (int64_t(1) << 20), AWQ_ERROR_INVALID_VALUE,
              "K=%lld must be a positive multiple of 8, at most 2^20", (long long)K);
  if (int st = check_aligned({{x, "x"}, {s, "s"}, {xs, "xs"}})) return st;
  return device_status(awq::launch_scale_input(x, s, M, K, xs, as_stream(stream)), "awq_scale_input");
  AWQ_GUARD_END
}

// The scaled input through a buffer of M * K halfs: awq_scale_input, then the
// product awq_gemm_bits would run on it.
static hipError_t gemm_scaled_via(const void* x, const float* s, const void* packed, const void* scales,
                                  const void* zeros, void* y, int64_t M, int64_t N, int64_t K, int32_t bits,
                                  void* xs, hipStream_t hs) {
  hipError_t e = awq::launch_scale_input(x, s, M, K, xs, hs);
  if (e != hipSuccess) return e;
  return launch_product(xs, packed, scales, zeros, y, M, N, K, bits, hs);
}

size_t awq_gemm_scaled_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t bits) {
  if (M < 1 || N < 1 || K < 1 || (bits != 4 && bits != 3)) return 0;
  return (size_t)((M * K * 2 + 255) / 256 * 256);
}

int awq_gemm_scaled(const void* x, const float* s, const void* packed, const void* scales, const void* zeros,
                    void* y, int64_t M, int64_t N, int64_t K, int32_t group, int32_t bits, void* workspace,
                    size_t workspace_bytes, void* stream) {
  AWQ_GUARD_BEGIN
  AWQ_REQUIRE(x && s && packed && scales && zeros && y && workspace, AWQ_ERROR_INVALID_VALUE,
              "x, s, packed, scales, zeros, y and workspace must not be NULL");
  int st = check_layer(N, K, group);
  if (st == AWQ_OK) st = check_bits(bits);
  if (st != AWQ_OK) return st;
  AWQ_REQUIRE(M >= 1 && M <= (int64_t(1) << 22), AWQ_ERROR_INVALID_VALUE, "M=%lld outside [1, 2^22]", (long long)M);
  if (int st2 = check_aligned({{x, "x"}, {s, "s"}, {packed, "packed"}, {scales, "scales"}, {zeros, "zeros"},
                                {y, "y"}, {workspace, "workspace"}}))
    return st2;
  const size_t need = awq_gemm_scaled_workspace_bytes(M, N, K, bits);
  AWQ_REQUIRE(workspace_bytes >= need, AWQ_ERROR_WORKSPACE_TOO_SMALL,
              "workspace_bytes=%zu below awq_gemm_scaled_workspace_bytes=%zu", workspace_bytes, need);
  return device_status(gemm_scaled_via(x, s, packed, scales, zeros, y, M, N, K, bits, workspace, as_stream(stream)),
                       "awq_gemm_scaled");
  AWQ_GUARD_END
}

int awq_gemm_scaled_static(const void* x, const float* s, const void* packed, const void* scales, const void* zeros,
                           void* y, int64_t M, int64_t N, int64_t K, int32_t group, int32_t bits, void* stream) {
  AWQ_GUARD_BEGIN
  AWQ_REQUIRE(x && s && packed && scales && zeros && y, AWQ_ERROR_INVALID_VALUE,
              "x, s, packed, scales, zeros and y must not be NULL");
  int st = check_layer(N, K, group);
  if (st == AWQ_OK) st = check_bits(bits);
  if (st != AWQ_OK) return st;
  AWQ_REQUIRE(M >= 1 && M <= (int64_t(1) << 22), AWQ_ERROR_INVALID_VALUE, "M=%lld outside [1, 2^22]", (long long)M);
  const size_t need = awq_gemm_scaled_workspace_bytes(M, N, K, bits);
  AWQ_REQUIRE(need <= AWQ_STATIC_SCRATCH_BYTES, AWQ_ERROR_INVALID_VALUE,
              "M * K * 2 = %zu bytes exceeds the static scratch of %u bytes", (size_t)(M * K * 2),
              (unsigned)AWQ_STATIC_SCRATCH_BYTES);
  if (int st2 = check_aligned({{x, "x"}, {s, "s"}, {packed, "packed"}, {scales, "scales"}, {zeros, "zeros"},
                                {y, "y"}}))
    return st2;
  void* xs = nullptr;
  if (int st2 = device_scratch(&xs)) return st2;
  return device_status(gemm_scaled_via(x, s, packed, scales, zeros, y, M, N, K, bits, xs, as_stream(stream)),
                       "awq_gemm_scaled_static");
  AWQ_GUARD_END
}

int awq_unpack(const void* packed, const void* zeros, int64_t N, int64_t K, int32_t group, uint8_t* codes,
               uint8_t* zeros_u8, void* stream) {
  return awq_unpack_bits(packed, zeros, N, K, group, 4, codes, zeros_u8, stream);
}

int awq_unpack_bits(const void* packed, const void* zeros, int64_t N, int64_t K, int32_t group, int32_t bits,
                    uint8_t* codes, uint8_t* zeros_u8, void* stream) {
  AWQ_GUARD_BEGIN
  AWQ_REQUIRE(packed && zeros && codes && zeros_u8, AWQ_ERROR_INVALID_VALUE, "pointers must not be NULL");
  int st = check_layer(N, K, group);
  if (st == AWQ_OK) st = check_bits(bits);
  if (st != AWQ_OK) return st;
  if (int st2 = check_aligned({{packed, "packed"}, {zeros, "zeros"}, {codes, "codes"}, {zeros_u8, "zeros_u8"}}))
    return st2;
  return device_status(awq::launch_unpack(packed, zeros, N, K, bits, codes, zeros_u8, as_stream(stream)),
                       "awq_unpack");
  AWQ_GUARD_END
}

}  // extern "C"
