// C ABI of the Q4 x Q8 library (declared in include/q4q8.h).
//
// Every entry point validates its arguments on the host, launches on the
// caller's stream and returns a status.  Conventions follow the supports_op
// idea of "GGML：Backend 抽象与硬件加速" (section "注册顺序决定默认优先级"):
// a request the library cannot serve is rejected explicitly, never computed
// wrongly.
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/q4q8.h"
#include "common.h"

#define Q4Q8_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return Q4Q8_OK;
}

std::atomic<int> g_path{Q4Q8_PATH_AUTO};
std::atomic<uint64_t> g_counts[4];

constexpr int kMaxDevices = 64;
std::atomic<int> g_arch[kMaxDevices];  // 0 unknown, 1 gfx950, -1 other
std::mutex g_arch_mu;

int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0)
    return fail(Q4Q8_E_ARCH, "no current HIP device");
  if (dev >= kMaxDevices) return fail(Q4Q8_E_ARCH, "device index %d out of range", dev);
  int st = g_arch[dev].load(std::memory_order_acquire);
  if (st == 0) {
    std::lock_guard<std::mutex> lk(g_arch_mu);
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
      return fail(Q4Q8_E_ARCH, "hipGetDeviceProperties failed for device %d", dev);
    st = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    g_arch[dev].store(st, std::memory_order_release);
  }
  if (st != 1) return fail(Q4Q8_E_ARCH, "device %d is not gfx950", dev);
  return Q4Q8_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(Q4Q8_E_LAUNCH, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

int check_k(int64_t K) {
  if (K <= 0 || K % q4q8::kQK) return fail(Q4Q8_E_ARG, "K = %lld must be a positive multiple of 32", (long long)K);
  if (K > (int64_t)1 << 24) return fail(Q4Q8_E_ARG, "K = %lld exceeds 2^24", (long long)K);
  return Q4Q8_OK;
}

int check_dims(int64_t M, int64_t B) {
  if (M < 0 || B < 0) return fail(Q4Q8_E_ARG, "negative dimension (M = %lld, B = %lld)", (long long)M, (long long)B);
  if (M > INT32_MAX || B > INT32_MAX) return fail(Q4Q8_E_ARG, "dimension exceeds 2^31 - 1");
  return Q4Q8_OK;
}

int check_matmul_args(const uint8_t* qs, const uint16_t* d, int64_t M, int64_t K, const int8_t* xq,
                      const float* xd, int64_t B, const float* y) {
  int st;
  if ((st = check_k(K)) || (st = check_dims(M, B))) return st;
  if (M == 0 || B == 0) return Q4Q8_OK;
  if (!qs || !d || !xq || !xd || !y) return fail(Q4Q8_E_ARG, "null pointer argument");
  if (!aligned(qs, 16) || !aligned(xq, 16)) return fail(Q4Q8_E_ALIGN, "qs and xq must be 16-byte aligned");
  if (!aligned(d, 2) || !aligned(xd, 4) || !aligned(y, 4)) return fail(Q4Q8_E_ALIGN, "d, xd or y misaligned");
  if ((int64_t)M * (K / q4q8::kQK) > ((int64_t)1 << 40)) return fail(Q4Q8_E_ARG, "matrix too large");
  return Q4Q8_OK;
}

int matmul_common(const uint8_t* qs, const uint16_t* d, int64_t M, int64_t K, const int8_t* xq,
                  const float* xd, int64_t B, float* y, int32_t* I, void* stream) {
  int st = check_matmul_args(qs, d, M, K, xq, xd, B, y);
  if (st) return st;
  if (I && !aligned(I, 4)) return fail(Q4Q8_E_ALIGN, "I misaligned");
  if (M == 0 || B == 0) return ok();
  if ((st = check_device())) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const int path = g_path.load(std::memory_order_relaxed);
  const bool gemv_ok = q4q8::gemv_supported(M, K, B);
  bool use_gemv;
  if (path == Q4Q8_PATH_GEMV) {
    if (!gemv_ok) return fail(Q4Q8_E_UNSUPPORTED, "GEMV route forced but B = %lld, K = %lld does not fit it", (long long)B, (long long)K);
    use_gemv = true;
  } else if (path == Q4Q8_PATH_GEMM) {
    use_gemv = false;
  } else {
    use_gemv = gemv_ok;
  }
  if (use_gemv) {
    g_counts[0].fetch_add(1, std::memory_order_relaxed);
    return launched(q4q8::launch_gemv(qs, d, M, K, xq, xd, B, y, I, s), "gemv");
  }
  if (B > (int64_t)65535 * 128) return fail(Q4Q8_E_UNSUPPORTED, "B = %lld exceeds the GEMM grid", (long long)B);
  g_counts[1].fetch_add(1, std::memory_order_relaxed);
  return launched(q4q8::launch_gemm(qs, d, M, K, xq, xd, B, y, I, s), "gemm");
}

}  // namespace

Q4Q8_EXPORT const char* q4q8_last_error(void) { return g_err; }

Q4Q8_EXPORT int q4q8_version(void) { return 100; }

Q4Q8_EXPORT int q4_quantize(const float* w, int64_t M, int64_t K, uint8_t* qs, uint16_t* d, void* stream) {
  int st;
  if ((st = check_k(K)) || (st = check_dims(M, 1))) return st;
  if (M == 0) return ok();
  if (!w || !qs || !d) return fail(Q4Q8_E_ARG, "null pointer argument");
  if (!aligned(w, 16) || !aligned(qs, 16) || !aligned(d, 2)) return fail(Q4Q8_E_ALIGN, "w/qs must be 16-byte aligned, d 2-byte");
  if ((st = check_device())) return st;
  return launched(q4q8::launch_q4_quantize(w, M, K, qs, d, static_cast<hipStream_t>(stream)), "q4_quantize");
}

Q4Q8_EXPORT int q8_quantize_rmsnorm(const float* x, int64_t B, int64_t K, const float* g, float eps,
                                    uint32_t flags, int8_t* xq, float* xd, int32_t* xs, void* stream) {
  int st;
  if ((st = check_k(K)) || (st = check_dims(1, B))) return st;
  if (K > q4q8::kMaxPrologueK) return fail(Q4Q8_E_ARG, "K = %lld exceeds %d", (long long)K, q4q8::kMaxPrologueK);
  if (flags & ~Q8_NO_NORM) return fail(Q4Q8_E_ARG, "unknown flags 0x%x", flags);
  const bool no_norm = (flags & Q8_NO_NORM) != 0;
  if (B == 0) return ok();
  if (!x || !xq || !xd || (!no_norm && !g)) return fail(Q4Q8_E_ARG, "null pointer argument");
  if (!aligned(x, 16) || !aligned(xq, 16) || (!no_norm && !aligned(g, 16)) || !aligned(xd, 4) || (xs && !aligned(xs, 4)))
    return fail(Q4Q8_E_ALIGN, "x, g, xq must be 16-byte aligned; xd, xs 4-byte");
  if (!no_norm && !(eps >= 0.0f)) return fail(Q4Q8_E_ARG, "eps must be >= 0");
  if ((st = check_device())) return st;
  g_counts[3].fetch_add(1, std::memory_order_relaxed);
  return launched(q4q8::launch_q8_rmsnorm(x, B, K, g, eps, no_norm, xq, xd, xs, static_cast<hipStream_t>(stream)),
                  "q8_quantize_rmsnorm");
}

Q4Q8_EXPORT int mul_mat_q4q8(const uint8_t* qs, const uint16_t* d, int64_t M, int64_t K, const int8_t* xq,
                             const float* xd, int64_t B, float* y, void* stream) {
  return matmul_common(qs, d, M, K, xq, xd, B, y, nullptr, stream);
}

Q4Q8_EXPORT int mul_mat_q4q8_blocksums(const uint8_t* qs, const uint16_t* d, int64_t M, int64_t K,
                                       const int8_t* xq, const float* xd, int64_t B, float* y, int32_t* I,
                                       void* stream) {
  if (!I && M > 0 && B > 0) return fail(Q4Q8_E_ARG, "null pointer argument (I)");
  return matmul_common(qs, d, M, K, xq, xd, B, y, I, stream);
}

Q4Q8_EXPORT size_t mul_mat_id_q4q8_workspace(int64_t E, int64_t T, int64_t top_k) {
  if (E < 0 || T < 0 || top_k < 0) return 0;
  return q4q8::moe_workspace_bytes(E, T, top_k);
}

Q4Q8_EXPORT int mul_mat_id_q4q8(const uint8_t* qs, const uint16_t* d, int64_t E, int64_t M, int64_t K,
                                const int8_t* xq, const float* xd, int64_t n_x_slots, const int32_t* ids,
                                int64_t T, int64_t top_k, float* y, void* ws, size_t ws_bytes, void* stream) {
  int st;
  if ((st = check_k(K)) || (st = check_dims(M, T))) return st;
  if (E <= 0 || E > 16384) return fail(Q4Q8_E_ARG, "E = %lld must be in [1, 16384]", (long long)E);
  if (top_k <= 0 || top_k > 64) return fail(Q4Q8_E_ARG, "top_k = %lld must be in [1, 64]", (long long)top_k);
  if (n_x_slots != 1 && n_x_slots != top_k) return fail(Q4Q8_E_ARG, "n_x_slots must be 1 or top_k");
  if (T * top_k > 65536) return fail(Q4Q8_E_ARG, "T * top_k exceeds 65536");
  if (M == 0 || T == 0) return ok();
  if (!qs || !d || !xq || !xd || !ids || !y || !ws) return fail(Q4Q8_E_ARG, "null pointer argument");
  if (!aligned(qs, 16) || !aligned(xq, 16) || !aligned(ws, 16) || !aligned(d, 2) || !aligned(xd, 4) ||
      !aligned(ids, 4) || !aligned(y, 4))
    return fail(Q4Q8_E_ALIGN, "misaligned pointer argument");
  if (ws_bytes < q4q8::moe_workspace_bytes(E, T, top_k))
    return fail(Q4Q8_E_ARG, "workspace of %zu bytes is smaller than the %zu required", ws_bytes,
                q4q8::moe_workspace_bytes(E, T, top_k));
  const size_t lds = 4 * (size_t)K + 8 * 4 * (size_t)(K / q4q8::kQK);
  if (lds > 64 * 1024) return fail(Q4Q8_E_UNSUPPORTED, "K = %lld too large for the routed kernel", (long long)K);
  if ((st = check_device())) return st;
  g_counts[2].fetch_add(1, std::memory_order_relaxed);
  return launched(q4q8::launch_moe(qs, d, E, M, K, xq, xd, n_x_slots, ids, T, top_k, y, ws,
                                   static_cast<hipStream_t>(stream)),
                  "mul_mat_id_q4q8");
}

Q4Q8_EXPORT int q4q8_set_path(int path) {
  if (path != Q4Q8_PATH_AUTO && path != Q4Q8_PATH_GEMV && path != Q4Q8_PATH_GEMM)
    return fail(Q4Q8_E_ARG, "unknown path %d", path);
  g_path.store(path, std::memory_order_relaxed);
  return ok();
}

Q4Q8_EXPORT int q4q8_dispatch_counts(uint64_t out[4], int reset) {
  if (!out) return fail(Q4Q8_E_ARG, "null pointer argument");
  for (int i = 0; i < 4; ++i) out[i] = reset ? g_counts[i].exchange(0) : g_counts[i].load();
  return ok();
}
