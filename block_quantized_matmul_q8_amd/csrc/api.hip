// C ABI of the Q4 x Q8 library (declared in include/q4q8.h).
//
// Every entry point validates its arguments on the host, launches on the
// caller's stream and returns a status.  Conventions follow the supports_op
// idea of "GGML：Backend 抽象与硬件加速" (section "注册顺序决定默认优先级"):
// a request the library cannot serve is rejected explicitly, never computed
// wrongly.
#include <cxxabi.h>

#include <atomic>
#include <cstdarg>
#include <cstdlib>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <algorithm>
#include <vector>

#include "../../include/q4q8.h"
#include "common.h"

#define Q4Q8_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

thread_local char g_err[512] = "";
thread_local const void* g_last_kernel = nullptr;
thread_local char g_last_kernel_name[512] = "";

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

q4q8::GemvProblem single_problem(const uint8_t* qs, const uint16_t* d, int64_t M, int64_t K, float* y) {
  q4q8::GemvProblem p;
  memset(&p, 0, sizeof p);
  p.qs = qs;
  p.d = d;
  p.y = y;
  p.M = (int32_t)M;
  p.K = (int32_t)K;
  p.win_begin = 0;
  return p;
}

// wf: weight format of qs (q4q8::WeightFormat); both routes serve both.
int matmul_common(const uint8_t* qs, const uint16_t* d, int64_t M, int64_t K, const int8_t* xq,
                  const float* xd, int64_t B, float* y, int32_t* I, void* stream,
                  int wf = q4q8::kWeightQ4) {
  int st = check_matmul_args(qs, d, M, K, xq, xd, B, y);
  if (st) return st;
  if (I && !aligned(I, 4)) return fail(Q4Q8_E_ALIGN, "I misaligned");
  if (M == 0 || B == 0) return ok();
  if ((st = check_device())) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const int path = g_path.load(std::memory_order_relaxed);
  // the multi-column kernel reads the scale planes in 16-byte pieces
  const bool mfma_ok = path != Q4Q8_PATH_GEMV_LANES && q4q8::gemv_mfma_ok(M, K, B, wf) && aligned(d, 16) &&
                       aligned(xd, 16);
  const bool gemv_ok = B <= 8 && (mfma_ok || q4q8::gemv_supported(M, K, B));
  bool use_gemv;
  if (path == Q4Q8_PATH_GEMV || path == Q4Q8_PATH_GEMV_LANES) {
    if (!gemv_ok) return fail(Q4Q8_E_UNSUPPORTED, "GEMV route forced but B = %lld, K = %lld does not fit it", (long long)B, (long long)K);
    use_gemv = true;
  } else if (path == Q4Q8_PATH_GEMM) {
    use_gemv = false;
  } else {
    use_gemv = gemv_ok;
  }
  if (use_gemv && mfma_ok) {
    q4q8::GemvProblem p = single_problem(qs, d, M, K, y);
    p.xq = xq;
    p.xd = xd;
    p.mode = q4q8::kModeQ8;
    p.wf = wf;
    const int win = q4q8::gemv_mfma_window_rows();
    p.n_win = (int32_t)((M + win - 1) / win);
    g_counts[0].fetch_add(1, std::memory_order_relaxed);
    return launched(q4q8::launch_gemv_mfma(p, nullptr, nullptr, p.n_win, 0, B, I, s, wf), "gemv (multi-column)");
  }
  if (use_gemv) {
    q4q8::GemvProblem p = single_problem(qs, d, M, K, y);
    p.xq = xq;
    p.xd = xd;
    p.mode = q4q8::kModeQ8;
    p.wf = wf;
    const int win = q4q8::gemv_window_rows(K, B, wf);
    p.n_win = (int32_t)((M + win - 1) / win);
    g_counts[0].fetch_add(1, std::memory_order_relaxed);
    return launched(q4q8::launch_gemv_table(p, nullptr, nullptr, p.n_win, K, B, false, I, s, wf), "gemv");
  }
  const int64_t tiles = q4q8::gemm_tiles(M, B);
  if (tiles > INT32_MAX || B > INT32_MAX)
    return fail(Q4Q8_E_UNSUPPORTED, "M = %lld, B = %lld exceed the GEMM grid", (long long)M, (long long)B);
  q4q8::GemvProblem p = single_problem(qs, d, M, K, y);
  p.xq = xq;
  p.xd = xd;
  p.wf = wf;
  p.n_win = (int32_t)tiles;
  g_counts[1].fetch_add(1, std::memory_order_relaxed);
  return launched(q4q8::launch_gemm(p, nullptr, nullptr, tiles, B, I, s, wf), "gemm");
}

}  // namespace

namespace q4q8 {
void note_launch(const void* kernel) { g_last_kernel = kernel; }
}  // namespace q4q8

Q4Q8_EXPORT const char* q4q8_last_error(void) { return g_err; }

Q4Q8_EXPORT const char* q4q8_last_kernel(void) {
  g_last_kernel_name[0] = '\0';
  if (!g_last_kernel) return g_last_kernel_name;
  const char* raw = hipKernelNameRefByPtr(g_last_kernel, nullptr);
  if (!raw) return g_last_kernel_name;
  int st = -1;
  char* dem = abi::__cxa_demangle(raw, nullptr, nullptr, &st);
  snprintf(g_last_kernel_name, sizeof g_last_kernel_name, "%s", (st == 0 && dem) ? dem : raw);
  free(dem);
  return g_last_kernel_name;
}

Q4Q8_EXPORT int q4q8_version(void) { return 100; }

// One thread per 32-block: the launch grid must stay within 2^31 workgroups.
static int check_blocks(int64_t M, int64_t K) {
  if (M * (K / q4q8::kQK) > ((int64_t)1 << 38)) return fail(Q4Q8_E_ARG, "matrix too large (M * K / 32 > 2^38)");
  return Q4Q8_OK;
}

Q4Q8_EXPORT int q4_quantize(const float* w, int64_t M, int64_t K, uint8_t* qs, uint16_t* d, void* stream) {
  int st;
  if ((st = check_k(K)) || (st = check_dims(M, 1)) || (st = check_blocks(M, K))) return st;
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

Q4Q8_EXPORT int q8_quantize_rmsnorm_add(const float* x, int64_t B, int64_t K, const float* g, const float* a,
                                        int64_t a_row_stride, float eps, int8_t* xq, float* xd, int32_t* xs,
                                        void* stream) {
  int st;
  if ((st = check_k(K)) || (st = check_dims(1, B))) return st;
  if (K > q4q8::kMaxPrologueK) return fail(Q4Q8_E_ARG, "K = %lld exceeds %d", (long long)K, q4q8::kMaxPrologueK);
  if (a_row_stride != 0 && a_row_stride != K)
    return fail(Q4Q8_E_ARG, "a_row_stride = %lld must be 0 or K", (long long)a_row_stride);
  if (B == 0) return ok();
  if (!x || !g || !a || !xq || !xd) return fail(Q4Q8_E_ARG, "null pointer argument");
  if (!aligned(x, 16) || !aligned(g, 16) || !aligned(a, 16) || !aligned(xq, 16) || !aligned(xd, 4) ||
      (xs && !aligned(xs, 4)))
    return fail(Q4Q8_E_ALIGN, "x, g, a, xq must be 16-byte aligned; xd, xs 4-byte");
  if (!(eps >= 0.0f)) return fail(Q4Q8_E_ARG, "eps must be >= 0");
  if ((st = check_device())) return st;
  g_counts[3].fetch_add(1, std::memory_order_relaxed);
  return launched(q4q8::launch_q8_rmsnorm(x, B, K, g, eps, false, xq, xd, xs, static_cast<hipStream_t>(stream), a,
                                          a_row_stride),
                  "q8_quantize_rmsnorm_add");
}

Q4Q8_EXPORT int q8_quantize_swiglu(const float* gate, const float* up, int64_t B, int64_t F, int64_t row_stride,
                                   int8_t* xq, float* xd, int32_t* xs, void* stream) {
  int st;
  if ((st = check_k(F)) || (st = check_dims(1, B))) return st;
  if (row_stride < F || row_stride % 4)
    return fail(Q4Q8_E_ARG, "row_stride = %lld must be >= F and a multiple of 4", (long long)row_stride);
  // eight lanes per 32-block, 256 per workgroup: the grid stays within 2^31
  if (B * (F / 32) > (int64_t)INT32_MAX * 8) return fail(Q4Q8_E_ARG, "B * F / 32 > 2^34");
  if (B == 0) return ok();
  if (!gate || !up || !xq || !xd) return fail(Q4Q8_E_ARG, "null pointer argument");
  if (!aligned(gate, 16) || !aligned(up, 16) || !aligned(xq, 16) || !aligned(xd, 4) || (xs && !aligned(xs, 4)))
    return fail(Q4Q8_E_ALIGN, "gate, up, xq must be 16-byte aligned; xd, xs 4-byte");
  if ((st = check_device())) return st;
  g_counts[3].fetch_add(1, std::memory_order_relaxed);
  return launched(q4q8::launch_swiglu_q8(gate, up, B, F, row_stride, xq, xd, xs, static_cast<hipStream_t>(stream)),
                  "q8_quantize_swiglu");
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

Q4Q8_EXPORT int q8_0_quantize(const float* w, int64_t M, int64_t K, int8_t* qw, uint16_t* d, void* stream) {
  int st;
  if ((st = check_k(K)) || (st = check_dims(M, 1)) || (st = check_blocks(M, K))) return st;
  if (M == 0) return ok();
  if (!w || !qw || !d) return fail(Q4Q8_E_ARG, "null pointer argument");
  if (!aligned(w, 16) || !aligned(qw, 16) || !aligned(d, 2))
    return fail(Q4Q8_E_ALIGN, "w/qw must be 16-byte aligned, d 2-byte");
  if ((st = check_device())) return st;
  return launched(q4q8::launch_q8w_quantize(w, M, K, qw, d, static_cast<hipStream_t>(stream)), "q8_0_quantize");
}

Q4Q8_EXPORT int mul_mat_q8_0_q8(const int8_t* qw, const uint16_t* d, int64_t M, int64_t K, const int8_t* xq,
                                const float* xd, int64_t B, float* y, void* stream) {
  return matmul_common(reinterpret_cast<const uint8_t*>(qw), d, M, K, xq, xd, B, y, nullptr, stream,
                       q4q8::kWeightQ8);
}

Q4Q8_EXPORT int mul_mat_q8_0_q8_blocksums(const int8_t* qw, const uint16_t* d, int64_t M, int64_t K,
                                          const int8_t* xq, const float* xd, int64_t B, float* y, int32_t* I,
                                          void* stream) {
  if (!I && M > 0 && B > 0) return fail(Q4Q8_E_ARG, "null pointer argument (I)");
  return matmul_common(reinterpret_cast<const uint8_t*>(qw), d, M, K, xq, xd, B, y, I, stream,
                       q4q8::kWeightQ8);
}

Q4Q8_EXPORT size_t mul_mat_id_q4q8_workspace(int64_t E, int64_t T, int64_t top_k) {
  if (E < 0 || T < 0 || top_k < 0) return 0;
  return q4q8::moe_workspace_bytes(E, T, top_k);
}

// Checks shared by the two routed entry points (everything but the workspace).
static int check_moe_args(const uint8_t* qs, const uint16_t* d, int64_t E, int64_t M, int64_t K, const int8_t* xq,
                          const float* xd, int64_t n_x_slots, const int32_t* ids, int64_t T, int64_t top_k,
                          const float* y) {
  int st;
  if ((st = check_k(K)) || (st = check_dims(M, T))) return st;
  if (E <= 0 || E > 4096) return fail(Q4Q8_E_ARG, "E = %lld must be in [1, 4096]", (long long)E);
  if (top_k <= 0 || top_k > 64) return fail(Q4Q8_E_ARG, "top_k = %lld must be in [1, 64]", (long long)top_k);
  if (n_x_slots != 1 && n_x_slots != top_k) return fail(Q4Q8_E_ARG, "n_x_slots must be 1 or top_k");
  if (T * top_k > 65536) return fail(Q4Q8_E_ARG, "T * top_k exceeds 65536");
  if (M == 0 || T == 0) return Q4Q8_OK;
  if (!qs || !d || !xq || !xd || !ids || !y) return fail(Q4Q8_E_ARG, "null pointer argument");
  if (!aligned(qs, 16) || !aligned(xq, 16) || !aligned(d, 2) || !aligned(xd, 4) || !aligned(ids, 4) ||
      !aligned(y, 4))
    return fail(Q4Q8_E_ALIGN, "misaligned pointer argument");
  if (!q4q8::gemv_supported(1, K, 8))
    return fail(Q4Q8_E_UNSUPPORTED, "K = %lld too large for the routed kernel", (long long)K);
  if (q4q8::moe_schedule_cost_bound(E, M, K, T * top_k) >= INT32_MAX)
    return fail(Q4Q8_E_UNSUPPORTED, "M = %lld with E = %lld is too large for the routed schedule", (long long)M,
                (long long)E);
  return Q4Q8_OK;
}

Q4Q8_EXPORT int mul_mat_id_q4q8(const uint8_t* qs, const uint16_t* d, int64_t E, int64_t M, int64_t K,
                                const int8_t* xq, const float* xd, int64_t n_x_slots, const int32_t* ids,
                                int64_t T, int64_t top_k, float* y, void* ws, size_t ws_bytes, void* stream) {
  int st;
  if ((st = check_moe_args(qs, d, E, M, K, xq, xd, n_x_slots, ids, T, top_k, y))) return st;
  if (M == 0 || T == 0) return ok();
  if (!ws) return fail(Q4Q8_E_ARG, "null pointer argument (ws)");
  if (!aligned(ws, 16)) return fail(Q4Q8_E_ALIGN, "misaligned pointer argument (ws)");
  if (ws_bytes < q4q8::moe_workspace_bytes(E, T, top_k))
    return fail(Q4Q8_E_ARG, "workspace of %zu bytes is smaller than the %zu required", ws_bytes,
                q4q8::moe_workspace_bytes(E, T, top_k));
  if ((st = check_device())) return st;
  g_counts[2].fetch_add(1, std::memory_order_relaxed);
  return launched(q4q8::launch_moe(qs, d, E, M, K, xq, xd, n_x_slots, ids, T, top_k, y, ws,
                                   static_cast<hipStream_t>(stream)),
                  "mul_mat_id_q4q8");
}

Q4Q8_EXPORT int mul_mat_id_q4q8_noalloc(const uint8_t* qs, const uint16_t* d, int64_t E, int64_t M, int64_t K,
                                        const int8_t* xq, const float* xd, int64_t n_x_slots, const int32_t* ids,
                                        int64_t T, int64_t top_k, float* y, void* stream) {
  int st;
  if ((st = check_moe_args(qs, d, E, M, K, xq, xd, n_x_slots, ids, T, top_k, y))) return st;
  if (M == 0 || T == 0) return ok();
  const size_t need = q4q8::moe_workspace_bytes(E, T, top_k);
  if (need > q4q8::moe_scratch_bytes())
    return fail(Q4Q8_E_UNSUPPORTED, "routing of E = %lld, T * top_k = %lld needs %zu bytes, beyond the %zu-byte scratch",
                (long long)E, (long long)(T * top_k), need, q4q8::moe_scratch_bytes());
  if ((st = check_device())) return st;
  void* ws = nullptr;
  hipError_t err = q4q8::moe_scratch(&ws);
  if (err != hipSuccess) return fail(Q4Q8_E_LAUNCH, "scratch address: %s", hipGetErrorString(err));
  g_counts[2].fetch_add(1, std::memory_order_relaxed);
  return launched(q4q8::launch_moe(qs, d, E, M, K, xq, xd, n_x_slots, ids, T, top_k, y, ws,
                                   static_cast<hipStream_t>(stream)),
                  "mul_mat_id_q4q8_noalloc");
}

Q4Q8_EXPORT int moe_expert_sum_f32(const float* y, const float* w, int64_t T, int64_t top_k, int64_t M,
                                   float* out, void* stream) {
  if (T < 0 || M < 0 || top_k < 1 || top_k > 64)
    return fail(Q4Q8_E_ARG, "T = %lld, M = %lld must be >= 0 and top_k = %lld in [1, 64]", (long long)T,
                (long long)M, (long long)top_k);
  if (T > 65535) return fail(Q4Q8_E_ARG, "T = %lld exceeds 65535", (long long)T);
  if (M > INT32_MAX / 2) return fail(Q4Q8_E_ARG, "M exceeds 2^30");
  if (T == 0 || M == 0) return ok();
  if (!y || !out) return fail(Q4Q8_E_ARG, "null pointer argument");
  if (!aligned(y, 4) || !aligned(out, 4) || (w && !aligned(w, 4)))
    return fail(Q4Q8_E_ALIGN, "y, w, out must be 4-byte aligned");
  const uintptr_t y0 = reinterpret_cast<uintptr_t>(y), y1 = y0 + (uintptr_t)(T * top_k * M) * 4;
  const uintptr_t o0 = reinterpret_cast<uintptr_t>(out), o1 = o0 + (uintptr_t)(T * M) * 4;
  if (o0 < y1 && y0 < o1) return fail(Q4Q8_E_ARG, "out must not overlap y");
  int st;
  if ((st = check_device())) return st;
  return launched(q4q8::launch_moe_expert_sum(y, w, T, top_k, M, out, static_cast<hipStream_t>(stream)),
                  "moe_expert_sum_f32");
}

Q4Q8_EXPORT int mul_mat_q4q8_rmsnorm(const uint8_t* qs, const uint16_t* d, int64_t M, int64_t K,
                                     const float* x, const float* g, float eps, uint32_t flags, int64_t B,
                                     float* y, void* stream) {
  int st;
  if ((st = check_k(K)) || (st = check_dims(M, B))) return st;
  if (flags & ~Q8_NO_NORM) return fail(Q4Q8_E_ARG, "unknown flags 0x%x", flags);
  const bool no_norm = (flags & Q8_NO_NORM) != 0;
  if (M == 0 || B == 0) return ok();
  if (!qs || !d || !x || !y || (!no_norm && !g)) return fail(Q4Q8_E_ARG, "null pointer argument");
  if (!aligned(qs, 16) || !aligned(x, 16) || (!no_norm && !aligned(g, 16)) || !aligned(d, 2) || !aligned(y, 4))
    return fail(Q4Q8_E_ALIGN, "qs, x, g must be 16-byte aligned; d 2-byte; y 4-byte");
  if (!no_norm && !(eps >= 0.0f)) return fail(Q4Q8_E_ARG, "eps must be >= 0");
  if (!q4q8::gemv_fused_supported(K, B))
    return fail(Q4Q8_E_UNSUPPORTED, "B = %lld, K = %lld too large for the folded-in prologue", (long long)B,
                (long long)K);
  if ((st = check_device())) return st;
  q4q8::GemvProblem p = single_problem(qs, d, M, K, y);
  p.x = x;
  p.g = no_norm ? nullptr : g;
  p.eps = eps;
  p.mode = no_norm ? q4q8::kModeRaw : q4q8::kModeNorm;
  const int win = q4q8::gemv_window_rows(K, B, q4q8::kWeightQ4, true);
  p.n_win = (int32_t)((M + win - 1) / win);
  g_counts[0].fetch_add(1, std::memory_order_relaxed);
  g_counts[3].fetch_add(1, std::memory_order_relaxed);
  return launched(q4q8::launch_gemv_table(p, nullptr, nullptr, p.n_win, K, B, true, nullptr,
                                          static_cast<hipStream_t>(stream)),
                  "mul_mat_q4q8_rmsnorm");
}

namespace {
constexpr uint32_t kGroupMagic = 0x51344738u;  // "Q4G8"

}  // namespace

Q4Q8_EXPORT int q4q8_group_build(const q4q8_gemv_desc* descs, int32_t n, int64_t B, void* workspace,
                                 size_t workspace_bytes, void* table_host, size_t table_bytes,
                                 q4q8_group_plan* plan) {
  if (!plan) return fail(Q4Q8_E_ARG, "null plan");
  memset(plan, 0, sizeof *plan);
  if (n <= 0 || n > (1 << 20)) return fail(Q4Q8_E_ARG, "n = %d must be in [1, 2^20]", n);
  if (!descs) return fail(Q4Q8_E_ARG, "null pointer argument");
  if (B < 1 || B > 65535) return fail(Q4Q8_E_UNSUPPORTED, "B = %lld: grouped products take 1 <= B <= 65535", (long long)B);
  const bool tiled = B > 8;  // the matrix route; B <= 8 streams
  for (int32_t i = 0; i < n; ++i) {
    const q4q8_gemv_desc& e = descs[i];
    int st;
    if ((st = check_k(e.K)) || (st = check_dims(e.M, B))) {
      char msg[sizeof g_err];
      memcpy(msg, g_err, sizeof msg);
      return fail(st, "descriptor %d: %s", i, msg);
    }
    if (e.M == 0) continue;
    if (!e.qs || !e.d || !e.y) return fail(Q4Q8_E_ARG, "descriptor %d: null pointer", i);
    if (!aligned(e.qs, 16) || !aligned(e.d, 2) || !aligned(e.y, 4)) return fail(Q4Q8_E_ALIGN, "descriptor %d: misaligned", i);
    if (e.flags & ~(Q8_NO_NORM | Q4Q8_WEIGHTS_Q8_0)) return fail(Q4Q8_E_ARG, "descriptor %d: unknown flags", i);
    if (!tiled && !q4q8::gemv_route_supported(e.M, e.K, B,
                                              (e.flags & Q4Q8_WEIGHTS_Q8_0) ? q4q8::kWeightQ8 : q4q8::kWeightQ4))
      return fail(Q4Q8_E_UNSUPPORTED, "descriptor %d: K = %lld with B = %lld exceeds the streaming kernel", i,
                  (long long)e.K, (long long)B);
    if (e.xq) {
      if (!e.xd) return fail(Q4Q8_E_ARG, "descriptor %d: xq without xd", i);
      if (!aligned(e.xq, 16) || !aligned(e.xd, 4)) return fail(Q4Q8_E_ALIGN, "descriptor %d: misaligned", i);
    } else {
      const bool no_norm = (e.flags & Q8_NO_NORM) != 0;
      if (!e.x || (!no_norm && !e.g)) return fail(Q4Q8_E_ARG, "descriptor %d: needs xq/xd or x (and g)", i);
      if (!aligned(e.x, 16) || (!no_norm && !aligned(e.g, 16))) return fail(Q4Q8_E_ALIGN, "descriptor %d: misaligned", i);
      if (!no_norm && !(e.eps >= 0.0f)) return fail(Q4Q8_E_ARG, "descriptor %d: eps must be >= 0", i);
      if (e.K > q4q8::kMaxPrologueK)
        return fail(Q4Q8_E_ARG, "descriptor %d: K = %lld exceeds %d for fp32 rows", i, (long long)e.K,
                    q4q8::kMaxPrologueK);
    }
  }
  // Distinct fp32 inputs, in order of first use; each gets its Q8 planes in
  // the workspace: codes [B][K] then scales [B][K/32], each 16-byte aligned.
  struct Input {
    const float* x;
    const float* g;
    int64_t K;
    uint32_t eps_bits;
    uint32_t raw;
    int64_t ws_off;
  };
  std::vector<Input> inputs;
  std::vector<int32_t> input_of(n, -1);
  int64_t ws_total = 0;
  for (int32_t i = 0; i < n; ++i) {
    const q4q8_gemv_desc& e = descs[i];
    if (e.M == 0 || e.xq) continue;
    const uint32_t raw = (e.flags & Q8_NO_NORM) ? 1u : 0u;
    const float* g = raw ? nullptr : e.g;
    uint32_t eps_bits = 0;
    if (!raw) memcpy(&eps_bits, &e.eps, sizeof eps_bits);
    int32_t found = -1;
    for (size_t k = 0; k < inputs.size(); ++k) {
      const Input& in = inputs[k];
      if (in.x == e.x && in.g == g && in.K == e.K && in.eps_bits == eps_bits && in.raw == raw) {
        found = (int32_t)k;
        break;
      }
    }
    if (found < 0) {
      found = (int32_t)inputs.size();
      inputs.push_back({e.x, g, e.K, eps_bits, raw, ws_total});
      ws_total += (B * e.K + 15) / 16 * 16 + (B * (e.K / q4q8::kQK) * 4 + 15) / 16 * 16;
    }
    input_of[i] = found;
  }
  // The streaming pass of B = 5..8 columns runs the multi-column MFMA kernel
  // when it serves every product and all weights have one format, else the
  // lane-per-block kernel (which must then serve every product).
  bool mfma_group = !tiled && B >= q4q8::kGemvMfmaMinB && B <= 8 &&
                    g_path.load(std::memory_order_relaxed) != Q4Q8_PATH_GEMV_LANES;
  int mfma_wf = -1;
  for (int32_t i = 0; i < n && mfma_group; ++i) {
    const q4q8_gemv_desc& e = descs[i];
    if (e.M == 0) continue;
    const int wf = (e.flags & Q4Q8_WEIGHTS_Q8_0) ? q4q8::kWeightQ8 : q4q8::kWeightQ4;
    if (mfma_wf < 0) mfma_wf = wf;
    if (wf != mfma_wf || !q4q8::gemv_mfma_ok(e.M, e.K, B, wf) || !aligned(e.d, 16) || (e.xq && !aligned(e.xd, 16)))
      mfma_group = false;
  }
  if (!tiled && !mfma_group)
    for (int32_t i = 0; i < n; ++i)
      if (descs[i].M > 0 && !q4q8::gemv_supported(descs[i].M, descs[i].K, B))
        return fail(Q4Q8_E_UNSUPPORTED,
                    "descriptor %d: K = %lld with B = %lld needs the multi-column kernel, which does not serve "
                    "every product of the group", i, (long long)descs[i].K, (long long)B);
  // Product records in the caller's order, all in one streaming launch (the
  // kernel dispatches per product on its register-blocking class).
  std::vector<q4q8::GemvProblem> recs;
  std::vector<int64_t> rec_tiles;
  int64_t tiles = 0, max_k = 0;
  for (int32_t i = 0; i < n; ++i) {
    const q4q8_gemv_desc& e = descs[i];
    if (e.M == 0) continue;
    q4q8::GemvProblem p = single_problem(e.qs, e.d, e.M, e.K, e.y);
    p.mode = q4q8::kModeQ8;
    p.wf = (e.flags & Q4Q8_WEIGHTS_Q8_0) ? q4q8::kWeightQ8 : q4q8::kWeightQ4;
    if (e.xq) {
      p.xq = e.xq;
      p.xd = e.xd;
    } else if (workspace) {
      char* base = static_cast<char*>(workspace) + inputs[input_of[i]].ws_off;
      p.xq = reinterpret_cast<const int8_t*>(base);
      p.xd = reinterpret_cast<const float*>(base + (B * e.K + 15) / 16 * 16);
    }
    int64_t t;
    if (tiled) {
      t = q4q8::gemm_tiles(e.M, B);
    } else {
      const int win = mfma_group ? q4q8::gemv_mfma_window_rows() : q4q8::gemv_window_rows(e.K, B, p.wf);
      t = (e.M + win - 1) / win;
    }
    tiles += t;
    if (tiles > INT32_MAX) return fail(Q4Q8_E_ARG, "too many windows");
    p.n_win = (int32_t)t;
    if (e.K > max_k) max_k = e.K;
    recs.push_back(p);
    rec_tiles.push_back(t);
  }
  // Work order: streamed products in the caller's order; tiled products
  // longest K first (their tiles take longest), ties in the caller's order.
  std::vector<int32_t> order(recs.size());
  for (size_t r = 0; r < recs.size(); ++r) order[r] = (int32_t)r;
  if (tiled)
    std::stable_sort(order.begin(), order.end(),
                     [&](int32_t a, int32_t b) { return recs[a].K > recs[b].K; });
  // Multi-column groups: the windows are packed into one bin per workgroup
  // (cost of a window = K / 32 blocks per row, its 64 rows being common), and
  // each run of consecutive windows of one product in a bin becomes a record
  // of its own (win_off: its first window within the product).  Other
  // routes: one record per product, its windows consecutive.
  std::vector<q4q8::MfRun> runs;
  std::vector<int64_t> bounds;
  int64_t mfma_grid = 0;
  if (mfma_group && !recs.empty()) {
    std::vector<int64_t> cost(recs.size());
    int64_t total = 0;
    for (size_t r = 0; r < recs.size(); ++r) {
      cost[r] = recs[r].K / q4q8::kQK;
      total += rec_tiles[r] * cost[r];
    }
    if (total > INT32_MAX)
      return fail(Q4Q8_E_UNSUPPORTED, "group too large for the multi-column route (windows x K / 32 > 2^31)");
    mfma_grid = std::min<int64_t>(q4q8::gemv_mfma_group_grid(mfma_wf), tiles);
    q4q8::gemv_mfma_pack(rec_tiles, cost, mfma_grid, runs, bounds);
  } else {
    int64_t first = 0;
    for (int32_t r : order) {
      recs[r].win_begin = (int32_t)first;
      first += rec_tiles[r];
    }
  }
  const int64_t n_records = mfma_grid ? (int64_t)runs.size() : (int64_t)recs.size();
  plan->B = (int32_t)B;
  plan->n_records = (int32_t)n_records;
  plan->n_prologue = (int32_t)inputs.size();
  plan->n_windows = tiles;
  plan->max_k = max_k;
  plan->map_offset = n_records * (int64_t)sizeof(q4q8::GemvProblem);
  plan->prologue_offset =
      (plan->map_offset + (tiles + (mfma_grid ? mfma_grid + 1 : 0)) * (int64_t)sizeof(int32_t) + 15) / 16 * 16;
  plan->table_bytes = plan->prologue_offset + (int64_t)(inputs.size() * sizeof(q4q8::PrologueJob));
  plan->workspace_bytes = ws_total;
  plan->weight_formats = 0;
  for (const q4q8::GemvProblem& r : recs) plan->weight_formats |= 1 << r.wf;
  plan->max_prologue_k = 0;
  for (const Input& in : inputs) plan->max_prologue_k = std::max(plan->max_prologue_k, (int32_t)in.K);
  plan->mfma_columns = mfma_grid ? 1 : 0;
  plan->mfma_grid = (int32_t)mfma_grid;
  plan->magic = kGroupMagic;
  if (!table_host) return ok();
  const char* why = nullptr;
  int st = Q4Q8_E_ARG;
  if (table_bytes < (size_t)plan->table_bytes) {
    why = "table buffer is smaller than plan->table_bytes";
  } else if (!aligned(table_host, 16)) {
    why = "table buffer must be 16-byte aligned";
    st = Q4Q8_E_ALIGN;
  } else if (ws_total > 0 && !workspace) {
    why = "products take fp32 rows: a workspace of plan->workspace_bytes is required";
  } else if (ws_total > 0 && workspace_bytes < (size_t)ws_total) {
    why = "workspace is smaller than plan->workspace_bytes";
  } else if (ws_total > 0 && !aligned(workspace, 16)) {
    why = "workspace must be 16-byte aligned";
    st = Q4Q8_E_ALIGN;
  }
  if (why) {
    plan->magic = 0;
    return fail(st, "%s", why);
  }
  char* out = static_cast<char*>(table_host);
  memset(out, 0, (size_t)plan->table_bytes);
  int32_t* map = reinterpret_cast<int32_t*>(out + plan->map_offset);
  if (mfma_grid) {
    q4q8::GemvProblem* rec_out = reinterpret_cast<q4q8::GemvProblem*>(out);
    int64_t m = 0;
    for (size_t i = 0; i < runs.size(); ++i) {
      q4q8::GemvProblem p = recs[runs[i].rec];
      p.win_begin = (int32_t)m;
      p.n_win = runs[i].count;
      p.win_off = runs[i].first;
      rec_out[i] = p;
      for (int32_t t = 0; t < runs[i].count; ++t) map[m++] = (int32_t)i;
    }
    for (size_t g = 0; g < bounds.size(); ++g) map[tiles + g] = (int32_t)bounds[g];
  } else {
    memcpy(out, recs.data(), recs.size() * sizeof(q4q8::GemvProblem));
    int64_t m = 0;
    for (int32_t r : order)
      for (int64_t t = 0; t < rec_tiles[r]; ++t) map[m++] = r;
  }
  q4q8::PrologueJob* jobs = reinterpret_cast<q4q8::PrologueJob*>(out + plan->prologue_offset);
  for (size_t k = 0; k < inputs.size(); ++k) {
    const Input& in = inputs[k];
    char* base = static_cast<char*>(workspace) + in.ws_off;
    q4q8::PrologueJob j;
    memset(&j, 0, sizeof j);
    j.x = in.x;
    j.g = in.g;
    j.xq = reinterpret_cast<int8_t*>(base);
    j.xd = reinterpret_cast<float*>(base + (B * in.K + 15) / 16 * 16);
    j.K = (int32_t)in.K;
    memcpy(&j.eps, &in.eps_bits, sizeof j.eps);
    j.raw = (int32_t)in.raw;
    jobs[k] = j;
  }
  return ok();
}

Q4Q8_EXPORT int mul_mat_q4q8_group(const void* table_dev, const q4q8_group_plan* plan, void* stream) {
  if (!plan || plan->magic != kGroupMagic) return fail(Q4Q8_E_ARG, "plan not built by q4q8_group_build");
  if (plan->n_records == 0) return ok();
  if (!table_dev) return fail(Q4Q8_E_ARG, "null table");
  if (!aligned(table_dev, 16)) return fail(Q4Q8_E_ALIGN, "table must be 16-byte aligned");
  const bool tiled = plan->B > 8;
  if (plan->n_records < 0 || plan->B < 1 || plan->B > 65535 || plan->n_windows < plan->n_records ||
      plan->n_windows > INT32_MAX || plan->n_prologue < 0 || plan->n_prologue > plan->n_records ||
      plan->max_k < q4q8::kQK || plan->max_k % q4q8::kQK != 0 ||
      plan->mfma_columns < 0 || plan->mfma_columns > 1 ||
      (plan->mfma_columns ? plan->mfma_grid < 1 || plan->mfma_grid > plan->n_windows : plan->mfma_grid != 0) ||
      (plan->mfma_columns && (tiled || plan->B < q4q8::kGemvMfmaMinB || plan->max_k < 512 || plan->max_k % 128 != 0 ||
                                 plan->weight_formats == 3)) ||
      (!tiled && !plan->mfma_columns && !q4q8::gemv_supported(1, plan->max_k, plan->B)) ||
      plan->map_offset != (int64_t)plan->n_records * (int64_t)sizeof(q4q8::GemvProblem) ||
      plan->prologue_offset != (plan->map_offset +
                                (plan->n_windows + (plan->mfma_columns ? plan->mfma_grid + 1 : 0)) *
                                    (int64_t)sizeof(int32_t) +
                                15) / 16 * 16 ||
      plan->table_bytes != plan->prologue_offset + plan->n_prologue * (int64_t)sizeof(q4q8::PrologueJob) ||
      plan->weight_formats < 1 || plan->weight_formats > 3 || plan->max_prologue_k < 0 ||
      plan->max_prologue_k > plan->max_k || plan->max_prologue_k % q4q8::kQK != 0 ||
      plan->max_prologue_k > q4q8::kMaxPrologueK || (plan->n_prologue > 0) != (plan->max_prologue_k > 0))
    return fail(Q4Q8_E_ARG, "corrupt plan");
  // the kernel instance: single-format groups take the leaner ones
  const int wf = plan->weight_formats == 1   ? q4q8::kWeightQ4
                 : plan->weight_formats == 2 ? q4q8::kWeightQ8
                                             : q4q8::kWeightMixed;
  int st;
  if ((st = check_device())) return st;
  const char* base = static_cast<const char*>(table_dev);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (plan->n_prologue > 0) {
    g_counts[3].fetch_add(1, std::memory_order_relaxed);
    st = launched(q4q8::launch_group_prologue(
                      reinterpret_cast<const q4q8::PrologueJob*>(base + plan->prologue_offset),
                      plan->n_prologue, plan->B, plan->max_prologue_k, s),
                  "mul_mat_q4q8_group (prologue pass)");
    if (st) return st;
  }
  q4q8::GemvProblem unused;
  memset(&unused, 0, sizeof unused);
  if (tiled) {
    g_counts[1].fetch_add(1, std::memory_order_relaxed);
    return launched(q4q8::launch_gemm(unused, reinterpret_cast<const q4q8::GemvProblem*>(base),
                                      reinterpret_cast<const int32_t*>(base + plan->map_offset), plan->n_windows,
                                      plan->B, nullptr, s, wf),
                    "mul_mat_q4q8_group (tiled)");
  }
  g_counts[0].fetch_add(1, std::memory_order_relaxed);
  if (plan->mfma_columns)
    return launched(q4q8::launch_gemv_mfma(unused, reinterpret_cast<const q4q8::GemvProblem*>(base),
                                           reinterpret_cast<const int32_t*>(base + plan->map_offset),
                                           plan->n_windows, plan->mfma_grid, plan->B, nullptr, s, wf),
                    "mul_mat_q4q8_group (multi-column)");
  return launched(q4q8::launch_gemv_table(unused, reinterpret_cast<const q4q8::GemvProblem*>(base),
                                          reinterpret_cast<const int32_t*>(base + plan->map_offset),
                                          plan->n_windows, plan->max_k, plan->B, false, nullptr, s, wf),
                  "mul_mat_q4q8_group");
}

Q4Q8_EXPORT int q4q8_set_path(int path) {
  if (path != Q4Q8_PATH_AUTO && path != Q4Q8_PATH_GEMV && path != Q4Q8_PATH_GEMM && path != Q4Q8_PATH_GEMV_LANES)
    return fail(Q4Q8_E_ARG, "unknown path %d", path);
  g_path.store(path, std::memory_order_relaxed);
  return ok();
}

Q4Q8_EXPORT int q4q8_dispatch_counts(uint64_t out[4], int reset) {
  if (!out) return fail(Q4Q8_E_ARG, "null pointer argument");
  for (int i = 0; i < 4; ++i) out[i] = reset ? g_counts[i].exchange(0) : g_counts[i].load();
  return ok();
}
