// Streaming Q4 x Q8 matrix x vector kernel for gfx950 (the decode route; the
// mmvq role in "GGML：Backend 抽象与硬件加速", section "CUDA：mmvq、mmq、cublas
// 三条矩阵路": decode is a quantised matrix x vector product, and a dedicated
// vector kernel is cheaper to launch than the matrix path).
//
// The plain (one product) and grouped (a device table of products plus a
// window -> record map) kernels over the streaming segment of gemv_dev.h,
// and their host-side launchers.
#include <mutex>
#include <utility>
#include <vector>

#include "gemv_dev.h"

namespace q4q8 {

// Persistent grid: workgroup g streams the g-th equal share of the window
// list (the windows of all products, product after product), so every
// workgroup carries the same load from start to end and the launch has no
// rounds of short-lived workgroups.  A share spans few products; the next
// product's record is requested when a segment starts, so it is at hand when
// the segment ends.  A grouped instance serves every blocking class of its
// column width up to its template J (the workgroup dispatches uniformly on
// each product's class) and reads Q8 planes only; single-product instances
// compile their own class only.  The grouped and single-product forms are separate instances because
// selecting between the kernel argument and the table at run time would make
// every access a generic flat access.
#ifndef Q4Q8_GEMV_MIN_WG_PER_CU
#define Q4Q8_GEMV_MIN_WG_PER_CU 1
#endif

enum GemvKind : int {
  kKindGroup = 0,      // table of products, Q8 planes
  kKindSingle = 1,     // one product, Q8 planes
  kKindFold = 2,       // one product, fp32 rows, prologue folded in
  kKindBlockSums = 3,  // one product, Q8 planes, per-block sums written out
};

// Workgroups per CU an instance is built for.  A grouped instance holds the
// segments of every blocking class up to J, so its registers are the largest
// of theirs; the single-column Q4 instance without the 8-block classes (every
// product with K <= 32768) and the two-column one without the 4-block
// classes (K <= 16384) fit two workgroups per CU at the full rows in flight,
// which measured 1.3-2.5% faster on the Llama-3.2-1B decode step.
// With an 8-block class it needs more than 256 registers; holding it to 256
// spills, and halving that class's rows instead cost 3% on K = 14336.
__host__ __device__ constexpr int gemv_min_wg_per_cu(int BT, int J, int KIND, int WF) {
  return KIND == kKindGroup && WF == kWeightQ4 && ((BT == 1 && J <= 4) || (BT == 2 && J <= 2))
             ? 2
             : Q4Q8_GEMV_MIN_WG_PER_CU;
}

// WF: weight format of the products (kWeightMixed, grouped only: each
// record's format decides; the folded prologue serves Q4 weights).  A Q8_0
// block is two loads, so it keeps half the rows in flight for the same bytes
// in flight.  A mixed instance holds both segments (the larger register
// footprint of the two), so uniform groups take the single-format ones.
// Grouped instances (KIND == kKindGroup): J is the largest blocking class
// served (every product's class must have at most J blocks per lane).
template <int BT, int J, int S, int KIND, int WF = kWeightQ4>
__global__ __launch_bounds__(kGemvThreads, gemv_min_wg_per_cu(BT, J, KIND, WF)) void gemv_kernel(
    GemvProblem p0, const GemvProblem* __restrict__ table, const int32_t* __restrict__ win_map,
    int n_windows, int B, int32_t* __restrict__ Iout) {
  constexpr bool GROUPED = KIND == kKindGroup;
  constexpr bool FOLD = KIND == kKindFold;
  constexpr bool WRITE_I = KIND == kKindBlockSums;
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ SplitScratch split;
  const int64_t G = gridDim.x, g = blockIdx.x;
  const int w_begin = (int)(n_windows * g / G);
  const int w_end = (int)(n_windows * (g + 1) / G);
  int parity = 0;
  if constexpr (GROUPED) {
    int rec = win_map[w_begin];
    const int rec_last = win_map[w_end - 1];
    GemvProblem P = table[rec];
    for (int w = w_begin; w < w_end;) {
      const int seg_end = min(w_end, P.win_begin + P.n_win);
      const GemvProblem Pn = table[min(rec + 1, rec_last)];
      const int wl0 = w - P.win_begin, wl1 = seg_end - P.win_begin;
      const GemvClass cls = gemv_class_of(P.K, BT, WF == kWeightMixed ? P.wf : WF);
      dispatch_class<BT>(cls.J, cls.S, [&]<int JJ, int SS>() {
        if constexpr (JJ > J) return;
        if (WF == kWeightQ8 || (WF == kWeightMixed && P.wf == kWeightQ8))
          gemv_segment<BT, JJ, SS, false, false, DenseCols, gemv_rif(BT, kWeightQ8), kWeightQ8>(
              P, DenseCols(P), B, wl0, wl1, smem, &split, parity, Iout);
        else
          gemv_segment<BT, JJ, SS, false, false, DenseCols, gemv_rif(BT, kWeightQ4)>(
              P, DenseCols(P), B, wl0, wl1, smem, &split, parity, Iout);
      });
      w = seg_end;
      P = Pn;
      ++rec;
    }
  } else {
    if (w_begin < w_end)
      gemv_segment<BT, J, S, FOLD, WRITE_I, DenseCols, gemv_rif(BT, WF), WF>(p0, DenseCols(p0), B, w_begin, w_end,
                                                                             smem, &split, parity, Iout);
  }
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------

static size_t fused_lds_bytes(int64_t K, int64_t B) {
  const int64_t nb = K / kQK;
  return (size_t)(B * K + 8 * B * nb + 8 * sizeof(float));
}

bool gemv_supported(int64_t M, int64_t K, int64_t B) {
  (void)M;
  return gemv_class_of(K, B).J != 0;
}

bool gemv_mfma_ok(int64_t M, int64_t K, int64_t B, int wf) {
  // rows of at least four whole 128-byte segments (Q4: K a multiple of 256,
  // at least 1024; Q8_0: a multiple of 128, at least 512).  Five or more
  // columns: up to four, the lane-per-block kernel streams faster (it runs
  // four columns without padding; the matrix kernel pays for the activation
  // operands and the exchange of partial sums whatever B is).
  const int64_t row_bytes = wf == kWeightQ8 ? K : K / 2;
  return (wf == kWeightQ4 || wf == kWeightQ8) && B >= kGemvMfmaMinB && B <= 8 && row_bytes >= 512 &&
         row_bytes % 128 == 0 &&
         K % 64 == 0 && M >= 1 && M * row_bytes < ((int64_t)1 << 31) && B * K < ((int64_t)1 << 30);
}

bool gemv_route_supported(int64_t M, int64_t K, int64_t B, int wf) {
  return gemv_mfma_ok(M, K, B, wf) || gemv_class_of(K, B).J != 0;
}

bool gemv_fused_supported(int64_t K, int64_t B) {
  const GemvClass c = gemv_class_unsplit(K, B);
  return B <= 4 && c.J != 0 && c.S == 1 && fused_lds_bytes(K, B) <= kGemvMaxLds;
}

int gemv_window_rows(int64_t K, int64_t B, int wf, bool fold) {
  if (B < 1 || B > 8) return 0;
  return gemv_window_rows_bt(K, gemv_bt((int)B), gemv_rif(gemv_bt((int)B), wf), fold || wf == kWeightQ8);
}

// Workgroups that can be resident at once for one kernel instance and LDS
// size, times the CU count (queried once per instance, size and device).
static int64_t resident_workgroups(const void* kernel, size_t lds) {
  struct Key {
    const void* k;
    size_t lds;
    int dev;
  };
  static std::mutex mu;
  static std::vector<std::pair<Key, int64_t>> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  std::lock_guard<std::mutex> lk(mu);
  for (const auto& e : cache)
    if (e.first.k == kernel && e.first.lds == lds && e.first.dev == dev) return e.second;
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kGemvThreads, lds) != hipSuccess ||
      per_cu < 1)
    per_cu = 1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    cus = 256;
  const int64_t n = (int64_t)per_cu * cus;
  cache.push_back({Key{kernel, lds, dev}, n});
  return n;
}

template <int BT, int J, int S, int KIND, int WF = kWeightQ4>
static hipError_t launch_kind(const GemvProblem& p, const GemvProblem* table, const int32_t* map,
                              int64_t n_windows, int B, size_t lds, int32_t* I, hipStream_t s) {
  const void* k = (const void*)gemv_kernel<BT, J, S, KIND, WF>;
  int64_t grid = resident_workgroups(k, lds);
  if (grid > n_windows) grid = n_windows;
  note_launch(k);
  hipLaunchKernelGGL((gemv_kernel<BT, J, S, KIND, WF>), dim3((unsigned)grid), dim3(kGemvThreads), lds, s, p,
                     table, map, (int)n_windows, B, I);
  return hipGetLastError();
}

template <int BT>
static hipError_t launch_bt(const GemvProblem& p, const GemvProblem* table, const int32_t* map,
                            int64_t n_windows, int64_t max_k, int B, bool fold, int32_t* I, hipStream_t s,
                            int wf) {
  if (table) {
    // max_k is the group's largest K: every product's class is at most its class
    if (wf == kWeightQ8) return launch_kind<BT, 8, 1, kKindGroup, kWeightQ8>(p, table, map, n_windows, B, 0, I, s);
    if (wf == kWeightMixed)
      return launch_kind<BT, 8, 1, kKindGroup, kWeightMixed>(p, table, map, n_windows, B, 0, I, s);
    if constexpr (BT == 1) {
      const GemvClass c = gemv_class_of(max_k, BT);
      if (c.J <= 4) return launch_kind<BT, 4, 1, kKindGroup>(p, table, map, n_windows, B, 0, I, s);
    }
    if constexpr (BT == 2) {
      const GemvClass c = gemv_class_of(max_k, BT);
      if (c.J <= 2) return launch_kind<BT, 2, 1, kKindGroup>(p, table, map, n_windows, B, 0, I, s);
    }
    return launch_kind<BT, 8, 1, kKindGroup>(p, table, map, n_windows, B, 0, I, s);
  }
  if (wf == kWeightQ8) {
    if (fold) return hipErrorInvalidValue;
    const GemvClass c = gemv_class_of(max_k, B, kWeightQ8);
    hipError_t err = hipErrorInvalidValue;
    dispatch_class<BT>(c.J, c.S, [&]<int JJ, int SS>() {
      if (I)
        err = launch_kind<BT, JJ, SS, kKindBlockSums, kWeightQ8>(p, nullptr, nullptr, n_windows, B, 0, I, s);
      else
        err = launch_kind<BT, JJ, SS, kKindSingle, kWeightQ8>(p, nullptr, nullptr, n_windows, B, 0, I, s);
    });
    return err;
  }
  const GemvClass c = fold ? gemv_class_unsplit(max_k, B) : gemv_class_of(max_k, B);
  const size_t lds = fold ? fused_lds_bytes(max_k, B) : 0;
  hipError_t err = hipErrorInvalidValue;
  dispatch_class<BT>(c.J, c.S, [&]<int JJ, int SS>() {
    if constexpr (SS == 1) {
      if (fold) {
        err = launch_kind<BT, JJ, SS, kKindFold>(p, nullptr, nullptr, n_windows, B, lds, I, s);
        return;
      }
    }
    if (fold) return;
    if (I)
      err = launch_kind<BT, JJ, SS, kKindBlockSums>(p, nullptr, nullptr, n_windows, B, 0, I, s);
    else
      err = launch_kind<BT, JJ, SS, kKindSingle>(p, nullptr, nullptr, n_windows, B, 0, I, s);
  });
  return err;
}

hipError_t launch_gemv_table(const GemvProblem& p, const GemvProblem* table, const int32_t* map,
                             int64_t n_windows, int64_t max_k, int64_t B, bool any_fused, int32_t* I,
                             hipStream_t s, int wf) {
  if (table && (any_fused || I)) return hipErrorInvalidValue;  // grouped launches read Q8 planes
  if (wf != kWeightQ4 && wf != kWeightQ8 && !(table && wf == kWeightMixed)) return hipErrorInvalidValue;
  if (gemv_class_of(max_k, B).J == 0) return hipErrorInvalidValue;
  switch (gemv_bt((int)B)) {
    case 1: return launch_bt<1>(p, table, map, n_windows, max_k, (int)B, any_fused, I, s, wf);
    case 2: return launch_bt<2>(p, table, map, n_windows, max_k, (int)B, any_fused, I, s, wf);
    case 4: return launch_bt<4>(p, table, map, n_windows, max_k, (int)B, any_fused, I, s, wf);
    default: return launch_bt<8>(p, table, map, n_windows, max_k, (int)B, any_fused, I, s, wf);
  }
}

}  // namespace q4q8
