// Expert-routed Q4 x Q8 product (MUL_MAT_ID) for gfx950.
//
// "GGML：Backend 抽象与硬件加速", section "调度器三遍切图，pipeline 四个副本":
// an expert matmul only touches the expert slices that are actually used.
// Here that holds on one device: the routing runs on the GPU (no host sync)
// and one streaming launch covers the row windows of the selected experts
// only: an expert that no token selected is never visited.
//
// Workspace layout (int32): offsets[E + 1] | list[n] | rank[n] | sel[E] |
// ctl[4], n = T * top_k.
//   list holds, grouped by expert, the flat (token, slot) index t * top_k + s
//   of every routed pair; the order inside a group is not fixed, and does not
//   matter because every output element is computed independently.
//   sel lists the selected experts, those with the most pairs first; ctl[0]
//   is the number of work items of the streaming launch, ctl[1] the counter
//   its workgroups take items from.
#include <mutex>

#include "gemv_dev.h"

namespace q4q8 {

constexpr int kRouteThreads = 1024;

constexpr int kMoeChunk = 4;  // windows per work item of the streaming launch (2, 6, 8 measured slower)

size_t moe_workspace_bytes(int64_t E, int64_t T, int64_t top_k) {
  const size_t n = (size_t)(T * top_k);
  const size_t words = (size_t)E + 1 + 2 * n + (size_t)E + 4;
  return (words * sizeof(int32_t) + 15) & ~(size_t)15;
}

// Routing: one workgroup.  Pass 1 reads every id once: a valid pair takes
// its rank within its expert (LDS atomics), an invalid one is written to the
// tail of `list` (valid pairs fill it from the front, so the two never
// meet).  The per-expert counts are scanned in chunks (a thread per chunk,
// a shuffle scan per wave, one thread over the wave totals), the pairs are
// scattered into the
// grouped list, and the rows of invalid pairs are filled with quiet NaNs.
// LDS: counts[E + 1] | wave totals[kRouteThreads / 64].
__global__ __launch_bounds__(kRouteThreads) void moe_route_kernel(
    const int32_t* __restrict__ ids, int n, int E, int M, int chunks, int32_t* __restrict__ offsets,
    int32_t* __restrict__ list, int32_t* __restrict__ rank, int32_t* __restrict__ sel,
    int32_t* __restrict__ ctl, float* __restrict__ y) {
  extern __shared__ int lds[];
  int* cnt = lds;                         // E + 1
  int* chunk = lds + E + 1;               // kRouteThreads / 64
  __shared__ int n_bad;
  const int tid = threadIdx.x;
  for (int e = tid; e <= E; e += kRouteThreads) cnt[e] = 0;
  if (tid == 0) n_bad = 0;
  __syncthreads();
  for (int i = tid; i < n; i += kRouteThreads) {
    const int e = ids[i];
    if (e >= 0 && e < E)
      rank[i] = atomicAdd(&cnt[e], 1);
    else
      list[n - 1 - atomicAdd(&n_bad, 1)] = i;
  }
  __syncthreads();
  // exclusive scan of cnt[0..E) into cnt, total into cnt[E]: chunk sums per
  // thread, an inclusive scan of them within each wave (shuffles), the wave
  // totals scanned by one thread, then each chunk scanned from its offset
  const int per = (E + kRouteThreads - 1) / kRouteThreads;
  const int lo = min(E, tid * per), hi = min(E, lo + per);
  int sum = 0;
  for (int e = lo; e < hi; ++e) sum += cnt[e];
  const int lane = tid & 63, wv = tid >> 6;
  int incl = sum;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int t = __shfl_up(incl, off, 64);
    if (lane >= off) incl += t;
  }
  if (lane == 63) chunk[wv] = incl;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int w = 0; w < kRouteThreads / 64; ++w) {
      const int c = chunk[w];
      chunk[w] = run;
      run += c;
    }
    cnt[E] = run;
  }
  __syncthreads();
  int run = chunk[wv] + incl - sum;
  for (int e = lo; e < hi; ++e) {
    const int c = cnt[e];
    cnt[e] = run;
    run += c;
  }
  __syncthreads();
  for (int e = tid; e <= E; e += kRouteThreads) offsets[e] = cnt[e];
  // Selected experts, heaviest class first (5+ pairs, 3-4, 2, 1): the work
  // items of an expert with many pairs cost the most, so they start first.
  __shared__ int cls_n[4], cls_at[4];
  if (tid < 4) cls_n[tid] = 0;
  __syncthreads();
  for (int e = tid; e < E; e += kRouteThreads) {
    const int c = cnt[e + 1] - cnt[e];
    if (c > 0) atomicAdd(&cls_n[c >= 5 ? 0 : c >= 3 ? 1 : c == 2 ? 2 : 3], 1);
  }
  __syncthreads();
  if (tid == 0) {
    int at = 0;
    for (int k = 0; k < 4; ++k) {
      cls_at[k] = at;
      at += cls_n[k];
    }
    ctl[0] = at * chunks;  // work items
    ctl[1] = 0;            // item counter
  }
  __syncthreads();
  for (int e = tid; e < E; e += kRouteThreads) {
    const int c = cnt[e + 1] - cnt[e];
    if (c > 0) sel[atomicAdd(&cls_at[c >= 5 ? 0 : c >= 3 ? 1 : c == 2 ? 2 : 3], 1)] = e;
  }
  for (int i = tid; i < n; i += kRouteThreads) {
    const int e = ids[i];
    if (e >= 0 && e < E) list[cnt[e] + rank[i]] = i;
  }
  // Pairs with an id outside [0, E) get a row of quiet NaNs.
  const float qnan = __builtin_bit_cast(float, 0x7FC00000u);
  const int nb_bad = n_bad;
  for (int k = 0; k < nb_bad; ++k) {
    const int64_t row = (int64_t)list[n - 1 - k] * M;
    for (int m = tid; m < M; m += kRouteThreads) y[row + m] = qnan;
  }
}

// Rows per window of the routed launch: the largest streaming window over the
// column widths an expert can take (1, 2, 4, 8 routed pairs per pass); every
// width's window divides it (all are powers of two).
static int moe_window_rows(int64_t K) {
  int u = 1;
  for (int bt = 1; bt <= 8; bt *= 2) {
    const int w = gemv_window_rows_bt(K, bt);
    if (w > u) u = w;
  }
  return u;
}

// Work items are (selected expert, chunk of kMoeChunk windows), heaviest
// experts first; each workgroup takes the next item from the counter in the
// workspace (one global atomic per item, requested one item ahead), so an
// expert with many routed pairs does not hold back a fixed share of the
// grid.  Every workgroup leaves once the counter passes the item count.
// Per item the routed pairs are taken up to 8 at a time, each pass with the
// narrowest column width that holds it.
// KMAX: the power-of-two band of K (2048, 4096, 8192 or 16384); within a band
// every column width has one blocking class, so each instance compiles four
// segment variants only.
template <int KMAX>
__global__ __launch_bounds__(kGemvThreads, 1) void moe_stream_kernel(
    const uint8_t* __restrict__ qs, const uint16_t* __restrict__ d, int M, int K,
    const int8_t* __restrict__ xq, const float* __restrict__ xd, int per_slot, int top_k,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ list, const int32_t* __restrict__ sel,
    int32_t* __restrict__ ctl, float* __restrict__ y, int n_win, int chunks, int unit) {
  __shared__ SplitScratch split;
  __shared__ int s_item;
  const int tid = threadIdx.x;
  const int nb = K >> 5;
  const int n_items = ctl[0];
  int parity = 0;
  if (tid == 0) s_item = atomicAdd(&ctl[1], 1);
  __syncthreads();
  int item = s_item;
  while (item < n_items) {
    __syncthreads();  // every wave has read s_item
    if (tid == 0) s_item = atomicAdd(&ctl[1], 1);  // the next item, in flight meanwhile
    const int e = sel[item / chunks];
    const int wl0 = (item % chunks) * kMoeChunk, wl1 = min(n_win, wl0 + kMoeChunk);
    const int beg = offsets[e], cnt = offsets[e + 1] - beg;
    GemvProblem P;
    P.qs = qs + (int64_t)e * M * (K >> 1);
    P.d = d + (int64_t)e * M * nb;
    P.xq = nullptr;
    P.xd = nullptr;
    P.x = nullptr;
    P.g = nullptr;
    P.y = nullptr;
    P.M = M;
    P.K = K;
    P.eps = 0.0f;
    P.mode = kModeQ8;
    P.win_begin = 0;
    P.n_win = n_win;
    for (int c0 = 0; c0 < cnt; c0 += 8) {
      const int nc = min(8, cnt - c0);
      RoutedCols cols;
      cols.xq = xq;
      cols.xd = xd;
      cols.y = y;
      cols.list = list;
      cols.beg = beg + c0;
      cols.K = K;
      cols.nb = nb;
      cols.M = M;
      cols.top_k = top_k;
      cols.per_slot = per_slot;
      auto run = [&]<int BT>() {
        constexpr GemvClass cls = gemv_class_of(KMAX, BT);
        static_assert(cls.J != 0, "unsupported band");
        const int f = unit / GemvShape<BT, cls.J, cls.S>::WIN;
        gemv_segment<BT, cls.J, cls.S, false, false>(P, cols, nc, wl0 * f, wl1 * f, nullptr, &split, parity,
                                                     nullptr);
      };
      if (nc == 1)
        run.template operator()<1>();
      else if (nc == 2)
        run.template operator()<2>();
      else if (nc <= 4)
        run.template operator()<4>();
      else
        run.template operator()<8>();
    }
    __syncthreads();  // s_item holds the next item
    item = s_item;
  }
}

hipError_t launch_moe(const uint8_t* qs, const uint16_t* d, int64_t E, int64_t M, int64_t K,
                      const int8_t* xq, const float* xd, int64_t n_x_slots, const int32_t* ids,
                      int64_t T, int64_t top_k, float* y, void* ws, hipStream_t s) {
  const int n = (int)(T * top_k);
  int32_t* offsets = static_cast<int32_t*>(ws);
  int32_t* list = offsets + E + 1;
  int32_t* rank = list + n;
  int32_t* sel = rank + n;
  int32_t* ctl = sel + E;
  const int unit = moe_window_rows(K);
  const int64_t n_win = (M + unit - 1) / unit;
  const int chunks = (int)((n_win + kMoeChunk - 1) / kMoeChunk);
  const size_t route_lds = ((size_t)E + 1 + kRouteThreads / 64) * sizeof(int);
  hipLaunchKernelGGL(moe_route_kernel, dim3(1), dim3(kRouteThreads), route_lds, s, ids, n, (int)E, (int)M, chunks,
                     offsets, list, rank, sel, ctl, y);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  auto go = [&](auto kernel) {
    static std::mutex mu;
    static int resident = 0;
    {
      std::lock_guard<std::mutex> lk(mu);
      if (resident == 0) {
        int per_cu = 0, cus = 0, dev = 0;
        if (hipGetDevice(&dev) != hipSuccess) dev = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)kernel, kGemvThreads, 0) !=
                hipSuccess || per_cu < 1)
          per_cu = 1;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
          cus = 256;
        resident = per_cu * cus;
      }
    }
    int64_t grid = resident;
    if (grid > E * chunks) grid = E * chunks;
    hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kGemvThreads), 0, s, qs, d, (int)M, (int)K, xq, xd,
                       n_x_slots == 1 ? 0 : 1, (int)top_k, offsets, list, sel, ctl, y, (int)n_win, chunks, unit);
  };
  if (K <= 2048)
    go(moe_stream_kernel<2048>);
  else if (K <= 4096)
    go(moe_stream_kernel<4096>);
  else if (K <= 8192)
    go(moe_stream_kernel<8192>);
  else if (K <= 16384)
    go(moe_stream_kernel<16384>);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace q4q8
