// Expert-routed Q4 x Q8 product (MUL_MAT_ID) for gfx950.
//
// "GGML：Backend 抽象与硬件加速", section "调度器三遍切图，pipeline 四个副本":
// an expert matmul only touches the expert slices that are actually used.
// Here that holds on one device: the routing runs on the GPU (no host sync)
// and one streaming launch covers the row windows of the selected experts
// only: an expert that no token selected is never visited.
//
// Workspace layout (int32): offsets[E + 1] | list[n] | rank[n] | sel[E] |
// costp[E + 1] | ctl[4], n = T * top_k.
//   list holds, grouped by expert, the flat (token, slot) index t * top_k + s
//   of every routed pair; the order inside a group is not fixed, and does not
//   matter because every output element is computed independently.
//   sel lists the selected experts in expert order, costp the prefix of their
//   streaming costs (costp[i] = cost of sel[0..i)); ctl[0] is their number.
#include <mutex>
#include <utility>
#include <vector>

#include "../../include/q4q8.h"
#include "gemv_dev.h"

namespace q4q8 {

constexpr int kRouteThreads = 1024;

size_t moe_workspace_bytes(int64_t E, int64_t T, int64_t top_k) {
  const size_t n = (size_t)(T * top_k);
  const size_t words = (size_t)E + 1 + 2 * n + (size_t)E + (size_t)E + 1 + 4;
  return (words * sizeof(int32_t) + 15) & ~(size_t)15;
}

// Relative cost of streaming one window of an expert with c routed pairs in
// K band `band`: the pairs are taken up to 8 per pass, and a pass of width
// 1 / 2 / 4 / 8 costs (the routed kernel's time per call with every expert of
// a 64-expert layer at that width, less a few microseconds of fixed cost):
//   1536 band (16 lanes per row up to width 4): 16 / 17 / 20 / 43 units
//     (21.8 / 22.5 / 25.8 / 50 us per call, K = 1408, 2048 rows);
//   2048 band: 16 / 16 / 18 / 28 (37.3 / 38.3 / 41.5 / 62.3 us, K = 2048,
//     2816 rows);
//   wider bands: 16 / 16 / 21 / 33 (an earlier calibration of the 2048 band).
// In the 1536 band two passes of width 4 cost less than one of width 8 (40
// against 43 units, and 5 pairs as 4 + 1 cost 36), so its passes take at
// most 4 pairs and the instance holds no width-8 segment.
constexpr int kMoeMaxWindowCost = 43;
__host__ __device__ constexpr int moe_max_pass(int band) { return band == 1536 ? 4 : 8; }
__host__ __device__ inline int moe_window_cost(int c, int band) {
  const int w2 = band == 1536 ? 17 : 16;
  const int w4 = band == 1536 ? 20 : band == 2048 ? 18 : 21;
  const int w8 = band == 1536 ? 43 : band == 2048 ? 28 : 33;
  int cost = 0;
  for (int c0 = 0; c0 < c; c0 += moe_max_pass(band)) {
    const int nc = min(moe_max_pass(band), c - c0);
    cost += nc == 1 ? 16 : nc == 2 ? w2 : nc <= 4 ? w4 : w8;
  }
  return cost;
}

// In-place exclusive scan of v[0..count) by all NT threads, total into
// v[count]: a contiguous chunk per thread, a shuffle scan within each wave,
// one thread over the wave totals (wave_tot: NT / 64 ints).
template <int NT>
__device__ void block_exclusive_scan(int* v, int count, int* wave_tot, int tid) {
  const int per = (count + NT - 1) / NT;
  const int lo = min(count, tid * per), hi = min(count, lo + per);
  int sum = 0;
  for (int e = lo; e < hi; ++e) sum += v[e];
  const int lane = tid & 63, wv = tid >> 6;
  int incl = sum;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int t = __shfl_up(incl, off, 64);
    if (lane >= off) incl += t;
  }
  if (lane == 63) wave_tot[wv] = incl;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int w = 0; w < NT / 64; ++w) {
      const int c = wave_tot[w];
      wave_tot[w] = run;
      run += c;
    }
    v[count] = run;
  }
  __syncthreads();
  int run = wave_tot[wv] + incl - sum;
  for (int e = lo; e < hi; ++e) {
    const int c = v[e];
    v[e] = run;
    run += c;
  }
  __syncthreads();
}

// Routing by one workgroup of NT threads.  Pass 1 reads every id once: a
// valid pair takes its rank within its expert (LDS atomics), an invalid one
// is written to the tail of `list` (valid pairs fill it from the front, so
// the two never meet).  Block scans give the per-expert offsets, the selected
// experts' indices and the prefix of their streaming costs; the pairs are
// scattered into the grouped list, and (when nan_rows) the rows of invalid
// pairs are filled with quiet NaNs.  cnt, sidx, cpre: E + 1 ints of LDS each,
// wave_tot NT / 64, n_bad one; the outputs (offsets .. ctl, the workspace
// layout above) may live in LDS or global memory.
template <int NT>
__device__ __forceinline__ void moe_route(const int32_t* __restrict__ ids, int n, int E, int n_win, int band, int* cnt,
                                          int* sidx, int* cpre, int* wave_tot, int* n_bad, int32_t* offsets,
                                          int32_t* list, int32_t* rank, int32_t* sel, int32_t* costp,
                                          int32_t* ctl, bool nan_rows, int M, float* __restrict__ y) {
  const int tid = threadIdx.x;
  for (int e = tid; e <= E; e += NT) cnt[e] = 0;
  if (tid == 0) *n_bad = 0;
  __syncthreads();
  for (int i = tid; i < n; i += NT) {
    const int e = ids[i];
    if (e >= 0 && e < E)
      rank[i] = atomicAdd(&cnt[e], 1);
    else
      list[n - 1 - atomicAdd(n_bad, 1)] = i;
  }
  __syncthreads();
  if (E <= kWave) {
    // Up to one expert per lane: wave 0 takes the three prefix sums with
    // shuffles (no block scans and their barriers).
    if (tid < kWave) {
      const int e = tid;
      const int c = e < E ? cnt[e] : 0;
      const int si = c > 0 ? 1 : 0;
      const int cp = c > 0 ? n_win * moe_window_cost(c, band) : 0;
      int ic = c, is = si, ip = cp;
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const int tc = __shfl_up(ic, off, kWave), ts = __shfl_up(is, off, kWave), tq = __shfl_up(ip, off, kWave);
        if (e >= off) {
          ic += tc;
          is += ts;
          ip += tq;
        }
      }
      const int tot_c = __shfl(ic, kWave - 1, kWave), tot_s = __shfl(is, kWave - 1, kWave);
      const int tot_p = __shfl(ip, kWave - 1, kWave);
      if (e < E) {
        cnt[e] = ic - c;
        offsets[e] = ic - c;
        if (c > 0) {
          sel[is - si] = e;
          costp[is - si] = ip - cp;
        }
      }
      if (e == 0) {
        cnt[E] = tot_c;
        offsets[E] = tot_c;
        costp[tot_s] = tot_p;
        ctl[0] = tot_s;
      }
    }
    __syncthreads();
  } else {
    for (int e = tid; e < E; e += NT) {
      const int c = cnt[e];
      sidx[e] = c > 0 ? 1 : 0;
      cpre[e] = c > 0 ? n_win * moe_window_cost(c, band) : 0;
    }
    __syncthreads();
    block_exclusive_scan<NT>(cnt, E, wave_tot, tid);
    block_exclusive_scan<NT>(sidx, E, wave_tot, tid);
    block_exclusive_scan<NT>(cpre, E, wave_tot, tid);
    for (int e = tid; e <= E; e += NT) offsets[e] = cnt[e];
    // Selected experts in expert order with the prefix of their costs.
    for (int e = tid; e < E; e += NT) {
      if (cnt[e + 1] > cnt[e]) {
        sel[sidx[e]] = e;
        costp[sidx[e]] = cpre[e];
      }
    }
    if (tid == 0) {
      costp[sidx[E]] = cpre[E];
      ctl[0] = sidx[E];
    }
  }
  for (int i = tid; i < n; i += NT) {
    const int e = ids[i];
    if (e >= 0 && e < E) list[cnt[e] + rank[i]] = i;
  }
  if (nan_rows) {
    // Pairs with an id outside [0, E) get a row of quiet NaNs.
    const float qnan = __builtin_bit_cast(float, 0x7FC00000u);
    const int nb_bad = *n_bad;
    for (int k = 0; k < nb_bad; ++k) {
      const int64_t row = (int64_t)list[n - 1 - k] * M;
      for (int m = tid; m < M; m += NT) y[row + m] = qnan;
    }
  }
}

// The routing as its own launch (one workgroup), results in the workspace.
// LDS: counts, selected indices, cost prefix (E + 1 each) | wave totals.
__global__ __launch_bounds__(kRouteThreads) void moe_route_kernel(
    const int32_t* __restrict__ ids, int n, int E, int n_win, int band, int32_t* __restrict__ offsets,
    int32_t* __restrict__ list, int32_t* __restrict__ rank, int32_t* __restrict__ sel,
    int32_t* __restrict__ costp, int32_t* __restrict__ ctl, int M, float* __restrict__ y) {
  extern __shared__ int lds[];
  __shared__ int n_bad;
  moe_route<kRouteThreads>(ids, n, E, n_win, band, lds, lds + E + 1, lds + 2 * (E + 1), lds + 3 * (E + 1), &n_bad,
                           offsets, list, rank, sel, costp, ctl, true, M, y);
}

// Small routings (few experts and pairs) run inside every workgroup of the
// streaming launch instead, in LDS: one launch per call instead of two.
// LDS ints: cnt, sidx, cpre, offsets, costp (E + 1 each), sel (E), list,
// rank (n each), wave totals (kGemvThreads / 64), n_bad, ctl.
constexpr int kFusedRouteMaxInts = 4096;
__host__ __device__ constexpr int64_t moe_fused_route_ints(int64_t E, int64_t n) {
  return 5 * (E + 1) + E + 2 * n + kGemvThreads / 64 + 2;
}

// Blocking of a column width BT in a K band: J blocks per lane, K split over
// S waves, LPR lanes per row (GemvShape).  Rows of up to 48 blocks (the 1536
// band, e.g. K = 1408: 44 blocks) take 16 lanes per row and 3 blocks per lane
// for up to four columns, so a load instruction covers four rows and 44 of
// its 48 block slots carry data, where a row per instruction keeps 20 of 64
// lanes idle; eight columns would need 3 x 8 activation blocks per lane and
// keep a row per instruction.
struct MoeClass {
  int J, S, LPR;
};
__host__ __device__ constexpr MoeClass moe_class(int band, int BT) {
  if (band == 1536 && BT <= 4) return {3, 1, 16};
  const GemvClass c = gemv_class_of(band == 1536 ? 2048 : band, BT);
  return {c.J, c.S, kWave};
}

// 16-byte weight loads each lane keeps in flight per row group, per column
// width (1, 2, 4, 8 routed pairs per pass) and K band.  The 1536 band keeps
// two row slots (8 rows, 6 loads per lane) at one and two columns and two
// (12 loads) at four: 32-row windows like the 2048 band's.  One kernel instance
// holds the segments of all four widths, so its register allocation is the
// largest of theirs.  The 2048 band takes 8 / 8 / 16 / 8, which fits two
// workgroups per CU (245 VGPRs) and measured fastest: 4.1 TB/s for the MoE
// step against 3.6 with 16 at width 8 and one workgroup per CU, 3.0 with 8 at
// width 4 (one per CU) and 3.3 with 4 at width 8.  The larger bands take
// 8 / 8 / 16 / 16 at one workgroup per CU, and the 16384 band keeps width 4
// at 8 so that its instance stays free of scratch spills.
__host__ __device__ constexpr int moe_rif(int BT, int band) {
  if (band == 1536) return moe_class(band, BT).LPR != kWave ? (BT <= 2 ? 6 : 12) : moe_rif(BT, 2048);
  if (band <= 2048) return BT <= 2 ? 8 : BT <= 4 ? 16 : 8;
  return BT <= 2 ? 8 : BT <= 4 ? (band >= 16384 ? 8 : 16) : 16;
}

// Workgroups per CU the streaming instance of a K band is built for.  The
// 2048 band's per-wave instance needs 150 VGPRs, so three fit (steadier and
// about 1% faster on the MoE step than two, six interleaved runs each).
__host__ __device__ constexpr int moe_waves_per_simd(int band) { return band == 2048 ? 3 : band < 2048 ? 2 : 1; }

// The band of K whose blocking classes an instance compiles: 1536, 2048,
// 4096, 8192 or 16384 (0: K too large).  Within a band every column width
// has one class.
static int moe_band(int64_t K) {
  return K <= 1536 ? 1536 : K <= 2048 ? 2048 : K <= 4096 ? 4096 : K <= 8192 ? 8192 : K <= 16384 ? 16384 : 0;
}

// Bands whose every width keeps K in one wave (S = 1) schedule per wave:
// each wave of a workgroup takes its own share of the cost, in windows of
// its own rows (a quarter of a workgroup window), so the shares end within a
// small window of their target.
template <int BAND>
constexpr bool moe_per_wave() {
  return moe_class(BAND, 1).S == 1 && moe_class(BAND, 2).S == 1 && moe_class(BAND, 4).S == 1 &&
         moe_class(BAND, 8).S == 1;
}

template <int BAND, int BT>
constexpr int moe_win() {
  constexpr MoeClass c = moe_class(BAND, BT);
  using Sh = GemvShape<BT, c.J, c.S, moe_rif(BT, BAND), c.LPR>;
  return moe_per_wave<BAND>() ? Sh::RU * Sh::RPI : Sh::WIN;
}

// Rows per window of the routed launch: the largest streaming window over the
// column widths; every width's window divides it (all are powers of two).
template <int BAND>
constexpr int moe_window_rows_c() {
  constexpr int w1 = moe_win<BAND, 1>(), w2 = moe_win<BAND, 2>(), w4 = moe_win<BAND, 4>(), w8 = moe_win<BAND, 8>();
  constexpr int u = w1 > w2 ? w1 : w2, v = w4 > w8 ? w4 : w8;
  constexpr int m = u > v ? u : v;
  static_assert(m % w1 == 0 && m % w2 == 0 && m % w4 == 0 && m % w8 == 0, "windows must divide the unit");
  return m;
}
static int moe_window_rows(int64_t K) {
  switch (moe_band(K)) {
    case 1536: return moe_window_rows_c<1536>();
    case 2048: return moe_window_rows_c<2048>();
    case 4096: return moe_window_rows_c<4096>();
    case 8192: return moe_window_rows_c<8192>();
    case 16384: return moe_window_rows_c<16384>();
    default: return 1;
  }
}

// Static cost-balanced schedule: window j of selected expert i starts at
// cost costp[i] + j * cost_i (cost_i = moe_window_cost of its pair count),
// and workgroup g streams the windows whose start lies in its equal share
// [C g / G, C (g + 1) / G) of the total cost C -- a contiguous run across
// experts, so each workgroup keeps its windows in flight from one to the
// next, and an expert with many routed pairs gets proportionally fewer
// windows per workgroup.  Per expert the routed pairs are taken up to 8 at a
// time, each pass with the narrowest column width that holds it.
// KMAX: the band of K (moe_band), so each instance compiles four segment
// variants only.
// FUSED: the workgroup first routes the ids itself (moe_route in LDS;
// workgroup 0 also fills the NaN rows), else the routing comes from the
// workspace written by moe_route_kernel.
template <int KMAX, bool FUSED>
__global__ __launch_bounds__(kGemvThreads, moe_waves_per_simd(KMAX)) void moe_stream_kernel(
    const uint8_t* __restrict__ qs, const uint16_t* __restrict__ d, int M, int K,
    const int8_t* __restrict__ xq, const float* __restrict__ xd, int per_slot, int top_k,
    const int32_t* __restrict__ g_offsets, const int32_t* __restrict__ g_list, const int32_t* __restrict__ g_sel,
    const int32_t* __restrict__ g_costp, const int32_t* __restrict__ g_ctl, float* __restrict__ y, int n_win,
    int unit, const int32_t* __restrict__ ids, int n, int E) {
  __shared__ SplitScratch split;
  extern __shared__ int rl[];
  const int32_t* offsets = g_offsets;
  const int32_t* list = g_list;
  const int32_t* sel = g_sel;
  const int32_t* costp = g_costp;
  const int32_t* ctl = g_ctl;
  if constexpr (FUSED) {
    int* cnt = rl;
    int* sidx = cnt + E + 1;
    int* cpre = sidx + E + 1;
    int* l_off = cpre + E + 1;
    int* l_costp = l_off + E + 1;
    int* l_sel = l_costp + E + 1;
    int* l_list = l_sel + E;
    int* l_rank = l_list + n;
    int* wave_tot = l_rank + n;
    int* n_bad = wave_tot + kGemvThreads / 64;
    int* l_ctl = n_bad + 1;
    moe_route<kGemvThreads>(ids, n, E, n_win, KMAX, cnt, sidx, cpre, wave_tot, n_bad, l_off, l_list, l_rank, l_sel,
                            l_costp, l_ctl, blockIdx.x == 0, M, y);
    __syncthreads();
    offsets = l_off;
    list = l_list;
    sel = l_sel;
    costp = l_costp;
    ctl = l_ctl;
  }
  const int lane = threadIdx.x & 63;
  const int nb = K >> 5;
  const int n_sel = ctl[0];
  if (n_sel == 0) return;
  const int64_t C = costp[n_sel];
  // per-wave shares (moe_per_wave): wave w of workgroup b takes share 4 b + w
  constexpr bool PW = moe_per_wave<KMAX>();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
  const int64_t G = (int64_t)gridDim.x * (PW ? kGemvWaves : 1), g = PW ? (int64_t)blockIdx.x * kGemvWaves + wave
                                                                         : (int64_t)blockIdx.x;
  const int64_t c_lo = C * g / G, c_hi = C * (g + 1) / G;
  // first selected expert whose cost range reaches past c_lo (wave-wide ballot)
  int i = -1;
  for (int base = 0; base < n_sel && i < 0; base += 64) {
    const int k = base + lane;
    const bool hit = k < n_sel && costp[k + 1] > c_lo;
    const uint64_t mask = __ballot(hit);
    if (mask) i = base + __builtin_ctzll(mask);
  }
  int parity = 0;
  for (; i >= 0 && i < n_sel && costp[i] < c_hi; ++i) {
    const int e = sel[i];
    const int beg = offsets[e], cnt = offsets[e + 1] - beg;
    const int64_t wc = moe_window_cost(cnt, KMAX);
    // windows of this expert whose start cost lies in [c_lo, c_hi)
    const int64_t r_lo = c_lo - costp[i], r_hi = c_hi - costp[i];
    const int wl0 = r_lo <= 0 ? 0 : (int)((r_lo + wc - 1) / wc);
    const int wl1 = (int)min((int64_t)n_win, (r_hi + wc - 1) / wc);
    if (wl0 >= wl1) continue;
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
    for (int c0 = 0; c0 < cnt; c0 += moe_max_pass(KMAX)) {
      const int nc = min(moe_max_pass(KMAX), cnt - c0);
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
        constexpr MoeClass cls = moe_class(KMAX, BT);
        static_assert(cls.J != 0, "unsupported band");
        constexpr int RIF = moe_rif(BT, KMAX);
        const int f = unit / moe_win<KMAX, BT>();
        gemv_segment<BT, cls.J, cls.S, false, false, RoutedCols, RIF, kWeightQ4, cls.LPR, PW>(
            P, cols, nc, wl0 * f, wl1 * f, nullptr, &split, parity, nullptr);
      };
      if (nc == 1)
        run.template operator()<1>();
      else if (nc == 2)
        run.template operator()<2>();
      else if (KMAX == 1536 || nc <= 4)
        run.template operator()<4>();
      else
        run.template operator()<8>();
    }
  }
}

// Workgroups of a streaming instance resident at once (per CU times CUs),
// queried once per instance and device with the largest fused-routing LDS.
static int64_t moe_resident_workgroups(const void* kernel) {
  static std::mutex mu;
  static std::vector<std::pair<std::pair<const void*, int>, int64_t>> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  std::lock_guard<std::mutex> lk(mu);
  for (const auto& e : cache)
    if (e.first.first == kernel && e.first.second == dev) return e.second;
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kGemvThreads,
                                                   (size_t)kFusedRouteMaxInts * sizeof(int)) != hipSuccess ||
      per_cu < 1)
    per_cu = 1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 256;
  const int64_t n = (int64_t)per_cu * cus;
  cache.push_back({{kernel, dev}, n});
  return n;
}

// Built-in scratch of the allocation-free routed entry point: the routing
// workspace (offsets, list, rank, selected experts, cost prefix, control
// words) of a call that cannot bring one.  Every valid call fits (E <= 4096
// and T * top_k <= 65536 need at most 573,464 bytes).  Each GPU holds its own
// copy until the process ends; in host code `scratch` is only a host-side
// stand-in, so kernels get the device address that hipGetSymbolAddress
// returns for the current device, looked up once per device.
constexpr size_t kMoeScratchBytes = Q4Q8_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kMoeScratchBytes];

size_t moe_scratch_bytes() { return kMoeScratchBytes; }

hipError_t moe_scratch(void** out) {
  constexpr int kMaxDev = 64;
  static std::mutex mu;
  static void* ptr[kMaxDev] = {};
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDev) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(mu);
  if (!ptr[dev]) {
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return err;
    if (!p) return hipErrorInvalidSymbol;
    ptr[dev] = p;
  }
  *out = ptr[dev];
  return hipSuccess;
}

int64_t moe_schedule_cost_bound(int64_t E, int64_t M, int64_t K, int64_t n) {
  const int unit = moe_window_rows(K);
  const int64_t n_win = (M + unit - 1) / unit;
  return n_win * kMoeMaxWindowCost * ((n + 7) / 8 + E);
}

hipError_t launch_moe(const uint8_t* qs, const uint16_t* d, int64_t E, int64_t M, int64_t K,
                      const int8_t* xq, const float* xd, int64_t n_x_slots, const int32_t* ids,
                      int64_t T, int64_t top_k, float* y, void* ws, hipStream_t s) {
  const int n = (int)(T * top_k);
  int32_t* offsets = static_cast<int32_t*>(ws);
  int32_t* list = offsets + E + 1;
  int32_t* rank = list + n;
  int32_t* sel = rank + n;
  int32_t* costp = sel + E;
  int32_t* ctl = costp + E + 1;
  const int unit = moe_window_rows(K);
  const int64_t n_win = (M + unit - 1) / unit;
  // (the widest band keeps the separate routing launch: its instance has no
  // registers to spare for the fused routing)
  const bool fused = moe_fused_route_ints(E, n) <= kFusedRouteMaxInts && moe_band(K) <= 8192;
  const size_t fused_lds = fused ? (size_t)moe_fused_route_ints(E, n) * sizeof(int) : 0;
  if (!fused) {
    const size_t route_lds = (3 * ((size_t)E + 1) + kRouteThreads / 64) * sizeof(int);
    note_launch((const void*)moe_route_kernel);
    hipLaunchKernelGGL(moe_route_kernel, dim3(1), dim3(kRouteThreads), route_lds, s, ids, n, (int)E, (int)n_win,
                       moe_band(K), offsets, list, rank, sel, costp, ctl, (int)M, y);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  auto go = [&](auto kernel) {
    int64_t grid = moe_resident_workgroups((const void*)kernel);
    if (grid > E * n_win) grid = E * n_win;
    note_launch((const void*)kernel);
    hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kGemvThreads), fused_lds, s, qs, d, (int)M, (int)K, xq,
                       xd, n_x_slots == 1 ? 0 : 1, (int)top_k, offsets, list, sel, costp, ctl, y, (int)n_win, unit,
                       ids, n, (int)E);
  };
  auto band = [&](auto k_fused, auto k_ws) {
    if (fused)
      go(k_fused);
    else
      go(k_ws);
  };
  switch (moe_band(K)) {
    case 1536: band(moe_stream_kernel<1536, true>, moe_stream_kernel<1536, false>); break;
    case 2048: band(moe_stream_kernel<2048, true>, moe_stream_kernel<2048, false>); break;
    case 4096: band(moe_stream_kernel<4096, true>, moe_stream_kernel<4096, false>); break;
    case 8192: band(moe_stream_kernel<8192, true>, moe_stream_kernel<8192, false>); break;
    case 16384: go(moe_stream_kernel<16384, false>); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Expert-plane sum after MUL_MAT_ID ("llama.cpp b10981发布：OpenVINO后端优化
// 有状态解码与GPU MoE推理": the planes are added by a chain of ADD ops, and a
// reordered reduction drifts in f32).  out[t][m] is the in-order chain over
// the slots of fl(w[t][s] * y[t][s][m]), one rounding per product and per sum
// and no contraction, so it equals that chain bit for bit.  Thread per
// element; a workgroup covers 256 consecutive m of one token, so the weights
// of the token are uniform and the plane reads are coalesced.
constexpr int kSumThreads = 256;

__global__ __launch_bounds__(kSumThreads) void moe_expert_sum_kernel(const float* __restrict__ y,
                                                                    const float* __restrict__ w, int top_k,
                                                                    int64_t M, float* __restrict__ out) {
  const int64_t t = blockIdx.y;
  const int64_t m = (int64_t)blockIdx.x * kSumThreads + threadIdx.x;
  if (m >= M) return;
  const float* yp = y + t * top_k * M + m;
  float acc = 0.0f;
  for (int s = 0; s < top_k; ++s) {
    const float yv = gptr(yp)[(int64_t)s * M];
    const float v = w ? __fmul_rn(gptr(w)[t * top_k + s], yv) : yv;
    acc = s == 0 ? v : __fadd_rn(acc, v);
  }
  gptr_w(out)[t * M + m] = acc;
}

hipError_t launch_moe_expert_sum(const float* y, const float* w, int64_t T, int64_t top_k, int64_t M, float* out,
                                 hipStream_t s) {
  const dim3 grid((unsigned)((M + kSumThreads - 1) / kSumThreads), (unsigned)T);
  note_launch((const void*)moe_expert_sum_kernel);
  hipLaunchKernelGGL(moe_expert_sum_kernel, grid, dim3(kSumThreads), 0, s, y, w, (int)top_k, M, out);
  return hipGetLastError();
}

}  // namespace q4q8
