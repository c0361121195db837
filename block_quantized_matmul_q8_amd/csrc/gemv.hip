// Streaming Q4 x Q8 matrix x vector kernel for gfx950 (the decode route; the
// mmvq role in "GGML：Backend 抽象与硬件加速", section "CUDA：mmvq、mmq、cublas
// 三条矩阵路": batch-1 decode is a quantised matrix x vector product, and a
// dedicated vector kernel is cheaper to launch than the matrix path).
//
// One persistent kernel serves a single product and a grouped launch over
// many products (a device table of GemvProblem records plus a window ->
// record map).  Per product segment of a workgroup:
//   - the weight loads of each wave's first row group are issued first, so
//     they are in flight while the activations are prepared;
//   - activations come either as Q8 planes (loaded straight into registers)
//     or as fp32 x + norm weight g, in which case the workgroup runs the
//     RMSNorm * g -> Q8 prologue itself (prologue_dev.h, bit-identical to the
//     standalone prologue) and stages the codes through LDS;
//   - lane l holds the activation codes of blocks l, l + 64, ... in
//     registers for the whole tile; each row is streamed with one 16-byte
//     load per lane per 64 blocks (a whole 32-block, 1 KiB per wave load,
//     fully coalesced), nibbles unpacked in registers, v_dot4_i32_i8 on the
//     unsigned codes with the offset removed through the code sums
//     (I = sum q x - 8 sum x, exact), fp32 fma for the block scale;
//   - RU rows are in flight per wave (the next group is loaded while the
//     current one is computed) and finished with one multi-row butterfly.
#include <mutex>
#include <utility>
#include <vector>

#include "prologue_dev.h"

namespace q4q8 {

constexpr int kGemvThreads = 256;
constexpr size_t kGemvMaxLds = 64 * 1024;

// Butterfly sum of N values per lane over the 64 lanes.  Lane L returns the
// total of value index L >> (6 - log2 N); each exchange step halves the
// number of values a lane carries, so the cost is N - 1 + 6 - log2 N
// shuffles instead of 6 N.
template <int N>
__device__ __forceinline__ float multi_reduce(float (&v)[N], int lane) {
#pragma unroll
  for (int s = N / 2, off = 32; s >= 1; s /= 2, off /= 2) {
    const bool upper = (lane & off) != 0;
#pragma unroll
    for (int i = 0; i < s; ++i) {
      // The empty asm pins both values in registers: otherwise the compiler
      // folds the lane-dependent choice into a load from a selected address,
      // which moves the array to scratch memory.
      float a = v[i], b = v[i + s];
      __asm__("" : "+v"(a), "+v"(b));
      const float send = upper ? a : b;
      const float keep = upper ? b : a;
      v[i] = keep + __shfl_xor(send, off, kWave);
    }
  }
  float r = v[0];
#pragma unroll
  for (int off = 32 / N; off >= 1; off /= 2) r += __shfl_xor(r, off, kWave);
  return r;
}

constexpr int ilog2_c(int n) { return n <= 1 ? 0 : 1 + ilog2_c(n / 2); }
constexpr int pow2_ceil_c(int n) { return n <= 1 ? 1 : 2 * pow2_ceil_c((n + 1) / 2); }

__device__ __forceinline__ int code_sum8(const i32x4 a, const i32x4 b) {
  int s = 0;
  s = __builtin_amdgcn_sdot4(a.x, 0x01010101, s, false);
  s = __builtin_amdgcn_sdot4(a.y, 0x01010101, s, false);
  s = __builtin_amdgcn_sdot4(a.z, 0x01010101, s, false);
  s = __builtin_amdgcn_sdot4(a.w, 0x01010101, s, false);
  s = __builtin_amdgcn_sdot4(b.x, 0x01010101, s, false);
  s = __builtin_amdgcn_sdot4(b.y, 0x01010101, s, false);
  s = __builtin_amdgcn_sdot4(b.z, 0x01010101, s, false);
  s = __builtin_amdgcn_sdot4(b.w, 0x01010101, s, false);
  return 8 * s;
}

#ifndef Q4Q8_GEMV_ROWS_IN_FLIGHT
#define Q4Q8_GEMV_ROWS_IN_FLIGHT 16  // 16-byte loads per lane in flight per row group
#endif

// Rows a wave keeps in flight per group for B columns and J blocks per lane.
__host__ __device__ constexpr int gemv_rows_per_wave(int B, int J) {
  return B <= 2 ? (Q4Q8_GEMV_ROWS_IN_FLIGHT / J > 0 ? Q4Q8_GEMV_ROWS_IN_FLIGHT / J : 1)
                : (Q4Q8_GEMV_ROWS_IN_FLIGHT / J / 2 > 0 ? Q4Q8_GEMV_ROWS_IN_FLIGHT / J / 2 : 1);
}

template <int B, int J>
struct GemvShape {
  static constexpr int RU = gemv_rows_per_wave(B, J);
  static constexpr int WIN = 4 * RU;  // rows per window (one row group per wave)
  static constexpr int NV = RU * B;   // values reduced per row group
  static constexpr int NP = pow2_ceil_c(NV);
  static constexpr int SHIFT = 6 - ilog2_c(NP);
};

__host__ __device__ __forceinline__ int blocks_per_lane_of(int K) {
  const int j = (K / kQK + kWave - 1) / kWave;
  return j <= 1 ? 1 : j <= 2 ? 2 : j <= 4 ? 4 : j <= 8 ? 8 : 16;
}

// Streams windows [wl0, wl1) of product P (window i = rows i*WIN .. +WIN;
// wave w takes the RU rows at w*RU of each window) with J blocks per lane.
template <int B, int J, bool FOLD, bool WRITE_I>
__device__ __forceinline__ void gemv_segment(const GemvProblem& P, int wl0, int wl1,
                                             unsigned char* smem, int32_t* __restrict__ Iout) {
  using S = GemvShape<B, J>;
  constexpr int RU = S::RU, WIN = S::WIN, NV = S::NV, NP = S::NP, SHIFT = S::SHIFT;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int M = P.M, K = P.K, nb = K >> 5;
  const int64_t row_bytes = K >> 1;

  // Loads are unconditional, from addresses clamped into the segment's rows
  // (so an overrun re-reads a row just loaded, from cache, and never touches
  // rows another workgroup streams) and the block range: a guarded or masked
  // load becomes a branch that waits for its own data, which would serialise
  // the rows a wave keeps in flight.  Nothing needs masking: blocks past nb
  // meet zeroed activation registers (their product is exactly 0) and rows
  // past the segment are never stored.  Scales stay raw fp16 bits until used,
  // so no conversion waits on a prefetch.  Weights and scales are read once:
  // non-temporal loads keep them from displacing reusable lines.
  const int row_last = min(M, wl1 * WIN) - 1;
  auto load_group = [&](int row0, u32x4 (&w)[RU][J], uint32_t (&dw)[RU][J]) {
#pragma unroll
    for (int r = 0; r < RU; ++r) {
      const int rowc = min(row0 + r, row_last);
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int bc = min(lane + kWave * j, nb - 1);
        w[r][j] = __builtin_nontemporal_load(
            &gptr(reinterpret_cast<const u32x4*>(P.qs))[rowc * (row_bytes / 16) + bc]);
        dw[r][j] = __builtin_nontemporal_load(&gptr(P.d)[(int64_t)rowc * nb + bc]);
      }
    }
  };

  u32x4 wA[RU][J], wB[RU][J];
  uint32_t dA[RU][J], dB[RU][J];
  i32x4 xa[B][J], xb[B][J];
  float xdr[B][J];
  int xsr[B][J];
  if constexpr (!FOLD) {
    // Q8 planes: the activation loads go first (they are small and mostly
    // L2-resident), then the first two windows; loads complete in issue
    // order, so the first compute waits for the activations and window A
    // only while window B is already in flight.
#pragma unroll
    for (int c = 0; c < B; ++c)
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int b = lane + kWave * j;
        const int bc = min(b, nb - 1);
        const Q4Q8_GLOBAL i32x4* src =
            gptr(reinterpret_cast<const i32x4*>(P.xq + (int64_t)c * K + (int64_t)bc * kQK));
        xa[c][j] = src[0];
        xb[c][j] = src[1];
        xdr[c][j] = gptr(P.xd)[(int64_t)c * nb + bc];
      }
    load_group(wl0 * WIN + wave * RU, wA, dA);
    load_group((wl0 + 1) * WIN + wave * RU, wB, dB);
#pragma unroll
    for (int c = 0; c < B; ++c)
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const bool valid = lane + kWave * j < nb;
        const i32x4 zero = {0, 0, 0, 0};
        xa[c][j] = valid ? xa[c][j] : zero;
        xb[c][j] = valid ? xb[c][j] : zero;
        xdr[c][j] = valid ? xdr[c][j] : 0.0f;
        xsr[c][j] = code_sum8(xa[c][j], xb[c][j]);
      }
  } else {
    // Folded-in prologue: window A is requested first, then the whole
    // workgroup quantises the activation rows (prologue_dev.h, the
    // register/butterfly form of the same steps) and stages the codes
    // through LDS; window B follows.
    load_group(wl0 * WIN + wave * RU, wA, dA);
    int8_t* sx = reinterpret_cast<int8_t*>(smem);                  // [B][K]
    float* sxd = reinterpret_cast<float*>(smem + (size_t)B * K);   // [B][nb]
    int* sxs = reinterpret_cast<int*>(sxd + B * nb);               // [B][nb]
    float* groups = reinterpret_cast<float*>(sxs + B * nb);        // [8]
    const bool raw = P.mode == kModeRaw;
    for (int c = 0; c < B; ++c)
      wg_q8_row_fast(P.x + (int64_t)c * K, P.g, K, P.eps, raw, sx + (size_t)c * K, sxd + c * nb,
                     sxs + c * nb, groups, tid);
#pragma unroll
    for (int c = 0; c < B; ++c)
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int b = lane + kWave * j;
        if (b < nb) {
          const i32x4* src = reinterpret_cast<const i32x4*>(sx + (size_t)c * K + (size_t)b * kQK);
          xa[c][j] = src[0];
          xb[c][j] = src[1];
          xdr[c][j] = sxd[c * nb + b];
          xsr[c][j] = 8 * sxs[c * nb + b];
        } else {
          xa[c][j] = i32x4{0, 0, 0, 0};
          xb[c][j] = i32x4{0, 0, 0, 0};
          xdr[c][j] = 0.0f;
          xsr[c][j] = 0;
        }
      }
    load_group((wl0 + 1) * WIN + wave * RU, wB, dB);
  }

  // One row group: block sums, scale, multi-row reduction, store.
  auto compute_group = [&](int row0, const u32x4 (&w)[RU][J], const uint32_t (&dw)[RU][J]) {
    float acc[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i) acc[i] = 0.0f;
#pragma unroll
    for (int j = 0; j < J; ++j)
#pragma unroll
      for (int r = 0; r < RU; ++r) {
        const float dwf = f16_bits_to_f32((uint16_t)dw[r][j]);
#pragma unroll
        for (int c = 0; c < B; ++c) {
          const int I = dot_block(w[r][j], xa[c][j], xb[c][j]) - xsr[c][j];
          acc[r * B + c] = __builtin_fmaf((float)I, dwf * xdr[c][j], acc[r * B + c]);
          if (WRITE_I) {
            const int b = lane + kWave * j;
            const int row = row0 + r;
            if (b < nb && row <= row_last) Iout[((int64_t)c * M + row) * nb + b] = I;
          }
        }
      }
    const float v = multi_reduce<NP>(acc, lane);
    const int k = lane >> SHIFT;
    if ((lane & ((1 << SHIFT) - 1)) == 0 && k < NV) {
      const int row = row0 + k / B;
      if (row <= row_last) gptr_w(P.y)[(int64_t)(k % B) * M + row] = v;
    }
  };

  // Ping-pong over two register buffers: while one window is computed the
  // other is in flight; a buffer is refilled right after it is consumed.
  for (int wi = wl0; wi < wl1; wi += 2) {
    const int r0 = wi * WIN + wave * RU;
    compute_group(r0, wA, dA);
    load_group(r0 + 2 * WIN, wA, dA);
    if (wi + 1 >= wl1) break;
    compute_group(r0 + WIN, wB, dB);
    load_group(r0 + 3 * WIN, wB, dB);
  }
}

// Persistent grid: workgroup g streams the g-th equal share of the window
// list (the windows of all products, product after product), so every
// workgroup carries the same load from start to end and the launch has no
// rounds of short-lived workgroups.  A share spans few products; the next
// product's record is requested when a segment starts, so it is at hand when
// the segment ends.  The grouped instance serves products of every blocking
// class up to JMAX (the workgroup dispatches uniformly on each product's own
// J) and reads Q8 planes only; single-product instances compile their own
// class only.  The grouped and single-product forms are separate instances
// because selecting between the kernel argument and the table at run time
// would make every access a generic flat access.
#ifndef Q4Q8_GEMV_MIN_WG_PER_CU
#define Q4Q8_GEMV_MIN_WG_PER_CU 1
#endif

enum GemvKind : int {
  kKindGroup = 0,      // table of products, Q8 planes
  kKindSingle = 1,     // one product, Q8 planes
  kKindFold = 2,       // one product, fp32 rows, prologue folded in
  kKindBlockSums = 3,  // one product, Q8 planes, per-block sums written out
};

template <int B, int JMAX, int KIND>
__global__ __launch_bounds__(kGemvThreads, Q4Q8_GEMV_MIN_WG_PER_CU) void gemv_kernel(GemvProblem p0,
                                                            const GemvProblem* __restrict__ table,
                                                            const int32_t* __restrict__ win_map,
                                                            int n_windows,
                                                            int32_t* __restrict__ Iout) {
  constexpr bool GROUPED = KIND == kKindGroup;
  constexpr bool FOLD = KIND == kKindFold;
  constexpr bool WRITE_I = KIND == kKindBlockSums;
  extern __shared__ __align__(16) unsigned char smem[];
  const int64_t G = gridDim.x, g = blockIdx.x;
  const int w_begin = (int)(n_windows * g / G);
  const int w_end = (int)(n_windows * (g + 1) / G);
  if constexpr (GROUPED) {
    int rec = win_map[w_begin];
    const int rec_last = win_map[w_end - 1];
    GemvProblem P = table[rec];
    for (int w = w_begin; w < w_end;) {
      const int seg_end = min(w_end, P.win_begin + P.n_win);
      const GemvProblem Pn = table[min(rec + 1, rec_last)];
      const int wl0 = w - P.win_begin, wl1 = seg_end - P.win_begin;
      const int J = blocks_per_lane_of(P.K);
      if constexpr (JMAX >= 8 && B * 8 <= 8) {
        if (J == 8) gemv_segment<B, 8, false, false>(P, wl0, wl1, smem, Iout);
      }
      if constexpr (JMAX >= 4 && B * 4 <= 8) {
        if (J == 4) gemv_segment<B, 4, false, false>(P, wl0, wl1, smem, Iout);
      }
      if constexpr (JMAX >= 2 && B * 2 <= 8) {
        if (J == 2) gemv_segment<B, 2, false, false>(P, wl0, wl1, smem, Iout);
      }
      if (J == 1) gemv_segment<B, 1, false, false>(P, wl0, wl1, smem, Iout);
      w = seg_end;
      P = Pn;
      ++rec;
    }
  } else {
    if (w_begin < w_end) gemv_segment<B, JMAX, FOLD, WRITE_I>(p0, w_begin, w_end, smem, Iout);
  }
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------

static int blocks_per_lane(int64_t K) { return blocks_per_lane_of((int)K); }

static size_t fused_lds_bytes(int64_t K, int64_t B) {
  const int64_t nb = K / kQK;
  return (size_t)(B * K + 8 * B * nb + 8 * sizeof(float));
}

bool gemv_supported(int64_t M, int64_t K, int64_t B) {
  (void)M;
  if (B < 1 || B > 4) return false;
  const int J = blocks_per_lane(K);
  return J <= 8 && B * J <= 8;
}

bool gemv_fused_supported(int64_t K, int64_t B) {
  return gemv_supported(1, K, B) && fused_lds_bytes(K, B) <= kGemvMaxLds;
}

int gemv_window_rows(int64_t K, int64_t B) {
  return 4 * gemv_rows_per_wave((int)B, blocks_per_lane(K));
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

template <int B, int JMAX, int KIND>
static hipError_t launch_kind(const GemvProblem& p, const GemvProblem* table, const int32_t* map,
                              int64_t n_windows, size_t lds, int32_t* I, hipStream_t s) {
  const void* k = (const void*)gemv_kernel<B, JMAX, KIND>;
  int64_t grid = resident_workgroups(k, lds);
  if (grid > n_windows) grid = n_windows;
  hipLaunchKernelGGL((gemv_kernel<B, JMAX, KIND>), dim3((unsigned)grid), dim3(kGemvThreads), lds, s, p, table,
                     map, (int)n_windows, I);
  return hipGetLastError();
}

template <int B, int JMAX>
static hipError_t launch_bj(const GemvProblem& p, const GemvProblem* table, const int32_t* map,
                            int64_t n_windows, bool fold, size_t lds, int32_t* I, hipStream_t s) {
  if (table) return launch_kind<B, JMAX, kKindGroup>(p, table, map, n_windows, 0, I, s);
  if (fold) return launch_kind<B, JMAX, kKindFold>(p, table, map, n_windows, lds, I, s);
  if (I) return launch_kind<B, JMAX, kKindBlockSums>(p, table, map, n_windows, 0, I, s);
  return launch_kind<B, JMAX, kKindSingle>(p, table, map, n_windows, 0, I, s);
}

hipError_t launch_gemv_table(const GemvProblem& p, const GemvProblem* table, const int32_t* map,
                             int64_t n_windows, int64_t max_k, int64_t B, bool any_fused, int32_t* I,
                             hipStream_t s) {
  const int J = blocks_per_lane(max_k);
  if (table && (any_fused || I)) return hipErrorInvalidValue;  // grouped launches read Q8 planes
  const size_t lds = any_fused ? fused_lds_bytes(max_k, B) : 0;
#define Q4Q8_GEMV_CASE(BB, JJ) \
  if (B == BB && J == JJ) return launch_bj<BB, JJ>(p, table, map, n_windows, any_fused, lds, I, s);
  Q4Q8_GEMV_CASE(1, 1)
  Q4Q8_GEMV_CASE(1, 2)
  Q4Q8_GEMV_CASE(1, 4)
  Q4Q8_GEMV_CASE(1, 8)
  Q4Q8_GEMV_CASE(2, 1)
  Q4Q8_GEMV_CASE(2, 2)
  Q4Q8_GEMV_CASE(2, 4)
  Q4Q8_GEMV_CASE(3, 1)
  Q4Q8_GEMV_CASE(3, 2)
  Q4Q8_GEMV_CASE(4, 1)
  Q4Q8_GEMV_CASE(4, 2)
#undef Q4Q8_GEMV_CASE
  return hipErrorInvalidValue;
}

}  // namespace q4q8
