// Internal declarations shared by the gfx950 kernels and the C-ABI layer.
// Not installed; the public interface is include/q4q8.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <vector>

#define Q4Q8_HIDDEN __attribute__((visibility("hidden")))

namespace q4q8 {

constexpr int kQK = 32;              // elements per quantisation block
constexpr int kWave = 64;            // CDNA wavefront width
constexpr int kMaxPrologueK = 131072;

// MFMA accumulator seed: the int32 result of an i8 MFMA started from these
// bits, read as fp32, is 1.5 * 2^23 + I exactly for |I| < 2^22, so
// fma(F, d, -1.5 * 2^23 * d) gives fl(I * d) without a separate conversion.
constexpr int kMagicBits = 0x4B400000;
constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23

// Pointers read from a record in memory are generic (flat) pointers; loads
// through them are flat loads, which also count against the LDS counter and
// force coarser waits.  All buffers here are global memory, so accesses go
// through explicit global-address-space pointers.
#define Q4Q8_GLOBAL __attribute__((address_space(1)))
// Native vector types (HIP's float4 / uint4 classes cannot be copied out of
// an explicitly global pointer).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
template <typename T>
__device__ __forceinline__ const Q4Q8_GLOBAL T* gptr(const T* p) {
  return (const Q4Q8_GLOBAL T*)(p);
}
template <typename T>
__device__ __forceinline__ Q4Q8_GLOBAL T* gptr_w(T* p) {
  return (Q4Q8_GLOBAL T*)(p);
}

__device__ __forceinline__ float f16_bits_to_f32(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

__device__ __forceinline__ uint16_t f32_to_f16_bits_rne(float f) {
  // v_cvt_f16_f32 rounds to nearest even in the default mode and keeps
  // fp16 subnormals.
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}

// Correctly rounded fp32 square root.  On gfx950 both sqrtf and __fsqrt_rn
// lower to the hardware estimate, which is not always the nearest float.  The
// estimate is moved to the float whose rounding interval contains x: the
// interval ends are the midpoints between neighbouring floats, each with at
// most 25 significant bits, so their squares are exact in fp64.  (No fp32 x
// has a square root exactly on a midpoint, so there are no ties.)
// Zero, negative, infinite and NaN inputs return the hardware result.
__device__ __forceinline__ float sqrt_rn(float x) {
  float y = __builtin_sqrtf(x);
  if (!(x > 0.0f) || x == __builtin_inff()) return y;
  const double xd = (double)x;
#pragma unroll 1
  for (int it = 0; it < 8; ++it) {
    const uint32_t b = __builtin_bit_cast(uint32_t, y);
    const float lo = __builtin_bit_cast(float, b - 1u);
    const double mlo = ((double)lo + (double)y) * 0.5;
    if (xd < mlo * mlo) {
      y = lo;
      continue;
    }
    const float hi = __builtin_bit_cast(float, b + 1u);
    const double mhi = ((double)y + (double)hi) * 0.5;
    if (xd >= mhi * mhi) {
      y = hi;
      continue;
    }
    break;
  }
  return y;
}

// Exact int32 block product s0 + sum_j q_j * x_j of one Q4 block (16 bytes of
// packed unsigned codes) with one Q8 block (two int4 of codes).
__device__ __forceinline__ int dot_block(const u32x4 w, const i32x4 xa, const i32x4 xb, int s0 = 0) {
  // lo nibbles of byte j = code j (pairs with x codes 0..15 = xa);
  // hi nibbles of byte j = code j+16 (pairs with x codes 16..31 = xb).
  const uint32_t m = 0x0F0F0F0Fu;
  int s = s0;
  s = __builtin_amdgcn_sdot4((int)(w.x & m), xa.x, s, false);
  s = __builtin_amdgcn_sdot4((int)(w.y & m), xa.y, s, false);
  s = __builtin_amdgcn_sdot4((int)(w.z & m), xa.z, s, false);
  s = __builtin_amdgcn_sdot4((int)(w.w & m), xa.w, s, false);
  s = __builtin_amdgcn_sdot4((int)((w.x >> 4) & m), xb.x, s, false);
  s = __builtin_amdgcn_sdot4((int)((w.y >> 4) & m), xb.y, s, false);
  s = __builtin_amdgcn_sdot4((int)((w.z >> 4) & m), xb.z, s, false);
  s = __builtin_amdgcn_sdot4((int)((w.w >> 4) & m), xb.w, s, false);
  return s;
}

// Exact int32 block product s0 + sum_j w_j * x_j of one Q8_0 weight block
// (32 int8 codes in w0 = codes 0..15, w1 = codes 16..31) with one Q8 block.
__device__ __forceinline__ int dot_block_q8(const u32x4 w0, const u32x4 w1, const i32x4 xa, const i32x4 xb,
                                            int s0) {
  int s = s0;
  s = __builtin_amdgcn_sdot4((int)w0.x, xa.x, s, false);
  s = __builtin_amdgcn_sdot4((int)w0.y, xa.y, s, false);
  s = __builtin_amdgcn_sdot4((int)w0.z, xa.z, s, false);
  s = __builtin_amdgcn_sdot4((int)w0.w, xa.w, s, false);
  s = __builtin_amdgcn_sdot4((int)w1.x, xb.x, s, false);
  s = __builtin_amdgcn_sdot4((int)w1.y, xb.y, s, false);
  s = __builtin_amdgcn_sdot4((int)w1.z, xb.z, s, false);
  s = __builtin_amdgcn_sdot4((int)w1.w, xb.w, s, false);
  return s;
}

// Workgroup barrier that orders LDS accesses only.  __syncthreads() also
// fences global memory, which makes every wave wait for all of its global
// loads in flight -- a streaming kernel would drain its prefetch at every
// exchange.  Here the fences are limited to the local (LDS) address space, so
// the barrier waits for this wave's LDS accesses and nothing else.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// Weight block formats (qs of a GemvProblem): per 32-element block,
// kWeightQ4 = 16 bytes of packed 4-bit codes (offset 8), kWeightQ8 = Q8_0,
// 32 int8 codes; both with one fp16 scale per block in d.
enum WeightFormat : int {
  kWeightQ4 = 0,
  kWeightQ8 = 1,
  kWeightMixed = 2,  // grouped launches only: each record's wf decides
};

// One product of a (grouped) GEMV launch, as the kernel reads it.
enum GemvMode : int32_t {
  kModeQ8 = 0,    // activations given as Q8 planes xq / xd
  kModeNorm = 1,  // fp32 x and norm weight g: RMSNorm * g -> Q8 folded in
  kModeRaw = 2,   // fp32 x quantised as it is
};

struct alignas(16) GemvProblem {
  const uint8_t* qs;   // [M][K/2] Q4, or [M][K] Q8_0 (wf)
  const uint16_t* d;   // [M][K/32]
  const int8_t* xq;    // [B][K]       (kModeQ8)
  const float* xd;     // [B][K/32]    (kModeQ8)
  const float* x;      // [B][K]       (kModeNorm, kModeRaw)
  const float* g;      // [K]          (kModeNorm)
  float* y;            // [B][M]
  int32_t M;
  int32_t K;
  float eps;
  int32_t mode;
  int32_t win_begin;   // index of this problem's first window in the launch
  int32_t n_win;       // windows of this problem (ceil(M / window rows))
  int32_t wf;          // weight format of qs (WeightFormat)
  int32_t win_off;     // index, within its product, of this record's first window (multi-column
                       // groups split a product's windows over several records; else 0)
};
static_assert(sizeof(GemvProblem) == 96, "GemvProblem layout");

// One fp32 input of a grouped launch, quantised by the prologue pass into
// Q8 planes that the streaming pass then reads.
struct alignas(16) PrologueJob {
  const float* x;  // [B][K]
  const float* g;  // [K] (null when raw)
  int8_t* xq;      // [B][K]
  float* xd;       // [B][K/32]
  int32_t K;
  float eps;
  int32_t raw;     // quantise x as it is
  int32_t pad;
};
static_assert(sizeof(PrologueJob) == 48, "PrologueJob layout");


// Records the kernel instance a launch site is about to launch (host pointer
// of the __global__ function), per calling thread, for q4q8_last_kernel().
Q4Q8_HIDDEN void note_launch(const void* kernel);

// Route selection helpers (host).  gemv_supported: the lane-per-block
// streaming kernel (gemv_dev.h, also the routed MoE kernel) serves K with B
// columns; gemv_route_supported: either streaming kernel serves the product
// (the MFMA kernel of gemv_mfma.hip takes B = 5..8 where gemv_mfma_ok).
Q4Q8_HIDDEN bool gemv_supported(int64_t M, int64_t K, int64_t B);
Q4Q8_HIDDEN bool gemv_route_supported(int64_t M, int64_t K, int64_t B, int wf);
// The multi-column MFMA kernel serves B = 5..8 columns on Q8 planes with
// rows of at least four whole 128-byte segments (K a multiple of 256 and at
// least 1024 for Q4, a multiple of 128 and at least 512 for Q8_0)
// and weight planes under 2 GiB (32-bit buffer offsets); its callers also
// require d and xd 16-byte aligned, and one weight format per launch.
constexpr int kGemvMfmaMinB = 5;
Q4Q8_HIDDEN bool gemv_mfma_ok(int64_t M, int64_t K, int64_t B, int wf);
// Rows per window of the MFMA multi-column kernel, and its launcher.  A
// single product (table == nullptr) is split into equal shares of its
// windows; a group launches `groups` workgroups over a table whose map
// (window -> record, n_windows entries) is followed by groups + 1 window
// indices: workgroup g streams windows [bounds[g], bounds[g + 1]).
Q4Q8_HIDDEN int gemv_mfma_window_rows();
Q4Q8_HIDDEN hipError_t launch_gemv_mfma(const GemvProblem& p, const GemvProblem* table, const int32_t* map,
                                        int64_t n_windows, int64_t groups, int64_t B, int32_t* I, hipStream_t s,
                                        int wf);
// Workgroups a grouped multi-column launch takes on the current device (all
// resident at once; 2 per CU x 256 CUs when no device answers).
Q4Q8_HIDDEN int64_t gemv_mfma_group_grid(int wf);
// Packs the windows of a multi-column group into `groups` workgroup bins of
// near-equal cost (a window of record r costs cost[r] = K / 32, its 64 rows
// being common).  Output, in launch order: runs of consecutive windows of one
// record (rec, first window within it, count), and groups + 1 bounds (bin g
// holds launch windows [bounds[g], bounds[g + 1])).
struct MfRun {
  int32_t rec, first, count;
};
Q4Q8_HIDDEN void gemv_mfma_pack(const std::vector<int64_t>& n_win, const std::vector<int64_t>& cost, int64_t groups,
                                std::vector<MfRun>& runs, std::vector<int64_t>& bounds);
Q4Q8_HIDDEN bool gemv_fused_supported(int64_t K, int64_t B);
// Rows per window (the unit a workgroup streams) for a product with K and B;
// wf: weight format (kWeightQ4 or kWeightQ8); fold: the folded-prologue form.
Q4Q8_HIDDEN int gemv_window_rows(int64_t K, int64_t B, int wf = kWeightQ4, bool fold = false);
// Persistent launch over the products of a device `table`, window w of the
// launch belonging to record map[w]; or, when table == nullptr, over the
// single record `p`.  `n_windows` = total windows; `max_k` = largest K among
// the products (selects the kernel instance and the LDS size).  wf: the weight
// format of `p`, or of every table record (kWeightMixed: read per record).
Q4Q8_HIDDEN hipError_t launch_gemv_table(const GemvProblem& p, const GemvProblem* table,
                                         const int32_t* map, int64_t n_windows, int64_t max_k,
                                         int64_t B, bool any_fused, int32_t* I, hipStream_t s,
                                         int wf = kWeightQ4);

// Launchers: enqueue on `s`, return the launch status.
Q4Q8_HIDDEN hipError_t launch_q4_quantize(const float* w, int64_t M, int64_t K, uint8_t* qs,
                                          uint16_t* d, hipStream_t s);
Q4Q8_HIDDEN hipError_t launch_q8w_quantize(const float* w, int64_t M, int64_t K, int8_t* qw, uint16_t* d,
                                           hipStream_t s);
// a: addend rows (RMS_NORM+MUL+ADD; row b at a + b * a_row_stride) or null.
Q4Q8_HIDDEN hipError_t launch_q8_rmsnorm(const float* x, int64_t B, int64_t K, const float* g,
                                         float eps, bool no_norm, int8_t* xq, float* xd,
                                         int32_t* xs, hipStream_t s, const float* a = nullptr,
                                         int64_t a_row_stride = 0);
Q4Q8_HIDDEN hipError_t launch_swiglu_q8(const float* gate, const float* up, int64_t B, int64_t F,
                                        int64_t row_stride, int8_t* xq, float* xd, int32_t* xs, hipStream_t s);
Q4Q8_HIDDEN hipError_t launch_group_prologue(const PrologueJob* jobs, int64_t n_jobs, int64_t B,
                                             int64_t max_k, hipStream_t s);
// Tiles (128 weight rows x 128 tokens) of one product on the tiled route.
Q4Q8_HIDDEN int64_t gemm_tiles(int64_t M, int64_t B);
// Tiled route over the single record `p` (table == nullptr, n_tiles =
// gemm_tiles(p.M, B)) or over the products of a device `table`, tile t of the
// launch belonging to record tile_map[t] (its first tile is win_begin); wf as
// for launch_gemv_table.
Q4Q8_HIDDEN hipError_t launch_gemm(const GemvProblem& p, const GemvProblem* table, const int32_t* tile_map,
                                   int64_t n_tiles, int64_t B, int32_t* I, hipStream_t s,
                                   int wf = kWeightQ4);
Q4Q8_HIDDEN size_t moe_workspace_bytes(int64_t E, int64_t T, int64_t top_k);
// The library-owned routing scratch of the current device (device address)
// and its size: the workspace of mul_mat_id_q4q8_noalloc.
Q4Q8_HIDDEN size_t moe_scratch_bytes();
Q4Q8_HIDDEN hipError_t moe_scratch(void** out);
Q4Q8_HIDDEN hipError_t launch_moe_expert_sum(const float* y, const float* w, int64_t T, int64_t top_k,
                                             int64_t M, float* out, hipStream_t s);
// Upper bound of the routed launch's total schedule cost (it must fit int32).
Q4Q8_HIDDEN int64_t moe_schedule_cost_bound(int64_t E, int64_t M, int64_t K, int64_t n);
Q4Q8_HIDDEN hipError_t launch_moe(const uint8_t* qs, const uint16_t* d, int64_t E, int64_t M,
                                  int64_t K, const int8_t* xq, const float* xd, int64_t n_x_slots,
                                  const int32_t* ids, int64_t T, int64_t top_k, float* y,
                                  void* ws, hipStream_t s);

}  // namespace q4q8
