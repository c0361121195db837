// Multi-column Q4 x Q8 decode kernel on int8 MFMA for gfx950: the streaming
// matrix x vector route of "GGML：Backend 抽象与硬件加速" (section "CUDA：mmvq、
// mmq、cublas 三条矩阵路") for B = 5..8 activation columns (the kernel
// serves any B up to 8; with up to four columns the lane-per-block kernel is
// faster and the route takes that).
//
// Why a matrix instruction for a vector product: with several columns the
// lane-per-block dot4 kernel (gemv_dev.h) spends ~8 v_dot4 per block and
// column plus a cross-lane reduction per output, and from five columns on
// (padded to eight) its vector ALU becomes the bound.  v_mfma_i32_16x16x64_i8 forms the exact block sums of
// 16 weight rows with up to 8 columns for TWO 32-element blocks at once:
//   A (16 x 64, activations): row m = 2c + b holds column c's codes of
//     block 2p + b in k = 32b .. 32b + 31 and zeros in the other half;
//   B (64 x 16, weights): column n holds weight row n's codes of blocks 2p
//     (k < 32) and 2p + 1 (k >= 32), as signed bytes (16 (q - 8) for Q4,
//     see mf_chunk);
//   D = A B: D[2c + b][n] = I(column c, row n, block 2p + b), exact in
//     int32 (|16 I| <= 520192 < 2^22, as the seeded accumulator needs).
// Lane layout of the instruction (checked on gfx950): lane l supplies row
// l % 16 of A and column l % 16 of B, k = 16 (l / 16) .. + 15, and holds
// D rows 4 (l / 16) + i, column l % 16.  So lane l = 16 g + n owns weight
// row n, columns 2g and 2g + 1, blocks 2p and 2p + 1: each output element
// costs the two fp32 fmas of the per-block rescale (seeded accumulator, as in
// the tiled kernel) and nothing else -- no cross-lane reduction at all.
//
// Memory: an MFMA operand holds 16 bytes of each of 16 rows, so weights
// loaded straight into operand registers touch every 128-byte line of a row
// from eight instructions, and HBM sees short scattered requests.  Instead
// each wave stages its weights through its own LDS region with direct-to-LDS
// buffer loads of whole 128-byte row segments: a chunk is 64 rows x 128
// bytes (4 block pairs of Q4, 2 of Q8_0) plus the rows' block scales.  The
// row segments land in LDS with their 16-byte pieces rotated by row, so that
// the operand reads of 16 rows hit 16 distinct bank groups.  A landed chunk
// is read out into registers at once and its buffer refilled, so two chunks
// per wave are in flight while one is computed.  Activation operands and
// scales (a few KiB per product, resident in L2) go straight to registers,
// one chunk ahead.
//
// Work: a window is 64 weight rows of one product over all of K, streamed by
// the four waves of a workgroup together, wave w taking chunks w, w + 4,
// w + 8, ...: at any time the workgroup reads 512 contiguous bytes of each of
// 64 rows and 64 contiguous bytes of each row's scales -- long runs that HBM
// serves well (a wave alone on a window would read 128 bytes per row and 16
// bytes of scales, and the scale lines, revisited chunk after chunk, leave
// L2 in between).  At a window's end the four partial sums meet in LDS and
// are added in wave order, so results do not depend on timing.  A single
// product is split into equal shares of its windows.  A group's windows are
// packed on the host into one bin per workgroup, of near-equal cost (rows x
// K), so that products with long and short K mix evenly: a row's sum never
// depends on which workgroup streams its window, so the packing leaves every
// result bit-identical.
#include <algorithm>
#include <mutex>
#include <utility>
#include <vector>

#include "common.h"

namespace q4q8 {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
#define Q4Q8_LDS __attribute__((address_space(3)))

constexpr int kMfThreads = 256;
constexpr int kMfWaves = kMfThreads / kWave;
constexpr int kMfRg = 4;                          // row groups of 16 per window
constexpr int kMfRows = 16 * kMfRg;               // rows per window
constexpr int kMfSegBytes = 128;                  // weight bytes of a row per chunk
constexpr int kMfWBytes = kMfRows * kMfSegBytes;  // 8 KiB of weights per chunk
constexpr int kMfBufBytes = kMfWBytes + 1024;     // + the scales of 64 rows
// Word 3 of a raw buffer resource on gfx9-family GPUs (32-bit data format,
// no swizzle, stride 0): loads then take a 32-bit per-lane offset plus a
// wave-uniform one, and a lane whose offset lies past the buffer's size reads
// zeros (and writes zeros to LDS).
constexpr int kBufferWord3 = 0x00020000;
constexpr uint32_t kOutOfRange = 0x7FFFFFF0u;  // a per-lane offset past every buffer here

// Block pairs per chunk: 128 bytes of a row are 4 pairs of Q4 blocks (16
// bytes each) or 2 pairs of Q8_0 blocks (32 bytes each).
template <int WF>
__host__ __device__ constexpr int mf_pairs_per_chunk() {
  return WF == kWeightQ8 ? 2 : 4;
}

// A wave's window: 64 rows of one product (uniform across the wave).
struct MfWindow {
  const uint8_t* qs;
  const uint16_t* d;
  const int8_t* xq;
  const float* xd;
  float* y;
  int M, K, nb, row0, nch;
};

template <int WF>
__device__ __forceinline__ MfWindow mf_window(const GemvProblem& P, int w) {
  MfWindow W;
  W.qs = P.qs;
  W.d = P.d;
  W.xq = P.xq;
  W.xd = P.xd;
  W.y = P.y;
  W.M = P.M;
  W.K = P.K;
  W.nb = P.K >> 5;
  W.row0 = (w - P.win_begin + P.win_off) * kMfRows;
  W.nch = (P.K >> 6) / mf_pairs_per_chunk<WF>();  // the route takes K of >= 4 whole chunks only
  return W;
}


// Load addresses of a window for the wave's lanes, at chunk 0 (chunk c adds
// a uniform offset).  Weight stream (direct-to-LDS):
//   ow[j]: weight load j (rows 8j .. 8j + 7, 16 bytes per lane): lane i
//     fills slot i % 8 of row r = 8j + i / 8, which holds the row's piece
//     (slot - rot(r)) mod 8, rot(r) = (r % 16) / 2; rows past M read zeros.
//   od: the lane's row (lane i = row i) of the scale plane.
struct MfDmaFront {
  __amdgpu_buffer_rsrc_t rw, rd;
  uint32_t ow[8];
  uint32_t od;
};
// Activation stream (registers): oa, the lane's A operand; ox, the scales
// of columns 2g and 2g + 1.
struct MfRegFront {
  __amdgpu_buffer_rsrc_t ra, rx;
  uint32_t oa, ox[2];
};

template <int WF>
__device__ __forceinline__ MfDmaFront mf_dma_front(const MfWindow& W, int lane) {
  const uint32_t row_bytes = WF == kWeightQ8 ? (uint32_t)W.K : (uint32_t)W.K >> 1;
  MfDmaFront F;
  F.rw = __builtin_amdgcn_make_buffer_rsrc((void*)W.qs, (short)0, (int)((uint32_t)W.M * row_bytes), kBufferWord3);
  F.rd = __builtin_amdgcn_make_buffer_rsrc((void*)W.d, (short)0, W.M * W.nb * 2, kBufferWord3);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = 8 * j + lane / 8;
    const int piece = ((lane & 7) - (4 * (j & 1) + lane / 16)) & 7;
    const int row = W.row0 + r;
    F.ow[j] = row < W.M ? (uint32_t)row * row_bytes + 16u * (uint32_t)piece : kOutOfRange;
  }
  const int drow = W.row0 + lane;
  F.od = drow < W.M ? (uint32_t)drow * (uint32_t)W.nb * 2u : kOutOfRange;
  return F;
}

template <int WF>
__device__ __forceinline__ MfRegFront mf_reg_front(const MfWindow& W, int lane, int B) {
  const int n = lane & 15, g = lane >> 4;
  MfRegFront F;
  F.ra = __builtin_amdgcn_make_buffer_rsrc((void*)W.xq, (short)0, B * W.K, kBufferWord3);
  F.rx = __builtin_amdgcn_make_buffer_rsrc((void*)W.xd, (short)0, B * W.nb * 4, kBufferWord3);
  // A operand of lane (g, m = n): column m >> 1, block 2p + (m & 1), which
  // lies in this lane's k range 16 g .. 16 g + 15 only when (m & 1) == g >> 1
  const int col = n >> 1;
  F.oa = ((n & 1) == (g >> 1) && col < B) ? (uint32_t)(col * W.K + 16 * g) : kOutOfRange;
#pragma unroll
  for (int j = 0; j < 2; ++j) F.ox[j] = (uint32_t)min(2 * g + j, B - 1) * (uint32_t)W.nb * 4u;
  return F;
}

// Register part of a chunk: the activation operands of its pairs, and the
// activation scales of columns 2g and 2g + 1 (fp32 bits), four blocks (two
// pairs) per vector.
template <int WF>
struct MfRegs {
  v4i a[mf_pairs_per_chunk<WF>()];
  u32x4 x[2][mf_pairs_per_chunk<WF>() / 2];
};

// A chunk's weights and scales, read out of LDS: the lane's 16 bytes of
// pair s in row group r, and the fp16 scales of its rows (Q4: the chunk's 8
// blocks of each of its 4 rows, as one vector per row group; Q8_0: blocks
// 2s, 2s + 1 per word).
template <int WF>
struct MfChunkW {
  u32x4 w[mf_pairs_per_chunk<WF>()][kMfRg];
  uint32_t ds[mf_pairs_per_chunk<WF>()][kMfRg];
};

// Vector memory instructions of the two issue steps: direct-to-LDS loads
// (8 of weights, 1 or 2 of scales) and register loads.  Every one is a
// 16-byte load or a direct-to-LDS load, which the compiler can neither merge
// nor split, and each step is fenced against reordering, so the counts are
// exact.
template <int WF>
__host__ __device__ constexpr int mf_lds_loads() {
  return WF == kWeightQ8 ? 10 : 9;
}

// Direct-to-LDS loads of chunk c of the front's window into buffer `buf`.
template <int WF>
__device__ __forceinline__ void mf_issue_dma(const MfDmaFront& F, int c, Q4Q8_LDS uint8_t* buf) {
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < 8; ++j)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(F.rw, (Q4Q8_LDS void*)(buf + 1024 * j), 16, F.ow[j],
                                             kMfSegBytes * c, 0, 0);
  if constexpr (WF == kWeightQ8) {
    // 4 blocks per chunk: two 4-byte pieces per row, stored [piece][row]
    __builtin_amdgcn_raw_ptr_buffer_load_lds(F.rd, (Q4Q8_LDS void*)(buf + kMfWBytes), 4, F.od, 8 * c, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(F.rd, (Q4Q8_LDS void*)(buf + kMfWBytes + 256), 4, F.od, 8 * c + 4, 0,
                                             0);
  } else {
    // 8 blocks per chunk: 16 bytes per row, stored [row][16 bytes]
    __builtin_amdgcn_raw_ptr_buffer_load_lds(F.rd, (Q4Q8_LDS void*)(buf + kMfWBytes), 16, F.od, 16 * c, 0, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
}

// Register loads of chunk c of the front's window into `R`.
template <int WF>
__device__ __forceinline__ void mf_issue_reg(const MfRegFront& F, int c, MfRegs<WF>& R) {
  constexpr int CP = mf_pairs_per_chunk<WF>();
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int s = 0; s < CP; ++s) R.a[s] = __builtin_amdgcn_raw_buffer_load_b128(F.ra, F.oa, 64 * (c * CP + s), 0);
#pragma unroll
  for (int t = 0; t < CP / 2; ++t)
#pragma unroll
    for (int j = 0; j < 2; ++j)
      R.x[j][t] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(F.rx, F.ox[j], 8 * CP * c + 16 * t,
                                                                                  0));
  __builtin_amdgcn_sched_barrier(0);
}

// Waits until at most N vector memory instructions are in flight.  The
// compiler does not order LDS reads after direct-to-LDS loads by itself.
template <int N>
__device__ __forceinline__ void mf_wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Waits for every LDS read in flight (before a buffer is refilled).
__device__ __forceinline__ void mf_wait_lds_reads() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Reads a landed chunk out of LDS buffer `buf` into registers.
template <int WF>
__device__ __forceinline__ MfChunkW<WF> mf_read(const Q4Q8_LDS uint8_t* buf, int lane) {
  constexpr int CP = mf_pairs_per_chunk<WF>();
  const int n = lane & 15, g = lane >> 4, h = g & 1, bsel = g >> 1;
  // this lane's row within a 16-row group (128 bytes per row) and the
  // rotation of its pieces
  const int rowoff = n * kMfSegBytes;
  const int rot = n >> 1;
  MfChunkW<WF> CW;
#pragma unroll
  for (int s = 0; s < CP; ++s) {
    // the lane's 16 bytes: block 2s + bsel of the chunk (Q4: one piece per
    // block; Q8_0: two pieces per block, half h)
    const int piece = WF == kWeightQ8 ? 4 * s + 2 * bsel + h : 2 * s + bsel;
    const int woff = rowoff + ((piece + rot) & 7) * 16;
#pragma unroll
    for (int r = 0; r < kMfRg; ++r)
      CW.w[s][r] = *reinterpret_cast<const Q4Q8_LDS u32x4*>(buf + r * 16 * kMfSegBytes + woff);
  }
#pragma unroll
  for (int r = 0; r < kMfRg; ++r) {
    const int rr = 16 * r + n;  // row within the window
    if constexpr (WF == kWeightQ8) {
#pragma unroll
      for (int s = 0; s < CP; ++s)
        CW.ds[s][r] = *reinterpret_cast<const Q4Q8_LDS uint32_t*>(buf + kMfWBytes + 256 * s + 4 * rr);
    } else {
      const u32x4 v = *reinterpret_cast<const Q4Q8_LDS u32x4*>(buf + kMfWBytes + 16 * rr);
      CW.ds[0][r] = v.x;
      CW.ds[1][r] = v.y;
      CW.ds[2][r] = v.z;
      CW.ds[3][r] = v.w;
    }
  }
  return CW;
}

// Computes chunk c of window W from its weights `CW` and activations `R`.
template <int WF, bool WRITE_I>
__device__ __forceinline__ void mf_compute(const MfWindow& W, int c, const MfChunkW<WF>& CW, const MfRegs<WF>& R,
                                           int lane, int B, const v4i seed, float (&acc)[kMfRg][4],
                                           int32_t* __restrict__ Iout) {
  constexpr int CP = mf_pairs_per_chunk<WF>();
  const int n = lane & 15, g = lane >> 4, h = g & 1;
  // Q4 codes enter the product as 16 (q - 8): the lane's nibble (low for
  // codes 0..15, high for 16..31) moved to the high half of its byte with
  // the top bit flipped is that value as a signed byte, so two bit
  // operations per word replace a q - 8 conversion; the factor 16 stays in
  // the sums and is taken out of the final outputs (exact: a power of two).
  const uint32_t sh = 4u - 4u * (uint32_t)h;
#pragma unroll
  for (int s = 0; s < CP; ++s) {
    v4i F[kMfRg];
#pragma unroll
    for (int r = 0; r < kMfRg; ++r) {
      v4i b;
      if constexpr (WF == kWeightQ8)
        b = __builtin_bit_cast(v4i, CW.w[s][r]);
      else
        b = __builtin_bit_cast(v4i, ((CW.w[s][r] << sh) ^ 0x80808080u) & 0xF0F0F0F0u);
      F[r] = __builtin_amdgcn_mfma_i32_16x16x64_i8(R.a[s], b, seed, 0, 0, 0);
    }
    // (whole vectors reinterpreted: hipcc miscompiles a bit cast of one
    // element of a vector)
    const f32x4 x0 = __builtin_bit_cast(f32x4, R.x[0][s >> 1]), x1 = __builtin_bit_cast(f32x4, R.x[1][s >> 1]);
    const f32x2 xa = (s & 1) ? f32x2{x0.z, x0.w} : f32x2{x0.x, x0.y};
    const f32x2 xb = (s & 1) ? f32x2{x1.z, x1.w} : f32x2{x1.x, x1.y};
#pragma unroll
    for (int r = 0; r < kMfRg; ++r) {
      const uint32_t dw = CW.ds[s][r];
      const float d0 = f16_bits_to_f32((uint16_t)(dw & 0xFFFFu));  // block 2p
      const float d1 = f16_bits_to_f32((uint16_t)(dw >> 16));      // block 2p + 1
      const float c0 = -kMagic * d0, c1 = -kMagic * d1;
      const f32x4 Fv = __builtin_bit_cast(f32x4, F[r]);
      acc[r][0] = __builtin_fmaf(__builtin_fmaf(Fv.x, d0, c0), xa.x, acc[r][0]);
      acc[r][1] = __builtin_fmaf(__builtin_fmaf(Fv.y, d1, c1), xa.y, acc[r][1]);
      acc[r][2] = __builtin_fmaf(__builtin_fmaf(Fv.z, d0, c0), xb.x, acc[r][2]);
      acc[r][3] = __builtin_fmaf(__builtin_fmaf(Fv.w, d1, c1), xb.y, acc[r][3]);
      if constexpr (WRITE_I) {
        const int row = W.row0 + 16 * r + n, p = c * CP + s;
        v4i Iv = F[r] - seed;
        if constexpr (WF != kWeightQ8) Iv = Iv >> 4;  // exact: the sum is 16 I
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int col = 2 * g + (i >> 1), blk = 2 * p + (i & 1);
          int v;
          if (i == 0) v = Iv.x;
          else if (i == 1) v = Iv.y;
          else if (i == 2) v = Iv.z;
          else v = Iv.w;
          if (col < B && row < W.M) Iout[((int64_t)col * W.M + row) * W.nb + blk] = v;
        }
      }
    }
  }
}

// The outputs of a finished window, held until the wave's next issue point:
// columns 2g and 2g + 1 of row row0 + n.
struct MfOut {
  float v[2];
  float* y;
  int M, row0;
};

// Partial sums of a window on their way to the wave that adds them up:
// [row group r][slot of the sending wave among the other three][column 2g + j][lane].
struct MfExchange {
  float v[kMfRg][kMfWaves - 1][2][kWave];
};
static_assert(kMfRg == kMfWaves, "wave r adds up row group r");

// LDS writes done, then the workgroup's barrier.  Spelled out because the
// compiler's workgroup barrier may also wait for every vector memory load in
// flight.
__device__ __forceinline__ void mf_lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Ends a window: each lane adds its two block parities for columns 2g and
// 2g + 1 of its four rows; wave r adds the four waves' partials of row group
// r in wave order (scaled by 1/16 for Q4 codes, which enter the products as
// 16 (q - 8)) and holds them for storing; the sums restart from zero.
template <int WF>
__device__ __forceinline__ void mf_finish(const MfWindow& W, float (&acc)[kMfRg][4], MfOut& O,
                                          Q4Q8_LDS MfExchange* X, int lane, int wave) {
  constexpr float scale = WF == kWeightQ8 ? 1.0f : 0.0625f;
  float v[kMfRg][2];
#pragma unroll
  for (int r = 0; r < kMfRg; ++r) {
    v[r][0] = acc[r][0] + acc[r][1];
    v[r][1] = acc[r][2] + acc[r][3];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[r][i] = 0.0f;
  }
#pragma unroll
  for (int r = 0; r < kMfRg; ++r)
    if (r != wave) {
      const int slot = wave < r ? wave : wave - 1;
      X->v[r][slot][0][lane] = v[r][0];
      X->v[r][slot][1][lane] = v[r][1];
    }
  mf_lds_barrier();
  // this wave's own partials of row group `wave` (uniform selects, not a
  // dynamically indexed register array)
  float own[2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
    own[j] = wave == 0 ? v[0][j] : wave == 1 ? v[1][j] : wave == 2 ? v[2][j] : v[3][j];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    float t = 0.0f;
#pragma unroll
    for (int q = 0; q < kMfWaves; ++q) {
      const float x = q == wave ? own[j] : X->v[wave][q < wave ? q : q - 1][j][lane];
      t = q == 0 ? x : t + x;
    }
    O.v[j] = t * scale;
  }
  mf_lds_barrier();  // the exchange area is free again
  O.y = W.y;
  O.M = W.M;
  O.row0 = W.row0 + 16 * wave;
}

__device__ __forceinline__ void mf_store(const MfOut& O, int lane, int B) {
  const int n = lane & 15, g = lane >> 4;
  const int row = O.row0 + n;
  if (row < O.M) {
    if (2 * g < B) gptr_w(O.y)[(int64_t)(2 * g) * O.M + row] = O.v[0];
    if (2 * g + 1 < B) gptr_w(O.y)[(int64_t)(2 * g + 1) * O.M + row] = O.v[1];
  }
}

template <bool GROUPED, bool WRITE_I, int WF>
__global__ __launch_bounds__(kMfThreads, 2) void gemv_mfma_kernel(GemvProblem p0,
                                                                  const GemvProblem* __restrict__ table,
                                                                  const int32_t* __restrict__ win_map,
                                                                  int n_windows, int B, int32_t* __restrict__ Iout) {
  // one LDS object for the chunk buffers and the exchange area
  __shared__ __align__(16) uint8_t lds[kMfWaves * 2 * kMfBufBytes + sizeof(MfExchange)];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  // The window -> record map (and, after it, the workgroups' window bounds)
  // is read through the constant address space: scalar loads, which do not
  // wait behind the vector loads in flight.
  const __attribute__((address_space(4))) int32_t* cmap = (const __attribute__((address_space(4))) int32_t*)win_map;
  // this workgroup's windows
  const int64_t G = gridDim.x, gi = blockIdx.x;
  int w_lo, w_hi;
  if constexpr (GROUPED) {
    w_lo = cmap[n_windows + gi];
    w_hi = cmap[n_windows + gi + 1];
  } else {
    w_lo = (int)(n_windows * gi / G);
    w_hi = (int)(n_windows * (gi + 1) / G);
  }
  w_lo = __builtin_amdgcn_readfirstlane(w_lo);
  w_hi = __builtin_amdgcn_readfirstlane(w_hi);
  if (w_lo >= w_hi) return;  // the whole workgroup: no barrier is left waiting
  auto window = [&](int w) -> MfWindow {
    if constexpr (GROUPED)
      return mf_window<WF>(table[cmap[w]], w);
    else
      return mf_window<WF>(p0, w);
  };
  Q4Q8_LDS uint8_t* buf0 = (Q4Q8_LDS uint8_t*)&lds[(2 * wave) * kMfBufBytes];
  Q4Q8_LDS uint8_t* buf1 = (Q4Q8_LDS uint8_t*)&lds[(2 * wave + 1) * kMfBufBytes];
  Q4Q8_LDS MfExchange* X = (Q4Q8_LDS MfExchange*)&lds[kMfWaves * 2 * kMfBufBytes];

  v4i seed;
  {
    int v;
    asm volatile("v_mov_b32 %0, %1" : "=v"(v) : "s"(kMagicBits));
    seed = v4i{v, v, v, v};
  }
  float acc[kMfRg][4];
#pragma unroll
  for (int r = 0; r < kMfRg; ++r)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[r][i] = 0.0f;

  // Three fronts walk the wave's chunks (window by window; chunks wave,
  // wave + 4, ... of each, every window having at least four): the compute
  // front (window cw, chunk cc); the register front, one chunk ahead; the
  // direct-to-LDS front, two chunks ahead.  A chunk is read out of LDS into
  // registers as soon as it has landed, and its buffer is refilled at once.
  // Past the wave's last chunk the fronts re-issue it (unconditional loads:
  // a register loaded under a branch would merge with its old contents, and
  // the copies of such a merge wait for every load in flight).  Issue order
  // per step: register loads of chunk i + 1, then the direct-to-LDS loads of
  // chunk i + 2; so when chunk i is due, everything but the latest
  // direct-to-LDS loads must have landed.
  int cw = w_lo, cc = wave;
  MfWindow C = window(cw);
  int dw_ = w_lo, dc = wave, rw_ = w_lo, rc = wave;
  MfWindow DL = C, RL = C;
  MfDmaFront DF = mf_dma_front<WF>(DL, lane);
  MfRegFront RF = mf_reg_front<WF>(RL, lane, B);
  auto dma_advance = [&]() {
    if (dc + kMfWaves < DL.nch) {
      dc += kMfWaves;
    } else if (dw_ + 1 < w_hi) {
      ++dw_;
      dc = wave;
      DL = window(dw_);
      DF = mf_dma_front<WF>(DL, lane);
    }
  };
  auto reg_advance = [&]() {
    if (rc + kMfWaves < RL.nch) {
      rc += kMfWaves;
    } else if (rw_ + 1 < w_hi) {
      ++rw_;
      rc = wave;
      RL = window(rw_);
      RF = mf_reg_front<WF>(RL, lane, B);
    }
  };
  MfOut O;
  bool pending = false;
  // Ends the compute front's chunk (and, after the wave's last chunk of a
  // window, the window, with the workgroup); false when the share is done.
  auto compute_advance = [&]() {
    cc += kMfWaves;
    if (cc < C.nch) return true;
    mf_finish<WF>(C, acc, O, X, lane, wave);
    pending = true;
    if (++cw >= w_hi) return false;
    C = window(cw);
    cc = wave;
    return true;
  };
  MfRegs<WF> R0, R1;
  mf_issue_dma<WF>(DF, dc, buf0);
  dma_advance();
  mf_issue_reg<WF>(RF, rc, R0);
  reg_advance();
  mf_issue_dma<WF>(DF, dc, buf1);
  dma_advance();
  // Two chunks per iteration, so that the LDS buffer and register set of
  // each are fixed (buffer 0 / R0, then buffer 1 / R1).
  for (;;) {
    mf_wait_vm<mf_lds_loads<WF>()>();
    MfChunkW<WF> CW = mf_read<WF>(buf0, lane);
    mf_wait_lds_reads();
    // outputs of the window that ended last step, stored before the next
    // loads so that no wait above has to cover them
    if (pending) {
      mf_store(O, lane, B);
      pending = false;
    }
    mf_issue_reg<WF>(RF, rc, R1);
    reg_advance();
    mf_issue_dma<WF>(DF, dc, buf0);
    dma_advance();
    mf_compute<WF, WRITE_I>(C, cc, CW, R0, lane, B, seed, acc, Iout);
    // the sums' updates stay before the loads that reuse R0 (sunk below
    // them, they would keep R0 alive and force copies that wait for loads)
#pragma unroll
    for (int r = 0; r < kMfRg; ++r)
#pragma unroll
      for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(acc[r][i]));
    __builtin_amdgcn_sched_barrier(0);
    if (!compute_advance()) break;

    mf_wait_vm<mf_lds_loads<WF>()>();
    CW = mf_read<WF>(buf1, lane);
    mf_wait_lds_reads();
    if (pending) {
      mf_store(O, lane, B);
      pending = false;
    }
    mf_issue_reg<WF>(RF, rc, R0);
    reg_advance();
    mf_issue_dma<WF>(DF, dc, buf1);
    dma_advance();
    mf_compute<WF, WRITE_I>(C, cc, CW, R1, lane, B, seed, acc, Iout);
#pragma unroll
    for (int r = 0; r < kMfRg; ++r)
#pragma unroll
      for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(acc[r][i]));
    __builtin_amdgcn_sched_barrier(0);
    if (!compute_advance()) break;
  }
  mf_store(O, lane, B);
  // the fronts' last (repeated) chunks may still be landing in LDS
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------

int gemv_mfma_window_rows() { return kMfRows; }

// Workgroups of `kernel` resident at once on the current device.  Without a
// device (a plan built on a host with no GPU) the figure is the launch bound
// of these kernels on gfx950: 2 per CU x 256 CUs.
static int64_t mf_resident_workgroups(const void* kernel) {
  static std::mutex mu;
  static std::vector<std::pair<std::pair<const void*, int>, int64_t>> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 2 * 256;
  std::lock_guard<std::mutex> lk(mu);
  for (const auto& e : cache)
    if (e.first.first == kernel && e.first.second == dev) return e.second;
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kMfThreads, 0) != hipSuccess || per_cu < 1)
    per_cu = 2;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 256;
  const int64_t n = (int64_t)per_cu * cus;
  cache.push_back({{kernel, dev}, n});
  return n;
}

int64_t gemv_mfma_group_grid(int wf) {
  return mf_resident_workgroups(wf == kWeightQ8 ? (const void*)gemv_mfma_kernel<true, false, kWeightQ8>
                                                : (const void*)gemv_mfma_kernel<true, false, kWeightQ4>);
}

hipError_t launch_gemv_mfma(const GemvProblem& p, const GemvProblem* table, const int32_t* map, int64_t n_windows,
                            int64_t groups, int64_t B, int32_t* I, hipStream_t s, int wf) {
  if (B < 1 || B > 8 || n_windows < 1 || n_windows > INT32_MAX) return hipErrorInvalidValue;
  if (table && (I || groups < 1 || groups > n_windows)) return hipErrorInvalidValue;
  auto go = [&](auto kernel) {
    // a group: one workgroup per bin of the table; a single product: the
    // resident workgroups, each streaming whole windows (no more workgroups
    // than windows)
    int64_t grid = groups;
    if (!table) {
      grid = mf_resident_workgroups((const void*)kernel);
      if (grid > n_windows) grid = n_windows;
    }
    note_launch((const void*)kernel);
    hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kMfThreads), 0, s, p, table, map, (int)n_windows, (int)B,
                       I);
    return hipGetLastError();
  };
  if (table) {
    if (wf == kWeightQ4) return go(gemv_mfma_kernel<true, false, kWeightQ4>);
    if (wf == kWeightQ8) return go(gemv_mfma_kernel<true, false, kWeightQ8>);
    return hipErrorInvalidValue;  // one weight format per launch
  }
  if (wf == kWeightQ4)
    return I ? go(gemv_mfma_kernel<false, true, kWeightQ4>) : go(gemv_mfma_kernel<false, false, kWeightQ4>);
  if (wf == kWeightQ8)
    return I ? go(gemv_mfma_kernel<false, true, kWeightQ8>) : go(gemv_mfma_kernel<false, false, kWeightQ8>);
  return hipErrorInvalidValue;
}

// Bins are filled in launch order.  Bin g aims to bring the running cost to
// C * (g + 1) / G (C: the group's total), so a bin that falls short leaves
// the difference to the next one.  A bin takes the combination of windows
// whose cost comes closest to its room without exceeding it; among equal
// totals, the one with more of the costlier windows (those are the hard ones
// to place late).  Combinations are searched costliest class first, with a
// node budget past which the rest of a search takes the largest counts that
// fit; past 32 distinct costs (the search recurses once per cost) every bin
// takes the largest counts that fit, costliest first.  Within a cost class,
// windows go in record order, so a bin holds few runs.  The last bin takes
// whatever is left.
void gemv_mfma_pack(const std::vector<int64_t>& n_win, const std::vector<int64_t>& cost, int64_t groups,
                    std::vector<MfRun>& runs, std::vector<int64_t>& bounds) {
  struct Seg {
    int32_t rec;
    int64_t n;
  };
  struct Cls {
    int64_t c = 0, avail = 0, off = 0;
    size_t si = 0;
    std::vector<Seg> segs;
  };
  std::vector<Cls> cls;
  int64_t C = 0;
  for (size_t r = 0; r < n_win.size(); ++r) {
    if (n_win[r] <= 0) continue;
    size_t k = 0;
    while (k < cls.size() && cls[k].c != cost[r]) ++k;
    if (k == cls.size()) {
      cls.emplace_back();
      cls.back().c = cost[r];
    }
    cls[k].segs.push_back({(int32_t)r, n_win[r]});
    cls[k].avail += n_win[r];
    C += n_win[r] * cost[r];
  }
  std::stable_sort(cls.begin(), cls.end(), [](const Cls& a, const Cls& b) { return a.c > b.c; });
  const int m = (int)cls.size();
  runs.clear();
  bounds.assign(1, 0);
  int64_t placed = 0, n_placed = 0;
  auto take = [&](Cls& k, int64_t cnt) {
    while (cnt > 0) {
      const Seg& sg = k.segs[k.si];
      const int64_t t = std::min(cnt, sg.n - k.off);
      if (!runs.empty() && runs.back().rec == sg.rec && runs.back().first + runs.back().count == k.off)
        runs.back().count += (int32_t)t;
      else
        runs.push_back({sg.rec, (int32_t)k.off, (int32_t)t});
      k.off += t;
      k.avail -= t;
      cnt -= t;
      n_placed += t;
      placed += t * k.c;
      if (k.off == sg.n) {
        ++k.si;
        k.off = 0;
      }
    }
  };
  constexpr int64_t kNodeBudget = 1 << 14;
  constexpr int kMaxSearchClasses = 32;
  std::vector<int64_t> x(m), best(m);
  for (int64_t g = 0; g < groups; ++g) {
    if (g + 1 == groups) {
      for (Cls& k : cls) take(k, k.avail);
    } else {
      const int64_t room = C * (g + 1) / groups - placed;
      int64_t best_sum = -1, nodes = 0;
      auto search = [&](auto&& self, int i, int64_t rem, int64_t sum) -> void {
        if (i == m) {
          if (sum > best_sum) {
            best_sum = sum;
            best = x;
          }
          return;
        }
        const int64_t hi = std::min(cls[i].avail, rem > 0 ? rem / cls[i].c : 0);
        for (int64_t v = hi; v >= 0; --v) {
          x[i] = v;
          self(self, i + 1, rem - v * cls[i].c, sum + v * cls[i].c);
          if (best_sum == room || ++nodes > kNodeBudget) break;
        }
        x[i] = 0;
      };
      if (m <= kMaxSearchClasses) {
        search(search, 0, room, 0);
      } else {
        int64_t rem = room;
        for (int i = 0; i < m; ++i) {
          best[i] = std::min(cls[i].avail, rem > 0 ? rem / cls[i].c : 0);
          rem -= best[i] * cls[i].c;
        }
      }
      for (int i = 0; i < m; ++i) take(cls[i], best[i]);
    }
    bounds.push_back(n_placed);
  }
}

}  // namespace q4q8
