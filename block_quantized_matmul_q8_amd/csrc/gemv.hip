// Streaming Q4 x Q8 matrix x vector kernel for gfx950 (the decode route; the
// mmvq role in "GGML：Backend 抽象与硬件加速", section "CUDA：mmvq、mmq、cublas
// 三条矩阵路": batch-1 decode is a quantised matrix x vector product).
//
// Design:
//   - The B activation columns (codes, scales, and 8 * code sums) are staged
//     once per workgroup in LDS; every weight byte is read exactly once from
//     HBM with 16-byte loads (one whole 32-block per lane; 64 lanes read 1 KiB
//     of one row per instruction, fully coalesced).
//   - Nibbles are unpacked in registers; v_dot4_i32_i8 forms sum q * x on the
//     unsigned codes and the offset is removed with the code sums:
//     I = sum (q - 8) x = sum q x - 8 sum x, exact in int32.
//   - Each wave owns RU rows at a time (independent loads in flight), scales
//     with fp32 fma and finishes each row with a cross-lane butterfly.
#include "common.h"

namespace q4q8 {

constexpr int kGemvThreads = 256;
constexpr int kGemvWaves = kGemvThreads / kWave;
constexpr size_t kGemvMaxLds = 64 * 1024;

template <int B, int RU, bool WRITE_I>
__global__ __launch_bounds__(kGemvThreads) void gemv_kernel(
    const uint8_t* __restrict__ qs, const uint16_t* __restrict__ d, int M, int K,
    const int8_t* __restrict__ xq, const float* __restrict__ xd, float* __restrict__ y,
    int32_t* __restrict__ Iout) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int nb = K / kQK;
  int8_t* sx = reinterpret_cast<int8_t*>(smem);                 // [B][K]
  float* sxd = reinterpret_cast<float*>(smem + (size_t)B * K);  // [B][nb]
  int* sxs = reinterpret_cast<int*>(sxd + B * nb);              // [B][nb], 8 * sum of codes
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;

  {
    const int n16 = B * K / 16;
    const int4* src = reinterpret_cast<const int4*>(xq);
    int4* dst = reinterpret_cast<int4*>(sx);
    for (int i = tid; i < n16; i += kGemvThreads) dst[i] = src[i];
    for (int i = tid; i < B * nb; i += kGemvThreads) sxd[i] = xd[i];
  }
  __syncthreads();
  for (int i = tid; i < B * nb; i += kGemvThreads) {
    const int* p = reinterpret_cast<const int*>(sx + (size_t)i * kQK);
    int s = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) s = __builtin_amdgcn_sdot4(p[k], 0x01010101, s, false);
    sxs[i] = 8 * s;
  }
  __syncthreads();

  const int64_t row_bytes = K / 2;
  const int nwaves = gridDim.x * kGemvWaves;
  for (int row0 = (blockIdx.x * kGemvWaves + wave) * RU; row0 < M; row0 += nwaves * RU) {
    float acc[RU][B];
#pragma unroll
    for (int r = 0; r < RU; ++r)
#pragma unroll
      for (int c = 0; c < B; ++c) acc[r][c] = 0.0f;

    for (int b0 = 0; b0 < nb; b0 += kWave) {
      const int b = b0 + lane;
      if (b < nb) {
        uint4 w[RU];
        float dw[RU];
#pragma unroll
        for (int r = 0; r < RU; ++r) {
          const int row = row0 + r;
          if (row < M) {
            w[r] = *reinterpret_cast<const uint4*>(qs + row * row_bytes + (int64_t)b * 16);
            dw[r] = f16_bits_to_f32(d[(int64_t)row * nb + b]);
          } else {
            w[r] = make_uint4(0, 0, 0, 0);
            dw[r] = 0.0f;
          }
        }
#pragma unroll
        for (int c = 0; c < B; ++c) {
          const int4* xp = reinterpret_cast<const int4*>(sx + (size_t)c * K + (size_t)b * kQK);
          const int4 xa = xp[0], xb = xp[1];
          const float xdc = sxd[c * nb + b];
          const int xsc = sxs[c * nb + b];
#pragma unroll
          for (int r = 0; r < RU; ++r) {
            const int I = dot_block(w[r], xa, xb) - xsc;
            acc[r][c] = __builtin_fmaf((float)I, dw[r] * xdc, acc[r][c]);
            if (WRITE_I) {
              const int row = row0 + r;
              if (row < M) Iout[((int64_t)c * M + row) * nb + b] = I;
            }
          }
        }
      }
    }
#pragma unroll
    for (int r = 0; r < RU; ++r)
#pragma unroll
      for (int c = 0; c < B; ++c) {
        const float v = wave_sum(acc[r][c]);
        const int row = row0 + r;
        if (lane == 0 && row < M) y[(int64_t)c * M + row] = v;
      }
  }
}

static size_t gemv_lds_bytes(int64_t K, int64_t B) {
  const int64_t nb = K / kQK;
  return (size_t)(B * K + 8 * B * nb);
}

bool gemv_supported(int64_t M, int64_t K, int64_t B) {
  (void)M;
  return B >= 1 && B <= 4 && gemv_lds_bytes(K, B) <= kGemvMaxLds;
}

template <int B, int RU>
static hipError_t launch_gemv_t(const uint8_t* qs, const uint16_t* d, int64_t M, int64_t K,
                                const int8_t* xq, const float* xd, float* y, int32_t* I,
                                hipStream_t s) {
  const size_t lds = gemv_lds_bytes(K, B);
  const int64_t groups = (M + RU - 1) / RU;
  int64_t grid = (groups + kGemvWaves - 1) / kGemvWaves;
  if (grid > 1024) grid = 1024;
  if (I)
    hipLaunchKernelGGL((gemv_kernel<B, RU, true>), dim3((unsigned)grid), dim3(kGemvThreads), lds,
                       s, qs, d, (int)M, (int)K, xq, xd, y, I);
  else
    hipLaunchKernelGGL((gemv_kernel<B, RU, false>), dim3((unsigned)grid), dim3(kGemvThreads),
                       lds, s, qs, d, (int)M, (int)K, xq, xd, y, I);
  return hipGetLastError();
}

hipError_t launch_gemv(const uint8_t* qs, const uint16_t* d, int64_t M, int64_t K,
                       const int8_t* xq, const float* xd, int64_t B, float* y, int32_t* I,
                       hipStream_t s) {
  switch (B) {
    case 1: return launch_gemv_t<1, 4>(qs, d, M, K, xq, xd, y, I, s);
    case 2: return launch_gemv_t<2, 4>(qs, d, M, K, xq, xd, y, I, s);
    case 3: return launch_gemv_t<3, 2>(qs, d, M, K, xq, xd, y, I, s);
    case 4: return launch_gemv_t<4, 2>(qs, d, M, K, xq, xd, y, I, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace q4q8
