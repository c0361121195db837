// Int8-MFMA Q4 x Q8 matrix kernel for gfx950 (the prefill route; the mmq role
// in "GGML：Backend 抽象与硬件加速", section "CUDA：mmvq、mmq、cublas 三条
// 矩阵路": larger quantised products go to a tiled matrix kernel).
//
// One v_mfma_i32_32x32x32_i8 covers exactly one 32-element quantisation block,
// so its int32 result is the exact block sum I for a 32 x 32 output tile.  The
// accumulator input is seeded with the bits of 1.5 * 2^23: the result read as
// fp32 is F = 1.5 * 2^23 + I exactly, and the per-block rescale is two fp32
// fmas per output element: t = fma(F, d_w, -1.5 * 2^23 * d_w) = fl(I * d_w),
// acc = fma(t, d_x, acc).
//
// Operand roles: A = activations (MFMA rows = tokens), B = weights (MFMA
// columns = weight rows).  Each lane then holds one weight row (one d_w per
// lane) and 16 token rows, and the output y[token][row] is stored with
// consecutive lanes on consecutive rows.
//
// Tiling: a workgroup of 4 waves computes 128 weight rows x 128 tokens; each
// wave a 64 x 64 quadrant (2 x 2 MFMA tiles).  Per LDS stage, two 32-blocks of
// K: weight nibbles are unpacked to signed int8 once per stage and shared by
// all 128 tokens.
#include "common.h"

namespace q4q8 {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kTM = 128;  // weight rows per workgroup
constexpr int kTN = 128;  // tokens per workgroup
constexpr int kKB = 2;    // 32-blocks per LDS stage
constexpr int kGemmThreads = 256;

__device__ __forceinline__ uint32_t nib_to_s8(uint32_t n) {
  // bytes in [0,15] -> signed bytes n - 8 (no carries cross byte lanes)
  return (n + 0x78787878u) ^ 0x80808080u;
}

template <bool WRITE_I>
__global__ __launch_bounds__(kGemmThreads) void gemm_kernel(
    const uint8_t* __restrict__ qs, const uint16_t* __restrict__ d, int M, int K,
    const int8_t* __restrict__ xq, const float* __restrict__ xd, int B, float* __restrict__ y,
    int32_t* __restrict__ Iout) {
  __shared__ __align__(16) int8_t sA[kKB][kTN][kQK];
  __shared__ __align__(16) int8_t sW[kKB][kTM][kQK];
  __shared__ __align__(16) float sDX[kKB][kTN];
  __shared__ float sDW[kKB][kTM];
  __shared__ float sCW[kKB][kTM];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wt = wave >> 1, ww = wave & 1;
  const int m0 = blockIdx.x * kTM, n0 = blockIdx.y * kTN;
  const int nb = K / kQK;
  const int64_t row_bytes = K / 2;
  const int l32 = lane & 31, h = lane >> 5;

  float acc[2][2][16];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  v16i seed;
#pragma unroll
  for (int r = 0; r < 16; ++r) seed[r] = kMagicBits;

  for (int kb0 = 0; kb0 < nb; kb0 += kKB) {
    {
      // activations: thread -> (token row, half) for each stage block
      const int ar = tid >> 1, ah = tid & 1;
#pragma unroll
      for (int blk = 0; blk < kKB; ++blk) {
        const int kb = kb0 + blk;
        int4 v = make_int4(0, 0, 0, 0);
        if (kb < nb && n0 + ar < B)
          v = *reinterpret_cast<const int4*>(xq + (int64_t)(n0 + ar) * K + kb * kQK + ah * 16);
        *reinterpret_cast<int4*>(&sA[blk][ar][ah * 16]) = v;
      }
      // weights: thread -> (weight row, stage block)
      const int wr = tid & (kTM - 1), wb = tid / kTM;
      const int kb = kb0 + wb;
      uint4 q = make_uint4(0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u);
      float dwv = 0.0f;
      if (kb < nb && m0 + wr < M) {
        q = *reinterpret_cast<const uint4*>(qs + (int64_t)(m0 + wr) * row_bytes + (int64_t)kb * 16);
        dwv = f16_bits_to_f32(d[(int64_t)(m0 + wr) * nb + kb]);
      }
      const uint32_t m4 = 0x0F0F0F0Fu;
      uint4 lo = make_uint4(nib_to_s8(q.x & m4), nib_to_s8(q.y & m4), nib_to_s8(q.z & m4),
                            nib_to_s8(q.w & m4));
      uint4 hi = make_uint4(nib_to_s8((q.x >> 4) & m4), nib_to_s8((q.y >> 4) & m4),
                            nib_to_s8((q.z >> 4) & m4), nib_to_s8((q.w >> 4) & m4));
      *reinterpret_cast<uint4*>(&sW[wb][wr][0]) = lo;
      *reinterpret_cast<uint4*>(&sW[wb][wr][16]) = hi;
      sDW[wb][wr] = dwv;
      sCW[wb][wr] = -kMagic * dwv;
      // token scales: thread -> (token row, stage block)
      float dxv = 0.0f;
      if (kb < nb && n0 + wr < B) dxv = xd[(int64_t)(n0 + wr) * nb + kb];
      sDX[wb][wr] = dxv;
    }
    __syncthreads();

#pragma unroll
    for (int blk = 0; blk < kKB; ++blk) {
      const int kb = kb0 + blk;
      if (kb < nb) {
        v4i a[2], b[2];
        float dw[2], cw[2];
        float dx[2][16];
#pragma unroll
        for (int it = 0; it < 2; ++it)
          a[it] = *reinterpret_cast<const v4i*>(&sA[blk][wt * 64 + it * 32 + l32][16 * h]);
#pragma unroll
        for (int jt = 0; jt < 2; ++jt) {
          const int wrow = ww * 64 + jt * 32 + l32;
          b[jt] = *reinterpret_cast<const v4i*>(&sW[blk][wrow][16 * h]);
          dw[jt] = sDW[blk][wrow];
          cw[jt] = sCW[blk][wrow];
        }
#pragma unroll
        for (int it = 0; it < 2; ++it)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const float4 v =
                *reinterpret_cast<const float4*>(&sDX[blk][wt * 64 + it * 32 + 8 * g + 4 * h]);
            dx[it][4 * g + 0] = v.x;
            dx[it][4 * g + 1] = v.y;
            dx[it][4 * g + 2] = v.z;
            dx[it][4 * g + 3] = v.w;
          }
#pragma unroll
        for (int it = 0; it < 2; ++it)
#pragma unroll
          for (int jt = 0; jt < 2; ++jt) {
            const v16i D = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[it], b[jt], seed, 0, 0, 0);
            // Reinterpret the whole result vector at once: hipcc (ROCm 7.2)
            // miscompiles a per-element int -> float bit cast of an MFMA
            // result, propagating element 0 to every element.
            const v16f Fv = __builtin_bit_cast(v16f, D);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const float F = Fv[r];
              const float t = __builtin_fmaf(F, dw[jt], cw[jt]);
              acc[it][jt][r] = __builtin_fmaf(t, dx[it][r], acc[it][jt][r]);
              if (WRITE_I) {
                const int n = n0 + wt * 64 + it * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                const int m = m0 + ww * 64 + jt * 32 + l32;
                if (n < B && m < M) Iout[((int64_t)n * M + m) * nb + kb] = D[r] - kMagicBits;
              }
            }
          }
      }
    }
    __syncthreads();
  }

#pragma unroll
  for (int it = 0; it < 2; ++it)
#pragma unroll
    for (int jt = 0; jt < 2; ++jt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int n = n0 + wt * 64 + it * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        const int m = m0 + ww * 64 + jt * 32 + l32;
        if (n < B && m < M) y[(int64_t)n * M + m] = acc[it][jt][r];
      }
}

hipError_t launch_gemm(const uint8_t* qs, const uint16_t* d, int64_t M, int64_t K,
                       const int8_t* xq, const float* xd, int64_t B, float* y, int32_t* I,
                       hipStream_t s) {
  const dim3 grid((unsigned)((M + kTM - 1) / kTM), (unsigned)((B + kTN - 1) / kTN));
  if (I)
    hipLaunchKernelGGL(gemm_kernel<true>, grid, dim3(kGemmThreads), 0, s, qs, d, (int)M, (int)K,
                       xq, xd, (int)B, y, I);
  else
    hipLaunchKernelGGL(gemm_kernel<false>, grid, dim3(kGemmThreads), 0, s, qs, d, (int)M, (int)K,
                       xq, xd, (int)B, y, I);
  return hipGetLastError();
}

}  // namespace q4q8
