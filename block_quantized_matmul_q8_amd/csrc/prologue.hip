// Quantisation kernels for gfx950: load-time Q4 weight quantisation and the
// fused RMSNorm * g -> Q8 activation prologue.
//
// Both produce codes and scales that must match a sequential fp32 reference
// bit for bit, so every floating-point step is a single IEEE-rounded operation
// (explicit __f*_rn intrinsics, and the file is built without FMA
// contraction); the reduction order of the RMS statistic is fixed (see
// rmsnorm_q8_kernel).
#include "common.h"

namespace q4q8 {

// ---------------------------------------------------------------------------
// Q4 quantisation.  One thread per (row, 32-block).  The block rule:
//   amax = max |w|; m = element of lowest index with |w| = amax;
//   d = m / -8; id = 1 / d; q = clamp(trunc(w * id + 8.5), 0, 15);
//   stored scale fp16(d) (RNE); all-zero block -> d = +0, codes 8.
// Packing: byte j of the block = code j | code (j + 16) << 4.
// (Load-time re-layout into kernel-friendly planes: "GGML：Backend 抽象与硬件
// 加速", section "构建开关如何变成运行时能力".)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void q4_quantize_kernel(const float* __restrict__ w, int64_t M,
                                                          int64_t K, uint8_t* __restrict__ qs,
                                                          uint16_t* __restrict__ d) {
  const int64_t nb = K / kQK;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= M * nb) return;
  const int64_t row = idx / nb, b = idx - row * nb;
  const float4* src = reinterpret_cast<const float4*>(w + row * K + b * kQK);
  float v[kQK];
#pragma unroll
  for (int i = 0; i < kQK / 4; ++i) {
    const float4 t = src[i];
    v[4 * i + 0] = t.x;
    v[4 * i + 1] = t.y;
    v[4 * i + 2] = t.z;
    v[4 * i + 3] = t.w;
  }
  float amax = 0.0f, mval = 0.0f;
#pragma unroll
  for (int j = 0; j < kQK; ++j) {
    const float a = fabsf(v[j]);
    if (a > amax) {  // strict: the lowest index wins a tie
      amax = a;
      mval = v[j];
    }
  }
  uint32_t packed[4];
  uint16_t dbits;
  if (amax == 0.0f) {
    dbits = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) packed[i] = 0x88888888u;
  } else {
    const float dd = __fdiv_rn(mval, -8.0f);
    const float id = __fdiv_rn(1.0f, dd);
    uint32_t q[kQK];
#pragma unroll
    for (int j = 0; j < kQK; ++j) {
      const float t = __fadd_rn(__fmul_rn(v[j], id), 8.5f);
      int qi = (int)t;  // truncation toward zero
      qi = qi > 15 ? 15 : qi;
      qi = qi < 0 ? 0 : qi;
      q[j] = (uint32_t)qi;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t word = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int j = 4 * i + k;
        word |= (q[j] | (q[j + 16] << 4)) << (8 * k);
      }
      packed[i] = word;
    }
    dbits = f32_to_f16_bits_rne(dd);
  }
  *reinterpret_cast<uint4*>(qs + row * (K / 2) + b * (kQK / 2)) =
      make_uint4(packed[0], packed[1], packed[2], packed[3]);
  d[row * nb + b] = dbits;
}

hipError_t launch_q4_quantize(const float* w, int64_t M, int64_t K, uint8_t* qs, uint16_t* d,
                              hipStream_t s) {
  const int64_t n = M * (K / kQK);
  const int64_t grid = (n + 255) / 256;
  hipLaunchKernelGGL(q4_quantize_kernel, dim3((unsigned)grid), dim3(256), 0, s, w, M, K, qs, d);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Fused RMSNorm * g -> Q8.  One workgroup per activation row.
//   Phase 1: thread b computes p_b = sum_{j<32} x_j^2 for block b, adding in
//            index order (one rounding per multiply and per add).
//   Phase 2: p is padded with +0 to P = next_pow2(nb) and reduced pairwise,
//            level by level: p[i] = p[2i] + p[2i+1] (ping-pong LDS buffers).
//   Phase 3: s = 1 / sqrt(ssq / K + eps) (correctly rounded div and sqrt;
//            see sqrt_rn).
//   Phase 4: v = (x * s) * g; per block d = amax / 127, id = 1 / d,
//            q = roundf(v * id) (halves away from zero), clamp +-127.
// The two roundings of phase 4 keep the fused kernel equal to the unfused
// RMS_NORM then MUL pair ("llama.cpp b10909：Metal后端融合表重构..." restores
// exactly that fusion).  With no_norm the row is quantised as it is.
// ---------------------------------------------------------------------------
constexpr int kPrologueThreads = 256;

__device__ __forceinline__ void load_block32(const float* p, float (&v)[kQK]) {
  const float4* s = reinterpret_cast<const float4*>(p);
#pragma unroll
  for (int i = 0; i < kQK / 4; ++i) {
    const float4 t = s[i];
    v[4 * i + 0] = t.x;
    v[4 * i + 1] = t.y;
    v[4 * i + 2] = t.z;
    v[4 * i + 3] = t.w;
  }
}

__global__ __launch_bounds__(kPrologueThreads) void rmsnorm_q8_kernel(
    const float* __restrict__ x, int K, const float* __restrict__ g, float eps, int no_norm,
    int P, int8_t* __restrict__ xq, float* __restrict__ xd, int32_t* __restrict__ xs) {
  extern __shared__ float red[];  // 2 * P floats
  __shared__ float s_scale;
  const int nb = K / kQK;
  const int64_t row = blockIdx.x;
  const float* xr = x + row * (int64_t)K;
  const int tid = threadIdx.x;

  float s = 1.0f;
  if (!no_norm) {
    for (int b = tid; b < P; b += kPrologueThreads) {
      float acc = 0.0f;
      if (b < nb) {
        float v[kQK];
        load_block32(xr + b * kQK, v);
#pragma unroll
        for (int j = 0; j < kQK; ++j) acc = __fadd_rn(acc, __fmul_rn(v[j], v[j]));
      }
      red[b] = acc;
    }
    __syncthreads();
    float* src = red;
    float* dst = red + P;
    for (int h = P / 2; h >= 1; h /= 2) {
      for (int i = tid; i < h; i += kPrologueThreads) dst[i] = __fadd_rn(src[2 * i], src[2 * i + 1]);
      __syncthreads();
      float* t = src;
      src = dst;
      dst = t;
    }
    if (tid == 0) {
      const float mean = __fdiv_rn(src[0], (float)K);
      const float r = sqrt_rn(__fadd_rn(mean, eps));
      s_scale = __fdiv_rn(1.0f, r);
    }
    __syncthreads();
    s = s_scale;
  }

  for (int b = tid; b < nb; b += kPrologueThreads) {
    float v[kQK];
    load_block32(xr + b * kQK, v);
    if (!no_norm) {
      float gv[kQK];
      load_block32(g + b * kQK, gv);
#pragma unroll
      for (int j = 0; j < kQK; ++j) v[j] = __fmul_rn(__fmul_rn(v[j], s), gv[j]);
    }
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < kQK; ++j) amax = fmaxf(amax, fabsf(v[j]));
    const float dd = __fdiv_rn(amax, 127.0f);
    const float id = dd != 0.0f ? __fdiv_rn(1.0f, dd) : 0.0f;
    int sum = 0;
    uint32_t packed[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t word = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        int qi = (int)roundf(__fmul_rn(v[4 * i + k], id));
        qi = qi > 127 ? 127 : (qi < -127 ? -127 : qi);
        sum += qi;
        word |= ((uint32_t)qi & 0xFFu) << (8 * k);
      }
      packed[i] = word;
    }
    uint4* dst = reinterpret_cast<uint4*>(xq + row * (int64_t)K + b * kQK);
    dst[0] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
    dst[1] = make_uint4(packed[4], packed[5], packed[6], packed[7]);
    xd[row * nb + b] = dd;
    if (xs) xs[row * nb + b] = sum;
  }
}

hipError_t launch_q8_rmsnorm(const float* x, int64_t B, int64_t K, const float* g, float eps,
                             bool no_norm, int8_t* xq, float* xd, int32_t* xs, hipStream_t s) {
  const int nb = (int)(K / kQK);
  int P = 1;
  while (P < nb) P *= 2;
  const size_t lds = no_norm ? 0 : 2 * (size_t)P * sizeof(float);
  hipLaunchKernelGGL(rmsnorm_q8_kernel, dim3((unsigned)B), dim3(kPrologueThreads), lds, s, x,
                     (int)K, g, eps, no_norm ? 1 : 0, P, xq, xd, xs);
  return hipGetLastError();
}

}  // namespace q4q8
