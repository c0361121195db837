// Quantisation kernels for gfx950: load-time Q4 weight quantisation and the
// fused RMSNorm * g -> Q8 activation prologue.
//
// Both produce codes and scales that must match a sequential fp32 reference
// bit for bit, so every floating-point step is a single IEEE-rounded operation
// (explicit __f*_rn intrinsics, and the file is built without FMA
// contraction); the reduction order of the RMS statistic is fixed (see
// rmsnorm_q8_kernel).
#include "prologue_dev.h"

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
  note_launch((const void*)q4_quantize_kernel);
  hipLaunchKernelGGL(q4_quantize_kernel, dim3((unsigned)grid), dim3(256), 0, s, w, M, K, qs, d);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// fp32 weights -> Q8_0 blocks (32 int8 codes, fp16 scale), one thread per
// block.  The codes follow the Q8 block rule with the fp32 scale; the stored
// scale is that scale rounded to fp16 (the Q8_0 type of "GGML：Backend 抽象与
// 硬件加速", sections "Metal 与 Vulkan：默认路径和生成路径" and "对照本栈",
// read as 32-element blocks with an fp16 scale).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void q8w_quantize_kernel(const float* __restrict__ w, int64_t M, int64_t K,
                                                           int8_t* __restrict__ qw, uint16_t* __restrict__ d) {
  const int64_t nb = K / kQK;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= M * nb) return;
  const int64_t row = idx / nb, b = idx - row * nb;
  float v[kQK];
  load_block32(w + row * K + b * kQK, v);
  uint32_t packed[8];
  float dd;
  int sum;
  q8_pack_block(v, packed, dd, sum);
  uint4* dst = reinterpret_cast<uint4*>(qw + row * K + b * kQK);
  dst[0] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
  dst[1] = make_uint4(packed[4], packed[5], packed[6], packed[7]);
  d[row * nb + b] = f32_to_f16_bits_rne(dd);
}

hipError_t launch_q8w_quantize(const float* w, int64_t M, int64_t K, int8_t* qw, uint16_t* d, hipStream_t s) {
  const int64_t n = M * (K / kQK);
  const int64_t grid = (n + 255) / 256;
  note_launch((const void*)q8w_quantize_kernel);
  hipLaunchKernelGGL(q8w_quantize_kernel, dim3((unsigned)grid), dim3(256), 0, s, w, M, K, qw, d);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Fused RMSNorm * g -> Q8 (standalone prologue).  One workgroup per activation
// row; the steps and their order are those of prologue_dev.h.  Rows of up to
// 16384 elements take the register form (one pass over x), longer rows the
// LDS-tree form; both give the same bits.  With no_norm the row is quantised
// as it is.
// ---------------------------------------------------------------------------
constexpr int kPrologueThreads = 256;
// Grouped calls of up to this many columns (decode) take the 1024-thread
// prologue workgroups; wider ones (prefill) the 256-thread ones, whose total
// instruction count is lower.
constexpr int kWidePrologueMaxB = 8;

__global__ __launch_bounds__(kPrologueThreads) void rmsnorm_q8_kernel(
    const float* __restrict__ x, int K, const float* __restrict__ g, float eps, int no_norm,
    int P, int8_t* __restrict__ xq, float* __restrict__ xd, int32_t* __restrict__ xs,
    const float* __restrict__ a, int64_t a_row_stride) {
  extern __shared__ float red[];  // 2 * P floats (long rows only)
  __shared__ float s_slot;
  __shared__ float groups[8];
  const int nb = K / kQK;
  const int64_t row = blockIdx.x;
  const float* xr = x + row * (int64_t)K;
  const int tid = threadIdx.x;
  const float* ar = a ? a + row * a_row_stride : nullptr;
  if (K <= kFastPrologueK) {
    wg_q8_row_fast(xr, g, K, eps, no_norm != 0, xq + row * (int64_t)K, xd + row * nb,
                   xs ? xs + row * nb : nullptr, groups, tid, ar);
    return;
  }
  const float s = no_norm ? 1.0f : wg_rms_scale(xr, K, eps, P, red, &s_slot, tid, kPrologueThreads);
  for (int b = tid; b < nb; b += kPrologueThreads) {
    uint32_t packed[8];
    float dd;
    int sum;
    q8_block_codes(xr, g, b, s, no_norm != 0, packed, dd, sum, ar);
    uint4* dst = reinterpret_cast<uint4*>(xq + row * (int64_t)K + b * kQK);
    dst[0] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
    dst[1] = make_uint4(packed[4], packed[5], packed[6], packed[7]);
    xd[row * nb + b] = dd;
    if (xs) xs[row * nb + b] = sum;
  }
}

// The standalone prologue for a few rows (decode): one 1024-thread
// workgroup per row, the forms of group_prologue_wide_kernel.
__global__ __launch_bounds__(kWideThreads) void rmsnorm_q8_wide_kernel(
    const float* __restrict__ x, int K, const float* __restrict__ g, float eps, int no_norm, int P,
    int8_t* __restrict__ xq, float* __restrict__ xd, int32_t* __restrict__ xs, const float* __restrict__ a,
    int64_t a_row_stride) {
  extern __shared__ float red[];  // 2 * P floats (rows beyond 32768 elements only)
  __shared__ float s_slot;
  __shared__ float groups[kWideWaves];
  const int nb = K / kQK;
  const int64_t row = blockIdx.x;
  const float* xr = x + row * (int64_t)K;
  const int tid = threadIdx.x;
  const float* ar = a ? a + row * a_row_stride : nullptr;
  int8_t* xqr = xq + row * (int64_t)K;
  float* xdr = xd + row * nb;
  int32_t* xsr = xs ? xs + row * nb : nullptr;
  if (K <= kWideMaxK && tid / kWave >= wide_active_waves(K)) return;  // holds no lane of the row
  if (K <= kQuadMaxK) {
    wide_q8_row_lanes<4>(xr, g, K, eps, no_norm != 0, xqr, xdr, xsr, groups, tid, ar);
    return;
  }
  if (K <= kPairMaxK) {
    wide_q8_row_lanes<2>(xr, g, K, eps, no_norm != 0, xqr, xdr, xsr, groups, tid, ar);
    return;
  }
  if (K <= kWideMaxK) {
    wide_q8_row_single(xr, g, K, eps, no_norm != 0, xqr, xdr, xsr, groups, tid, ar);
    return;
  }
  const float s = no_norm ? 1.0f : wg_rms_scale(xr, K, eps, P, red, &s_slot, tid, kWideThreads);
  for (int b = tid; b < nb; b += kWideThreads) {
    uint32_t packed[8];
    float dd;
    int sum;
    q8_block_codes(xr, g, b, s, no_norm != 0, packed, dd, sum, ar);
    uint4* dst = reinterpret_cast<uint4*>(xqr + b * kQK);
    dst[0] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
    dst[1] = make_uint4(packed[4], packed[5], packed[6], packed[7]);
    xdr[b] = dd;
    if (xsr) xsr[b] = sum;
  }
}

hipError_t launch_q8_rmsnorm(const float* x, int64_t B, int64_t K, const float* g, float eps,
                             bool no_norm, int8_t* xq, float* xd, int32_t* xs, hipStream_t s,
                             const float* a, int64_t a_row_stride) {
  const int P = next_pow2_int((int)(K / kQK));
  if (B <= kWidePrologueMaxB) {
    const size_t lds = (no_norm || K <= kWideMaxK) ? 0 : 2 * (size_t)P * sizeof(float);
    note_launch((const void*)rmsnorm_q8_wide_kernel);
    hipLaunchKernelGGL(rmsnorm_q8_wide_kernel, dim3((unsigned)B), dim3(kWideThreads), lds, s, x, (int)K, g, eps,
                       no_norm ? 1 : 0, P, xq, xd, xs, a, a_row_stride);
    return hipGetLastError();
  }
  const size_t lds = (no_norm || K <= kFastPrologueK) ? 0 : 2 * (size_t)P * sizeof(float);
  note_launch((const void*)rmsnorm_q8_kernel);
  hipLaunchKernelGGL(rmsnorm_q8_kernel, dim3((unsigned)B), dim3(kPrologueThreads), lds, s, x,
                     (int)K, g, eps, no_norm ? 1 : 0, P, xq, xd, xs, a, a_row_stride);
  return hipGetLastError();
}

// SwiGLU -> Q8 (the producer of the down projection's input): eight lanes
// per (row, 32-block), four elements each; h = fl(silu(gate) * up), then
// the Q8 block rule with the block's amax and code sum combined over the
// eight lanes by DPP (quad swaps, then the mirror within each half-row of 8
// lanes).  Rows of gate and up start row_stride floats apart (a stacked
// [B][2F] gate|up buffer: gate = buffer, up = buffer + F, row_stride = 2F).
__global__ __launch_bounds__(256) void swiglu_q8_kernel(const float* __restrict__ gate,
                                                        const float* __restrict__ up, int64_t B, int64_t F,
                                                        int64_t row_stride, int8_t* __restrict__ xq,
                                                        float* __restrict__ xd, int32_t* __restrict__ xs) {
  const int64_t nb = F / kQK;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t blk = idx >> 3;
  const int part = (int)(idx & 7);
  if (blk >= B * nb) return;  // whole groups of eight lanes leave together
  const int64_t row = blk / nb, b = blk - row * nb;
  const f32x4 gv = *gptr(reinterpret_cast<const f32x4*>(gate + row * row_stride + b * kQK + 4 * part));
  const f32x4 uv = *gptr(reinterpret_cast<const f32x4*>(up + row * row_stride + b * kQK + 4 * part));
  float v[4];
  v[0] = __fmul_rn(silu_q(gv.x), uv.x);
  v[1] = __fmul_rn(silu_q(gv.y), uv.y);
  v[2] = __fmul_rn(silu_q(gv.z), uv.z);
  v[3] = __fmul_rn(silu_q(gv.w), uv.w);
  float m = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
  m = quad_max(m);
  m = fmaxf(m, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, m), 0x141, 0xF,
                                                                      0xF, false)));
  const float d = __fdiv_rn(m, 127.0f);
  const float id = d != 0.0f ? __fdiv_rn(1.0f, d) : 0.0f;
  uint32_t word = 0;
  int csum = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    int qi = round_half_away_i32(__fmul_rn(v[k], id));
    qi = qi > 127 ? 127 : (qi < -127 ? -127 : qi);
    csum += qi;
    word |= ((uint32_t)qi & 0xFFu) << (8 * k);
  }
  gptr_w(reinterpret_cast<uint32_t*>(xq + row * F + b * kQK + 4 * part))[0] = word;
  if (xs) {
    csum += __builtin_amdgcn_update_dpp(0, csum, 0xB1, 0xF, 0xF, false);
    csum += __builtin_amdgcn_update_dpp(0, csum, 0x4E, 0xF, 0xF, false);
    csum += __builtin_amdgcn_update_dpp(0, csum, 0x141, 0xF, 0xF, false);
  }
  if (part == 0) {
    gptr_w(xd)[row * nb + b] = d;
    if (xs) gptr_w(xs)[row * nb + b] = csum;
  }
}

hipError_t launch_swiglu_q8(const float* gate, const float* up, int64_t B, int64_t F, int64_t row_stride,
                            int8_t* xq, float* xd, int32_t* xs, hipStream_t s) {
  const int64_t n = B * (F / kQK) * 8;
  note_launch((const void*)swiglu_q8_kernel);
  hipLaunchKernelGGL(swiglu_q8_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, gate, up, B, F,
                     row_stride, xq, xd, xs);
  return hipGetLastError();
}

// Prologue pass of a grouped launch: workgroup (j, c) quantises row c of the
// fp32 input of job j into the job's Q8 planes, in the register form for
// rows of up to 16384 elements and the LDS-tree form beyond (dynamic LDS of
// 2 * next_pow2(K / 32) floats for the longest row of the launch).
__global__ __launch_bounds__(kPrologueThreads) void group_prologue_kernel(
    const PrologueJob* __restrict__ jobs) {
  extern __shared__ float red[];
  __shared__ float s_slot;
  __shared__ float groups[8];
  const PrologueJob& J = jobs[blockIdx.x];
  const int c = blockIdx.y;
  const int K = J.K, nb = K / kQK, tid = threadIdx.x;
  const float* xr = J.x + (int64_t)c * K;
  int8_t* xq = J.xq + (int64_t)c * K;
  float* xd = J.xd + (int64_t)c * nb;
  if (K <= kFastPrologueK) {
    wg_q8_row_fast(xr, J.g, K, J.eps, J.raw != 0, xq, xd, nullptr, groups, tid);
    return;
  }
  const int P = next_pow2_int(nb);
  const float s = J.raw ? 1.0f : wg_rms_scale(xr, K, J.eps, P, red, &s_slot, tid, kPrologueThreads);
  for (int b = tid; b < nb; b += kPrologueThreads) {
    uint32_t packed[8];
    float dd;
    int sum;
    q8_block_codes(xr, J.g, b, s, J.raw != 0, packed, dd, sum);
    uint4* dst = reinterpret_cast<uint4*>(xq + b * kQK);
    dst[0] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
    dst[1] = make_uint4(packed[4], packed[5], packed[6], packed[7]);
    xd[b] = dd;
  }
}

// The same pass for a few columns (decode): 1024-thread workgroups, so that
// each row's serial stretches are short -- four lanes per block up to K =
// 8192, two up to 16384, one up to 32768, the LDS-tree form beyond.
__global__ __launch_bounds__(kWideThreads) void group_prologue_wide_kernel(const PrologueJob* __restrict__ jobs) {
  extern __shared__ float red[];
  __shared__ float s_slot;
  __shared__ float groups[kWideWaves];
  const PrologueJob& J = jobs[blockIdx.x];
  const int c = blockIdx.y;
  const int K = J.K, nb = K / kQK, tid = threadIdx.x;
  const float* xr = J.x + (int64_t)c * K;
  int8_t* xq = J.xq + (int64_t)c * K;
  float* xd = J.xd + (int64_t)c * nb;
  if (K <= kWideMaxK && tid / kWave >= wide_active_waves(K)) return;  // holds no lane of the row
  if (K <= kQuadMaxK) {
    wide_q8_row_lanes<4>(xr, J.g, K, J.eps, J.raw != 0, xq, xd, nullptr, groups, tid);
    return;
  }
  if (K <= kPairMaxK) {
    wide_q8_row_lanes<2>(xr, J.g, K, J.eps, J.raw != 0, xq, xd, nullptr, groups, tid);
    return;
  }
  if (K <= kWideMaxK) {
    wide_q8_row_single(xr, J.g, K, J.eps, J.raw != 0, xq, xd, nullptr, groups, tid);
    return;
  }
  const int P = next_pow2_int(nb);
  const float s = J.raw ? 1.0f : wg_rms_scale(xr, K, J.eps, P, red, &s_slot, tid, kWideThreads);
  for (int b = tid; b < nb; b += kWideThreads) {
    uint32_t packed[8];
    float dd;
    int sum;
    q8_block_codes(xr, J.g, b, s, J.raw != 0, packed, dd, sum);
    uint4* dst = reinterpret_cast<uint4*>(xq + b * kQK);
    dst[0] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
    dst[1] = make_uint4(packed[4], packed[5], packed[6], packed[7]);
    xd[b] = dd;
  }
}

hipError_t launch_group_prologue(const PrologueJob* jobs, int64_t n_jobs, int64_t B, int64_t max_k,
                                 hipStream_t s) {
  if (B <= kWidePrologueMaxB) {
    const size_t lds = max_k > kWideMaxK ? 2 * (size_t)next_pow2_int((int)(max_k / kQK)) * sizeof(float) : 0;
    note_launch((const void*)group_prologue_wide_kernel);
    hipLaunchKernelGGL(group_prologue_wide_kernel, dim3((unsigned)n_jobs, (unsigned)B), dim3(kWideThreads), lds,
                       s, jobs);
    return hipGetLastError();
  }
  const size_t lds = max_k > kFastPrologueK ? 2 * (size_t)next_pow2_int((int)(max_k / kQK)) * sizeof(float) : 0;
  note_launch((const void*)group_prologue_kernel);
  hipLaunchKernelGGL(group_prologue_kernel, dim3((unsigned)n_jobs, (unsigned)B), dim3(kPrologueThreads), lds,
                     s, jobs);
  return hipGetLastError();
}

}  // namespace q4q8
