// Expert-routed Q4 x Q8 product (MUL_MAT_ID) for gfx950.
//
// "GGML：Backend 抽象与硬件加速", section "调度器三遍切图，pipeline 四个副本":
// an expert matmul only touches the expert slices that are actually used.
// Here that holds on one device: the routing runs on the GPU (no host sync)
// and the grouped product launches a workgroup grid over (row tile, expert)
// whose workgroups for unselected experts exit before reading any weight.
//
// Workspace layout (int32): offsets[E + 1] | list[n] | rank[n], n = T * top_k.
//   list holds, grouped by expert, the flat (token, slot) index t * top_k + s
//   of every routed pair; the order inside a group is not fixed, and does not
//   matter because every output element is computed independently.
#include "common.h"

namespace q4q8 {

constexpr int kRouteThreads = 1024;
constexpr int kMoeThreads = 256;
constexpr int kMoeWaves = kMoeThreads / kWave;
constexpr int kMoeCols = 4;      // routed columns staged per pass
constexpr int kMoeRowsPerWg = 64;
constexpr int kMoeRU = 2;        // rows per wave in flight

size_t moe_workspace_bytes(int64_t E, int64_t T, int64_t top_k) {
  const size_t n = (size_t)(T * top_k);
  const size_t words = (size_t)E + 1 + 2 * n;
  return (words * sizeof(int32_t) + 15) & ~(size_t)15;
}

__global__ __launch_bounds__(kRouteThreads) void moe_route_kernel(
    const int32_t* __restrict__ ids, int n, int E, int M, int32_t* __restrict__ offsets,
    int32_t* __restrict__ list, int32_t* __restrict__ rank, float* __restrict__ y) {
  extern __shared__ int cnt[];  // E + 1
  const int tid = threadIdx.x;
  for (int e = tid; e <= E; e += kRouteThreads) cnt[e] = 0;
  __syncthreads();
  for (int i = tid; i < n; i += kRouteThreads) {
    const int e = ids[i];
    if (e >= 0 && e < E) rank[i] = atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int e = 0; e < E; ++e) {
      const int c = cnt[e];
      cnt[e] = run;
      run += c;
    }
    cnt[E] = run;
  }
  __syncthreads();
  for (int e = tid; e <= E; e += kRouteThreads) offsets[e] = cnt[e];
  for (int i = tid; i < n; i += kRouteThreads) {
    const int e = ids[i];
    if (e >= 0 && e < E) list[cnt[e] + rank[i]] = i;
  }
  // Pairs with an id outside [0, E) get a row of quiet NaNs.
  const float qnan = __builtin_bit_cast(float, 0x7FC00000u);
  for (int i = 0; i < n; ++i) {
    const int e = ids[i];
    if (e < 0 || e >= E)
      for (int m = tid; m < M; m += kRouteThreads) y[(int64_t)i * M + m] = qnan;
  }
}

__global__ __launch_bounds__(kMoeThreads) void moe_gemv_kernel(
    const uint8_t* __restrict__ qs, const uint16_t* __restrict__ d, int M, int K,
    const int8_t* __restrict__ xq, const float* __restrict__ xd, int n_x_slots, int top_k,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ list, float* __restrict__ y) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int e = blockIdx.y;
  const int beg = offsets[e];
  const int cnt = offsets[e + 1] - beg;
  if (cnt == 0) return;  // expert not selected: its weights are never read
  const int m_begin = blockIdx.x * kMoeRowsPerWg;
  const int m_end = min(M, m_begin + kMoeRowsPerWg);
  const int nb = K / kQK;
  const int64_t row_bytes = K / 2;
  const uint8_t* qs_e = qs + (int64_t)e * M * row_bytes;
  const uint16_t* d_e = d + (int64_t)e * M * nb;

  int8_t* sx = reinterpret_cast<int8_t*>(smem);                          // [C][K]
  float* sxd = reinterpret_cast<float*>(smem + (size_t)kMoeCols * K);    // [C][nb]
  int* sxs = reinterpret_cast<int*>(sxd + kMoeCols * nb);                // [C][nb]
  __shared__ int s_pair[kMoeCols];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;

  for (int c0 = 0; c0 < cnt; c0 += kMoeCols) {
    const int nc = min(kMoeCols, cnt - c0);
    __syncthreads();  // previous pass finished reading the staged columns
    if (tid < kMoeCols) s_pair[tid] = tid < nc ? list[beg + c0 + tid] : -1;
    __syncthreads();
    for (int c = 0; c < kMoeCols; ++c) {
      const int p = s_pair[c];
      int4* dst = reinterpret_cast<int4*>(sx + (size_t)c * K);
      if (p >= 0) {
        const int t = p / top_k, s = p - t * top_k;
        const int64_t xrow = (int64_t)t * n_x_slots + (n_x_slots == 1 ? 0 : s);
        const int4* src = reinterpret_cast<const int4*>(xq + xrow * K);
        for (int i = tid; i < K / 16; i += kMoeThreads) dst[i] = src[i];
        for (int i = tid; i < nb; i += kMoeThreads) sxd[c * nb + i] = xd[xrow * nb + i];
      } else {
        for (int i = tid; i < K / 16; i += kMoeThreads) dst[i] = make_int4(0, 0, 0, 0);
        for (int i = tid; i < nb; i += kMoeThreads) sxd[c * nb + i] = 0.0f;
      }
    }
    __syncthreads();
    for (int i = tid; i < kMoeCols * nb; i += kMoeThreads) {
      const int* p = reinterpret_cast<const int*>(sx + (size_t)i * kQK);
      int s = 0;
#pragma unroll
      for (int k = 0; k < 8; ++k) s = __builtin_amdgcn_sdot4(p[k], 0x01010101, s, false);
      sxs[i] = 8 * s;
    }
    __syncthreads();

    for (int row0 = m_begin + wave * kMoeRU; row0 < m_end; row0 += kMoeWaves * kMoeRU) {
      float acc[kMoeRU][kMoeCols];
#pragma unroll
      for (int r = 0; r < kMoeRU; ++r)
#pragma unroll
        for (int c = 0; c < kMoeCols; ++c) acc[r][c] = 0.0f;
      for (int b0 = 0; b0 < nb; b0 += kWave) {
        const int b = b0 + lane;
        if (b < nb) {
          u32x4 w[kMoeRU];
          float dw[kMoeRU];
#pragma unroll
          for (int r = 0; r < kMoeRU; ++r) {
            const int row = row0 + r;
            if (row < m_end) {
              w[r] = *reinterpret_cast<const u32x4*>(qs_e + row * row_bytes + (int64_t)b * 16);
              dw[r] = f16_bits_to_f32(d_e[(int64_t)row * nb + b]);
            } else {
              w[r] = u32x4{0, 0, 0, 0};
              dw[r] = 0.0f;
            }
          }
#pragma unroll
          for (int c = 0; c < kMoeCols; ++c) {
            if (c < nc) {
              const i32x4* xp = reinterpret_cast<const i32x4*>(sx + (size_t)c * K + (size_t)b * kQK);
              const i32x4 xa = xp[0], xb = xp[1];
              const float xdc = sxd[c * nb + b];
              const int xsc = sxs[c * nb + b];
#pragma unroll
              for (int r = 0; r < kMoeRU; ++r) {
                const int I = dot_block(w[r], xa, xb) - xsc;
                acc[r][c] = __builtin_fmaf((float)I, dw[r] * xdc, acc[r][c]);
              }
            }
          }
        }
      }
#pragma unroll
      for (int r = 0; r < kMoeRU; ++r)
#pragma unroll
        for (int c = 0; c < kMoeCols; ++c) {
          const float v = wave_sum(acc[r][c]);
          const int row = row0 + r;
          if (lane == 0 && row < m_end && c < nc) y[(int64_t)s_pair[c] * M + row] = v;
        }
    }
  }
}

hipError_t launch_moe(const uint8_t* qs, const uint16_t* d, int64_t E, int64_t M, int64_t K,
                      const int8_t* xq, const float* xd, int64_t n_x_slots, const int32_t* ids,
                      int64_t T, int64_t top_k, float* y, void* ws, hipStream_t s) {
  const int n = (int)(T * top_k);
  int32_t* offsets = static_cast<int32_t*>(ws);
  int32_t* list = offsets + E + 1;
  int32_t* rank = list + n;
  hipLaunchKernelGGL(moe_route_kernel, dim3(1), dim3(kRouteThreads), (size_t)(E + 1) * sizeof(int),
                     s, ids, n, (int)E, (int)M, offsets, list, rank, y);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int nb = (int)(K / kQK);
  const size_t lds = (size_t)kMoeCols * K + 8 * (size_t)kMoeCols * nb;
  const dim3 grid((unsigned)((M + kMoeRowsPerWg - 1) / kMoeRowsPerWg), (unsigned)E);
  hipLaunchKernelGGL(moe_gemv_kernel, grid, dim3(kMoeThreads), lds, s, qs, d, (int)M, (int)K, xq,
                     xd, (int)n_x_slots, (int)top_k, offsets, list, y);
  return hipGetLastError();
}

}  // namespace q4q8
