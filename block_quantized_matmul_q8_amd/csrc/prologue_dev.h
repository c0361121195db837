// Device-side steps of the RMSNorm * g -> Q8 prologue, shared by the
// standalone prologue kernel and the GEMV kernel that folds the prologue in.
// Both therefore produce the same codes and scales bit for bit.
//
// Order of operations (each a single IEEE-rounded fp32 operation):
//   p_b  = sum_{j<32} x_j * x_j over block b, in index order;
//   the p_b are padded with +0 to P = next_pow2(nb) values and reduced
//   pairwise, adjacent pairs, level by level (p[i] = p[2i] + p[2i+1]);
//   s    = 1 / sqrt(ssq / K + eps);
//   v_j  = (x_j * s) * g_j   (or v = x when the norm is skipped);
//   with an addend row a (RMS_NORM+MUL+ADD): v_j = ((x_j * s) * g_j) + a_j;
//   per 32-block: d = amax(|v|) / 127, id = 1 / d (0 if d == 0),
//   q_j = roundf(v_j * id) (halves away from zero), clamped to [-127, 127].
// The two roundings in v keep the fused RMS_NORM+MUL equal to the unfused
// pair ("llama.cpp b10909：Metal后端融合表重构..." restores that fusion).
#pragma once

#include "common.h"

namespace q4q8 {

__device__ __forceinline__ void load_block32(const float* p, float (&v)[kQK]) {
  const Q4Q8_GLOBAL f32x4* s = gptr(reinterpret_cast<const f32x4*>(p));
#pragma unroll
  for (int i = 0; i < kQK / 4; ++i) {
    const f32x4 t = s[i];
    v[4 * i + 0] = t.x;
    v[4 * i + 1] = t.y;
    v[4 * i + 2] = t.z;
    v[4 * i + 3] = t.w;
  }
}

__host__ __device__ __forceinline__ int next_pow2_int(int n) {
  int p = 1;
  while (p < n) p *= 2;
  return p;
}

// Sum over the 64 lanes of a wave as a pairwise tree: level k adds lane
// groups of 2^k that are neighbours (lane ^ 2^k), so every lane ends with the
// tree sum of the wave (fp32 addition is commutative, so the operand order
// within a pair does not matter).  Levels 1..8 are DPP lane permutations
// folded into the add (quad_perm [1,0,3,2], [2,3,0,1], row_half_mirror,
// row_mirror: each maps a lane group onto its neighbour group), levels 16 and
// 32 v_permlane16/32_swap, whose two results hold the pair's two values in
// every lane -- no LDS round trip at any level.
__device__ __forceinline__ float wave_tree_sum(float v) {
  v = __fadd_rn(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false)));
  v = __fadd_rn(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false)));
  v = __fadd_rn(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false)));
  v = __fadd_rn(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false)));
  // Elements of the swap pairs are copied into scalars before any bit cast
  // (hipcc miscompiles a bit cast of one element of a vector value).
  const auto p16 = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, v), __builtin_bit_cast(unsigned, v),
                                                    false, false);
  const unsigned a0 = p16[0], a1 = p16[1];
  v = __fadd_rn(__builtin_bit_cast(float, a0), __builtin_bit_cast(float, a1));
  const auto p32 = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, v), __builtin_bit_cast(unsigned, v),
                                                    false, false);
  const unsigned b0 = p32[0], b1 = p32[1];
  return __fadd_rn(__builtin_bit_cast(float, b0), __builtin_bit_cast(float, b1));
}

// Largest |v_j| of a block, as a tree (the maximum does not depend on the
// order, and a tree is 5 dependent steps instead of 31).
__device__ __forceinline__ float block_amax(const float (&v)[kQK]) {
  float m[kQK / 2];
#pragma unroll
  for (int j = 0; j < kQK / 2; ++j) m[j] = fmaxf(fabsf(v[2 * j]), fabsf(v[2 * j + 1]));
#pragma unroll
  for (int w = kQK / 4; w >= 1; w /= 2)
#pragma unroll
    for (int j = 0; j < w; ++j) m[j] = fmaxf(m[2 * j], m[2 * j + 1]);
  return m[0];
}

// RMS scale s of one row, computed cooperatively by all `nthreads` threads of
// the workgroup (every thread must call it).  `red` is LDS scratch of 2 * P
// floats; `s_slot` one LDS float.  Returns s to every thread.
__device__ __forceinline__ float wg_rms_scale(const float* __restrict__ xr, int K, float eps, int P,
                                              float* red, float* s_slot, int tid, int nthreads) {
  const int nb = K / kQK;
  for (int b = tid; b < P; b += nthreads) {
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
    for (int i = tid; i < h; i += nthreads) dst[i] = __fadd_rn(src[2 * i], src[2 * i + 1]);
    __syncthreads();
    float* t = src;
    src = dst;
    dst = t;
  }
  if (tid == 0) {
    const float mean = __fdiv_rn(src[0], (float)K);
    const float r = sqrt_rn(__fadd_rn(mean, eps));
    *s_slot = __fdiv_rn(1.0f, r);
  }
  __syncthreads();
  return *s_slot;
}

// roundf(t) (halves away from zero) as an int, for any finite t whose
// rounded value fits an int: fl(t + copysign(0.5 - 2^-25, t)) truncated.
// Adding the largest float below one half, with round-to-nearest-even, never
// carries t past the next integer unless roundf does: for frac(t) < 1/2 the
// sum stays more than a rounding step below it, for frac(t) >= 1/2 it lands
// within half a step of it (the tie at t = 1/2 goes to the even 1.0); at
// 2^23 and above every float is an integer and the sum rounds back to t.
// Two instructions and a truncating convert instead of roundf's six.
__device__ __forceinline__ int round_half_away_i32(float t) {
  return (int)__fadd_rn(t, __builtin_copysignf(0.49999997f, t));
}

// The Q8 block rule on 32 values: d = amax(|v|) / 127, id = 1 / d (0 for an
// all-zero block), q = roundf(v * id) clamped to [-127, 127].  packed[8]
// holds the codes in index order (4 per dword, little-endian), sum their sum.
__device__ __forceinline__ void q8_pack_block(const float (&v)[kQK], uint32_t (&packed)[8], float& d, int& sum) {
  const float amax = block_amax(v);
  d = __fdiv_rn(amax, 127.0f);
  const float id = d != 0.0f ? __fdiv_rn(1.0f, d) : 0.0f;
  sum = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t word = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      int qi = round_half_away_i32(__fmul_rn(v[4 * i + k], id));
      qi = qi > 127 ? 127 : (qi < -127 ? -127 : qi);
      sum += qi;
      word |= ((uint32_t)qi & 0xFFu) << (8 * k);
    }
    packed[i] = word;
  }
}

// Q8 codes of block b of one row: packed[8] holds the 32 int8 codes in index
// order (4 per dword, little-endian), d the fp32 scale, sum the code sum.
// ar: the row's addend (RMS_NORM+MUL+ADD) or null.
__device__ __forceinline__ void q8_block_codes(const float* __restrict__ xr, const float* __restrict__ g,
                                               int b, float s, bool no_norm, uint32_t (&packed)[8],
                                               float& d, int& sum, const float* __restrict__ ar = nullptr) {
  float v[kQK];
  load_block32(xr + b * kQK, v);
  if (!no_norm) {
    float gv[kQK];
    load_block32(g + b * kQK, gv);
#pragma unroll
    for (int j = 0; j < kQK; ++j) v[j] = __fmul_rn(__fmul_rn(v[j], s), gv[j]);
  }
  if (ar) {
    float av[kQK];
    load_block32(ar + b * kQK, av);
#pragma unroll
    for (int j = 0; j < kQK; ++j) v[j] = __fadd_rn(v[j], av[j]);
  }
  q8_pack_block(v, packed, d, sum);
}

// SwiGLU producer: a fixed fp32 exponential, so that the Q8 codes of
// silu(gate) * up are reproducible bit for bit.  W. J. Cody and W. Waite's
// argument reduction (t = n ln2 + r, ln2 split into a high part with 8
// trailing zero bits, so n * ln2_hi is exact), exp(r) by its degree-7 Taylor
// polynomial in Horner form (coefficients the fp32 values nearest 1/k!), and
// exact scaling by 2^n.  Every step is one fp32 rounding; no fused
// multiply-add.  Domain [-17, 88]: below it 1 + exp(t) == 1 in fp32 anyway
// (0 is returned), above it +inf.  Maximal error about 1.2 ulp.
__device__ __forceinline__ float exp_q(float t) {
  if (t != t) return t;
  if (t > 88.0f) return __builtin_inff();
  if (t < -17.0f) return 0.0f;
  const float l2e = __builtin_bit_cast(float, 0x3fb8aa3bu);
  const float ln2_hi = __builtin_bit_cast(float, 0x3f317200u);
  const float ln2_lo = __builtin_bit_cast(float, 0x35bfbe8eu);
  const float nf = rintf(__fmul_rn(t, l2e));
  const float r = __fadd_rn(__fadd_rn(t, -__fmul_rn(nf, ln2_hi)), -__fmul_rn(nf, ln2_lo));
  float c = __builtin_bit_cast(float, 0x39500d01u);                       // 1/7!
  c = __fadd_rn(__fmul_rn(c, r), __builtin_bit_cast(float, 0x3ab60b61u));  // 1/6!
  c = __fadd_rn(__fmul_rn(c, r), __builtin_bit_cast(float, 0x3c088889u));  // 1/5!
  c = __fadd_rn(__fmul_rn(c, r), __builtin_bit_cast(float, 0x3d2aaaabu));  // 1/4!
  c = __fadd_rn(__fmul_rn(c, r), __builtin_bit_cast(float, 0x3e2aaaabu));  // 1/3!
  c = __fadd_rn(__fmul_rn(c, r), 0.5f);
  c = __fadd_rn(__fmul_rn(c, r), 1.0f);
  const float p = __fadd_rn(__fmul_rn(c, r), 1.0f);
  const float scale = __builtin_bit_cast(float, (uint32_t)((int)nf + 127) << 23);
  return __fmul_rn(p, scale);
}

// silu(g) = g / (1 + exp(-g)).
__device__ __forceinline__ float silu_q(float g) { return __fdiv_rn(g, __fadd_rn(1.0f, exp_q(-g))); }

// The same prologue for one row, latency-optimised for a workgroup that
// folds it into a product kernel (K <= 16384, i.e. at most 2 blocks per
// thread of a 256-thread workgroup).  Produces bit for bit what
// wg_rms_scale + q8_block_codes produce:
//   - each thread loads x (and g) of its blocks once, into registers;
//   - per-block sums in index order; the first six levels of the pairwise
//     tree are a 64-lane xor butterfly within each wave (block = 64 * group +
//     lane, so the butterfly pairs exactly the tree's pairs, and the zero
//     padding of missing blocks adds exact zeros); one barrier publishes the
//     per-wave group sums; every thread finishes the tree over the groups
//     and computes s itself;
//   - each thread quantises its blocks from the registers it holds.
// Writes codes to sx [K] (int8), scales to sxd [nb] and, when sxs is not
// null, code sums to sxs [nb] (LDS or global memory); `groups` is LDS scratch
// of 8 floats; ar: the row's addend (RMS_NORM+MUL+ADD) or null.  Ends with a
// barrier.
constexpr int kFastPrologueK = 16384;

__device__ __forceinline__ void wg_q8_row_fast(const float* __restrict__ xr,
                                               const float* __restrict__ g, int K, float eps,
                                               bool raw, int8_t* sx, float* sxd, int* sxs,
                                               float* groups, int tid, const float* __restrict__ ar = nullptr) {
  constexpr int kThreads = 256;
  const int nb = K / kQK;
  const int lane = tid & 63, wave = tid >> 6;
  float xv[2][kQK], gv[2][kQK];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int b = tid + kThreads * h;
    if (b < nb) {
      load_block32(xr + b * kQK, xv[h]);
      if (!raw) load_block32(g + b * kQK, gv[h]);
    }
  }
  float s = 1.0f;
  if (!raw) {
    float gsum[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int b = tid + kThreads * h;
      float acc = 0.0f;
      if (b < nb) {
#pragma unroll
        for (int j = 0; j < kQK; ++j) acc = __fadd_rn(acc, __fmul_rn(xv[h][j], xv[h][j]));
      }
      gsum[h] = wave_tree_sum(acc);
    }
    if (lane == 0) {
      groups[wave] = gsum[0];
      groups[4 + wave] = gsum[1];
    }
    __syncthreads();
    // The tree's levels above the wave groups.  Groups past the padded count
    // hold +0 and adding +0 to a non-negative sum is exact, so a fixed
    // three-level tree over all 8 slots gives the bits of the tree over the
    // next_pow2(nb) / 64 slots for every row length.
    float t[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) t[i] = groups[i];
#pragma unroll
    for (int h = 4; h >= 1; h /= 2)
#pragma unroll
      for (int i = 0; i < h; ++i) t[i] = __fadd_rn(t[2 * i], t[2 * i + 1]);
    const float mean = __fdiv_rn(t[0], (float)K);
    const float r = sqrt_rn(__fadd_rn(mean, eps));
    s = __fdiv_rn(1.0f, r);
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int b = tid + kThreads * h;
    if (b < nb) {
      float v[kQK];
#pragma unroll
      for (int j = 0; j < kQK; ++j) v[j] = raw ? xv[h][j] : __fmul_rn(__fmul_rn(xv[h][j], s), gv[h][j]);
      if (ar) {
        float av[kQK];
        load_block32(ar + b * kQK, av);
#pragma unroll
        for (int j = 0; j < kQK; ++j) v[j] = __fadd_rn(v[j], av[j]);
      }
      float d;
      int sum;
      uint32_t packed[8];
      q8_pack_block(v, packed, d, sum);
      u32x4* dst = reinterpret_cast<u32x4*>(sx + (size_t)b * kQK);
      dst[0] = u32x4{packed[0], packed[1], packed[2], packed[3]};
      dst[1] = u32x4{packed[4], packed[5], packed[6], packed[7]};
      sxd[b] = d;
      if (sxs) sxs[b] = sum;
    }
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// The same prologue on a 1024-thread workgroup, for the latency-bound decode
// rows (a handful of rows per call, each on its own workgroup): more lanes per
// row shorten every serial stretch of the row's work.  Bit for bit the steps
// above: per-block sums in index order, the pairwise tree over the padded
// block sums, then s, v and the Q8 block rule.
// ---------------------------------------------------------------------------
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
constexpr int kWideThreads = 1024;
constexpr int kWideWaves = kWideThreads / kWave;
constexpr int kQuadMaxK = kQK * kWideThreads / 4;  // 8192: four lanes per block
constexpr int kPairMaxK = kQK * kWideThreads / 2;  // 16384: two lanes per block
constexpr int kWideMaxK = kQK * kWideThreads;      // 32768: one lane per block

// Waves of the 1024-thread workgroup that hold lanes of a row of K (K <=
// kWideMaxK): 4, 2 or 1 lanes per block by the row forms below.  The others
// have no part in the row; the kernels let them leave the workgroup before
// any barrier (a barrier waits for the waves that have not ended only).
__host__ __device__ constexpr int wide_active_waves(int K) {
  const int nb = K / kQK;
  const int lanes = nb * (K <= kQuadMaxK ? 4 : K <= kPairMaxK ? 2 : 1);
  return lanes <= kWave ? 1 : (lanes + kWave - 1) / kWave;
}

// DPP within each group of L lanes (L = 2 or 4; groups aligned in quads):
// lane_from_prev hands lane r the value of lane r - 1 (quad_perm [0,0,1,2]
// for L = 4, [0,0,2,2] for L = 2); group_max and group_isum combine the
// group by swapping neighbours ([1,0,3,2]) and, for L = 4, pairs
// ([2,3,0,1]).
template <int L>
__device__ __forceinline__ float lane_from_prev(float v) {
  constexpr int sel = L == 4 ? 0x90 : 0xA0;
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), sel, 0xF, 0xF, false));
}
template <int L>
__device__ __forceinline__ float group_max(float m) {
  m = fmaxf(m, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, m), 0xB1, 0xF, 0xF, false)));
  if constexpr (L == 4)
    m = fmaxf(m, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, m), 0x4E, 0xF, 0xF, false)));
  return m;
}
template <int L>
__device__ __forceinline__ int group_isum(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);
  if constexpr (L == 4) v += __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);
  return v;
}
__device__ __forceinline__ float quad_max(float m) { return group_max<4>(m); }

// s from the per-wave partial trees: lane 0 of every wave publishes its
// wave's sum, one barrier, and every thread finishes the tree over the 16
// wave slots (slots past the row's padded block count hold +0, and adding +0
// to a non-negative sum is exact, so the fixed four-level tree gives the bits
// of the tree over next_pow2(nb) blocks).  Only the first n_waves waves hold
// lanes of the row (wide_active_waves); the others have left the workgroup,
// and their slots are taken as +0.
__device__ __forceinline__ float wide_rms_scale(float wave_sum, int K, float eps, float* groups, int tid,
                                                int n_waves) {
  if ((tid & (kWave - 1)) == 0) groups[tid / kWave] = wave_sum;
  __syncthreads();
  float t[kWideWaves];
#pragma unroll
  for (int i = 0; i < kWideWaves; ++i) t[i] = i < n_waves ? groups[i] : 0.0f;
#pragma unroll
  for (int h = kWideWaves / 2; h >= 1; h /= 2)
#pragma unroll
    for (int i = 0; i < h; ++i) t[i] = __fadd_rn(t[2 * i], t[2 * i + 1]);
  const float mean = __fdiv_rn(t[0], (float)K);
  return __fdiv_rn(1.0f, sqrt_rn(__fadd_rn(mean, eps)));
}

// One row of at most 1024 / L blocks, L = 4 or 2 lanes per block: lane r of
// group b holds elements E r .. E r + E - 1 of block b (E = 32 / L).
//   - the block's squares are formed in parallel and summed in index order
//     by passing the running sum along the group (L rounds of E adds);
//   - the group's last lane holds p_b; with the other lanes at +0, the
//     wave's xor butterfly pairs exactly the tree's pairs of blocks (its
//     first log2 L levels add exact zeros);
//   - amax (and the code sum) over the group by DPP, then each lane codes
//     its E values.
// Writes codes to xq [K], scales to xd [nb] and, when xs is not null, code
// sums to xs [nb]; ar: the row's addend (RMS_NORM+MUL+ADD) or null; groups:
// LDS of 16 floats.
template <int L>
__device__ __forceinline__ void wide_q8_row_lanes(const float* __restrict__ xr, const float* __restrict__ g, int K,
                                                  float eps, bool raw, int8_t* __restrict__ xq,
                                                  float* __restrict__ xd, int32_t* __restrict__ xs, float* groups,
                                                  int tid, const float* __restrict__ ar = nullptr) {
  static_assert(L == 2 || L == 4, "two or four lanes per block");
  constexpr int E = kQK / L;
  const int nb = K / kQK;
  const int b = tid / L, r = tid % L;
  const bool on = b < nb;
  float xv[E], gv[E];
#pragma unroll
  for (int j = 0; j < E; ++j) xv[j] = gv[j] = 0.0f;
  if (on) {
    const Q4Q8_GLOBAL f32x4* px = gptr(reinterpret_cast<const f32x4*>(xr + b * kQK + E * r));
#pragma unroll
    for (int i = 0; i < E / 4; ++i) {
      const f32x4 t = px[i];
      xv[4 * i] = t.x, xv[4 * i + 1] = t.y, xv[4 * i + 2] = t.z, xv[4 * i + 3] = t.w;
    }
    if (!raw) {
      const Q4Q8_GLOBAL f32x4* pg = gptr(reinterpret_cast<const f32x4*>(g + b * kQK + E * r));
#pragma unroll
      for (int i = 0; i < E / 4; ++i) {
        const f32x4 t = pg[i];
        gv[4 * i] = t.x, gv[4 * i + 1] = t.y, gv[4 * i + 2] = t.z, gv[4 * i + 3] = t.w;
      }
    }
  }
  float s = 1.0f;
  if (!raw) {
    float sq[E];
#pragma unroll
    for (int j = 0; j < E; ++j) sq[j] = __fmul_rn(xv[j], xv[j]);
    // round k: lane k continues the block's sum from lane k - 1's result
    float cin = 0.0f, t = 0.0f;
#pragma unroll
    for (int k = 0; k < L; ++k) {
      t = cin;
#pragma unroll
      for (int j = 0; j < E; ++j) t = __fadd_rn(t, sq[j]);
      const float prev = lane_from_prev<L>(t);
      cin = r == k + 1 ? prev : cin;
    }
    s = wide_rms_scale(wave_tree_sum(r == L - 1 ? t : 0.0f), K, eps, groups, tid, (nb * L + kWave - 1) / kWave);
  }
  float v[E];
#pragma unroll
  for (int j = 0; j < E; ++j) v[j] = raw ? xv[j] : __fmul_rn(__fmul_rn(xv[j], s), gv[j]);
  if (ar && on) {
    const Q4Q8_GLOBAL f32x4* pa = gptr(reinterpret_cast<const f32x4*>(ar + b * kQK + E * r));
#pragma unroll
    for (int i = 0; i < E / 4; ++i) {
      const f32x4 t = pa[i];
      v[4 * i] = __fadd_rn(v[4 * i], t.x), v[4 * i + 1] = __fadd_rn(v[4 * i + 1], t.y);
      v[4 * i + 2] = __fadd_rn(v[4 * i + 2], t.z), v[4 * i + 3] = __fadd_rn(v[4 * i + 3], t.w);
    }
  }
  float m = 0.0f;
#pragma unroll
  for (int j = 0; j < E; j += 2) m = fmaxf(m, fmaxf(fabsf(v[j]), fabsf(v[j + 1])));
  const float amax = group_max<L>(m);
  const float d = __fdiv_rn(amax, 127.0f);
  const float id = d != 0.0f ? __fdiv_rn(1.0f, d) : 0.0f;
  uint32_t w[E / 4];
  int csum = 0;
#pragma unroll
  for (int h = 0; h < E / 4; ++h) {
    uint32_t word = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      int qi = round_half_away_i32(__fmul_rn(v[4 * h + k], id));
      qi = qi > 127 ? 127 : (qi < -127 ? -127 : qi);
      csum += qi;
      word |= ((uint32_t)qi & 0xFFu) << (8 * k);
    }
    w[h] = word;
  }
  if (xs) csum = group_isum<L>(csum);  // exact integer adds
  if (on) {
    if constexpr (E == 8) {
      *gptr_w(reinterpret_cast<u32x2_t*>(xq + b * kQK + E * r)) = u32x2_t{w[0], w[1]};
    } else {
      *gptr_w(reinterpret_cast<u32x4*>(xq + b * kQK + E * r)) = u32x4{w[0], w[1], w[2], w[3]};
    }
    if (r == 0) {
      gptr_w(xd)[b] = d;
      if (xs) gptr_w(xs)[b] = csum;
    }
  }
}

// One row of at most 1024 blocks (K <= 32768), one lane per block: the
// register form of wg_q8_row_fast on 16 waves.
__device__ __forceinline__ void wide_q8_row_single(const float* __restrict__ xr, const float* __restrict__ g, int K,
                                                   float eps, bool raw, int8_t* __restrict__ xq,
                                                   float* __restrict__ xd, int32_t* __restrict__ xs, float* groups,
                                                   int tid, const float* __restrict__ ar = nullptr) {
  const int nb = K / kQK;
  const int b = tid;
  const bool on = b < nb;
  float xv[kQK], gv[kQK];
#pragma unroll
  for (int j = 0; j < kQK; ++j) xv[j] = gv[j] = 0.0f;
  if (on) {
    load_block32(xr + b * kQK, xv);
    if (!raw) load_block32(g + b * kQK, gv);
  }
  float s = 1.0f;
  if (!raw) {
    float acc = 0.0f;
#pragma unroll
    for (int j = 0; j < kQK; ++j) acc = __fadd_rn(acc, __fmul_rn(xv[j], xv[j]));
    s = wide_rms_scale(wave_tree_sum(acc), K, eps, groups, tid, (nb + kWave - 1) / kWave);
  }
  if (on) {
    float v[kQK];
#pragma unroll
    for (int j = 0; j < kQK; ++j) v[j] = raw ? xv[j] : __fmul_rn(__fmul_rn(xv[j], s), gv[j]);
    if (ar) {
      float av[kQK];
      load_block32(ar + b * kQK, av);
#pragma unroll
      for (int j = 0; j < kQK; ++j) v[j] = __fadd_rn(v[j], av[j]);
    }
    float d;
    int sum;
    uint32_t packed[8];
    q8_pack_block(v, packed, d, sum);
    u32x4* dst = reinterpret_cast<u32x4*>(xq + (size_t)b * kQK);
    gptr_w(dst)[0] = u32x4{packed[0], packed[1], packed[2], packed[3]};
    gptr_w(dst)[1] = u32x4{packed[4], packed[5], packed[6], packed[7]};
    gptr_w(xd)[b] = d;
    if (xs) gptr_w(xs)[b] = sum;
  }
}

}  // namespace q4q8
