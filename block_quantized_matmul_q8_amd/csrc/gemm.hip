// Int8-MFMA Q4 x Q8 matrix kernel for gfx950 (the prefill route; the mmq role
// in "GGML：Backend 抽象与硬件加速", section "CUDA：mmvq、mmq、cublas 三条
// 矩阵路": larger quantised products go to a tiled matrix kernel).
//
// One v_mfma_i32_32x32x32_i8 covers exactly one 32-element quantisation block,
// so its int32 result is the exact block sum I for a 32 x 32 output tile.  The
// accumulator input is seeded with the bits of 1.5 * 2^23: the result read as
// fp32 is F = 1.5 * 2^23 + I exactly (|I| < 2^22), and the per-block rescale
// is two fp32 fmas per output element: t = fma(F, d_w, -1.5 * 2^23 * d_w) =
// fl(I * d_w) (the product 1.5 * 2^23 * d_w is exact for an fp16 d_w), then
// acc = fma(t, d_x, acc).  Those two fmas per output and block are the
// kernel's bound: the vector ALU, not the matrix core.
//
// Operand roles: A = activations (MFMA rows = tokens), B = weights (MFMA
// columns = weight rows).  Each lane then holds one weight row (one d_w per
// lane) and 16 token rows, and the output y[token][row] is stored with
// consecutive lanes on consecutive rows.
//
// Tiling: a workgroup of 4 waves computes 128 tokens x 128 weight rows; each
// wave a 64 x 64 quadrant (2 x 2 MFMA tiles).  A stage is 4 blocks of K (128
// bytes of activation codes per token, 64 bytes of packed weight codes per
// row), so every global load instruction covers whole cache lines.  Two LDS
// stage buffers: while stage s is computed, stage s + 1 travels from global
// memory into registers and then into the other buffer (weights unpacked to
// signed int8 once, shared by all 128 tokens), so each stage costs one
// barrier.  Loads are unconditional from clamped addresses; rows, tokens and
// blocks past the end get zero scales, so they add exact zeros.
//
// Q8_0 weights (32 signed int8 codes and one fp16 scale per block) take the
// same path: a stage then holds 128 bytes of codes per weight row, fetched as
// four 16-byte pieces per thread and stored to LDS as they are (no unpack);
// everything after the LDS stage is shared with the Q4 route.
//
// One launch serves one product or a group of products (a device table of
// records plus a tile -> record map; the map lists the long-K products
// first).  Tiles of a product are ordered weight-tile major (consecutive
// tiles share the weight tile); the token tiles of one weight tile run on one
// XCD, so the weight tile is reused from that XCD's L2.
#include "common.h"

namespace q4q8 {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kTM = 128;  // weight rows per workgroup
constexpr int kTN = 128;  // tokens per workgroup
constexpr int kIT = kTN / 64;  // 32-token MFMA tiles per wave
constexpr int kNA = kTN / 32;  // 16-byte activation chunks per thread per stage
constexpr int kNBuf = 2;       // LDS stage buffers
constexpr int kKB = 4;             // 32-blocks per stage
constexpr int kGemmThreads = 256;
constexpr int kXcds = 8;

__device__ __forceinline__ uint32_t nib_to_s8(uint32_t n) {
  // bytes in [0,15] -> signed bytes n - 8 (no carries cross byte lanes)
  return (n + 0x78787878u) ^ 0x80808080u;
}

struct GemmStage {
  int8_t a[kKB][kTN][kQK];   // activation codes
  int8_t w[kKB][kTM][kQK];   // weight codes as signed int8
  float dx[kKB][kTN];        // activation scales (0 past the end)
  float dw[kKB][kTM];        // weight scales (0 past the end)
  float cw[kKB][kTM];        // -1.5 * 2^23 * dw
};

// Tile L of product P (its tiles start at P.win_begin): n_nt token tiles per
// weight tile; st: the workgroup's LDS stage buffers.
template <bool WRITE_I, int WF>
__device__ __forceinline__ void gemm_tile(const GemvProblem& P, int L, int n_nt, int B, GemmStage* st,
                                          int32_t* __restrict__ Iout) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wt = wave >> 1, ww = wave & 1;
  const int l32 = lane & 31, h = lane >> 5;
  const int M = P.M, K = P.K;
  const uint8_t* __restrict__ qs = P.qs;
  const uint16_t* __restrict__ d = P.d;
  const int8_t* __restrict__ xq = P.xq;
  const float* __restrict__ xd = P.xd;
  float* __restrict__ y = P.y;
  const int nb = K / kQK;
  constexpr int kNW = WF == kWeightQ8 ? 4 : 2;  // 16-byte weight chunks per thread per stage
  const int64_t row_bytes = WF == kWeightQ8 ? K : K / 2;
  const int lt = L - P.win_begin;
  const int m0 = (lt / n_nt) * kTM, n0 = (lt % n_nt) * kTN;

  // Thread -> data of a stage: activation chunk c = 256 i + tid is token
  // c / 8, 16-byte piece c % 8 (two pieces per block); Q4 weight chunk
  // c = 256 i + tid is row c / 4, block c % 4, Q8_0 weight chunk row c / 8,
  // piece c % 8 like the activations; scales: row / token tid / 2,
  // blocks 2 (tid % 2) and 2 (tid % 2) + 1 (read one value each: d rows are
  // only 2-byte aligned).
  auto fetch = [&](int kb0, i32x4 (&a)[kNA], u32x4 (&w)[kNW], uint32_t (&dw)[2], float (&dx)[2]) {
#pragma unroll
    for (int i = 0; i < kNA; ++i) {
      const int c = 256 * i + tid;
      const int n = min(n0 + c / 8, B - 1);
      const int blk = min(kb0 + (c % 8) / 2, nb - 1);
      a[i] = *gptr(reinterpret_cast<const i32x4*>(xq + (int64_t)n * K + (int64_t)blk * kQK + 16 * (c % 2)));
    }
#pragma unroll
    for (int i = 0; i < kNW; ++i) {
      const int c = 256 * i + tid;
      if constexpr (WF == kWeightQ8) {
        const int m = min(m0 + c / 8, M - 1);
        const int blk = min(kb0 + (c % 8) / 2, nb - 1);
        w[i] = __builtin_nontemporal_load(gptr(
            reinterpret_cast<const u32x4*>(qs + (int64_t)m * row_bytes + (int64_t)blk * kQK + 16 * (c % 2))));
      } else {
        const int m = min(m0 + c / 4, M - 1);
        const int blk = min(kb0 + c % 4, nb - 1);
        w[i] = __builtin_nontemporal_load(
            gptr(reinterpret_cast<const u32x4*>(qs + (int64_t)m * row_bytes + (int64_t)blk * 16)));
      }
    }
    const int m = min(m0 + tid / 2, M - 1);
    const int n = min(n0 + tid / 2, B - 1);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int blk = min(kb0 + 2 * (tid % 2) + e, nb - 1);
      dw[e] = gptr(d)[(int64_t)m * nb + blk];
      if (tid / 2 < kTN) dx[e] = gptr(xd)[(int64_t)n * nb + blk];
    }
  };

  auto store_stage = [&](GemmStage& sg, int kb0, const i32x4 (&a)[kNA], const u32x4 (&w)[kNW],
                         const uint32_t (&dwb)[2], const float (&dxv)[2]) {
#pragma unroll
    for (int i = 0; i < kNA; ++i) {
      const int c = 256 * i + tid;
      *reinterpret_cast<i32x4*>(&sg.a[(c % 8) / 2][c / 8][16 * (c % 2)]) = a[i];
    }
    if constexpr (WF == kWeightQ8) {
#pragma unroll
      for (int i = 0; i < kNW; ++i) {
        const int c = 256 * i + tid;
        *reinterpret_cast<u32x4*>(&sg.w[(c % 8) / 2][c / 8][16 * (c % 2)]) = w[i];
      }
    } else {
      const uint32_t m4 = 0x0F0F0F0Fu;
#pragma unroll
      for (int i = 0; i < kNW; ++i) {
        const int c = 256 * i + tid;
        const u32x4 qv = w[i];
        const u32x4 lo = {nib_to_s8(qv.x & m4), nib_to_s8(qv.y & m4), nib_to_s8(qv.z & m4), nib_to_s8(qv.w & m4)};
        const u32x4 hi = {nib_to_s8((qv.x >> 4) & m4), nib_to_s8((qv.y >> 4) & m4), nib_to_s8((qv.z >> 4) & m4),
                          nib_to_s8((qv.w >> 4) & m4)};
        *reinterpret_cast<u32x4*>(&sg.w[c % 4][c / 4][0]) = lo;
        *reinterpret_cast<u32x4*>(&sg.w[c % 4][c / 4][16]) = hi;
      }
    }
    const int r = tid / 2;
    const bool row_ok = m0 + r < M, tok_ok = n0 + r < B;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int blk = 2 * (tid % 2) + e;
      const bool blk_ok = kb0 + blk < nb;
      const float dwf = (row_ok && blk_ok) ? f16_bits_to_f32((uint16_t)dwb[e]) : 0.0f;
      sg.dw[blk][r] = dwf;
      sg.cw[blk][r] = -kMagic * dwf;
      if (r < kTN) sg.dx[blk][r] = (tok_ok && blk_ok) ? dxv[e] : 0.0f;
    }
  };

  float acc[kIT][2][16];
#pragma unroll
  for (int i = 0; i < kIT; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  v16i seed;
#pragma unroll
  for (int r = 0; r < 16; ++r) seed[r] = kMagicBits;

  i32x4 fa[kNA];
  u32x4 fw[kNW];
  uint32_t fdw[2];
  float fdx[2];
  fetch(0, fa, fw, fdw, fdx);
  if constexpr (kNBuf == 2) {
    store_stage(st[0], 0, fa, fw, fdw, fdx);
    __syncthreads();
  }

  int buf = 0;
  for (int kb0 = 0; kb0 < nb; kb0 += kKB) {
    const bool more = kb0 + kKB < nb;
    if constexpr (kNBuf == 1) {
      __syncthreads();  // the previous stage has been read
      store_stage(st[0], kb0, fa, fw, fdw, fdx);
      __syncthreads();
    }
    if (more) fetch(kb0 + kKB, fa, fw, fdw, fdx);  // in flight during this stage's compute
    const GemmStage& sg = st[kNBuf == 2 ? buf : 0];

#pragma unroll
    for (int blk = 0; blk < kKB; ++blk) {
      if (kb0 + blk < nb) {
        v4i a[kIT], b[2];
        float dw[2], cw[2];
#pragma unroll
        for (int it = 0; it < kIT; ++it)
          a[it] = *reinterpret_cast<const v4i*>(&sg.a[blk][wt * (kTN / 2) + it * 32 + l32][16 * h]);
#pragma unroll
        for (int jt = 0; jt < 2; ++jt) {
          const int wrow = ww * 64 + jt * 32 + l32;
          b[jt] = *reinterpret_cast<const v4i*>(&sg.w[blk][wrow][16 * h]);
          dw[jt] = sg.dw[blk][wrow];
          cw[jt] = sg.cw[blk][wrow];
        }
        // The four block products go to the matrix core first, into
        // separate registers, so it works while the vector ALU rescales.
        v16i Di[kIT][2];
        v16f Fv[kIT][2];
#pragma unroll
        for (int it = 0; it < kIT; ++it)
#pragma unroll
          for (int jt = 0; jt < 2; ++jt) {
            // Reinterpret the whole result vector at once: hipcc (ROCm 7.2)
            // miscompiles a per-element int <-> float bit cast of an MFMA
            // result, propagating element 0 to every element.
            Di[it][jt] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[it], b[jt], seed, 0, 0, 0);
            Fv[it][jt] = __builtin_bit_cast(v16f, Di[it][jt]);
          }
#pragma unroll
        for (int it = 0; it < kIT; ++it) {
          float dx[16];
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f32x4 v = *reinterpret_cast<const f32x4*>(&sg.dx[blk][wt * (kTN / 2) + it * 32 + 8 * g + 4 * h]);
            dx[4 * g + 0] = v.x;
            dx[4 * g + 1] = v.y;
            dx[4 * g + 2] = v.z;
            dx[4 * g + 3] = v.w;
          }
#pragma unroll
          for (int jt = 0; jt < 2; ++jt) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const float t = __builtin_fmaf(Fv[it][jt][r], dw[jt], cw[jt]);
              acc[it][jt][r] = __builtin_fmaf(t, dx[r], acc[it][jt][r]);
              if (WRITE_I) {
                const int n = n0 + wt * (kTN / 2) + it * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                const int m = m0 + ww * 64 + jt * 32 + l32;
                if (n < B && m < M) Iout[((int64_t)n * M + m) * nb + kb0 + blk] = Di[it][jt][r] - kMagicBits;
              }
            }
          }
        }
      }
    }
    if constexpr (kNBuf == 2) {
      // The other buffer was last read in the previous stage, which every
      // wave finished before the barrier that ended it.
      if (more) store_stage(st[buf ^ 1], kb0 + kKB, fa, fw, fdw, fdx);
      __syncthreads();
      buf ^= 1;
    }
  }

#pragma unroll
  for (int it = 0; it < kIT; ++it)
#pragma unroll
    for (int jt = 0; jt < 2; ++jt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int n = n0 + wt * (kTN / 2) + it * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        const int m = m0 + ww * 64 + jt * 32 + l32;
        if (n < B && m < M) y[(int64_t)n * M + m] = acc[it][jt][r];
      }
}


// Q8_0 and Q4 tiles share the LDS stage layout.  WF = kWeightMixed (grouped
// only): each record's format decides, uniformly over a workgroup; that
// instance holds both tile bodies, so uniform groups take the single-format
// ones.
template <bool WRITE_I, bool GROUPED, int WF = kWeightQ4>
__global__ __launch_bounds__(kGemmThreads, WRITE_I ? 1 : 2) void gemm_kernel(
    GemvProblem p0, const GemvProblem* __restrict__ table, const int32_t* __restrict__ tile_map,
    int n_tiles, int B, int32_t* __restrict__ Iout) {
  __shared__ __align__(16) GemmStage st[kNBuf];

  // Tile of this workgroup.  The tile list is dealt to the XCDs (workgroup
  // bid runs on XCD bid % 8) in chunks of n_nt consecutive tiles -- the token
  // tiles of one weight tile -- round robin: a weight tile stays on one XCD
  // (reused from its L2) while long and short products spread over all XCDs.
  const int n_nt = (B + kTN - 1) / kTN;
  const int bid = blockIdx.x;
  const int span = kXcds * n_nt;
  int L = bid;
  if (bid < n_tiles / span * span) {
    const int x = bid % kXcds, pos = bid / kXcds;
    L = ((pos / n_nt) * kXcds + x) * n_nt + pos % n_nt;
  }
  if constexpr (GROUPED && WF == kWeightMixed) {
    const GemvProblem P = table[tile_map[L]];
    if (P.wf == kWeightQ8)
      gemm_tile<WRITE_I, kWeightQ8>(P, L, n_nt, B, st, Iout);
    else
      gemm_tile<WRITE_I, kWeightQ4>(P, L, n_nt, B, st, Iout);
  } else if constexpr (GROUPED) {
    gemm_tile<WRITE_I, WF>(table[tile_map[L]], L, n_nt, B, st, Iout);
  } else {
    gemm_tile<WRITE_I, WF>(p0, L, n_nt, B, st, Iout);
  }
}

int64_t gemm_tiles(int64_t M, int64_t B) { return ((M + kTM - 1) / kTM) * ((B + kTN - 1) / kTN); }

hipError_t launch_gemm(const GemvProblem& p, const GemvProblem* table, const int32_t* tile_map,
                       int64_t n_tiles, int64_t B, int32_t* I, hipStream_t s, int wf) {
  const dim3 grid((unsigned)n_tiles), block(kGemmThreads);
  auto go = [&](auto kernel) {
    note_launch((const void*)kernel);
    hipLaunchKernelGGL(kernel, grid, block, 0, s, p, table, tile_map, (int)n_tiles, (int)B, I);
    return hipGetLastError();
  };
  if (table) {
    if (I) return hipErrorInvalidValue;
    if (wf == kWeightQ4) return go(gemm_kernel<false, true, kWeightQ4>);
    if (wf == kWeightQ8) return go(gemm_kernel<false, true, kWeightQ8>);
    if (wf == kWeightMixed) return go(gemm_kernel<false, true, kWeightMixed>);
    return hipErrorInvalidValue;
  }
  if (wf == kWeightQ4) return I ? go(gemm_kernel<true, false, kWeightQ4>) : go(gemm_kernel<false, false, kWeightQ4>);
  if (wf == kWeightQ8) return I ? go(gemm_kernel<true, false, kWeightQ8>) : go(gemm_kernel<false, false, kWeightQ8>);
  return hipErrorInvalidValue;
}

}  // namespace q4q8
