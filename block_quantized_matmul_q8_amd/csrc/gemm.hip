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
// acc = fma(t, d_x, acc).  Q4 weights enter the MFMA as the bytes 16 (q - 8)
// (two bit operations per four codes, no add), so F = 1.5 * 2^23 + 16 I
// (|16 I| < 2^22 still) and the fmas take d_w / 16 and -1.5 * 2^23 * d_w / 16,
// both exact: t keeps the bits of fl(I * d_w).
//
// What bounds it on gfx950 (measured): a 32x32x32 i8 MFMA occupies the
// matrix core of its SIMD for 32-37 cycles, and a SIMD's vector ALU retires
// one wave64 fp32 fma about every 4 cycles when two or more waves feed it
// (one wave alone: one every ~6 cycles).  The matrix core and the vector ALU
// run concurrently (instructions of other waves, or independent ones of the
// same wave, issue while an MFMA executes), so a 32 x 32 tile-block costs
// about 4 x 32 = 128 vector-ALU cycles against 32 on the matrix core: the
// rescale fmas are the bound (near 25% of the int8 peak at 2.4 GHz, less at
// the clock the chip holds under this load), and every other vector
// instruction adds to it.  Waves stall where an MFMA or fma waits for an
// LDS read or for the MFMA result it consumes; with two waves per SIMD (the
// register budget of this tiling) such stalls leave the vector ALU idle
// unless the other wave has work, so LDS operands are read one MFMA ahead.
//
// Operand roles: A = activations (MFMA rows = tokens), B = weights (MFMA
// columns = weight rows).  Each lane then holds one weight row per 32-row
// tile (one d_w per lane) and 16 token rows: 8 (r / 4) + 4 (lane / 32) +
// (r % 4) for result register r.
//
// Tiling: a workgroup of 4 waves computes 128 tokens x 128 weight rows; each
// wave 32 tokens x 128 rows (4 MFMA tiles side by side), so the 16 token
// scales a lane needs per block are read once and serve 4 tiles.  A stage is
// 4 blocks of K.  Stage layout in LDS, per block: activations and weight
// codes as [32-row group][half][32 rows][16 bytes], so that the operand read
// of a wave (lane = half * 32 + row) is one contiguous 1 KiB; the row slot is
// XOR-ed with 8 * half, which keeps those reads contiguous per half and
// with padded block planes spreads the stage writes over the banks.  Two LDS
// stage buffers: while stage s is computed, stage s + 1 travels from global
// memory into registers and then into the other buffer (Q4 codes unpacked to
// 16 (q - 8) once, shared by all 128 tokens), so each stage costs one
// barrier.  Global loads are shaped for few cache lines per instruction
// (whole 128-byte lines of a token or row; the 4 scales of a token or row of
// a stage in one load) and take no vector instructions in a full stage (a
// uniform base plus per-lane offsets fixed per tile).  Loads are
// unconditional from clamped addresses; rows and tokens past the end are
// computed but never stored, and blocks past the end are skipped.
//
// Q8_0 weights (32 signed int8 codes and one fp16 scale per block) take the
// same path: their codes go to LDS as they are (no unpack); everything after
// the LDS stage is shared with the Q4 route.
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
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kTM = 128;            // weight rows per workgroup
constexpr int kTN = 128;            // tokens per workgroup
constexpr int kJT = kTM / 32;       // 32-row MFMA tiles per wave
constexpr int kKB = 4;              // 32-blocks per stage
constexpr int kGemmThreads = 256;
constexpr int kXcds = 8;

// Four Q4 codes held in the high nibbles of v's bytes -> the signed bytes
// 16 (q - 8): the low nibbles cleared and each byte's top bit flipped (no
// carries cross byte lanes).  The MFMA then sums 16 I, which the rescale
// takes with d_w / 16 (both exact: powers of two).
__device__ __forceinline__ uint32_t nib_hi_to_s8x16(uint32_t v) { return (v ^ 0x80808080u) & 0xF0F0F0F0u; }

// Block planes are padded (activation codes by 32 bytes, weight codes by
// 64), so that the stage writes of 16 consecutive lanes -- 2 tokens x 4
// blocks x 2 halves of activation codes, 4 rows x 4 blocks of Q4 codes --
// fall on 16 distinct 16-byte bank slots.
struct GemmStage {
  struct {
    int8_t v[kTN / 32][2][32][16];     // activation codes [token group][half][token ^ 8 half][16 B]
    int8_t pad[32];
  } a[kKB];
  struct {
    int8_t v[kTM / 32][2][32][16];     // weight codes as signed int8, same layout over rows
    int8_t pad[64];
  } w[kKB];
  float dx[kKB][kTN];                  // activation scales
  f32x2 dwc[kKB][kTM];                 // (d_w, -1.5 * 2^23 * d_w)
};

// Byte offset of the 16-byte piece (half h, row r) inside a [32-row group]
// region of the a / w arrays (one block).
__device__ __forceinline__ int piece_off(int r, int h) { return h * 512 + ((r & 31) ^ (8 * h)) * 16; }

// Tile L of product P (its tiles start at P.win_begin): n_nt token tiles per
// weight tile; st: the workgroup's LDS stage buffers.
template <bool WRITE_I, int WF>
__device__ __forceinline__ void gemm_tile(const GemvProblem& P, int L, int n_nt, int B, GemmStage* st,
                                          int32_t* __restrict__ Iout) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  const int M = P.M, K = P.K;
  const uint8_t* __restrict__ qs = P.qs;
  const uint16_t* __restrict__ d = P.d;
  const int8_t* __restrict__ xq = P.xq;
  const float* __restrict__ xd = P.xd;
  float* __restrict__ y = P.y;
  const int nb = K / kQK;
  const int64_t row_bytes = WF == kWeightQ8 ? K : K / 2;
  const int lt = L - P.win_begin;
  const int m0 = (lt / n_nt) * kTM, n0 = (lt % n_nt) * kTN;

  // Per stage and thread, through registers:
  //   - activation chunks c = 256 i + tid: token c / 8, 16-byte piece c % 8
  //     (block (c % 8) / 2, half c % 2), so 8 lanes read one token's 128
  //     contiguous bytes;
  //   - Q4 weight chunks c = 256 i + tid: row c / 4, block c % 4 (16 bytes
  //     holding codes j and j + 16 per byte); Q8_0: row c / 8, piece c % 8
  //     like the activations;
  //   - scales of the stage's 4 blocks: the activation scales of token
  //     tid % 128 (16 bytes) and the weight scales of row tid % 128 (8
  //     bytes); threads below 128 store the former, the others the latter.
  // A full stage whose scale rows keep that alignment (K a multiple of 128;
  // the usual case) addresses each of them as a uniform base -- the tile's
  // first row, advanced by the stage -- plus a 32-bit per-lane offset
  // computed once per tile (rows past the end clamped to the last one): no
  // vector instructions and no branches, so that nothing makes the wave wait
  // for the loads before the stage store that consumes them.  Any other stage
  // clamps every row and block index and reads the scales one at a time.
  constexpr int kNA = kTN / 32;
  constexpr int kNW = WF == kWeightQ8 ? 4 : 2;
  constexpr int kWB = WF == kWeightQ8 ? kQK : kQK / 2;  // weight bytes per row and block
  const int sr = tid & 127;
  const int8_t* __restrict__ xtile = xq + (int64_t)n0 * K;
  const uint8_t* __restrict__ wtile = qs + (int64_t)m0 * row_bytes;
  const float* __restrict__ xdtile = xd + (int64_t)n0 * nb;
  const uint16_t* __restrict__ dtile = d + (int64_t)m0 * nb;
  uint32_t aoff[kNA], woff[kNW];
#pragma unroll
  for (int i = 0; i < kNA; ++i) {
    const int c = 256 * i + tid;
    aoff[i] = (uint32_t)min(c / 8, B - 1 - n0) * (uint32_t)K + 32u * ((c % 8) / 2) + 16u * (c % 2);
  }
#pragma unroll
  for (int i = 0; i < kNW; ++i) {
    const int c = 256 * i + tid;
    if constexpr (WF == kWeightQ8)
      woff[i] = (uint32_t)min(c / 8, M - 1 - m0) * (uint32_t)row_bytes + 32u * ((c % 8) / 2) + 16u * (c % 2);
    else
      woff[i] = (uint32_t)min(c / 4, M - 1 - m0) * (uint32_t)row_bytes + 16u * (c % 4);
  }
  const uint32_t xsoff = (uint32_t)min(sr, B - 1 - n0) * (uint32_t)nb;
  const uint32_t wsoff = (uint32_t)min(sr, M - 1 - m0) * (uint32_t)nb;
  const bool fast_ok = (nb & 3) == 0 && (reinterpret_cast<uintptr_t>(xd) & 15) == 0 &&
                       (reinterpret_cast<uintptr_t>(d) & 7) == 0;

  // Staged data of one stage: packed weight scales in sw, activation scales
  // (or, from the general fetch, the weight scales one per word) in sx.
  struct Staged {
    i32x4 a[kNA];
    u32x4 w[kNW];
    u32x4 sx;
    u32x2 sw;
  };
  auto fetch_fast = [&](int kb0, Staged& f) {
    const int8_t* xs = xtile + (int64_t)kb0 * kQK;
    const uint8_t* ws = wtile + (int64_t)kb0 * kWB;
#pragma unroll
    for (int i = 0; i < kNA; ++i) f.a[i] = *gptr(reinterpret_cast<const i32x4*>(xs + aoff[i]));
#pragma unroll
    for (int i = 0; i < kNW; ++i) f.w[i] = __builtin_nontemporal_load(gptr(reinterpret_cast<const u32x4*>(ws + woff[i])));
    f.sx = *gptr(reinterpret_cast<const u32x4*>(xdtile + kb0 + xsoff));
    f.sw = *gptr(reinterpret_cast<const u32x2*>(dtile + kb0 + wsoff));
  };
  auto fetch_any = [&](int kb0, Staged& f) {
#pragma unroll
    for (int i = 0; i < kNA; ++i) {
      const int c = 256 * i + tid;
      const int n = min(n0 + c / 8, B - 1);
      const int blk = min(kb0 + (c % 8) / 2, nb - 1);
      f.a[i] = *gptr(reinterpret_cast<const i32x4*>(xq + (int64_t)n * K + (int64_t)blk * kQK + 16 * (c % 2)));
    }
#pragma unroll
    for (int i = 0; i < kNW; ++i) {
      const int c = 256 * i + tid;
      if constexpr (WF == kWeightQ8) {
        const int m = min(m0 + c / 8, M - 1);
        const int blk = min(kb0 + (c % 8) / 2, nb - 1);
        f.w[i] = __builtin_nontemporal_load(gptr(
            reinterpret_cast<const u32x4*>(qs + (int64_t)m * row_bytes + (int64_t)blk * kQK + 16 * (c % 2))));
      } else {
        const int m = min(m0 + c / 4, M - 1);
        const int blk = min(kb0 + c % 4, nb - 1);
        f.w[i] = __builtin_nontemporal_load(
            gptr(reinterpret_cast<const u32x4*>(qs + (int64_t)m * row_bytes + (int64_t)blk * 16)));
      }
    }
    if (tid < 128) {
      const Q4Q8_GLOBAL uint32_t* p = gptr(reinterpret_cast<const uint32_t*>(xdtile + xsoff));
      f.sx = u32x4{p[min(kb0, nb - 1)], p[min(kb0 + 1, nb - 1)], p[min(kb0 + 2, nb - 1)], p[min(kb0 + 3, nb - 1)]};
    } else {
      const Q4Q8_GLOBAL uint16_t* p = gptr(dtile + wsoff);
      f.sx = u32x4{p[min(kb0, nb - 1)], p[min(kb0 + 1, nb - 1)], p[min(kb0 + 2, nb - 1)], p[min(kb0 + 3, nb - 1)]};
    }
    f.sw = u32x2{0u, 0u};  // every field written on both paths: nothing to merge
  };

  // packed: the weight scales are in sw (fetch_fast), else one per word of sx.
  auto store_stage = [&](GemmStage& sg, bool packed, const Staged& f) {
#pragma unroll
    for (int i = 0; i < kNA; ++i) {
      const int c = 256 * i + tid;
      const int t = c / 8, blk = (c % 8) / 2, hh = c % 2;
      *reinterpret_cast<i32x4*>(&sg.a[blk].v[t / 32][0][0][0] + piece_off(t, hh)) = f.a[i];
    }
    if constexpr (WF == kWeightQ8) {
#pragma unroll
      for (int i = 0; i < kNW; ++i) {
        const int c = 256 * i + tid;
        const int r = c / 8, blk = (c % 8) / 2, hh = c % 2;
        *reinterpret_cast<u32x4*>(&sg.w[blk].v[r / 32][0][0][0] + piece_off(r, hh)) = f.w[i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < kNW; ++i) {
        const int c = 256 * i + tid;
        const int r = c / 4, blk = c % 4;
        const u32x4 qv = f.w[i];
        const u32x4 lo = {nib_hi_to_s8x16(qv.x << 4), nib_hi_to_s8x16(qv.y << 4), nib_hi_to_s8x16(qv.z << 4),
                          nib_hi_to_s8x16(qv.w << 4)};
        const u32x4 hi = {nib_hi_to_s8x16(qv.x), nib_hi_to_s8x16(qv.y), nib_hi_to_s8x16(qv.z),
                          nib_hi_to_s8x16(qv.w)};
        *reinterpret_cast<u32x4*>(&sg.w[blk].v[r / 32][0][0][0] + piece_off(r, 0)) = lo;
        *reinterpret_cast<u32x4*>(&sg.w[blk].v[r / 32][0][0][0] + piece_off(r, 1)) = hi;
      }
    }
    if (tid < 128) {
      // reinterpret the whole vector (hipcc miscompiles a bit cast of one
      // element of a vector value: it reads element 0)
      const f32x4 v = __builtin_bit_cast(f32x4, f.sx);
      sg.dx[0][sr] = v.x;
      sg.dx[1][sr] = v.y;
      sg.dx[2][sr] = v.z;
      sg.dx[3][sr] = v.w;
    } else {
      const uint32_t b0 = packed ? f.sw.x & 0xFFFFu : f.sx.x, b1 = packed ? f.sw.x >> 16 : f.sx.y;
      const uint32_t b2 = packed ? f.sw.y & 0xFFFFu : f.sx.z, b3 = packed ? f.sw.y >> 16 : f.sx.w;
      // Q4: the MFMA sums 16 I, so the scale is taken as d_w / 16 (exact)
      constexpr float ws = WF == kWeightQ8 ? 1.0f : 0.0625f;
      const float w0 = ws * f16_bits_to_f32((uint16_t)b0), w1 = ws * f16_bits_to_f32((uint16_t)b1);
      const float w2 = ws * f16_bits_to_f32((uint16_t)b2), w3 = ws * f16_bits_to_f32((uint16_t)b3);
      sg.dwc[0][sr] = f32x2{w0, -kMagic * w0};
      sg.dwc[1][sr] = f32x2{w1, -kMagic * w1};
      sg.dwc[2][sr] = f32x2{w2, -kMagic * w2};
      sg.dwc[3][sr] = f32x2{w3, -kMagic * w3};
    }
  };

  float acc[kJT][16];
#pragma unroll
  for (int j = 0; j < kJT; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.0f;
  // The seed lives in vector registers for the whole tile (the MFMA reads it
  // as its accumulator input); materialised through asm so that the compiler
  // does not keep it in scalar registers and copy it over before every MFMA.
  v16i seed;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    int v;
    asm volatile("v_mov_b32 %0, %1" : "=v"(v) : "s"(kMagicBits));
    seed[r] = v;
  }
  const int loff = piece_off(l32, h);  // this lane's 16-byte piece in a row-group region

  // Stage pipeline: stage s + 1 is fetched (the fast form when it is full
  // and the scale rows are aligned) while stage s is computed, and stored to
  // the other LDS buffer after it; one barrier per stage.
  Staged f;
  fetch_any(0, f);
  store_stage(st[0], false, f);
  __syncthreads();
  // Q4 tiles without block-sum output take two stages per iteration of the
  // outer loop (the inner loop unrolled), so that the buffer index is a
  // constant and every LDS address a per-lane offset plus a constant (fewer
  // vector instructions per stage); the other instances have no registers to
  // spare for the second set of addresses.
  constexpr int kUnroll = (!WRITE_I && WF == kWeightQ4) ? 2 : 1;
  for (int kb00 = 0; kb00 < nb; kb00 += kUnroll * kKB) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int kb0 = kb00 + u * kKB;
      if (kb0 >= nb) break;
      const int buf = kUnroll == 2 ? u : (kb0 / kKB) & 1;
      const bool more = kb0 + kKB < nb;
      const bool fast = fast_ok && kb0 + 2 * kKB <= nb;
      if (more) {  // in flight during this stage's compute
        if (fast)
          fetch_fast(kb0 + kKB, f);
        else
          fetch_any(kb0 + kKB, f);
      }
      const GemmStage& sg = st[buf];
      auto lds_a = [&](int blk) { return *reinterpret_cast<const v4i*>(&sg.a[blk].v[wave][0][0][0] + loff); };
      auto lds_w = [&](int blk, int jt) { return *reinterpret_cast<const v4i*>(&sg.w[blk].v[jt][0][0][0] + loff); };
      auto lds_dwc = [&](int blk, int jt) { return sg.dwc[blk][jt * 32 + l32]; };
      // LDS operands are read one MFMA ahead of their use (kAhead): a block's
      // first two weight fragments (and the activation fragment) during the
      // previous block's last tiles, fragments 2 and 3 while tile 0 is
      // rescaled, so that no MFMA waits for an LDS read that was issued just
      // before it.  The block-sum instances read each fragment just before its
      // MFMA: their block-sum stores leave no registers for operands in flight.
      constexpr bool kAhead = !WRITE_I;
      v4i a, bf[kJT];
      f32x2 dwf[kJT];
      if constexpr (kAhead) {
        a = lds_a(0);
        bf[0] = lds_w(0, 0);
        bf[1] = lds_w(0, 1);
        dwf[0] = lds_dwc(0, 0);
        dwf[1] = lds_dwc(0, 1);
      }
#pragma unroll
      for (int blk = 0; blk < kKB; ++blk) {
        if (kb0 + blk < nb) {
          float dx[16];
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f32x4 v = *reinterpret_cast<const f32x4*>(&sg.dx[blk][wave * 32 + 8 * g + 4 * h]);
            dx[4 * g + 0] = v.x;
            dx[4 * g + 1] = v.y;
            dx[4 * g + 2] = v.z;
            dx[4 * g + 3] = v.w;
          }
          // The 4 tiles of the block in a pipeline: tile jt + 1's MFMA is
          // issued before tile jt is rescaled, so at most two results are live
          // (the register budget of two workgroups per CU).  Scheduling
          // barriers keep that order.
          // Whole result vectors are reinterpreted: hipcc (ROCm 7.2)
          // miscompiles a per-element int <-> float bit cast of an MFMA
          // result, propagating element 0 to every element.
          if constexpr (!kAhead) {
            a = lds_a(blk);
            bf[0] = lds_w(blk, 0);
            dwf[0] = lds_dwc(blk, 0);
          }
          v16i Di = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, bf[0], seed, 0, 0, 0);
          if constexpr (kAhead) {
            bf[2] = lds_w(blk, 2);
            dwf[2] = lds_dwc(blk, 2);
          }
#pragma unroll
          for (int jt = 0; jt < kJT; ++jt) {
            v16i Dn;
            if (jt + 1 < kJT) {
              if constexpr (!kAhead) {
                bf[jt + 1] = lds_w(blk, jt + 1);
                dwf[jt + 1] = lds_dwc(blk, jt + 1);
              }
              Dn = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, bf[jt + 1], seed, 0, 0, 0);
            }
            if (kAhead && jt == 0) {
              bf[3] = lds_w(blk, 3);
              dwf[3] = lds_dwc(blk, 3);
            }
            if (kAhead && jt == kJT - 2 && blk + 1 < kKB) {  // the last MFMA of the block has read a
              a = lds_a(blk + 1);
              bf[0] = lds_w(blk + 1, 0);
              bf[1] = lds_w(blk + 1, 1);
              dwf[0] = lds_dwc(blk + 1, 0);
              dwf[1] = lds_dwc(blk + 1, 1);
            }
            __builtin_amdgcn_sched_barrier(0);
            if (WRITE_I) {
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const int n = n0 + wave * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                const int m = m0 + jt * 32 + l32;
                // Q4 operands carry 16 (q - 8): the exact multiple of 16 is shifted back
                const int I = WF == kWeightQ8 ? Di[r] - kMagicBits : (Di[r] - kMagicBits) >> 4;
                if (n < B && m < M) Iout[((int64_t)n * M + m) * nb + kb0 + blk] = I;
              }
            }
            // Two passes, so that no fma waits on the one just before it
            // (back-to-back dependent vector instructions stall on gfx950):
            // t = fl(I * d_w) in place of F for all 16 elements, then the sums.
            const f32x2 dwc = dwf[jt];
            v16f Fv = __builtin_bit_cast(v16f, Di);
#pragma unroll
            for (int r = 0; r < 16; ++r) Fv[r] = __builtin_fmaf(Fv[r], dwc.x, dwc.y);
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[jt][r] = __builtin_fmaf(Fv[r], dx[r], acc[jt][r]);
            __builtin_amdgcn_sched_barrier(0);
            if (jt + 1 < kJT) Di = Dn;
          }
        }
      }
      // The other buffer was last read in the previous stage, which every wave
      // finished before the barrier that ended it.
      if (more) store_stage(st[buf ^ 1], fast, f);
      __syncthreads();
    }
  }

#pragma unroll
  for (int jt = 0; jt < kJT; ++jt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int n = n0 + wave * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
      const int m = m0 + jt * 32 + l32;
      if (n < B && m < M) y[(int64_t)n * M + m] = acc[jt][r];
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
  __shared__ __align__(16) GemmStage st[2];

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
