// Device side of the streaming Q4 x Q8 matrix x vector kernel for gfx950:
// the register blocking classes, the window / segment streaming loop and the
// column policies.  gemv.hip builds the plain and grouped kernels on it,
// moe.hip the expert-routed one.
//
// One persistent kernel serves a single product and a grouped launch over
// many products (a device table of GemvProblem records plus a window ->
// record map).  Per product segment of a workgroup:
//   - lane l holds the activation codes of blocks kb0 + l, kb0 + l + 64, ...
//     in registers for the whole segment; each row is streamed with one
//     16-byte load per lane per 64 blocks (a whole 32-block, 1 KiB per wave
//     load, fully coalesced), nibbles unpacked in registers, v_dot4_i32_i8 on
//     the unsigned codes with the offset removed through the code sums
//     (I = sum q x - 8 sum x, exact), fp32 fma for the block scale;
//   - when B columns times the blocks per lane would not fit in registers,
//     K is split over S = 2 or 4 waves that stream the same rows (wave part
//     kp covers blocks kb0 = kp * 64 * J onwards); their per-row partial sums
//     meet in LDS and are added in part order;
//   - activations come either as Q8 planes (loaded straight into registers)
//     or, for a single product, as fp32 x + norm weight g, in which case the
//     workgroup runs the RMSNorm * g -> Q8 prologue itself (prologue_dev.h,
//     bit-identical to the standalone prologue) and stages the codes through
//     LDS;
//   - RU rows are in flight per wave in each of two register buffers (one is
//     computed while the other loads) and finished with one multi-row
//     butterfly.
// Column counts are padded to BT in {1, 2, 4, 8}; the true count B is a
// launch argument (columns past B read nothing and store nothing).
#pragma once

#include "prologue_dev.h"

namespace q4q8 {

constexpr int kGemvThreads = 256;
constexpr int kGemvWaves = kGemvThreads / kWave;
constexpr size_t kGemvMaxLds = 64 * 1024;

// Butterfly sum of N values per lane over each group of L consecutive lanes
// (L = 64: the whole wave).  Lane l returns the total, over its group, of
// value index (l % L) >> (log2 L - log2 N) (N <= L); each exchange step
// halves the number of values a lane carries, so the cost is
// N - 1 + log2 L - log2 N shuffles instead of N log2 L.
template <int N, int L = kWave>
__device__ __forceinline__ float multi_reduce(float (&v)[N], int lane) {
  static_assert(N <= L, "more values than lanes in a group");
#pragma unroll
  for (int s = N / 2, off = L / 2; s >= 1; s /= 2, off /= 2) {
    const bool upper = (lane & off) != 0;
#pragma unroll
    for (int i = 0; i < s; ++i) {
      // The empty asm pins both values in registers: otherwise the compiler
      // folds the lane-dependent choice into a load from a selected address,
      // which moves the array to scratch memory.
      float a = v[i], b = v[i + s];
      __asm__("" : "+v"(a), "+v"(b));
      const float send = upper ? a : b;
      const float keep = upper ? b : a;
      v[i] = keep + __shfl_xor(send, off, kWave);
    }
  }
  float r = v[0];
#pragma unroll
  for (int off = L / 2 / N; off >= 1; off /= 2) r += __shfl_xor(r, off, kWave);
  return r;
}

constexpr int ilog2_c(int n) { return n <= 1 ? 0 : 1 + ilog2_c(n / 2); }
constexpr int pow2_ceil_c(int n) { return n <= 1 ? 1 : 2 * pow2_ceil_c((n + 1) / 2); }

__device__ __forceinline__ int code_sum8(const i32x4 a, const i32x4 b) {
  int s = 0;
  s = __builtin_amdgcn_sdot4(a.x, 0x01010101, s, false);
  s = __builtin_amdgcn_sdot4(a.y, 0x01010101, s, false);
  s = __builtin_amdgcn_sdot4(a.z, 0x01010101, s, false);
  s = __builtin_amdgcn_sdot4(a.w, 0x01010101, s, false);
  s = __builtin_amdgcn_sdot4(b.x, 0x01010101, s, false);
  s = __builtin_amdgcn_sdot4(b.y, 0x01010101, s, false);
  s = __builtin_amdgcn_sdot4(b.z, 0x01010101, s, false);
  s = __builtin_amdgcn_sdot4(b.w, 0x01010101, s, false);
  return 8 * s;
}

#ifndef Q4Q8_GEMV_ROWS_IN_FLIGHT
#define Q4Q8_GEMV_ROWS_IN_FLIGHT 16  // 16-byte loads per lane in flight per row group
#endif

// 16-byte loads per lane in flight per row group for column width BT and
// weight format wf: a Q8_0 block takes two loads per lane, so half the rows
// keep the same bytes in flight.  (Raising it for 3..8 columns costs the
// second workgroup per CU and measured slower at every width.)
__host__ __device__ constexpr int gemv_rif(int BT, int wf) {
  (void)BT;
  return wf == kWeightQ8 ? Q4Q8_GEMV_ROWS_IN_FLIGHT / 2 : Q4Q8_GEMV_ROWS_IN_FLIGHT;
}

// Padded column count of the kernel instance serving B columns.
__host__ __device__ constexpr int gemv_bt(int B) { return B <= 1 ? 1 : B <= 2 ? 2 : B <= 4 ? 4 : 8; }

// Activation blocks (columns x blocks per lane) a lane may hold.
__host__ __device__ constexpr int gemv_act_budget(int BT) { return BT <= 4 ? 8 : 16; }

// Rows a wave keeps in flight per group for BT columns and J blocks per lane
// (at least 1; at most 64 / BT, so a group's outputs fit one value per lane).
__host__ __device__ constexpr int gemv_rows_per_wave(int BT, int J, int rif = Q4Q8_GEMV_ROWS_IN_FLIGHT) {
  const int r = rif / J / (BT <= 2 ? 1 : BT <= 4 ? 2 : 4);
  return r < 1 ? 1 : r > 64 / BT ? 64 / BT : r;
}

// Register blocking class of a product: J blocks per lane, K split over S
// waves (the smallest S whose blocks fit the register budget).  J == 0: the
// streaming kernel does not serve the shape.
struct GemvClass {
  int J, S;
};
// The class with the fewest waves per row whose blocks fit the register
// budget.  The folded prologue takes this class (it needs K in one wave).
__host__ __device__ constexpr GemvClass gemv_class_unsplit(int64_t K, int64_t B) {
  if (B < 1 || B > 8 || K < kQK) return {0, 0};
  const int64_t nb = K / kQK;
  const int BT = gemv_bt((int)B);
  for (int S = 1; S <= 4; S *= 2) {
    const int64_t per = (nb + 64 * S - 1) / (64 * S);
    const int J = per <= 1 ? 1 : per <= 2 ? 2 : per <= 4 ? 4 : per <= 8 ? 8 : 16;
    if (J <= 8 && BT * J <= gemv_act_budget(BT)) return {J, S};
  }
  return {0, 0};
}

// The class of every other streaming launch.  With Q4 weights one column
// prefers at most 4 blocks per lane and two columns at most 2, splitting K
// over 2 or 4 waves before they take more: a grouped instance without the
// larger classes fits two workgroups per CU (Llama-3-8B, K = 14336: 1.5-2%
// faster at B = 1 and at B = 2 than the larger classes at one workgroup per
// CU).  Q8_0 weights keep the unsplit class: the split measured 3-5% slower
// for them at B = 1.
__host__ __device__ constexpr GemvClass gemv_class_of(int64_t K, int64_t B, int wf = kWeightQ4) {
  if (B < 1 || B > 8 || K < kQK) return {0, 0};
  if (wf == kWeightQ8) return gemv_class_unsplit(K, B);
  const int64_t nb = K / kQK;
  if (gemv_bt((int)B) == 1)
    for (int S = 1; S <= 4; S *= 2) {
      const int64_t per = (nb + 64 * S - 1) / (64 * S);
      if (per <= 4) return {per <= 1 ? 1 : per <= 2 ? 2 : 4, S};
    }
  if (gemv_bt((int)B) == 2)
    for (int S = 1; S <= 4; S *= 2) {
      const int64_t per = (nb + 64 * S - 1) / (64 * S);
      if (per <= 2) return {per <= 1 ? 1 : 2, S};
    }
  return gemv_class_unsplit(K, B);
}

// Rows per window of the class serving K with column width BT (0: none);
// unsplit: the folded prologue's class, and the class of Q8_0 weights.
__host__ __device__ inline int gemv_window_rows_bt(int64_t K, int BT, int rif = Q4Q8_GEMV_ROWS_IN_FLIGHT,
                                                   bool unsplit = false) {
  const GemvClass c = unsplit ? gemv_class_unsplit(K, BT) : gemv_class_of(K, BT);
  if (c.J == 0) return 0;
  return (kGemvWaves / c.S) * gemv_rows_per_wave(BT, c.J, rif);
}

// rif: 16-byte loads per lane in flight per row group (fewer rows per wave
// leave registers for a second workgroup per CU).  LPR: lanes per row.  With
// LPR = 64 a row's blocks are spread over the whole wave; with LPR < 64 a
// load instruction covers 64 / LPR rows, one per group of LPR lanes, so rows
// of fewer than 64 blocks fill the wave (a row slot then holds 64 / LPR rows).
template <int BT, int J, int S, int RIF = Q4Q8_GEMV_ROWS_IN_FLIGHT, int LPR = kWave>
struct GemvShape {
  static constexpr int RPI = kWave / LPR;        // rows per load instruction
  static constexpr int RU = gemv_rows_per_wave(BT, J, RIF);  // row slots per wave
  static constexpr int SLOTS = kGemvWaves / S;  // row groups per window
  static constexpr int WIN = SLOTS * RU * RPI;  // rows per window
  static constexpr int NV = RU * BT;            // values reduced per lane group
  static constexpr int NP = pow2_ceil_c(NV);
  static constexpr int SHIFT = ilog2_c(LPR) - ilog2_c(NP);
  static_assert(NP <= LPR, "a lane group holds at most one value per lane");
};
constexpr int kMaxNP = 32;  // largest NP over all classes (checked below)

// LDS exchange of the K-split partial sums: two parities x waves x values.
struct SplitScratch {
  float v[2][kGemvWaves][kMaxNP];
};

// Where column c of a segment reads its Q8 activation row and writes its
// output row.  Dense: B consecutive rows of the product's own planes.
struct DenseCols {
  static constexpr bool kWeightsFirst = false;
  const int8_t* xq;
  const float* xd;
  float* y;
  int K, nb, M;
  __device__ __forceinline__ DenseCols(const GemvProblem& P)
      : xq(P.xq), xd(P.xd), y(P.y), K(P.K), nb(P.K >> 5), M(P.M) {}
  __device__ __forceinline__ const int8_t* act(int c) const { return xq + (int64_t)c * K; }
  __device__ __forceinline__ const float* scale(int c) const { return xd + (int64_t)c * nb; }
  __device__ __forceinline__ float* out(int c) const { return y + (int64_t)c * M; }
};

// Routed (expert) columns: column c is the (token, slot) pair
// list[beg + c] = t * top_k + s; its activation row is token t's (one row
// per token) or pair p's (one row per token and slot), its output row is
// pair p's in y [T][top_k][M].
struct RoutedCols {
  static constexpr bool kWeightsFirst = true;
  const int8_t* xq;
  const float* xd;
  float* y;
  const int32_t* list;
  int beg, K, nb, M, top_k, per_slot;
  __device__ __forceinline__ int pair(int c) const { return list[beg + c]; }
  __device__ __forceinline__ int64_t xrow(int c) const {
    const int p = pair(c);
    return per_slot ? (int64_t)p : (int64_t)(p / top_k);
  }
  __device__ __forceinline__ const int8_t* act(int c) const { return xq + xrow(c) * K; }
  __device__ __forceinline__ const float* scale(int c) const { return xd + xrow(c) * nb; }
  __device__ __forceinline__ float* out(int c) const { return y + (int64_t)pair(c) * M; }
};

// Streams windows [wl0, wl1) of product P (window i = rows i*WIN .. +WIN;
// the waves of row slot rs take the RU rows at rs*RU of each window, wave
// part kp its share of K) with J blocks per lane.  `parity` alternates over
// every compute of the workgroup (also across products) so that a K-split
// exchange never overwrites values a slower wave has yet to read.  WF: the
// weight format; a Q8_0 block is two loads, so the caller passes half the
// rows in flight (RIF) for the same bytes in flight.  LPR: lanes per row
// (GemvShape); lane l takes blocks kb0 + l % LPR + LPR j of row slot rows
// r * 64 / LPR + l / LPR.  PW: windows of one wave (RU * 64 / LPR rows; K in
// one wave only): the caller gives each wave its own window range, so the
// waves of a workgroup stream independently.
template <int BT, int J, int S, bool FOLD, bool WRITE_I, class Cols, int RIF = Q4Q8_GEMV_ROWS_IN_FLIGHT,
          int WF = kWeightQ4, int LPR = kWave, bool PW = false>
__device__ __forceinline__ void gemv_segment(const GemvProblem& P, const Cols& cols, int B, int wl0, int wl1,
                                             unsigned char* smem, SplitScratch* split, int& parity,
                                             int32_t* __restrict__ Iout) {
  using Sh = GemvShape<BT, J, S, RIF, LPR>;
  constexpr int RU = Sh::RU, NV = Sh::NV, NP = Sh::NP, SHIFT = Sh::SHIFT, RPI = Sh::RPI;
  constexpr int WIN = PW ? RU * RPI : Sh::WIN;  // rows per window (of the workgroup, or of this wave)
  static_assert(NP <= kMaxNP, "split scratch too small");
  static_assert(!FOLD || S == 1, "the folded prologue serves unsplit products");
  static_assert(!FOLD || WF == kWeightQ4, "the folded prologue serves Q4 weights");
  static_assert(LPR == kWave || (S == 1 && !FOLD), "rows shared by lane groups are neither split nor folded");
  static_assert(!PW || (S == 1 && !FOLD), "per-wave windows keep K in one wave");
  constexpr int NL = WF == kWeightQ8 ? 2 : 1;  // 16-byte loads per block and lane
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  int bl = lane, rl = 0;  // lane within its row's lane group; the group's row within a row slot
  if constexpr (LPR != kWave) {
    bl = lane & (LPR - 1);
    rl = lane / LPR;
  }
  if constexpr (LPR != kWave || Cols::kWeightsFirst) {
    // Opaque from here on (routed segments, which a caller runs in loops
    // beside the other widths' segments): otherwise the compiler hoists the
    // segment's per-lane 64-bit addresses out of those loops, where they stay
    // live across the other segments and spill.
    asm volatile("" : "+v"(bl), "+v"(rl));
  }
  const int rs = PW ? 0 : wave / S, kp = wave % S;
  const int kb0 = kp * LPR * J;
  const int M = P.M, K = P.K, nb = K >> 5;
  const int64_t row_bytes = WF == kWeightQ8 ? K : K >> 1;

  // Loads are unconditional, from addresses clamped into the segment's rows
  // (so an overrun re-reads a row just loaded, from cache, and never touches
  // rows another workgroup streams) and the block range: a guarded or masked
  // load becomes a branch that waits for its own data, which would serialise
  // the rows a wave keeps in flight.  Nothing needs masking: blocks past nb
  // meet zeroed activation registers (their product is exactly 0) and rows
  // past the segment are never stored.  Scales stay raw fp16 bits until used,
  // so no conversion waits on a prefetch.  Weights and scales are read once:
  // non-temporal loads keep them from displacing reusable lines.
  const int row_last = min(M, wl1 * WIN) - 1;
  auto load_group = [&](int row0, u32x4 (&w)[RU][J * NL], uint32_t (&dw)[RU][J]) {
#pragma unroll
    for (int r = 0; r < RU; ++r) {
      const int rowc = min(row0 + r * RPI + rl, row_last);
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int bc = min(kb0 + bl + LPR * j, nb - 1);
#pragma unroll
        for (int h = 0; h < NL; ++h)
          w[r][j * NL + h] = __builtin_nontemporal_load(
              &gptr(reinterpret_cast<const u32x4*>(P.qs))[rowc * (row_bytes / 16) + bc * NL + h]);
        dw[r][j] = __builtin_nontemporal_load(&gptr(P.d)[(int64_t)rowc * nb + bc]);
      }
    }
  };

  u32x4 wA[RU][J * NL], wB[RU][J * NL];
  uint32_t dA[RU][J], dB[RU][J];
  i32x4 xa[BT][J], xb[BT][J];
  float xdr[BT][J];
  int xsr[BT][J];
  if constexpr (!FOLD) {
    // Q8 planes: the activation loads go first (they are small and mostly
    // L2-resident), then the first two windows; loads complete in issue
    // order, so the first compute waits for the activations and window A
    // only while window B is already in flight.  Routed columns first look
    // their rows up in the routing list (two dependent reads), so there the
    // weight windows are requested before that lookup.
    if constexpr (Cols::kWeightsFirst) {
      load_group(wl0 * WIN + rs * RU * RPI, wA, dA);
      load_group((wl0 + 1) * WIN + rs * RU * RPI, wB, dB);
    }
#pragma unroll
    for (int c = 0; c < BT; ++c)
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int cc = min(c, B - 1);
        const int bc = min(kb0 + bl + LPR * j, nb - 1);
        const Q4Q8_GLOBAL i32x4* src =
            gptr(reinterpret_cast<const i32x4*>(cols.act(cc) + (int64_t)bc * kQK));
        xa[c][j] = src[0];
        xb[c][j] = src[1];
        xdr[c][j] = gptr(cols.scale(cc))[bc];
      }
    if constexpr (!Cols::kWeightsFirst) {
      load_group(wl0 * WIN + rs * RU * RPI, wA, dA);
      load_group((wl0 + 1) * WIN + rs * RU * RPI, wB, dB);
    }
#pragma unroll
    for (int c = 0; c < BT; ++c)
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const bool valid = c < B && kb0 + bl + LPR * j < nb;
        const i32x4 zero = {0, 0, 0, 0};
        xa[c][j] = valid ? xa[c][j] : zero;
        xb[c][j] = valid ? xb[c][j] : zero;
        xdr[c][j] = valid ? xdr[c][j] : 0.0f;
        // Q4 codes are unsigned (offset 8): remove 8 * sum x through the seed
        xsr[c][j] = WF == kWeightQ8 ? kMagicBits : kMagicBits - code_sum8(xa[c][j], xb[c][j]);
      }
  } else {
    // Folded-in prologue: window A is requested first, then the whole
    // workgroup quantises the activation rows (prologue_dev.h, the
    // register/butterfly form of the same steps) and stages the codes
    // through LDS; window B follows.
    load_group(wl0 * WIN + rs * RU, wA, dA);
    int8_t* sx = reinterpret_cast<int8_t*>(smem);                  // [B][K]
    float* sxd = reinterpret_cast<float*>(smem + (size_t)B * K);   // [B][nb]
    int* sxs = reinterpret_cast<int*>(sxd + B * nb);               // [B][nb]
    float* groups = reinterpret_cast<float*>(sxs + B * nb);        // [8]
    const bool raw = P.mode == kModeRaw;
    for (int c = 0; c < B; ++c)
      wg_q8_row_fast(P.x + (int64_t)c * K, P.g, K, P.eps, raw, sx + (size_t)c * K, sxd + c * nb,
                     sxs + c * nb, groups, tid);
#pragma unroll
    for (int c = 0; c < BT; ++c)
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int b = lane + kWave * j;
        if (c < B && b < nb) {
          const i32x4* src = reinterpret_cast<const i32x4*>(sx + (size_t)c * K + (size_t)b * kQK);
          xa[c][j] = src[0];
          xb[c][j] = src[1];
          xdr[c][j] = sxd[c * nb + b];
          xsr[c][j] = kMagicBits - 8 * sxs[c * nb + b];
        } else {
          xa[c][j] = i32x4{0, 0, 0, 0};
          xb[c][j] = i32x4{0, 0, 0, 0};
          xdr[c][j] = 0.0f;
          xsr[c][j] = kMagicBits;
        }
      }
    load_group((wl0 + 1) * WIN + rs * RU, wB, dB);
  }

  // The column a lane stores is fixed for the segment (value index
  // bl >> SHIFT of every row group), so its output row is looked up once.
  const int my_k = bl >> SHIFT, my_c = my_k % BT;
  float* const my_out = cols.out(min(my_c, B - 1));

  // One row group: block sums, scale, multi-row reduction, store (through
  // the part exchange when K is split).
  // The block sum is accumulated onto kMagicBits - 8 sum x for Q4 codes, onto
  // kMagicBits for Q8_0 codes (xsr holds that seed), so its bits read as the
  // float 1.5 * 2^23 + I (exact: |I| < 2^22 for both formats)
  // and I * d_w comes out of one fma against -1.5 * 2^23 * d_w (exact: 2 + 11
  // significant bits) with a single rounding -- no integer subtract, no
  // conversion, and the column's d_x is applied by a second fma.
  auto compute_group = [&](int row0, const u32x4 (&w)[RU][J * NL], const uint32_t (&dw)[RU][J]) {
    float acc[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i) acc[i] = 0.0f;
#pragma unroll
    for (int j = 0; j < J; ++j)
#pragma unroll
      for (int r = 0; r < RU; ++r) {
        const float dwf = f16_bits_to_f32((uint16_t)dw[r][j]);
        const float cwf = -kMagic * dwf;
#pragma unroll
        for (int c = 0; c < BT; ++c) {
          int Fb;
          if constexpr (WF == kWeightQ8)
            Fb = dot_block_q8(w[r][2 * j], w[r][2 * j + 1], xa[c][j], xb[c][j], xsr[c][j]);
          else
            Fb = dot_block(w[r][j], xa[c][j], xb[c][j], xsr[c][j]);
          const float t = __builtin_fmaf(__builtin_bit_cast(float, Fb), dwf, cwf);
          acc[r * BT + c] = __builtin_fmaf(t, xdr[c][j], acc[r * BT + c]);
          if (WRITE_I) {
            const int I = Fb - kMagicBits;
            const int b = kb0 + bl + LPR * j;
            const int row = row0 + r * RPI + rl;
            if (c < B && b < nb && row <= row_last) Iout[((int64_t)c * M + row) * nb + b] = I;
          }
        }
      }
    const float v = multi_reduce<NP, LPR>(acc, lane);
    const int k = my_k, c = my_c;
    const bool holder = (bl & ((1 << SHIFT) - 1)) == 0 && k < NV;
    const int row = row0 + (k / BT) * RPI + rl;
    if constexpr (S == 1) {
      if (holder && c < B && row <= row_last) gptr_w(my_out)[row] = v;
    } else {
      if (holder) split->v[parity][wave][k] = v;
      lds_barrier();
      if (kp == 0 && holder && c < B && row <= row_last) {
        float t = v;
#pragma unroll
        for (int q = 1; q < S; ++q) t += split->v[parity][wave + q][k];
        gptr_w(my_out)[row] = t;
      }
      parity ^= 1;
    }
  };

  // Ping-pong over two register buffers: while one window is computed the
  // other is in flight; a buffer is refilled right after it is consumed.
  for (int wi = wl0; wi < wl1; wi += 2) {
    const int r0 = wi * WIN + rs * RU * RPI;
    compute_group(r0, wA, dA);
    load_group(r0 + 2 * WIN, wA, dA);
    if (wi + 1 >= wl1) break;
    compute_group(r0 + WIN, wB, dB);
    load_group(r0 + 3 * WIN, wB, dB);
  }
}


// Calls f.template operator()<J, S>() for the blocking class (J, S) of
// column width BT; every class gemv_class_of can return for BT is listed.
template <int BT, typename F>
__host__ __device__ __forceinline__ void dispatch_class(int J, int S, F&& f) {
  if constexpr (BT == 1) {
    if (S == 1 && J == 1) f.template operator()<1, 1>();
    if (S == 1 && J == 2) f.template operator()<2, 1>();
    if (S == 1 && J == 4) f.template operator()<4, 1>();
    if (S == 2 && J == 4) f.template operator()<4, 2>();
    if (S == 4 && J == 4) f.template operator()<4, 4>();
    if (S == 1 && J == 8) f.template operator()<8, 1>();
    if (S == 2 && J == 8) f.template operator()<8, 2>();
    if (S == 4 && J == 8) f.template operator()<8, 4>();
  } else if constexpr (BT == 2) {
    if (S == 1 && J == 1) f.template operator()<1, 1>();
    if (S == 1 && J == 2) f.template operator()<2, 1>();
    if (S == 1 && J == 4) f.template operator()<4, 1>();
    if (S == 2 && J == 4) f.template operator()<4, 2>();
    if (S == 4 && J == 4) f.template operator()<4, 4>();
    if (S == 2 && J == 2) f.template operator()<2, 2>();
    if (S == 4 && J == 2) f.template operator()<2, 4>();
  } else {
    if (S == 1 && J == 1) f.template operator()<1, 1>();
    if (S == 1 && J == 2) f.template operator()<2, 1>();
    if (S == 2 && J == 2) f.template operator()<2, 2>();
    if (S == 4 && J == 2) f.template operator()<2, 4>();
  }
}


}  // namespace q4q8
