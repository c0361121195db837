/*
 * Q4-weight x Q8-activation oracle: plain, slow, single-threaded CPU code.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library may include,
 * link or call this file; only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark use it.  It shares no code, header, table or
 * helper with the HIP path.
 *
 * What it computes.  The page "GGML：Backend 抽象与硬件加速" (sections
 * "Metal 与 Vulkan：默认路径和生成路径" and "硬件选择怎样映射到本栈") states
 * that every backend honours one convention -- 4-bit quantised weights dotted
 * with 8-bit quantised activations -- and that hardware changes only the
 * kernel, never that arithmetic.  The block format itself is defined in an
 * earlier chapter that is not among the pages; this oracle uses the fixed
 * format of this project:
 *   - blocks of 32 consecutive elements along K;
 *   - a Q4 block is an fp16 scale d plus 32 4-bit codes q in [0,15] that
 *     stand for the values (q - 8) * d;
 *   - a Q8 block is an fp32 scale plus 32 int8 codes;
 *   - each block's integer dot product is exact in int32, is multiplied by
 *     d_w * d_x and the products are summed in fp32.
 * The fused RMSNorm -> multiply-by-norm-weight prologue follows the page
 * "llama.cpp b10909：Metal后端融合表重构..." (the RMS_NORM+MUL fusion it
 * restores).  Readings of every point the pages leave open are listed in the
 * function comments below.
 *
 * Parity status: every reading taken below is pinned by a test that the
 * plausible alternative reading fails: closed forms, hand-derived examples
 * re-derived on exact rationals, library routines or brute force.  The block
 * rules' reciprocal-multiply (id = 1/d, then w * id rather than w / d) and
 * their codes from the fp32 scale (not the stored fp16 one) are pinned by
 * blocks that sit on a rounding boundary between the two readings; the
 * within-block order of the sum of squares by a block whose sequential and
 * pairwise sums differ.  The fp32 summation order of the products is not a
 * reading: every order is correct there, and outputs are compared within a
 * tolerance.
 *
 * Plane layouts (all row-major, no padding):
 *   qs  u8  [M][K/2]  block b of row m occupies bytes m*K/2 + 16b .. +15;
 *                     byte j holds code j in its low nibble and code j+16
 *                     in its high nibble.
 *   d   u16 [M][K/32] fp16 bit patterns of the block scales.
 *   xq  i8  [B][K]    activation codes.
 *   xd  f32 [B][K/32] activation block scales.
 *   xs  i32 [B][K/32] sum of the 32 codes of each activation block.
 */
#ifndef Q4Q8_ORACLE_H
#define Q4Q8_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* IEEE 754 binary32 -> binary16, round to nearest even, with subnormals,
 * overflow to +-inf, NaN kept quiet. */
uint16_t orc_f32_to_f16(float f);
/* binary16 -> binary32 (exact). */
float orc_f16_to_f32(uint16_t h);

/* Bulk forms of the two conversions (for exhaustive tests). */
void orc_f32_to_f16_array(const float* in, int64_t n, uint16_t* out);
void orc_f16_to_f32_array(const uint16_t* in, int64_t n, float* out);

/* Q4 quantisation of W [M][K] (K % 32 == 0) into the qs / d planes. */
void orc_q4_quantize(const float* w, int64_t M, int64_t K, uint8_t* qs, uint16_t* d);

/* Unpack codes: q [M][K] u8 in [0,15] from the qs plane (layout inverse). */
void orc_q4_unpack_codes(const uint8_t* qs, int64_t M, int64_t K, uint8_t* q);

/* RMS normalisation of each row: out = x * s, s = 1/sqrt(mean(x^2) + eps),
 * with the fixed reduction order described in the source. */
void orc_rmsnorm(const float* x, int64_t B, int64_t K, float eps, float* out, float* scale_out);

/* Elementwise out[b][k] = v[b][k] * g[k] (the MUL of RMS_NORM+MUL). */
void orc_mul_rows(const float* v, int64_t B, int64_t K, const float* g, float* out);

/* Q8 quantisation of rows v [B][K] into xq / xd (/ xs if non-null). */
void orc_q8_quantize(const float* v, int64_t B, int64_t K, int8_t* xq, float* xd, int32_t* xs);

/* Fused prologue: RMSNorm, multiply by g, Q8 quantise.  Equal bit for bit
 * to orc_rmsnorm -> orc_mul_rows -> orc_q8_quantize.  no_norm != 0 skips
 * the norm and the multiply and quantises x as it is (g may be NULL). */
void orc_q8_quantize_rmsnorm(const float* x, int64_t B, int64_t K, const float* g, float eps,
                             int no_norm, int8_t* xq, float* xd, int32_t* xs);

/* Exact per-block integer dot products I [B][M][K/32] (int32). */
void orc_block_dots(const uint8_t* qs, int64_t M, int64_t K, const int8_t* xq, int64_t B, int32_t* I);

/* y [B][M] fp32: per row, blocks in ascending order,
 *   acc = acc + float(I) * (f32(d_w) * d_x).
 * y64 (nullable) [B][M]: the same terms summed in fp64 (exact products). */
void orc_mul_mat(const uint8_t* qs, const uint16_t* d, int64_t M, int64_t K,
                 const int8_t* xq, const float* xd, int64_t B, float* y, double* y64);

/* Same result, output rows split over nthreads POSIX threads.  Each output
 * element is computed by the identical sequential code, so the result is bit
 * for bit that of orc_mul_mat. */
void orc_mul_mat_mt(const uint8_t* qs, const uint16_t* d, int64_t M, int64_t K,
                    const int8_t* xq, const float* xd, int64_t B, float* y, double* y64,
                    int nthreads);

/* Expert-routed product.  Weights qs [E][M][K/2], d [E][M][K/32];
 * activations xq [T][n_x_slots][K], xd [T][n_x_slots][K/32] with
 * n_x_slots == 1 (one row per token, shared by its slots) or == top_k (one
 * row per token and slot); ids [T][top_k] int32.
 *   y[t][s][:] = orc_mul_mat(expert ids[t][s], row (t, n_x_slots==1 ? 0 : s))
 * An id outside [0, E) gives a row of quiet NaNs.  y [T][top_k][M]. */
void orc_mul_mat_id(const uint8_t* qs, const uint16_t* d, int64_t E, int64_t M, int64_t K,
                    const int8_t* xq, const float* xd, int64_t n_x_slots,
                    const int32_t* ids, int64_t T, int64_t top_k, float* y, int nthreads);

/* Q8_0 weights: the second weight type of the contract.  The GGML backend
 * page ("GGML：Backend 抽象与硬件加速", sections "Metal 与 Vulkan：默认路径和生
 * 成路径" and "对照本栈") has the conversion bridge pick Q4_K or Q8_0 and new
 * types appended to the type list, every backend kernel set learning each
 * one.  Reading: 32-element blocks, an fp16 scale and 32 int8 codes; the block
 * rule is the Q8 rule of the activations with the scale stored as fp16:
 *   amax = max |w|; d = fl(amax / 127); id = fl(1 / d) (0 if d == 0);
 *   q = roundf(fl(w * id)) (halves away from zero), clamped to [-127, 127];
 *   stored scale fp16(d), nearest even; codes from the fp32 d (as for Q4).
 * Planes: qw i8 [M][K] (block b of row m at m*K + 32b), d u16 [M][K/32].
 * The product is the Q4 product with I = sum_j qw_j * x_j (exact in int32:
 * |I| <= 32 * 127 * 127). */
void orc_q8w_quantize(const float* w, int64_t M, int64_t K, int8_t* qw, uint16_t* d);
void orc_block_dots_q8w(const int8_t* qw, int64_t M, int64_t K, const int8_t* xq, int64_t B, int32_t* I);
void orc_mul_mat_q8w_mt(const int8_t* qw, const uint16_t* d, int64_t M, int64_t K, const int8_t* xq,
                        const float* xd, int64_t B, float* y, double* y64, int nthreads);

/* RMS_NORM + MUL + ADD prologue.  The Metal fusion page ("llama.cpp
 * b10909：Metal后端融合表重构...", its fusion-pattern counts) lists the
 * RMS_NORM+MUL+ADD pattern beside RMS_NORM+MUL; reading: the three ops in that
 * order, each rounded as its own op, then Q8:
 *   v[b][k] = fl( fl( fl(x[b][k] * s_b) * g[k] ) + a_b[k] ),
 * s_b the RMS scale of orc_rmsnorm, a_b = a + b * a_row_stride (stride 0: one
 * [K] addend for every row; stride K: an addend row per row), then
 * orc_q8_quantize(v). */
void orc_q8_quantize_rmsnorm_add(const float* x, int64_t B, int64_t K, const float* g, const float* a,
                                 int64_t a_row_stride, float eps, int8_t* xq, float* xd, int32_t* xs);

/* SwiGLU -> Q8, the producer of the down projection's input.  The OpenVINO
 * page ("llama.cpp b10981发布...") handles the GLU op swiglu (with clamp) and
 * its f16 rounding drift; the op is silu(gate) * up.  Because the Q8 codes
 * must be bit-exact, the exponential is fixed here as an fp32 algorithm
 * (Cody-Waite argument reduction by ln 2 with a split constant, a degree-7
 * Taylor polynomial in Horner form, exact scaling by 2^n; every step one
 * fp32 rounding, no fused multiply-add):
 *   exp_q(t): NaN -> NaN; t > 88 -> +inf; t < -17 -> 0 (then 1 + e == 1 in
 *     fp32 anyway);  n = rint(fl(t * L2E)) (nearest even),
 *     r = fl(fl(t - fl(n * LN2_HI)) - fl(n * LN2_LO)),
 *     c = C7, then c = fl(fl(c * r) + C_k) for k = 6..1, p = fl(fl(c * r) + 1),
 *     e = p * 2^n (exact: n in [-25, 127], the result stays normal);
 *     L2E = 0x3fb8aa3b, LN2_HI = 0x3f317200 (8 trailing zero bits, so n * LN2_HI
 *     is exact), LN2_LO = 0x35bfbe8e, C_k = fp32(1 / k!) (C1 = 1).
 *   silu(g) = fl(g / fl(1 + exp_q(-g)));  h = fl(silu(gate) * up);
 * then orc_q8_quantize of h.  Rows: gate + b * row_stride, up + b * row_stride
 * (row_stride >= F; a stacked [B][2F] gate|up buffer uses row_stride = 2F). */
float orc_exp_q(float t);
float orc_silu(float g);
void orc_silu_array(const float* in, int64_t n, float* out);
void orc_exp_q_array(const float* in, int64_t n, float* out);
void orc_q8_quantize_swiglu(const float* gate, const float* up, int64_t B, int64_t F, int64_t row_stride,
                            int8_t* xq, float* xd, int32_t* xs);

/* Sum of the expert planes of a MUL_MAT_ID result.  The page "llama.cpp
 * b10981发布：OpenVINO后端优化有状态解码与GPU MoE推理" describes the expert
 * planes being added by a chain of ADD ops (and a reordered reduction of that
 * chain drifting in f32).  Each plane is first scaled by its routing weight
 * (a MUL), then the chain runs over the slots in order:
 *   v_s = fl(w[t][s] * y[t][s][m])              (w == NULL: v_s = y[t][s][m])
 *   out[t][m] = fl(...fl(fl(v_0 + v_1) + v_2)... + v_{top_k-1})
 * one fp32 rounding per product and per sum, no fused multiply-add.  A NaN
 * plane (an invalid expert id) makes the output NaN.  y [T][top_k][M],
 * w [T][top_k], out [T][M]; top_k >= 1. */
void orc_moe_expert_sum(const float* y, const float* w, int64_t T, int64_t top_k, int64_t M, float* out);

#ifdef __cplusplus
}
#endif
#endif
