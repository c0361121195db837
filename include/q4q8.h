/*
 * q4q8.h -- C ABI of the MI355X (gfx950) Q4-weight x Q8-activation library.
 *
 * The operation.  "GGML：Backend 抽象与硬件加速", sections "Metal 与 Vulkan：
 * 默认路径和生成路径" and "硬件选择怎样映射到本栈": every backend multiplies
 * 4-bit block-quantised weights by 8-bit block-quantised activations with the
 * same arithmetic; only the kernel changes with the hardware.  Section "CUDA：
 * mmvq、mmq、cublas 三条矩阵路" of the same page routes a quantised
 * matrix x vector product (decode) to a dedicated vector kernel and larger
 * quantised products (prefill) to a matrix kernel.  The page "llama.cpp
 * b10909：Metal后端融合表重构，修复约5% token生成性能回退" restores the fused
 * RMS_NORM+MUL pattern whose loss cost about 5% of token generation; here it is
 * the prologue that normalises, scales and quantises each activation row.
 *
 * Block format (fixed by this project; the pages defer it to a chapter that is
 * not among them):
 *   - 32 consecutive elements along K form a block; K must be a multiple of 32;
 *   - Q4 weights: per block an fp16 scale d_w and 32 codes q in [0,15]
 *     meaning (q - 8) * d_w;
 *   - Q8 activations: per block an fp32 scale d_x and 32 int8 codes;
 *   - I = sum_j (q_j - 8) * x_j is exact in int32; the output is the fp32 sum
 *     over blocks of I * d_w * d_x.
 *
 * Plane layouts (row-major, caller-owned device memory):
 *   qs u8  [M][K/2]   block b of row m at byte m*K/2 + 16b; byte j holds code j
 *                     in its low nibble and code j+16 in its high nibble
 *   d  u16 [M][K/32]  fp16 bit patterns of the weight block scales
 *   xq i8  [B][K]     activation codes, one row per activation column / token
 *   xd f32 [B][K/32]  activation block scales
 *   xs i32 [B][K/32]  (optional) sum of the 32 codes of each activation block
 *   y  f32 [B][M]     output, y[n][m] = sum over blocks of row m and column n
 *
 * Conventions common to every entry point:
 *   - All array pointers are device pointers owned by the caller; the library
 *     never frees, retains or allocates them.  Calls allocate no device memory.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  All
 *     work is enqueued asynchronously on it; the call returns after launch.
 *     Inputs must stay unmodified and outputs unread until the stream reaches
 *     the call (synchronise before reusing buffers).
 *   - Arguments are validated on the host before anything is launched.  A bad
 *     call returns a negative status, launches nothing and writes nothing;
 *     q4q8_last_error() then returns a message for the calling thread.
 *   - Empty problems (M == 0 or B == 0 or T == 0) are valid and launch nothing.
 *   - NaN or infinite inputs give unspecified (but memory-safe) results.
 *   - The current HIP device must be a gfx950 GPU.
 */
#ifndef Q4Q8_H
#define Q4Q8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define Q4Q8_OK 0
#define Q4Q8_E_ARG (-1)         /* null pointer, bad dimension, K % 32 != 0, ... */
#define Q4Q8_E_ALIGN (-2)       /* a pointer violates its alignment requirement */
#define Q4Q8_E_ARCH (-3)        /* current device is not gfx950 */
#define Q4Q8_E_LAUNCH (-4)      /* the HIP runtime reported a launch error */
#define Q4Q8_E_UNSUPPORTED (-5) /* valid request outside what is built */

/* Flags of q8_quantize_rmsnorm (and of a q4q8_gemv_desc). */
#define Q8_NO_NORM 1u /* quantise x as it is: no normalisation, g ignored */
/* Flag of a q4q8_gemv_desc: the product's weights are Q8_0 planes (qs points
 * to int8 codes [M][K], 16-byte aligned; d as for Q4), see mul_mat_q8_0_q8. */
#define Q4Q8_WEIGHTS_Q8_0 2u

/* Message describing the last failed call on this thread ("" if none).  The
 * error convention follows the supports_op idea of "GGML：Backend 抽象与硬件
 * 加速" (section "注册顺序决定默认优先级"): a request the library cannot serve
 * is rejected explicitly with a reason, never computed wrongly.  The string
 * lives in thread-local storage owned by the library and stays valid until
 * the thread's next library call; the call never fails. */
const char* q4q8_last_error(void);

/* Library version as major*10000 + minor*100 + patch. */
int q4q8_version(void);

/*
 * q4_quantize -- load-time quantisation of fp32 weights to the Q4 planes.
 * Rule per 32-block: amax = max |w|; m = the element of lowest index with
 * |w| = amax; d = m / -8 (fp32); codes = clamp(trunc(w * (1/d) + 8.5), 0, 15)
 * from that fp32 d; stored scale = fp16(d) rounded to nearest even; an
 * all-zero block stores d = +0 and codes 8.  (The page on the GGML backends,
 * section "构建开关如何变成运行时能力", places weight re-layout at load time;
 * this call is where the kernel-friendly SoA planes are produced.)
 *   w  [M][K] f32, 16-byte aligned      qs [M][K/2] u8, 16-byte aligned
 *   d  [M][K/32] u16, 2-byte aligned     M * K / 32 <= 2^38 (else Q4Q8_E_ARG)
 */
int q4_quantize(const float* w, int64_t M, int64_t K, uint8_t* qs, uint16_t* d, void* stream);

/*
 * q8_quantize_rmsnorm -- fused activation prologue (RMS_NORM + MUL + Q8).
 * Per row x[0..K-1]: p_b = fp32 sum of x^2 over block b in index order; the
 * p_b are padded with zeros to a power-of-two count and summed pairwise,
 * adjacent pairs, level by level; s = 1 / sqrt(sum / K + eps); v = (x * s) * g
 * (two roundings, so the result equals the unfused RMS_NORM then MUL).  Then
 * per 32-block: d = amax(|v|) / 127 (fp32), codes = roundf(v * (1/d)) with
 * halves away from zero, clamped to [-127, 127]; an all-zero block gives d = 0
 * and codes 0.  Codes and scales are bit-exact results of those fp32 steps.
 * flags & Q8_NO_NORM: v = x (g may be NULL, eps ignored).
 *   x  [B][K] f32, 16-byte aligned      g  [K] f32, 16-byte aligned
 *   xq [B][K] i8, 16-byte aligned       xd [B][K/32] f32, 4-byte aligned
 *   xs [B][K/32] i32 or NULL
 *   K <= 131072.
 */
int q8_quantize_rmsnorm(const float* x, int64_t B, int64_t K, const float* g, float eps,
                        uint32_t flags, int8_t* xq, float* xd, int32_t* xs, void* stream);

/*
 * q8_quantize_rmsnorm_add -- activation prologue RMS_NORM + MUL + ADD + Q8.
 * The Metal fusion page ("llama.cpp b10909：Metal后端融合表重构，修复约5% token
 * 生成性能回退", its fusion-pattern counts) lists RMS_NORM+MUL+ADD beside
 * RMS_NORM+MUL.  Per row: s as for q8_quantize_rmsnorm, then
 *   v = ((x * s) * g) + a_row        (three fp32 roundings, in this order)
 * and the same per-block Q8 quantisation; codes, scales and code sums are
 * bit-exact results of those steps.
 *   a  addend: a_row_stride == 0 -> one [K] row for every input row,
 *      a_row_stride == K -> [B][K], row b at a + b * K; 16-byte aligned
 *   other arguments as q8_quantize_rmsnorm (no flags: the norm is applied)
 *   K <= 131072.
 */
int q8_quantize_rmsnorm_add(const float* x, int64_t B, int64_t K, const float* g, const float* a,
                            int64_t a_row_stride, float eps, int8_t* xq, float* xd, int32_t* xs, void* stream);

/*
 * q8_quantize_swiglu -- SwiGLU -> Q8, the producer of the down projection's
 * input.  The OpenVINO page ("llama.cpp b10981发布：OpenVINO后端优化有状态解码
 * 与GPU MoE推理") handles the GLU op swiglu and its rounding drift; the op is
 * silu(gate) * up.  Per element h = fl(silu(gate) * up) with
 * silu(g) = fl(g / fl(1 + exp_q(-g))), exp_q a fixed fp32 algorithm (Cody-Waite
 * reduction by ln 2, degree-7 Taylor polynomial, exact 2^n scaling; domain
 * [-17, 88], 0 below, +inf above; about 1.2 ulp), so that the Q8 codes, scales
 * and code sums of h (the q8_quantize_rmsnorm block rule) are bit-exact.
 *   gate, up  rows of F f32, row b at gate + b * row_stride and up + b * row_stride
 *             (a stacked [B][2F] gate|up buffer: up = gate + F, row_stride = 2F);
 *             16-byte aligned, row_stride >= F and a multiple of 4
 *   xq [B][F] i8 (16-byte aligned), xd [B][F/32] f32, xs [B][F/32] i32 or NULL
 *   B * F / 32 <= 2^34 (else Q4Q8_E_ARG)
 * Outputs must not overlap the inputs.  Non-finite inputs give unspecified codes.
 */
int q8_quantize_swiglu(const float* gate, const float* up, int64_t B, int64_t F, int64_t row_stride, int8_t* xq,
                       float* xd, int32_t* xs, void* stream);

/*
 * mul_mat_q4q8 -- y = W x for M x K Q4 weights and B Q8 activation columns of
 * length K.  Route (section "CUDA：mmvq、mmq、cublas 三条矩阵路" of the GGML
 * backend page): small B takes the streaming matrix x vector kernel (the mmvq
 * role), larger B the int8-MFMA tiled kernel (the mmq role).  Both compute the
 * same block sums exactly; the fp32 accumulation order differs from the
 * sequential reference, so outputs agree to rounding only.
 *   qs [M][K/2] u8, 16-byte aligned     d  [M][K/32] u16, 2-byte aligned
 *   xq [B][K] i8, 16-byte aligned       xd [B][K/32] f32, 4-byte aligned
 *   y  [B][M] f32, 4-byte aligned, must not overlap the inputs
 */
int mul_mat_q4q8(const uint8_t* qs, const uint16_t* d, int64_t M, int64_t K, const int8_t* xq,
                 const float* xd, int64_t B, float* y, void* stream);

/*
 * Q8_0 weights -- the second weight type.  The GGML backend page (sections
 * "Metal 与 Vulkan：默认路径和生成路径" and "对照本栈") names Q8_0 beside Q4 as a
 * type the conversion bridge emits and every backend kernel set must learn.
 * A Q8_0 block is 32 signed int8 codes and one fp16 scale; its product with a
 * Q8 activation block is I = sum_j q_j x_j (exact in int32) times d_w d_x.
 *
 * q8_0_quantize -- fp32 weights to Q8_0 planes.  Rule per 32-block: the Q8
 * block rule of q8_quantize_rmsnorm (d = fl(amax / 127), id = fl(1 / d) or 0,
 * q = roundf(fl(w * id)) clamped to [-127, 127]) with codes from the fp32 d
 * and the stored scale fp16(d), nearest even.
 *   w  [M][K] f32, 16-byte aligned      qw [M][K] i8, 16-byte aligned
 *   d  [M][K/32] u16, 2-byte aligned     M * K / 32 <= 2^38 (else Q4Q8_E_ARG)
 */
int q8_0_quantize(const float* w, int64_t M, int64_t K, int8_t* qw, uint16_t* d, void* stream);

/*
 * mul_mat_q8_0_q8 -- y = W x for M x K Q8_0 weights and B Q8 activation
 * columns: mul_mat_q4q8 with the weight planes qw [M][K] i8 (16-byte aligned)
 * and d [M][K/32] u16.  Same routes (streaming kernel for B <= 8 within its
 * register classes, int8-MFMA tiled kernel otherwise), same exact block sums,
 * same rounding contract and errors.  Grouped launches take Q8_0 products
 * through the Q4Q8_WEIGHTS_Q8_0 descriptor flag; no folded-prologue or MoE
 * variant takes Q8_0 weights.
 */
int mul_mat_q8_0_q8(const int8_t* qw, const uint16_t* d, int64_t M, int64_t K, const int8_t* xq,
                    const float* xd, int64_t B, float* y, void* stream);

/*
 * mul_mat_q4q8_rmsnorm -- mul_mat_q4q8 with the activation prologue folded in:
 * the B fp32 activation rows x [B][K] go through exactly the steps of
 * q8_quantize_rmsnorm (same codes and scales, bit for bit) inside the product
 * kernel, so the Q8 planes never travel through HBM.  flags & Q8_NO_NORM
 * quantises x as it is (g may then be NULL).  Served by the streaming route
 * only: B <= 4, B * ceil(K / 2048) <= 8 (rounded up to a power of two), and
 * B*K + 8*B*(K/32) + 32 <= 65536 bytes of staging; otherwise
 * Q4Q8_E_UNSUPPORTED (call q8_quantize_rmsnorm, then mul_mat_q4q8).
 *   x [B][K] f32, g [K] f32 (both 16-byte aligned), y [B][M] f32.
 */
int mul_mat_q4q8_rmsnorm(const uint8_t* qs, const uint16_t* d, int64_t M, int64_t K, const float* x,
                         const float* g, float eps, uint32_t flags, int64_t B, float* y, void* stream);

/*
 * Grouped streaming products.  Decode issues many small independent products
 * (the Q/K/V projections share one activation row, gate/up another); on this
 * GPU a kernel launch costs more than streaming a small matrix, so one launch
 * serves a whole list.  (The GGML backend page's CUDA section gives launch
 * cost as the reason batch-1 products take the vector kernel.)
 *
 * Usage: fill q4q8_gemv_desc records on the host; q4q8_group_build validates
 * them and writes a table image into caller host memory plus a plan; the
 * caller copies the image unchanged to device memory (16-byte aligned) once;
 * mul_mat_q4q8_group then launches from the device table, any number of times
 * (it is safe to capture in a HIP graph).  Products with M == 0 are dropped.
 * Every product uses B activation columns, 1 <= B <= 65535: B <= 8 takes the
 * streaming kernel (every K must fit its register classes), larger B the
 * tiled int8-MFMA kernel.  Products must not write overlapping outputs.  Each
 * product's weights are Q4 planes, or Q8_0 planes with flags &
 * Q4Q8_WEIGHTS_Q8_0; one group may mix both.
 *
 * A product's activations are either Q8 planes (xq, xd; x == NULL) or fp32
 * rows x (xq == NULL) that go through the prologue of q8_quantize_rmsnorm
 * (g and eps, or flags & Q8_NO_NORM).  Each distinct fp32 input (same x, g,
 * K, eps and Q8_NO_NORM) is quantised once per call, by a prologue pass that runs
 * before the streaming pass, into the caller's device workspace
 * (plan->workspace_bytes, 16-byte aligned, passed to q4q8_group_build because
 * the table records point into it).  The workspace belongs to the group:
 * calls of one group that may overlap in time (different streams) race on it.
 * Products sharing an input therefore see the same codes, bit for bit those
 * of q8_quantize_rmsnorm.  One call is one launch, or two when any product
 * takes fp32 rows.
 */
typedef struct q4q8_gemv_desc {
  const uint8_t* qs;  /* [M][K/2] Q4 (or [M][K] Q8_0 codes, see flags), 16-byte aligned */
  const uint16_t* d;  /* [M][K/32] */
  int64_t M;
  int64_t K;
  const int8_t* xq;   /* [B][K] Q8 codes, or NULL */
  const float* xd;    /* [B][K/32] Q8 scales (with xq) */
  const float* x;     /* [B][K] fp32 activations (when xq == NULL), 16-byte aligned */
  const float* g;     /* [K] norm weight, 16-byte aligned (with x, unless Q8_NO_NORM) */
  float eps;
  uint32_t flags;     /* Q8_NO_NORM (fp32 rows quantised as they are), Q4Q8_WEIGHTS_Q8_0 */
  float* y;           /* [B][M] */
} q4q8_gemv_desc;

typedef struct q4q8_group_plan {
  uint32_t magic;          /* set by q4q8_group_build */
  int32_t B;
  int32_t n_records;       /* records in the table image: one per product, or on the multi-column
                              route one per run of a product's windows within a bin */
  int32_t n_prologue;      /* distinct fp32 inputs the prologue pass quantises */
  int64_t n_windows;       /* work windows of the streaming pass (rows of ~32 KiB of weights) */
  int64_t max_k;           /* largest K of a product (also selects the kernel instance) */
  int64_t map_offset;      /* byte offset of the window -> record map in the image */
  int64_t prologue_offset; /* byte offset of the prologue records in the image */
  int64_t table_bytes;     /* size of the table image */
  int64_t workspace_bytes; /* device workspace the prologue pass writes (0 if none) */
  int32_t weight_formats;  /* 1: all products Q4, 2: all Q8_0, 3: both (selects the kernel instance) */
  int32_t max_prologue_k;  /* largest K among the fp32 inputs of the prologue pass (0 if none);
                              sizes that pass's LDS, which Q8-plane products never enter */
  int32_t mfma_columns;    /* 1: the streaming pass runs the multi-column int8-MFMA kernel (B = 5..8,
                              one weight format, every K a multiple of 256 and >= 1024 for Q4, or
                              of 128 and >= 512 for Q8_0,
                              d and xd 16-byte aligned; windows of 64 rows), 0: the
                              lane-per-block one */
  int32_t mfma_grid;       /* multi-column route: workgroups of the streaming launch, the ones
                              resident at once on the device current at build time (2 per CU;
                              512 when no device answers).  The host packs the windows into one bin
                              of near-equal cost (rows x K) per workgroup; a product's windows may
                              then span several records, and the map is followed by mfma_grid + 1
                              window indices (the bins' bounds).  0 on the other routes. */
} q4q8_group_plan;
/* Every field is written by q4q8_group_build and read as it left them: a
 * launch checks their consistency but cannot detect every edited value. */

/* Validate n descriptors and fill the plan.  With table_host == NULL only the
 * plan is computed (table_bytes and workspace_bytes tell the sizes; workspace
 * may then be NULL); otherwise the table image (table_bytes >=
 * plan->table_bytes, 16-byte aligned host memory) is written, with the
 * records pointing into `workspace` (device memory of workspace_bytes >=
 * plan->workspace_bytes, 16-byte aligned; may be NULL when no product takes
 * fp32 rows).  Host only; no device work. */
int q4q8_group_build(const q4q8_gemv_desc* descs, int32_t n, int64_t B, void* workspace,
                     size_t workspace_bytes, void* table_host, size_t table_bytes,
                     q4q8_group_plan* plan);
/* Launch every product of a built group from its device table image. */
int mul_mat_q4q8_group(const void* table_dev, const q4q8_group_plan* plan, void* stream);

/*
 * mul_mat_id_q4q8 -- expert-routed product (MUL_MAT_ID).  The scheduler
 * section of the GGML backend page ("调度器三遍切图，pipeline 四个副本") notes
 * that an expert matmul only touches the expert slices actually used; here the
 * weights of experts that no token selects are never read.
 *   qs  [E][M][K/2] u8 (16-byte aligned), d [E][M][K/32] u16
 *   xq  [T][n_x_slots][K] i8 (16-byte aligned), xd [T][n_x_slots][K/32] f32;
 *       n_x_slots is 1 (each token's row is shared by its top_k slots, as for
 *       gate/up) or top_k (one row per token and slot, as for down)
 *   ids [T][top_k] i32, expert index per token and slot
 *   y   [T][top_k][M] f32: y[t][s] = W[ids[t][s]] * x[t][n_x_slots==1 ? 0 : s];
 *       a row whose id lies outside [0, E) is filled with quiet NaNs
 *   ws  device workspace of at least mul_mat_id_q4q8_workspace(E, T, top_k)
 *       bytes, 16-byte aligned, owned by the caller; its contents on entry do
 *       not matter and on exit are unspecified.  Calls that share a workspace
 *       must be ordered on one stream.
 *   1 <= E <= 4096, T * top_k <= 65536, top_k <= 64, K <= 16384; M times
 *   (E + T * top_k / 8) must stay below about 2^31 / 33 / rows-per-window
 *   (Q4Q8_E_UNSUPPORTED otherwise; no expert layer comes near it).
 * Each selected expert's weights are streamed once per call (its routed
 * pairs taken up to 8 at a time); the routing runs on the device, and the
 * selected experts' row windows are split over the grid in equal shares of
 * estimated streaming cost.
 */
size_t mul_mat_id_q4q8_workspace(int64_t E, int64_t T, int64_t top_k);
int mul_mat_id_q4q8(const uint8_t* qs, const uint16_t* d, int64_t E, int64_t M, int64_t K,
                    const int8_t* xq, const float* xd, int64_t n_x_slots, const int32_t* ids,
                    int64_t T, int64_t top_k, float* y, void* ws, size_t ws_bytes, void* stream);

/*
 * mul_mat_id_q4q8_noalloc -- mul_mat_id_q4q8 without a workspace argument, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation.  Same arguments,
 * layouts, results (bit for bit) and errors as mul_mat_id_q4q8; the routing
 * workspace is instead a library-owned scratch array of
 * Q4Q8_NOALLOC_SCRATCH_BYTES in each GPU's memory, held from the first call on
 * that device until the process ends.  The call allocates nothing (no
 * hipMalloc, no hipFree, no allocating library routine).
 *   - Every call on one device shares that device's scratch, which keeps the
 *     last call's contents: calls that overlap on one GPU (on different
 *     streams, or from different threads without ordering) race.  Order them
 *     on one stream.  No content needs clearing between calls (the routing
 *     writes every word it reads).
 *   - A routing that needs more than the scratch returns Q4Q8_E_UNSUPPORTED
 *     with a message; every call valid for mul_mat_id_q4q8 (E <= 4096,
 *     T * top_k <= 65536) needs at most 573,464 bytes and fits.
 */
#define Q4Q8_NOALLOC_SCRATCH_BYTES ((size_t)1 << 20)
int mul_mat_id_q4q8_noalloc(const uint8_t* qs, const uint16_t* d, int64_t E, int64_t M, int64_t K,
                            const int8_t* xq, const float* xd, int64_t n_x_slots, const int32_t* ids,
                            int64_t T, int64_t top_k, float* y, void* stream);

/*
 * moe_expert_sum_f32 -- sum of the expert planes of a MUL_MAT_ID result.  The
 * OpenVINO page ("llama.cpp b10981发布：OpenVINO后端优化有状态解码与GPU MoE推理")
 * describes those planes being added by a chain of ADD ops after the routing
 * weights are applied, and notes that a reordered f32 reduction of the chain
 * drifts from the reference.  This call computes the chain in order:
 *   out[t][m] = fl(...fl(v_0 + v_1)... + v_{top_k-1}),  v_s = fl(w[t][s] * y[t][s][m])
 * (v_s = y[t][s][m] when w is null), one fp32 rounding per product and per
 * sum, so the result is bit-identical to that chain.
 *   y   [T][top_k][M] f32 device (e.g. mul_mat_id_q4q8's output), 4-byte aligned
 *   w   [T][top_k] f32 device routing weights, or null
 *   out [T][M] f32 device, must not overlap y
 *   1 <= top_k <= 64, T <= 65535.  A NaN plane (invalid expert id) gives NaN.
 * Async on `stream`.  Q4Q8_E_ARG / Q4Q8_E_ALIGN on invalid arguments.
 */
int moe_expert_sum_f32(const float* y, const float* w, int64_t T, int64_t top_k, int64_t M, float* out,
                       void* stream);

/* ---------------------------------------------------------------------------
 * Test hooks (not for production use).  The GGML backend page's CUDA section
 * keeps switches that force one matrix route only for cross-checking; these
 * are the equivalent.
 * ------------------------------------------------------------------------- */

#define Q4Q8_PATH_AUTO 0
#define Q4Q8_PATH_GEMV 1
#define Q4Q8_PATH_GEMM 2
#define Q4Q8_PATH_GEMV_LANES 3

/* Force the route taken by mul_mat_q4q8 and mul_mat_q8_0_q8 (process-wide).
 * Forcing GEMV for a shape it cannot hold returns Q4Q8_E_UNSUPPORTED.
 * Q4Q8_PATH_GEMV_LANES forces the streaming route with the lane-per-block
 * kernel, never the multi-column MFMA one; group plans built while it is
 * set use the lane-per-block kernel too (plan->mfma_columns == 0). */
int q4q8_set_path(int path);

/* Like mul_mat_q4q8, and also writes the exact per-block integer sums
 * I [B][M][K/32] (int32, 4-byte aligned) computed by the same kernel that
 * produced y (a debug instance of the same kernel template). */
int mul_mat_q4q8_blocksums(const uint8_t* qs, const uint16_t* d, int64_t M, int64_t K,
                           const int8_t* xq, const float* xd, int64_t B, float* y, int32_t* I,
                           void* stream);

/* mul_mat_q8_0_q8 that also writes the exact block sums I [B][M][K/32]
 * (int32, 4-byte aligned), as mul_mat_q4q8_blocksums. */
int mul_mat_q8_0_q8_blocksums(const int8_t* qw, const uint16_t* d, int64_t M, int64_t K, const int8_t* xq,
                              const float* xd, int64_t B, float* y, int32_t* I, void* stream);

/* Per-route dispatch counters since load or the last reset:
 * out[0] GEMV launches, out[1] GEMM launches, out[2] routed (MUL_MAT_ID)
 * calls, out[3] prologue launches.  reset != 0 clears them after reading
 * (atomically per counter; the counters are process-wide).  The analogue of
 * the fusion statistics of "llama.cpp b10909：Metal后端融合表重构，修复约5%
 * token生成性能回退" (section "融合统计与回归测试": counting which fused
 * kernels ran, so that a silently lost fusion shows): here they show which
 * route a call took.  out must hold 4 values; returns Q4Q8_E_ARG if null. */
int q4q8_dispatch_counts(uint64_t out[4], int reset);

/* Name of the kernel instance (demangled, with its template arguments) that
 * the calling thread's last library call launched last -- for a grouped call
 * the streaming or tiled pass, for a routed call its streaming pass -- or ""
 * before any launch.  Like the dispatch counters above, the analogue of the
 * fusion statistics of the Metal fusion page (section "融合统计与回归测试":
 * which fused kernels actually ran), so that a measurement can name the
 * instance it timed.  The string lives in thread-local storage owned by the
 * library and stays valid until the thread's next call of this function;
 * the call never fails. */
const char* q4q8_last_kernel(void);

#ifdef __cplusplus
}
#endif
#endif /* Q4Q8_H */
