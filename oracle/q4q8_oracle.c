/*
 * Q4-weight x Q8-activation oracle.  TEST INFRASTRUCTURE ONLY: see the
 * header for what it computes, the plane layouts and who may call it.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math (no FMA
 * contraction anywhere: every fp32 operation below is one IEEE-rounded
 * operation, and x86-64 evaluates float arithmetic in single precision).
 */
#include "q4q8_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

#define QK 32 /* elements per block */

/* ------------------------------------------------------------------ */
/* fp16 <-> fp32, written from the IEEE 754 binary16 definition:       */
/* 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits; exponent 0 */
/* encodes +-0 and subnormals m * 2^-24; exponent 31 encodes inf/NaN.  */
/* ------------------------------------------------------------------ */

uint16_t orc_f32_to_f16(float f) {
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    const uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    const uint32_t ef = (u >> 23) & 0xFFu;
    const uint32_t mf = u & 0x7FFFFFu;

    if (ef == 0xFFu) { /* inf or NaN */
        if (mf == 0) return (uint16_t)(sign | 0x7C00u);
        return (uint16_t)(sign | 0x7E00u | (mf >> 13)); /* quiet NaN */
    }
    /* Exact value = S * 2^E with S an integer significand. */
    uint64_t S;
    int E;
    if (ef == 0) {
        S = mf;
        E = -149;
    } else {
        S = (uint64_t)(0x800000u | mf);
        E = (int)ef - 150;
    }
    if (S == 0) return sign;

    int p = 63 - __builtin_clzll(S); /* S in [2^p, 2^(p+1)) */
    int e = p + E;                   /* unbiased exponent of the value */
    /* Quantum (spacing of binary16 numbers) at this magnitude: 2^(e-10)
     * for normals, 2^-24 in the subnormal range. */
    int qe = e - 10;
    if (qe < -24) qe = -24;
    int shift = qe - E;
    uint64_t R;
    if (shift <= 0) {
        R = S << (-shift); /* exactly representable */
    } else if (shift > 40) {
        R = 0; /* far below half a quantum */
    } else {
        R = S >> shift;
        const uint64_t rem = S & ((1ull << shift) - 1);
        const uint64_t half = 1ull << (shift - 1);
        if (rem > half || (rem == half && (R & 1u))) R += 1; /* ties to even */
    }
    if (qe == -24) {
        /* subnormal range: value = R * 2^-24; R == 1024 is the smallest
         * normal, whose bit pattern is also 1024 (exponent 1, fraction 0). */
        return (uint16_t)(sign | (uint16_t)R);
    }
    if (R == 2048) { /* rounding carried into the next binade */
        R = 1024;
        qe += 1;
    }
    const int e16 = qe + 25; /* value = R * 2^qe = (1024 + frac) * 2^(e16 - 25) */
    if (e16 >= 31) return (uint16_t)(sign | 0x7C00u); /* overflow -> inf */
    return (uint16_t)(sign | (uint16_t)(e16 << 10) | (uint16_t)(R - 1024));
}

float orc_f16_to_f32(uint16_t h) {
    const uint32_t sign = ((uint32_t)h & 0x8000u) << 16;
    const uint32_t e16 = ((uint32_t)h >> 10) & 0x1Fu;
    const uint32_t m = (uint32_t)h & 0x3FFu;
    uint32_t u;
    if (e16 == 0) {
        /* +-0 or subnormal: m * 2^-24, exact in binary32 */
        float v = ldexpf((float)m, -24);
        memcpy(&u, &v, sizeof u);
        u |= sign;
    } else if (e16 == 31) {
        u = sign | 0x7F800000u | (m << 13) | (m ? 0x400000u : 0u);
    } else {
        u = sign | ((e16 - 15 + 127) << 23) | (m << 13);
    }
    float out;
    memcpy(&out, &u, sizeof out);
    return out;
}

void orc_f32_to_f16_array(const float* in, int64_t n, uint16_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_f32_to_f16(in[i]);
}

void orc_f16_to_f32_array(const uint16_t* in, int64_t n, float* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_f16_to_f32(in[i]);
}

/* ------------------------------------------------------------------ */
/* Q4 quantisation (one 32-block at a time).                           */
/* Reading of the rule (the defining chapter is not among the pages):  */
/*  - amax = largest |w_j|; m = w_j at the lowest j reaching amax, so   */
/*    the sign of the scale follows the first extreme element;          */
/*  - d = m / -8 in fp32, so that value m maps to code 0 and the whole  */
/*    range [-8, 7] of q - 8 is used;                                   */
/*  - id = 1 / d; code = trunc(w*id + 8.5), clamped to [0, 15]          */
/*    (round half up in the scaled domain, the +8 offset folded in);    */
/*  - codes come from the fp32 d; the stored scale is fp16(d), RNE;     */
/*  - an all-zero block stores d = +0 and codes 8.                      */
/* ------------------------------------------------------------------ */

static void q4_block(const float* w, uint8_t* qs16, uint16_t* dbits) {
    float amax = 0.0f;
    float mval = 0.0f;
    for (int j = 0; j < QK; ++j) {
        const float a = fabsf(w[j]);
        if (a > amax) { /* strict: the lowest index wins a tie */
            amax = a;
            mval = w[j];
        }
    }
    uint8_t q[QK];
    if (amax == 0.0f) {
        *dbits = 0x0000u;
        for (int j = 0; j < QK; ++j) q[j] = 8;
    } else {
        const float d = mval / -8.0f;
        const float id = 1.0f / d;
        for (int j = 0; j < QK; ++j) {
            float t = w[j] * id;
            t = t + 8.5f;
            int qi = (int)t; /* truncation toward zero */
            if (qi > 15) qi = 15;
            if (qi < 0) qi = 0;
            q[j] = (uint8_t)qi;
        }
        *dbits = orc_f32_to_f16(d);
    }
    for (int j = 0; j < QK / 2; ++j) qs16[j] = (uint8_t)(q[j] | (q[j + QK / 2] << 4));
}

void orc_q4_quantize(const float* w, int64_t M, int64_t K, uint8_t* qs, uint16_t* d) {
    const int64_t nb = K / QK;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t b = 0; b < nb; ++b)
            q4_block(w + m * K + b * QK, qs + m * (K / 2) + b * (QK / 2), d + m * nb + b);
}

void orc_q4_unpack_codes(const uint8_t* qs, int64_t M, int64_t K, uint8_t* q) {
    const int64_t nb = K / QK;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t b = 0; b < nb; ++b)
            for (int j = 0; j < QK; ++j) {
                const uint8_t byte = qs[m * (K / 2) + b * (QK / 2) + (j % (QK / 2))];
                q[m * K + b * QK + j] = (j < QK / 2) ? (uint8_t)(byte & 0x0F) : (uint8_t)(byte >> 4);
            }
}

/* ------------------------------------------------------------------ */
/* RMSNorm.  Textbook RMS normalisation with eps added to the mean of  */
/* squares inside the square root (the OpenVINO page notes that the    */
/* translation keeps GGML's epsilon position; we read it as this one). */
/* Bit-exact codes downstream make the reduction order part of the     */
/* contract.  Order chosen:                                            */
/*   p_b  = sum over the 32 elements of block b, index order, fp32;    */
/*   pad p to the next power of two P with +0;                         */
/*   while P > 1: p[i] = p[2i] + p[2i+1] for i < P/2; P /= 2;          */
/*   ssq = p[0]; mean = ssq / K; s = 1 / sqrt(mean + eps);             */
/*   out = x * s.                                                      */
/* ------------------------------------------------------------------ */

static int64_t next_pow2(int64_t n) {
    int64_t p = 1;
    while (p < n) p *= 2;
    return p;
}

static float row_rms_scale(const float* x, int64_t K, float eps) {
    const int64_t nb = K / QK;
    int64_t P = next_pow2(nb);
    float* p = (float*)calloc((size_t)P, sizeof(float));
    for (int64_t b = 0; b < nb; ++b) {
        float acc = 0.0f;
        for (int j = 0; j < QK; ++j) {
            const float sq = x[b * QK + j] * x[b * QK + j];
            acc = acc + sq;
        }
        p[b] = acc;
    }
    while (P > 1) {
        for (int64_t i = 0; i < P / 2; ++i) p[i] = p[2 * i] + p[2 * i + 1];
        P /= 2;
    }
    const float ssq = p[0];
    free(p);
    const float mean = ssq / (float)K;
    const float r = sqrtf(mean + eps);
    return 1.0f / r;
}

void orc_rmsnorm(const float* x, int64_t B, int64_t K, float eps, float* out, float* scale_out) {
    for (int64_t b = 0; b < B; ++b) {
        const float s = row_rms_scale(x + b * K, K, eps);
        if (scale_out) scale_out[b] = s;
        for (int64_t k = 0; k < K; ++k) out[b * K + k] = x[b * K + k] * s;
    }
}

void orc_mul_rows(const float* v, int64_t B, int64_t K, const float* g, float* out) {
    for (int64_t b = 0; b < B; ++b)
        for (int64_t k = 0; k < K; ++k) out[b * K + k] = v[b * K + k] * g[k];
}

/* ------------------------------------------------------------------ */
/* Q8 quantisation of one 32-block: symmetric, d = amax / 127 in fp32, */
/* id = 1/d, code = roundf(v * id) (halves away from zero), clamped to */
/* [-127, 127]; all-zero block -> d = 0, codes 0.  The scale is kept   */
/* in fp32 (the format allows fp16 or fp32; fp32 avoids a rounding).   */
/* ------------------------------------------------------------------ */

static void q8_block(const float* v, int8_t* q, float* d_out, int32_t* s_out) {
    float amax = 0.0f;
    for (int j = 0; j < QK; ++j) {
        const float a = fabsf(v[j]);
        if (a > amax) amax = a;
    }
    const float d = amax / 127.0f;
    const float id = (d != 0.0f) ? 1.0f / d : 0.0f;
    int32_t sum = 0;
    for (int j = 0; j < QK; ++j) {
        const float t = v[j] * id;
        long qi = lroundf(t);
        if (qi > 127) qi = 127;
        if (qi < -127) qi = -127;
        q[j] = (int8_t)qi;
        sum += (int32_t)qi;
    }
    *d_out = d;
    if (s_out) *s_out = sum;
}

void orc_q8_quantize(const float* v, int64_t B, int64_t K, int8_t* xq, float* xd, int32_t* xs) {
    const int64_t nb = K / QK;
    for (int64_t b = 0; b < B; ++b)
        for (int64_t kb = 0; kb < nb; ++kb)
            q8_block(v + b * K + kb * QK, xq + b * K + kb * QK, xd + b * nb + kb,
                     xs ? xs + b * nb + kb : NULL);
}

void orc_q8_quantize_rmsnorm(const float* x, int64_t B, int64_t K, const float* g, float eps,
                             int no_norm, int8_t* xq, float* xd, int32_t* xs) {
    if (no_norm) {
        orc_q8_quantize(x, B, K, xq, xd, xs);
        return;
    }
    float* t = (float*)malloc((size_t)(B * K) * sizeof(float));
    float* v = (float*)malloc((size_t)(B * K) * sizeof(float));
    orc_rmsnorm(x, B, K, eps, t, NULL);
    orc_mul_rows(t, B, K, g, v);
    orc_q8_quantize(v, B, K, xq, xd, xs);
    free(t);
    free(v);
}

void orc_q8_quantize_rmsnorm_add(const float* x, int64_t B, int64_t K, const float* g, const float* a,
                                 int64_t a_row_stride, float eps, int8_t* xq, float* xd, int32_t* xs) {
    float* t = (float*)malloc((size_t)(B * K) * sizeof(float));
    float* v = (float*)malloc((size_t)(B * K) * sizeof(float));
    orc_rmsnorm(x, B, K, eps, t, NULL);
    orc_mul_rows(t, B, K, g, v);
    for (int64_t b = 0; b < B; ++b) {
        const float* ar = a + b * a_row_stride;
        for (int64_t k = 0; k < K; ++k) v[b * K + k] = v[b * K + k] + ar[k];
    }
    orc_q8_quantize(v, B, K, xq, xd, xs);
    free(t);
    free(v);
}

/* ------------------------------------------------------------------ */
/* Block integer dot: I = sum_j (q4_j - 8) * q8_j, exact in int32      */
/* (|I| <= 32 * 8 * 127 = 32512).                                       */
/* ------------------------------------------------------------------ */

static int32_t block_dot(const uint8_t* qs16, const int8_t* x32) {
    int32_t sum = 0;
    for (int j = 0; j < QK; ++j) {
        const uint8_t byte = qs16[j % (QK / 2)];
        const int32_t q = (j < QK / 2) ? (byte & 0x0F) : (byte >> 4);
        sum += (q - 8) * (int32_t)x32[j];
    }
    return sum;
}

void orc_block_dots(const uint8_t* qs, int64_t M, int64_t K, const int8_t* xq, int64_t B, int32_t* I) {
    const int64_t nb = K / QK;
    for (int64_t b = 0; b < B; ++b)
        for (int64_t m = 0; m < M; ++m)
            for (int64_t kb = 0; kb < nb; ++kb)
                I[(b * M + m) * nb + kb] =
                    block_dot(qs + m * (K / 2) + kb * (QK / 2), xq + b * K + kb * QK);
}

/* ------------------------------------------------------------------ */
/* Scale and accumulate one output element: blocks in ascending order, */
/* acc = acc + float(I) * (f32(d_w) * d_x), all in fp32.                */
/* ------------------------------------------------------------------ */

static float out_element(const uint8_t* qs_row, const uint16_t* d_row, int64_t K,
                         const int8_t* x_row, const float* xd_row, double* y64) {
    const int64_t nb = K / QK;
    float acc = 0.0f;
    double acc64 = 0.0;
    for (int64_t kb = 0; kb < nb; ++kb) {
        const int32_t I = block_dot(qs_row + kb * (QK / 2), x_row + kb * QK);
        const float dw = orc_f16_to_f32(d_row[kb]);
        const float c = dw * xd_row[kb];
        const float t = (float)I * c;
        acc = acc + t;
        acc64 += (double)I * (double)dw * (double)xd_row[kb];
    }
    if (y64) *y64 = acc64;
    return acc;
}

void orc_mul_mat(const uint8_t* qs, const uint16_t* d, int64_t M, int64_t K,
                 const int8_t* xq, const float* xd, int64_t B, float* y, double* y64) {
    const int64_t nb = K / QK;
    for (int64_t b = 0; b < B; ++b)
        for (int64_t m = 0; m < M; ++m)
            y[b * M + m] = out_element(qs + m * (K / 2), d + m * nb, K, xq + b * K, xd + b * nb,
                                       y64 ? &y64[b * M + m] : NULL);
}

typedef struct {
    const uint8_t* qs;
    const uint16_t* d;
    int64_t M, K, B, m0, m1;
    const int8_t* xq;
    const float* xd;
    float* y;
    double* y64;
} mm_job;

static void* mm_worker(void* arg) {
    const mm_job* j = (const mm_job*)arg;
    const int64_t nb = j->K / QK;
    for (int64_t b = 0; b < j->B; ++b)
        for (int64_t m = j->m0; m < j->m1; ++m)
            j->y[b * j->M + m] =
                out_element(j->qs + m * (j->K / 2), j->d + m * nb, j->K, j->xq + b * j->K,
                            j->xd + b * nb, j->y64 ? &j->y64[b * j->M + m] : NULL);
    return NULL;
}

void orc_mul_mat_mt(const uint8_t* qs, const uint16_t* d, int64_t M, int64_t K,
                    const int8_t* xq, const float* xd, int64_t B, float* y, double* y64,
                    int nthreads) {
    if (nthreads < 1) nthreads = 1;
    if (nthreads > M) nthreads = (int)(M > 0 ? M : 1);
    pthread_t* th = (pthread_t*)malloc((size_t)nthreads * sizeof(pthread_t));
    mm_job* jobs = (mm_job*)malloc((size_t)nthreads * sizeof(mm_job));
    for (int t = 0; t < nthreads; ++t) {
        mm_job j = {qs, d, M, K, B, M * t / nthreads, M * (t + 1) / nthreads, xq, xd, y, y64};
        jobs[t] = j;
        pthread_create(&th[t], NULL, mm_worker, &jobs[t]);
    }
    for (int t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
    free(th);
    free(jobs);
}

/* ------------------------------------------------------------------ */
/* Expert-routed product.  The scheduler section of the GGML backend    */
/* page says an expert matmul only touches the expert slices that are   */
/* used; here that is simply: each (token, slot) pair multiplies its    */
/* activation row by the one expert its id names.                       */
/* ------------------------------------------------------------------ */

void orc_mul_mat_id(const uint8_t* qs, const uint16_t* d, int64_t E, int64_t M, int64_t K,
                    const int8_t* xq, const float* xd, int64_t n_x_slots,
                    const int32_t* ids, int64_t T, int64_t top_k, float* y, int nthreads) {
    const int64_t nb = K / QK;
    for (int64_t t = 0; t < T; ++t)
        for (int64_t s = 0; s < top_k; ++s) {
            float* yrow = y + (t * top_k + s) * M;
            const int32_t e = ids[t * top_k + s];
            if (e < 0 || e >= E) {
                for (int64_t m = 0; m < M; ++m) yrow[m] = nanf("");
                continue;
            }
            const int64_t slot = (n_x_slots == 1) ? 0 : s;
            const int8_t* xrow = xq + (t * n_x_slots + slot) * K;
            const float* xdrow = xd + (t * n_x_slots + slot) * nb;
            orc_mul_mat_mt(qs + (int64_t)e * M * (K / 2), d + (int64_t)e * M * nb, M, K, xrow, xdrow, 1,
                           yrow, NULL, nthreads);
        }
}

void orc_moe_expert_sum(const float* y, const float* w, int64_t T, int64_t top_k, int64_t M, float* out) {
    for (int64_t t = 0; t < T; ++t)
        for (int64_t m = 0; m < M; ++m) {
            float acc = 0.0f;
            for (int64_t s = 0; s < top_k; ++s) {
                const float yv = y[(t * top_k + s) * M + m];
                const float v = w ? w[t * top_k + s] * yv : yv;
                acc = (s == 0) ? v : acc + v;
            }
            out[t * M + m] = acc;
        }
}

/* ------------------------------------------------------------------ */
/* SwiGLU -> Q8 (see the header for the fixed exponential).             */
/* ------------------------------------------------------------------ */

static float bits_to_f32(uint32_t u) {
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

float orc_exp_q(float t) {
    if (t != t) return t;
    if (t > 88.0f) return INFINITY;
    if (t < -17.0f) return 0.0f;
    const float l2e = bits_to_f32(0x3fb8aa3bu);
    const float ln2_hi = bits_to_f32(0x3f317200u);
    const float ln2_lo = bits_to_f32(0x35bfbe8eu);
    /* C_k = fp32 nearest 1 / k!, k = 7 .. 2 */
    const float c7 = bits_to_f32(0x39500d01u), c6 = bits_to_f32(0x3ab60b61u), c5 = bits_to_f32(0x3c088889u);
    const float c4 = bits_to_f32(0x3d2aaaabu), c3 = bits_to_f32(0x3e2aaaabu), c2 = 0.5f;
    const float nf = rintf(t * l2e);
    const float hi = nf * ln2_hi;
    const float lo = nf * ln2_lo;
    const float r = (t - hi) - lo;
    float c = c7;
    c = c * r + c6;
    c = c * r + c5;
    c = c * r + c4;
    c = c * r + c3;
    c = c * r + c2;
    c = c * r + 1.0f;
    const float p = c * r + 1.0f;
    const int n = (int)nf;
    const float scale = bits_to_f32((uint32_t)(n + 127) << 23);
    return p * scale;
}

float orc_silu(float g) {
    const float e = orc_exp_q(-g);
    return g / (1.0f + e);
}

void orc_silu_array(const float* in, int64_t n, float* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_silu(in[i]);
}

void orc_exp_q_array(const float* in, int64_t n, float* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_exp_q(in[i]);
}

void orc_q8_quantize_swiglu(const float* gate, const float* up, int64_t B, int64_t F, int64_t row_stride,
                            int8_t* xq, float* xd, int32_t* xs) {
    float* h = (float*)malloc((size_t)(B * F) * sizeof(float));
    for (int64_t b = 0; b < B; ++b)
        for (int64_t k = 0; k < F; ++k)
            h[b * F + k] = orc_silu(gate[b * row_stride + k]) * up[b * row_stride + k];
    orc_q8_quantize(h, B, F, xq, xd, xs);
    free(h);
}

/* ------------------------------------------------------------------ */
/* Q8_0 weights (see the header).                                      */
/* ------------------------------------------------------------------ */

void orc_q8w_quantize(const float* w, int64_t M, int64_t K, int8_t* qw, uint16_t* d) {
    const int64_t nb = K / QK;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t b = 0; b < nb; ++b) {
            const float* v = w + m * K + b * QK;
            float amax = 0.0f;
            for (int j = 0; j < QK; ++j) {
                const float a = fabsf(v[j]);
                if (a > amax) amax = a;
            }
            const float dd = amax / 127.0f;
            const float id = (dd != 0.0f) ? 1.0f / dd : 0.0f;
            for (int j = 0; j < QK; ++j) {
                long qi = lroundf(v[j] * id);
                if (qi > 127) qi = 127;
                if (qi < -127) qi = -127;
                qw[m * K + b * QK + j] = (int8_t)qi;
            }
            d[m * nb + b] = orc_f32_to_f16(dd);
        }
}

static int32_t block_dot_q8w(const int8_t* w32, const int8_t* x32) {
    int32_t sum = 0;
    for (int j = 0; j < QK; ++j) sum += (int32_t)w32[j] * (int32_t)x32[j];
    return sum;
}

void orc_block_dots_q8w(const int8_t* qw, int64_t M, int64_t K, const int8_t* xq, int64_t B, int32_t* I) {
    const int64_t nb = K / QK;
    for (int64_t b = 0; b < B; ++b)
        for (int64_t m = 0; m < M; ++m)
            for (int64_t kb = 0; kb < nb; ++kb)
                I[(b * M + m) * nb + kb] = block_dot_q8w(qw + m * K + kb * QK, xq + b * K + kb * QK);
}

static float out_element_q8w(const int8_t* w_row, const uint16_t* d_row, int64_t K, const int8_t* x_row,
                             const float* xd_row, double* y64) {
    const int64_t nb = K / QK;
    float acc = 0.0f;
    double acc64 = 0.0;
    for (int64_t kb = 0; kb < nb; ++kb) {
        const int32_t I = block_dot_q8w(w_row + kb * QK, x_row + kb * QK);
        const float dw = orc_f16_to_f32(d_row[kb]);
        const float c = dw * xd_row[kb];
        const float t = (float)I * c;
        acc = acc + t;
        acc64 += (double)I * (double)dw * (double)xd_row[kb];
    }
    if (y64) *y64 = acc64;
    return acc;
}

typedef struct {
    const int8_t* qw;
    const uint16_t* d;
    int64_t M, K, B, m0, m1;
    const int8_t* xq;
    const float* xd;
    float* y;
    double* y64;
} mm8_job;

static void* mm8_worker(void* arg) {
    const mm8_job* j = (const mm8_job*)arg;
    const int64_t nb = j->K / QK;
    for (int64_t b = 0; b < j->B; ++b)
        for (int64_t m = j->m0; m < j->m1; ++m)
            j->y[b * j->M + m] = out_element_q8w(j->qw + m * j->K, j->d + m * nb, j->K, j->xq + b * j->K,
                                                 j->xd + b * nb, j->y64 ? &j->y64[b * j->M + m] : NULL);
    return NULL;
}

void orc_mul_mat_q8w_mt(const int8_t* qw, const uint16_t* d, int64_t M, int64_t K, const int8_t* xq,
                        const float* xd, int64_t B, float* y, double* y64, int nthreads) {
    if (nthreads < 1) nthreads = 1;
    if (nthreads > M) nthreads = (int)(M > 0 ? M : 1);
    pthread_t* th = (pthread_t*)malloc((size_t)nthreads * sizeof(pthread_t));
    mm8_job* jobs = (mm8_job*)malloc((size_t)nthreads * sizeof(mm8_job));
    for (int t = 0; t < nthreads; ++t) {
        mm8_job j = {qw, d, M, K, B, M * t / nthreads, M * (t + 1) / nthreads, xq, xd, y, y64};
        jobs[t] = j;
        pthread_create(&th[t], NULL, mm8_worker, &jobs[t]);
    }
    for (int t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
    free(th);
    free(jobs);
}
