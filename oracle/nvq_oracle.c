/*
 * nvq_oracle.c -- plain scalar C reference (TEST INFRASTRUCTURE ONLY; see the header).
 *
 * Build: gcc -std=c99 -O2 -fno-tree-vectorize -ffp-contract=off -fPIC -shared
 * (no fast-math: float division and rintf must be IEEE, round to nearest even).
 */
#include "nvq_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------- */
/* Element decodes                                                            */
/* ------------------------------------------------------------------------- */

/* NVFP4 element: the 4-bit float E2M1 ([HANDOFF] section 3: "NVFP4" weights whose
 * integer LUT spans -12..12 around the +12 bias, i.e. twice E2M1). */
double nvqo_e2m1(int code)
{
    int s = (code >> 3) & 1;
    int e = (code >> 1) & 3;
    int m = code & 1;
    double v;
    if (e == 0)
        v = 0.5 * m;                          /* subnormal: m * 2^(1-1) * 2^-1 */
    else
        v = ldexp(1.0 + 0.5 * m, e - 1);      /* (1 + m/2) * 2^(e - bias), bias 1 */
    return s ? -v : v;
}

/* NVFP4 subblock scale: UE4M3, one per 16 weights ([HANDOFF] section 3, the
 * UE4M3 table and the per-16 scale sd16).  Reading: "unsigned E4M3", bias 7,
 * subnormals at exponent 0, 0x7F is NaN, a set bit 7 is not a valid scale. */
double nvqo_ue4m3(int byte)
{
    if (byte < 0 || byte > 255 || (byte & 0x80) || byte == 0x7F)
        return NAN;
    int e = byte >> 3;
    int m = byte & 7;
    if (e == 0)
        return ldexp((double)m, -9);          /* m/8 * 2^(1-7) */
    return ldexp(1.0 + m / 8.0, e - 7);
}

/* IEEE 754 binary16 (the Q8_0 block's d; [GGUF] type table). */
double nvqo_f16_to_f64(uint16_t h)
{
    int s = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int m = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(m + 1024), e - 25);
    return s ? -v : v;
}

uint16_t nvqo_f32_to_f16(float f)
{
    uint32_t x;
    memcpy(&x, &f, 4);
    uint32_t sign = (x >> 16) & 0x8000u;
    uint32_t exp = (x >> 23) & 0xFFu;
    uint32_t man = x & 0x7FFFFFu;

    if (exp == 0xFFu)                               /* inf / NaN */
        return (uint16_t)(sign | 0x7C00u | (man ? (0x200u | (man >> 13)) : 0u));

    int e = (int)exp - 127 + 15;                    /* binary16 biased exponent */
    if (e >= 31)
        return (uint16_t)(sign | 0x7C00u);          /* overflow */

    if (e <= 0) {                                   /* binary16 subnormal or zero */
        if (e < -10)
            return (uint16_t)sign;                  /* below half the smallest subnormal */
        man |= 0x800000u;
        int shift = 14 - e;                         /* value / 2^-24 = man >> shift */
        uint32_t res = man >> shift;
        uint32_t rem = man & ((1u << shift) - 1u);
        uint32_t half = 1u << (shift - 1);
        if (rem > half || (rem == half && (res & 1u)))
            res++;                                  /* may carry into the smallest normal */
        return (uint16_t)(sign | res);
    }

    uint32_t res = ((uint32_t)e << 10) | (man >> 13);
    uint32_t rem = man & 0x1FFFu;
    if (rem > 0x1000u || (rem == 0x1000u && (res & 1u)))
        res++;                                      /* carry may reach inf: correct */
    return (uint16_t)(sign | res);
}

/* ------------------------------------------------------------------------- */
/* Q8_0 activation quantization                                               */
/* ------------------------------------------------------------------------- */

/* Q8_0 ([GGUF] type table: 32 values, 34 bytes = 32 int8 + fp16 d; [HANDOFF]
 * section 3, block_q8_0 activations and their per-16 code sums "bsums").
 * Readings: d32 = amax / 127 in fp32; the stored scale is fp16(d32) rounded to
 * nearest even; the codes are rint(x / d32) (IEEE fp32 division by the unrounded
 * d32, ties to even) clamped to +-127; an all-zero block stores d = 0 and q = 0,
 * and so does a block of float32 subnormals so small that d32 rounds to 0 (x / 0
 * names no integer code; the block's dequantized values d * q are 0 either way). */
void nvqo_quantize_q8_0(const float* x, int64_t M, int64_t K,
                        int8_t* q, uint16_t* d16, int16_t* bsum16)
{
    int64_t nb = K / 32;
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t b = 0; b < nb; ++b) {
            const float* xb = x + m * K + b * 32;
            int8_t* qb = q + m * K + b * 32;
            float amax = 0.0f;
            for (int j = 0; j < 32; ++j) {
                float a = fabsf(xb[j]);
                if (a > amax)
                    amax = a;
            }
            float d = amax / 127.0f;
            d16[m * nb + b] = nvqo_f32_to_f16(d);
            for (int j = 0; j < 32; ++j) {
                int v = 0;
                if (d != 0.0f) {
                    float t = xb[j] / d;
                    float r = rintf(t);
                    if (r > 127.0f) r = 127.0f;
                    if (r < -127.0f) r = -127.0f;
                    v = (int)r;
                }
                qb[j] = (int8_t)v;
            }
            if (bsum16) {
                for (int h = 0; h < 2; ++h) {
                    int s = 0;
                    for (int j = 0; j < 16; ++j)
                        s += qb[16 * h + j];
                    bsum16[m * (K / 16) + 2 * b + h] = (int16_t)s;
                }
            }
        }
    }
}

/* ------------------------------------------------------------------------- */
/* NVFP4 x Q8_0                                                               */
/* ------------------------------------------------------------------------- */

/* Integer per-16 sums ([HANDOFF] section 3: the vec_dot keeps one int32 sum per
 * 16-subblock before any scale is applied).  L(c) = 2*E2M1(c) is an integer. */
void nvqo_isums_nvfp4(const uint8_t* codes, const int8_t* q,
                      int64_t M, int64_t N, int64_t K, int32_t* isums)
{
    int64_t ns = K / 16;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            for (int64_t s = 0; s < ns; ++s) {
                int32_t acc = 0;
                for (int j = 0; j < 16; ++j) {
                    int64_t k = 16 * s + j;
                    int l = (int)(2.0 * nvqo_e2m1(codes[n * K + k]));
                    acc += l * (int32_t)q[m * K + k];
                }
                isums[(m * N + n) * ns + s] = acc;
            }
}

/* Dequantize one NVFP4 weight row to double: W[k] = S_t * UE4M3(scale[k/16]) * E2M1(code[k]). */
static void dequant_nvfp4_row(const uint8_t* codes, const uint8_t* scales, float w_scale,
                              int64_t K, double* w)
{
    for (int64_t k = 0; k < K; ++k)
        w[k] = (double)w_scale * nvqo_ue4m3(scales[k / 16]) * nvqo_e2m1(codes[k]);
}

/* Dequantize one Q8_0 activation row to double: A[k] = fp16(d16[k/32]) * q[k]. */
static void dequant_q8_0_row(const int8_t* q, const uint16_t* d16, int64_t K, double* a)
{
    for (int64_t k = 0; k < K; ++k)
        a[k] = nvqo_f16_to_f64(d16[k / 32]) * (double)q[k];
}

/* The product the path computes, as its plain definition: dequantize both
 * operands exactly, take the dot product in double, round once to float. */
static void dot_rows(const double* w, const double* a, int64_t K, float* y, double* abs_wa)
{
    double acc = 0.0, aacc = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        double p = w[k] * a[k];
        acc += p;
        aacc += fabs(p);
    }
    *y = (float)acc;
    if (abs_wa)
        *abs_wa = aacc;
}

void nvqo_matmul_nvfp4(const uint8_t* codes, const uint8_t* scales, float w_scale,
                       const int8_t* q, const uint16_t* d16,
                       int64_t M, int64_t N, int64_t K,
                       const int64_t* cols, int64_t ncols,
                       float* y, double* abs_wa)
{
    if (!cols)
        ncols = N;
    double* w = (double*)malloc(sizeof(double) * (size_t)K);
    double* a = (double*)malloc(sizeof(double) * (size_t)(M * K));
    if (!w || !a) {
        free(w);
        free(a);
        return;
    }
    for (int64_t m = 0; m < M; ++m)
        dequant_q8_0_row(q + m * K, d16 + m * (K / 32), K, a + m * K);
    for (int64_t j = 0; j < ncols; ++j) {
        int64_t n = cols ? cols[j] : j;
        dequant_nvfp4_row(codes + n * K, scales + n * (K / 16), w_scale, K, w);
        for (int64_t m = 0; m < M; ++m)
            dot_rows(w, a + m * K, K, &y[m * ncols + j],
                     abs_wa ? &abs_wa[m * ncols + j] : NULL);
    }
    free(w);
    free(a);
}

/* Expert-routed product ([HANDOFF] section 7 "Open items / next steps", item 1):
 * the plain product above, once per (token, routing slot), with the expert the slot
 * names.  Reading taken: the page gives only the shape of the routed step (K = 2048,
 * 256 experts, 6 active per token); each expert is a
 * complete NVFP4 matrix with its own per-tensor scale, and an expert index outside
 * the table selects nothing (NaN marks the row). */
void nvqo_matmul_nvfp4_routed(const uint8_t* codes, const uint8_t* scales, const float* w_scales,
                              const int32_t* ids, int64_t E, int64_t A,
                              const int8_t* q, const uint16_t* d16,
                              int64_t M, int64_t N, int64_t K,
                              const int64_t* cols, int64_t ncols,
                              float* y, double* abs_wa)
{
    if (!cols)
        ncols = N;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t a = 0; a < A; ++a) {
            int64_t job = m * A + a;
            int32_t e = ids[job];
            float* yj = y + job * ncols;
            double* aj = abs_wa ? abs_wa + job * ncols : NULL;
            if (e < 0 || e >= E) {
                for (int64_t j = 0; j < ncols; ++j) {
                    yj[j] = NAN;
                    if (aj)
                        aj[j] = 0.0;
                }
                continue;
            }
            nvqo_matmul_nvfp4(codes + e * N * K, scales + e * N * (K / 16), w_scales[e],
                              q + m * K, d16 + m * (K / 32), 1, N, K, cols, ncols, yj, aj);
        }
}

/* ------------------------------------------------------------------------- */
/* Q4_1 x Q8_0                                                                */
/* ------------------------------------------------------------------------- */

/* Q4_1 ([HANDOFF] section 1: the patch's Q4_1 kernels): per 32 weights an fp16
 * scale d and fp16 offset m, 4-bit codes q in 0..15, weight = d*q + m. */
void nvqo_isums_q4_1(const uint8_t* qw, const int8_t* q,
                     int64_t M, int64_t N, int64_t K, int32_t* isums)
{
    int64_t ns = K / 16;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            for (int64_t s = 0; s < ns; ++s) {
                int32_t acc = 0;
                for (int j = 0; j < 16; ++j) {
                    int64_t k = 16 * s + j;
                    acc += (int32_t)qw[n * K + k] * (int32_t)q[m * K + k];
                }
                isums[(m * N + n) * ns + s] = acc;
            }
}

static void dequant_q4_1_row(const uint8_t* qw, const uint16_t* dw, const uint16_t* mw,
                             int64_t K, double* w)
{
    for (int64_t k = 0; k < K; ++k)
        w[k] = nvqo_f16_to_f64(dw[k / 32]) * (double)qw[k] + nvqo_f16_to_f64(mw[k / 32]);
}

void nvqo_matmul_q4_1(const uint8_t* qw, const uint16_t* dw, const uint16_t* mw,
                      const int8_t* q, const uint16_t* d16,
                      int64_t M, int64_t N, int64_t K,
                      const int64_t* cols, int64_t ncols,
                      float* y, double* abs_wa)
{
    if (!cols)
        ncols = N;
    double* w = (double*)malloc(sizeof(double) * (size_t)K);
    double* a = (double*)malloc(sizeof(double) * (size_t)(M * K));
    if (!w || !a) {
        free(w);
        free(a);
        return;
    }
    for (int64_t m = 0; m < M; ++m)
        dequant_q8_0_row(q + m * K, d16 + m * (K / 32), K, a + m * K);
    for (int64_t j = 0; j < ncols; ++j) {
        int64_t n = cols ? cols[j] : j;
        dequant_q4_1_row(qw + n * K, dw + n * (K / 32), mw + n * (K / 32), K, w);
        for (int64_t m = 0; m < M; ++m)
            dot_rows(w, a + m * K, K, &y[m * ncols + j],
                     abs_wa ? &abs_wa[m * ncols + j] : NULL);
    }
    free(w);
    free(a);
}

/* ------------------------------------------------------------------------- */
/* Q4_K x Q8_0                                                                */
/* ------------------------------------------------------------------------- */

/* Q4_K ([HANDOFF] section 1 names Q4_K among the patch's formats; the llama.cpp
 * 2-bit GGUF tutorial's GGML type table gives its block: 256 values in 144 bytes).
 * Reading (the pages give the block size only): a super-block of 256 weights holds a
 * binary16 scale d and a binary16 min scale dmin, and each of its eight 32-weight
 * sub-blocks j a 6-bit scale sc_j and a 6-bit min mn_j; with 4-bit codes q,
 *     weight = d * sc_j * q - dmin * mn_j,
 * 2 + 2 + 16 * 6 / 8 + 256 / 2 = 144 bytes.  The per-16 integer sums are those of
 * Q4_1 (unsigned codes times activation codes), nvqo_isums_q4_1. */
static void dequant_q4_k_row(const uint8_t* qw, const uint8_t* sc, const uint8_t* mn,
                             const uint16_t* d, const uint16_t* dmin, int64_t K, double* w)
{
    for (int64_t k = 0; k < K; ++k) {
        int64_t s = k / 256, j = k / 32;
        w[k] = nvqo_f16_to_f64(d[s]) * (double)sc[j] * (double)qw[k]
             - nvqo_f16_to_f64(dmin[s]) * (double)mn[j];
    }
}

void nvqo_matmul_q4_k(const uint8_t* qw, const uint8_t* sc, const uint8_t* mn,
                      const uint16_t* d, const uint16_t* dmin,
                      const int8_t* q, const uint16_t* d16,
                      int64_t M, int64_t N, int64_t K,
                      const int64_t* cols, int64_t ncols,
                      float* y, double* abs_wa)
{
    if (!cols)
        ncols = N;
    double* w = (double*)malloc(sizeof(double) * (size_t)K);
    double* a = (double*)malloc(sizeof(double) * (size_t)(M * K));
    if (!w || !a) {
        free(w);
        free(a);
        return;
    }
    for (int64_t m = 0; m < M; ++m)
        dequant_q8_0_row(q + m * K, d16 + m * (K / 32), K, a + m * K);
    for (int64_t jc = 0; jc < ncols; ++jc) {
        int64_t n = cols ? cols[jc] : jc;
        dequant_q4_k_row(qw + n * K, sc + n * (K / 32), mn + n * (K / 32), d + n * (K / 256),
                         dmin + n * (K / 256), K, w);
        for (int64_t m = 0; m < M; ++m)
            dot_rows(w, a + m * K, K, &y[m * ncols + jc],
                     abs_wa ? &abs_wa[m * ncols + jc] : NULL);
    }
    free(w);
    free(a);
}

/* ------------------------------------------------------------------------- */
/* Q5_K and Q6_K x Q8_0                                                       */
/* ------------------------------------------------------------------------- */

/* Q5_K ([HANDOFF] section 1 names "Q4_K/Q5_K/Q6_K" among the patch's formats; the
 * pages give neither its block nor its rule).  Reading (the GGML format's, known from
 * outside the pages): Q4_K's super-block of 256 weights with binary16 d and dmin and
 * per 32-weight sub-block j a 6-bit scale sc_j and min mn_j, but 5-bit codes c:
 *     weight = d * sc_j * c - dmin * mn_j,   c in 0..31,
 * 2 + 2 + 12 + 32 (the codes' fifth bits) + 128 = 176 bytes.  The per-16 integer sums
 * are sum c * q, nvqo_isums_q4_1 applied to the 5-bit codes. */
static void dequant_q5_k_row(const uint8_t* qw, const uint8_t* sc, const uint8_t* mn,
                             const uint16_t* d, const uint16_t* dmin, int64_t K, double* w)
{
    for (int64_t k = 0; k < K; ++k) {
        double scale = nvqo_f16_to_f64(d[k / 256]) * (double)sc[k / 32];
        double offset = nvqo_f16_to_f64(dmin[k / 256]) * (double)mn[k / 32];
        w[k] = scale * (double)qw[k] - offset;
    }
}

void nvqo_matmul_q5_k(const uint8_t* qw, const uint8_t* sc, const uint8_t* mn,
                      const uint16_t* d, const uint16_t* dmin,
                      const int8_t* q, const uint16_t* d16,
                      int64_t M, int64_t N, int64_t K,
                      const int64_t* cols, int64_t ncols,
                      float* y, double* abs_wa)
{
    if (!cols)
        ncols = N;
    double* w = (double*)malloc(sizeof(double) * (size_t)K);
    double* a = (double*)malloc(sizeof(double) * (size_t)(M * K));
    if (!w || !a) {
        free(w);
        free(a);
        return;
    }
    for (int64_t m = 0; m < M; ++m)
        dequant_q8_0_row(q + m * K, d16 + m * (K / 32), K, a + m * K);
    for (int64_t jc = 0; jc < ncols; ++jc) {
        int64_t n = cols ? cols[jc] : jc;
        dequant_q5_k_row(qw + n * K, sc + n * (K / 32), mn + n * (K / 32), d + n * (K / 256),
                         dmin + n * (K / 256), K, w);
        for (int64_t m = 0; m < M; ++m)
            dot_rows(w, a + m * K, K, &y[m * ncols + jc],
                     abs_wa ? &abs_wa[m * ncols + jc] : NULL);
    }
    free(w);
    free(a);
}

/* Q6_K (named beside Q5_K; no block or rule in the pages).  Reading (the GGML
 * format's): a super-block of 256 weights holds a binary16 scale d and one signed
 * 8-bit scale sc_s per 16 weights; 6-bit codes c are stored with an offset of 32:
 *     weight = d * sc_s * (c - 32),   c in 0..63,   s = k / 16,
 * 128 (low four bits) + 64 (high two bits) + 16 + 2 = 210 bytes.  The per-16 integer
 * sums are sum (c - 32) * q. */
void nvqo_isums_q6_k(const uint8_t* qw, const int8_t* q,
                     int64_t M, int64_t N, int64_t K, int32_t* isums)
{
    int64_t ns = K / 16;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            for (int64_t s = 0; s < ns; ++s) {
                int32_t acc = 0;
                for (int j = 0; j < 16; ++j) {
                    int64_t k = 16 * s + j;
                    acc += ((int32_t)qw[n * K + k] - 32) * (int32_t)q[m * K + k];
                }
                isums[(m * N + n) * ns + s] = acc;
            }
}

static void dequant_q6_k_row(const uint8_t* qw, const int8_t* sc, const uint16_t* d, int64_t K, double* w)
{
    for (int64_t k = 0; k < K; ++k)
        w[k] = nvqo_f16_to_f64(d[k / 256]) * (double)sc[k / 16] * (double)((int)qw[k] - 32);
}

void nvqo_matmul_q6_k(const uint8_t* qw, const int8_t* sc, const uint16_t* d,
                      const int8_t* q, const uint16_t* d16,
                      int64_t M, int64_t N, int64_t K,
                      const int64_t* cols, int64_t ncols,
                      float* y, double* abs_wa)
{
    if (!cols)
        ncols = N;
    double* w = (double*)malloc(sizeof(double) * (size_t)K);
    double* a = (double*)malloc(sizeof(double) * (size_t)(M * K));
    if (!w || !a) {
        free(w);
        free(a);
        return;
    }
    for (int64_t m = 0; m < M; ++m)
        dequant_q8_0_row(q + m * K, d16 + m * (K / 32), K, a + m * K);
    for (int64_t jc = 0; jc < ncols; ++jc) {
        int64_t n = cols ? cols[jc] : jc;
        dequant_q6_k_row(qw + n * K, sc + n * (K / 16), d + n * (K / 256), K, w);
        for (int64_t m = 0; m < M; ++m)
            dot_rows(w, a + m * K, K, &y[m * ncols + jc],
                     abs_wa ? &abs_wa[m * ncols + jc] : NULL);
    }
    free(w);
    free(a);
}

/* ------------------------------------------------------------------------- */
/* IQ4_XS x Q8_0                                                              */
/* ------------------------------------------------------------------------- */

/* IQ4_XS ([HANDOFF] section 1 names IQ4_XS among the patch's formats; the GGUF
 * tutorial's type table gives its block: 256 values in 136 bytes).  Reading: a
 * 256-weight super-block holds a binary16 scale d, each of its eight 32-weight
 * sub-blocks a 6-bit scale ls_j taken as ls_j - 32, and 4-bit codes c that index a
 * 16-entry int8 value table V (non-linear; the pages do not print it, so it is an
 * input here):  weight = d * (ls_j - 32) * V[c];  2 + 6 + 128 = 136 bytes.  The per-16
 * integer sums are sum V[c] * q. */
void nvqo_isums_iq4_xs(const uint8_t* qw, const int8_t* table, const int8_t* q,
                       int64_t M, int64_t N, int64_t K, int32_t* isums)
{
    int64_t ns = K / 16;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            for (int64_t s = 0; s < ns; ++s) {
                int32_t acc = 0;
                for (int j = 0; j < 16; ++j) {
                    int64_t k = 16 * s + j;
                    acc += (int32_t)table[qw[n * K + k]] * (int32_t)q[m * K + k];
                }
                isums[(m * N + n) * ns + s] = acc;
            }
}

static void dequant_iq4_xs_row(const uint8_t* qw, const uint8_t* ls, const uint16_t* d,
                               const int8_t* table, int64_t K, double* w)
{
    for (int64_t k = 0; k < K; ++k)
        w[k] = nvqo_f16_to_f64(d[k / 256]) * (double)((int)ls[k / 32] - 32) * (double)table[qw[k]];
}

void nvqo_matmul_iq4_xs(const uint8_t* qw, const uint8_t* ls, const uint16_t* d, const int8_t* table,
                        const int8_t* q, const uint16_t* d16,
                        int64_t M, int64_t N, int64_t K,
                        const int64_t* cols, int64_t ncols,
                        float* y, double* abs_wa)
{
    if (!cols)
        ncols = N;
    double* w = (double*)malloc(sizeof(double) * (size_t)K);
    double* a = (double*)malloc(sizeof(double) * (size_t)(M * K));
    if (!w || !a) {
        free(w);
        free(a);
        return;
    }
    for (int64_t m = 0; m < M; ++m)
        dequant_q8_0_row(q + m * K, d16 + m * (K / 32), K, a + m * K);
    for (int64_t jc = 0; jc < ncols; ++jc) {
        int64_t n = cols ? cols[jc] : jc;
        dequant_iq4_xs_row(qw + n * K, ls + n * (K / 32), d + n * (K / 256), table, K, w);
        for (int64_t m = 0; m < M; ++m)
            dot_rows(w, a + m * K, K, &y[m * ncols + jc],
                     abs_wa ? &abs_wa[m * ncols + jc] : NULL);
    }
    free(w);
    free(a);
}
