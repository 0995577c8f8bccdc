/*
 * nvq_oracle.h -- plain scalar C reference for the NVFP4 x Q8_0 (and Q4_1 / Q4_K /
 * IQ4_XS x Q8_0) quantized matrix product.
 *
 * TEST INFRASTRUCTURE ONLY.  This code exists to check the GPU library, never to
 * serve results.  Only the test suite, the package smoke check and the CPU-baseline
 * leg of the benchmark may load it.  It shares no code, header, table or constant
 * with the GPU library, and it includes nothing from it.
 *
 * Sources (web pages, cited by title and section):
 *   [HANDOFF]  "HANDOFF: flint CPU optimization (Q4_1 + NVFP4)", section 3 "Code map"
 *              and the "Bias trick" paragraph under it: NVFP4 weights in 64-weight
 *              blocks with one UE4M3 scale per 16 weights, Q8_0 activations, integer
 *              sums per 16-subblock, per-16 activation code sums (bsums).
 *   [GGUF]     the llama.cpp 2-bit GGUF tutorial (spke.com, article 4846), the GGML
 *              type table: Q8_0 packs 32 values in 34 bytes (32 int8 + one fp16 d).
 * Where the pages leave a step open the reading taken is stated at the function.
 *
 * Precision: decode of every format is exact in double; products and sums are done
 * in double and rounded once to float at the end.  No lookup tables exist here: every
 * decode is a closed form evaluated on the spot, so nothing can be left
 * uninitialised.
 *
 * Parity pins: each function below is checked by the CPU test suite against
 * something other than itself (library decoders, brute force, closed-form special
 * cases, the bias identity).  Nothing here is "parity unpinned".
 */
#ifndef NVQ_ORACLE_H
#define NVQ_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- element decodes ------------------------------------------------------ */

/* E2M1 4-bit float: bit 3 sign, bits 2..1 exponent (bias 1), bit 0 mantissa.
 * Exponent field 0 is subnormal (m * 0.5).  Code 8 (negative zero) decodes to 0. */
double nvqo_e2m1(int code);

/* UE4M3: unsigned 8-bit float, 4 exponent bits (bias 7), 3 mantissa bits,
 * subnormals at exponent field 0.  Bit 7 set or 0x7F are not valid scales and
 * decode to NaN. */
double nvqo_ue4m3(int byte);

/* IEEE binary16 -> double (exact, subnormals kept). */
double nvqo_f16_to_f64(uint16_t h);

/* float -> IEEE binary16, round to nearest even, subnormals kept, overflow -> inf. */
uint16_t nvqo_f32_to_f16(float x);

/* ---- Q8_0 activation quantization ----------------------------------------- */

/* x [M][K] fp32 -> q [M][K] int8, d16 [M][K/32] fp16 bits, bsum16 [M][K/16] int16
 * (bsum16 may be NULL).  K must be a multiple of 32. */
void nvqo_quantize_q8_0(const float* x, int64_t M, int64_t K,
                        int8_t* q, uint16_t* d16, int16_t* bsum16);

/* ---- NVFP4 weights -------------------------------------------------------- */

/* codes [N][K] one byte per weight (0..15), q [M][K].
 * isums [M][N][K/16] = sum over the 16 weights of a subblock of L(code) * q,
 * with L(c) = 2 * E2M1(c) an integer in -12..12.  K must be a multiple of 16. */
void nvqo_isums_nvfp4(const uint8_t* codes, const int8_t* q,
                      int64_t M, int64_t N, int64_t K, int32_t* isums);

/* y[m][j] = float( sum_k W[n_j][k] * A[m][k] ),  W = w_scale * UE4M3(scale) * E2M1(code),
 * A = fp16(d16) * q.  cols lists the output columns n_j (NULL: all N, then ncols = N);
 * y is [M][ncols].  abs_wa (nullable) receives sum_k |W*A| in double, same shape. */
void nvqo_matmul_nvfp4(const uint8_t* codes, const uint8_t* scales, float w_scale,
                       const int8_t* q, const uint16_t* d16,
                       int64_t M, int64_t N, int64_t K,
                       const int64_t* cols, int64_t ncols,
                       float* y, double* abs_wa);

/* Expert-routed product (the "mul_mat_id" step of a mixture-of-experts layer,
 * [HANDOFF] section 7 "Open items / next steps", item 1): E expert matrices, and for
 * every token m and routing slot a, the product of token m with expert ids[m][a].
 * codes [E][N][K], scales [E][N][K/16], w_scales [E], ids [M][A] (int32),
 * q [M][K], d16 [M][K/32].  y [M][A][ncols] and abs_wa (nullable) as for
 * nvqo_matmul_nvfp4 per (m, a).  An id outside [0, E) selects no weights: its y row
 * is NaN and its abs_wa row 0. */
void nvqo_matmul_nvfp4_routed(const uint8_t* codes, const uint8_t* scales, const float* w_scales,
                              const int32_t* ids, int64_t E, int64_t A,
                              const int8_t* q, const uint16_t* d16,
                              int64_t M, int64_t N, int64_t K,
                              const int64_t* cols, int64_t ncols,
                              float* y, double* abs_wa);

/* ---- Q4_1 weights ---------------------------------------------------------- */

/* qw [N][K] one byte per weight (0..15); dw, mw [N][K/32] fp16 bits; W = d*q + m.
 * isums [M][N][K/16] = sum over 16 of qw * q (unsigned weight codes). */
void nvqo_isums_q4_1(const uint8_t* qw, const int8_t* q,
                     int64_t M, int64_t N, int64_t K, int32_t* isums);

void nvqo_matmul_q4_1(const uint8_t* qw, const uint16_t* dw, const uint16_t* mw,
                      const int8_t* q, const uint16_t* d16,
                      int64_t M, int64_t N, int64_t K,
                      const int64_t* cols, int64_t ncols,
                      float* y, double* abs_wa);

/* ---- Q4_K weights ---------------------------------------------------------- */

/* qw [N][K] one byte per weight (0..15); sc, mn [N][K/32] 6-bit sub-block scales and
 * mins (0..63); d, dmin [N][K/256] fp16 bits; W = d*sc*q - dmin*mn.  K % 256 == 0.
 * Outputs and cols as nvqo_matmul_nvfp4.  Integer sums: nvqo_isums_q4_1. */
void nvqo_matmul_q4_k(const uint8_t* qw, const uint8_t* sc, const uint8_t* mn,
                      const uint16_t* d, const uint16_t* dmin,
                      const int8_t* q, const uint16_t* d16,
                      int64_t M, int64_t N, int64_t K,
                      const int64_t* cols, int64_t ncols,
                      float* y, double* abs_wa);

/* ---- Q5_K and Q6_K weights -------------------------------------------------- */

/* Q5_K: qw [N][K] one byte per weight (0..31); sc, mn [N][K/32] 6-bit sub-block scales
 * and mins (0..63); d, dmin [N][K/256] fp16 bits; W = d*sc*qw - dmin*mn.  K % 256 == 0.
 * Integer sums: nvqo_isums_q4_1 (sum qw * q). */
void nvqo_matmul_q5_k(const uint8_t* qw, const uint8_t* sc, const uint8_t* mn,
                      const uint16_t* d, const uint16_t* dmin,
                      const int8_t* q, const uint16_t* d16,
                      int64_t M, int64_t N, int64_t K,
                      const int64_t* cols, int64_t ncols,
                      float* y, double* abs_wa);

/* Q6_K: qw [N][K] one byte per weight (0..63); sc [N][K/16] int8 scales; d [N][K/256]
 * fp16 bits; W = d * sc * (qw - 32).  K % 256 == 0.  isums [M][N][K/16] = sum over 16
 * of (qw - 32) * q. */
void nvqo_isums_q6_k(const uint8_t* qw, const int8_t* q,
                     int64_t M, int64_t N, int64_t K, int32_t* isums);

void nvqo_matmul_q6_k(const uint8_t* qw, const int8_t* sc, const uint16_t* d,
                      const int8_t* q, const uint16_t* d16,
                      int64_t M, int64_t N, int64_t K,
                      const int64_t* cols, int64_t ncols,
                      float* y, double* abs_wa);

/* ---- IQ4_XS weights --------------------------------------------------------- */

/* qw [N][K] one byte per weight (0..15, an index into table); table [16] int8 values;
 * ls [N][K/32] 6-bit sub-block scales (0..63, used as ls - 32); d [N][K/256] fp16 bits;
 * W = d * (ls - 32) * table[qw].  K % 256 == 0.  isums [M][N][K/16] = sum over 16 of
 * table[qw] * q.  Outputs and cols as nvqo_matmul_nvfp4. */
void nvqo_isums_iq4_xs(const uint8_t* qw, const int8_t* table, const int8_t* q,
                       int64_t M, int64_t N, int64_t K, int32_t* isums);

void nvqo_matmul_iq4_xs(const uint8_t* qw, const uint8_t* ls, const uint16_t* d, const int8_t* table,
                        const int8_t* q, const uint16_t* d16,
                        int64_t M, int64_t N, int64_t K,
                        const int64_t* cols, int64_t ncols,
                        float* y, double* abs_wa);

#ifdef __cplusplus
}
#endif
#endif /* NVQ_ORACLE_H */
