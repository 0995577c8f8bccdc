/*
 * nvq.h -- C ABI of libnvq: NVFP4 x Q8_0 (and Q4_1 x Q8_0) quantized matrix
 * products on AMD Instinct MI355X (gfx950).
 *
 * What is computed.  Weights W [N][K] ("out x in", row-major) are stored 4-bit;
 * activations X [M][K] (M tokens) are quantized on the fly to Q8_0; the product is
 *     y[m][n] = sum_k W[n][k] * A[m][k],   y float32 [M][N] row-major,
 * where A = d * q is the Q8_0-dequantized activation.  Sources (web pages, cited
 * by title and section):
 *   "HANDOFF: flint CPU optimization (Q4_1 + NVFP4)", section 3 ("Code map" and the
 *     bias-trick paragraph): NVFP4 weights in 64-weight blocks, one UE4M3 scale
 *     per 16 weights, integer partial sums per 16-subblock, per-16 activation code
 *     sums; batch-1 decode uses a vector dot, larger batches a tiled matmul;
 *     section 1 names the Q4_1 kernels of the same work.
 *   The llama.cpp 2-bit GGUF tutorial (spke.com, article 4846), GGML type table:
 *     Q8_0 is 32 values in 34 bytes (32 int8 codes + one fp16 scale).
 *
 * Element formats (bit-exact definitions):
 *   E2M1 code c (4 bits): sign = bit 3, exponent e = bits 2..1 (bias 1), mantissa
 *     m = bit 0; e == 0 gives m/2, otherwise (1 + m/2) * 2^(e-1).  Code 8 is 0.
 *   UE4M3 byte b (bit 7 must be 0, 0x7F is not allowed): exponent E = b >> 3
 *     (bias 7), mantissa M = b & 7; E == 0 gives M * 2^-9, otherwise
 *     (1 + M/8) * 2^(E-7).  Range 2^-9 .. 448.
 *   NVFP4 weight: W[n][k] = S * UE4M3(scale[n][k/16]) * E2M1(code[n][k]),
 *     S = float32 per-tensor scale (argument w_scale).
 *   Q4_1 weight: W[n][k] = d[n][k/32] * q[n][k] + m[n][k/32], q in 0..15,
 *     d and m IEEE binary16.
 *   Q8_0 activation, per row and per 32 consecutive k:
 *     amax = max |x|; d32 = amax / 127 (IEEE float32 division);
 *     d = binary16(d32) rounded to nearest even (stored);
 *     q = clamp(rint(x / d32), -127, 127) with IEEE float32 division by the
 *         unrounded d32 and ties to even; amax == 0 gives d = 0, q = 0.
 *     A[m][k] = d[m][k/32] * q[m][k].  bsum16[m][j] = sum of the 16 codes
 *     q[m][16j .. 16j+15] (int16).
 *
 * Packed weight buffers (produced on the host by nvq_pack_*; one contiguous
 * buffer, which the caller copies to device memory):
 *   NVFP4, tile-interleaved.  Let Np = N rounded up to 16, Kp = K rounded up to 128,
 *     T = Np/16 row tiles, C = Kp/128 chunks.  nvq_nvfp4_weight_bytes(N, K) =
 *     Np*Kp/2 + Np*Kp/16 bytes:
 *     [0, T*C*1024)         codes: tile t, chunk c at (t*C + c)*1024: 64 slots of
 *                           16 bytes; slot l = 16*g + n holds row 16t + n,
 *                           k = 128c + 32g .. 128c + 32g + 31; byte i of a slot holds
 *                           the code of k0 + 2i in bits 0..3 and of k0 + 2i + 1 in
 *                           bits 4..7.
 *     [T*C*1024, +T*C*128)  UE4M3 scales: tile t, chunk c at (t*C + c)*128: slot l
 *                           (2 bytes) holds the scales of the two 16-subblocks of
 *                           slot l's 32 codes, in k order.
 *     Rows >= N and k >= K are zero padding.  One slot is the 16-byte FP4 operand a
 *     lane of a 16x16x128 matrix-core instruction takes, so every 64-lane load of
 *     a tile-chunk reads 1 KB of contiguous memory.
 *   Q4_1, row-major, nvq_q4_1_weight_bytes(N, K) = N*K/2 + N*K/8 bytes:
 *     [0, N*K/2)            codes: row n at n*K/2; byte i of a row holds the code of
 *                           k = 2i in bits 0..3 and of k = 2i+1 in bits 4..7.
 *     [N*K/2, +N*K/8)       per 32 weights a 4-byte pair: binary16 d in the low
 *                           half, binary16 m in the high half, row-major [N][K/32].
 *
 * Conventions for every entry point:
 *   - All array arguments of the compute entries are DEVICE pointers owned by the
 *     caller; the packers take HOST pointers.  The library allocates no device
 *     memory and keeps no pointer after it returns; its only state is a
 *     per-device "is this gfx950" flag written on first use.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Compute entries only enqueue work; results are valid once the stream is
 *     synchronised.
 *   - Device pointers w, q, x and y must be 16-byte aligned, d_f16 and bsum16
 *     2-byte aligned and isums 4-byte aligned (NVQ_ERR_ALIGN otherwise).
 *   - Return value: NVQ_OK (0) or a negative nvq_status.  On any error nothing is
 *     enqueued and no output is touched (except NVQ_ERR_HIP, which reports a
 *     launch failure after validation passed).  nvq_last_error() returns a
 *     thread-local message describing the last error of the calling thread.
 *   - Results are deterministic: identical inputs give bitwise identical outputs.
 *   - The compute entries run only on gfx950 devices (NVQ_ERR_DEVICE otherwise);
 *     there is no other code path.
 */
#ifndef NVQ_H
#define NVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int nvq_status;

#define NVQ_OK             0
#define NVQ_ERR_NULL      -1  /* a required pointer is NULL */
#define NVQ_ERR_SHAPE     -2  /* M, N or K out of range or K not a multiple of the block */
#define NVQ_ERR_RANGE     -3  /* invalid code / scale byte, or bad enum argument */
#define NVQ_ERR_ALIGN     -4  /* pointer alignment requirement not met */
#define NVQ_ERR_DEVICE    -5  /* current device is not gfx950 */
#define NVQ_ERR_HIP       -6  /* HIP runtime error (see nvq_last_error) */
#define NVQ_ERR_WORKSPACE -7  /* workspace missing or too small */

#define NVQ_FMT_NVFP4 0
#define NVQ_FMT_Q4_1  1
#define NVQ_PATH_GEMV      0  /* decode GEMV, matrix-core inner loop (production) */
#define NVQ_PATH_GEMM      1  /* tiled GEMM */
#define NVQ_PATH_GEMV_DOT4 2  /* decode GEMV, v_perm + v_dot4 inner loop (NVFP4 only) */

/* Largest M accepted by the GEMV entries; the GEMM entries accept M >= 16. */
#define NVQ_GEMV_MAX_M 15

/* ---- sizes (pure functions) ------------------------------------------------ */

/* Bytes of a packed NVFP4 weight buffer [N][K]: Np*Kp*9/16 with Np = N rounded up
 * to 16 and Kp = K rounded up to 128.  0 if N < 1 or K is not a positive multiple
 * of 64. */
size_t nvq_nvfp4_weight_bytes(int64_t N, int64_t K);

/* Bytes of a packed Q4_1 weight buffer [N][K]: N*K*5/8.  0 if N < 1 or K is not a
 * positive multiple of 32. */
size_t nvq_q4_1_weight_bytes(int64_t N, int64_t K);

/* Device workspace bytes nvq_gemm_nvfp4 / nvq_gemm_q4_1 need for this shape (fmt
 * is NVQ_FMT_*): with M > 16 and K % 64 == 0, the fp32 partial tiles of the K-split
 * work items that even out the last round of tiles over the chip's 256 compute units
 * (at most 32 MiB); otherwise 0.  Pure function.
 * When it is 0 the workspace pointer may be NULL. */
size_t nvq_gemm_workspace_bytes(int fmt, int64_t M, int64_t N, int64_t K);

/* ---- packers (host memory in, host memory out) ------------------------------ */

/* codes: [N][K] bytes, one E2M1 code (0..15) per byte; ue4m3: [N][K/16] bytes.
 * Writes nvq_nvfp4_weight_bytes(N, K) bytes to dst_host.  K % 64 == 0.
 * NVQ_ERR_RANGE if a code exceeds 15 or a scale byte has bit 7 set or equals 0x7F
 * (dst_host is then left unspecified). */
nvq_status nvq_pack_nvfp4(const uint8_t* codes, const uint8_t* ue4m3,
                          int64_t N, int64_t K, void* dst_host);

/* q: [N][K] bytes (0..15); d_f16, m_f16: [N][K/32] binary16 bit patterns.
 * Writes nvq_q4_1_weight_bytes(N, K) bytes to dst_host.  K % 32 == 0.
 * NVQ_ERR_RANGE if a code exceeds 15. */
nvq_status nvq_pack_q4_1(const uint8_t* q, const uint16_t* d_f16, const uint16_t* m_f16,
                         int64_t N, int64_t K, void* dst_host);

/* ---- activation quantization ------------------------------------------------ */

/* Q8_0 quantization of x [M][K] float32 into q [M][K] int8, d_f16 [M][K/32]
 * (binary16 bits) and, if bsum16 is not NULL, bsum16 [M][K/16] int16.  M >= 1,
 * K % 32 == 0.  Bit-exact with the definition above.  Non-finite x, or
 * amax > 65504 * 127, are outside the contract. */
nvq_status nvq_quantize_act_q8_0(const float* x, int64_t M, int64_t K,
                                 int8_t* q, uint16_t* d_f16, int16_t* bsum16, void* stream);

/* ---- NVFP4 products ----------------------------------------------------------- */

/* Decode GEMV (the single-token case of the product): 1 <= M <= NVQ_GEMV_MAX_M,
 * N >= 1, K % 64 == 0.  w: packed NVFP4 [N][K]; q, d_f16: Q8_0 activations [M][K];
 * y [M][N] float32 (overwritten).  M == 1 runs the decode kernel whose per-16
 * integer sums come from the matrix cores reading the FP4 codes directly (K up to
 * what its on-chip activation table holds, about 70000; longer rows run the tiled
 * kernel).  2 <= M runs the batched kernel (M * K < 2^32, NVQ_ERR_SHAPE otherwise),
 * all tokens in one launch streaming the weights once: exact binary16 operands (E2M1 * UE4M3 weights;
 * d * q split exactly into two binary16 terms) on the fp16 matrix cores, any K.
 * Per output the error against the exact product is at most 1e-5 * sum_k |W*A|
 * + 1e-6 (float32 accumulation of exact terms). */
nvq_status nvq_gemv_nvfp4(const void* w, float w_scale, const int8_t* q, const uint16_t* d_f16,
                          int64_t M, int64_t N, int64_t K, float* y, void* stream);

/* The same decode GEMV with the per-16 integer sums computed on the vector unit:
 * E2M1 -> int8 by v_perm_b32 table lookups and v_dot4_i32_i8 (one launch per
 * token).  Same arguments, results within the same bound.  K is limited to what
 * the on-chip activation table holds (NVQ_ERR_SHAPE beyond, about 70000). */
nvq_status nvq_gemv_nvfp4_dot4(const void* w, float w_scale, const int8_t* q,
                               const uint16_t* d_f16, int64_t M, int64_t N, int64_t K,
                               float* y, void* stream);

/* Expert-routed decode GEMV: the "mul_mat_id" step of a mixture-of-experts layer
 * ("HANDOFF: flint CPU optimization (Q4_1 + NVFP4)", section 7 "Open items / next
 * steps", item 1, which names the shape K = 2048, 256 experts, 6 active per token).
 * w: n_experts packed NVFP4 [N][K] matrices back to back, expert e at byte offset
 * e * nvq_nvfp4_weight_bytes(N, K) (device, 16-byte aligned); w_scales: float32
 * [n_experts] per-tensor scales (device); ids: int32 [M][n_active] expert indices
 * (device, e.g. written by a router kernel); q, d_f16: Q8_0 activations [M][K];
 * y: float32 [M][n_active][N] (overwritten): y[m][a] = the nvq_gemv_nvfp4 result of
 * token m against expert ids[m][a] (same kernel, same error bound).  An id outside
 * [0, n_experts) is not an error the host can see: its y row is set to NaN and no
 * weights are read for it.  1 <= n_active, M * n_active <= 65535, K % 64 == 0 and
 * K within the decode GEMV's LDS limit (NVQ_ERR_SHAPE otherwise).  Each (token,
 * slot) streams its expert's weights on its own; tokens that share an expert are
 * not merged. */
nvq_status nvq_gemv_nvfp4_routed(const void* w, const float* w_scales, const int32_t* ids,
                                 int64_t n_experts, int64_t n_active, const int8_t* q,
                                 const uint16_t* d_f16, int64_t M, int64_t N, int64_t K, float* y,
                                 void* stream);

/* Prefill GEMM (many tokens take the tiled form): M >= 16, N >= 1,
 * K % 64 == 0; arguments as for the GEMV plus a device workspace (16-byte aligned,
 * contents on entry irrelevant, overwritten) of at least
 * nvq_gemm_workspace_bytes(NVQ_FMT_NVFP4, M, N, K) bytes; NULL is accepted when
 * that size is 0.  Calls that share a workspace must not overlap in time.
 * For M > 16 the kernel folds each activation scale into an exact pair of binary16
 * values (hi + lo = d * q); this is exact for |d * q| < 65520, i.e. activations
 * below the binary16 range limit.  A row with larger activations yields
 * non-finite outputs in that row (never silently wrong values); M = 16 and the
 * GEMV entry points have no such limit. */
nvq_status nvq_gemm_nvfp4(const void* w, float w_scale, const int8_t* q, const uint16_t* d_f16,
                          int64_t M, int64_t N, int64_t K, float* y,
                          void* workspace, size_t ws_bytes, void* stream);

/* ---- Q4_1 products ------------------------------------------------------------ */

/* Q4_1 GEMV (1 <= M <= NVQ_GEMV_MAX_M) and GEMM (M >= 16); K % 32 == 0.
 * bsum16 [M][K/16] (from nvq_quantize_act_q8_0) is required: the offset m of each
 * 32-block multiplies the sum of that block's activation codes.  Same error bound
 * as the NVFP4 entries.  The GEMM takes a device workspace as nvq_gemm_nvfp4 does,
 * of nvq_gemm_workspace_bytes(NVQ_FMT_Q4_1, M, N, K) bytes (NULL when that is 0).
 * For M > 16 with K % 64 == 0 the GEMM forms each weight in two binary16 terms
 * (after a per-row power-of-two scaling, so any finite d, m are fine) and folds
 * each activation scale into an exact pair of binary16 values, which holds for
 * |d * q| < 65520; a token row with larger activations yields non-finite outputs in
 * that row, as for nvq_gemm_nvfp4.  The GEMV has no such limit. */
nvq_status nvq_gemv_q4_1(const void* w, const int8_t* q, const uint16_t* d_f16,
                         const int16_t* bsum16, int64_t M, int64_t N, int64_t K, float* y,
                         void* stream);
nvq_status nvq_gemm_q4_1(const void* w, const int8_t* q, const uint16_t* d_f16,
                         const int16_t* bsum16, int64_t M, int64_t N, int64_t K, float* y,
                         void* workspace, size_t ws_bytes, void* stream);

/* ---- debug: integer per-16 partial sums --------------------------------------- */

/* isums [M][N][K/16] int32 = for each 16-subblock, sum_j L(code) * q (NVFP4, with
 * L(c) = 2*E2M1(c), an integer in -12..12) or sum_j code * q (Q4_1, unsigned codes).
 * fmt: NVQ_FMT_*; path: NVQ_PATH_GEMV, NVQ_PATH_GEMM or (NVFP4 only)
 * NVQ_PATH_GEMV_DOT4 selects which production kernel's data path (weight load,
 * code expansion, integer / matrix-core contraction) produces the sums, run with
 * unit scales.  Any M >= 1 is accepted for every path; K % 64 == 0 (NVFP4) or
 * K % 32 == 0 (Q4_1). */
nvq_status nvq_debug_isums(int fmt, int path, const void* w, const int8_t* q,
                           int64_t M, int64_t N, int64_t K, int32_t* isums, void* stream);

/* ---- errors ------------------------------------------------------------------- */

const char* nvq_status_str(nvq_status s);
const char* nvq_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* NVQ_H */
