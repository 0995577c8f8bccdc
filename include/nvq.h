/*
 * nvq.h -- C ABI of libnvq: NVFP4 x Q8_0 (and Q4_1 / Q4_K / Q5_K / Q6_K / IQ4_XS x Q8_0) quantized
 * matrix products on AMD Instinct MI355X (gfx950).
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
 *     section 1 names the Q4_1 kernels of the same work and IQ4_XS and Q4_K / Q5_K /
 *     Q6_K among its formats.
 *   The llama.cpp 2-bit GGUF tutorial (spke.com, article 4846), GGML type table:
 *     Q8_0 is 32 values in 34 bytes (32 int8 codes + one fp16 scale); Q4_K is 256
 *     values in 144 bytes, IQ4_XS 256 values in 136 bytes.
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
 *   Q4_K weight (the pages give only its block size; this is the reading taken):
 *     W[n][k] = d[n][k/256] * sc[n][k/32] * q[n][k] - dmin[n][k/256] * mn[n][k/32],
 *     q in 0..15, sc and mn 6-bit (0..63), d and dmin IEEE binary16; 2 + 2 + 12 + 128
 *     = 144 bytes per 256 weights.
 *   Q5_K weight (the pages give neither its block nor its rule; the rule taken is the
 *     GGML format's): as Q4_K with 5-bit codes q in 0..31; 2 + 2 + 12 + 32 + 128 = 176
 *     bytes per 256 weights.
 *   Q6_K weight (likewise the GGML format's rule): W[n][k] = d[n][k/256] *
 *     sc[n][k/16] * (q[n][k] - 32), q in 0..63, sc signed 8-bit, d IEEE binary16;
 *     128 + 64 + 16 + 2 = 210 bytes per 256 weights.
 *   IQ4_XS weight (the pages give only its block size; the rule taken is the GGML
 *     format's, with its 16-entry value table as an argument, since the pages print
 *     none): W[n][k] = d[n][k/256] * (ls[n][k/32] - 32) * table[c[n][k]], c in 0..15,
 *     ls 6-bit (0..63), table 16 int8 values, d IEEE binary16; 2 + 6 + 128 = 136 bytes
 *     per 256 weights.
 *   Q8_0 activation, per row and per 32 consecutive k:
 *     amax = max |x|; d32 = amax / 127 (IEEE float32 division);
 *     d = binary16(d32) rounded to nearest even (stored);
 *     q = clamp(rint(x / d32), -127, 127) with IEEE float32 division by the
 *         unrounded d32 and ties to even; a block whose d32 is 0 (amax == 0,
 *         or float32 subnormals below 127 * 2^-150) gives d = 0, q = 0.
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
 *   Q4_K, row-major, nvq_q4_k_weight_bytes(N, K) = N*K*144/256 bytes:
 *     [0, N*K/2)            codes, as Q4_1.
 *     [N*K/2, +N*K/16)      per 256 weights a 16-byte header, row-major [N][K/256]:
 *                           bytes 0-1 binary16 d, bytes 2-3 binary16 dmin, bytes
 *                           4-15 the 16 6-bit fields sc_0..sc_7, mn_0..mn_7 of its
 *                           eight 32-weight sub-blocks, field f at bits
 *                           [6f, 6f + 6) of those 12 bytes read as one
 *                           little-endian 96-bit number.
 *   Q5_K, row-major, nvq_q5_k_weight_bytes(N, K) = N*K*176/256 bytes:
 *     [0, N*K/2)            the codes' low four bits, as Q4_1.
 *     [N*K/2, +N*K/16)      the 16-byte headers, as Q4_K.
 *     [N*K/2 + N*K/16, +N*K/8)  per 32 weights a 4-byte little-endian word of the
 *                           codes' fifth bits, row-major [N][K/32]: bit e (0..15) of
 *                           the code of k = 2e, bit 16 + e of the code of k = 2e + 1
 *                           (k counted within the 32-block).
 *   Q6_K, row-major, nvq_q6_k_weight_bytes(N, K) = N*K*210/256 bytes:
 *     [0, N*K/2)            the codes' low four bits, as Q4_1.
 *     [N*K/2, +N*K/16)      the int8 scales, row-major [N][K/16].
 *     [N*K/2 + N*K/16, +N*K/4)  per 32 weights two 4-byte words, row-major [N][K/32]:
 *                           the codes' fifth bits, then their sixth bits, each
 *                           arranged as Q5_K's fifth-bit word.
 *     [N*K/2 + N*K/16 + N*K/4, +N*K/128)  binary16 d, row-major [N][K/256].
 *   IQ4_XS, row-major, nvq_iq4_xs_weight_bytes(N, K) = N*K*136/256 bytes:
 *     [0, N*K/2)            codes, as Q4_1.
 *     [N*K/2, +N*K/32)      per 256 weights an 8-byte header, row-major [N][K/256]:
 *                           bytes 0-1 binary16 d, bytes 2-7 the eight 6-bit fields
 *                           ls_0..ls_7, field j at bits [6j, 6j + 6) of those 6 bytes
 *                           read as one little-endian 48-bit number.
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
#define NVQ_FMT_Q4_K  2
#define NVQ_FMT_IQ4_XS 3
#define NVQ_FMT_Q5_K  4
#define NVQ_FMT_Q6_K  5
#define NVQ_PATH_GEMV      0  /* decode GEMV, matrix-core inner loop (production) */
#define NVQ_PATH_GEMM      1  /* tiled GEMM */
#define NVQ_PATH_GEMV_DOT4 2  /* decode GEMV, v_perm + v_dot4 inner loop (NVFP4 only) */

/* Largest M accepted by the GEMV entries; the GEMM entries accept M >= 16. */
#define NVQ_GEMV_MAX_M 15

/* ---- sizes (pure functions) ------------------------------------------------ */

/* Bytes of a packed NVFP4 weight buffer [N][K]: Np*Kp*9/16 with Np = N rounded up
 * to 16 and Kp = K rounded up to 128.  0 if N < 1 or K is not a positive multiple
 * of 64.  Follows: "HANDOFF: flint CPU optimization (Q4_1 + NVFP4)", section 3
 * (NVFP4 blocks of 64 weights: 4-bit codes plus one UE4M3 byte per 16, i.e. 4.5 bits
 * per weight); the tile-interleaved order is this library's own. */
size_t nvq_nvfp4_weight_bytes(int64_t N, int64_t K);

/* Bytes of a packed Q4_1 weight buffer [N][K]: N*K*5/8.  0 if N < 1 or K is not a
 * positive multiple of 32.  Follows: the llama.cpp 2-bit GGUF tutorial, GGML type
 * table (Q4_1: 32 weights per block, 4-bit codes plus a binary16 scale and offset). */
size_t nvq_q4_1_weight_bytes(int64_t N, int64_t K);

/* Bytes of a packed Q4_K weight buffer [N][K]: N*K*144/256.  0 if N < 1 or K is not a
 * positive multiple of 256.  Follows: the llama.cpp 2-bit GGUF tutorial, GGML type
 * table (Q4_K: 256 values in 144 bytes). */
size_t nvq_q4_k_weight_bytes(int64_t N, int64_t K);

/* Bytes of a packed Q5_K / Q6_K weight buffer [N][K]: N*K*176/256 / N*K*210/256.  0 if
 * N < 1 or K is not a positive multiple of 256.  Follows: "HANDOFF: flint CPU
 * optimization (Q4_1 + NVFP4)", section 1 (Q5_K and Q6_K among the patch's formats; the
 * pages give no block size for them, these are the GGML formats' 176 and 210 bytes). */
size_t nvq_q5_k_weight_bytes(int64_t N, int64_t K);
size_t nvq_q6_k_weight_bytes(int64_t N, int64_t K);

/* Bytes of a packed IQ4_XS weight buffer [N][K]: N*K*136/256.  0 if N < 1 or K is not
 * a positive multiple of 256.  Follows: the llama.cpp 2-bit GGUF tutorial, GGML type
 * table (IQ4_XS: 256 values in 136 bytes). */
size_t nvq_iq4_xs_weight_bytes(int64_t N, int64_t K);

/* Device workspace bytes nvq_gemm_nvfp4 / nvq_gemm_q4_1 / nvq_gemm_q4_k / nvq_gemm_q5_k /
 * nvq_gemm_q6_k / nvq_gemm_iq4_xs need for this shape (fmt is NVQ_FMT_*): with M > 16
 * and K % 64 == 0 (Q4_K, Q5_K, Q6_K, IQ4_XS: K % 256 == 0, and also M <= 16 with
 * K > 20480), the fp32 partial
 * tiles of the K-split
 * work items that even out the last round of tiles over the chip's 256 compute units
 * (at most 64 MiB: 256 work items x 512 threads x 128 floats); otherwise 0.  Pure
 * function.  When it is 0 the workspace pointer may be NULL.  (A scheduling detail
 * of this library; the pages have no counterpart.) */
size_t nvq_gemm_workspace_bytes(int fmt, int64_t M, int64_t N, int64_t K);

/* ---- packers (host memory in, host memory out) ------------------------------ */

/* codes: [N][K] bytes, one E2M1 code (0..15) per byte; ue4m3: [N][K/16] bytes.
 * Writes nvq_nvfp4_weight_bytes(N, K) bytes to dst_host.  K % 64 == 0.
 * NVQ_ERR_RANGE if a code exceeds 15 or a scale byte has bit 7 set or equals 0x7F
 * (dst_host is then left unspecified).  Host memory only, caller-owned.
 * Follows: "HANDOFF: flint CPU optimization (Q4_1 + NVFP4)", section 3 (E2M1 codes,
 * one UE4M3 scale per 16 weights). */
nvq_status nvq_pack_nvfp4(const uint8_t* codes, const uint8_t* ue4m3,
                          int64_t N, int64_t K, void* dst_host);

/* q: [N][K] bytes (0..15); d_f16, m_f16: [N][K/32] binary16 bit patterns.
 * Writes nvq_q4_1_weight_bytes(N, K) bytes to dst_host.  K % 32 == 0.
 * NVQ_ERR_RANGE if a code exceeds 15.  Host memory only, caller-owned.
 * Follows: the llama.cpp 2-bit GGUF tutorial, GGML type table (Q4_1), and "HANDOFF:
 * flint CPU optimization (Q4_1 + NVFP4)", section 1 (Q4_1 weights in the same work). */
nvq_status nvq_pack_q4_1(const uint8_t* q, const uint16_t* d_f16, const uint16_t* m_f16,
                         int64_t N, int64_t K, void* dst_host);

/* q: [N][K] bytes (0..15); sc, mn: [N][K/32] bytes (6-bit, 0..63); d_f16, dmin_f16:
 * [N][K/256] binary16 bit patterns.  Writes nvq_q4_k_weight_bytes(N, K) bytes to
 * dst_host.  K % 256 == 0.  NVQ_ERR_RANGE if a code exceeds 15 or a scale or min
 * exceeds 63.  Host memory only, caller-owned.
 * Follows: the llama.cpp 2-bit GGUF tutorial, GGML type table (Q4_K: 256 values in
 * 144 bytes) and "HANDOFF: flint CPU optimization (Q4_1 + NVFP4)", section 1 (Q4_K
 * among the formats of the same work). */
nvq_status nvq_pack_q4_k(const uint8_t* q, const uint8_t* sc, const uint8_t* mn, const uint16_t* d_f16,
                         const uint16_t* dmin_f16, int64_t N, int64_t K, void* dst_host);

/* q: [N][K] bytes (0..31); sc, mn: [N][K/32] bytes (6-bit, 0..63); d_f16, dmin_f16:
 * [N][K/256] binary16 bit patterns.  Writes nvq_q5_k_weight_bytes(N, K) bytes to
 * dst_host.  K % 256 == 0.  NVQ_ERR_RANGE if a code exceeds 31 or a scale or min 63.
 * Host memory only, caller-owned.
 * Follows: "HANDOFF: flint CPU optimization (Q4_1 + NVFP4)", section 1 (Q5_K among the
 * formats of the same work; its rule is the GGML format's, not the pages'). */
nvq_status nvq_pack_q5_k(const uint8_t* q, const uint8_t* sc, const uint8_t* mn, const uint16_t* d_f16,
                         const uint16_t* dmin_f16, int64_t N, int64_t K, void* dst_host);

/* q: [N][K] bytes (0..63, used as q - 32); sc: [N][K/16] int8 scales; d_f16: [N][K/256]
 * binary16 bit patterns.  Writes nvq_q6_k_weight_bytes(N, K) bytes to dst_host.
 * K % 256 == 0.  NVQ_ERR_RANGE if a code exceeds 63.  Host memory only.
 * Follows: "HANDOFF: flint CPU optimization (Q4_1 + NVFP4)", section 1 (Q6_K among the
 * formats of the same work; its rule is the GGML format's, not the pages'). */
nvq_status nvq_pack_q6_k(const uint8_t* q, const int8_t* sc, const uint16_t* d_f16, int64_t N, int64_t K,
                         void* dst_host);

/* q: [N][K] bytes (0..15, indices into the value table); ls: [N][K/32] bytes (6-bit,
 * 0..63); d_f16: [N][K/256] binary16 bit patterns.  Writes nvq_iq4_xs_weight_bytes(N, K)
 * bytes to dst_host.  K % 256 == 0.  NVQ_ERR_RANGE if a code exceeds 15 or a scale 63.
 * The value table is not part of the buffer; the products take it.  Host memory only.
 * Follows: the llama.cpp 2-bit GGUF tutorial, GGML type table (IQ4_XS: 256 values in
 * 136 bytes) and "HANDOFF: flint CPU optimization (Q4_1 + NVFP4)", section 1 (IQ4_XS
 * among the formats of the same work). */
nvq_status nvq_pack_iq4_xs(const uint8_t* q, const uint8_t* ls, const uint16_t* d_f16, int64_t N, int64_t K,
                           void* dst_host);

/* ---- activation quantization ------------------------------------------------ */

/* Q8_0 quantization of x [M][K] float32 into q [M][K] int8, d_f16 [M][K/32]
 * (binary16 bits) and, if bsum16 is not NULL, bsum16 [M][K/16] int16 (all device).
 * M >= 1, K % 32 == 0.  Bit-exact with the definition above.  Non-finite x, or
 * amax > 65504 * 127, are outside the contract.
 * Follows: the llama.cpp 2-bit GGUF tutorial, GGML type table (Q8_0: 32 int8 codes
 * and one binary16 d per block); "HANDOFF: flint CPU optimization (Q4_1 + NVFP4)",
 * section 3, bias-trick paragraph (the per-16 sums of the activation codes). */
nvq_status nvq_quantize_act_q8_0(const float* x, int64_t M, int64_t K,
                                 int8_t* q, uint16_t* d_f16, int16_t* bsum16, void* stream);

/* ---- NVFP4 products ----------------------------------------------------------- */

/* Decode GEMV (the single-token case of the product): 1 <= M <= NVQ_GEMV_MAX_M,
 * N >= 1, K % 64 == 0.  w: packed NVFP4 [N][K]; q, d_f16: Q8_0 activations [M][K];
 * y [M][N] float32 (overwritten).  M == 1 runs the decode kernel whose per-16
 * integer sums come from the matrix cores reading the FP4 codes directly (K up to
 * what its on-chip activation table holds, about 70000; longer rows run the tiled
 * kernel).  2 <= M runs the batched kernel (M * K < 2^32, NVQ_ERR_SHAPE otherwise),
 * all tokens in one launch streaming the weights once: exact binary16 operands
 * (E2M1 * UE4M3 weights; d * q split exactly into two binary16 terms, activation
 * blocks with d >= 512 in a second pass at d / 256) on the fp16 matrix cores, any K.
 * Per output the error against the exact product is at most 1e-5 * sum_k |W*A|
 * + 1e-6 (float32 accumulation of exact terms).
 * Follows: "HANDOFF: flint CPU optimization (Q4_1 + NVFP4)", section 3, Code map
 * (the batch-1 vector dot: one integer sum per 16-subblock, scaled once by the
 * subblock's UE4M3 and the block's activation scale). */
nvq_status nvq_gemv_nvfp4(const void* w, float w_scale, const int8_t* q, const uint16_t* d_f16,
                          int64_t M, int64_t N, int64_t K, float* y, void* stream);

/* Decode GEMV of one token with its Q8_0 activation quantization fused in: x [K]
 * float32 (device, 16-byte aligned), y [N] float32 = the nvq_gemv_nvfp4 result for
 * the codes and scales nvq_quantize_act_q8_0 gives for x (same Q8_0 definition, bit
 * for bit; same error bound).  One launch: every block of the decode kernel
 * quantizes x into its on-chip activation table, so no quantization launch and no
 * round trip of the codes through memory precede the product.  q_out [K] int8 and
 * d_out [K/32] binary16 (device; both NULL or both given) receive the codes and
 * scales it used, e.g. for a later product on the same activations.  N >= 1,
 * K % 64 == 0, K within the decode kernel's LDS table (about 70000; NVQ_ERR_SHAPE
 * beyond).  Several tokens take nvq_quantize_act_q8_0 + nvq_gemv_nvfp4 (the batched
 * kernel streams the weights once for all of them).
 * Follows: "HANDOFF: flint CPU optimization (Q4_1 + NVFP4)", section 3, Code map
 * (the tiled path repacks the Q8_0 activations itself, tiled_unpack_src1) and
 * section 7 item 1 (decode is bandwidth-bound: every extra pass over memory costs). */
nvq_status nvq_gemv_nvfp4_fused(const void* w, float w_scale, const float* x, int64_t N, int64_t K, float* y,
                                int8_t* q_out, uint16_t* d_out, void* stream);

/* The same decode GEMV with the per-16 integer sums computed on the vector unit:
 * E2M1 -> int8 by v_perm_b32 table lookups and v_dot4_i32_i8 (one launch per
 * token).  Same arguments, results within the same bound.  K is limited to what
 * the on-chip activation table holds (NVQ_ERR_SHAPE beyond, about 70000).
 * Follows: "HANDOFF: flint CPU optimization (Q4_1 + NVFP4)", section 3, Code map and
 * bias-trick paragraph (integer LUT of the codes, int8 dot products per 16). */
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
 * values (hi + lo = d * q); activation blocks with d >= 512, whose d * q can pass
 * the binary16 range, are summed in a second pass at d / 256, so every finite
 * activation in the contract is exact.  Same error bound as the GEMV.
 * Follows: "HANDOFF: flint CPU optimization (Q4_1 + NVFP4)", section 3, Code map
 * (batches larger than one take a tiled matmul that unpacks weight and activation
 * tiles and applies the per-16 weight scale beside them). */
nvq_status nvq_gemm_nvfp4(const void* w, float w_scale, const int8_t* q, const uint16_t* d_f16,
                          int64_t M, int64_t N, int64_t K, float* y,
                          void* workspace, size_t ws_bytes, void* stream);

/* The same prefill GEMM for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation): no
 * workspace argument; the K-split partial tiles go to a static scratch array inside
 * the library, NVQ_NOALLOC_SCRATCH_BYTES (64 MiB) per GPU it runs on, held until the
 * process ends.  Every valid shape fits (the largest K-split plan needs exactly that
 * much); a shape that needed more would be rejected with NVQ_ERR_WORKSPACE.  The call
 * allocates nothing and needs no cleared memory.  Calls on one GPU share its scratch:
 * calls that overlap in time on one GPU (different streams, or different host threads)
 * race and give wrong results; serialise them.  Results equal nvq_gemm_nvfp4's. */
#define NVQ_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
nvq_status nvq_gemm_nvfp4_noalloc(const void* w, float w_scale, const int8_t* q, const uint16_t* d_f16,
                                  int64_t M, int64_t N, int64_t K, float* y, void* stream);

/* ---- Q4_1 products ------------------------------------------------------------ */

/* Q4_1 GEMV (1 <= M <= NVQ_GEMV_MAX_M) and GEMM (M >= 16); K % 32 == 0.
 * bsum16 [M][K/16] (from nvq_quantize_act_q8_0) is required: the offset m of each
 * 32-block multiplies the sum of that block's activation codes.  Same error bound
 * as the NVFP4 entries.  The GEMM takes a device workspace as nvq_gemm_nvfp4 does,
 * of nvq_gemm_workspace_bytes(NVQ_FMT_Q4_1, M, N, K) bytes (NULL when that is 0).
 * For M > 16 with K % 64 == 0 the GEMM sums code x activation code per 32-block
 * exactly on the int8 matrix cores and applies d, m and the activation scale in
 * float32 (any finite d, m and activation scale); each block's codes are taken
 * relative to the code nearest the block's zero crossing (-m / d), so the scale and
 * offset parts of a weight never dwarf the weight itself.
 * Follows: "HANDOFF: flint CPU optimization (Q4_1 + NVFP4)", section 1 (Q4_1 vec_dot
 * and tiled kernels beside the NVFP4 ones) and section 3, bias-trick paragraph (the
 * activation code sums that the offset term needs); the llama.cpp 2-bit GGUF
 * tutorial, GGML type table (Q4_1 block). */
nvq_status nvq_gemv_q4_1(const void* w, const int8_t* q, const uint16_t* d_f16,
                         const int16_t* bsum16, int64_t M, int64_t N, int64_t K, float* y,
                         void* stream);
nvq_status nvq_gemm_q4_1(const void* w, const int8_t* q, const uint16_t* d_f16,
                         const int16_t* bsum16, int64_t M, int64_t N, int64_t K, float* y,
                         void* workspace, size_t ws_bytes, void* stream);

/* ---- Q4_K products ------------------------------------------------------------ */

/* Q4_K GEMV (1 <= M <= NVQ_GEMV_MAX_M) and GEMM (M >= 16); K % 256 == 0; arguments
 * as the Q4_1 entries (bsum16 required: the min term multiplies each 32-block's
 * activation code sum), workspace of nvq_gemm_workspace_bytes(NVQ_FMT_Q4_K, M, N, K)
 * bytes for the GEMM.  Per 32-block a Q4_K weight is a Q4_1 weight with scale
 * d * sc and offset -dmin * mn (both exact in float32), and the Q4_1 kernels run it:
 * the integer-dot GEMV for rows up to 20480 weights, the integer-MFMA GEMM above that
 * and for M > 16.  Same error bound as the NVFP4 entries.
 * Follows: "HANDOFF: flint CPU optimization (Q4_1 + NVFP4)", section 1 (Q4_K among the
 * patch's formats, beside its Q4_1 vec_dot and tiled kernels); the llama.cpp 2-bit
 * GGUF tutorial, GGML type table (Q4_K block). */
nvq_status nvq_gemv_q4_k(const void* w, const int8_t* q, const uint16_t* d_f16,
                         const int16_t* bsum16, int64_t M, int64_t N, int64_t K, float* y,
                         void* stream);
nvq_status nvq_gemm_q4_k(const void* w, const int8_t* q, const uint16_t* d_f16,
                         const int16_t* bsum16, int64_t M, int64_t N, int64_t K, float* y,
                         void* workspace, size_t ws_bytes, void* stream);

/* ---- Q5_K and Q6_K products ------------------------------------------------ */

/* Q5_K GEMV (1 <= M <= NVQ_GEMV_MAX_M) and GEMM (M >= 16); K % 256 == 0; arguments and
 * workspace (NVQ_FMT_Q5_K) as the Q4_K entries, bsum16 required.  Per 32-block a Q5_K
 * weight is the Q4_K block's scale d * sc and offset -dmin * mn on a 5-bit code: the
 * GEMV kernel splices the fifth bits into the code bytes before v_dot4_i32_i8, the
 * integer-MFMA GEMM into its int8 code bytes.
 * Q6_K GEMV and GEMM: no bsum16 (no offset term); workspace NVQ_FMT_Q6_K.  One scale
 * d * sc per 16 weights on the values q - 32: the GEMV kernel sums (q - 32) * a as
 * v_dot4 of the 6-bit code bytes plus v_dot4 of bytes -32, per 16-block half; the
 * GEMM forms d * sc * (q - 32) exactly in float32 and splits it into two binary16
 * terms on the fp16 matrix cores (the per-16 scales would double the integer-MFMA
 * kernel's vector work).  Same dispatch and error bound as the Q4_K entries.
 * Follows: "HANDOFF: flint CPU optimization (Q4_1 + NVFP4)", section 1 (Q5_K and Q6_K
 * among the patch's formats); the rules are the GGML formats' (the pages give none). */
nvq_status nvq_gemv_q5_k(const void* w, const int8_t* q, const uint16_t* d_f16,
                         const int16_t* bsum16, int64_t M, int64_t N, int64_t K, float* y,
                         void* stream);
nvq_status nvq_gemm_q5_k(const void* w, const int8_t* q, const uint16_t* d_f16,
                         const int16_t* bsum16, int64_t M, int64_t N, int64_t K, float* y,
                         void* workspace, size_t ws_bytes, void* stream);
nvq_status nvq_gemv_q6_k(const void* w, const int8_t* q, const uint16_t* d_f16, int64_t M, int64_t N, int64_t K,
                         float* y, void* stream);
nvq_status nvq_gemm_q6_k(const void* w, const int8_t* q, const uint16_t* d_f16, int64_t M, int64_t N, int64_t K,
                         float* y, void* workspace, size_t ws_bytes, void* stream);

/* ---- IQ4_XS products ---------------------------------------------------------- */

/* IQ4_XS GEMV (1 <= M <= NVQ_GEMV_MAX_M) and GEMM (M >= 16); K % 256 == 0; table: the
 * 16 int8 values the codes index (HOST memory, read during the call; the kernels
 * receive it by value).  No bsum16 (the format has no offset term).  Workspace of
 * nvq_gemm_workspace_bytes(NVQ_FMT_IQ4_XS, M, N, K) bytes for the GEMM.  The Q4_1 / Q4_K
 * kernels run it: per 32-block the scale d * (ls - 32) (exact in float32), the codes
 * mapped through the table by v_perm_b32 lookups -- int8 values into v_dot4_i32_i8 in
 * the GEMV kernel and into the int8 matrix-core operands of the GEMM.
 * Same error bound as the NVFP4 entries.
 * Follows: "HANDOFF: flint CPU optimization (Q4_1 + NVFP4)", section 1 (IQ4_XS among the
 * patch's formats); the llama.cpp 2-bit GGUF tutorial, GGML type table (IQ4_XS block). */
nvq_status nvq_gemv_iq4_xs(const void* w, const int8_t* table, const int8_t* q, const uint16_t* d_f16,
                           int64_t M, int64_t N, int64_t K, float* y, void* stream);
nvq_status nvq_gemm_iq4_xs(const void* w, const int8_t* table, const int8_t* q, const uint16_t* d_f16,
                           int64_t M, int64_t N, int64_t K, float* y, void* workspace, size_t ws_bytes,
                           void* stream);

/* ---- debug: integer per-16 partial sums --------------------------------------- */

/* isums [M][N][K/16] int32 (device, overwritten) = for each 16-subblock,
 * sum_j L(code) * q (NVFP4, with L(c) = 2*E2M1(c), an integer in -12..12) or
 * sum_j code * q (Q4_1, Q4_K and Q5_K, unsigned codes) or sum_j (code - 32) * q (Q6_K).
 * fmt: NVQ_FMT_* (not IQ4_XS).  path picks the
 * product entry whose kernel computes the sums, run with unit scales (UE4M3 = 1,
 * d = 1; Q4_1 / Q4_K / Q5_K / Q6_K block scale 1, offset 0 or -32) through its own weight loads, code
 * expansion and integer or
 * matrix-core contraction -- the kernel that entry dispatches for this M:
 *   NVQ_PATH_GEMV      nvq_gemv_nvfp4 / nvq_gemv_q4_1: NVFP4 M = 1 the matrix-core
 *                      decode kernel (the tiled kernel past its LDS table), M >= 2 the
 *                      batched kernel (16 tokens per launch); Q4_1 the GEMV kernel;
 *   NVQ_PATH_GEMM      nvq_gemm_nvfp4 / nvq_gemm_q4_1 (any M >= 1): NVFP4 M = 1 the
 *                      tiled kernel, 2 <= M <= 16 the batched kernel, M > 16 the
 *                      two-term kernel of M's tile height with its K-split work items;
 *                      Q4_1 M <= 16 the GEMV kernel, M > 16 the integer-MFMA
 *                      kernel (K % 64 == 0; one int8 MFMA per 16-block, the other
 *                      half of the weight operand zeroed) or the tiled kernel;
 *                      Q4_K, Q5_K, Q6_K as their entries dispatch (GEMV kernel, or
 *                      the integer-MFMA kernel; Q6_K the two-term kernel);
 *   NVQ_PATH_GEMV_DOT4 nvq_gemv_nvfp4_dot4 (NVFP4 only): the v_dot4 decode kernel,
 *                      one launch per token.
 * K % 64 == 0 (NVFP4), K % 32 == 0 (Q4_1) or K % 256 == 0 (Q4_K, Q5_K, Q6_K).
 * Follows: "HANDOFF: flint CPU optimization (Q4_1 + NVFP4)", section 3, Code map
 * (one int32 sum per 16-subblock, lane k of the sum = subblock k/2) and bias-trick
 * paragraph; the integer sums are unique, so they are checked bit for bit. */
nvq_status nvq_debug_isums(int fmt, int path, const void* w, const int8_t* q,
                           int64_t M, int64_t N, int64_t K, int32_t* isums, void* stream);

/* The same for IQ4_XS weights, whose sums need the value table (host memory):
 * isums [M][N][K/16] = sum_j table[code] * q, from the kernel nvq_gemv_iq4_xs
 * (path NVQ_PATH_GEMV) or nvq_gemm_iq4_xs (NVQ_PATH_GEMM, any M >= 1) dispatches for
 * the shape, with unit block scales.  K % 256 == 0.
 * Follows: "HANDOFF: flint CPU optimization (Q4_1 + NVFP4)", section 3, Code map (one
 * int32 sum per 16-subblock). */
nvq_status nvq_debug_isums_iq4_xs(const int8_t* table, int path, const void* w, const int8_t* q,
                                  int64_t M, int64_t N, int64_t K, int32_t* isums, void* stream);

/* ---- errors ------------------------------------------------------------------- */

/* Name of a status code, and the calling thread's last error message (static
 * strings owned by the library).  The pages print no error API; "HANDOFF: flint CPU
 * optimization (Q4_1 + NVFP4)", section 3 (kernel tests pass silently on zeroed
 * decode tables unless the library is initialised) and its VNNI-only dispatch guard
 * are why this library has no silent init and no silent fallback path. */
const char* nvq_status_str(nvq_status s);
const char* nvq_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* NVQ_H */
