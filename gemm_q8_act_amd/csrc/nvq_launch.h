// nvq_launch.h -- host-side launchers of the gfx950 kernels (internal to libnvq).
// Argument validation is done by the C ABI layer before any of these is called;
// each launcher only picks a kernel configuration and enqueues it on `stream`.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvq {

hipError_t launch_act_quant(const float* x, int64_t M, int64_t K, int8_t* q, uint16_t* d16,
                            int16_t* bsum16, hipStream_t stream);

// NVFP4, M == 1 decode GEMV on the tile-interleaved layout.  mode 0: FP4 MFMA
// inner loop (production); mode 1: v_perm + v_dot4 inner loop.  isums != nullptr
// selects the debug variant (writes per-16 integer sums instead of y).
hipError_t launch_gemv_nvfp4_m1(const uint8_t* w, float w_scale, const int8_t* q,
                                const uint16_t* d16, int64_t N, int64_t K, float* y,
                                int32_t* isums, int mode, hipStream_t stream);
// NVFP4, one token: Q8_0 quantization of the float32 row x fused into the M == 1
// decode GEMV (every block quantizes the row into its LDS table); q_out / d_out, if
// not null, receive the row's codes and binary16 scales.  K within gemv_lds_bytes.
hipError_t launch_gemv_nvfp4_fused(const uint8_t* w, float w_scale, const float* x, int64_t N, int64_t K, float* y,
                                   int8_t* q_out, uint16_t* d_out, hipStream_t stream);
// NVFP4, 2 <= M <= 16 tokens: exact fp16 operands on the fp16 matrix core, one launch
// (one weight stream) per 16 tokens.  Any K with M * K < 2^32 (32-bit activation
// offsets; the callers check).  isums != nullptr selects the debug variant (per-16
// integer sums [M][N][K/16] of the same data path; d16 and y unused).
hipError_t launch_gemv_nvfp4_batch_f16(const uint8_t* w, float w_scale, const int8_t* q,
                                       const uint16_t* d16, int64_t M, int64_t N, int64_t K, float* y,
                                       int32_t* isums, hipStream_t stream);
// NVFP4 expert-routed decode GEMV: E packed expert matrices back to back, ids [M][A]
// (device int32), y [M][A][N]; one launch, grid.y = M * A jobs.
hipError_t launch_gemv_nvfp4_routed(const uint8_t* w, const float* w_scales, const int32_t* ids, int64_t E,
                                    int64_t A, int64_t M, const int8_t* q, const uint16_t* d16, int64_t N,
                                    int64_t K, float* y, hipStream_t stream);
// LDS bytes the decode GEMV needs for a row length K.
size_t gemv_lds_bytes(int64_t K);

// NVFP4 GEMM paths (any M >= 1): M = 1 the tiled kernel (rows too long for the decode
// kernels), 2 <= M <= 16 the batched decode kernel, M > 16 the split-activation
// kernel, whose K-split parts need gemm_nvfp4_workspace(M, N, K) bytes of device
// workspace (may be 0).  isums != nullptr selects the debug variant of the kernel the
// shape dispatches to (per-16 integer sums, no workspace).
hipError_t launch_gemm_nvfp4(const uint8_t* w, float w_scale, const int8_t* q,
                             const uint16_t* d16, int64_t M, int64_t N, int64_t K, float* y,
                             int32_t* isums, float* workspace, hipStream_t stream);
size_t gemm_nvfp4_workspace(int64_t M, int64_t N, int64_t K);
// The same NVFP4 GEMM dispatch with the K-split partials in the library's static
// per-device scratch array (no allocation; calls on one GPU must not overlap), and
// that array's size.
hipError_t launch_gemm_nvfp4_noalloc(const uint8_t* w, float w_scale, const int8_t* q, const uint16_t* d16,
                                     int64_t M, int64_t N, int64_t K, float* y, hipStream_t stream);
size_t gemm_nvfp4_noalloc_scratch_bytes();

// Q4_1 GEMV (any M; used for M <= 16), integer-dot path; with isums the
// debug sums [M][N][K/16].
hipError_t launch_gemv_q4_1(const uint8_t* w, const int8_t* q, const uint16_t* d16,
                            const int16_t* bsum16, int64_t M, int64_t N, int64_t K, float* y,
                            int32_t* isums, hipStream_t stream);

// Q4_1 GEMM paths (any M >= 1): M <= 16 the GEMV kernel, M > 16 the integer-MFMA
// kernel when K % 64 == 0 (it needs gemm_q4_1_workspace(M, N, K) bytes of device
// workspace, may be 0), else the tiled kernel.  isums != nullptr selects the debug
// variant of the kernel the shape dispatches to.
hipError_t launch_gemm_q4_1(const uint8_t* w, const int8_t* q, const uint16_t* d16,
                            const int16_t* bsum16, int64_t M, int64_t N, int64_t K, float* y,
                            int32_t* isums, float* workspace, hipStream_t stream);
size_t gemm_q4_1_workspace(int64_t M, int64_t N, int64_t K);

// Q4_K (K % 256 == 0) on the Q4_1 kernels with the Q4_K block scales.  GEMV entry
// (M <= 16): the GEMV kernel, or for rows longer than 20480 the integer-MFMA kernel
// (Q6_K: the two-term kernel) with one work item per tile.  GEMM (any M >= 1): M <= 16
// (rows up to 20480) the GEMV
// kernel, else the integer-MFMA kernel (Q6_K: the two-term kernel) with
// gemm_q4_k_workspace(M, N, K, fmt is Q6_K) bytes of device workspace (may be 0).
// isums != nullptr: the debug sums of the dispatched kernel.
hipError_t launch_gemv_q4_k(const uint8_t* w, const int8_t* q, const uint16_t* d16,
                            const int16_t* bsum16, int64_t M, int64_t N, int64_t K, float* y,
                            int32_t* isums, hipStream_t stream);
hipError_t launch_gemm_q4_k(const uint8_t* w, const int8_t* q, const uint16_t* d16,
                            const int16_t* bsum16, int64_t M, int64_t N, int64_t K, float* y,
                            int32_t* isums, float* workspace, hipStream_t stream);
size_t gemm_q4_k_workspace(int64_t M, int64_t N, int64_t K, bool q6k);

// IQ4_XS (K % 256 == 0; table: the 16 int8 values the codes index, host memory) on the
// same kernels and with the same dispatch as Q4_K; its workspace is gemm_q4_k_workspace's.
hipError_t launch_gemv_iq4_xs(const uint8_t* w, const int8_t* table, const int8_t* q, const uint16_t* d16,
                              int64_t M, int64_t N, int64_t K, float* y, int32_t* isums, hipStream_t stream);
hipError_t launch_gemm_iq4_xs(const uint8_t* w, const int8_t* table, const int8_t* q, const uint16_t* d16,
                              int64_t M, int64_t N, int64_t K, float* y, int32_t* isums, float* workspace,
                              hipStream_t stream);

// Q5_K and Q6_K (K % 256 == 0) on the same kernels and with the same dispatch as Q4_K;
// their workspace is gemm_q4_k_workspace's.  Q6_K takes no bsum16.
hipError_t launch_gemv_q5_k(const uint8_t* w, const int8_t* q, const uint16_t* d16,
                            const int16_t* bsum16, int64_t M, int64_t N, int64_t K, float* y,
                            int32_t* isums, hipStream_t stream);
hipError_t launch_gemm_q5_k(const uint8_t* w, const int8_t* q, const uint16_t* d16,
                            const int16_t* bsum16, int64_t M, int64_t N, int64_t K, float* y,
                            int32_t* isums, float* workspace, hipStream_t stream);
hipError_t launch_gemv_q6_k(const uint8_t* w, const int8_t* q, const uint16_t* d16, int64_t M, int64_t N,
                            int64_t K, float* y, int32_t* isums, hipStream_t stream);
hipError_t launch_gemm_q6_k(const uint8_t* w, const int8_t* q, const uint16_t* d16, int64_t M, int64_t N,
                            int64_t K, float* y, int32_t* isums, float* workspace, hipStream_t stream);

// Measurement probes (probe.hip): a streaming read of n16 16-byte units over `blocks`
// blocks of 256 threads (sink: 4 words per block); the decode GEMV's weight loads
// alone for waves in {4, 8, 16}, batch in {3, 5} and `splits` blocks per tile (sink:
// waves words per block); a register-only MFMA loop (out: 256 floats per block).
hipError_t launch_probe_read(const void* src, int64_t n16, int blocks, uint32_t* sink, hipStream_t stream);
hipError_t launch_probe_gemv_loads(const uint8_t* w, int64_t N, int64_t K, int splits, int waves, int batch,
                                   uint32_t* sink, hipStream_t stream);
hipError_t launch_probe_mfma(int blocks, int64_t iters, int random_operands, float* out, hipStream_t stream);

}  // namespace nvq
