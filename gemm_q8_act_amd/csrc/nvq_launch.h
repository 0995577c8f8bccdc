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
// NVFP4, 2 <= M <= 16 tokens: exact fp16 operands on the fp16 matrix core, one launch
// (one weight stream) per 16 tokens.  Any K with M * K < 2^32 (32-bit activation
// offsets; the callers check).
hipError_t launch_gemv_nvfp4_batch_f16(const uint8_t* w, float w_scale, const int8_t* q,
                                       const uint16_t* d16, int64_t M, int64_t N, int64_t K, float* y,
                                       hipStream_t stream);
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
// workspace (may be 0).  isums != nullptr selects the tiled debug variant.
hipError_t launch_gemm_nvfp4(const uint8_t* w, float w_scale, const int8_t* q,
                             const uint16_t* d16, int64_t M, int64_t N, int64_t K, float* y,
                             int32_t* isums, float* workspace, hipStream_t stream);
size_t gemm_nvfp4_workspace(int64_t M, int64_t N, int64_t K);

// Q4_1 GEMV (any M; used for M <= 16), integer-dot path; with isums the
// debug sums [M][N][K/16].
hipError_t launch_gemv_q4_1(const uint8_t* w, const int8_t* q, const uint16_t* d16,
                            const int16_t* bsum16, int64_t M, int64_t N, int64_t K, float* y,
                            int32_t* isums, hipStream_t stream);

// Q4_1 GEMM paths (any M >= 1): M <= 16 the GEMV kernel, M > 16 the two-term fp16
// kernel when K % 64 == 0 (it needs gemm_q4_1_workspace(M, N, K) bytes of device
// workspace, may be 0), else the tiled kernel, which also gives the debug sums.
hipError_t launch_gemm_q4_1(const uint8_t* w, const int8_t* q, const uint16_t* d16,
                            const int16_t* bsum16, int64_t M, int64_t N, int64_t K, float* y,
                            int32_t* isums, float* workspace, hipStream_t stream);
size_t gemm_q4_1_workspace(int64_t M, int64_t N, int64_t K);

}  // namespace nvq
