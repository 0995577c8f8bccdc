/* nvq_probe.h -- measurement probes of libnvq: the ceilings its kernels are compared with.
 *
 * Follows: "Roofline-First Decoding: results" (each kernel is reported as a fraction of a
 * measured ceiling, not only of the published peak).  None of these entries computes any
 * part of the NVFP4 x Q8_0 product; they exist so that a kernel's time can be set against
 * what the chip gives a kernel of the same shape:
 *   - nvq_probe_read: the streaming-read rate of a long buffer;
 *   - nvq_probe_gemv_loads: the weight loads of a decode GEMV launch and nothing else,
 *     i.e. the loads-only floor of that launch shape;
 *   - nvq_probe_mfma: the rate of back-to-back fp16 MFMAs on register operands.
 *
 * Conventions are those of nvq.h: device pointers are caller-owned, calls are asynchronous
 * on `stream` (a hipStream_t, NULL for the default stream), arguments are validated on
 * the host before anything is enqueued (negative nvq_status on error, detail in
 * nvq_last_error), and only gfx950 devices are accepted.  Each probe stores one value per
 * wavefront (an XOR or a sum of what it read or computed) so that no load or MFMA is
 * dead code; the stored values carry no meaning beyond that.
 */
#ifndef NVQ_PROBE_H
#define NVQ_PROBE_H

#include "nvq.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Reads `bytes` bytes of device memory at src with 16-byte non-temporal loads, eight in
 * flight per thread, over `blocks` blocks of 256 threads, each block streaming
 * contiguous 32 KB segments (segment j + blocks after segment j).  src 16-byte
 * aligned; bytes > 0 and a multiple of 16; 1 <= blocks <= 65536.  sink: device,
 * 4 * blocks uint32 (4-byte aligned), one word per wavefront.  Bytes read per call:
 * `bytes`. */
nvq_status nvq_probe_read(const void* src, size_t bytes, int blocks, uint32_t* sink, void* stream);

/* The weight loads of the single-token decode GEMV (nvq_gemv_nvfp4 at M = 1) over the
 * packed NVFP4 matrix w (N x K, the layout of nvq_pack_nvfp4; K % 64 == 0, w 16-byte
 * aligned) and nothing else: `splits` blocks per 16-row tile (1..8, at most the tile's
 * ceil(K/128) chunks), each of `waves` wavefronts (4, 8 or 16) walking its contiguous
 * share of the tile's 128-k chunks in batches of `batch` (3 or 5) -- per lane and chunk
 * a 16-byte code load and a 2-byte scale load, non-temporal, in the GEMV kernel's order.
 * splits = 1 with the GEMV's own (waves, batch) is that launch's loads-only floor.
 * sink: device, waves * ceil(N/16) * splits uint32 (4-byte aligned).  Bytes read per
 * call: N * K * 9 / 16 (the packed weights). */
nvq_status nvq_probe_gemv_loads(const void* w, int64_t N, int64_t K, int splits, int waves, int batch,
                                uint32_t* sink, void* stream);

/* Back-to-back v_mfma_f32_32x32x16_f16 on register operands: `blocks` blocks of 256
 * threads (512 blocks put two wavefronts on every SIMD of a 256-compute-unit chip), each
 * wavefront issuing 12 * iters MFMAs into four accumulators from two operand sets.
 * random_operands != 0 draws every lane's fp16 operands from an integer hash (values in
 * [-1, 1), many bits toggling), 0 keeps them constant.  1 <= blocks <= 65536,
 * 1 <= iters <= 2^31.  out: device, 256 * blocks floats (4-byte aligned), each thread's
 * accumulator sum.  Flops per call: blocks * 4 * 12 * iters * 32768. */
nvq_status nvq_probe_mfma(int blocks, int64_t iters, int random_operands, float* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NVQ_PROBE_H */
