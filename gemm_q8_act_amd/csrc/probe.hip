// probe.hip -- measurement probes: the ceilings the product kernels are compared with.
//
// None of these computes anything of the method.  They measure what the chip gives a
// kernel of a given shape, so that a kernel's time can be read as a fraction of a
// measured ceiling as well as of the published peaks ("Roofline-First Decoding:
// results" reports each kernel against a measured bandwidth ceiling):
//
//  * probe_read_kernel: a plain streaming read (16-byte non-temporal loads, eight in
//    flight per thread) -- the chip's read rate on a long stream.
//  * probe_gemv_loads_kernel: exactly the weight loads of the single-token decode
//    GEMV (gemv_nvfp4.hip: one block of W wavefronts per 16-row tile, wavefront v
//    taking chunks v, v + W, ... in batches of P, a 16-byte code load and a 2-byte
//    scale load per lane and chunk, non-temporal, indices clamped), optionally with
//    each tile's chunks split over S blocks -- the loads-only floor of a launch shape.
//  * probe_mfma_kernel: back-to-back v_mfma_f32_32x32x16_f16 on register operands,
//    constant or hashed per lane -- the matrix-core rate the board sustains (it lowers
//    its clock when the operands toggle many bits).
//
// Every kernel folds what it read or computed into one value per wavefront and stores
// it, so no load or MFMA is dead code.
#include "nvq_device.h"
#include "nvq_launch.h"

namespace nvq {

namespace {

// XOR over the 64 lanes of a wavefront (every lane receives it)
__device__ __forceinline__ uint32_t wave_xor(uint32_t v) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) v ^= __shfl_xor(v, o, 64);
  return v;
}

constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 8;

// Each block streams contiguous 32 KB segments (256 threads x 8 loads of 16 bytes,
// every load instruction of a wavefront covering 1 KB), segment j + gridDim.x after
// segment j: measured 7.0-7.1 TB/s at 2048-16384 blocks, against 6.1-6.8 TB/s for a
// grid-stride order whose eight loads per thread lie a whole grid apart.
__global__ __launch_bounds__(kReadThreads) void probe_read_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                                  uint32_t* __restrict__ sink) {
  constexpr int64_t kSeg = (int64_t)kReadThreads * kReadUnroll;
  uint32_t acc = 0u;
  for (int64_t seg = (int64_t)blockIdx.x * kSeg; seg < n16; seg += (int64_t)gridDim.x * kSeg) {
    u32x4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) {
      const int64_t i = seg + threadIdx.x + kReadThreads * u;
      v[u] = i < n16 ? __builtin_nontemporal_load(src + i) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  acc = wave_xor(acc);
  if ((threadIdx.x & 63) == 0) sink[blockIdx.x * (kReadThreads / 64) + (threadIdx.x >> 6)] = acc;
}

template <int W, int P>
__global__ __launch_bounds__(64 * W) void probe_gemv_loads_kernel(const uint8_t* __restrict__ w, int64_t N, int K,
                                                                  int S, uint32_t* __restrict__ sink) {
  const int nch = (K + 127) >> 7;
  const int64_t ntiles = (N + 15) >> 4;
  const int64_t tile = blockIdx.x / S;
  const int s = (int)(blockIdx.x % S);
  const int c_lo = (int)((int64_t)s * nch / S), c_hi = (int)((int64_t)(s + 1) * nch / S);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint8_t* __restrict__ wt = w + tile * nch * 1024 + 16 * lane;
  const uint8_t* __restrict__ st = w + ntiles * nch * 1024 + tile * nch * 128 + 2 * lane;
  uint32_t acc = 0u;
  for (int c0 = c_lo + wave; c0 < c_hi; c0 += W * P) {
    u32x4 bb[P];
    uint32_t ss[P];
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int c = min(c0 + W * p, c_hi - 1);
      bb[p] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wt + (int64_t)c * 1024));
      ss[p] = __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(st + (int64_t)c * 128));
    }
#pragma unroll
    for (int p = 0; p < P; ++p) acc ^= bb[p].x ^ bb[p].y ^ bb[p].z ^ bb[p].w ^ ss[p];
  }
  acc = wave_xor(acc);
  if (lane == 0) sink[(int64_t)blockIdx.x * W + wave] = acc;
}

constexpr int kMfmaThreads = 256;

// 12 MFMAs per iteration over four accumulators and two operand sets
__global__ __launch_bounds__(kMfmaThreads) void probe_mfma_kernel(int64_t iters, int rnd, float* __restrict__ out) {
  const uint32_t tid = blockIdx.x * kMfmaThreads + threadIdx.x;
  half8_t a0, a1, b0, b1;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (rnd) {
      // a 32-bit integer hash (multiply-xorshift) of (thread, element) -> [-1, 1)
      auto h = [&](uint32_t k) {
        uint32_t x = tid * 0x9E3779B9u + k * 0x85EBCA6Bu + 0x27D4EB2Fu;
        x ^= x >> 15;
        x *= 0x2C1B3C6Du;
        x ^= x >> 12;
        return (_Float16)((float)(x >> 8) * (1.0f / 8388608.0f) - 1.0f);
      };
      a0[i] = h(4 * i);
      a1[i] = h(4 * i + 1);
      b0[i] = h(4 * i + 2);
      b1[i] = h(4 * i + 3);
    } else {
      a0[i] = a1[i] = (_Float16)(0.001f * (i + 1));
      b0[i] = b1[i] = (_Float16)(0.002f * (i + 3));
    }
  }
  floatx16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int64_t it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, b0, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, b1, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, b1, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, b0, c3, 0, 0, 0);
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, b1, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, b0, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, b0, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, b1, c3, 0, 0, 0);
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, b1, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, b0, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, b0, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, b1, c3, 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  out[tid] = s;
}

}  // namespace

hipError_t launch_probe_read(const void* src, int64_t n16, int blocks, uint32_t* sink, hipStream_t stream) {
  hipLaunchKernelGGL(probe_read_kernel, dim3((unsigned)blocks), dim3(kReadThreads), 0, stream,
                     static_cast<const u32x4*>(src), n16, sink);
  return hipGetLastError();
}

hipError_t launch_probe_gemv_loads(const uint8_t* w, int64_t N, int64_t K, int splits, int waves, int batch,
                                   uint32_t* sink, hipStream_t stream) {
  const unsigned grid = (unsigned)(((N + 15) >> 4) * splits);
#define NVQ_PROBE_CASE(W_, P_)                                                                       \
  if (waves == W_ && batch == P_) {                                                                  \
    hipLaunchKernelGGL((probe_gemv_loads_kernel<W_, P_>), dim3(grid), dim3(64 * W_), 0, stream, w, N, \
                       (int)K, splits, sink);                                                        \
    return hipGetLastError();                                                                        \
  }
  NVQ_PROBE_CASE(4, 3)
  NVQ_PROBE_CASE(4, 5)
  NVQ_PROBE_CASE(8, 3)
  NVQ_PROBE_CASE(8, 5)
  NVQ_PROBE_CASE(16, 3)
  NVQ_PROBE_CASE(16, 5)
#undef NVQ_PROBE_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_probe_mfma(int blocks, int64_t iters, int random_operands, float* out, hipStream_t stream) {
  hipLaunchKernelGGL(probe_mfma_kernel, dim3((unsigned)blocks), dim3(kMfmaThreads), 0, stream, iters,
                     random_operands ? 1 : 0, out);
  return hipGetLastError();
}

}  // namespace nvq
