// act_quant.hip -- Q8_0 activation quantization on gfx950.
//
// Q8_0 (llama.cpp 2-bit GGUF tutorial, GGML type table: 32 values in 34 bytes) with
// the per-16 code sums the NVFP4 path consumes ("HANDOFF: flint CPU optimization
// (Q4_1 + NVFP4)", section 3, bias-trick paragraph: bsums are per-16 sums of the
// int8 activation codes).
//
// Mapping: the [M][K] input is a flat sequence of M*K/32 blocks (rows are whole
// blocks because K % 32 == 0).  Eight lanes own one block, four floats each, so a
// wavefront reads 1 KB of contiguous float4 and writes 256 B of contiguous codes per
// block group; on large inputs each thread keeps two such groups' loads in flight.
// HBM-bound: 4 B read + 1 B written per element (+ 2 B per 32 and 2 B per 16).
#include "nvq_device.h"
#include "nvq_launch.h"

namespace nvq {

// Large inputs: each thread issues the loads of U = 2 blocks (2 x 16 B in flight)
// before computing either, for more bytes in flight per wavefront (M = 2048,
// K = 17408: 29 us instead of 33).  Small inputs keep U = 1: there the kernel is a
// latency chain, and a second block per thread lengthens it (M = 1: 2.0 vs 2.2 us).
constexpr int64_t kQuantWideBlocks = 1 << 16;

// one 32-value block: lanes 8g .. 8g+7 of the wavefront hold its 32 floats (4 each)
__device__ __forceinline__ void quant_block(float4 v, int64_t g, int p, bool valid, int8_t* __restrict__ q,
                                            uint16_t* __restrict__ d16, int16_t* __restrict__ bsum16) {
  // block amax over the 8 lanes of the block (lanes are 8-aligned groups)
  float a = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
  a = fmaxf(a, __shfl_xor(a, 1, 64));
  a = fmaxf(a, __shfl_xor(a, 2, 64));
  a = fmaxf(a, __shfl_xor(a, 4, 64));

  // d32 = amax / 127 and q = rint(x / d32): IEEE float32 division (this file is
  // compiled without fast-math, so '/' is correctly rounded), ties to even.  A
  // block whose d32 is 0 (all zero, or float32 subnormals below 127 * 2^-150)
  // keeps q = 0: x / 0 names no code, and d * q is 0 either way.
  const float d = a / 127.0f;
  int qi[4] = {0, 0, 0, 0};
  if (d != 0.0f) {
    const float xs[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float r = __builtin_rintf(xs[i] / d);
      r = fminf(fmaxf(r, -127.0f), 127.0f);
      qi[i] = (int)r;
    }
  }
  const uint32_t packed = (uint32_t)(qi[0] & 0xFF) | ((uint32_t)(qi[1] & 0xFF) << 8) |
                          ((uint32_t)(qi[2] & 0xFF) << 16) | ((uint32_t)(qi[3] & 0xFF) << 24);

  // per-16 code sums: lanes p = 0..3 cover the first 16 codes, 4..7 the second
  int s = qi[0] + qi[1] + qi[2] + qi[3];
  s += __shfl_xor(s, 1, 64);
  s += __shfl_xor(s, 2, 64);

  if (valid) {
    *reinterpret_cast<uint32_t*>(q + g * 32 + 4 * p) = packed;
    if (p == 0) d16[g] = __builtin_bit_cast(uint16_t, (_Float16)d);  // v_cvt_f16_f32: RNE
    if (bsum16 && (p & 3) == 0) bsum16[2 * g + (p >> 2)] = (int16_t)s;
  }
}

// Workgroup w covers blocks 32 U w .. 32 U (w + 1) - 1; in pass u thread t takes
// block 32 U w + 32 u + t / 8, floats 4 (t % 8) .. + 3 of it, so every pass reads
// 4 KB of contiguous floats.
template <int U>
__global__ __launch_bounds__(256) void act_quant_q8_0_kernel(const float* __restrict__ x,
                                                             int64_t nblk, int8_t* __restrict__ q,
                                                             uint16_t* __restrict__ d16,
                                                             int16_t* __restrict__ bsum16) {
  const int p = (int)(threadIdx.x & 7);  // which 4 floats of the block
  const int64_t g0 = (int64_t)blockIdx.x * (32 * U) + (threadIdx.x >> 3);
  float4 v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t g = g0 + 32 * u;
    v[u] = g < nblk ? *reinterpret_cast<const float4*>(x + g * 32 + 4 * p) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t g = g0 + 32 * u;
    quant_block(v[u], g, p, g < nblk, q, d16, bsum16);
  }
}

hipError_t launch_act_quant(const float* x, int64_t M, int64_t K, int8_t* q, uint16_t* d16,
                            int16_t* bsum16, hipStream_t stream) {
  const int64_t nblk = M * (K / 32);
  if (nblk >= kQuantWideBlocks) {
    hipLaunchKernelGGL(act_quant_q8_0_kernel<2>, dim3((unsigned)((nblk + 63) / 64)), dim3(256), 0, stream, x,
                       nblk, q, d16, bsum16);
  } else {
    hipLaunchKernelGGL(act_quant_q8_0_kernel<1>, dim3((unsigned)((nblk + 31) / 32)), dim3(256), 0, stream, x,
                       nblk, q, d16, bsum16);
  }
  return hipGetLastError();
}

}  // namespace nvq
