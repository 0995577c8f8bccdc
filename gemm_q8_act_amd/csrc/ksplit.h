// ksplit.h -- work items and the ordered K-split reduction shared by the two-term
// GEMM kernels (gemm_nvfp4.hip, q4_1.hip).
//
// A GEMM of T output tiles runs as one work item per tile while whole rounds over
// the chip's 256 compute units fill up; the r = T mod 256 tiles of an incomplete last
// round are each split along K into up to 16 parts (at most one per 64-k stage), so
// the last round has about 256 items too.  A split part writes its fp32 accumulators
// to the workspace, element-major (slot e of producer thread t at e * 512 + t), and
// ksplit_reduce_kernel sums the parts of each tile in part order -- deterministic,
// no atomics.
#pragma once

#include <algorithm>
#include <type_traits>

#include "nvq_device.h"

namespace nvq {

constexpr int kKSplitSlots = 256;   // compute units of the chip: work items of the last round
constexpr int kKSplitMax = 16;      // parts per split tile
constexpr int kKSplitThreads = 512; // threads of a GEMM work item

struct KSplitPlan {
  int64_t tiles_n, tiles, full, split_tiles;
  int split;  // K parts per split tile (1: no split)
  int stages; // 64-k stages of K
};

template <int BN, int BM>
inline KSplitPlan ksplit_plan(int64_t M, int64_t N, int64_t K) {
  KSplitPlan p;
  p.tiles_n = (N + BN - 1) / BN;
  p.tiles = p.tiles_n * ((M + BM - 1) / BM);
  p.stages = (int)(K / 64);
  const int64_t r = p.tiles % kKSplitSlots;
  p.split = 1;
  if (r != 0) p.split = (int)std::min<int64_t>({kKSplitSlots / r, (int64_t)kKSplitMax, (int64_t)p.stages});
  if (p.split < 2) p.split = 1;
  p.split_tiles = p.split > 1 ? r : 0;
  p.full = p.tiles - p.split_tiles;
  return p;
}

// workspace bytes of configuration C (fields BN, BM, kAcc: fp32 accumulators per thread)
template <class C>
inline size_t ksplit_workspace(int64_t M, int64_t N, int64_t K) {
  const KSplitPlan p = ksplit_plan<C::BN, C::BM>(M, N, K);
  return (size_t)(p.split_tiles * p.split) * kKSplitThreads * C::kAcc * sizeof(float);
}

// Sums the K parts of every split tile in part order (s = part 0, s += part 1, ...),
// multiplies by `scale` and stores the tile.  Block (split tile, 16 accumulator slots
// e0 .. e0 + 15 = one v_mfma_f32_32x32x16 tile of every producer thread): thread t
// takes slots e0 + 8 (t / 512) .. + 7 of producer thread t % 512, so each load of a
// part is a coalesced 2 KB row and one block writes whole 128-byte lines of y.
// C describes the producer: WM wavefronts along m, TN x TM MFMA tiles per wavefront.
// producers whose MFMA rows are tokens (C::kRowsM, the integer-MFMA kernel) rather
// than weight rows
template <class C, class = void>
struct ksplit_rows_m : std::false_type {};
template <class C>
struct ksplit_rows_m<C, std::void_t<decltype(C::kRowsM)>> : std::integral_constant<bool, C::kRowsM> {};

template <class C>
__global__ __launch_bounds__(1024) void ksplit_reduce_kernel(const float* __restrict__ part_ws, int64_t N,
                                                             int64_t M, float scale, float* __restrict__ y,
                                                             KSplitPlan plan) {
  constexpr int WM = C::WM, TN = C::TN, TM = C::TM, kAcc = C::kAcc, kTiles = TN * TM;
  const int half = threadIdx.x >> 9, ptid = threadIdx.x & 511;
  const int lane = ptid & 63, wave = ptid >> 6;
  const int wn = wave / WM, wm = wave % WM;
  const int64_t st = blockIdx.x / kTiles;  // split tile index
  const int ij = blockIdx.x % kTiles, i = ij / TM, j = ij % TM;
  const int e0 = 16 * ij + 8 * half;
  const int64_t tile = plan.full + st;
  const int64_t n0 = (tile % plan.tiles_n) * C::BN, m0 = (tile / plan.tiles_n) * C::BM;
  const float* src = part_ws + (st * plan.split * kAcc + e0) * kKSplitThreads + ptid;
  float s[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) s[e] = src[e * kKSplitThreads];
  // later parts four at a time, their loads issued before the adds
  for (int p0 = 1; p0 < plan.split; p0 += 4) {
    float v[4][8];
#pragma unroll
    for (int pp = 0; pp < 4; ++pp)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        v[pp][e] = p0 + pp < plan.split ? src[((int64_t)(p0 + pp) * kAcc + e) * kKSplitThreads] : 0.0f;
#pragma unroll
    for (int pp = 0; pp < 4; ++pp)
      if (p0 + pp < plan.split) {
#pragma unroll
        for (int e = 0; e < 8; ++e) s[e] += v[pp][e];
      }
  }
  if constexpr (ksplit_rows_m<C>::value) {
    // tile ij = (token tile i, weight tile j) with i = ij / TN; slot e0 + 4 h + rr holds
    // token row 8 ((e0 % 16) / 4 + h) + 4 (lane >> 5) + rr of weight row lane % 32
    const int ti = ij / TN, tj = ij % TN;
    const int64_t n = n0 + wn * (32 * TN) + 32 * tj + (lane & 31);
    if (n >= N) return;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int64_t m = m0 + wm * (32 * TM) + 32 * ti + 8 * ((e0 & 15) / 4 + h) + 4 * (lane >> 5) + rr;
        if (m < M) y[m * N + n] = s[4 * h + rr] * scale;
      }
    return;
  }
  const int64_t m = m0 + wm * (32 * TM) + 32 * j + (lane & 31);
  if (m >= M) return;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    // slot e0 + 4 h + rr of the producer holds row 8 ((e0 % 16) / 4 + h) + 4 (lane >> 5) + rr
    const int64_t n = n0 + wn * (32 * TN) + 32 * i + 8 * ((e0 & 15) / 4 + h) + 4 * (lane >> 5);
    const floatx4 o = {s[4 * h] * scale, s[4 * h + 1] * scale, s[4 * h + 2] * scale, s[4 * h + 3] * scale};
    if ((N & 3) == 0 && n + 3 < N) {
      *reinterpret_cast<floatx4*>(y + m * N + n) = o;
    } else {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
        if (n + rr < N) y[m * N + n + rr] = o[rr];
    }
  }
}

template <class C>
inline hipError_t launch_ksplit_reduce(const float* part_ws, int64_t N, int64_t M, float scale, float* y,
                                       const KSplitPlan& plan, hipStream_t stream) {
  hipLaunchKernelGGL(ksplit_reduce_kernel<C>, dim3((unsigned)(plan.split_tiles * C::TN * C::TM)), dim3(1024), 0,
                     stream, part_ws, N, M, scale, y, plan);
  return hipGetLastError();
}

}  // namespace nvq
