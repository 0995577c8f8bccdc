// gemm_nvfp4.hip -- tiled MFMA products, NVFP4 weights x Q8_0 activations, gfx950.
//
// Method ("HANDOFF: flint CPU optimization (Q4_1 + NVFP4)", section 3, Code map:
// the tiled path unpacks weight and activation tiles, then runs a microkernel with
// a per-16 weight scale cached beside the unpacked tile).  On gfx950 the
// contraction runs on the matrix cores, on an exact fp16 expansion of the weights:
// w16 = E2M1(code) * UE4M3(scale) has at most 6 significant bits and lies in
// [2^-10, 2688], so it is exact in fp16; activation codes q (|q| <= 127) are exact
// in fp16 too.  Two kernels:
//
//   * gemm_nvfp4_tile_kernel (the debug sums, and M = 1 rows too long for the decode
//     kernels' activation table).  Per 32-k chunk (one Q8_0 block) one v_mfma_f32_16x16x32_f16
//     with a zero accumulator gives P[n][m] = sum_k w16 * q, exact in fp32; the
//     chunk's activation scale is applied on the vector unit,
//     acc[n][m] += d[m][chunk] * P[n][m].  Weights are the MFMA A operand (rows n)
//     and activations B (columns m), so one d value per lane scales all of that
//     lane's accumulators.  A 256-thread block computes BN weight rows x BM tokens
//     per 128-k step from double-buffered LDS.
//   * gemm_nvfp4_kernel (M > 16), below: the activation scale is folded into an
//     exact two-term fp16 split of the activations so the matrix core accumulates
//     the whole row by itself.
// A GEMM of 2 <= M <= 16 tokens runs the batched decode kernel (gemv_batch_f16.hip).
#include <algorithm>
#include <mutex>

#include "ksplit.h"
#include "nvq_device.h"
#include "nvq_launch.h"

namespace nvq {

template <int BM, int BN, bool DEBUG>
__global__ __launch_bounds__(256) void gemm_nvfp4_tile_kernel(const uint8_t* __restrict__ w,
                                                         int64_t N, int K,
                                                         const int8_t* __restrict__ q,
                                                         const uint16_t* __restrict__ d16,
                                                         int64_t M, float w_scale,
                                                         float* __restrict__ y,
                                                         int32_t* __restrict__ isums) {
  constexpr int BK = 128;        // one tile-chunk of the packed layout per step
  constexpr int WN = BN / 4;     // weight rows per wavefront
  constexpr int NT = WN / 16;    // 16-row subtiles per wavefront
  constexpr int MT = BM / 16;    // 16-token subtiles
  constexpr int LDH = BK + 8;    // fp16 per LDS row (272 B: conflict-free 16-byte reads)
  constexpr int WT = (BN * 4 + 255) / 256;  // 32-weight lane slots per thread
  constexpr int AT = (BM * 8 + 255) / 256;  // 16-code activation segments per thread
  static_assert(NT >= 1 && MT >= 1, "tile");

  __shared__ __align__(16) _Float16 lw[2][BN * LDH];
  __shared__ __align__(16) _Float16 la[2][BM * LDH];
  __shared__ float ldv[2][BM * 4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t n0 = (int64_t)blockIdx.x * BN;
  const int64_t m0 = (int64_t)blockIdx.y * BM;
  const int64_t nb32 = K >> 5;
  const int64_t nsb = K >> 4;
  const int nch = (K + BK - 1) / BK;
  const int64_t ntiles = (N + 15) >> 4;
  const uint8_t* __restrict__ sc = w + ntiles * nch * 1024;

  uint4 wreg[WT];
  uint32_t sreg[WT];
  uint4 areg[AT];
  float dval = 0.0f;

  auto gload = [&](int ks) {
#pragma unroll
    for (int i = 0; i < WT; ++i) {
      const int task = tid + 256 * i;
      const int64_t tile = n0 / 16 + (task >> 6);
      if (task < BN * 4 && tile < ntiles) {
        const int64_t blk = tile * nch + ks;
        wreg[i] = *reinterpret_cast<const uint4*>(w + blk * 1024 + 16 * (task & 63));
        sreg[i] = *reinterpret_cast<const uint16_t*>(sc + blk * 128 + 2 * (task & 63));
      } else {
        wreg[i] = make_uint4(0u, 0u, 0u, 0u);
        sreg[i] = 0u;
      }
    }
#pragma unroll
    for (int i = 0; i < AT; ++i) {
      const int task = tid + 256 * i;
      const int r = task >> 3, p = task & 7;
      const int64_t m = m0 + r;
      const int64_t k = (int64_t)ks * BK + 16 * p;
      if (task < BM * 8 && m < M && k < K)
        areg[i] = *reinterpret_cast<const uint4*>(q + m * K + k);
      else
        areg[i] = make_uint4(0u, 0u, 0u, 0u);
    }
    if (!DEBUG && tid < BM * 4) {
      const int64_t m = m0 + (tid >> 2);
      const int64_t b = (int64_t)ks * 4 + (tid & 3);
      dval = (m < M && b < nb32) ? f16_bits_to_f32(d16[m * nb32 + b]) : 0.0f;
    }
  };

  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < WT; ++i) {
      const int task = tid + 256 * i;
      if (task < BN * 4) {
        const int l = task & 63;
        const int r = 16 * (task >> 6) + (l & 15);   // row within the block tile
        const int kq = l >> 4;                        // 32-k quarter of the chunk
        const _Float16 u0 = DEBUG ? (_Float16)1.0f : (_Float16)ue4m3_to_f32<0>(sreg[i]);
        const _Float16 u1 = DEBUG ? (_Float16)1.0f : (_Float16)ue4m3_to_f32<1>(sreg[i]);
        const half2_t s0 = {u0, u0}, s1 = {u1, u1};
        const uint32_t c[4] = {wreg[i].x, wreg[i].y, wreg[i].z, wreg[i].w};
        _Float16* dst = &lw[buf][r * LDH + 32 * kq];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const half2_t s = d < 2 ? s0 : s1;
          half8_t v;
          const half2_t p0 = e2m1x2_to_f16<0>(c[d]) * s;
          const half2_t p1 = e2m1x2_to_f16<1>(c[d]) * s;
          const half2_t p2 = e2m1x2_to_f16<2>(c[d]) * s;
          const half2_t p3 = e2m1x2_to_f16<3>(c[d]) * s;
          v[0] = p0[0]; v[1] = p0[1]; v[2] = p1[0]; v[3] = p1[1];
          v[4] = p2[0]; v[5] = p2[1]; v[6] = p3[0]; v[7] = p3[1];
          *reinterpret_cast<half8_t*>(dst + 8 * d) = v;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < AT; ++i) {
      const int task = tid + 256 * i;
      if (task < BM * 8) {
        const int r = task >> 3, p = task & 7;
        const uint32_t c[4] = {areg[i].x, areg[i].y, areg[i].z, areg[i].w};
        _Float16* dst = &la[buf][r * LDH + 16 * p];
#pragma unroll
        for (int d = 0; d < 4; d += 2) {
          half2_t a0, a1, b0, b1;
          i8x4_to_f16x4(c[d], a0, a1);
          i8x4_to_f16x4(c[d + 1], b0, b1);
          half8_t v;
          v[0] = a0[0]; v[1] = a0[1]; v[2] = a1[0]; v[3] = a1[1];
          v[4] = b0[0]; v[5] = b0[1]; v[6] = b1[0]; v[7] = b1[1];
          *reinterpret_cast<half8_t*>(dst + 4 * d) = v;
        }
      }
    }
    if (!DEBUG && tid < BM * 4) ldv[buf][tid] = dval;
  };

  floatx4 acc[NT][MT];
#pragma unroll
  for (int i = 0; i < NT; ++i)
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[i][t] = floatx4{0.f, 0.f, 0.f, 0.f};

  const int fr = lane & 15;   // fragment row (A) / column (B)
  const int fg = lane >> 4;   // k group: k = 8*fg .. 8*fg+7 of the 32-k block
  const floatx4 zero4 = {0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int buf, int ks) {
#pragma unroll
    for (int c = 0; c < BK / 32; ++c) {
      half8_t a[NT], b[MT];
#pragma unroll
      for (int i = 0; i < NT; ++i)
        a[i] = *reinterpret_cast<const half8_t*>(&lw[buf][(wave * WN + 16 * i + fr) * LDH + 32 * c + 8 * fg]);
#pragma unroll
      for (int t = 0; t < MT; ++t)
        b[t] = *reinterpret_cast<const half8_t*>(&la[buf][(16 * t + fr) * LDH + 32 * c + 8 * fg]);
      if (!DEBUG) {
        float dv[MT];
#pragma unroll
        for (int t = 0; t < MT; ++t) dv[t] = ldv[buf][(16 * t + fr) * 4 + c];
#pragma unroll
        for (int i = 0; i < NT; ++i)
#pragma unroll
          for (int t = 0; t < MT; ++t) {
            const floatx4 p = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[i], b[t], zero4, 0, 0, 0);
            acc[i][t] += dv[t] * p;
          }
      } else {
        const half8_t z8 = {};
#pragma unroll
        for (int i = 0; i < NT; ++i)
#pragma unroll
          for (int t = 0; t < MT; ++t) {
#pragma unroll
            for (int hsub = 0; hsub < 2; ++hsub) {
              // keep only the k groups of one 16-subblock: groups 0,1 or 2,3
              const half8_t bb = ((fg >> 1) == hsub) ? b[t] : z8;
              const floatx4 p = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[i], bb, zero4, 0, 0, 0);
              const int64_t m = m0 + 16 * t + fr;
              const int64_t s = (int64_t)ks * 8 + 2 * c + hsub;
#pragma unroll
              for (int rr = 0; rr < 4; ++rr) {
                const int64_t n = n0 + wave * WN + 16 * i + 4 * fg + rr;
                if (m < M && n < N && s < nsb) isums[(m * N + n) * nsb + s] = (int32_t)(2.0f * p[rr]);
              }
            }
          }
      }
    }
  };

  gload(0);
  lstore(0);
  __syncthreads();
  for (int ks = 0; ks < nch; ++ks) {
    const bool more = ks + 1 < nch;
    if (more) gload(ks + 1);
    compute(ks & 1, ks);
    if (more) lstore((ks + 1) & 1);
    __syncthreads();
  }

  if (!DEBUG) {
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const int64_t m = m0 + 16 * t + fr;
      if (m >= M) continue;
#pragma unroll
      for (int i = 0; i < NT; ++i) {
        const int64_t n = n0 + wave * WN + 16 * i + 4 * fg;
        const floatx4 v = acc[i][t] * w_scale;
        if ((N & 3) == 0 && n + 3 < N) {
          *reinterpret_cast<floatx4*>(y + m * N + n) = v;
        } else {
#pragma unroll
          for (int rr = 0; rr < 4; ++rr)
            if (n + rr < N) y[m * N + n + rr] = v[rr];
        }
      }
    }
  }
}

namespace {
template <int BM, int BN, bool DEBUG>
hipError_t launch_tile(const uint8_t* w, float w_scale, const int8_t* q, const uint16_t* d16,
                       int64_t M, int64_t N, int64_t K, float* y, int32_t* isums,
                       hipStream_t stream) {
  dim3 grid((unsigned)((N + BN - 1) / BN), (unsigned)((M + BM - 1) / BM));
  hipLaunchKernelGGL((gemm_nvfp4_tile_kernel<BM, BN, DEBUG>), grid, dim3(256), 0, stream, w, N, (int)K,
                     q, d16, M, w_scale, y, isums);
  return hipGetLastError();
}
}  // namespace

// ---------------------------------------------------------------------------------
// Two-term kernel (M > 16): exact two-term split of the scaled activations.
//
// The per-32 activation scale d is folded into the activation operand instead of
// being applied to partial products on the vector unit: d * q has at most 18
// significant bits (11 of the binary16 d, 7 of |q| <= 127), so it is the exact sum
// of two binary16 values, hi = fp16(d * q) (one v_pk_mul_f16, round to nearest)
// and lo = fma(d, q, -hi) (one v_pk_fma_f16; the exact difference is representable,
// so the fused result is exact).  Then y = S * (W16 . hi + W16 . lo) with the
// matrix core accumulating across the whole row: twice the MFMA work of a single
// pass, but no per-block vector FMA and no partial-product registers.  hi stays
// finite while |d * q| < 65520; a 32-value block whose d is 512 or more (where
// |d * q| can pass that) is left out of the main pass (d -> 0) and done by a second
// pass, taken only by blocks that met such a d, with d / 256 into the same
// accumulators scaled by 2^-8 before and 2^8 after (both exact): every finite
// activation is handled exactly, and the main pass carries no extra MFMA work.
//
// Block: 512 threads, WN x WM wavefronts, each a (32 TN) x (32 TM) tile of
// v_mfma_f32_32x32x16_f16 products; the block tile is 256 weight rows by
// BM = 32 WM TM tokens (64 for 16 < M <= 64, 128 up to M = 128, 256 above).  LDS holds two 64-k
// stages (double buffered): weights expanded to fp16 (E2M1 * UE4M3, exact), raw
// int8 activation codes and their binary16 scales.  Each wavefront splits its own
// activation fragments into (hi, lo) in registers.  Fragments of the next 32-k
// substep are read while the MFMAs of the current one issue; global loads run two
// stages ahead; staging of stage t+1 overlaps the MFMAs of stage t.
//
// Work items: full tiles, then -- for the tiles of an incomplete last round over
// the 256 compute units -- K-split parts whose fp32 partial tiles go to the
// workspace and are summed in part order by ksplit_reduce_kernel (ksplit.h;
// deterministic: no atomics).
//
// DEBUG instance (the integer per-16 sums of this kernel's data path): the same
// staging, fp16 weight expansion, activation split and MFMAs with unit scales
// (UE4M3 = 1, d = 1, so hi = q and lo = 0); each 16-k half of a 32-k substep is one
// subblock, so two MFMAs (hi, lo) with a zero accumulator give 32 x 32 per-subblock
// sums sum E2M1 * q, exact in fp32 (|2 sum| <= 24384), written as L = 2 E2M1 sums.
// Each work item (K-split parts included) writes the subblocks of its own k range.
// ---------------------------------------------------------------------------------
namespace {
constexpr int kBigThreads = 512;
constexpr int kBigLRW = 72;   // halves per LDS weight row (64 k + 8 pad)
constexpr int kBigLRA = 72;   // bytes per LDS activation row (64 codes + 8 pad: 18 dwords, so the
                              // 8-byte fragment reads of 16 consecutive rows hit distinct banks)

template <int WN_, int WM_, int TN_, int TM_>
struct NvCfg {
  static constexpr int WN = WN_, WM = WM_, TN = TN_, TM = TM_;
  static constexpr int BN = 32 * WN * TN, BM = 32 * WM * TM;
  static constexpr int kAcc = 16 * TN * TM;  // fp32 accumulators per thread
  static constexpr int kStageW = BN * kBigLRW * 2, kStageA = BM * kBigLRA, kStageD = BM * 4;
  static constexpr int kStage = kStageW + kStageA + kStageD;
  static constexpr int kLds = 2 * kStage;
  static constexpr int ABT = BM * 64 / kBigThreads;  // activation bytes staged per thread
  static constexpr int APR = 64 / ABT;               // threads per activation row
  static_assert(WN * WM * 64 == kBigThreads, "8 wavefronts");
  static_assert(BN == 256, "weight staging: 32 codes (one packed lane slot) per thread and stage");
  static_assert(ABT == 8 || ABT == 16 || ABT == 32, "activation staging width");
  static_assert(kLds <= 160 * 1024, "LDS");
};
using NvBig = NvCfg<1, 8, 8, 1>;  // 256 weight rows x 256 tokens: each wavefront all 256 rows x 32
                                  // tokens, so every token's activation split is done once
                                  // per block (2 x 4 wavefronts of 128 x 64: 3 % slower)
using NvM128 = NvCfg<2, 4, 4, 1>; // 256 weight rows x 128 tokens (4 x 2 wavefronts of 64 x 64: 2-6 % slower)
using NvMid = NvCfg<4, 2, 2, 1>;  // 256 weight rows x 64 tokens

// which kernel runs an NVFP4 GEMM of M tokens: M = 1 only for rows too long for the
// decode kernels' activation table; the batched kernel indexes activations in 32 bits
enum NvPath { kNvTiled, kNvBatched, kNvMid, kNvM128, kNvBig };
NvPath nv_path(int64_t M, int64_t K) {
  if (M == 1) return kNvTiled;
  if (M <= 16 && M * K < (int64_t(1) << 32)) return kNvBatched;
  if (M <= 64) return kNvMid;
  return M <= 128 ? kNvM128 : kNvBig;
}

}  // namespace

size_t gemm_nvfp4_workspace(int64_t M, int64_t N, int64_t K) {
  switch (nv_path(M, K)) {
    case kNvMid: return ksplit_workspace<NvMid>(M, N, K);
    case kNvM128: return ksplit_workspace<NvM128>(M, N, K);
    case kNvBig: return ksplit_workspace<NvBig>(M, N, K);
    default: return 0;
  }
}

template <class C, bool DEBUG>
__global__ __launch_bounds__(512, 1) void gemm_nvfp4_kernel(const uint8_t* __restrict__ w, int64_t N,
                                                            int K, const int8_t* __restrict__ q,
                                                            const uint16_t* __restrict__ d16, int64_t M,
                                                            float w_scale, float* __restrict__ y,
                                                            float* __restrict__ part_ws,
                                                            int32_t* __restrict__ isums, KSplitPlan plan) {
  constexpr int BN = C::BN, BM = C::BM, WM = C::WM, TN = C::TN, TM = C::TM;
  constexpr int LRW = kBigLRW, LRA = kBigLRA, ABT = C::ABT, APR = C::APR;
  extern __shared__ __align__(16) uint8_t smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = wave / WM, wm = wave % WM;
  // work item -> tile and stage range
  const int64_t item = blockIdx.x;
  int64_t tile, part = -1;
  int t0 = 0, t1 = plan.stages;
  if (item < plan.full) {
    tile = item;
  } else {
    const int64_t it = item - plan.full;
    tile = plan.full + it / plan.split;
    part = it % plan.split;
    t0 = (int)(part * plan.stages / plan.split);
    t1 = (int)((part + 1) * plan.stages / plan.split);
  }
  const int64_t n0 = (tile % plan.tiles_n) * BN, m0 = (tile / plan.tiles_n) * BM;
  const int nch = (K + 127) >> 7;
  const int64_t ntiles = (N + 15) >> 4;
  const uint8_t* __restrict__ sc = w + ntiles * nch * 1024;
  const int nb32 = K >> 5;

  // staging task of this thread: 32 weight codes (one 16 B lane slot) of row wrow and
  // k-quarter (2 (t & 1) + whh) of chunk t >> 1; ABT activation codes of row arow; for
  // tid < 2 BM one activation scale.  Rows beyond N / M are clamped to valid memory:
  // their results are never stored.
  const int wrow = tid >> 1, whh = tid & 1;
  const int64_t wtile = min(n0 / 16 + (wrow >> 4), ntiles - 1);
  const uint8_t* __restrict__ wbase = w + wtile * nch * 1024 + 16 * (wrow & 15);
  const uint8_t* __restrict__ sbase = sc + wtile * nch * 128 + 2 * (wrow & 15);
  const int arow = tid / APR, aoff = ABT * (tid % APR);
  const int8_t* __restrict__ abase = q + min(m0 + arow, M - 1) * K + aoff;
  const bool dtask = 2 * BM >= kBigThreads || tid < 2 * BM;
  const int drow = tid % BM, dblk = (tid / BM) & 1;
  const uint16_t* __restrict__ dbase = DEBUG ? nullptr : d16 + min(m0 + drow, M - 1) * nb32 + dblk;
  bool anybig = false;  // this thread staged an activation scale d >= 512
  struct Stage { Words<ABT / 4> a; u32x4 wr; uint32_t sr, dr; };
  auto gload = [&](int t, Stage& x) {
    const int c = t >> 1, g = 2 * (t & 1) + whh;
    x.wr = *reinterpret_cast<const u32x4*>(wbase + (int64_t)c * 1024 + 256 * g);
    x.sr = *reinterpret_cast<const uint16_t*>(sbase + (int64_t)c * 128 + 32 * g);
    x.a = load_words<ABT / 4>(abase + 64 * t);
    if constexpr (DEBUG) x.dr = 0x3C00u;  // d = 1
    else x.dr = dtask ? dbase[2 * t] : 0u;
  };
  // pass 0: the main pass (blocks with d >= 512 get d = 0); pass 1: those blocks only,
  // with d / 256
  auto lstore = [&](int b, const Stage& x, int pass) {
    uint8_t* st = smem + b * C::kStage;
    _Float16* lw = reinterpret_cast<_Float16*>(st);
    uint8_t* la = st + C::kStageW;
    uint16_t* ld = reinterpret_cast<uint16_t*>(st + C::kStageW + C::kStageA);
    const _Float16 u0 = DEBUG ? (_Float16)1.0f : (_Float16)ue4m3_to_f32<0>(x.sr);
    const _Float16 u1 = DEBUG ? (_Float16)1.0f : (_Float16)ue4m3_to_f32<1>(x.sr);
    const half2_t s0 = {u0, u0}, s1 = {u1, u1};
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const half2_t s = d < 2 ? s0 : s1;
      const uint32_t cw = x.wr[d];
      const half2_t p0 = e2m1x2_to_f16<0>(cw) * s;
      const half2_t p1 = e2m1x2_to_f16<1>(cw) * s;
      const half2_t p2 = e2m1x2_to_f16<2>(cw) * s;
      const half2_t p3 = e2m1x2_to_f16<3>(cw) * s;
      const half8_t v = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
      *reinterpret_cast<half8_t*>(lw + wrow * LRW + 32 * whh + 8 * d) = v;
    }
    store_words<ABT / 4>(la + arow * LRA + aoff, x.a);
    if (dtask) {
      uint32_t dr = x.dr;
      if constexpr (!DEBUG) {
        anybig |= act_scale_big(dr);
        dr = act_scale_for_pass(dr, pass);
      }
      ld[2 * drow + dblk] = (uint16_t)dr;
    }
  };

  floatx16 acc[TN][TM];
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j) acc[i][j] = floatx16{};
  const int fr = lane & 31, fk = 8 * (lane >> 5);
  // fragments of one 32-k substep u of a stage: weights for both 16-k halves, raw
  // activation codes, activation scales
  struct Frag { half8_t af[2][TN]; uint2 raw[2][TM]; uint32_t dd[TM]; };
  auto fread = [&](int b, int u, Frag& f) {
    const uint8_t* st = smem + b * C::kStage;
    const _Float16* lw = reinterpret_cast<const _Float16*>(st);
    const uint8_t* la = st + C::kStageW;
    const uint16_t* ld = reinterpret_cast<const uint16_t*>(st + C::kStageW + C::kStageA);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < TN; ++i)
        f.af[h][i] = *reinterpret_cast<const half8_t*>(lw + (wn * (32 * TN) + 32 * i + fr) * LRW + 32 * u + 16 * h + fk);
#pragma unroll
    for (int j = 0; j < TM; ++j) {
      const int r = wm * (32 * TM) + 32 * j + fr;
      f.dd[j] = ld[2 * r + u];
#pragma unroll
      for (int h = 0; h < 2; ++h) f.raw[h][j] = *reinterpret_cast<const uint2*>(la + r * LRA + 32 * u + 16 * h + fk);
    }
  };
  // the MFMAs of substep u of stage t (t, u only locate the subblocks of the DEBUG sums)
  auto mfmas = [&](const Frag& f, int t, int u) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      half8_t bh[TM], bl[TM];
#pragma unroll
      for (int j = 0; j < TM; ++j) {
        const _Float16 dh = __builtin_bit_cast(_Float16, (uint16_t)f.dd[j]);
        const half2_t d2 = {dh, dh};
        half2_t a0, a1, c0, c1;
        i8x4_to_f16x4(f.raw[h][j].x, a0, a1);
        i8x4_to_f16x4(f.raw[h][j].y, c0, c1);
        const half2_t h0 = a0 * d2, h1 = a1 * d2, h2 = c0 * d2, h3 = c1 * d2;
        const half2_t l0 = __builtin_elementwise_fma(a0, d2, -h0);
        const half2_t l1 = __builtin_elementwise_fma(a1, d2, -h1);
        const half2_t l2 = __builtin_elementwise_fma(c0, d2, -h2);
        const half2_t l3 = __builtin_elementwise_fma(c1, d2, -h3);
        bh[j] = half8_t{h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
        bl[j] = half8_t{l0[0], l0[1], l1[0], l1[1], l2[0], l2[1], l3[0], l3[1]};
      }
      if constexpr (DEBUG) {
        // subblock 4 t + 2 u + h: its sums for 32 weight rows x 32 tokens per (i, j)
        const int64_t sb = 4 * (int64_t)t + 2 * u + h, nsb = K >> 4;
#pragma unroll
        for (int i = 0; i < TN; ++i)
#pragma unroll
          for (int j = 0; j < TM; ++j) {
            floatx16 p = __builtin_amdgcn_mfma_f32_32x32x16_f16(f.af[h][i], bh[j], floatx16{}, 0, 0, 0);
            p = __builtin_amdgcn_mfma_f32_32x32x16_f16(f.af[h][i], bl[j], p, 0, 0, 0);
            const int64_t m = m0 + wm * (32 * TM) + 32 * j + fr;
            if (m >= M) continue;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              const int64_t n = n0 + wn * (32 * TN) + 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
              if (n < N) isums[(m * N + n) * nsb + sb] = (int32_t)(2.0f * p[e]);
            }
          }
      } else {
#pragma unroll
        for (int i = 0; i < TN; ++i)
#pragma unroll
          for (int j = 0; j < TM; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(f.af[h][i], bh[j], acc[i][j], 0, 0, 0);
#pragma unroll
        for (int i = 0; i < TN; ++i)
#pragma unroll
          for (int j = 0; j < TM; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(f.af[h][i], bl[j], acc[i][j], 0, 0, 0);
      }
    }
  };

  // pipeline over stages t0 .. t1-1 (every global load index is clamped to the range,
  // so no load is conditional and the in-order load counter stays exact).  The loop
  // body has no branch: after the last stage the staging writes a clamped copy to the
  // free buffer and the fragment read takes it, both unused; one basic block lets the
  // scheduler spread the staging and the fragment reads between the MFMAs.
  Stage x;
  gload(t0, x);
  lstore(0, x, 0);
  gload(min(t0 + 1, t1 - 1), x);
  __syncthreads();
  Frag f0, f1;
  fread(0, 0, f0);
  for (int t = t0; t < t1; ++t) {
    const int b = (t - t0) & 1;
    fread(b, 1, f1);
    lstore(b ^ 1, x, 0);               // stage t+1, loaded one stage ago
    mfmas(f0, t, 0);
    gload(min(t + 2, t1 - 1), x);
    __syncthreads();                   // stage t+1 visible; stage t-1's buffer free
    fread(b ^ 1, 0, f0);
    mfmas(f1, t, 1);
  }
  if constexpr (DEBUG) return;

  // second pass over the stages for blocks with d >= 512 (activations near the
  // binary16 range; not taken otherwise): plain staging through buffer 0, into the
  // accumulators scaled by 2^-8 (exact) and restored by 2^8 afterwards
  if (__syncthreads_or(anybig)) {
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
      for (int j = 0; j < TM; ++j) acc[i][j] *= 0.00390625f;
    for (int t = t0; t < t1; ++t) {
      gload(t, x);
      __syncthreads();                 // every read of buffer 0 done
      lstore(0, x, 1);
      __syncthreads();
      fread(0, 0, f0);
      mfmas(f0, t, 0);
      fread(0, 1, f1);
      mfmas(f1, t, 1);
    }
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
      for (int j = 0; j < TM; ++j) acc[i][j] *= 256.0f;
  }

  if (part >= 0) {
    // partial tile: thread-private accumulators to the workspace, element-major
    float* dst = part_ws + ((item - plan.full) * C::kAcc) * kBigThreads + tid;
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
      for (int j = 0; j < TM; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) dst[((i * TM + j) * 16 + e) * kBigThreads] = acc[i][j][e];
    return;
  }
#pragma unroll
  for (int j = 0; j < TM; ++j) {
    const int64_t m = m0 + wm * (32 * TM) + 32 * j + fr;
    if (m >= M) continue;
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int64_t n = n0 + wn * (32 * TN) + 32 * i + 8 * e4 + 4 * (lane >> 5);
        const floatx4 v = {acc[i][j][4 * e4] * w_scale, acc[i][j][4 * e4 + 1] * w_scale,
                           acc[i][j][4 * e4 + 2] * w_scale, acc[i][j][4 * e4 + 3] * w_scale};
        if ((N & 3) == 0 && n + 3 < N) {
          *reinterpret_cast<floatx4*>(y + m * N + n) = v;
        } else {
#pragma unroll
          for (int rr = 0; rr < 4; ++rr)
            if (n + rr < N) y[m * N + n + rr] = v[rr];
        }
      }
  }
}

namespace {
// isums != nullptr: the DEBUG instance (per-16 sums, no workspace, no reduction)
template <class C>
hipError_t launch_two_term(const uint8_t* w, float w_scale, const int8_t* q, const uint16_t* d16, int64_t M,
                           int64_t N, int64_t K, float* y, int32_t* isums, float* workspace, hipStream_t stream) {
  const KSplitPlan plan = ksplit_plan<C::BN, C::BM>(M, N, K);
  const int64_t items = plan.full + plan.split_tiles * plan.split;
  if (isums) {
    hipError_t ea = hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_nvfp4_kernel<C, true>),
                                        hipFuncAttributeMaxDynamicSharedMemorySize, C::kLds);
    if (ea != hipSuccess) return ea;
    hipLaunchKernelGGL((gemm_nvfp4_kernel<C, true>), dim3((unsigned)items), dim3(kBigThreads), C::kLds, stream, w,
                       N, (int)K, q, d16, M, 1.0f, y, nullptr, isums, plan);
    return hipGetLastError();
  }
  if (plan.split_tiles && !workspace) return hipErrorInvalidValue;  // callers size it first
  hipError_t ea = hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_nvfp4_kernel<C, false>),
                                      hipFuncAttributeMaxDynamicSharedMemorySize, C::kLds);
  if (ea != hipSuccess) return ea;
  hipLaunchKernelGGL((gemm_nvfp4_kernel<C, false>), dim3((unsigned)items), dim3(kBigThreads), C::kLds, stream, w,
                     N, (int)K, q, d16, M, w_scale, y, workspace, nullptr, plan);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || plan.split_tiles == 0) return e;
  return launch_ksplit_reduce<C>(workspace, N, M, w_scale, y, plan, stream);
}
}  // namespace

hipError_t launch_gemm_nvfp4(const uint8_t* w, float w_scale, const int8_t* q,
                             const uint16_t* d16, int64_t M, int64_t N, int64_t K, float* y,
                             int32_t* isums, float* workspace, hipStream_t stream) {
  switch (nv_path(M, K)) {
    case kNvBatched: return launch_gemv_nvfp4_batch_f16(w, w_scale, q, d16, M, N, K, y, isums, stream);
    case kNvMid: return launch_two_term<NvMid>(w, w_scale, q, d16, M, N, K, y, isums, workspace, stream);
    case kNvM128: return launch_two_term<NvM128>(w, w_scale, q, d16, M, N, K, y, isums, workspace, stream);
    case kNvBig: return launch_two_term<NvBig>(w, w_scale, q, d16, M, N, K, y, isums, workspace, stream);
    default:
      if (isums) return launch_tile<16, 64, true>(w, w_scale, q, d16, M, N, K, y, isums, stream);
      return launch_tile<16, 128, false>(w, w_scale, q, d16, M, N, K, y, isums, stream);
  }
}

// ---------------------------------------------------------------------------------
// Static scratch for callers that cannot allocate (nvq_gemm_nvfp4_noalloc): the
// K-split partial tiles go to this file-scope device array instead of a workspace
// argument.  Every GPU the library runs on holds its own copy until the process ends.
// No shape needs more: at most 256 K-split work items (one round over the compute
// units), each one 512-thread partial tile of at most 128 float accumulators per
// thread.  Its contents need no clearing: every part writes its whole partial tile
// before the reduction reads it.  Calls that overlap in time on one GPU share it and
// race.  In host code `scratch` only names the host-side stand-in of the symbol;
// its device address on each GPU comes from hipGetSymbolAddress, taken once per
// device on that device's first call and kept in g_scratch_dev.
// ---------------------------------------------------------------------------------
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
static_assert(kNoAllocScratchBytes == (size_t)kKSplitSlots * kKSplitThreads * 128 * sizeof(float),
              "largest K-split plan: 256 items x 512 threads x 128 accumulators");
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_dev[64];  // device address of `scratch` per device index
}  // namespace

size_t gemm_nvfp4_noalloc_scratch_bytes() { return kNoAllocScratchBytes; }

hipError_t launch_gemm_nvfp4_noalloc(const uint8_t* w, float w_scale, const int8_t* q, const uint16_t* d16,
                                     int64_t M, int64_t N, int64_t K, float* y, hipStream_t stream) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  void* ptr = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_dev[dev] == nullptr) {
      void* p = nullptr;
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      g_scratch_dev[dev] = p;
    }
    ptr = g_scratch_dev[dev];
  }
  if (gemm_nvfp4_workspace(M, N, K) > kNoAllocScratchBytes) return hipErrorInvalidValue;  // callers check first
  return launch_gemm_nvfp4(w, w_scale, q, d16, M, N, K, y, nullptr, static_cast<float*>(ptr), stream);
}

}  // namespace nvq
