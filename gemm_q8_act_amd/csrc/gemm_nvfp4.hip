// gemm_nvfp4.hip -- tiled MFMA product, NVFP4 weights x Q8_0 activations, gfx950.
//
// Method ("HANDOFF: flint CPU optimization (Q4_1 + NVFP4)", section 3, Code map:
// the tiled path unpacks weight and activation tiles, then runs a microkernel with
// a per-16 weight scale cached beside the unpacked tile).  On gfx950 the
// contraction runs on the matrix cores:
//
//   * Exact fp16 expansion.  w16 = E2M1(code) * UE4M3(scale) has at most 6
//     significant bits and lies in [2^-10, 2688], so it is exact in fp16; the
//     UE4M3 scale is folded into the weights once per tile.  Activation codes q
//     (|q| <= 127) are exact in fp16 too.
//   * Per 32-k chunk (one Q8_0 block) one v_mfma_f32_16x16x32_f16 with a zero
//     accumulator gives P[n][m] = sum_k w16 * q; products are exact in fp32.
//   * The chunk's activation scale d[m] differs per chunk, so it is applied on the
//     vector unit: acc[n][m] += d[m][chunk] * P[n][m]; y = S * acc at the end.
//     With weights as the MFMA A operand (rows = n) and activations as B
//     (columns = m), every lane owns a single column m, so one d value per lane
//     scales all of that lane's accumulators.
//
// Tiling: a 256-thread block computes BN weight rows x BM tokens.  Per 128-k step
// the block loads BN/16 tile-chunks of the packed layout (1 KB of codes + 128 scale
// bytes each, contiguous) and BM x 128 B of activation codes, expands both to fp16
// in LDS (double-buffered, rows padded to 272 B so 16-byte fragment reads are
// bank-conflict free), and each of the 4 wavefronts runs (BN/64) x (BM/16) MFMAs
// per 32-k block.  Global loads of step k+1 are issued before the MFMAs of step k.
#include "nvq_device.h"
#include "nvq_launch.h"

namespace nvq {

template <int BM, int BN, bool DEBUG>
__global__ __launch_bounds__(256) void gemm_nvfp4_kernel(const uint8_t* __restrict__ w,
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
  hipLaunchKernelGGL((gemm_nvfp4_kernel<BM, BN, DEBUG>), grid, dim3(256), 0, stream, w, N, (int)K,
                     q, d16, M, w_scale, y, isums);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_gemm_nvfp4(const uint8_t* w, float w_scale, const int8_t* q,
                             const uint16_t* d16, int64_t M, int64_t N, int64_t K, float* y,
                             int32_t* isums, hipStream_t stream) {
  if (isums) return launch_tile<16, 64, true>(w, w_scale, q, d16, M, N, K, y, isums, stream);
  if (M <= 16) return launch_tile<16, 128, false>(w, w_scale, q, d16, M, N, K, y, isums, stream);
  return launch_tile<64, 128, false>(w, w_scale, q, d16, M, N, K, y, isums, stream);
}

}  // namespace nvq
