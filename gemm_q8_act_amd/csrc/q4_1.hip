// q4_1.hip -- Q4_1 weights x Q8_0 activations on gfx950 (GEMV and tiled MFMA).
//
// Q4_1 ("HANDOFF: flint CPU optimization (Q4_1 + NVFP4)", section 1: the same work
// carries Q4_1 vec_dot and tiled kernels): per 32 weights an fp16 scale d and
// offset m, 4-bit codes c in 0..15, weight = d*c + m.  With Q8_0 activations
// (da, q) over the same 32-block:
//     sum_k w*a = da * (d * sum_k c*q + m * sum_k q),
// the second sum being the block's activation code sum (two bsum16 values).
//
// GEMV (M == 1): same lane mapping as the NVFP4 GEMV -- a unit is one 32-weight
// block (16 B of codes + one 4-byte (d, m) pair), the codes are unsigned nibbles
// used directly as int8 by v_dot4_i32_i8.
//
// GEMM: like the NVFP4 tiled kernel with a 32-k stage; codes become exact
// integer-valued fp16, P = sum c*q over the block is an exact fp32 integer
// (|P| <= 32*15*127 = 60960), and per element acc += da*(d*P + m*bsum32).
#include "nvq_device.h"
#include "nvq_launch.h"

namespace nvq {

constexpr int kQ41MaxUPL = 10;
__host__ __device__ constexpr int q41_rg(int upl) { return upl >= 7 ? 1 : (upl >= 4 ? 2 : 4); }

// 8 unsigned 4-bit codes (byte i: code 2i low nibble, 2i+1 high) dotted with the
// matching even / odd activation codes.
__device__ __forceinline__ int dot8_u4(uint32_t c, uint32_t qe, uint32_t qo, int acc) {
  acc = dot4(c & 0x0F0F0F0Fu, qe, acc);
  acc = dot4((c >> 4) & 0x0F0F0F0Fu, qo, acc);
  return acc;
}

template <int LPR, int UPL, bool DEBUG>
__global__ __launch_bounds__(256) void gemv_q4_1_m1_kernel(const uint8_t* __restrict__ w,
                                                           int64_t N, int K,
                                                           const int8_t* __restrict__ q,
                                                           const uint16_t* __restrict__ d16,
                                                           const int16_t* __restrict__ bsum16,
                                                           float* __restrict__ y,
                                                           int32_t* __restrict__ isums) {
  constexpr int RG = q41_rg(UPL);
  constexpr int RPG = 64 / LPR;
  constexpr int RPW = RPG * RG;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int sub = lane % LPR;
  const int slot = lane / LPR;
  const int units = K >> 5;
  const int64_t crow = K >> 1;
  const int64_t nb = K >> 5;
  const uint32_t* __restrict__ dm = reinterpret_cast<const uint32_t*>(w + N * crow);
  const int64_t row0 = ((int64_t)blockIdx.x * 4 + wave) * RPW;

  uint4 cw[RG][UPL];
  uint32_t pw[RG][UPL];
#pragma unroll
  for (int r = 0; r < RG; ++r) {
    const int64_t row = row0 + r * RPG + slot;
#pragma unroll
    for (int j = 0; j < UPL; ++j) {
      const int u = sub + LPR * j;
      if (row < N && u < units) {
        cw[r][j] = *reinterpret_cast<const uint4*>(w + row * crow + 16 * (int64_t)u);
        pw[r][j] = dm[row * nb + u];
      } else {
        cw[r][j] = make_uint4(0u, 0u, 0u, 0u);
        pw[r][j] = 0u;
      }
    }
  }

  uint32_t qe[UPL][4], qo[UPL][4];
  float da[UPL], bs[UPL];
#pragma unroll
  for (int j = 0; j < UPL; ++j) {
    const int u = sub + LPR * j;
    if (u < units) {
      const uint4 a = *reinterpret_cast<const uint4*>(q + 32 * (int64_t)u);
      const uint4 b = *reinterpret_cast<const uint4*>(q + 32 * (int64_t)u + 16);
      split_even_odd(a.x, a.y, qe[j][0], qo[j][0]);
      split_even_odd(a.z, a.w, qe[j][1], qo[j][1]);
      split_even_odd(b.x, b.y, qe[j][2], qo[j][2]);
      split_even_odd(b.z, b.w, qe[j][3], qo[j][3]);
      if (!DEBUG) {
        da[j] = f16_bits_to_f32(d16[u]);
        bs[j] = (float)((int)bsum16[2 * u] + (int)bsum16[2 * u + 1]);
      } else {
        da[j] = bs[j] = 0.0f;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) qe[j][i] = qo[j][i] = 0u;
      da[j] = bs[j] = 0.0f;
    }
  }

#pragma unroll
  for (int r = 0; r < RG; ++r) {
    const int64_t row = row0 + r * RPG + slot;
    float acc = 0.0f;
#pragma unroll
    for (int j = 0; j < UPL; ++j) {
      const int i0 = dot8_u4(cw[r][j].y, qe[j][1], qo[j][1], dot8_u4(cw[r][j].x, qe[j][0], qo[j][0], 0));
      const int i1 = dot8_u4(cw[r][j].w, qe[j][3], qo[j][3], dot8_u4(cw[r][j].z, qe[j][2], qo[j][2], 0));
      if (DEBUG) {
        const int u = sub + LPR * j;
        if (row < N && u < units) {
          isums[row * (K >> 4) + 2 * u] = i0;
          isums[row * (K >> 4) + 2 * u + 1] = i1;
        }
      } else {
        const float dw = f16_bits_to_f32((uint16_t)(pw[r][j] & 0xFFFFu));
        const float mw = f16_bits_to_f32((uint16_t)(pw[r][j] >> 16));
        acc = fmaf(da[j], fmaf(dw, (float)(i0 + i1), mw * bs[j]), acc);
      }
    }
    if (!DEBUG) {
      acc = group_sum<LPR>(acc);
      if (sub == 0 && row < N) y[row] = acc;
    }
  }
}

template <int BM, int BN, bool DEBUG>
__global__ __launch_bounds__(256) void gemm_q4_1_kernel(const uint8_t* __restrict__ w, int64_t N,
                                                        int K, const int8_t* __restrict__ q,
                                                        const uint16_t* __restrict__ d16,
                                                        const int16_t* __restrict__ bsum16,
                                                        int64_t M, float* __restrict__ y,
                                                        int32_t* __restrict__ isums) {
  constexpr int BK = 32;
  constexpr int WN = BN / 4;
  constexpr int NT = WN / 16;
  constexpr int MT = BM / 16;
  constexpr int LDH = BK + 8;               // 80 B rows: 16-byte fragment reads stay conflict free
  constexpr int WT = (BN + 255) / 256;      // one 32-weight task per row
  constexpr int AT = (BM * 2 + 255) / 256;  // two 16-code tasks per token
  __shared__ __align__(16) _Float16 lw[2][BN * LDH];
  __shared__ __align__(16) _Float16 la[2][BM * LDH];
  __shared__ __align__(16) float ldm[2][BN * 2];   // (d, m) per weight row
  __shared__ __align__(16) float lab[2][BM * 2];   // (da, bsum32) per token

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t n0 = (int64_t)blockIdx.x * BN, m0 = (int64_t)blockIdx.y * BM;
  const int64_t crow = K >> 1, nb = K >> 5, ns = K >> 4;
  const int nks = K / BK;
  const uint32_t* __restrict__ dm = reinterpret_cast<const uint32_t*>(w + N * crow);

  uint4 wreg[WT];
  uint32_t preg[WT];
  uint4 areg[AT];
  float av0 = 0.f, av1 = 0.f;

  auto gload = [&](int ks) {
#pragma unroll
    for (int i = 0; i < WT; ++i) {
      const int r = tid + 256 * i;
      const int64_t row = n0 + r;
      if (r < BN && row < N) {
        wreg[i] = *reinterpret_cast<const uint4*>(w + row * crow + (int64_t)ks * 16);
        preg[i] = dm[row * nb + ks];
      } else {
        wreg[i] = make_uint4(0u, 0u, 0u, 0u);
        preg[i] = 0u;
      }
    }
#pragma unroll
    for (int i = 0; i < AT; ++i) {
      const int task = tid + 256 * i;
      const int r = task >> 1, p = task & 1;
      const int64_t m = m0 + r;
      if (task < BM * 2 && m < M)
        areg[i] = *reinterpret_cast<const uint4*>(q + m * K + (int64_t)ks * 32 + 16 * p);
      else
        areg[i] = make_uint4(0u, 0u, 0u, 0u);
    }
    if (!DEBUG && tid < BM) {
      const int64_t m = m0 + tid;
      if (m < M) {
        av0 = f16_bits_to_f32(d16[m * nb + ks]);
        av1 = (float)((int)bsum16[m * ns + 2 * ks] + (int)bsum16[m * ns + 2 * ks + 1]);
      } else {
        av0 = av1 = 0.f;
      }
    }
  };

  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < WT; ++i) {
      const int r = tid + 256 * i;
      if (r < BN) {
        const uint32_t c[4] = {wreg[i].x, wreg[i].y, wreg[i].z, wreg[i].w};
        _Float16* dst = &lw[buf][r * LDH];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          // code byte j -> (low nibble, high nibble) as exact integer fp16 via 1024 + c
          half8_t v;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t b = (c[d] >> (8 * j)) & 0xFFu;
            const uint32_t bits = 0x64006400u | (b & 0xFu) | ((b & 0xF0u) << 12);
            const half2_t h = __builtin_bit_cast(half2_t, bits) - half2_t{(_Float16)1024.0f, (_Float16)1024.0f};
            v[2 * j] = h[0];
            v[2 * j + 1] = h[1];
          }
          *reinterpret_cast<half8_t*>(dst + 8 * d) = v;
        }
        if (!DEBUG) {
          ldm[buf][2 * r] = f16_bits_to_f32((uint16_t)(preg[i] & 0xFFFFu));
          ldm[buf][2 * r + 1] = f16_bits_to_f32((uint16_t)(preg[i] >> 16));
        }
      }
    }
#pragma unroll
    for (int i = 0; i < AT; ++i) {
      const int task = tid + 256 * i;
      if (task < BM * 2) {
        const int r = task >> 1, p = task & 1;
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
    if (!DEBUG && tid < BM) {
      lab[buf][2 * tid] = av0;
      lab[buf][2 * tid + 1] = av1;
    }
  };

  floatx4 acc[NT][MT];
#pragma unroll
  for (int i = 0; i < NT; ++i)
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[i][t] = floatx4{0.f, 0.f, 0.f, 0.f};
  const int fr = lane & 15, fg = lane >> 4;
  const floatx4 zero4 = {0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int buf, int ks) {
    half8_t a[NT], b[MT];
#pragma unroll
    for (int i = 0; i < NT; ++i)
      a[i] = *reinterpret_cast<const half8_t*>(&lw[buf][(wave * WN + 16 * i + fr) * LDH + 8 * fg]);
#pragma unroll
    for (int t = 0; t < MT; ++t)
      b[t] = *reinterpret_cast<const half8_t*>(&la[buf][(16 * t + fr) * LDH + 8 * fg]);
    if (!DEBUG) {
      float dav[MT], bsv[MT];
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        dav[t] = lab[buf][2 * (16 * t + fr)];
        bsv[t] = lab[buf][2 * (16 * t + fr) + 1];
      }
#pragma unroll
      for (int i = 0; i < NT; ++i) {
        const int rb = wave * WN + 16 * i + 4 * fg;
        const floatx4 dw = {ldm[buf][2 * rb], ldm[buf][2 * rb + 2], ldm[buf][2 * rb + 4], ldm[buf][2 * rb + 6]};
        const floatx4 mw = {ldm[buf][2 * rb + 1], ldm[buf][2 * rb + 3], ldm[buf][2 * rb + 5], ldm[buf][2 * rb + 7]};
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          const floatx4 p = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[i], b[t], zero4, 0, 0, 0);
#pragma unroll
          for (int rr = 0; rr < 4; ++rr)
            acc[i][t][rr] = fmaf(dav[t], fmaf(dw[rr], p[rr], mw[rr] * bsv[t]), acc[i][t][rr]);
        }
      }
    } else {
      const half8_t z8 = {};
#pragma unroll
      for (int i = 0; i < NT; ++i)
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
          for (int hsub = 0; hsub < 2; ++hsub) {
            const half8_t bb = ((fg >> 1) == hsub) ? b[t] : z8;
            const floatx4 p = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[i], bb, zero4, 0, 0, 0);
            const int64_t m = m0 + 16 * t + fr;
            const int64_t s = 2 * (int64_t)ks + hsub;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
              const int64_t n = n0 + wave * WN + 16 * i + 4 * fg + rr;
              if (m < M && n < N) isums[(m * N + n) * ns + s] = (int32_t)p[rr];
            }
          }
    }
  };

  gload(0);
  lstore(0);
  __syncthreads();
  for (int ks = 0; ks < nks; ++ks) {
    const bool more = ks + 1 < nks;
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
        if ((N & 3) == 0 && n + 3 < N) {
          *reinterpret_cast<floatx4*>(y + m * N + n) = acc[i][t];
        } else {
#pragma unroll
          for (int rr = 0; rr < 4; ++rr)
            if (n + rr < N) y[m * N + n + rr] = acc[i][t][rr];
        }
      }
    }
  }
}

namespace {
typedef void (*gemv_q41_fn)(const uint8_t*, int64_t, int, const int8_t*, const uint16_t*,
                            const int16_t*, float*, int32_t*);
template <int LPR, bool DEBUG>
gemv_q41_fn pick_q41(int upl) {
  switch (upl) {
    case 1: return gemv_q4_1_m1_kernel<LPR, 1, DEBUG>;
    case 2: return gemv_q4_1_m1_kernel<LPR, 2, DEBUG>;
    case 3: return gemv_q4_1_m1_kernel<LPR, 3, DEBUG>;
    case 4: return gemv_q4_1_m1_kernel<LPR, 4, DEBUG>;
    case 5: return gemv_q4_1_m1_kernel<LPR, 5, DEBUG>;
    case 6: return gemv_q4_1_m1_kernel<LPR, 6, DEBUG>;
    case 7: return gemv_q4_1_m1_kernel<LPR, 7, DEBUG>;
    case 8: return gemv_q4_1_m1_kernel<LPR, 8, DEBUG>;
    case 9: return gemv_q4_1_m1_kernel<LPR, 9, DEBUG>;
    case 10: return gemv_q4_1_m1_kernel<LPR, 10, DEBUG>;
    default: return nullptr;
  }
}
template <int BM, int BN, bool DEBUG>
hipError_t launch_q41_tile(const uint8_t* w, const int8_t* q, const uint16_t* d16,
                           const int16_t* bsum16, int64_t M, int64_t N, int64_t K, float* y,
                           int32_t* isums, hipStream_t stream) {
  dim3 grid((unsigned)((N + BN - 1) / BN), (unsigned)((M + BM - 1) / BM));
  hipLaunchKernelGGL((gemm_q4_1_kernel<BM, BN, DEBUG>), grid, dim3(256), 0, stream, w, N, (int)K,
                     q, d16, bsum16, M, y, isums);
  return hipGetLastError();
}
}  // namespace

// Lanes-per-row and units-per-lane for a row of K weights: the LPR in {64, 32, 16}
// with the fewest idle unit slots (ties to the wider LPR), subject to UPL <= 10.
static void gemv_m1_config(int64_t K, int* lpr_out, int* upl_out) {
  const int units = (int)(K / 32);
  int best_lpr = 0, best_upl = 0;
  double best_eff = -1.0;
  const int lprs[3] = {64, 32, 16};
  for (int i = 0; i < 3; ++i) {
    const int lpr = lprs[i];
    const int upl = (units + lpr - 1) / lpr;
    if (upl > kQ41MaxUPL) continue;
    const double eff = (double)units / (double)(lpr * upl);
    if (eff > best_eff + 1e-9) {
      best_eff = eff;
      best_lpr = lpr;
      best_upl = upl;
    }
  }
  *lpr_out = best_lpr;
  *upl_out = best_upl;
}

hipError_t launch_gemv_q4_1_m1(const uint8_t* w, const int8_t* q, const uint16_t* d16,
                               const int16_t* bsum16, int64_t N, int64_t K, float* y,
                               int32_t* isums, hipStream_t stream) {
  const bool debug = isums != nullptr;
  int lpr = 0, upl = 0;
  gemv_m1_config(K, &lpr, &upl);
  if (lpr == 0) {
    // very long rows: the tiled kernel handles any K
    return launch_gemm_q4_1(w, q, d16, bsum16, 1, N, K, y, isums, stream);
  }
  gemv_q41_fn fn = nullptr;
  if (lpr == 64) fn = debug ? pick_q41<64, true>(upl) : pick_q41<64, false>(upl);
  if (lpr == 32) fn = debug ? pick_q41<32, true>(upl) : pick_q41<32, false>(upl);
  if (lpr == 16) fn = debug ? pick_q41<16, true>(upl) : pick_q41<16, false>(upl);
  if (!fn) return hipErrorInvalidValue;
  const int64_t rows_per_block = 4 * (64 / lpr) * q41_rg(upl);
  const int64_t grid = (N + rows_per_block - 1) / rows_per_block;
  hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(256), 0, stream, w, N, (int)K, q, d16, bsum16,
                     y, isums);
  return hipGetLastError();
}

hipError_t launch_gemm_q4_1(const uint8_t* w, const int8_t* q, const uint16_t* d16,
                            const int16_t* bsum16, int64_t M, int64_t N, int64_t K, float* y,
                            int32_t* isums, hipStream_t stream) {
  if (isums) return launch_q41_tile<16, 64, true>(w, q, d16, bsum16, M, N, K, y, isums, stream);
  if (M <= 16) return launch_q41_tile<16, 128, false>(w, q, d16, bsum16, M, N, K, y, isums, stream);
  return launch_q41_tile<64, 128, false>(w, q, d16, bsum16, M, N, K, y, isums, stream);
}

}  // namespace nvq
