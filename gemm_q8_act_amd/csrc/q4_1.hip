// q4_1.hip -- Q4_1 weights x Q8_0 activations on gfx950 (GEMV and tiled MFMA).
//
// Q4_1 ("HANDOFF: flint CPU optimization (Q4_1 + NVFP4)", section 1: the same work
// carries Q4_1 vec_dot and tiled kernels): per 32 weights an fp16 scale d and
// offset m, 4-bit codes c in 0..15, weight = d*c + m.  With Q8_0 activations
// (da, q) over the same 32-block:
//     sum_k w*a = da * (d * sum_k c*q + m * sum_k q),
// the second sum being the block's activation code sum (two bsum16 values).
//
// GEMV (M <= 16): same lane mapping as the NVFP4 GEMV -- a unit is one 32-weight
// block (16 B of codes + one 4-byte (d, m) pair), the codes are unsigned nibbles
// used directly as int8 by v_dot4_i32_i8.  A wavefront holds its rows' weights in
// registers and walks the tokens, reading each token's activations (cache-resident)
// once per row group.
//
// GEMM, tiled (K % 64 != 0, and the debug sums): like the NVFP4 tiled kernel with a
// 32-k stage; codes become exact integer-valued fp16, P = sum c*q over the block is an
// exact fp32 integer (|P| <= 32*15*127 = 60960), and per element
// acc += da*(d*P + m*bsum32).
//
// GEMM, M > 16 and K % 64 == 0: both operands as two binary16 terms, so the matrix
// core accumulates whole rows (see gemm_q4_1_f16x2_kernel below).
#include <algorithm>

#include "ksplit.h"
#include "nvq_device.h"
#include "nvq_launch.h"

namespace nvq {

constexpr int kQ41MaxUPL = 10;
__host__ __device__ constexpr int q41_rg(int upl) { return upl >= 7 ? 1 : (upl >= 4 ? 2 : 4); }
// tokens whose activations a GEMV wavefront holds at once (8 UPL registers each)
__host__ __device__ constexpr int q41_tb(int upl) { return upl <= 2 ? 4 : (upl <= 4 ? 2 : 1); }

// 8 unsigned 4-bit codes (byte i: code 2i low nibble, 2i+1 high) dotted with the
// matching even / odd activation codes.
__device__ __forceinline__ int dot8_u4(uint32_t c, uint32_t qe, uint32_t qo, int acc) {
  acc = dot4(c & 0x0F0F0F0Fu, qe, acc);
  acc = dot4((c >> 4) & 0x0F0F0F0Fu, qo, acc);
  return acc;
}

template <int LPR, int UPL, bool MULTI, bool DEBUG>
__global__ __launch_bounds__(256) void gemv_q4_1_m1_kernel(const uint8_t* __restrict__ w,
                                                           int64_t N, int K,
                                                           const int8_t* __restrict__ q,
                                                           const uint16_t* __restrict__ d16,
                                                           const int16_t* __restrict__ bsum16,
                                                           float* __restrict__ y,
                                                           int32_t* __restrict__ isums, int M) {
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

  // tokens in groups of TB: the activation loads of a group are issued together,
  // so a group costs one cache round trip; tokens past M load token M-1 and store
  // nothing
  constexpr int TB = MULTI ? q41_tb(UPL) : 1;
  if (!MULTI && !DEBUG) M = 1;  // the single-token production instance
  for (int m0 = 0; m0 < M; m0 += TB) {
    uint32_t qe[TB][UPL][4], qo[TB][UPL][4];
    float da[TB][UPL], bs[TB][UPL];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      const int64_t m = min(m0 + tb, M - 1);
      const int8_t* __restrict__ qm = q + m * K;
#pragma unroll
      for (int j = 0; j < UPL; ++j) {
        const int u = sub + LPR * j;
        if (u < units) {
          const uint4 a = *reinterpret_cast<const uint4*>(qm + 32 * (int64_t)u);
          const uint4 b = *reinterpret_cast<const uint4*>(qm + 32 * (int64_t)u + 16);
          split_even_odd(a.x, a.y, qe[tb][j][0], qo[tb][j][0]);
          split_even_odd(a.z, a.w, qe[tb][j][1], qo[tb][j][1]);
          split_even_odd(b.x, b.y, qe[tb][j][2], qo[tb][j][2]);
          split_even_odd(b.z, b.w, qe[tb][j][3], qo[tb][j][3]);
          if (!DEBUG) {
            da[tb][j] = f16_bits_to_f32(d16[m * nb + u]);
            bs[tb][j] = (float)((int)bsum16[m * 2 * nb + 2 * u] + (int)bsum16[m * 2 * nb + 2 * u + 1]);
          } else {
            da[tb][j] = bs[tb][j] = 0.0f;
          }
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) qe[tb][j][i] = qo[tb][j][i] = 0u;
          da[tb][j] = bs[tb][j] = 0.0f;
        }
      }
    }

#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      const int64_t m = m0 + tb;
      if (TB > 1 && m >= M) break;
#pragma unroll
      for (int r = 0; r < RG; ++r) {
        const int64_t row = row0 + r * RPG + slot;
        float acc = 0.0f;
#pragma unroll
        for (int j = 0; j < UPL; ++j) {
          const int i0 = dot8_u4(cw[r][j].y, qe[tb][j][1], qo[tb][j][1], dot8_u4(cw[r][j].x, qe[tb][j][0], qo[tb][j][0], 0));
          const int i1 = dot8_u4(cw[r][j].w, qe[tb][j][3], qo[tb][j][3], dot8_u4(cw[r][j].z, qe[tb][j][2], qo[tb][j][2], 0));
          if (DEBUG) {
            const int u = sub + LPR * j;
            if (row < N && u < units) {
              isums[(m * N + row) * (K >> 4) + 2 * u] = i0;
              isums[(m * N + row) * (K >> 4) + 2 * u + 1] = i1;
            }
          } else {
            const float dw = f16_bits_to_f32((uint16_t)(pw[r][j] & 0xFFFFu));
            const float mw = f16_bits_to_f32((uint16_t)(pw[r][j] >> 16));
            acc = fmaf(da[tb][j], fmaf(dw, (float)(i0 + i1), mw * bs[tb][j]), acc);
          }
        }
        if (!DEBUG) {
          acc = group_sum<LPR>(acc);
          if (sub == 0 && row < N) y[m * N + row] = acc;
        }
      }
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

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
                            const int16_t*, float*, int32_t*, int);
template <int LPR, bool MULTI, bool DEBUG>
gemv_q41_fn pick_q41(int upl) {
  switch (upl) {
    case 1: return gemv_q4_1_m1_kernel<LPR, 1, MULTI, DEBUG>;
    case 2: return gemv_q4_1_m1_kernel<LPR, 2, MULTI, DEBUG>;
    case 3: return gemv_q4_1_m1_kernel<LPR, 3, MULTI, DEBUG>;
    case 4: return gemv_q4_1_m1_kernel<LPR, 4, MULTI, DEBUG>;
    case 5: return gemv_q4_1_m1_kernel<LPR, 5, MULTI, DEBUG>;
    case 6: return gemv_q4_1_m1_kernel<LPR, 6, MULTI, DEBUG>;
    case 7: return gemv_q4_1_m1_kernel<LPR, 7, MULTI, DEBUG>;
    case 8: return gemv_q4_1_m1_kernel<LPR, 8, MULTI, DEBUG>;
    case 9: return gemv_q4_1_m1_kernel<LPR, 9, MULTI, DEBUG>;
    case 10: return gemv_q4_1_m1_kernel<LPR, 10, MULTI, DEBUG>;
    default: return nullptr;
  }
}
// one token (or the debug sums) at a time, or TB tokens per pass
template <int LPR>
gemv_q41_fn pick_q41_for(int upl, bool multi, bool debug) {
  if (debug) return pick_q41<LPR, false, true>(upl);
  return multi ? pick_q41<LPR, true, false>(upl) : pick_q41<LPR, false, false>(upl);
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
hipError_t launch_q41_tiled(const uint8_t* w, const int8_t* q, const uint16_t* d16,
                            const int16_t* bsum16, int64_t M, int64_t N, int64_t K, float* y,
                            int32_t* isums, hipStream_t stream) {
  if (isums) return launch_q41_tile<16, 64, true>(w, q, d16, bsum16, M, N, K, y, isums, stream);
  if (M <= 16) return launch_q41_tile<16, 128, false>(w, q, d16, bsum16, M, N, K, y, isums, stream);
  return launch_q41_tile<64, 128, false>(w, q, d16, bsum16, M, N, K, y, isums, stream);
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

hipError_t launch_gemv_q4_1(const uint8_t* w, const int8_t* q, const uint16_t* d16,
                            const int16_t* bsum16, int64_t M, int64_t N, int64_t K, float* y,
                            int32_t* isums, hipStream_t stream) {
  const bool debug = isums != nullptr;
  int lpr = 0, upl = 0;
  gemv_m1_config(K, &lpr, &upl);
  if (lpr == 0) {
    // very long rows: the tiled kernel handles any K
    return launch_q41_tiled(w, q, d16, bsum16, M, N, K, y, isums, stream);
  }
  gemv_q41_fn fn = nullptr;
  const bool multi = M > 1;
  if (lpr == 64) fn = pick_q41_for<64>(upl, multi, debug);
  if (lpr == 32) fn = pick_q41_for<32>(upl, multi, debug);
  if (lpr == 16) fn = pick_q41_for<16>(upl, multi, debug);
  if (!fn) return hipErrorInvalidValue;
  const int64_t rows_per_block = 4 * (64 / lpr) * q41_rg(upl);
  const int64_t grid = (N + rows_per_block - 1) / rows_per_block;
  hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(256), 0, stream, w, N, (int)K, q, d16, bsum16,
                     y, isums, (int)M);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------
// Two-term fp16 Q4_1 kernel (K % 64 == 0).  The weight w = d*c + m (binary16 d, m;
// c in 0..15) is formed in fp32 as w' = 2^s * w (one rounding) and split into
// hi = fp16(w') and lo = fp16(w' - hi).  The power of two 2^s is chosen per weight row
// (over the k range of the work item) from the bound |m| + 15|d| of its blocks so
// that |w'| < 2^15: hi never overflows and lo is a normal binary16 number unless
// |w'| < 2^-3, so hi + lo = w' to 2^-23 |w'|, or to 2^-25 absolute, i.e. 2^-39 of the
// row's largest weight.  The activation is split exactly as in the NVFP4 large-M
// kernel (d*q = hi + lo).  The matrix core then accumulates whole rows of
//     W'.A = Wh.Ah + Wh.Al + Wl.Ah (+ Wl.Al, dropped: at most 2^-22 |W.A|),
// three MFMA passes, with no per-block vector work; the offset term m * sum(a) is
// inside W, and the result is multiplied by 2^-s (exact).  Error per output: a few
// 2^-22 of sum |w*a| plus float32 accumulation, far inside the 1e-5 bound.
//
// Block: 512 threads, WN x WM wavefronts, each a (32 TN) x (32 TM) tile of
// v_mfma_f32_32x32x16_f16 products; block tile BN = 32 WN TN weight rows by
// BM = 32 WM TM tokens (256 x 64 for 16 < M <= 64, 128 x 128 up to M = 128,
// 128 x 256 above).  LDS holds two 64-k stages: the two weight planes (fp16 hi,
// lo), raw int8 activation codes and their binary16 scales; each wavefront splits its
// activation fragments in registers.  Work items and the ordered K-split reduction
// follow the NVFP4 large-M kernel.
// ---------------------------------------------------------------------------------
namespace {
constexpr int kQThreads = 512;
constexpr int kQLRW = 72;  // halves per LDS weight row (64 k + 8 pad)
constexpr int kQLRA = 72;  // bytes per LDS activation row (64 codes + 8 pad)

template <int WN_, int WM_, int TN_, int TM_>
struct Q41Cfg {
  static constexpr int WN = WN_, WM = WM_, TN = TN_, TM = TM_;
  static constexpr int BN = 32 * WN * TN, BM = 32 * WM * TM;
  static constexpr int kAcc = 16 * TN * TM;  // fp32 accumulators per thread
  static constexpr int kStageW = BN * kQLRW * 2, kStageA = BM * kQLRA, kStageD = BM * 4;
  static constexpr int kStage = 2 * kStageW + kStageA + kStageD;
  static constexpr int kLds = 2 * kStage + BN * 4;  // + 2^-s of each weight row
  static constexpr int CPT = BN * 64 / kQThreads;   // weight codes staged per thread
  static constexpr int TPR = 64 / CPT;              // threads per weight row
  static constexpr int ABT = BM * 64 / kQThreads;   // activation bytes staged per thread
  static constexpr int APR = 64 / ABT;              // threads per activation row
  static_assert(WN * WM * 64 == kQThreads, "8 wavefronts");
  static_assert(CPT == 16 || CPT == 32, "one 32-block per thread and stage");
  static_assert(ABT == 8 || ABT == 16 || ABT == 32, "activation staging width");
  static_assert(kLds <= 160 * 1024, "LDS");
};
using Q41Big = Q41Cfg<2, 4, 2, 2>;   // 128 weight rows x 256 tokens
using Q41M128 = Q41Cfg<2, 4, 2, 1>;  // 128 weight rows x 128 tokens
using Q41Mid = Q41Cfg<4, 2, 2, 1>;   // 256 weight rows x 64 tokens

// which kernel runs a Q4_1 GEMM of this shape (the GEMV kernel falls back to the
// tiled one for rows longer than 20480)
constexpr int kQ41GemvMaxM = 16;
enum Q41Path { kQ41Gemv, kQ41Tiled, kQ41Mid, kQ41M128, kQ41Big };
Q41Path q41_path(int64_t M, int64_t K) {
  if (M <= kQ41GemvMaxM) return kQ41Gemv;
  if (K % 64 != 0) return kQ41Tiled;
  if (M <= 64) return kQ41Mid;
  return M <= 128 ? kQ41M128 : kQ41Big;
}

}  // namespace

size_t gemm_q4_1_workspace(int64_t M, int64_t N, int64_t K) {
  switch (q41_path(M, K)) {
    case kQ41Mid: return ksplit_workspace<Q41Mid>(M, N, K);
    case kQ41M128: return ksplit_workspace<Q41M128>(M, N, K);
    case kQ41Big: return ksplit_workspace<Q41Big>(M, N, K);
    default: return 0;
  }
}

template <class C>
__global__ __launch_bounds__(512, 1) void gemm_q4_1_f16x2_kernel(const uint8_t* __restrict__ w, int64_t N, int K,
                                                                 const int8_t* __restrict__ q,
                                                                 const uint16_t* __restrict__ d16, int64_t M,
                                                                 float* __restrict__ y, float* __restrict__ part_ws,
                                                                 KSplitPlan plan) {
  constexpr int BN = C::BN, BM = C::BM, WM = C::WM, TN = C::TN, TM = C::TM;
  constexpr int LRW = kQLRW, LRA = kQLRA, CPT = C::CPT, TPR = C::TPR, ABT = C::ABT, APR = C::APR;
  extern __shared__ __align__(16) uint8_t smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave / WM, wm = wave % WM;
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
  const int64_t crow = K >> 1;  // code bytes per weight row
  const int nb32 = K >> 5;
  const uint32_t* __restrict__ dmw = reinterpret_cast<const uint32_t*>(w + N * crow);

  // staging task of this thread: CPT weight codes of row wrow at k-offset CPT wq of
  // the stage, all in one 32-block, with that block's (d, m); ABT activation codes of
  // row arow; for tid < 2 BM one activation scale.  Rows beyond N / M are clamped to
  // valid memory and their results never stored.
  const int wrow = tid / TPR, wq = tid % TPR;
  const int64_t wr = min(n0 + wrow, N - 1);
  const uint8_t* __restrict__ wbase = w + wr * crow + (CPT / 2) * wq;
  const uint32_t* __restrict__ dmbase = dmw + wr * nb32 + (CPT * wq) / 32;
  const int arow = tid / APR, aoff = ABT * (tid % APR);
  const int8_t* __restrict__ abase = q + min(m0 + arow, M - 1) * K + aoff;
  const bool dtask = 2 * BM >= kQThreads || tid < 2 * BM;
  const int drow = tid % BM, dblk = (tid / BM) & 1;
  const uint16_t* __restrict__ dbase = d16 + min(m0 + drow, M - 1) * nb32 + dblk;
  struct Stage { Words<ABT / 4> a; Words<CPT / 8> wc; uint32_t dm, dr; };

  // row scale 2^s: the largest bound |m| + 15|d| of this row's blocks in [t0, t1),
  // taken by the TPR threads that stage the row, placed in [2^14, 2^15).  A zero row
  // takes s = 0; a non-finite d or m gives a non-finite row anyway.
  float bmax = 0.0f;
  const uint32_t* __restrict__ dmrow = dmw + wr * nb32;
#pragma unroll 4
  for (int b = 2 * t0 + wq; b < 2 * t1; b += TPR) {
    const uint32_t v = dmrow[b];
    bmax = fmaxf(bmax, fabsf(f16_bits_to_f32((uint16_t)(v >> 16))) + 15.0f * fabsf(f16_bits_to_f32((uint16_t)(v & 0xFFFFu))));
  }
  bmax = fmaxf(bmax, __shfl_xor(bmax, 1));
  if constexpr (TPR == 4) bmax = fmaxf(bmax, __shfl_xor(bmax, 2));
  // a nonzero bound is at least 2^-24 (binary16's least magnitude), so it is a
  // normal float: bmax in [2^(E-127), 2^(E-126)) with E its biased exponent
  int rexp = 0;
  if (bmax > 0.0f && bmax <= 3.0e38f) rexp = 15 - ((int)((__float_as_uint(bmax) >> 23) & 0xFF) - 126);
  const float rscale = ldexpf(1.0f, rexp);
  if (wq == 0) reinterpret_cast<float*>(smem + 2 * C::kStage)[wrow] = ldexpf(1.0f, -rexp);

  auto gload = [&](int t, Stage& x) {
    x.wc = load_words<CPT / 8>(wbase + (int64_t)t * 32);
    x.dm = dmbase[2 * t];
    x.a = load_words<ABT / 4>(abase + 64 * t);
    x.dr = dtask ? dbase[2 * t] : 0u;
  };
  auto lstore = [&](int b, const Stage& x) {
    uint8_t* st = smem + b * C::kStage;
    _Float16* lh = reinterpret_cast<_Float16*>(st);
    _Float16* ll = reinterpret_cast<_Float16*>(st + C::kStageW);
    uint8_t* la = st + 2 * C::kStageW;
    uint16_t* ld = reinterpret_cast<uint16_t*>(st + 2 * C::kStageW + C::kStageA);
    const float dw = rscale * f16_bits_to_f32((uint16_t)(x.dm & 0xFFFFu));
    const float mw = rscale * f16_bits_to_f32((uint16_t)(x.dm >> 16));
#pragma unroll
    for (int h = 0; h < CPT / 8; ++h) {
      const uint32_t cw = x.wc.v[h];
      half8_t vh, vl;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float c = (float)((cw >> (4 * j)) & 0xFu);  // byte j/2: code 2i low nibble, 2i+1 high
        const float wf = fmaf(dw, c, mw);
        const _Float16 hi = (_Float16)wf;
        vh[j] = hi;
        vl[j] = (_Float16)(wf - (float)hi);
      }
      *reinterpret_cast<half8_t*>(lh + wrow * LRW + CPT * wq + 8 * h) = vh;
      *reinterpret_cast<half8_t*>(ll + wrow * LRW + CPT * wq + 8 * h) = vl;
    }
    store_words<ABT / 4>(la + arow * LRA + aoff, x.a);
    if (dtask) ld[2 * drow + dblk] = (uint16_t)x.dr;
  };

  floatx16 acc[TN][TM];
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j) acc[i][j] = floatx16{};
  const int fr = lane & 31, fk = 8 * (lane >> 5);
  struct Frag { half8_t ah[2][TN], al[2][TN]; uint2 raw[2][TM]; uint32_t dd[TM]; };
  auto fread = [&](int b, int u, Frag& f) {
    const uint8_t* st = smem + b * C::kStage;
    const _Float16* lh = reinterpret_cast<const _Float16*>(st);
    const _Float16* ll = reinterpret_cast<const _Float16*>(st + C::kStageW);
    const uint8_t* la = st + 2 * C::kStageW;
    const uint16_t* ld = reinterpret_cast<const uint16_t*>(st + 2 * C::kStageW + C::kStageA);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < TN; ++i) {
        const int off = (wn * (32 * TN) + 32 * i + fr) * LRW + 32 * u + 16 * h + fk;
        f.ah[h][i] = *reinterpret_cast<const half8_t*>(lh + off);
        f.al[h][i] = *reinterpret_cast<const half8_t*>(ll + off);
      }
#pragma unroll
    for (int j = 0; j < TM; ++j) {
      const int r = wm * (32 * TM) + 32 * j + fr;
      f.dd[j] = ld[2 * r + u];
#pragma unroll
      for (int h = 0; h < 2; ++h) f.raw[h][j] = *reinterpret_cast<const uint2*>(la + r * LRA + 32 * u + 16 * h + fk);
    }
  };
  auto mfmas = [&](const Frag& f) {
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
#pragma unroll
      for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(f.ah[h][i], bh[j], acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(f.ah[h][i], bl[j], acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(f.al[h][i], bh[j], acc[i][j], 0, 0, 0);
        }
    }
  };

  // pipeline over stages t0 .. t1-1; loads clamped, loop body branch-free (after the
  // last stage the staging writes a clamped copy nobody reads)
  Stage x;
  gload(t0, x);
  lstore(0, x);
  gload(min(t0 + 1, t1 - 1), x);
  __syncthreads();
  Frag f0, f1;
  fread(0, 0, f0);
  for (int t = t0; t < t1; ++t) {
    const int b = (t - t0) & 1;
    fread(b, 1, f1);
    lstore(b ^ 1, x);
    mfmas(f0);
    gload(min(t + 2, t1 - 1), x);
    __syncthreads();
    fread(b ^ 1, 0, f0);
    mfmas(f1);
  }

  // undo the row scales (the first barrier of the pipeline ordered their stores)
  const float* rinv = reinterpret_cast<const float*>(smem + 2 * C::kStage);
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {
      const floatx4 r = *reinterpret_cast<const floatx4*>(rinv + wn * (32 * TN) + 32 * i + 8 * e4 + 4 * (lane >> 5));
#pragma unroll
      for (int j = 0; j < TM; ++j)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) acc[i][j][4 * e4 + rr] *= r[rr];
    }
  if (part >= 0) {
    float* dst = part_ws + ((item - plan.full) * C::kAcc) * kQThreads + tid;
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
      for (int j = 0; j < TM; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) dst[((i * TM + j) * 16 + e) * kQThreads] = acc[i][j][e];
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
        const floatx4 v = {acc[i][j][4 * e4], acc[i][j][4 * e4 + 1], acc[i][j][4 * e4 + 2], acc[i][j][4 * e4 + 3]};
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
template <class C>
hipError_t launch_q41_f16x2(const uint8_t* w, const int8_t* q, const uint16_t* d16, int64_t M, int64_t N,
                            int64_t K, float* y, float* workspace, hipStream_t stream) {
  const KSplitPlan plan = ksplit_plan<C::BN, C::BM>(M, N, K);
  if (plan.split_tiles && !workspace) return hipErrorInvalidValue;  // callers size it first
  hipError_t ea = hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_q4_1_f16x2_kernel<C>),
                                      hipFuncAttributeMaxDynamicSharedMemorySize, C::kLds);
  if (ea != hipSuccess) return ea;
  const int64_t items = plan.full + plan.split_tiles * plan.split;
  hipLaunchKernelGGL(gemm_q4_1_f16x2_kernel<C>, dim3((unsigned)items), dim3(kQThreads), C::kLds, stream, w, N,
                     (int)K, q, d16, M, y, workspace, plan);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || plan.split_tiles == 0) return e;
  return launch_ksplit_reduce<C>(workspace, N, M, 1.0f, y, plan, stream);
}
}  // namespace

hipError_t launch_gemm_q4_1(const uint8_t* w, const int8_t* q, const uint16_t* d16,
                            const int16_t* bsum16, int64_t M, int64_t N, int64_t K, float* y,
                            int32_t* isums, float* workspace, hipStream_t stream) {
  if (isums) return launch_q41_tiled(w, q, d16, bsum16, M, N, K, y, isums, stream);
  switch (q41_path(M, K)) {
    case kQ41Gemv: return launch_gemv_q4_1(w, q, d16, bsum16, M, N, K, y, nullptr, stream);
    case kQ41Big: return launch_q41_f16x2<Q41Big>(w, q, d16, M, N, K, y, workspace, stream);
    case kQ41Mid: return launch_q41_f16x2<Q41Mid>(w, q, d16, M, N, K, y, workspace, stream);
    case kQ41M128: return launch_q41_f16x2<Q41M128>(w, q, d16, M, N, K, y, workspace, stream);
    default: return launch_q41_tiled(w, q, d16, bsum16, M, N, K, y, isums, stream);
  }
}

}  // namespace nvq
