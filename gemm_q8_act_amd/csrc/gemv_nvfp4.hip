// gemv_nvfp4.hip -- batch-1 decode GEMV, NVFP4 weights x Q8_0 activations, gfx950.
//
// Method ("HANDOFF: flint CPU optimization (Q4_1 + NVFP4)", section 3, Code map and
// bias-trick paragraph): per 16-weight subblock an exact integer sum of
// L(code) * q with L = 2 * E2M1, then one float scale per subblock,
//     y[n] = S * sum_s 0.5 * UE4M3(scale[n][s]) * d[s/2] * isum16[n][s].
// The page's x86 kernel biases codes to 0..24 because the VNNI multiply is
// unsigned x signed; v_dot4_i32_i8 is signed x signed, so the signed L is used
// directly and the bias (and the bsum16 correction) is not needed here.
//
// Mapping (HBM-bound stream of 9/16 byte per weight):
//   * a "unit" is 32 consecutive weights of a row: 16 B of codes (one 128-bit
//     load) + 2 UE4M3 bytes + one Q8_0 block of activations;
//   * LPR lanes share a row and take units sub, sub + LPR, ... so each load
//     instruction of a wavefront reads 64/LPR runs of LPR*16 contiguous bytes;
//   * every lane keeps the activation codes of its units in VGPRs (pre-split into
//     even/odd positions to match the nibble order) and reuses them for all the
//     rows it visits; RG row groups are loaded before any is reduced so that
//     RG*UPL 128-bit loads per lane are in flight;
//   * E2M1 -> int8 is two v_perm_b32 table lookups per 4 codes whose sum is L,
//     consumed by two v_dot4_i32_i8 (see nvq_device.h);
//   * per unit: 2 integer sums -> float, times UE4M3 (v_cvt_f32_fp8) and the
//     lane's 0.5*d, accumulated in float; the LPR partial sums of a row are
//     reduced across lanes and the first lane writes y.
#include "nvq_device.h"
#include "nvq_launch.h"

namespace nvq {

constexpr int kGemvMaxUPL = 10;

__host__ __device__ constexpr int gemv_rg(int upl) { return upl >= 7 ? 1 : (upl >= 4 ? 2 : 4); }

template <int LPR, int UPL, bool DEBUG>
__global__ __launch_bounds__(256) void gemv_nvfp4_m1_kernel(const uint8_t* __restrict__ w,
                                                            int64_t N, int K,
                                                            const int8_t* __restrict__ q,
                                                            const uint16_t* __restrict__ d16,
                                                            float w_scale, float* __restrict__ y,
                                                            int32_t* __restrict__ isums) {
  constexpr int RG = gemv_rg(UPL);
  constexpr int RPG = 64 / LPR;   // rows side by side in one wavefront
  constexpr int RPW = RPG * RG;   // rows per wavefront
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int sub = lane % LPR;
  const int slot = lane / LPR;
  const int units = K >> 5;
  const int64_t crow = K >> 1;   // code bytes per row
  const int64_t srow = K >> 4;   // scale bytes per row
  const uint8_t* __restrict__ sc = w + N * crow;
  const int64_t row0 = ((int64_t)blockIdx.x * 4 + wave) * RPW;

  // 1. weight loads of all RG row groups first (RG*UPL 16-byte loads in flight)
  uint4 cw[RG][UPL];
  uint32_t sw[RG][UPL];
#pragma unroll
  for (int r = 0; r < RG; ++r) {
    const int64_t row = row0 + r * RPG + slot;
#pragma unroll
    for (int j = 0; j < UPL; ++j) {
      const int u = sub + LPR * j;
      if (row < N && u < units) {
        cw[r][j] = *reinterpret_cast<const uint4*>(w + row * crow + 16 * (int64_t)u);
        sw[r][j] = *reinterpret_cast<const uint16_t*>(sc + row * srow + 2 * (int64_t)u);
      } else {
        cw[r][j] = make_uint4(0u, 0u, 0u, 0u);
        sw[r][j] = 0u;
      }
    }
  }

  // 2. activation codes of this lane's units, split into even / odd positions
  uint32_t qe[UPL][4], qo[UPL][4];
  float dq[UPL];
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
      dq[j] = DEBUG ? 0.0f : 0.5f * f16_bits_to_f32(d16[u]);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) qe[j][i] = qo[j][i] = 0u;
      dq[j] = 0.0f;
    }
  }

  // 3. integer dots, per-subblock scaling, row reduction
#pragma unroll
  for (int r = 0; r < RG; ++r) {
    const int64_t row = row0 + r * RPG + slot;
    float acc = 0.0f;
#pragma unroll
    for (int j = 0; j < UPL; ++j) {
      int i0 = dot8_e2m1(cw[r][j].x, qe[j][0], qo[j][0], 0);
      i0 = dot8_e2m1(cw[r][j].y, qe[j][1], qo[j][1], i0);
      int i1 = dot8_e2m1(cw[r][j].z, qe[j][2], qo[j][2], 0);
      i1 = dot8_e2m1(cw[r][j].w, qe[j][3], qo[j][3], i1);
      if (DEBUG) {
        const int u = sub + LPR * j;
        if (row < N && u < units) {
          isums[row * srow + 2 * u] = i0;
          isums[row * srow + 2 * u + 1] = i1;
        }
      } else {
        const float u0 = ue4m3_to_f32<0>(sw[r][j]);
        const float u1 = ue4m3_to_f32<1>(sw[r][j]);
        acc = fmaf(fmaf((float)i0, u0, (float)i1 * u1), dq[j], acc);
      }
    }
    if (!DEBUG) {
      acc = group_sum<LPR>(acc);
      if (sub == 0 && row < N) y[row] = acc * w_scale;
    }
  }
}

// Generic fallback for K beyond kGemvMaxUPL*64*32 weights: one wavefront per row,
// activations re-read per unit (from cache).  Same arithmetic as the fast kernel.
template <bool DEBUG>
__global__ __launch_bounds__(256) void gemv_nvfp4_m1_long_kernel(
    const uint8_t* __restrict__ w, int64_t N, int K, const int8_t* __restrict__ q,
    const uint16_t* __restrict__ d16, float w_scale, float* __restrict__ y,
    int32_t* __restrict__ isums) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= N) return;  // whole wavefront exits together
  const int units = K >> 5;
  const int64_t crow = K >> 1, srow = K >> 4;
  const uint8_t* __restrict__ sc = w + N * crow;
  float acc = 0.0f;
  for (int u = lane; u < units; u += 64) {
    const uint4 c = *reinterpret_cast<const uint4*>(w + row * crow + 16 * (int64_t)u);
    const uint32_t s = *reinterpret_cast<const uint16_t*>(sc + row * srow + 2 * (int64_t)u);
    const uint4 a = *reinterpret_cast<const uint4*>(q + 32 * (int64_t)u);
    const uint4 b = *reinterpret_cast<const uint4*>(q + 32 * (int64_t)u + 16);
    uint32_t e0, o0, e1, o1, e2, o2, e3, o3;
    split_even_odd(a.x, a.y, e0, o0);
    split_even_odd(a.z, a.w, e1, o1);
    split_even_odd(b.x, b.y, e2, o2);
    split_even_odd(b.z, b.w, e3, o3);
    int i0 = dot8_e2m1(c.y, e1, o1, dot8_e2m1(c.x, e0, o0, 0));
    int i1 = dot8_e2m1(c.w, e3, o3, dot8_e2m1(c.z, e2, o2, 0));
    if (DEBUG) {
      isums[row * srow + 2 * u] = i0;
      isums[row * srow + 2 * u + 1] = i1;
    } else {
      const float dqv = 0.5f * f16_bits_to_f32(d16[u]);
      acc = fmaf(fmaf((float)i0, ue4m3_to_f32<0>(s), (float)i1 * ue4m3_to_f32<1>(s)), dqv, acc);
    }
  }
  if (!DEBUG) {
    acc = group_sum<64>(acc);
    if (lane == 0) y[row] = acc * w_scale;
  }
}

namespace {

typedef void (*gemv_fn)(const uint8_t*, int64_t, int, const int8_t*, const uint16_t*, float,
                        float*, int32_t*);

template <int LPR, bool DEBUG>
gemv_fn pick_upl(int upl) {
  switch (upl) {
    case 1: return gemv_nvfp4_m1_kernel<LPR, 1, DEBUG>;
    case 2: return gemv_nvfp4_m1_kernel<LPR, 2, DEBUG>;
    case 3: return gemv_nvfp4_m1_kernel<LPR, 3, DEBUG>;
    case 4: return gemv_nvfp4_m1_kernel<LPR, 4, DEBUG>;
    case 5: return gemv_nvfp4_m1_kernel<LPR, 5, DEBUG>;
    case 6: return gemv_nvfp4_m1_kernel<LPR, 6, DEBUG>;
    case 7: return gemv_nvfp4_m1_kernel<LPR, 7, DEBUG>;
    case 8: return gemv_nvfp4_m1_kernel<LPR, 8, DEBUG>;
    case 9: return gemv_nvfp4_m1_kernel<LPR, 9, DEBUG>;
    case 10: return gemv_nvfp4_m1_kernel<LPR, 10, DEBUG>;
    default: return nullptr;
  }
}

}  // namespace

// Choose lanes-per-row and units-per-lane for a K: the LPR in {64, 32, 16} with
// the fewest idle unit slots (ties to the wider LPR), subject to UPL <= 10.
void gemv_m1_config(int64_t K, int* lpr_out, int* upl_out) {
  const int units = (int)(K / 32);
  int best_lpr = 0, best_upl = 0;
  double best_eff = -1.0;
  const int lprs[3] = {64, 32, 16};
  for (int i = 0; i < 3; ++i) {
    const int lpr = lprs[i];
    const int upl = (units + lpr - 1) / lpr;
    if (upl > kGemvMaxUPL) continue;
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

hipError_t launch_gemv_nvfp4_m1(const uint8_t* w, float w_scale, const int8_t* q,
                                const uint16_t* d16, int64_t N, int64_t K, float* y,
                                int32_t* isums, hipStream_t stream) {
  const bool debug = isums != nullptr;
  int lpr = 0, upl = 0;
  gemv_m1_config(K, &lpr, &upl);
  if (lpr == 0) {
    const int64_t grid = (N + 3) / 4;
    if (debug)
      hipLaunchKernelGGL(gemv_nvfp4_m1_long_kernel<true>, dim3((unsigned)grid), dim3(256), 0,
                         stream, w, N, (int)K, q, d16, w_scale, y, isums);
    else
      hipLaunchKernelGGL(gemv_nvfp4_m1_long_kernel<false>, dim3((unsigned)grid), dim3(256), 0,
                         stream, w, N, (int)K, q, d16, w_scale, y, isums);
    return hipGetLastError();
  }
  gemv_fn fn = nullptr;
  if (lpr == 64) fn = debug ? pick_upl<64, true>(upl) : pick_upl<64, false>(upl);
  if (lpr == 32) fn = debug ? pick_upl<32, true>(upl) : pick_upl<32, false>(upl);
  if (lpr == 16) fn = debug ? pick_upl<16, true>(upl) : pick_upl<16, false>(upl);
  if (!fn) return hipErrorInvalidValue;
  const int64_t rows_per_block = 4 * (64 / lpr) * gemv_rg(upl);
  const int64_t grid = (N + rows_per_block - 1) / rows_per_block;
  hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(256), 0, stream, w, N, (int)K, q, d16,
                     w_scale, y, isums);
  return hipGetLastError();
}

}  // namespace nvq
