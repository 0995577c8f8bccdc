// gemv_nvfp4.hip -- single-token decode GEMV, NVFP4 weights x Q8_0 activations, gfx950.
//
// What is computed ("HANDOFF: flint CPU optimization (Q4_1 + NVFP4)", section 3,
// Code map and bias-trick paragraph): for every 16-weight subblock an exact integer
// sum of the weight codes' values times the activation codes, then one float scale
// per subblock:
//     y[n] = S * sum_s UE4M3(scale[n][s]) * d[s/2] * sum_{k in s} E2M1(code[n][k]) * q[k].
//
// Weights use the tile-interleaved packed layout (include/nvq.h): a 16-row x 128-k
// tile-chunk is 1 KB of codes in MFMA lane order (lane l = 16*g + n holds row n,
// k = 32g..32g+31) followed elsewhere by its 128 scale bytes (lane l: the two scales
// of subblocks 2g, 2g+1).  Every wavefront load is therefore 1 KB contiguous.
//
// Two inner loops share one skeleton.  A block of W wavefronts owns one 16-row tile;
// wavefront v takes the chunks c = v, v + W, ... in batches of P, issuing the loads of
// a batch before computing it.  The activation table is built once per block in LDS.
// Order of the prologue matters: the activation codes are loaded first and every
// global load is unconditional (indices are clamped into the buffers), so the table
// build waits only for those codes (loads retire in order) and runs while the first
// weight batch is still in flight.  Partial sums are reduced through LDS at the end.
//
//  * MODE_MX (production).  gfx950's matrix cores read E2M1 natively: the 16 packed
//    bytes a lane loads are, unchanged, its FP4 operand of one
//    v_mfma_scale_f32_16x16x128_f8f6f4.  The FP8 (E4M3) operand carries the
//    activations: each code q = 16*h + l with h = q >> 4 in [-8, 7] and l = q & 15,
//    both exact in E4M3 (a byte b <= 15 encodes exactly b * 2^-9, which the
//    operand's MX scale 2^9 undoes; h is stored sign-magnitude).  Its 16 rows are
//    (subblock sb, part) variants that are zero outside subblock sb, so one MFMA
//    returns, for 16 weight rows, the 8 per-subblock sums of both parts:
//    isum = 16 * D_h + D_l is exact.  The vector unit only applies
//    UE4M3 * d per subblock (about 10 instructions per 2048 weights), so the
//    kernel stays under the HBM stream instead of being bound by code expansion.
//
//  * MODE_DOT4.  The same sums with the vector unit only: E2M1 -> int8 by two
//    v_perm_b32 table lookups per four codes, summed inside v_dot4_i32_i8 (see
//    nvq_device.h).  About 13 full-rate instructions per 8 weights: on MI355X this
//    costs as much time as streaming the bytes, so it is the slower of the two.

#include "nvq_device.h"
#include "nvq_launch.h"

namespace nvq {

typedef int v8i __attribute__((ext_vector_type(8)));

// Four activation codes -> the high parts h = q >> 4 as sign-magnitude E4M3 bytes
// (|h| <= 8, value |h| * 2^-9 with the sign bit).
__device__ __forceinline__ uint32_t act_hi_e4m3(uint32_t q) {
  const uint32_t nib = (q >> 4) & 0x0F0F0F0Fu;   // h as a two's complement nibble
  const uint32_t neg = (nib >> 3) & 0x01010101u;  // 1 where h < 0
  const uint32_t m = (neg << 4) - neg;            // 0x0F where h < 0
  const uint32_t mag = (nib ^ m) + neg;           // |h|
  return mag | (neg << 7);
}

// LDS carve-up shared by kernel and launcher: activation table [nch + 1][256 B] (the
// last chunk slot takes the writes of out-of-range threads), 16 zero bytes, d table
// [nch * 4 + 4] floats (the last 4 likewise), partial sums [W][64] floats.
__host__ __device__ constexpr int64_t gemv_tab_bytes(int64_t nch) { return (nch + 1) * 256; }
__host__ __device__ constexpr int64_t gemv_dtab_off(int64_t nch) { return gemv_tab_bytes(nch) + 16; }
__host__ __device__ constexpr int64_t gemv_red_off(int64_t nch) { return gemv_dtab_off(nch) + (nch * 4 + 4) * 4; }

// One 16-row tile of the product (the body of both kernels below).
template <int MODE, bool DEBUG, int W, int P>
__device__ __forceinline__ void gemv_tile(const uint8_t* __restrict__ w, int64_t N, int K,
                                          const int8_t* __restrict__ q, const uint16_t* __restrict__ d16,
                                          float w_scale, float* __restrict__ y, int32_t* __restrict__ isums,
                                          int64_t tile) {
  constexpr int NT = 64 * W;
  extern __shared__ __align__(16) uint8_t smem[];
  const int nch = (K + 127) >> 7;
  const int nsb = K >> 4;
  const int nq16 = K >> 4;  // 16-code groups of the activation row
  const int nd = K >> 5;    // activation scales
  uint8_t* tab = smem;
  uint8_t* zero16 = smem + gemv_tab_bytes(nch);
  float* dtab = reinterpret_cast<float*>(smem + gemv_dtab_off(nch));
  float* red = reinterpret_cast<float*>(smem + gemv_red_off(nch));
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nl = lane & 15, g = lane >> 4;
  const int64_t ntiles = (N + 15) >> 4;
  const uint8_t* __restrict__ wt = w + tile * nch * 1024 + 16 * lane;
  const uint8_t* __restrict__ st = w + ntiles * nch * 1024 + tile * nch * 128 + 2 * lane;

  // 1. activation codes and scales first (at most two 16-code groups per thread here)
  const u32x4* __restrict__ q16 = reinterpret_cast<const u32x4*>(q);
  const u32x4 qa = q16[min(tid, nq16 - 1)];
  const u32x4 qb = q16[min(tid + NT, nq16 - 1)];
  uint32_t da = 0u;
  if (!DEBUG) da = d16[min(tid, nd - 1)];
  __builtin_amdgcn_sched_barrier(0);

  // 2. first batch of weight loads (chunk indices clamped: loads past the row's last
  //    chunk re-read it and are never consumed)
  u32x4 bb[P];
  uint32_t ss[P];
  auto issue = [&](int c0) {
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int c = min(c0 + W * p, nch - 1);
      bb[p] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wt + (int64_t)c * 1024));
      ss[p] = __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(st + (int64_t)c * 128));
    }
  };
  int c0 = wave;
  issue(c0);
  __builtin_amdgcn_sched_barrier(0);

  // 3. activation table.  MX: per 128-k chunk [h parts 128 B | l parts 128 B].
  //    DOT4: per 32-k quarter [even codes 16 B | odd codes 16 B].
  auto put = [&](int j, const u32x4& v) {  // the 16 codes k = 16 j .. 16 j + 15
    const int k = 16 * j, c = k >> 7, o = k & 127;
    if (MODE == 0) {
      const u32x4 hi = {act_hi_e4m3(v[0]), act_hi_e4m3(v[1]), act_hi_e4m3(v[2]), act_hi_e4m3(v[3])};
      const u32x4 lo = {v[0] & 0x0F0F0F0Fu, v[1] & 0x0F0F0F0Fu, v[2] & 0x0F0F0F0Fu, v[3] & 0x0F0F0F0Fu};
      *reinterpret_cast<u32x4*>(tab + c * 256 + o) = hi;
      *reinterpret_cast<u32x4*>(tab + c * 256 + 128 + o) = lo;
    } else {
      uint32_t e0, o0, e1, o1;
      split_even_odd(v[0], v[1], e0, o0);
      split_even_odd(v[2], v[3], e1, o1);
      const int base = c * 256 + (o >> 5) * 64 + 8 * ((o & 31) >> 4);
      *reinterpret_cast<uint2*>(tab + base) = make_uint2(e0, e1);
      *reinterpret_cast<uint2*>(tab + base + 16) = make_uint2(o0, o1);
    }
  };
  const int junk = nch * 8;  // 16-code group index of the spare chunk slot
  put(tid < nq16 ? tid : junk, qa);
  put(tid + NT < nq16 ? tid + NT : junk, qb);
  for (int j = tid + 2 * NT; j < nq16; j += NT) put(j, q16[j]);
  for (int j = nq16 + tid; j < nch * 8; j += NT) put(j, u32x4{0u, 0u, 0u, 0u});
  if (!DEBUG) {
    dtab[tid < nd ? tid : nch * 4] = f16_bits_to_f32((uint16_t)da);
    for (int b = tid + NT; b < nd; b += NT) dtab[b] = f16_bits_to_f32(d16[b]);
    for (int b = nd + tid; b < nch * 4; b += NT) dtab[b] = 0.0f;
  }
  if (tid < 4) reinterpret_cast<uint32_t*>(zero16)[tid] = 0u;
  __syncthreads();

  // 4. compute
  const int sbv = nl >> 1, part = nl & 1;
  const uint32_t pal = in_vgpr(kPA_lo), pah = in_vgpr(kPA_hi);
  const uint32_t pbl = in_vgpr(kPB_lo), pbh = in_vgpr(kPB_hi);
  const uint32_t m4 = in_vgpr(0x0F0F0F0Fu), m3 = in_vgpr(0x07070707u);
  const int64_t row = tile * 16 + nl;
  float acc = 0.0f;
  while (true) {
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int c = c0 + W * p;
      if (c >= nch) continue;
      float i0, i1;  // the two per-16 sums (E2M1 units) of subblocks 8c+2g, 8c+2g+1
      if (MODE == 0) {
        const uint8_t* pa = (sbv == g) ? tab + c * 256 + part * 128 + 16 * g : zero16;
        const uint8_t* pb = (sbv == g + 4) ? tab + c * 256 + part * 128 + 64 + 16 * g : zero16;
        const u32x4 a0 = *reinterpret_cast<const u32x4*>(pa);
        const u32x4 a1 = *reinterpret_cast<const u32x4*>(pb);
        const v8i av = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3],
                        (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
        const v8i bv = {(int)bb[p][0], (int)bb[p][1], (int)bb[p][2], (int)bb[p][3], 0, 0, 0, 0};
        // A: FP8 activation variants (scale 2^9), B: FP4 weights (scale 1)
        const floatx4 D = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            av, bv, floatx4{0.f, 0.f, 0.f, 0.f}, 0, 4, 0, 127 + 9, 0, 127);
        i0 = fmaf(D[0], 16.0f, D[1]);
        i1 = fmaf(D[2], 16.0f, D[3]);
      } else {
        const u32x4 qe = *reinterpret_cast<const u32x4*>(tab + c * 256 + g * 64);
        const u32x4 qo = *reinterpret_cast<const u32x4*>(tab + c * 256 + g * 64 + 16);
        int a0 = 0, b0 = 0, a1 = 0, b1 = 0;
        dot8_e2m1_ab(bb[p][0], qe[0], qo[0], a0, b0, pal, pah, pbl, pbh, m4, m3);
        dot8_e2m1_ab(bb[p][1], qe[1], qo[1], a0, b0, pal, pah, pbl, pbh, m4, m3);
        dot8_e2m1_ab(bb[p][2], qe[2], qo[2], a1, b1, pal, pah, pbl, pbh, m4, m3);
        dot8_e2m1_ab(bb[p][3], qe[3], qo[3], a1, b1, pal, pah, pbl, pbh, m4, m3);
        i0 = 0.5f * (float)(a0 + b0);  // L = 2 * E2M1
        i1 = 0.5f * (float)(a1 + b1);
      }
      if (DEBUG) {
        const int s0 = 8 * c + 2 * g;
        if (row < N && s0 < nsb) {
          isums[row * nsb + s0] = (int32_t)(2.0f * i0);
          isums[row * nsb + s0 + 1] = (int32_t)(2.0f * i1);
        }
      } else {
        const float t = fmaf(i0, ue4m3_to_f32<0>(ss[p]), i1 * ue4m3_to_f32<1>(ss[p]));
        acc = fmaf(t, dtab[4 * c + g], acc);
      }
    }
    c0 += W * P;
    if (c0 >= nch) break;
    issue(c0);
  }
  if (DEBUG) return;

  // 5. reduce the 4 W partial sums of each row (4 lane groups x W wavefronts)
  red[wave * 64 + lane] = acc;
  __syncthreads();
  if (tid < 16) {
    float s = 0.0f;
#pragma unroll
    for (int ww = 0; ww < W; ++ww)
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) s += red[ww * 64 + gg * 16 + tid];
    const int64_t r = tile * 16 + tid;
    if (r < N) y[r] = s * w_scale;
  }
}

template <int MODE, bool DEBUG, int W, int P>
__global__ __launch_bounds__(64 * W) void gemv_nvfp4_kernel(const uint8_t* __restrict__ w, int64_t N,
                                                            int K, const int8_t* __restrict__ q,
                                                            const uint16_t* __restrict__ d16,
                                                            float w_scale, float* __restrict__ y,
                                                            int32_t* __restrict__ isums) {
  gemv_tile<MODE, DEBUG, W, P>(w, N, K, q, d16, w_scale, y, isums, blockIdx.x);
}

// Expert-routed form (the "mul_mat_id" step of a mixture-of-experts layer; "HANDOFF:
// flint CPU optimization (Q4_1 + NVFP4)", section 7 "Open items / next steps", item 1):
// grid.y enumerates the (token, routing slot) jobs, job = m * A + a.  The block reads
// its expert id once (wavefront-uniform), and runs the same tile on that expert's
// packed matrix, its per-tensor scale and token m's activations, into y[job][N].  An
// id outside [0, E) reads no weights and writes NaN to its rows.
template <int W, int P>
__global__ __launch_bounds__(64 * W) void gemv_nvfp4_routed_kernel(const uint8_t* __restrict__ w,
                                                                   int64_t expert_bytes,
                                                                   const float* __restrict__ w_scales,
                                                                   const int32_t* __restrict__ ids, int E,
                                                                   int A, int64_t N, int K,
                                                                   const int8_t* __restrict__ q,
                                                                   const uint16_t* __restrict__ d16,
                                                                   float* __restrict__ y) {
  const int job = blockIdx.y;
  const int e = ids[job];
  float* yj = y + (int64_t)job * N;
  if (e < 0 || e >= E) {
    const int64_t r = (int64_t)blockIdx.x * 16 + threadIdx.x;
    if (threadIdx.x < 16 && r < N) yj[r] = __builtin_nanf("");
    return;
  }
  const int64_t m = job / A;
  gemv_tile<0, false, W, P>(w + (int64_t)e * expert_bytes, N, K, q + m * K, d16 + m * (K >> 5), w_scales[e], yj,
                            nullptr, blockIdx.x);
}

// Launch shape: 4 wavefronts x 5-chunk batches, or 8 x 3 for long rows over few tiles
// (the down projection: K = 17408 over 320 tiles), where more wavefronts per tile keep
// more loads in flight per block.
static bool gemv_wide(int64_t ntiles, int64_t nch) { return nch >= 64 && ntiles <= 1024; }

size_t gemv_lds_bytes(int64_t K) {
  const int64_t nch = (K + 127) / 128;
  return (size_t)(gemv_red_off(nch) + 8 * 64 * 4);  // room for the widest block (W = 8)
}

template <int MODE, bool DEBUG, int W, int P>
static hipError_t launch_gemv(const uint8_t* w, float w_scale, const int8_t* q, const uint16_t* d16,
                              int64_t N, int64_t K, float* y, int32_t* isums, hipStream_t stream) {
  const int64_t ntiles = (N + 15) / 16;
  const int64_t nch = (K + 127) / 128;
  const size_t lds = (size_t)(gemv_red_off(nch) + W * 64 * 4);
  auto fn = gemv_nvfp4_kernel<MODE, DEBUG, W, P>;
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(fn, dim3((unsigned)ntiles), dim3(64 * W), lds, stream, w, N, (int)K, q, d16,
                     w_scale, y, isums);
  return hipGetLastError();
}

hipError_t launch_gemv_nvfp4_m1(const uint8_t* w, float w_scale, const int8_t* q,
                                const uint16_t* d16, int64_t N, int64_t K, float* y,
                                int32_t* isums, int mode, hipStream_t stream) {
  const int64_t ntiles = (N + 15) / 16;
  const int64_t nch = (K + 127) / 128;
  if (isums != nullptr)
    return mode == 0 ? launch_gemv<0, true, 4, 5>(w, w_scale, q, d16, N, K, y, isums, stream)
                     : launch_gemv<1, true, 4, 5>(w, w_scale, q, d16, N, K, y, isums, stream);
  if (mode != 0) return launch_gemv<1, false, 4, 5>(w, w_scale, q, d16, N, K, y, isums, stream);
  if (gemv_wide(ntiles, nch)) return launch_gemv<0, false, 8, 3>(w, w_scale, q, d16, N, K, y, isums, stream);
  return launch_gemv<0, false, 4, 5>(w, w_scale, q, d16, N, K, y, isums, stream);
}

template <int W, int P>
static hipError_t launch_routed(const uint8_t* w, const float* w_scales, const int32_t* ids, int64_t E,
                                int64_t A, int64_t M, const int8_t* q, const uint16_t* d16, int64_t N,
                                int64_t K, float* y, hipStream_t stream) {
  const int64_t ntiles = (N + 15) / 16;
  const int64_t nch = (K + 127) / 128;
  const size_t lds = (size_t)(gemv_red_off(nch) + W * 64 * 4);
  const int64_t expert_bytes = ntiles * nch * (1024 + 128);
  auto fn = gemv_nvfp4_routed_kernel<W, P>;
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(fn, dim3((unsigned)ntiles, (unsigned)(M * A)), dim3(64 * W), lds, stream, w, expert_bytes,
                     w_scales, ids, (int)E, (int)A, N, (int)K, q, d16, y);
  return hipGetLastError();
}

hipError_t launch_gemv_nvfp4_routed(const uint8_t* w, const float* w_scales, const int32_t* ids, int64_t E,
                                    int64_t A, int64_t M, const int8_t* q, const uint16_t* d16, int64_t N,
                                    int64_t K, float* y, hipStream_t stream) {
  const int64_t ntiles = (N + 15) / 16;
  const int64_t nch = (K + 127) / 128;
  if (gemv_wide(ntiles * M * A, nch))
    return launch_routed<8, 3>(w, w_scales, ids, E, A, M, q, d16, N, K, y, stream);
  return launch_routed<4, 5>(w, w_scales, ids, E, A, M, q, d16, N, K, y, stream);
}

}  // namespace nvq
