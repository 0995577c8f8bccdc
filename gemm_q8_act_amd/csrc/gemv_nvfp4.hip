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
//
// Fused quantization (gemv_tile_fused, MODE_MX, one token): the block reads the
// float32 row x instead of its Q8_0 codes and quantizes it into its LDS table, each
// wavefront exactly the chunks it consumes (no block barrier: no wavefront reads
// another's entries).  The float4 loads are issued first, then the first batch of
// weight loads, and the quantization runs while that batch is in flight.  No separate
// quantization launch (and no round trip of the codes through memory) precedes the
// product.  The codes are bit-exact with nvq_quantize_act_q8_0 (see q8_0_pack4).

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

// d32 = fl(amax / 127) without the division sequence: q0 = amax * fl(1/127), then one
// fma correction, d = fma(fma(-q0, 127, amax), fl(1/127), q0).  Checked exhaustively
// against IEEE float32 division: equal for every non-negative finite float (2^31
// values, subnormals included).
__device__ __forceinline__ float div127(float a) {
  constexpr float kInv127 = 0x1.020408p-7f;  // fl(1 / 127)
  const float q0 = a * kInv127;
  return __builtin_fmaf(__builtin_fmaf(-q0, 127.0f, a), kInv127, q0);
}

// max over the 8 lanes of each aligned 8-lane group (DPP: quad_perm [1,0,3,2],
// quad_perm [2,3,0,1], row_half_mirror), no LDS traffic
__device__ __forceinline__ float max8(float v) {
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, true)));
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, true)));
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, true)));
  return v;
}

// Q8_0 codes of 4 values of a 32-value block whose scale is d32 = fl(amax / 127):
// q = clamp(rint(fl(x / d32)), -127, 127), packed one byte each; d32 == 0 gives 0.
// Each quotient is taken as u = fma(x, r, 128) with r = v_rcp_f32(d32) (1 ulp):
// |x / d32| <= 127.00002, so |u - 128 - fl(x / d32)| <= 127.00002 (2^-23 + 2^-24) +
// 2^-18 + 2^-17 < 4.2e-5; whenever u lies more than 2^-14 (6.1e-5) inside the
// interval of its nearest integer k, k - 128 is also rint(fl(x / d32)) and |k - 128|
// <= 127.  The biased code k (1..255) is packed with v_cvt_pk_u8_f32 and the bias
// removed by flipping each byte's top bit.  Quotients nearer a rounding tie, and
// every quotient of a block with 0 < d32 < 2^-100 (whose reciprocal could leave the
// normal range), take the IEEE division and the clamp themselves.
__device__ __forceinline__ uint32_t q8_0_pack4(const float4& v, float d) {
  const bool exact = d > 0.0f && d < 0x1.0p-100f;
  const float r = d > 0.0f ? __builtin_amdgcn_rcpf(d) : 0.0f;
  const float xs[4] = {v.x, v.y, v.z, v.w};
  uint32_t packed = 0u;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float u = __builtin_fmaf(xs[i], r, 128.0f);
    float k = __builtin_rintf(u);
    if (exact || fabsf(u - k) > 0.49993896484375f) k = fminf(fmaxf(__builtin_rintf(xs[i] / d), -127.0f), 127.0f) + 128.0f;
    packed = __builtin_amdgcn_cvt_pk_u8_f32(k, (uint32_t)i, packed);
  }
  return packed ^ 0x80808080u;
}

// One 16-row tile of the product (the body of both kernels below).  OWN: the activation
// table is built per wavefront (below) instead of by the whole block.
template <int MODE, bool DEBUG, int W, int P, bool OWN>
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

  // OWN (the plain kernel's many-tile launch shape, 8 wavefronts x 5-chunk batches, and
  // the expert-routed kernel; matrix-core loop, no debug sums): each wavefront builds the table entries of the chunks it consumes (v, v + W,
  // ...) and needs no block barrier, since no wavefront reads another's entries.  Lane l
  // takes 16-code group l % 8 of the chunks v + W (l / 8 + 8 u) and activation scale l % 4
  // of the chunks v + W (l / 4 + 16 u); the first two code groups and the first scale are
  // loaded before the weights.  Measured against the block-cooperative build: gate+up
  // 34816 x 5120 17.1 -> 16.75 us; on the other shapes it was 0.5-1.6 % slower (down
  // 11.70 -> 11.89 us), so they keep the cooperative build.  Routed 6 of 256 experts (2048 x 2048): 5.12 -> 5.05 us.
  constexpr bool kOwn = OWN && MODE == 0 && !DEBUG;
  const u32x4* __restrict__ q16 = reinterpret_cast<const u32x4*>(q);
  const int oc = lane >> 3, og = lane & 7;  // chunk slot (of 8 per pass) and 16-code group
  // 1. activation codes and scales first (at most two 16-code groups per thread here)
  u32x4 qa, qb;
  uint32_t da = 0u;
  if constexpr (kOwn) {
    qa = q16[min(8 * (wave + W * oc) + og, nq16 - 1)];
    qb = q16[min(8 * (wave + W * (oc + 8)) + og, nq16 - 1)];
    da = d16[min(4 * (wave + W * (lane >> 2)) + (lane & 3), nd - 1)];
  } else {
    qa = q16[min(tid, nq16 - 1)];
    qb = q16[min(tid + NT, nq16 - 1)];
    if (!DEBUG) da = d16[min(tid, nd - 1)];
  }
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
  if constexpr (kOwn) {
    // 16-code group j of chunk c: in the row (j < nq16), zero past the row's end in its
    // last chunk, the spare slot for chunks past the row
    auto own_put = [&](int c, const u32x4& v) {
      const int j = 8 * c + og;
      put(c < nch ? j : junk, j < nq16 ? v : u32x4{0u, 0u, 0u, 0u});
    };
    own_put(wave + W * oc, qa);
    own_put(wave + W * (oc + 8), qb);
    for (int u = 2; wave + W * 8 * u < nch; ++u) {
      const int c = wave + W * (oc + 8 * u);
      own_put(c, q16[min(8 * c + og, nq16 - 1)]);
    }
    // scales: lane l takes scale l % 4 of the chunk v + W (l / 4 + 16 u)
    auto own_d = [&](int c, uint32_t dv) {
      const int bi = 4 * c + (lane & 3);
      dtab[c < nch ? bi : nch * 4] = bi < nd ? f16_bits_to_f32((uint16_t)dv) : 0.0f;
    };
    own_d(wave + W * (lane >> 2), da);
    for (int u = 1; wave + W * 16 * u < nch; ++u) {
      const int c = wave + W * ((lane >> 2) + 16 * u);
      own_d(c, d16[min(4 * c + (lane & 3), nd - 1)]);
    }
    if (lane < 4) reinterpret_cast<uint32_t*>(zero16)[lane] = 0u;  // every wavefront writes the same zeros
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  } else {
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
  }

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

// One 16-row tile of the product with the Q8_0 quantization of the float32 row x
// fused in (MODE_MX inner loop, as gemv_tile).  Prologue: wavefront v consumes the
// chunks c = v, v + W, ...; its lane l loads the float4 group 32 c + l % 32 (k = 128 c
// + 4 (l % 32) .. + 3) of chunks c = v + W (2 u + l / 32), u < XU (8 consecutive lanes
// hold one 32-value block, all in the row or all past it), then issues the first
// weight batch, then quantizes those groups into the LDS table while the weights
// stream in (loads retire in order, so the quantization waits for x only); rows with
// more than 2 XU chunks per wavefront load the rest as they go.  q_out / d_out, if not
// null, receive the row's codes and binary16 scales (block of tile 0).
template <int W, int P, int XU>
__device__ __forceinline__ void gemv_tile_fused(const uint8_t* __restrict__ w, int64_t N, int K,
                                                const float* __restrict__ x, float w_scale, float* __restrict__ y,
                                                int8_t* __restrict__ q_out, uint16_t* __restrict__ d_out,
                                                int64_t tile) {
  constexpr int NT = 64 * W;
  extern __shared__ __align__(16) uint8_t smem[];
  const int nch = (K + 127) >> 7;
  const int n4 = K >> 2, nd = K >> 5;
  uint8_t* tab = smem;
  uint8_t* zero16 = smem + gemv_tab_bytes(nch);
  float* dtab = reinterpret_cast<float*>(smem + gemv_dtab_off(nch));
  float* red = reinterpret_cast<float*>(smem + gemv_red_off(nch));
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nl = lane & 15, g = lane >> 4;
  const int64_t ntiles = (N + 15) >> 4;
  const uint8_t* __restrict__ wt = w + tile * nch * 1024 + 16 * lane;
  const uint8_t* __restrict__ st = w + ntiles * nch * 1024 + tile * nch * 128 + 2 * lane;
  const float4* __restrict__ x4 = reinterpret_cast<const float4*>(x);

  const int xh = lane >> 5, xl = lane & 31;
  float4 xv[XU];
  // 1. the float32 activations of this wavefront's own chunks first: lane half h takes
  //    chunks c = wave + W (2 u + h), lane l (of 32) its float4 group 32 c + l
#pragma unroll
  for (int u = 0; u < XU; ++u) xv[u] = x4[min(32 * (wave + W * (2 * u + xh)) + xl, n4 - 1)];
  __builtin_amdgcn_sched_barrier(0);

  // 2. first batch of weight loads (chunk indices clamped, as in gemv_tile)
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

  const bool write_q = tile == 0 && q_out != nullptr;
  // 3. quantize this wavefront's chunks into the table (MX layout of gemv_tile).  Only
  //    this wavefront reads them, so no block barrier: chunks past the row go to the
  //    spare slot nch, groups past the row's end (K % 128 == 64) get zero codes and scale.
  auto quant_put = [&](const float4& v, int c) {
    const float a = max8(fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
    const float d = div127(a);  // = fl(amax / 127)
    const uint32_t pk = q8_0_pack4(v, d);
    const int g4 = 32 * c + xl, cs = min(c, nch), o = 4 * xl;
    const bool in_row = g4 < n4;
    *reinterpret_cast<uint32_t*>(tab + cs * 256 + o) = in_row ? act_hi_e4m3(pk) : 0u;
    *reinterpret_cast<uint32_t*>(tab + cs * 256 + 128 + o) = in_row ? pk & 0x0F0F0F0Fu : 0u;
    const _Float16 dh = (_Float16)d;  // the stored binary16 scale (round to nearest even)
    if ((xl & 7) == 0) dtab[4 * cs + (xl >> 3)] = in_row ? (float)dh : 0.0f;
    if (write_q && in_row) {
      *reinterpret_cast<uint32_t*>(q_out + 4 * g4) = pk;
      if ((xl & 7) == 0) d_out[g4 >> 3] = __builtin_bit_cast(uint16_t, dh);
    }
  };
#pragma unroll
  for (int u = 0; u < XU; ++u) quant_put(xv[u], wave + W * (2 * u + xh));
  for (int u = XU; wave + W * 2 * u < nch; ++u) {
    const int c = wave + W * (2 * u + xh);
    quant_put(x4[min(32 * c + xl, n4 - 1)], c);
  }
  if (lane < 4) reinterpret_cast<uint32_t*>(zero16)[lane] = 0u;  // every wavefront writes the same zeros
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  // 4. compute (the MX loop of gemv_tile)
  const int sbv = nl >> 1, part = nl & 1;
  float acc = 0.0f;
  while (true) {
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int c = c0 + W * p;
      if (c >= nch) continue;
      const uint8_t* pa = (sbv == g) ? tab + c * 256 + part * 128 + 16 * g : zero16;
      const uint8_t* pb = (sbv == g + 4) ? tab + c * 256 + part * 128 + 64 + 16 * g : zero16;
      const u32x4 a0 = *reinterpret_cast<const u32x4*>(pa);
      const u32x4 a1 = *reinterpret_cast<const u32x4*>(pb);
      const v8i av = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
      const v8i bv = {(int)bb[p][0], (int)bb[p][1], (int)bb[p][2], (int)bb[p][3], 0, 0, 0, 0};
      const floatx4 D = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, floatx4{0.f, 0.f, 0.f, 0.f}, 0, 4,
                                                                        0, 127 + 9, 0, 127);
      const float i0 = fmaf(D[0], 16.0f, D[1]), i1 = fmaf(D[2], 16.0f, D[3]);
      const float t = fmaf(i0, ue4m3_to_f32<0>(ss[p]), i1 * ue4m3_to_f32<1>(ss[p]));
      acc = fmaf(t, dtab[4 * c + g], acc);
    }
    c0 += W * P;
    if (c0 >= nch) break;
    issue(c0);
  }

  // 5. reduce the 4 W partial sums of each row
  red[wave * 64 + lane] = acc;
  __syncthreads();
  if (tid < 16) {
    float sum = 0.0f;
#pragma unroll
    for (int ww = 0; ww < W; ++ww)
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) sum += red[ww * 64 + gg * 16 + tid];
    const int64_t r = tile * 16 + tid;
    if (r < N) y[r] = sum * w_scale;
  }
}

template <int MODE, bool DEBUG, int W, int P>
__global__ __launch_bounds__(64 * W) void gemv_nvfp4_kernel(const uint8_t* __restrict__ w, int64_t N,
                                                            int K, const int8_t* __restrict__ q,
                                                            const uint16_t* __restrict__ d16,
                                                            float w_scale, float* __restrict__ y,
                                                            int32_t* __restrict__ isums) {
  gemv_tile<MODE, DEBUG, W, P, W == 8 && P == 5>(w, N, K, q, d16, w_scale, y, isums, blockIdx.x);
}

// Fused quantization + decode GEMV (one token): y = S * W . Q8_0(x).
// At least 8 wavefronts per SIMD (at most 64 VGPRs): two 16-wavefront blocks must share
// a compute unit on the down projection's grid (320 blocks), and the wavefront-owned
// quantization would otherwise take 65 VGPRs there (down 13.0 us with this bound and
// one spilled register, 15.7 without it)
template <int W, int P, int XU>
__global__ __launch_bounds__(64 * W, 8) void gemv_nvfp4_fused_kernel(const uint8_t* __restrict__ w, int64_t N, int K,
                                                                  const float* __restrict__ x, float w_scale,
                                                                  float* __restrict__ y, int8_t* __restrict__ q_out,
                                                                  uint16_t* __restrict__ d_out) {
  gemv_tile_fused<W, P, XU>(w, N, K, x, w_scale, y, q_out, d_out, blockIdx.x);
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
  gemv_tile<0, false, W, P, true>(w + (int64_t)e * expert_bytes, N, K, q + m * K, d16 + m * (K >> 5), w_scales[e],
                                  yj, nullptr, blockIdx.x);
}

// Launch shape: 4 wavefronts x 5-chunk batches; 8 x 3 for long rows over few tiles
// (the down projection: K = 17408 over 320 tiles), where more wavefronts per tile keep
// more loads in flight per block; 8 x 5 from 1024 tiles up (gate+up 34816 x 5120:
// 16.9 us against 17.2 with 4 x 5; QKV and O, under 1024 tiles, are 5 % slower with it).
static bool gemv_wide(int64_t ntiles, int64_t nch) { return nch >= 64 && ntiles <= 1024; }

size_t gemv_lds_bytes(int64_t K) {
  const int64_t nch = (K + 127) / 128;
  return (size_t)(gemv_red_off(nch) + 16 * 64 * 4);  // room for the widest block (W = 16)
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
  if (ntiles >= 1024) return launch_gemv<0, false, 8, 5>(w, w_scale, q, d16, N, K, y, isums, stream);
  return launch_gemv<0, false, 4, 5>(w, w_scale, q, d16, N, K, y, isums, stream);
}

template <int W, int P, int XU>
static hipError_t launch_fused(const uint8_t* w, float w_scale, const float* x, int64_t N, int64_t K, float* y,
                               int8_t* q_out, uint16_t* d_out, hipStream_t stream) {
  const int64_t ntiles = (N + 15) / 16;
  const int64_t nch = (K + 127) / 128;
  const size_t lds = (size_t)(gemv_red_off(nch) + W * 64 * 4);
  auto fn = gemv_nvfp4_fused_kernel<W, P, XU>;
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(fn, dim3((unsigned)ntiles), dim3(64 * W), lds, stream, w, N, (int)K, x, w_scale, y, q_out,
                     d_out);
  return hipGetLastError();
}

// XU = the float4 groups per thread that cover the row (at most 9 preloaded)
template <int W, int P>
static hipError_t launch_fused_w(const uint8_t* w, float w_scale, const float* x, int64_t N, int64_t K, float* y,
                                 int8_t* q_out, uint16_t* d_out, hipStream_t stream) {
  const int64_t xu = (K / 4 + 64 * W - 1) / (64 * W);
  switch (xu < 9 ? xu : 9) {
    case 1: return launch_fused<W, P, 1>(w, w_scale, x, N, K, y, q_out, d_out, stream);
    case 2: return launch_fused<W, P, 2>(w, w_scale, x, N, K, y, q_out, d_out, stream);
    case 3: return launch_fused<W, P, 3>(w, w_scale, x, N, K, y, q_out, d_out, stream);
    case 4: return launch_fused<W, P, 4>(w, w_scale, x, N, K, y, q_out, d_out, stream);
    case 5: return launch_fused<W, P, 5>(w, w_scale, x, N, K, y, q_out, d_out, stream);
    case 6: return launch_fused<W, P, 6>(w, w_scale, x, N, K, y, q_out, d_out, stream);
    case 7: return launch_fused<W, P, 7>(w, w_scale, x, N, K, y, q_out, d_out, stream);
    case 8: return launch_fused<W, P, 8>(w, w_scale, x, N, K, y, q_out, d_out, stream);
    default: return launch_fused<W, P, 9>(w, w_scale, x, N, K, y, q_out, d_out, stream);
  }
}

// Launch shape of the fused kernel, by measurement on the layer shapes (the per-block
// quantization of the row is the extra cost, so larger blocks pay off on small grids):
// short rows (at most 12 chunks) 4 wavefronts x 3-chunk batches (4864 x 896: 2.9 us
// against 3.1 with 4 x 5); fewer than 1024 tiles with long rows 16 x 3 (down 5120 x
// 17408: 13.3 us against 13.9 with 16 x 2 and 15.1 with 8 x 3), else 8 x 3 (QKV
// 7168 x 5120 / O 5120 x 5120: 6.7 / 6.5 us against 7.1 / 7.0 with 4 x 5); many tiles
// 8 x 5 (gate+up 34816 x 5120: 18.2 us against 18.4 with 4 x 5 and 8 x 3; 17.8 against 21.5
// with 16 x 3 on another box).  The layer
// step of the four took 44.1 us against 44.8 with the former 16 x 2 / 4 x 5 choice.
hipError_t launch_gemv_nvfp4_fused(const uint8_t* w, float w_scale, const float* x, int64_t N, int64_t K, float* y,
                                   int8_t* q_out, uint16_t* d_out, hipStream_t stream) {
  const int64_t ntiles = (N + 15) / 16;
  const int64_t nch = (K + 127) / 128;
  if (nch <= 12) return launch_fused_w<4, 3>(w, w_scale, x, N, K, y, q_out, d_out, stream);
  if (ntiles < 1024 && nch >= 64) return launch_fused_w<16, 3>(w, w_scale, x, N, K, y, q_out, d_out, stream);
  if (ntiles < 1024) return launch_fused_w<8, 3>(w, w_scale, x, N, K, y, q_out, d_out, stream);
  return launch_fused_w<8, 5>(w, w_scale, x, N, K, y, q_out, d_out, stream);
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
