// gemv_batch_f16.hip -- batched decode GEMV (2 <= M <= 16 tokens per launch), NVFP4
// weights x Q8_0 activations, on gfx950's fp16 matrix cores.
//
// What is computed ("HANDOFF: flint CPU optimization (Q4_1 + NVFP4)", section 3):
//     y[m][n] = S * sum_s UE4M3(scale[n][s]) * sum_{k in s} E2M1(code[n][k]) * d[m][k/32] * q[m][k].
//
// Both scales are folded into exact fp16 operands, so the matrix core accumulates the
// whole row and the vector unit never touches a partial product:
//  * weights: w16 = E2M1 * UE4M3 has at most 6 significant bits and lies in
//    [2^-10, 2688], so it is an exact binary16 value (v_cvt_scalef32_pk_f16_fp4, then
//    one v_pk_mul_f16 by the UE4M3 value);
//  * activations: d * q has at most 18 significant bits (11 of the binary16 d, 7 of
//    |q| <= 127), so it is exactly hi + lo with hi = fp16(d * q) and
//    lo = fma(d, q, -hi) (the difference is representable, so the fused result is
//    exact).  hi and lo become two columns of the fp16 operand: column j < 8 holds
//    token j's hi values, column j + 8 its lo values, and y[m] = S * (D[m] + D[m + 8]).
//  * hi overflows once |d * q| reaches 65520.  A 32-value block whose d is 512 or
//    more (|d * q| can then exceed the binary16 range) is left out of the main loop
//    and done by a second pass, taken only by wavefronts that met such a block, with
//    d / 256 (exact: a power of two, and d / 256 >= 2 stays normal) into a second
//    accumulator that is multiplied by 256 at the end.  So every finite activation is
//    handled exactly, and the main loop carries no extra work for it.
//
// One v_mfma_f32_16x16x32_f16 covers 16 weight rows x 32 k x 16 columns.  A wavefront's
// 16 B weight load per chunk (lane l = 16 g + r: row r, k = 32 g .. 32 g + 31 of the
// 128-k chunk) feeds four of them: MFMA t reads from lane l the codes k = 32 g + 8 t
// .. + 7, which is the operand's "k group g" -- the reduction index is only permuted,
// identically for both operands.  The activation operand of lane l (column l % 16, k
// group g) is therefore the 32 codes q[m][128 c + 32 g .. + 31] and their one scale
// d[m][4 c + g], read straight from global memory (the row is L2-resident: 16 bytes
// per lane, the other 16 from the partner lane of the same token) and expanded in
// registers.  The expansion (about 72 vector
// instructions per chunk) is shared by the T tiles a block owns, so a wavefront
// streams T KB of weights per chunk against one activation expansion.
//
// Block: W wavefronts, T consecutive 16-row tiles; wavefront v takes chunks
// v, v + W, ... through D register slots of loads (software pipelined: while one chunk
// is expanded and multiplied, the loads of the next D - 1 are in flight).  The W
// partial tiles are summed through LDS at the end.
//
// DEBUG instance (the integer per-16 sums of this kernel's data path): the same
// loads, expansions and fp16 MFMAs with unit scales (UE4M3 = 1, d = 1, so the hi
// column of a token is q and its lo column 0).  MFMA u of a chunk holds, in k group g,
// the 8 codes k = 32 g + 8 u .. + 7, i.e. part of subblock 2 g + (u >> 1); so per k
// group g and subblock half the activation operand is masked to group g and two
// MFMAs (u = 2 half, 2 half + 1) sum the 16 codes of subblock 2 g + half, exact in
// fp32.  A token's sum is its hi column plus its lo column (lanes l and l ^ 8),
// written as L = 2 E2M1 sums.  Each chunk is written by the one wavefront that owns it.
#include "nvq_device.h"

namespace nvq {

template <int T, int W, int D, int G, bool DEBUG>
__global__ __launch_bounds__(64 * W) void gemv_nvfp4_f16_kernel(const uint8_t* __restrict__ w, int64_t N, int K,
                                                                const int8_t* __restrict__ q,
                                                                const uint16_t* __restrict__ d16, int M,
                                                                float w_scale, float* __restrict__ y,
                                                                int32_t* __restrict__ isums) {
  constexpr int NT = 64 * W;
  __shared__ floatx4 red[W * T * 64];
  // the wavefront index is uniform (readfirstlane tells the compiler so, which keeps
  // the chunk loop's indices in scalar registers)
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int fr = lane & 15, fg = lane >> 4;
  const int nch = (K + 127) >> 7;
  const int nb = K >> 5;
  const int64_t ntiles = (N + 15) >> 4;
  const int64_t tile0 = (int64_t)blockIdx.x * T;

  // per-tile bases are wavefront-uniform; lane offsets are 32-bit, so the loads use
  // scalar base + vector offset addressing
  const uint8_t* wt[T];
  const uint8_t* st[T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const int64_t tile = tile0 + t < ntiles ? tile0 + t : ntiles - 1;
    wt[t] = w + tile * nch * 1024;
    st[t] = w + ntiles * nch * 1024 + tile * nch * 128;
  }
  const uint32_t wl = 16 * lane, sl = 2 * lane;
  // this lane's activation column in token group gi: token 8 gi + fr % 8 (columns of
  // absent tokens repeat the last token and are never stored), part hi (fr < 8) or
  // lo (fr >= 8)
  const bool lo_lane = fr >= 8;
  uint32_t qoff[G], doff[G];
#pragma unroll
  for (int gi = 0; gi < G; ++gi) {
    const int m = min(8 * gi + (fr & 7), M - 1);
    qoff[gi] = (uint32_t)m * (uint32_t)K;
    doff[gi] = (uint32_t)m * (uint32_t)nb;
  }

  // D load slots, each one chunk ahead of the next: slot j holds chunk c + W j.  The
  // hi and lo lanes of a token need the same 32 codes: each loads 16 of them (hi lanes
  // the first half, lo lanes the second) and takes the other half from its partner
  // lane (fr ^ 8) when the chunk is consumed.
  u32x4 qa[G][D], bw[D][T];
  uint32_t dv[G][D], bs[D][T];
  auto issue = [&](int j, int c) {
    // chunk index clamped (loads past the row's last chunk are never consumed); k
    // groups past the row's end (a last chunk of 64) read the row's last 32 codes and
    // get scale 0 when consumed, so they contribute nothing
    c = min(c, nch - 1);
    const int b = min(4 * c + fg, nb - 1);
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
      qa[gi][j] = *reinterpret_cast<const u32x4*>(q + (qoff[gi] + 32 * b + (lo_lane ? 16 : 0)));
      dv[gi][j] = DEBUG ? 0x3C00u : (uint32_t)d16[doff[gi] + b];  // DEBUG: d = 1
    }
#pragma unroll
    for (int t = 0; t < T; ++t) {
      bw[j][t] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wt[t] + (int64_t)c * 1024 + wl));
      bs[j][t] = __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(st[t] + (int64_t)c * 128 + sl));
    }
  };

  floatx4 acc[G][T];
#pragma unroll
  for (int gi = 0; gi < G; ++gi)
#pragma unroll
    for (int t = 0; t < T; ++t) acc[gi][t] = floatx4{0.f, 0.f, 0.f, 0.f};

  // one chunk of slot j with the token groups' activation scales dd[] (binary16 bits):
  // for each of the 4 k groups, the activation operand of every token group, then the
  // T weight operands (expanded once for all groups) and MFMAs into a[][]
  auto chunk = [&](int j, const uint32_t* dd, floatx4 (*a)[T]) {
    const half2_t z2 = {(_Float16)0.0f, (_Float16)0.0f};
    half2_t d2[G], dl2[G];
    u32x4 qlo[G], qhi[G];
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
      const _Float16 dh = __builtin_bit_cast(_Float16, (uint16_t)dd[gi]);
      d2[gi] = half2_t{dh, dh};
      dl2[gi] = lo_lane ? d2[gi] : z2;
      // the partner's 16 codes (row_ror:8 swaps lanes fr and fr ^ 8 of each row of 16)
      u32x4 oth;
#pragma unroll
      for (int i = 0; i < 4; ++i) oth[i] = (uint32_t)__builtin_amdgcn_mov_dpp((int)qa[gi][j][i], 0x128, 0xF, 0xF, false);
      qlo[gi] = lo_lane ? oth : qa[gi][j];
      qhi[gi] = lo_lane ? qa[gi][j] : oth;
    }
    half2_t s[T];  // the lane's two UE4M3 scales (low word of its 16-bit load), exact in fp16
#pragma unroll
    for (int t = 0; t < T; ++t) s[t] = DEBUG ? half2_t{(_Float16)1.0f, (_Float16)1.0f} : ue4m3x2_to_f16(bs[j][t]);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      half8_t B[G];
#pragma unroll
      for (int gi = 0; gi < G; ++gi) {
        const u32x4& qq = u < 2 ? qlo[gi] : qhi[gi];
        const uint32_t w0 = qq[2 * (u & 1)], w1 = qq[2 * (u & 1) + 1];
        half2_t x0, x1, x2, x3;
        i8x4_to_f16x4(w0, x0, x1);
        i8x4_to_f16x4(w1, x2, x3);
        // hi lanes: fma(q, d, -0) = fp16(d q); lo lanes: fma(q, d, -fp16(d q)) = lo
        const half2_t b0 = __builtin_elementwise_fma(x0, d2[gi], -(x0 * dl2[gi]));
        const half2_t b1 = __builtin_elementwise_fma(x1, d2[gi], -(x1 * dl2[gi]));
        const half2_t b2 = __builtin_elementwise_fma(x2, d2[gi], -(x2 * dl2[gi]));
        const half2_t b3 = __builtin_elementwise_fma(x3, d2[gi], -(x3 * dl2[gi]));
        B[gi] = half8_t{b0[0], b0[1], b1[0], b1[1], b2[0], b2[1], b3[0], b3[1]};
      }
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const half2_t sc = {s[t][u >> 1], s[t][u >> 1]};  // subblock 2g + (u >> 1)
        const uint32_t cw = bw[j][t][u];
        const half2_t p0 = e2m1x2_to_f16<0>(cw) * sc;
        const half2_t p1 = e2m1x2_to_f16<1>(cw) * sc;
        const half2_t p2 = e2m1x2_to_f16<2>(cw) * sc;
        const half2_t p3 = e2m1x2_to_f16<3>(cw) * sc;
        const half8_t A = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
#pragma unroll
        for (int gi = 0; gi < G; ++gi) a[gi][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, B[gi], a[gi][t], 0, 0, 0);
      }
    }
  };

  // DEBUG: the per-16 sums of slot j's chunk c (unit scales), written to isums
  auto chunk_sums = [&](int j, int c) {
    const int64_t nsb = K >> 4;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      // operands of MFMAs u = 2 half and 2 half + 1, as in chunk() with d = 1, UE4M3 = 1
      half8_t A[2][T], B[2][G];
#pragma unroll
      for (int uu = 0; uu < 2; ++uu) {
        const int u = 2 * half + uu;
#pragma unroll
        for (int gi = 0; gi < G; ++gi) {
          u32x4 oth;
#pragma unroll
          for (int i = 0; i < 4; ++i) oth[i] = (uint32_t)__builtin_amdgcn_mov_dpp((int)qa[gi][j][i], 0x128, 0xF, 0xF, false);
          const u32x4 qq = (u < 2) == lo_lane ? oth : qa[gi][j];  // hi lanes hold the first 16 codes
          half2_t x0, x1, x2, x3;
          i8x4_to_f16x4(qq[2 * (u & 1)], x0, x1);
          i8x4_to_f16x4(qq[2 * (u & 1) + 1], x2, x3);
          const half2_t one = {(_Float16)1.0f, (_Float16)1.0f}, z2 = {(_Float16)0.0f, (_Float16)0.0f};
          const half2_t dl = lo_lane ? one : z2;
          const half2_t b0 = __builtin_elementwise_fma(x0, one, -(x0 * dl));
          const half2_t b1 = __builtin_elementwise_fma(x1, one, -(x1 * dl));
          const half2_t b2 = __builtin_elementwise_fma(x2, one, -(x2 * dl));
          const half2_t b3 = __builtin_elementwise_fma(x3, one, -(x3 * dl));
          B[uu][gi] = half8_t{b0[0], b0[1], b1[0], b1[1], b2[0], b2[1], b3[0], b3[1]};
        }
#pragma unroll
        for (int t = 0; t < T; ++t) {
          const uint32_t cw = bw[j][t][u];
          const half2_t p0 = e2m1x2_to_f16<0>(cw), p1 = e2m1x2_to_f16<1>(cw);
          const half2_t p2 = e2m1x2_to_f16<2>(cw), p3 = e2m1x2_to_f16<3>(cw);
          A[uu][t] = half8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
        }
      }
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int64_t sb = 8 * (int64_t)c + 2 * g + half;
#pragma unroll
        for (int gi = 0; gi < G; ++gi)
#pragma unroll
          for (int t = 0; t < T; ++t) {
            floatx4 p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int uu = 0; uu < 2; ++uu) {
              const half8_t bm = fg == g ? B[uu][gi] : half8_t{};
              p = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[uu][t], bm, p, 0, 0, 0);
            }
            // column fr: token 8 gi + fr % 8, hi (fr < 8) or lo part; rows 4 fg + rr
            const int m = 8 * gi + fr;
            const int64_t row0 = (tile0 + t) * 16 + 4 * fg;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
              const float v = p[rr] + __shfl_xor(p[rr], 8);
              if (fr < 8 && m < M && row0 + rr < N && sb < nsb)
                isums[((int64_t)m * N + row0 + rr) * nsb + sb] = (int32_t)(2.0f * v);
            }
          }
      }
    }
  };

  // scales of slot j's chunk c for this lane (one per token group): 0 past the row's
  // end; blocks with d >= 512 are left out here (scale 0) and done by the second pass
  // below, which takes d / 256 for them and 0 for the others (act_scale_for_pass)
  auto scales = [&](int j, int c, bool second, uint32_t* dd) {
    bool any = false;
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
      const uint32_t d = 4 * c + fg < nb ? dv[gi][j] : 0u;
      any |= act_scale_big(d);
      dd[gi] = act_scale_for_pass(d, second ? 1 : 0);
    }
    return any;
  };

  // software pipeline: slot j is consumed, then refilled with the chunk D slots later,
  // so D chunks of loads stay in flight while one is computed
  uint64_t any_big = 0;
#pragma unroll
  for (int j = 0; j < D; ++j) issue(j, wave + W * j);
  for (int c = wave; c < nch; c += W * D) {
#pragma unroll
    for (int j = 0; j < D; ++j) {
      if (c + W * j < nch) {
        if constexpr (DEBUG) {
          chunk_sums(j, c + W * j);
        } else {
          uint32_t dd[G];
          any_big |= __builtin_amdgcn_ballot_w64(scales(j, c + W * j, false, dd));
          chunk(j, dd, acc);
        }
      }
      issue(j, c + W * (j + D));
    }
  }
  if constexpr (DEBUG) return;
  // blocks with |d| >= 512 (only for activations near the binary16 range): one more
  // pass over this wavefront's chunks into the accumulator that is scaled by 256
  if (any_big) {
    floatx4 accb[G][T];
#pragma unroll
    for (int gi = 0; gi < G; ++gi)
#pragma unroll
      for (int t = 0; t < T; ++t) accb[gi][t] = floatx4{0.f, 0.f, 0.f, 0.f};
    for (int c = wave; c < nch; c += W) {
      issue(0, c);
      uint32_t dd[G];
      (void)scales(0, c, true, dd);
      chunk(0, dd, accb);
    }
#pragma unroll
    for (int gi = 0; gi < G; ++gi)
#pragma unroll
      for (int t = 0; t < T; ++t) acc[gi][t] += 256.0f * accb[gi][t];
  }

  // reduce the W wavefronts' partial tiles, one token group at a time (so the LDS
  // buffer holds one group: T = 9 fits for two groups too); in token group gi, column
  // j < 8 + column j + 8 = token 8 gi + j
  const float* rf = reinterpret_cast<const float*>(red);
#pragma unroll
  for (int gi = 0; gi < G; ++gi) {
    if (gi > 0) __syncthreads();  // the previous group's sums are read
#pragma unroll
    for (int t = 0; t < T; ++t) red[(wave * T + t) * 64 + lane] = acc[gi][t];
    __syncthreads();
    for (int o = tid; o < 8 * 16 * T; o += NT) {
      const int j = o / (16 * T), rr = o % (16 * T);
      const int t = rr >> 4, r = rr & 15, mo = 8 * gi + j;
      const int64_t row = (tile0 + t) * 16 + r;
      if (mo >= M || row >= N) continue;
      const int l_hi = j + 16 * (r >> 2), l_lo = l_hi + 8, v = r & 3;
      float s = 0.0f;
#pragma unroll
      for (int ww = 0; ww < W; ++ww) {
        const int base = (ww * T + t) * 64;
        s += rf[(base + l_hi) * 4 + v] + rf[(base + l_lo) * 4 + v];
      }
      y[(int64_t)mo * N + row] = s * w_scale;
    }
  }
}

template <int T, int W, int D, int G>
static hipError_t launch_f16(const uint8_t* w, float w_scale, const int8_t* q, const uint16_t* d16, int M,
                             int64_t N, int64_t K, float* y, int32_t* isums, hipStream_t stream) {
  const int64_t ntiles = (N + 15) / 16;
  const unsigned blocks = (unsigned)((ntiles + T - 1) / T);
  if (isums)
    hipLaunchKernelGGL((gemv_nvfp4_f16_kernel<T, W, D, G, true>), dim3(blocks), dim3(64 * W), 0, stream, w, N,
                       (int)K, q, d16, M, w_scale, y, isums);
  else
    hipLaunchKernelGGL((gemv_nvfp4_f16_kernel<T, W, D, G, false>), dim3(blocks), dim3(64 * W), 0, stream, w, N,
                       (int)K, q, d16, M, w_scale, y, nullptr);
  return hipGetLastError();
}

template <int G>
static hipError_t launch_f16_group(int T, const uint8_t* w, float w_scale, const int8_t* q, const uint16_t* d16,
                                   int M, int64_t N, int64_t K, float* y, int32_t* isums, hipStream_t stream) {
  switch (T) {
    case 4: return launch_f16<4, 4, 2, G>(w, w_scale, q, d16, M, N, K, y, isums, stream);
    case 5: return launch_f16<5, 4, 2, G>(w, w_scale, q, d16, M, N, K, y, isums, stream);
    case 6: return launch_f16<6, 4, 2, G>(w, w_scale, q, d16, M, N, K, y, isums, stream);
    case 7: return launch_f16<7, 4, 2, G>(w, w_scale, q, d16, M, N, K, y, isums, stream);
    case 8: return launch_f16<8, 4, 2, G>(w, w_scale, q, d16, M, N, K, y, isums, stream);
    case 9: return launch_f16<9, 4, 2, G>(w, w_scale, q, d16, M, N, K, y, isums, stream);
    default: return launch_f16<2, 8, 2, G>(w, w_scale, q, d16, M, N, K, y, isums, stream);
  }
}

// Tiles per block for many tiles.  The vector work of a block per chunk is about
// 32 T + 72 G instructions (weights of T tiles + one activation expansion per token
// group), and a compute unit runs ceil(blocks / 256) blocks' worth of it, so the launch
// takes the T in 4 .. 9 that minimises
// ceil(ceil(tiles / T) / 256) * (32 T + 72 G).  Measured at M = 8: gate+up (2176
// tiles) 24.2 us with T = 3, 22.4 with T = 5 and 20.8-21.3 with T = 9 (one block per
// compute unit); N = 17408 (1088 tiles) 16.2 us with T = 3 and 12.8 with T = 5.  T = 3
// never wins this from 1024 tiles up (it did under the former choice between 3 and 4
// only), so it is not built.
static int tiles_per_block(int64_t ntiles, int G) {
  int best = 4;
  int64_t best_cost = -1;
  for (int t = 4; t <= 9; ++t) {
    const int64_t per_cu = ((ntiles + t - 1) / t + 255) / 256;
    const int64_t cost = per_cu * (32 * t + 72 * G);
    if (best_cost < 0 || cost < best_cost) best = t, best_cost = cost;
  }
  return best;
}

// Tokens in launches of at most 16, each streaming the weights once: up to 8 tokens
// as one group of MFMA columns, 9 to 16 as two groups that share every weight
// expansion.  Fewer than 1024 tiles (QKV, O, down at hidden 5120): 2 tiles x 8
// wavefronts x 2 slots, so the blocks keep enough loads in flight (3 slots measured
// 4-8 % slower); more: T tiles x 4 wavefronts x 2 slots (every wavefront resident at
// once).
hipError_t launch_gemv_nvfp4_batch_f16(const uint8_t* w, float w_scale, const int8_t* q, const uint16_t* d16,
                                       int64_t M, int64_t N, int64_t K, float* y, int32_t* isums,
                                       hipStream_t stream) {
  const int64_t ntiles = (N + 15) / 16;
  for (int64_t m0 = 0; m0 < M; m0 += 16) {
    const int mb = (int)(M - m0 < 16 ? M - m0 : 16);
    const int G = mb > 8 ? 2 : 1;
    const int T = ntiles < 1024 ? 0 : tiles_per_block(ntiles, G);
    const int8_t* qb = q + m0 * K;
    const uint16_t* db = isums ? nullptr : d16 + m0 * (K / 32);
    float* yb = isums ? nullptr : y + m0 * N;
    int32_t* ib = isums ? isums + m0 * N * (K / 16) : nullptr;
    const hipError_t e = G == 2 ? launch_f16_group<2>(T, w, w_scale, qb, db, mb, N, K, yb, ib, stream)
                                : launch_f16_group<1>(T, w, w_scale, qb, db, mb, N, K, yb, ib, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace nvq
