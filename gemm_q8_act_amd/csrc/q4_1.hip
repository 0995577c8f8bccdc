// q4_1.hip -- Q4_1 (and Q4_K, Q5_K, Q6_K, IQ4_XS) weights x Q8_0 activations on gfx950
// (GEMV and tiled MFMA).
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
// GEMM, M > 16 and K % 64 == 0: the int8 matrix cores sum c*q per 32-block exactly and
// the vector unit applies the block scales in fp32 (gemm_q4x_i8_kernel below); Q6_K,
// with one scale per 16 weights, takes both operands as two binary16 terms instead, so
// the fp16 matrix core accumulates whole rows (gemm_q4_1_f16x2_kernel).
//
// Q4_K (the same patch's "Q4_K" format; the llama.cpp 2-bit GGUF tutorial's GGML type
// table gives its block, 256 values in 144 bytes): a 256-weight super-block holds
// binary16 d and dmin, and each 32-weight sub-block j a 6-bit scale sc_j and a 6-bit
// min mn_j, weight = d*sc_j*c - dmin*mn_j.  Per 32-block that is a Q4_1 block with
// scale d*sc_j and offset -dmin*mn_j (each product exact in fp32: 11 x 6 significant
// bits), so the GEMV and integer-MFMA kernels run it with a format parameter that only
// changes where a block's (scale, offset) pair comes from (BlockScales).  Device layout:
// the codes as Q4_1 ([N][K/2], byte i = codes 2i low, 2i+1 high nibble), then one
// 16-byte header per (row, super-block): binary16 d, binary16 dmin, and the 16 6-bit
// fields sc_0..sc_7, mn_0..mn_7, field f at bits [6f, 6f + 6) of the 96-bit
// little-endian number in bytes 4..15.
//
// IQ4_XS (also named by the patch; 256 values in 136 bytes in the type table): a
// binary16 d per 256 weights, a 6-bit scale ls_j per 32 (used as ls_j - 32), and 4-bit
// codes that index a 16-entry int8 value table V, weight = d*(ls_j - 32)*V[c].  The
// same two kernels run it: per 32-block the scale d*(ls_j - 32) (exact in fp32) and no
// offset, the codes mapped through V by v_perm_b32 lookups (lut16) -- int8 values for
// v_dot4 in the GEMV and for the int8 operands of the GEMM.  Layout:
// the codes as Q4_1, then one 8-byte header per (row, super-block): binary16 d and the
// eight 6-bit ls_j as a little-endian 48-bit number.  V is a call argument.
#include <algorithm>
#include <type_traits>

#include "ksplit.h"
#include "nvq_device.h"
#include "nvq_launch.h"

namespace nvq {

constexpr int kQ41MaxUPL = 10;
// Row groups per wavefront (rows = RG x 64 / LPR): fewer for one token, where the
// kernel is latency-bound and more wavefronts in flight pay (N = K = 4096 at M = 1: Q4_1
// 4.39 us with 2 against 4.53 with 4; Q4_K 4.46 against 4.68), and one for IQ4_XS,
// whose table lookups make each unit's vector work ~6x longer (5.2 us against 7.3 with 4).
// fmt: the weight format (NVQ_FMT_* value, 3 = IQ4_XS).
__host__ __device__ constexpr int q41_rg(int upl, bool multi, int fmt) {
  return fmt == 3 || fmt == 5 ? 1 : (upl >= 7 ? 1 : (upl >= 4 || !multi ? 2 : 4));
}
// tokens whose activations a GEMV wavefront holds at once (8 UPL registers each)
__host__ __device__ constexpr int q41_tb(int upl) { return upl <= 2 ? 4 : (upl <= 4 ? 2 : 1); }

// 8 unsigned 4-bit codes (byte i: code 2i low nibble, 2i+1 high) dotted with the
// matching even / odd activation codes.
__device__ __forceinline__ int dot8_u4(uint32_t c, uint32_t qe, uint32_t qo, int acc) {
  acc = dot4(c & 0x0F0F0F0Fu, qe, acc);
  acc = dot4((c >> 4) & 0x0F0F0F0Fu, qo, acc);
  return acc;
}

// weight formats of the kernels below (the NVQ_FMT_* values)
constexpr int kQ41 = 1, kQ4K = 2, kIQ4 = 3, kQ5K = 4, kQ6K = 5;

// 4 bits (x & 15) spread to the low bit of each byte: bit t -> bit 8 t (the four
// shifted copies x, x << 7, x << 14, x << 21 overlap in no bit, so the product adds
// without carries)
__device__ __forceinline__ uint32_t spread4(uint32_t x) { return ((x & 15u) * 0x00204081u) & 0x01010101u; }

// The even (ce) and odd (co) code bytes of word i (codes 8 i .. 8 i + 7 of a 32-block)
// from the packed low nibbles cwi and the format's high-bit words h: Q5_K adds the
// fifth bit (h[0]), Q6_K the fifth and sixth (h[0], h[1]); bit e of a high-bit word
// belongs to even code 2 e, bit 16 + e to odd code 2 e + 1.
template <int HW>
__device__ __forceinline__ void code_bytes(uint32_t cwi, int i, const uint32_t* h, uint32_t& ce, uint32_t& co) {
  ce = cwi & 0x0F0F0F0Fu;
  co = (cwi >> 4) & 0x0F0F0F0Fu;
#pragma unroll
  for (int b = 0; b < HW; ++b) {
    ce |= spread4(h[b] >> (4 * i)) << (4 + b);
    co |= spread4(h[b] >> (16 + 4 * i)) << (4 + b);
  }
}

// IQ4_XS: 4 values of a 16-entry byte table (words t0..t3 = entries 0-3, .., 12-15) for
// 4 index bytes idx (each 0..15): entries 0..7 and 8..15 by one v_perm_b32 each, then
// a third picks per byte by the index's bit 3
__device__ __forceinline__ uint32_t lut16(uint32_t idx, const u32x4& t) {
  const uint32_t i7 = idx & 0x07070707u;
  const uint32_t lo = perm(t[1], t[0], i7);
  const uint32_t hi = perm(t[3], t[2], i7);
  return perm(hi, lo, 0x03020100u | ((idx & 0x08080808u) >> 1));
}
// sum over 8 codes (one packed word) of table[code] * q: the int8 table values against
// the even / odd activation codes
__device__ __forceinline__ int iq4_dot8(uint32_t c, uint32_t qe, uint32_t qo, int acc, const u32x4& t) {
  acc = dot4(lut16(c & 0x0F0F0F0Fu, t), qe, acc);
  acc = dot4(lut16((c >> 4) & 0x0F0F0F0Fu, t), qo, acc);
  return acc;
}

// Q4_K: the (scale, offset) of sub-block j of the super-block with header h (see the
// layout above), as float32 (both products exact)
__device__ __forceinline__ void q4k_block_scales(const u32x4& h, int j, float& dw, float& mw) {
  const uint64_t lo = (uint64_t)h[2] << 32 | h[1], hi = (uint64_t)h[3] << 32 | h[2];
  const uint32_t sc = (uint32_t)(j < 6 ? lo >> (6 * j) : hi >> (6 * j - 32)) & 63u;
  const uint32_t mn = (uint32_t)(hi >> (16 + 6 * j)) & 63u;  // field 8 + j (bit 48 + 6 j >= 32)
  dw = f16_bits_to_f32((uint16_t)(h[0] & 0xFFFFu)) * (float)sc;
  mw = -(f16_bits_to_f32((uint16_t)(h[0] >> 16)) * (float)mn);
}

// The scale source of a weight format: Q4_1 one 4-byte (d, m) binary16 pair per
// 32-block after the codes; Q4_K one 16-byte header per 256-block after the codes;
// IQ4_XS one 8-byte header per 256-block (binary16 d, then the eight 6-bit sub-block
// scales ls_j as a little-endian 48-bit number; scale d * (ls_j - 32), no offset).
// kBound bounds |weight| / |scale| + |offset| / |scale| per block (the code range).
template <int FMT>
struct BlockScales {
  static constexpr bool kKq = FMT == kQ4K || FMT == kQ5K;  // the 16-byte K-quant header
  static constexpr int kWords = kKq ? 4 : (FMT == kIQ4 ? 2 : 1);
  // bound of |code value| (Q4: 15, Q5_K: 31, Q6_K: |c - 32| <= 32, IQ4_XS: |V| <= 128)
  static constexpr float kBound = FMT == kIQ4 ? 128.0f : (FMT == kQ5K ? 31.0f : (FMT == kQ6K ? 32.0f : 15.0f));
  const uint32_t* base;  // first word of the scale region
  int64_t per_row;       // words per weight row (Q6_K: bytes of int8 scales per row)
  const uint16_t* dbase;  // Q6_K: the binary16 d of each 256-block, [N][K/256]
  __device__ BlockScales(const uint8_t* w, int64_t N, int K)
      : base(reinterpret_cast<const uint32_t*>(w + N * (int64_t)(K >> 1))),
        per_row(kKq ? (int64_t)(K >> 8) * 4
                    : (FMT == kIQ4 ? (int64_t)(K >> 8) * 2 : (FMT == kQ6K ? (int64_t)(K >> 4) : (int64_t)(K >> 5)))),
        dbase(FMT == kQ6K ? reinterpret_cast<const uint16_t*>(w + N * (int64_t)(K >> 1) + N * (int64_t)(K >> 4) +
                                                              N * (int64_t)(K >> 2))
                          : nullptr) {}
  // the raw words that hold 32-block b of a row (Q6_K: its two int8 scales in bits
  // 0..15, the super-block's binary16 d in bits 16..31)
  __device__ __forceinline__ void load(int64_t row, int64_t b, uint32_t* v) const {
    if constexpr (FMT == kQ6K) {
      const uint16_t pair = reinterpret_cast<const uint16_t*>(reinterpret_cast<const uint8_t*>(base) + row * per_row)[b];
      v[0] = (uint32_t)pair | ((uint32_t)dbase[row * (per_row >> 4) + (b >> 3)] << 16);
    } else if constexpr (kKq) {
      const u32x4 h = *reinterpret_cast<const u32x4*>(base + row * per_row + 4 * (b >> 3));
      v[0] = h[0]; v[1] = h[1]; v[2] = h[2]; v[3] = h[3];
    } else if constexpr (FMT == kIQ4) {
      const u32x2 h = *reinterpret_cast<const u32x2*>(base + row * per_row + 2 * (b >> 3));
      v[0] = h[0]; v[1] = h[1];
    } else {
      v[0] = base[row * per_row + b];
    }
  }
  // (scale, offset) of 32-block b from its raw words; Q6_K: the larger of its two
  // 16-scales and no offset (what bounds the block; the products use decode_half)
  __device__ __forceinline__ static void decode(const uint32_t* v, int64_t b, float& dw, float& mw) {
    if constexpr (FMT == kQ6K) {
      const float d = f16_bits_to_f32((uint16_t)(v[0] >> 16));
      const int s0 = (int8_t)(v[0] & 0xFFu), s1 = (int8_t)((v[0] >> 8) & 0xFFu);
      dw = d * (float)max(abs(s0), abs(s1));
      mw = 0.0f;
    } else if constexpr (kKq) {
      q4k_block_scales(u32x4{v[0], v[1], v[2], v[3]}, (int)(b & 7), dw, mw);
    } else if constexpr (FMT == kIQ4) {
      const uint64_t f = (uint64_t)v[1] << 16 | (v[0] >> 16);  // the 48 bits of ls_0 .. ls_7
      const int ls = (int)((f >> (6 * (b & 7))) & 63u);
      dw = f16_bits_to_f32((uint16_t)(v[0] & 0xFFFFu)) * (float)(ls - 32);
      mw = 0.0f;
    } else {
      dw = f16_bits_to_f32((uint16_t)(v[0] & 0xFFFFu));
      mw = f16_bits_to_f32((uint16_t)(v[0] >> 16));
    }
  }
  // Q6_K: the scale d * sc of 16-block half (0, 1) of the 32-block (exact in fp32)
  __device__ __forceinline__ static float decode_half(const uint32_t* v, int half) {
    const int sc = (int8_t)((v[0] >> (8 * half)) & 0xFFu);
    return f16_bits_to_f32((uint16_t)(v[0] >> 16)) * (float)sc;
  }
};

// The high-bit words of Q5_K (one per 32-block: the codes' fifth bits) and Q6_K (two:
// fifth and sixth bits), row-major after the scale region.
template <int FMT>
struct HighBits {
  static constexpr int kHW = FMT == kQ5K ? 1 : (FMT == kQ6K ? 2 : 0);
  static constexpr int kSlots = kHW > 0 ? kHW : 1;  // register slots (unused without high bits)
  const uint32_t* base;
  int64_t per_row;  // words per weight row
  __device__ HighBits(const uint8_t* w, int64_t N, int K)
      : base(reinterpret_cast<const uint32_t*>(w + N * (int64_t)(K >> 1) + N * (int64_t)(K >> 4))),
        per_row((int64_t)(K >> 5) * kHW) {}
  __device__ __forceinline__ void load(int64_t row, int64_t b, uint32_t* h) const {
    if constexpr (kHW == 1) {
      h[0] = base[row * per_row + b];
    } else if constexpr (kHW == 2) {
      const u32x2 t = *reinterpret_cast<const u32x2*>(base + row * per_row + 2 * b);
      h[0] = t[0];
      h[1] = t[1];
    } else {
      h[0] = 0u;
    }
  }
};

template <int FMT, int LPR, int UPL, bool MULTI, bool DEBUG>
__global__ __launch_bounds__(256) void gemv_q4_1_m1_kernel(const uint8_t* __restrict__ w,
                                                           int64_t N, int K,
                                                           const int8_t* __restrict__ q,
                                                           const uint16_t* __restrict__ d16,
                                                           const int16_t* __restrict__ bsum16,
                                                           float* __restrict__ y,
                                                           int32_t* __restrict__ isums, int M, u32x4 vtab) {
  constexpr int RG = q41_rg(UPL, MULTI, FMT);
  constexpr int RPG = 64 / LPR;
  constexpr int RPW = RPG * RG;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int sub = lane % LPR;
  const int slot = lane / LPR;
  const int units = K >> 5;
  const int64_t crow = K >> 1;
  const int64_t nb = K >> 5;
  const BlockScales<FMT> bsc(w, N, K);
  constexpr int PW = BlockScales<FMT>::kWords;
  const HighBits<FMT> hbits(w, N, K);
  constexpr int HW = HighBits<FMT>::kHW, HS = HighBits<FMT>::kSlots;
  const int64_t row0 = ((int64_t)blockIdx.x * 4 + wave) * RPW;

  uint4 cw[RG][UPL];
  uint32_t pw[RG][UPL][PW];  // raw scale words of each unit's 32-block (not read for the debug sums)
  uint32_t hw[RG][UPL][HS];  // Q5_K / Q6_K: the unit's high-bit words
#pragma unroll
  for (int r = 0; r < RG; ++r) {
    const int64_t row = row0 + r * RPG + slot;
#pragma unroll
    for (int j = 0; j < UPL; ++j) {
      const int u = sub + LPR * j;
      if (row < N && u < units) {
        cw[r][j] = *reinterpret_cast<const uint4*>(w + row * crow + 16 * (int64_t)u);
        if (!DEBUG) bsc.load(row, u, pw[r][j]);
        else for (int e = 0; e < PW; ++e) pw[r][j][e] = 0u;
        if (HW > 0) hbits.load(row, u, hw[r][j]);
        else hw[r][j][0] = 0u;
      } else {
        cw[r][j] = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
        for (int e = 0; e < PW; ++e) pw[r][j][e] = 0u;
#pragma unroll
        for (int e = 0; e < HS; ++e) hw[r][j][e] = 0u;
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
            // IQ4_XS and Q6_K have no offset term (and take no bsum16)
            bs[tb][j] = FMT == kIQ4 || FMT == kQ6K
                            ? 0.0f
                            : (float)((int)bsum16[m * 2 * nb + 2 * u] + (int)bsum16[m * 2 * nb + 2 * u + 1]);
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
          int i0, i1;
          if constexpr (FMT == kIQ4) {  // table values of the codes
            i0 = iq4_dot8(cw[r][j].y, qe[tb][j][1], qo[tb][j][1], iq4_dot8(cw[r][j].x, qe[tb][j][0], qo[tb][j][0], 0, vtab), vtab);
            i1 = iq4_dot8(cw[r][j].w, qe[tb][j][3], qo[tb][j][3], iq4_dot8(cw[r][j].z, qe[tb][j][2], qo[tb][j][2], 0, vtab), vtab);
          } else if constexpr (HW > 0) {
            // 5- or 6-bit codes c (0..63 fit a signed byte); Q6_K's values are c - 32: the
            // bytes 0xE0 (-32) dotted with the same activation codes add -32 sum q
            const uint32_t cws[4] = {cw[r][j].x, cw[r][j].y, cw[r][j].z, cw[r][j].w};
            int is[2] = {0, 0};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              uint32_t ce, co;
              code_bytes<HW>(cws[i], i, hw[r][j], ce, co);
              int a = dot4(ce, qe[tb][j][i], is[i >> 1]);
              a = dot4(co, qo[tb][j][i], a);
              if constexpr (FMT == kQ6K) {
                a = dot4(0xE0E0E0E0u, qe[tb][j][i], a);
                a = dot4(0xE0E0E0E0u, qo[tb][j][i], a);
              }
              is[i >> 1] = a;
            }
            i0 = is[0];
            i1 = is[1];
          } else {
            i0 = dot8_u4(cw[r][j].y, qe[tb][j][1], qo[tb][j][1], dot8_u4(cw[r][j].x, qe[tb][j][0], qo[tb][j][0], 0));
            i1 = dot8_u4(cw[r][j].w, qe[tb][j][3], qo[tb][j][3], dot8_u4(cw[r][j].z, qe[tb][j][2], qo[tb][j][2], 0));
          }
          if (DEBUG) {
            const int u = sub + LPR * j;
            if (row < N && u < units) {
              isums[(m * N + row) * (K >> 4) + 2 * u] = i0;
              isums[(m * N + row) * (K >> 4) + 2 * u + 1] = i1;
            }
          } else if constexpr (FMT == kQ6K) {
            // one scale per 16-block half
            const float dw0 = BlockScales<FMT>::decode_half(pw[r][j], 0);
            const float dw1 = BlockScales<FMT>::decode_half(pw[r][j], 1);
            acc = fmaf(da[tb][j], fmaf(dw0, (float)i0, dw1 * (float)i1), acc);
          } else {
            float dw, mw;
            BlockScales<FMT>::decode(pw[r][j], sub + LPR * j, dw, mw);
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
                            const int16_t*, float*, int32_t*, int, u32x4);
template <int FMT, int LPR, bool MULTI, bool DEBUG>
gemv_q41_fn pick_q41(int upl) {
  switch (upl) {
    case 1: return gemv_q4_1_m1_kernel<FMT, LPR, 1, MULTI, DEBUG>;
    case 2: return gemv_q4_1_m1_kernel<FMT, LPR, 2, MULTI, DEBUG>;
    case 3: return gemv_q4_1_m1_kernel<FMT, LPR, 3, MULTI, DEBUG>;
    case 4: return gemv_q4_1_m1_kernel<FMT, LPR, 4, MULTI, DEBUG>;
    case 5: return gemv_q4_1_m1_kernel<FMT, LPR, 5, MULTI, DEBUG>;
    case 6: return gemv_q4_1_m1_kernel<FMT, LPR, 6, MULTI, DEBUG>;
    case 7: return gemv_q4_1_m1_kernel<FMT, LPR, 7, MULTI, DEBUG>;
    case 8: return gemv_q4_1_m1_kernel<FMT, LPR, 8, MULTI, DEBUG>;
    case 9: return gemv_q4_1_m1_kernel<FMT, LPR, 9, MULTI, DEBUG>;
    case 10: return gemv_q4_1_m1_kernel<FMT, LPR, 10, MULTI, DEBUG>;
    default: return nullptr;
  }
}
// one token (or the debug sums) at a time, or TB tokens per pass
template <int FMT, int LPR>
gemv_q41_fn pick_q41_for(int upl, bool multi, bool debug) {
  if (debug) return pick_q41<FMT, LPR, false, true>(upl);
  return multi ? pick_q41<FMT, LPR, true, false>(upl) : pick_q41<FMT, LPR, false, false>(upl);
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

// rows this GEMV kernel takes (at most kQ41MaxUPL 32-blocks per lane at 64 lanes per row)
static bool q41_gemv_fits(int64_t K) {
  int lpr = 0, upl = 0;
  gemv_m1_config(K, &lpr, &upl);
  return lpr != 0;
}

template <int FMT>
static hipError_t launch_gemv_q4x(const uint8_t* w, const int8_t* q, const uint16_t* d16, const int16_t* bsum16,
                                  int64_t M, int64_t N, int64_t K, float* y, int32_t* isums, hipStream_t stream,
                                  u32x4 vtab = u32x4{0u, 0u, 0u, 0u}) {
  const bool debug = isums != nullptr;
  int lpr = 0, upl = 0;
  gemv_m1_config(K, &lpr, &upl);
  gemv_q41_fn fn = nullptr;
  const bool multi = M > 1;
  if (lpr == 64) fn = pick_q41_for<FMT, 64>(upl, multi, debug);
  if (lpr == 32) fn = pick_q41_for<FMT, 32>(upl, multi, debug);
  if (lpr == 16) fn = pick_q41_for<FMT, 16>(upl, multi, debug);
  if (!fn) return hipErrorInvalidValue;
  const int64_t rows_per_block = 4 * (64 / lpr) * q41_rg(upl, multi && !debug, FMT);
  const int64_t grid = (N + rows_per_block - 1) / rows_per_block;
  hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(256), 0, stream, w, N, (int)K, q, d16, bsum16,
                     y, isums, (int)M, vtab);
  return hipGetLastError();
}

hipError_t launch_gemv_q4_1(const uint8_t* w, const int8_t* q, const uint16_t* d16,
                            const int16_t* bsum16, int64_t M, int64_t N, int64_t K, float* y,
                            int32_t* isums, hipStream_t stream) {
  // very long rows: the tiled kernel handles any K
  if (!q41_gemv_fits(K)) return launch_q41_tiled(w, q, d16, bsum16, M, N, K, y, isums, stream);
  return launch_gemv_q4x<kQ41>(w, q, d16, bsum16, M, N, K, y, isums, stream);
}

// ---------------------------------------------------------------------------------
// Two-term fp16 kernel (K % 64 == 0), written for Q4_1 and run for Q6_K, whose one
// scale per 16 weights suits it better than the integer-MFMA kernel below (which would
// need two half-zeroed MFMAs and twice the vector work per 32-block); every format
// can still instantiate it.  The weight w = d*c + m (binary16 d, m;
// c in 0..15) is formed in fp32 as w' = 2^s * w (one rounding) and split into
// hi = fp16(w') and lo = fp16(w' - hi).  The power of two 2^s is chosen per weight row
// (over the k range of the work item) from the bound |m| + 15|d| of its blocks so
// that |w'| < 2^15: hi never overflows and lo is a normal binary16 number unless
// |w'| < 2^-3, so hi + lo = w' to 2^-23 |w'|, or to 2^-25 absolute, i.e. 2^-39 of the
// row's largest weight.  The activation is split exactly as in the NVFP4 large-M
// kernel (d*q = hi + lo; blocks with d >= 512 go through the same second pass with
// d / 256).  The matrix core then accumulates whole rows of
//     W'.A = Wh.Ah + Wh.Al + Wl.Ah (+ Wl.Al, dropped: at most 2^-22 |W.A|),
// three MFMA passes, with no per-block vector work; the offset term m * sum(a) is
// inside W, and the result is multiplied by 2^-s (exact).  Error per output: a few
// 2^-22 of sum |w*a| plus float32 accumulation, far inside the 1e-5 bound.
//
// Block: 512 threads, WN x WM wavefronts, each a (32 TN) x (32 TM) tile of
// v_mfma_f32_32x32x16_f16 products; block tile BN = 32 WN TN weight rows by
// BM = 32 WM TM tokens (256 x 64 for 16 < M <= 64, 128 x 128 up to M = 128,
// 128 x 256 above).  LDS holds two 64-k stages: the two weight planes (fp16 hi,
// lo), the activation codes and their binary16 scales; each wavefront splits its
// activation fragments in registers.  With 128 or 256 tokens per tile the codes are
// staged already converted to binary16 (one conversion per block instead of one per
// wavefront column that reads them; the 256 x 64 tile's two stages have no room for
// it).  Work items and the ordered K-split reduction follow the NVFP4 large-M kernel.
//
// DEBUG instance (the integer per-16 sums sum c * q of this kernel's data path): the
// same staging and MFMAs with d = 1 and m = 0 for every weight block and d = 1 for
// every activation block.  The row bound is then 15, so w' = 2^11 c (exact in
// binary16, lo = 0) and the activation split is hi = q, lo = 0; the three MFMAs of a
// 16-k half with a zero accumulator give 2^11 sum c * q, exact in fp32 (every partial
// sum is a multiple of 2^11 below 2^26), and the row factor 2^-11 makes it an integer.
// IQ4_XS: the bound is 128, so w' = 2^7 V[c] (|V| <= 128: exact in binary16), and the
// sums 2^7 sum V[c] * q (below 2^25) are exact the same way.
// ---------------------------------------------------------------------------------
namespace {
constexpr int kQThreads = 512;
constexpr int kQLRW = 72;  // halves per LDS weight row (64 k + 8 pad)
constexpr int kQLRA = 72;  // codes per LDS activation row (64 + 8 pad)

template <int WN_, int WM_, int TN_, int TM_>
struct Q41Cfg {
  static constexpr int WN = WN_, WM = WM_, TN = TN_, TM = TM_;
  static constexpr int BN = 32 * WN * TN, BM = 32 * WM * TM;
  static constexpr int kAcc = 16 * TN * TM;  // fp32 accumulators per thread
  // A16: activation codes staged as binary16 values (converted once per block rather
  // than once per wavefront that reads them) where the two LDS stages have room
  static constexpr bool A16 = BM >= 128;
  static constexpr int kStageW = BN * kQLRW * 2, kStageA = BM * kQLRA * (A16 ? 2 : 1), kStageD = BM * 4;
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
// The integer-MFMA kernel takes 128 x 128 tiles up to M = 512 (half the K-split parts
// of the 128 x 256 tile: N = K = 4096, M = 256 / 512: 35.7 / 52.1 us against 37.9 /
// 53.0), the two-term kernel (Q6_K) only up to M = 128 (at M = 512: 72.9 us against 67.4)
constexpr int kI8M128Max = 512, kF16M128Max = 128;
enum Q41Path { kQ41Gemv, kQ41Tiled, kQ41Mid, kQ41M128, kQ41Big };
Q41Path q41_path(int64_t M, int64_t K) {
  if (M <= kQ41GemvMaxM) return kQ41Gemv;
  if (K % 64 != 0) return kQ41Tiled;
  if (M <= 64) return kQ41Mid;
  return M <= kI8M128Max ? kQ41M128 : kQ41Big;
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

template <class C, int FMT, bool DEBUG>
__global__ __launch_bounds__(512, 1) void gemm_q4_1_f16x2_kernel(const uint8_t* __restrict__ w, int64_t N, int K,
                                                                 const int8_t* __restrict__ q,
                                                                 const uint16_t* __restrict__ d16, int64_t M,
                                                                 float* __restrict__ y, float* __restrict__ part_ws,
                                                                 int32_t* __restrict__ isums, KSplitPlan plan,
                                                                 u32x4 vtab) {
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
  const int nb32 = K >> 5;      // activation scales per token row
  const BlockScales<FMT> bsc(w, N, K);
  constexpr int PW = BlockScales<FMT>::kWords;
  const HighBits<FMT> hbits(w, N, K);
  constexpr int HW = HighBits<FMT>::kHW, HS = HighBits<FMT>::kSlots;

  // staging task of this thread: CPT weight codes of row wrow at k-offset CPT wq of
  // the stage, all in one 32-block, with that block's (d, m); ABT activation codes of
  // row arow; for tid < 2 BM one activation scale.  Rows beyond N / M are clamped to
  // valid memory and their results never stored.
  const int wrow = tid / TPR, wq = tid % TPR;
  const int64_t wr = min(n0 + wrow, N - 1);
  const uint8_t* __restrict__ wbase = w + wr * crow + (CPT / 2) * wq;
  const int wblk = (CPT * wq) / 32;  // this thread's 32-block within a 64-k stage
  const int arow = tid / APR, aoff = ABT * (tid % APR);
  const int8_t* __restrict__ abase = q + min(m0 + arow, M - 1) * K + aoff;
  const bool dtask = 2 * BM >= kQThreads || tid < 2 * BM;
  const int drow = tid % BM, dblk = (tid / BM) & 1;
  const uint16_t* __restrict__ dbase = DEBUG ? nullptr : d16 + min(m0 + drow, M - 1) * nb32 + dblk;
  bool anybig = false;  // this thread staged an activation scale d >= 512
  struct Stage { Words<ABT / 4> a; Words<CPT / 8> wc; uint32_t dm[PW]; uint32_t hb[HS]; uint32_t dr; int blk; };
  // (scale, offset) of a staged 32-block; DEBUG: d = 1, m = 0 for every weight block
  auto block_scales = [&](const uint32_t* v, int64_t b, float& dwf, float& mwf) {
    if constexpr (DEBUG) {
      dwf = 1.0f;
      mwf = 0.0f;
    } else {
      BlockScales<FMT>::decode(v, b, dwf, mwf);
    }
  };

  // row scale 2^s: the largest bound |m| + 15|d| of this row's blocks in [t0, t1),
  // taken by the TPR threads that stage the row, placed in [2^14, 2^15).  A zero row
  // takes s = 0; a non-finite d or m gives a non-finite row anyway.
  float bmax = 0.0f;
#pragma unroll 4
  for (int b = 2 * t0 + wq; b < 2 * t1; b += TPR) {
    uint32_t v[PW] = {};
    if (!DEBUG) bsc.load(wr, b, v);
    float dwf, mwf;
    block_scales(v, b, dwf, mwf);
    bmax = fmaxf(bmax, fabsf(mwf) + BlockScales<FMT>::kBound * fabsf(dwf));
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
    x.blk = 2 * t + wblk;
    if (!DEBUG) bsc.load(wr, x.blk, x.dm);
    if (HW > 0) hbits.load(wr, x.blk, x.hb);
    x.a = load_words<ABT / 4>(abase + 64 * t);
    if constexpr (DEBUG) x.dr = 0x3C00u;  // d = 1
    else x.dr = dtask ? dbase[2 * t] : 0u;
  };
  // pass 0: the main pass (activation blocks with d >= 512 get d = 0); pass 1: those
  // blocks only, with d / 256
  auto lstore = [&](int b, const Stage& x, int pass) {
    uint8_t* st = smem + b * C::kStage;
    _Float16* lh = reinterpret_cast<_Float16*>(st);
    _Float16* ll = reinterpret_cast<_Float16*>(st + C::kStageW);
    uint8_t* la = st + 2 * C::kStageW;
    uint16_t* ld = reinterpret_cast<uint16_t*>(st + 2 * C::kStageW + C::kStageA);
    float dwf, mwf;
    block_scales(x.dm, x.blk, dwf, mwf);
    float dw = rscale * dwf;
    // IQ4_XS: the weight is dw * table[c]; the table is read as table + 128 (bytes
    // 0..255, exact floats), so w = fma(dw, table[c] + 128, -128 dw): one rounding of
    // the exact dw * table[c], as the Q4 formats' fma(dw, c, mw)
    float mw = FMT == kIQ4 ? -128.0f * dw : rscale * mwf;
    // Q5_K / Q6_K: this thread's high bits of its CPT codes (even codes from bit
    // ebase of a high-bit word, odd codes from bit 16 + ebase)
    const int ebase = ((CPT * wq) & 31) >> 1;
    uint32_t he[HS], ho[HS];
#pragma unroll
    for (int b = 0; b < HS; ++b) {
      he[b] = x.hb[b] >> ebase;
      ho[b] = x.hb[b] >> (16 + ebase);
    }
#pragma unroll
    for (int h = 0; h < CPT / 8; ++h) {
      const uint32_t cw = x.wc.v[h];
      if constexpr (FMT == kQ6K) {
        // the 16-block half of these 8 codes: w = d sc (c - 32) = fma(dw, c, -32 dw),
        // exact in fp32 (d sc c has at most 11 + 7 + 6 significant bits)
        const int half = ((CPT * wq + 8 * h) >> 4) & 1;
        dw = rscale * (DEBUG ? 1.0f : BlockScales<FMT>::decode_half(x.dm, half));
        mw = -32.0f * dw;
      }
      uint32_t ve = 0u, vo = 0u;  // IQ4_XS: biased table values of the even / odd codes
      if constexpr (FMT == kIQ4) {
        const u32x4 tb = vtab ^ u32x4{0x80808080u, 0x80808080u, 0x80808080u, 0x80808080u};
        ve = lut16(cw & 0x0F0F0F0Fu, tb);
        vo = lut16((cw >> 4) & 0x0F0F0F0Fu, tb);
      }
      half8_t vh, vl;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        // byte j/2 of the codes: code 2i low nibble, 2i+1 high
        uint32_t ci = (cw >> (4 * j)) & 0xFu;
#pragma unroll
        for (int b = 0; b < HW; ++b) ci |= (((j & 1 ? ho[b] : he[b]) >> (4 * h + (j >> 1))) & 1u) << (4 + b);
        const float c = FMT == kIQ4 ? (float)(((j & 1 ? vo : ve) >> (8 * (j >> 1))) & 0xFFu) : (float)ci;
        const float wf = fmaf(dw, c, mw);
        const _Float16 hi = (_Float16)wf;
        vh[j] = hi;
        vl[j] = (_Float16)(wf - (float)hi);
      }
      *reinterpret_cast<half8_t*>(lh + wrow * LRW + CPT * wq + 8 * h) = vh;
      *reinterpret_cast<half8_t*>(ll + wrow * LRW + CPT * wq + 8 * h) = vl;
    }
    if constexpr (C::A16) {
#pragma unroll
      for (int v = 0; v < ABT / 4; v += 2) {
        half2_t p0, p1, p2, p3;
        i8x4_to_f16x4(x.a.v[v], p0, p1);
        i8x4_to_f16x4(x.a.v[v + 1], p2, p3);
        *reinterpret_cast<half8_t*>(reinterpret_cast<_Float16*>(la) + arow * LRA + aoff + 4 * v) =
            half8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
      }
    } else {
      store_words<ABT / 4>(la + arow * LRA + aoff, x.a);
    }
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
  // a fragment's activation codes: 8 binary16 values (A16) or 8 int8 codes
  using Raw = std::conditional_t<C::A16, half8_t, uint2>;
  struct Frag { half8_t ah[2][TN], al[2][TN]; Raw raw[2][TM]; uint32_t dd[TM]; };
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
      for (int h = 0; h < 2; ++h) {
        const int e = r * LRA + 32 * u + 16 * h + fk;  // element offset in the activation plane
        if constexpr (C::A16) f.raw[h][j] = *reinterpret_cast<const Raw*>(reinterpret_cast<const _Float16*>(la) + e);
        else f.raw[h][j] = *reinterpret_cast<const Raw*>(la + e);
      }
    }
  };
  const float* rinv = reinterpret_cast<const float*>(smem + 2 * C::kStage);
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
        if constexpr (C::A16) {
          const half8_t r = f.raw[h][j];
          a0 = half2_t{r[0], r[1]};
          a1 = half2_t{r[2], r[3]};
          c0 = half2_t{r[4], r[5]};
          c1 = half2_t{r[6], r[7]};
        } else {
          i8x4_to_f16x4(f.raw[h][j].x, a0, a1);
          i8x4_to_f16x4(f.raw[h][j].y, c0, c1);
        }
        const half2_t h0 = a0 * d2, h1 = a1 * d2, h2 = c0 * d2, h3 = c1 * d2;
        const half2_t l0 = __builtin_elementwise_fma(a0, d2, -h0);
        const half2_t l1 = __builtin_elementwise_fma(a1, d2, -h1);
        const half2_t l2 = __builtin_elementwise_fma(c0, d2, -h2);
        const half2_t l3 = __builtin_elementwise_fma(c1, d2, -h3);
        bh[j] = half8_t{h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
        bl[j] = half8_t{l0[0], l0[1], l1[0], l1[1], l2[0], l2[1], l3[0], l3[1]};
      }
      if constexpr (DEBUG) {
        // subblock 4 t + 2 u + h: 2^11 sum c * q for 32 weight rows x 32 tokens per (i, j)
        const int64_t sb = 4 * (int64_t)t + 2 * u + h, nsb = K >> 4;
#pragma unroll
        for (int i = 0; i < TN; ++i)
#pragma unroll
          for (int j = 0; j < TM; ++j) {
            floatx16 p = __builtin_amdgcn_mfma_f32_32x32x16_f16(f.ah[h][i], bh[j], floatx16{}, 0, 0, 0);
            p = __builtin_amdgcn_mfma_f32_32x32x16_f16(f.ah[h][i], bl[j], p, 0, 0, 0);
            p = __builtin_amdgcn_mfma_f32_32x32x16_f16(f.al[h][i], bh[j], p, 0, 0, 0);
            const int64_t m = m0 + wm * (32 * TM) + 32 * j + fr;
            if (m >= M) continue;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              const int r = wn * (32 * TN) + 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
              if (n0 + r < N) isums[(m * N + n0 + r) * nsb + sb] = (int32_t)(p[e] * rinv[r]);
            }
          }
      } else {
#pragma unroll
        for (int i = 0; i < TN; ++i)
#pragma unroll
          for (int j = 0; j < TM; ++j) {
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(f.ah[h][i], bh[j], acc[i][j], 0, 0, 0);
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(f.ah[h][i], bl[j], acc[i][j], 0, 0, 0);
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(f.al[h][i], bh[j], acc[i][j], 0, 0, 0);
          }
      }
    }
  };

  // pipeline over stages t0 .. t1-1; loads clamped, loop body branch-free (after the
  // last stage the staging writes a clamped copy nobody reads)
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
    // keep the substep-1 fragment reads ahead of the staging work: left to itself the
    // scheduler sinks each read next to its first MFMA and waits on it there
    __builtin_amdgcn_sched_barrier(0);
    lstore(b ^ 1, x, 0);
    mfmas(f0, t, 0);
    gload(min(t + 2, t1 - 1), x);
    __syncthreads();
    fread(b ^ 1, 0, f0);
    mfmas(f1, t, 1);
  }
  if constexpr (DEBUG) return;

  // second pass for activation blocks with d >= 512 (not taken otherwise): plain
  // staging through buffer 0, into the accumulators scaled by 2^-8 and restored by
  // 2^8 afterwards (both exact)
  if (__syncthreads_or(anybig)) {
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
      for (int j = 0; j < TM; ++j) acc[i][j] *= 0.00390625f;
    for (int t = t0; t < t1; ++t) {
      gload(t, x);
      __syncthreads();  // every read of buffer 0 done
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

  // undo the row scales (the first barrier of the pipeline ordered their stores)
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

// ---------------------------------------------------------------------------------
// Integer-MFMA kernel for the formats with one (scale, offset) per 32 weights: Q4_1,
// Q4_K, Q5_K, IQ4_XS (K % 64 == 0).  Per 32-block b of a row the weight is
// w = dw_b * v + mw_b with an integer code value v (Q4_1 / Q4_K: 0..15, Q5_K: 0..31,
// IQ4_XS: the table value, -128..127, and mw = 0), so
//     y[m][n] = sum_b da[m][b] * (dw[n][b] * S[m][n][b] + mw[n][b] * Q[m][b]),
// S = sum over the block of v * q (an integer) and Q = sum of q.  One
// v_mfma_i32_32x32x32_i8 gives S exactly for 32 tokens x 32 weight rows: its int8
// operands are the activation codes and the weights' code values, both as staged.
// The vector unit then takes each S to float and adds (S * dw) * da into a float32
// accumulator (one rounding per product and sum; no split terms, no second pass for
// large activation scales).  The offset term is a (K / 32)-deep product of
// mw[n][b] and da[m][b] * Q[m][b] (an exact float: 11 x 12 significant bits), done by
// v_mfma_f32_32x32x2f32, two blocks per instruction, into the same accumulators.
//
// Conditioning of the offset formats: a weight dw * c + mw can be far smaller than
// either part (the block's line crosses zero near code c), and the two products would
// then carry rounding errors of the parts' size.  So each block's codes are staged
// shifted by the integer z nearest the root -mw / dw (clamped to the code range):
// w = dw * (c - z) + (mw + dw * z).  With the root in range |mw + dw z| <= |dw| / 2,
// so both parts of every weight are at most twice the weight; with the root outside,
// the parts have one sign.  Either way the errors stay a few 2^-24 of sum |w * a|.
// c - z fits int8 (|c - z| <= 31).
//
// MFMA rows are tokens and columns weight rows, so each lane has one weight row
// (one dw per block and column tile) and 16 tokens, whose binary16 da are read from
// LDS in the lanes' row order and used as fp16 operands of v_fma_mix.  Block: 512
// threads, WN x WM wavefronts of (32 TM tokens) x (32 TN weight rows); the tile shapes,
// work items and K-split parts are those of the two-term kernel, so the workspace is
// the same.  LDS holds two 64-k stages: the weight code values and the activation
// codes as int8 rows, the blocks' dw and mw (float32), da (binary16) and da * Q.
// Q is summed here from the staged codes (v_dot4 against ones).
//
// DEBUG instance (the per-16 sums of this kernel's data path): the same staging and
// int8 MFMAs, one per 16-block, with the weight operand's other 16-k half zeroed
// (each lane half holds one 16-k half of the block); the sums are written as they are.
// ---------------------------------------------------------------------------------
namespace {
constexpr int kI8Row = 80;  // bytes per LDS code row: 64 codes + 16 pad, 16-byte aligned

template <int WN_, int WM_, int TN_, int TM_>
struct QI8Cfg {
  static constexpr int WN = WN_, WM = WM_, TN = TN_, TM = TM_;
  static constexpr int BN = 32 * WN * TN, BM = 32 * WM * TM;
  static constexpr int kAcc = 16 * TN * TM;  // fp32 accumulators per thread
  static constexpr bool kRowsM = true;       // accumulator rows are tokens (K-split reduce)
  // one stage: weight codes [BN][80], activation codes [BM][80], then per 32-block
  // b = 0, 1 of the stage: dw [2][BN], mw [2][BN] (float32), da [2][BM] (binary16, in
  // lane order), da * Q [2][BM] (float32)
  static constexpr int kOffA = BN * kI8Row;
  static constexpr int kOffDW = kOffA + BM * kI8Row;
  static constexpr int kOffMW = kOffDW + 2 * BN * 4;
  static constexpr int kOffDA = kOffMW + 2 * BN * 4;
  static constexpr int kOffSA = kOffDA + 2 * BM * 2;
  static constexpr int kStage = kOffSA + 2 * BM * 4;
  static constexpr int kLds = 2 * kStage;
  static constexpr int CPT = BN * 64 / kQThreads;  // weight codes staged per thread
  static constexpr int TPR = 64 / CPT;             // threads per weight row
  static constexpr int ABT = BM * 64 / kQThreads;  // activation codes staged per thread
  static constexpr int APR = 64 / ABT;             // threads per activation row
  static_assert(WN * WM * 64 == kQThreads, "8 wavefronts");
  static_assert(CPT == 16 || CPT == 32, "one 32-block per thread and stage");
  static_assert(ABT == 8 || ABT == 16 || ABT == 32, "activation staging width");
  static_assert(kLds <= 160 * 1024, "LDS");
};
using QI8Big = QI8Cfg<2, 4, 2, 2>;   // 128 weight rows x 256 tokens
using QI8M128 = QI8Cfg<2, 4, 2, 1>;  // 128 weight rows x 128 tokens
using QI8Mid = QI8Cfg<4, 2, 2, 1>;   // 256 weight rows x 64 tokens

// position of token r (0..31) of a 32-token tile in the lane-ordered da row: lane half
// h = (r >> 2) & 1 reads 16 values, element e = 4 (r >> 3) + (r & 3)
__device__ __forceinline__ int i8_da_slot(int r) { return 16 * ((r >> 2) & 1) + 4 * (r >> 3) + (r & 3); }
}  // namespace

template <class C, int FMT, bool DEBUG>
__global__ __launch_bounds__(512, 1) void gemm_q4x_i8_kernel(const uint8_t* __restrict__ w, int64_t N, int K,
                                                             const int8_t* __restrict__ q,
                                                             const uint16_t* __restrict__ d16, int64_t M,
                                                             float* __restrict__ y, float* __restrict__ part_ws,
                                                             int32_t* __restrict__ isums, KSplitPlan plan,
                                                             u32x4 vtab) {
  static_assert(FMT != kQ6K, "per-16 scales: the two-term kernel");
  constexpr int BN = C::BN, BM = C::BM, WM = C::WM, TN = C::TN, TM = C::TM;
  constexpr int CPT = C::CPT, TPR = C::TPR, ABT = C::ABT, APR = C::APR;
  constexpr bool kOffset = FMT != kIQ4;  // formats with an offset term
  constexpr uint32_t kCodes = FMT == kQ5K ? 32u : 16u;  // code range of the offset formats
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
  const int nb32 = K >> 5;      // activation scales per token row
  const BlockScales<FMT> bsc(w, N, K);
  constexpr int PW = BlockScales<FMT>::kWords;
  const HighBits<FMT> hbits(w, N, K);
  constexpr int HW = HighBits<FMT>::kHW, HS = HighBits<FMT>::kSlots;

  // staging tasks: CPT codes of weight row wrow at k-offset CPT wq of the stage (all in
  // 32-block wblk of the stage), the block's scale words and high bits; ABT activation
  // codes of token arow at k-offset aoff (in block ablk) and the (token, block)'s
  // binary16 d.  The threads that share a 32-block store the same dw, mw (or da,
  // da * Q) to the same place, which keeps the staging free of branches.  Rows past
  // N / M are clamped to valid memory and their results never stored.
  const int wrow = tid / TPR, wq = tid % TPR;
  const int64_t wr = min(n0 + wrow, N - 1);
  const uint8_t* __restrict__ wbase = w + wr * crow + (CPT / 2) * wq;
  const int wblk = (CPT * wq) >> 5;
  const int arow = tid / APR, aoff = ABT * (tid % APR), ablk = aoff >> 5;
  const int8_t* __restrict__ abase = q + min(m0 + arow, M - 1) * K + aoff;
  const uint16_t* __restrict__ dbase = d16 + min(m0 + arow, M - 1) * nb32 + ablk;
  struct Stage { Words<ABT / 4> a; Words<CPT / 8> wc; uint32_t dm[PW]; uint32_t hb[HS]; uint32_t dr; int blk; };
  auto gload = [&](int t, Stage& x) {
    x.wc = load_words<CPT / 8>(wbase + (int64_t)t * 32);
    x.blk = 2 * t + wblk;
    if (!DEBUG) bsc.load(wr, x.blk, x.dm);
    if (HW > 0) hbits.load(wr, x.blk, x.hb);
    x.a = load_words<ABT / 4>(abase + 64 * t);
    x.dr = DEBUG ? 0x3C00u : (uint32_t)dbase[2 * t];
  };
  auto lstore = [&](int b, const Stage& x) {
    uint8_t* st = smem + b * C::kStage;
    // the block's scale and offset, and its code shift z (offset formats): the code
    // nearest the root -mw / dw of the block's weight line, clamped to the code range
    // (0 for a zero or non-finite dw)
    float dwf = 1.0f, mwf = 0.0f;
    uint32_t z = 0u;
    if constexpr (!DEBUG) {
      BlockScales<FMT>::decode(x.dm, x.blk, dwf, mwf);
      if constexpr (kOffset) {
        const float r = -mwf * __builtin_amdgcn_rcpf(dwf);
        z = (uint32_t)fminf(fmaxf(__builtin_rintf(r), 0.0f), (float)(kCodes - 1));
        mwf = __builtin_fmaf(dwf, (float)z, mwf);
      }
      reinterpret_cast<float*>(st + C::kOffDW)[wblk * BN + wrow] = dwf;
      if constexpr (kOffset) reinterpret_cast<float*>(st + C::kOffMW)[wblk * BN + wrow] = mwf;
    }
    // weight code values as int8 bytes in k order: per packed word (codes 2i in the low,
    // 2i + 1 in the high nibbles of byte i) the even and odd code bytes (with Q5_K's
    // fifth bits, or IQ4_XS's table values), interleaved by two v_perm_b32; offset
    // formats then store c - z: b = c + R - z lies in 1 .. 2R - 1 (no carry between
    // bytes) and b - R is b ^ R for b >= R, else (b ^ R) with the bits above R set
    Words<CPT / 4> cv;
#pragma unroll
    for (int h = 0; h < CPT / 8; ++h) {
      uint32_t ce, co;
      code_bytes<HW>(x.wc.v[h], ((CPT * wq) & 31) / 8 + h, x.hb, ce, co);
      if constexpr (FMT == kIQ4) {
        ce = lut16(ce, vtab);
        co = lut16(co, vtab);
      }
      cv.v[2 * h] = perm(co, ce, 0x05010400u);
      cv.v[2 * h + 1] = perm(co, ce, 0x07030602u);
    }
    if constexpr (kOffset && !DEBUG) {
      constexpr uint32_t kR = 0x01010101u * kCodes;
#pragma unroll
      for (int v = 0; v < CPT / 4; ++v) {
        const uint32_t bb = cv.v[v] + 0x01010101u * (kCodes - z);
        cv.v[v] = (bb ^ kR) | ((~bb & kR) * (256u / kCodes - 2u));
      }
    }
    store_words<CPT / 4>(st + wrow * kI8Row + CPT * wq, cv);
    store_words<ABT / 4>(st + C::kOffA + arow * kI8Row + aoff, x.a);
    if constexpr (!DEBUG) {
      // sum of the block's codes over the APR / 2 threads that stage it
      int s = 0;
#pragma unroll
      for (int v = 0; v < ABT / 4; ++v) s = dot4(x.a.v[v], 0x01010101u, s);
      if constexpr (ABT <= 16) s += __shfl_xor(s, 1);
      if constexpr (ABT == 8) s += __shfl_xor(s, 2);
      const int r = arow & 31, tb = arow & ~31;
      reinterpret_cast<uint16_t*>(st + C::kOffDA)[ablk * BM + tb + i8_da_slot(r)] = (uint16_t)x.dr;
      if constexpr (kOffset)
        reinterpret_cast<float*>(st + C::kOffSA)[ablk * BM + arow] = f16_bits_to_f32((uint16_t)x.dr) * (float)s;
    }
  };

  floatx16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = floatx16{};
  const int fr = lane & 31, hl = lane >> 5;
  typedef int i32x4 __attribute__((ext_vector_type(4)));
  typedef int i32x16 __attribute__((ext_vector_type(16)));
  // fragments of 32-block u of a stage: A (tokens) and B (weights) 16 codes per lane,
  // the lane's 16 token scales per token tile, its weight scale per weight tile; with
  // u = 1 also the stage's offset operands (da * Q of token fr, mw of row fr, block hl)
  struct Frag { i32x4 a[TM], b[TN]; half8_t da[TM][2]; float dw[TN]; float sa[TM], mw[TN]; };
  auto fread = [&](int b, int u, Frag& f) {
    const uint8_t* st = smem + b * C::kStage;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int r = wm * (32 * TM) + 32 * i;
      f.a[i] = *reinterpret_cast<const i32x4*>(st + C::kOffA + (r + fr) * kI8Row + 32 * u + 16 * hl);
      if constexpr (!DEBUG) {
        const half8_t* dp = reinterpret_cast<const half8_t*>(st + C::kOffDA + 2 * (u * BM + r + 16 * hl));
        f.da[i][0] = dp[0];
        f.da[i][1] = dp[1];
        if (kOffset && u == 1) f.sa[i] = reinterpret_cast<const float*>(st + C::kOffSA)[hl * BM + r + fr];
      }
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int r = wn * (32 * TN) + 32 * j + fr;
      f.b[j] = *reinterpret_cast<const i32x4*>(st + r * kI8Row + 32 * u + 16 * hl);
      if constexpr (!DEBUG) {
        f.dw[j] = reinterpret_cast<const float*>(st + C::kOffDW)[u * BN + r];
        if (kOffset && u == 1) f.mw[j] = reinterpret_cast<const float*>(st + C::kOffMW)[hl * BN + r];
      }
    }
  };
  const i32x16 zero16 = {};
  // the products of 32-block u of stage t (t, u only locate the DEBUG sums)
  auto mfmas = [&](const Frag& f, int t, int u) {
    if constexpr (DEBUG) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int64_t nsb = K >> 4;
          const int64_t n = n0 + wn * (32 * TN) + 32 * j + fr;
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const i32x4 bm = hl == hh ? f.b[j] : i32x4{0, 0, 0, 0};
            const i32x16 s = __builtin_amdgcn_mfma_i32_32x32x32_i8(f.a[i], bm, zero16, 0, 0, 0);
            const int64_t sb = 4 * (int64_t)t + 2 * u + hh;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              const int64_t m = m0 + wm * (32 * TM) + 32 * i + 8 * (e >> 2) + 4 * hl + (e & 3);
              if (m < M && n < N) isums[(m * N + n) * nsb + sb] = s[e];
            }
          }
        }
    } else {
      // tile k's MFMA is issued before tile k - 1's sums are scaled, so the vector work
      // covers the MFMA's latency instead of waiting for its own result
      constexpr int T = TM * TN;
      i32x16 sp = __builtin_amdgcn_mfma_i32_32x32x32_i8(f.a[0], f.b[0], zero16, 0, 0, 0);
#pragma unroll
      for (int k = 1; k <= T; ++k) {
        i32x16 sn = sp;
        if (k < T) sn = __builtin_amdgcn_mfma_i32_32x32x32_i8(f.a[k / TN], f.b[k % TN], zero16, 0, 0, 0);
        const int i = (k - 1) / TN, j = (k - 1) % TN;
#pragma unroll
        for (int e = 0; e < 16; ++e)
          acc[i][j][e] = __builtin_fmaf((float)sp[e] * f.dw[j], (float)f.da[i][e >> 3][e & 7], acc[i][j][e]);
        sp = sn;
      }
    }
    if constexpr (!DEBUG && kOffset) {
      if (u == 1) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(f.sa[i], f.mw[j], acc[i][j], 0, 0, 0);
      }
    }
  };

  // pipeline over stages t0 .. t1-1 (as the two-term kernel): loads clamped, loop body
  // branch-free (after the last stage the staging writes a clamped copy nobody reads)
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
    __builtin_amdgcn_sched_barrier(0);
    lstore(b ^ 1, x);
    mfmas(f0, t, 0);
    gload(min(t + 2, t1 - 1), x);
    __syncthreads();
    fread(b ^ 1, 0, f0);
    mfmas(f1, t, 1);
  }
  if constexpr (DEBUG) return;

  if (part >= 0) {
    float* dst = part_ws + ((item - plan.full) * C::kAcc) * kQThreads + tid;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) dst[((i * TN + j) * 16 + e) * kQThreads] = acc[i][j][e];
    return;
  }
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int64_t n = n0 + wn * (32 * TN) + 32 * j + fr;
    if (n >= N) continue;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t m = m0 + wm * (32 * TM) + 32 * i + 8 * (e >> 2) + 4 * hl + (e & 3);
        if (m < M) y[m * N + n] = acc[i][j][e];
      }
  }
}

namespace {
// isums != nullptr: the DEBUG instance (per-16 sums, no workspace, no reduction).
// split = false: one work item per tile (no workspace), for the GEMV entry's long rows.
template <class C, int FMT>
hipError_t launch_q4x_i8(const uint8_t* w, const int8_t* q, const uint16_t* d16, int64_t M, int64_t N, int64_t K,
                         float* y, int32_t* isums, float* workspace, hipStream_t stream, bool split, u32x4 vtab) {
  KSplitPlan plan = ksplit_plan<C::BN, C::BM>(M, N, K);
  if (!split) {
    plan.split = 1;
    plan.split_tiles = 0;
    plan.full = plan.tiles;
  }
  const int64_t items = plan.full + plan.split_tiles * plan.split;
  if (isums) {
    hipError_t ea = hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_q4x_i8_kernel<C, FMT, true>),
                                        hipFuncAttributeMaxDynamicSharedMemorySize, C::kLds);
    if (ea != hipSuccess) return ea;
    hipLaunchKernelGGL((gemm_q4x_i8_kernel<C, FMT, true>), dim3((unsigned)items), dim3(kQThreads), C::kLds,
                       stream, w, N, (int)K, q, d16, M, y, nullptr, isums, plan, vtab);
    return hipGetLastError();
  }
  if (plan.split_tiles && !workspace) return hipErrorInvalidValue;  // callers size it first
  hipError_t ea = hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_q4x_i8_kernel<C, FMT, false>),
                                      hipFuncAttributeMaxDynamicSharedMemorySize, C::kLds);
  if (ea != hipSuccess) return ea;
  hipLaunchKernelGGL((gemm_q4x_i8_kernel<C, FMT, false>), dim3((unsigned)items), dim3(kQThreads), C::kLds,
                     stream, w, N, (int)K, q, d16, M, y, workspace, nullptr, plan, vtab);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || plan.split_tiles == 0) return e;
  return launch_ksplit_reduce<C>(workspace, N, M, 1.0f, y, plan, stream);
}

// The Q4-family GEMM of tile shape C: the integer-MFMA kernel for the formats with one
// (scale, offset) per 32 weights, the two-term kernel for Q6_K (one scale per 16)
template <class C, int FMT>
hipError_t launch_q41_f16x2(const uint8_t* w, const int8_t* q, const uint16_t* d16, int64_t M, int64_t N,
                            int64_t K, float* y, int32_t* isums, float* workspace, hipStream_t stream,
                            bool split = true, u32x4 vtab = u32x4{0u, 0u, 0u, 0u}) {
  if constexpr (FMT != kQ6K)
    return launch_q4x_i8<QI8Cfg<C::WN, C::WM, C::TN, C::TM>, FMT>(w, q, d16, M, N, K, y, isums, workspace, stream,
                                                                  split, vtab);
  KSplitPlan plan = ksplit_plan<C::BN, C::BM>(M, N, K);
  if (!split) {
    plan.split = 1;
    plan.split_tiles = 0;
    plan.full = plan.tiles;
  }
  const int64_t items = plan.full + plan.split_tiles * plan.split;
  if (isums) {
    hipError_t ea = hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_q4_1_f16x2_kernel<C, FMT, true>),
                                        hipFuncAttributeMaxDynamicSharedMemorySize, C::kLds);
    if (ea != hipSuccess) return ea;
    hipLaunchKernelGGL((gemm_q4_1_f16x2_kernel<C, FMT, true>), dim3((unsigned)items), dim3(kQThreads), C::kLds,
                       stream, w, N, (int)K, q, d16, M, y, nullptr, isums, plan, vtab);
    return hipGetLastError();
  }
  if (plan.split_tiles && !workspace) return hipErrorInvalidValue;  // callers size it first
  hipError_t ea = hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_q4_1_f16x2_kernel<C, FMT, false>),
                                      hipFuncAttributeMaxDynamicSharedMemorySize, C::kLds);
  if (ea != hipSuccess) return ea;
  hipLaunchKernelGGL((gemm_q4_1_f16x2_kernel<C, FMT, false>), dim3((unsigned)items), dim3(kQThreads), C::kLds,
                     stream, w, N, (int)K, q, d16, M, y, workspace, nullptr, plan, vtab);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || plan.split_tiles == 0) return e;
  return launch_ksplit_reduce<C>(workspace, N, M, 1.0f, y, plan, stream);
}

// which kernel runs a Q4_K, Q5_K, IQ4_XS (i8) or Q6_K (!i8) product of this shape: the
// GEMV kernel up to 16 tokens (rows up to 20480 weights), else the integer-MFMA (or
// two-term) kernel in the tile shape for M (K % 256 == 0 always)
Q41Path q4k_path(int64_t M, int64_t K, bool i8 = true) {
  if (M <= kQ41GemvMaxM && q41_gemv_fits(K)) return kQ41Gemv;
  if (M <= 64) return kQ41Mid;
  return M <= (i8 ? kI8M128Max : kF16M128Max) ? kQ41M128 : kQ41Big;
}
}  // namespace

hipError_t launch_gemm_q4_1(const uint8_t* w, const int8_t* q, const uint16_t* d16,
                            const int16_t* bsum16, int64_t M, int64_t N, int64_t K, float* y,
                            int32_t* isums, float* workspace, hipStream_t stream) {
  switch (q41_path(M, K)) {
    case kQ41Gemv: return launch_gemv_q4_1(w, q, d16, bsum16, M, N, K, y, isums, stream);
    case kQ41Big: return launch_q41_f16x2<Q41Big, kQ41>(w, q, d16, M, N, K, y, isums, workspace, stream);
    case kQ41Mid: return launch_q41_f16x2<Q41Mid, kQ41>(w, q, d16, M, N, K, y, isums, workspace, stream);
    case kQ41M128: return launch_q41_f16x2<Q41M128, kQ41>(w, q, d16, M, N, K, y, isums, workspace, stream);
    default: return launch_q41_tiled(w, q, d16, bsum16, M, N, K, y, isums, stream);
  }
}

size_t gemm_q4_k_workspace(int64_t M, int64_t N, int64_t K, bool q6k) {
  switch (q4k_path(M, K, !q6k)) {
    case kQ41Mid: return ksplit_workspace<Q41Mid>(M, N, K);
    case kQ41M128: return ksplit_workspace<Q41M128>(M, N, K);
    case kQ41Big: return ksplit_workspace<Q41Big>(M, N, K);
    default: return 0;
  }
}

hipError_t launch_gemm_q4_k(const uint8_t* w, const int8_t* q, const uint16_t* d16,
                            const int16_t* bsum16, int64_t M, int64_t N, int64_t K, float* y,
                            int32_t* isums, float* workspace, hipStream_t stream) {
  switch (q4k_path(M, K)) {
    case kQ41Gemv: return launch_gemv_q4x<kQ4K>(w, q, d16, bsum16, M, N, K, y, isums, stream);
    case kQ41Big: return launch_q41_f16x2<Q41Big, kQ4K>(w, q, d16, M, N, K, y, isums, workspace, stream);
    case kQ41M128: return launch_q41_f16x2<Q41M128, kQ4K>(w, q, d16, M, N, K, y, isums, workspace, stream);
    default: return launch_q41_f16x2<Q41Mid, kQ4K>(w, q, d16, M, N, K, y, isums, workspace, stream);
  }
}

// IQ4_XS: the value table as 4 words (entries 4i .. 4i + 3 in word i, int8 bytes)
static u32x4 table_words(const int8_t* table) {
  u32x4 t = {0u, 0u, 0u, 0u};
  for (int i = 0; i < 16; ++i) t[i / 4] |= (uint32_t)(uint8_t)table[i] << (8 * (i % 4));
  return t;
}

hipError_t launch_gemm_iq4_xs(const uint8_t* w, const int8_t* table, const int8_t* q, const uint16_t* d16,
                              int64_t M, int64_t N, int64_t K, float* y, int32_t* isums, float* workspace,
                              hipStream_t stream) {
  const u32x4 t = table_words(table);
  switch (q4k_path(M, K)) {
    case kQ41Gemv: return launch_gemv_q4x<kIQ4>(w, q, d16, nullptr, M, N, K, y, isums, stream, t);
    case kQ41Big: return launch_q41_f16x2<Q41Big, kIQ4>(w, q, d16, M, N, K, y, isums, workspace, stream, true, t);
    case kQ41M128: return launch_q41_f16x2<Q41M128, kIQ4>(w, q, d16, M, N, K, y, isums, workspace, stream, true, t);
    default: return launch_q41_f16x2<Q41Mid, kIQ4>(w, q, d16, M, N, K, y, isums, workspace, stream, true, t);
  }
}

hipError_t launch_gemv_iq4_xs(const uint8_t* w, const int8_t* table, const int8_t* q, const uint16_t* d16,
                              int64_t M, int64_t N, int64_t K, float* y, int32_t* isums, hipStream_t stream) {
  const u32x4 t = table_words(table);
  if (q41_gemv_fits(K)) return launch_gemv_q4x<kIQ4>(w, q, d16, nullptr, M, N, K, y, isums, stream, t);
  return launch_q41_f16x2<Q41Mid, kIQ4>(w, q, d16, M, N, K, y, isums, nullptr, stream, false, t);
}

// The GEMV entry (M <= 16): the GEMV kernel, or for rows past its reach the two-term
// kernel with one work item per tile (no workspace)
hipError_t launch_gemv_q4_k(const uint8_t* w, const int8_t* q, const uint16_t* d16,
                            const int16_t* bsum16, int64_t M, int64_t N, int64_t K, float* y,
                            int32_t* isums, hipStream_t stream) {
  if (q41_gemv_fits(K)) return launch_gemv_q4x<kQ4K>(w, q, d16, bsum16, M, N, K, y, isums, stream);
  return launch_q41_f16x2<Q41Mid, kQ4K>(w, q, d16, M, N, K, y, isums, nullptr, stream, false);
}

// Q5_K and Q6_K: the same two kernels and dispatch as Q4_K (Q6_K takes no bsum16)
hipError_t launch_gemv_q5_k(const uint8_t* w, const int8_t* q, const uint16_t* d16,
                            const int16_t* bsum16, int64_t M, int64_t N, int64_t K, float* y,
                            int32_t* isums, hipStream_t stream) {
  if (q41_gemv_fits(K)) return launch_gemv_q4x<kQ5K>(w, q, d16, bsum16, M, N, K, y, isums, stream);
  return launch_q41_f16x2<Q41Mid, kQ5K>(w, q, d16, M, N, K, y, isums, nullptr, stream, false);
}

hipError_t launch_gemm_q5_k(const uint8_t* w, const int8_t* q, const uint16_t* d16,
                            const int16_t* bsum16, int64_t M, int64_t N, int64_t K, float* y,
                            int32_t* isums, float* workspace, hipStream_t stream) {
  switch (q4k_path(M, K)) {
    case kQ41Gemv: return launch_gemv_q4x<kQ5K>(w, q, d16, bsum16, M, N, K, y, isums, stream);
    case kQ41Big: return launch_q41_f16x2<Q41Big, kQ5K>(w, q, d16, M, N, K, y, isums, workspace, stream);
    case kQ41M128: return launch_q41_f16x2<Q41M128, kQ5K>(w, q, d16, M, N, K, y, isums, workspace, stream);
    default: return launch_q41_f16x2<Q41Mid, kQ5K>(w, q, d16, M, N, K, y, isums, workspace, stream);
  }
}

hipError_t launch_gemv_q6_k(const uint8_t* w, const int8_t* q, const uint16_t* d16, int64_t M, int64_t N,
                            int64_t K, float* y, int32_t* isums, hipStream_t stream) {
  if (q41_gemv_fits(K)) return launch_gemv_q4x<kQ6K>(w, q, d16, nullptr, M, N, K, y, isums, stream);
  return launch_q41_f16x2<Q41Mid, kQ6K>(w, q, d16, M, N, K, y, isums, nullptr, stream, false);
}

hipError_t launch_gemm_q6_k(const uint8_t* w, const int8_t* q, const uint16_t* d16, int64_t M, int64_t N,
                            int64_t K, float* y, int32_t* isums, float* workspace, hipStream_t stream) {
  switch (q4k_path(M, K, false)) {
    case kQ41Gemv: return launch_gemv_q4x<kQ6K>(w, q, d16, nullptr, M, N, K, y, isums, stream);
    case kQ41Big: return launch_q41_f16x2<Q41Big, kQ6K>(w, q, d16, M, N, K, y, isums, workspace, stream);
    case kQ41M128: return launch_q41_f16x2<Q41M128, kQ6K>(w, q, d16, M, N, K, y, isums, workspace, stream);
    default: return launch_q41_f16x2<Q41Mid, kQ6K>(w, q, d16, M, N, K, y, isums, workspace, stream);
  }
}

}  // namespace nvq
