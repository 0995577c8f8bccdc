// nvq_device.h -- device helpers shared by the gfx950 kernels of libnvq.
//
// Everything here is written for CDNA4 (gfx950) only: 64-wide wavefronts,
// v_perm_b32 byte selection, v_dot4_i32_i8, the OCP E4M3 / E2M1 conversion
// instructions and the 16x16x32 fp16 MFMA.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvq {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// NW 32-bit words moved as one 8-byte (NW = 2) or 16-byte vector access per 4 words;
// p must be aligned to the access size.  A plain array of scalars, so the compiler
// keeps it in registers.
template <int NW>
struct Words {
  uint32_t v[NW];
};
template <int NW>
__device__ __forceinline__ Words<NW> load_words(const void* p) {
  Words<NW> r;
  if constexpr (NW == 2) {
    const u32x2 t = *reinterpret_cast<const u32x2*>(p);
    r.v[0] = t[0];
    r.v[1] = t[1];
  } else {
#pragma unroll
    for (int h = 0; h < NW / 4; ++h) {
      const u32x4 t = reinterpret_cast<const u32x4*>(p)[h];
#pragma unroll
      for (int e = 0; e < 4; ++e) r.v[4 * h + e] = t[e];
    }
  }
  return r;
}
template <int NW>
__device__ __forceinline__ void store_words(void* p, const Words<NW>& w) {
  if constexpr (NW == 2) {
    *reinterpret_cast<u32x2*>(p) = u32x2{w.v[0], w.v[1]};
  } else {
#pragma unroll
    for (int h = 0; h < NW / 4; ++h)
      reinterpret_cast<u32x4*>(p)[h] = u32x4{w.v[4 * h], w.v[4 * h + 1], w.v[4 * h + 2], w.v[4 * h + 3]};
  }
}

// ---------------------------------------------------------------------------
// Byte permute and integer dot product.
// v_perm_b32(s0, s1, sel): result byte i = pool[sel_i] where pool bytes 0..3 come
// from s1 and 4..7 from s0; selector 12 gives 0x00 and selectors >= 13 give 0xFF;
// selectors 8..11 replicate the sign bit of pool bytes 1, 3, 5, 7.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t perm(uint32_t s0, uint32_t s1, uint32_t sel) {
  return __builtin_amdgcn_perm(s0, s1, sel);
}
__device__ __forceinline__ int dot4(uint32_t a, uint32_t b, int c) {
  return __builtin_amdgcn_sdot4((int)a, (int)b, c, false);
}

// ---------------------------------------------------------------------------
// E2M1 -> signed integer L(c) = 2 * E2M1(c) in -12..12, four codes per dword
// (one code per byte, values 0..15).  Two v_perm_b32 lookups whose sum is L:
//   PA indexed by the whole code:   codes 0..7 give 0,2,4,6,8,11,15,23; codes
//     8..12 give 0 (sign bits of non-negative pool bytes, or selector 12);
//     codes 13..15 give 0xFF = -1.
//   PB indexed by (code & 7):       0,-1,-2,-3,-4,-5,-7,-11.
// Sum: 0,1,2,3,4,6,8,12 for codes 0..7 and 0,-1,-2,-3,-4,-6,-8,-12 for 8..15.
// The two halves are summed inside the integer dot products (two v_dot4 per
// operand), so no byte-wise add (and no carry) is ever needed.
// ---------------------------------------------------------------------------
constexpr uint32_t kPA_lo = 0x06040200u, kPA_hi = 0x170F0B08u;
constexpr uint32_t kPB_lo = 0xFDFEFF00u, kPB_hi = 0xF5F9FBFCu;

// One dword of 8 packed codes (byte i: code of weight 2i in bits 0..3, weight 2i+1
// in bits 4..7) against activation dwords qe (the 4 even-position codes) and qo
// (the 4 odd-position codes).  Adds the PA part of L(code)*q to a and the PB part
// to b; a + b is the integer dot product.  pal/pah/pbl/pbh are the pools and
// m4/m3 the nibble masks, held in VGPRs by the caller.
__device__ __forceinline__ void dot8_e2m1_ab(uint32_t c, uint32_t qe, uint32_t qo, int& a, int& b,
                                             uint32_t pal, uint32_t pah, uint32_t pbl, uint32_t pbh,
                                             uint32_t m4, uint32_t m3) {
  const uint32_t lo = c & m4, lo7 = c & m3;
  const uint32_t t = c >> 4;
  const uint32_t hi = t & m4, hi7 = t & m3;
  a = dot4(perm(pah, pal, lo), qe, a);
  b = dot4(perm(pbh, pbl, lo7), qe, b);
  a = dot4(perm(pah, pal, hi), qo, a);
  b = dot4(perm(pbh, pbl, hi7), qo, b);
}

// Same, returning acc + sum_j L(code_j) * q_j (pools taken as constants).
__device__ __forceinline__ int dot8_e2m1(uint32_t c, uint32_t qe, uint32_t qo, int acc) {
  int a = acc, b = 0;
  dot8_e2m1_ab(c, qe, qo, a, b, kPA_lo, kPA_hi, kPB_lo, kPB_hi, 0x0F0F0F0Fu, 0x07070707u);
  return a + b;
}

// Split 8 activation bytes (two dwords, natural order) into even / odd positions.
__device__ __forceinline__ void split_even_odd(uint32_t a, uint32_t b, uint32_t& e, uint32_t& o) {
  e = perm(b, a, 0x06040200u);  // bytes a0 a2 b0 b2
  o = perm(b, a, 0x07050301u);  // bytes a1 a3 b1 b3
}

// ---------------------------------------------------------------------------
// UE4M3 scale byte -> float.  gfx950's v_cvt_f32_fp8 decodes OCP E4M3 (bias 7,
// subnormals, 0x7F NaN); a UE4M3 byte with bit 7 clear has the same bits.
// sel picks the byte of the dword.
// ---------------------------------------------------------------------------
template <int SEL>
__device__ __forceinline__ float ue4m3_to_f32(uint32_t v) {
  return __builtin_amdgcn_cvt_f32_fp8((int)v, SEL);
}

// The two UE4M3 bytes of the low 16 bits of v -> two fp16 values (byte 0 first).
// Every UE4M3 value (2^-9 .. 448, subnormals included) is exact in fp16; the
// instruction's scale operand only contributes its exponent, here 2^0.
__device__ __forceinline__ half2_t ue4m3x2_to_f16(uint32_t v) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v, 1.0f, false);
}

// ---------------------------------------------------------------------------
// Two E2M1 codes of byte SEL of v -> two fp16 values (low nibble first).  The
// instruction's scale operand only contributes its power-of-two exponent, so it
// is always 1.0 here and any other scale is applied with an exact fp16 multiply.
// ---------------------------------------------------------------------------
template <int SEL>
__device__ __forceinline__ half2_t e2m1x2_to_f16(uint32_t v) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(v, 1.0f, SEL);
}

// Activation scales d >= 512 (binary16 bits in [0x6000, 0x7C00): finite, exponent
// field >= 24), for which |d * q| can pass the binary16 range.  The kernels that fold
// d into binary16 operands leave such blocks out of their main pass (d -> 0) and
// take them in a second pass with d / 256 (exponent field - 8: exact, and still a
// normal number), whose accumulator is multiplied by 256 at the end.  Infinite or
// NaN d stay in the main pass, so they still give non-finite outputs.
__device__ __forceinline__ bool act_scale_big(uint32_t d) { return ((d & 0x7FFFu) - 0x6000u) < 0x1C00u; }
// the binary16 bits a block's d takes in pass 0 (main) or pass 1 (d >= 512 only)
__device__ __forceinline__ uint32_t act_scale_for_pass(uint32_t d, int pass) {
  const bool big = act_scale_big(d);
  return pass == 0 ? (big ? 0u : d) : (big ? d - 0x2000u : 0u);
}

// binary16 bits -> float (exact)
__device__ __forceinline__ float f16_bits_to_f32(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

// Four signed bytes -> four fp16 (exact for |v| <= 2048): bias to unsigned,
// splice under the exponent byte of 1024 (0x64) and subtract 1024 + 128.
__device__ __forceinline__ void i8x4_to_f16x4(uint32_t v, half2_t& lo, half2_t& hi) {
  const uint32_t u = v ^ 0x80808080u;
  const uint32_t a = perm(0x64646464u, u, 0x04010400u);  // [u0, 0x64, u1, 0x64]
  const uint32_t b = perm(0x64646464u, u, 0x04030402u);  // [u2, 0x64, u3, 0x64]
  const half2_t bias = {(_Float16)1152.0f, (_Float16)1152.0f};
  lo = __builtin_bit_cast(half2_t, a) - bias;
  hi = __builtin_bit_cast(half2_t, b) - bias;
}

// Keep a value in a VGPR (stops the compiler from re-materialising a constant
// operand of v_perm_b32 before every use).
__device__ __forceinline__ uint32_t in_vgpr(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

// Sum over the 16 lanes of each DPP row; every lane of the row receives the sum.
// quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror.
__device__ __forceinline__ float row16_sum(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, true));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, true));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, true));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x140, 0xF, 0xF, true));
  return v;
}

// Reduce a float over groups of LANES consecutive lanes (LANES = 16, 32 or 64).
// The result is valid in the first lane of each group (lane % LANES == 0).
// Rows of 16 are reduced with DPP (no LDS traffic); rows are combined with
// v_readlane into uniform values.
template <int LANES>
__device__ __forceinline__ float group_sum(float v) {
  v = row16_sum(v);
  if (LANES == 16) return v;
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
  if (LANES == 32) return (threadIdx.x & 32) ? (r2 + r3) : (r0 + r1);
  return (r0 + r1) + (r2 + r3);
}

}  // namespace nvq
