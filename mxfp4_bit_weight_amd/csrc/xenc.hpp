// xenc.hpp -- bf16 activations as two E4M3 terms under E8M0 block scales, the
// operand form of gfx950's block-scaled MFMA (v_mfma_scale_f32_16x16x128_f8f6f4).
//
// The product the pages define multiplies 16-bit activations with the decoded
// 4-bit weights and accumulates in fp32 (QATFactory page, section on how
// training repeats the engine's arithmetic).  gfx950 can feed E2M1 weight codes
// to the matrix core directly, but only against an 8-, 6- or 4-bit left operand.
// So each 32-element block of a row of x is split, exactly, into
//     x = 2^Eh * h + 2^El * l,     h, l in E4M3,
// with Eh = max(e - 7, -127) (e = floor(log2 of the block's largest |x|)) and
// El = max(Eh - 4, -127).  Why this is exact: v = x / 2^Eh is below 256 in
// magnitude and has at most 8 significant bits; h is v rounded to E4M3 (4 bits),
// so r = v - h is a multiple of ulp(v) no larger than 8 ulp(v) in magnitude
// (whatever the rounding direction, below 16 ulp), hence 16 r has at most 4
// significant bits and is an E4M3 value whenever ulp(16 r) >= 2^-9, i.e. when
// |v| >= 2^-6.  Elements more than 2^13 below their block's largest one may lose
// low bits: their error is at most 2^(El - 10), i.e. 2^-21 of the block maximum
// (2^-137 absolute for blocks whose maximum is below 2^-116).  A block holding
// an Inf or NaN gets the NaN scale 0xFF, which turns its row of the product NaN.
//
// The fp8 conversions used (v_cvt_scalef32_pk_fp8_bf16, v_cvt_scalef32_pk_f32_fp8,
// v_cvt_scalef32_pk_fp8_f32) divide or multiply by the power of two held in the
// scale operand's exponent field; their in-range results were checked on the
// device, including E4M3 subnormals and scale 2^-127.
#pragma once
#include "fp4w_device.hpp"

namespace fp4w {

typedef __attribute__((ext_vector_type(2))) short i16x2_t;

// Largest |x| of a 32-element block held by 4 consecutive lanes (8 elements
// each), as the 15 magnitude bits of bf16 (integer order = magnitude order,
// NaN above Inf).  All four lanes of the quad must be active.
__device__ __forceinline__ uint32_t quad_max_u32(uint32_t v) {
  uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);   // lane ^ 1
  v = o > v ? o : v;
  o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);            // lane ^ 2
  return o > v ? o : v;
}

struct XEnc8 {
  uint32_t h[2];     // 8 E4M3 bytes of the high term, element order
  uint32_t l[2];     // 8 E4M3 bytes of the low term
  uint32_t sch;      // E8M0 code of 2^Eh (0xFF: block not finite)
  uint32_t scl;      // E8M0 code of 2^El
};

// Encode the 8 bf16 elements `v` of this lane; the quad (lanes 4q..4q+3) holds
// one 32-element block.
__device__ __forceinline__ XEnc8 encode_x8(u32x4_t v) {
  uint32_t mb = 0;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const uint32_t a = v[i] & 0x7FFFu, b = (v[i] >> 16) & 0x7FFFu;
    const uint32_t m2 = a > b ? a : b;
    mb = m2 > mb ? m2 : mb;
  }
  mb = quad_max_u32(mb);
  const int field = (int)(mb >> 7);                       // biased exponent of the block max
  const int eh = field - 134 > -127 ? field - 134 : -127;
  const int el = eh - 4 > -127 ? eh - 4 : -127;
  // v = x / 2^Eh is formed by an exact power-of-two multiply (2^-Eh is a normal
  // fp32 for Eh in [-127, 120]); the remainder is taken in that scaled space,
  // where h * 2^Eh could not overflow even when h rounds up to 2^8.
  const float sh = pow2_scale_operand(eh);
  const float inv = __uint_as_float((uint32_t)(127 - eh) << 23);
  const float slh = pow2_scale_operand(el - eh);          // 2^(El - Eh), El - Eh in [-4, 0]
  XEnc8 r;
  const bool finite = field < 255;
  r.sch = finite ? (uint32_t)(eh + 127) : 0xFFu;
  r.scl = finite ? (uint32_t)(el + 127) : 0xFFu;
#pragma unroll
  for (int d = 0; d < 2; d++) {
    const uint32_t w0 = v[2 * d], w1 = v[2 * d + 1];
    i16x2_t hh = {0, 0};
    hh = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(hh, __builtin_bit_cast(bf16x2_t, w0), sh, false);
    hh = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(hh, __builtin_bit_cast(bf16x2_t, w1), sh, true);
    const uint32_t hw = __builtin_bit_cast(uint32_t, hh);
    const f32x2_t b0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hw, 1.0f, false);   // h exactly
    const f32x2_t b1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hw, 1.0f, true);
    const float r0 = bf16lo_f32(w0) * inv - b0.x, r1 = bf16hi_f32(w0) * inv - b0.y;   // exact remainders
    const float r2 = bf16lo_f32(w1) * inv - b1.x, r3 = bf16hi_f32(w1) * inv - b1.y;
    i16x2_t ll = {0, 0};
    ll = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(ll, r0, r1, slh, false);
    ll = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(ll, r2, r3, slh, true);
    r.h[d] = hw;
    r.l[d] = __builtin_bit_cast(uint32_t, ll);
  }
  return r;
}

}  // namespace fp4w
