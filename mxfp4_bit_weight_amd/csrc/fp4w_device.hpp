// fp4w_device.hpp -- device helpers shared by the gfx950 kernels of libfp4w.
//
// Formats (OCP bit layouts; the pages only name "an E2M1 code plus a shared
// block scale", Scale-QLoRA page, paragraph on the formats):
//   E2M1  sign | 2-bit exponent (bias 1) | 1-bit mantissa: 0, .5, 1, 1.5, 2, 3, 4, 6
//   E4M3  "FN": bias 7, subnormal m*2^-9, max 448 (0x7E), S.1111.111 = NaN
//   E8M0  2^(c-127), 0xFF = NaN
// gfx950 conversion instructions used here (their semantics were checked on the
// device against exact rationals):
//   v_cvt_scalef32_pk_fp4_f32 / _bf16 : RNE_sat(v / 2^exp(scale)) -> 2 nibbles,
//                                        ties to even, saturating at 6, -0 -> 0x8
//   v_cvt_scalef32_pk_{f32,bf16}_fp4  : e2m1 * 2^exp(scale), exact
//   v_cvt_f32_fp8                     : OCP E4M3FN decode
// where exp(scale) is the power of two held in the fp32 scale's exponent field
// (the mantissa is ignored; exponent field 0 means 2^-127).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4w {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;

constexpr int FMT_NVFP4 = 0;
constexpr int FMT_MXFP4 = 1;

// ---- bit helpers ------------------------------------------------------------

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }
__device__ __forceinline__ u32x4_t load16(const void* p) { return *reinterpret_cast<const u32x4_t*>(p); }

__device__ __forceinline__ float bf16lo_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi_f32(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t w) { return __builtin_bit_cast(bf16x2_t, w); }
__device__ __forceinline__ uint32_t as_u32(bf16x2_t v) { return __builtin_bit_cast(uint32_t, v); }

// Power of two 2^e (e in [-127, 127]) as the fp32 scale operand of the gfx950
// scaled conversions: only the exponent field is read, field 0 meaning 2^-127.
__device__ __forceinline__ float pow2_scale_operand(int e) {
  return __uint_as_float((uint32_t)(e + 127) << 23);
}
__device__ __forceinline__ float e8m0_scale_operand(uint32_t code) {
  return __uint_as_float((code & 0xFFu) << 23);
}

// E4M3FN byte -> fp32 (exact; 0x7F / 0xFF -> NaN).
__device__ __forceinline__ float e4m3_to_f32(uint32_t byte) {
  return __builtin_amdgcn_cvt_f32_fp8((int)(byte & 0xFFu), 0);
}

// E8M0 byte -> fp32 (exact; 0 -> 2^-127 subnormal; 0xFF -> NaN).
__device__ __forceinline__ float e8m0_to_f32(uint32_t code) {
  code &= 0xFFu;
  if (code == 0xFFu) return __builtin_nanf("");
  if (code == 0u) return __uint_as_float(0x00400000u);
  return __uint_as_float(code << 23);
}

// Two E2M1 codes (byte `sel` of `packed`, low nibble first) -> two exact bf16.
template <int SEL>
__device__ __forceinline__ uint32_t fp4x2_to_bf16x2(uint32_t packed) {
  return as_u32(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(packed, 1.0f, SEL));
}
template <int SEL>
__device__ __forceinline__ uint32_t fp4x2_to_bf16x2_scaled(uint32_t packed, float pow2) {
  return as_u32(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(packed, pow2, SEL));
}
template <int SEL>
__device__ __forceinline__ f32x2_t fp4x2_to_f32x2(uint32_t packed, float pow2) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(packed, pow2, SEL);
}

// fp32 -> bf16 bits, round to nearest even (finite or inf input; NaN kept NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;

// Two fp32 -> two bf16 (lo in bits 15:0) in one v_cvt_pk_bf16_f32: round to
// nearest even, the same bits as f32_to_bf16_rne for every input but NaN, which
// stays a NaN (all 2^32 inputs compared on gfx950).
__device__ __forceinline__ uint32_t f32x2_to_bf16x2_rne(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// acc + a.lo^2 + a.hi^2 for the two bf16 of a (v_dot2_f32_bf16).
__device__ __forceinline__ float bf16x2_sumsq(uint32_t a, float acc) {
  const bf16x2_t v = __builtin_bit_cast(bf16x2_t, a);
  return __builtin_amdgcn_fdot2_f32_bf16(v, v, acc, false);
}

// Round the exact value hi + lo (|lo| <= ulp(hi)/2, lo the exact remainder of
// the fp32 rounding that produced hi) once, to nearest even, to bf16 bits.
// Only an exact bf16 tie in hi needs lo: the exact value is above or below it.
__device__ __forceinline__ uint32_t bf16_rne_from_pair(float hi, float lo) {
  uint32_t u = __float_as_uint(hi);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  uint32_t low = u & 0xFFFFu;
  if (low == 0x8000u && lo != 0.0f) {
    // magnitude of the exact value vs the tie: lo with hi's sign is "above"
    bool above = (lo > 0.0f) == (hi > 0.0f);
    return above ? ((u >> 16) + 1u) : (u >> 16);
  }
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// ---- exact NVFP4 block-scale encode ------------------------------------------
// sb = RNE_sat(a / (6 s_t)) on the E4M3 grid for a >= 0, s_t > 0 finite.
// 6 s_t is exact in binary64 and the binary64 quotient decides exactly: a
// non-tie quotient is at least 2^-33 (relative) from any E4M3 midpoint, and an
// exact tie is representable, so the correctly rounded binary64 quotient lies on
// the same side of every midpoint as the real one.  Rounding to 3 mantissa bits
// is then done on the binary64 bit pattern (no intermediate binary32 rounding).
__device__ __forceinline__ uint32_t e4m3_rne_sat_from_f64(double q) {
  if (!(q < 448.0)) return 0x7Eu;                       // >= 448 (also +inf)
  if (q < 0.015625) {                                   // below 2^-6: subnormal step 2^-9
    double m = __builtin_rint(q * 512.0);               // RNE; 8 -> 0x08 = 2^-6
    return (uint32_t)m;
  }
  uint64_t b = (uint64_t)__double_as_longlong(q);
  uint64_t keep = (b >> 49) & 1ull;                     // lowest kept mantissa bit
  b += 0xFFFFFFFFFFFFull + keep;                        // round at bit 49, ties to even
  int e = (int)((b >> 52) & 0x7FF) - 1023;              // -6 .. 8
  uint32_t m = (uint32_t)((b >> 49) & 7u);
  uint32_t code = ((uint32_t)(e + 7) << 3) | m;
  return code > 0x7Eu ? 0x7Eu : code;
}

__device__ __forceinline__ uint32_t nvfp4_block_scale(float amax_b, float st) {
  if (!(st > 0.0f) || !(st <= 3.4028235e38f)) return 0u;   // s_t == 0 or non-finite
  double q = (double)amax_b / (6.0 * (double)st);
  return e4m3_rne_sat_from_f64(q);
}

// ---- exact E2M1 encode for one element (slow path) ---------------------------
// Magnitude code of RNE_sat(a / (d * s_t)), a = |w| >= 0, d = dec(sb) > 0.
// Each midpoint test is the sign of fma(mu * d, s_t, -a): mu * d has <= 7 bits
// so it is exact, and fma rounds once, which keeps the sign of the exact
// difference.  Tiny tensor scales are lifted by 2^64 (exact) so the difference
// never falls below the binary32 normal range.
__device__ __forceinline__ uint32_t e2m1_code_exact(float a, float d, float st) {
  float lift = st < 0x1p-64f ? 0x1p64f : 1.0f;
  float a2 = a * lift, st2 = st * lift;
  // midpoints between codes (i, i+1) and whether an exact tie goes up (to i+1)
  const float mids[7] = {0.25f, 0.75f, 1.25f, 1.75f, 2.5f, 3.5f, 5.0f};
  uint32_t code = 0;
#pragma unroll
  for (int i = 0; i < 7; i++) {
    float r = __builtin_fmaf(mids[i] * d, st2, -a2);    // sign(mu*S - a)
    bool tie_up = (i & 1) != 0;                         // upper code i+1 even <=> i odd
    code += (r < 0.0f || (r == 0.0f && tie_up)) ? 1u : 0u;
  }
  return code;
}

// ---- buffer loads ----------------------------------------------------------------
// Raw buffer resource (stride 0) over [base, base + bytes): a load at or past
// `bytes` returns zeros and makes no memory access, so predicated-off lanes are
// given an offset past the end instead of a branch.
constexpr uint32_t kBufferOob = 0xFFFFFFF0u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4_t buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// ---- small reductions ----------------------------------------------------------

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    uint32_t o = (uint32_t)__shfl_xor((int)v, off, 64);
    v = o > v ? o : v;
  }
  return v;
}

}  // namespace fp4w
