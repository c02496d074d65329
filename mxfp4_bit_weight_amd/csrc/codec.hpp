// codec.hpp -- decoding of NVFP4 / MXFP4 codes to the exact value rounded once,
// shared by the dequantize kernels and the fused fake-quant kernels, so that
// a fake-quantized weight is bit for bit the dequantized quantized weight.
//
// NVFP4: u = e2m1 * dec(sb) has at most 6 significant bits, so it is exact in
// fp32; u * s_t rounds once (the fp32 output).  For bf16, hi = fl32(u * s_t)
// and lo = fma(u, s_t, -hi) is the exact remainder, and bf16_rne_from_pair
// breaks the one case where rounding hi again would differ (hi exactly on a
// bf16 tie).  Tensor scales below 2^-90 could make the remainder underflow
// (`tiny`); the product is then formed in binary64 instead.
// MXFP4: the scaled conversions produce e2m1 * 2^e exactly; blocks whose
// exponent can overflow (sb >= 0xFD) or whose scale is NaN take the plain path.
#pragma once
#include "fp4w_device.hpp"

namespace fp4w {

__device__ __forceinline__ void nvfp4_pair(f32x2_t t, float d, float st, bool tiny, float& o0, float& o1,
                                           uint32_t& b01, bool want_bf16) {
  float u0 = t.x * d, u1 = t.y * d;                // exact
  if (!want_bf16) {
    o0 = u0 * st;
    o1 = u1 * st;
    return;
  }
  float h0, h1, l0, l1;
  if (!tiny) {
    h0 = u0 * st; l0 = __builtin_fmaf(u0, st, -h0);
    h1 = u1 * st; l1 = __builtin_fmaf(u1, st, -h1);
  } else {
    double v0 = (double)u0 * (double)st, v1 = (double)u1 * (double)st;   // exact
    h0 = (float)v0; l0 = (float)(v0 - (double)h0);
    h1 = (float)v1; l1 = (float)(v1 - (double)h1);
  }
  b01 = bf16_rne_from_pair(h0, l0) | (bf16_rne_from_pair(h1, l1) << 16);
}

__device__ __forceinline__ uint32_t canon_nan_f32(float v) {
  uint32_t u = __float_as_uint(v);
  return ((u & 0x7FFFFFFFu) > 0x7F800000u) ? 0x7FC00000u : u;
}

// Plain MXFP4 path: e2m1 as fp32, times 2^(sb-127) in one rounded multiply
// (exact, or +-inf on overflow), NaN for the NaN scale.
__device__ __forceinline__ void mx_plain8(uint32_t cw, uint32_t sb, float* v) {
  const bool nan_scale = sb == 0xFFu;
  const float p = e8m0_to_f32(sb);
  f32x2_t t0 = fp4x2_to_f32x2<0>(cw, 1.0f), t1 = fp4x2_to_f32x2<1>(cw, 1.0f);
  f32x2_t t2 = fp4x2_to_f32x2<2>(cw, 1.0f), t3 = fp4x2_to_f32x2<3>(cw, 1.0f);
  float e[8] = {t0.x, t0.y, t1.x, t1.y, t2.x, t2.y, t3.x, t3.y};
#pragma unroll
  for (int i = 0; i < 8; i++) v[i] = nan_scale ? __uint_as_float(0x7FC00000u) : e[i] * p;
}

}  // namespace fp4w
