// dequantize.hip -- codes + block scales -> bf16 or fp32 weights on gfx950.
//
// The decoded weight is the exact product e2m1(c) * dec(sb) * s_t (NVFP4) or
// e2m1(c) * 2^(sb-127) (MXFP4), rounded once to the output type.  This is the
// dequantization a fake-quant training forward inserts so that training sees the
// engine's values (QATFactory page, section on how training repeats the target
// engine's arithmetic).  One thread handles 32 elements (16 bytes of codes).
//
// The decoding itself (exactness arguments included) is in codec.hpp.
#include "codec.hpp"
#include "fp4w_device.hpp"
#include "fp4w_internal.hpp"

namespace fp4w {

template <bool OUT_F32>
__global__ __launch_bounds__(256) void nvfp4_dequant_kernel(const uint4* __restrict__ codes,
                                                            const uint8_t* __restrict__ scales,
                                                            const float* __restrict__ tensor_scale,
                                                            int64_t ngroups, void* __restrict__ out) {
  const float st = *tensor_scale;
  const bool tiny = !(st >= 0x1p-90f);
  for (int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x; g < ngroups; g += (int64_t)gridDim.x * 256) {
    uint4 c = codes[g];
    uint32_t cw[4] = {c.x, c.y, c.z, c.w};
    float d[2] = {e4m3_to_f32(scales[2 * g]), e4m3_to_f32(scales[2 * g + 1])};
    if (OUT_F32) {
      uint32_t o[32];
#pragma unroll
      for (int j = 0; j < 4; j++) {
        float dd = d[j >> 1];
        float v[8];
        uint32_t dummy;
        nvfp4_pair(fp4x2_to_f32x2<0>(cw[j], 1.0f), dd, st, tiny, v[0], v[1], dummy, false);
        nvfp4_pair(fp4x2_to_f32x2<1>(cw[j], 1.0f), dd, st, tiny, v[2], v[3], dummy, false);
        nvfp4_pair(fp4x2_to_f32x2<2>(cw[j], 1.0f), dd, st, tiny, v[4], v[5], dummy, false);
        nvfp4_pair(fp4x2_to_f32x2<3>(cw[j], 1.0f), dd, st, tiny, v[6], v[7], dummy, false);
#pragma unroll
        for (int e = 0; e < 8; e++) o[8 * j + e] = canon_nan_f32(v[e]);
      }
      uint4* dst = reinterpret_cast<uint4*>(out) + 8 * g;
#pragma unroll
      for (int q = 0; q < 8; q++) dst[q] = make_uint4(o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]);
    } else {
      uint32_t o[16];
#pragma unroll
      for (int j = 0; j < 4; j++) {
        float dd = d[j >> 1];
        float f0, f1;
        nvfp4_pair(fp4x2_to_f32x2<0>(cw[j], 1.0f), dd, st, tiny, f0, f1, o[4 * j + 0], true);
        nvfp4_pair(fp4x2_to_f32x2<1>(cw[j], 1.0f), dd, st, tiny, f0, f1, o[4 * j + 1], true);
        nvfp4_pair(fp4x2_to_f32x2<2>(cw[j], 1.0f), dd, st, tiny, f0, f1, o[4 * j + 2], true);
        nvfp4_pair(fp4x2_to_f32x2<3>(cw[j], 1.0f), dd, st, tiny, f0, f1, o[4 * j + 3], true);
      }
      uint4* dst = reinterpret_cast<uint4*>(out) + 4 * g;
#pragma unroll
      for (int q = 0; q < 4; q++) dst[q] = make_uint4(o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]);
    }
  }
}

template <bool OUT_F32>
__global__ __launch_bounds__(256) void mxfp4_dequant_kernel(const uint4* __restrict__ codes,
                                                            const uint8_t* __restrict__ scales,
                                                            int64_t ngroups, void* __restrict__ out) {
  for (int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x; g < ngroups; g += (int64_t)gridDim.x * 256) {
    uint4 c = codes[g];
    uint32_t cw[4] = {c.x, c.y, c.z, c.w};
    const uint32_t sb = scales[g];
    const bool plain = sb >= 0xFDu;
    if (OUT_F32) {
      uint32_t o[32];
      if (!plain) {
        const float s = e8m0_scale_operand(sb);
#pragma unroll
        for (int j = 0; j < 4; j++) {
          f32x2_t a = fp4x2_to_f32x2<0>(cw[j], s), b = fp4x2_to_f32x2<1>(cw[j], s);
          f32x2_t c2 = fp4x2_to_f32x2<2>(cw[j], s), d2 = fp4x2_to_f32x2<3>(cw[j], s);
          o[8 * j + 0] = __float_as_uint(a.x); o[8 * j + 1] = __float_as_uint(a.y);
          o[8 * j + 2] = __float_as_uint(b.x); o[8 * j + 3] = __float_as_uint(b.y);
          o[8 * j + 4] = __float_as_uint(c2.x); o[8 * j + 5] = __float_as_uint(c2.y);
          o[8 * j + 6] = __float_as_uint(d2.x); o[8 * j + 7] = __float_as_uint(d2.y);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; j++) {
          float v[8];
          mx_plain8(cw[j], sb, v);
#pragma unroll
          for (int e = 0; e < 8; e++) o[8 * j + e] = __float_as_uint(v[e]);
        }
      }
      uint4* dst = reinterpret_cast<uint4*>(out) + 8 * g;
#pragma unroll
      for (int q = 0; q < 8; q++) dst[q] = make_uint4(o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]);
    } else {
      uint32_t o[16];
      if (!plain) {
        const float s = e8m0_scale_operand(sb);
#pragma unroll
        for (int j = 0; j < 4; j++) {
          o[4 * j + 0] = fp4x2_to_bf16x2_scaled<0>(cw[j], s);
          o[4 * j + 1] = fp4x2_to_bf16x2_scaled<1>(cw[j], s);
          o[4 * j + 2] = fp4x2_to_bf16x2_scaled<2>(cw[j], s);
          o[4 * j + 3] = fp4x2_to_bf16x2_scaled<3>(cw[j], s);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; j++) {
          float v[8];
          mx_plain8(cw[j], sb, v);
          // values are exact in bf16 (<= 2 significant bits) or +-inf / NaN
#pragma unroll
          for (int e = 0; e < 4; e++)
            o[4 * j + e] = f32_to_bf16_rne(v[2 * e]) | (f32_to_bf16_rne(v[2 * e + 1]) << 16);
        }
      }
      uint4* dst = reinterpret_cast<uint4*>(out) + 4 * g;
#pragma unroll
      for (int q = 0; q < 4; q++) dst[q] = make_uint4(o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]);
    }
  }
}

// bf16 out with whole-wave stores: store instruction q of a wave writes 1 KB in
// one piece (lane l: the 8 elements of code dword l % 4 of group
// 64 w + 16 q + l / 4, 16 bytes at 1024 q + 16 l of the wave's 4 KB), and the
// code loads are 4 bytes a lane over 256 contiguous bytes.
template <int FMT>
__global__ __launch_bounds__(256) void dequant_bf16_kernel(const uint32_t* __restrict__ codes,
                                                           const uint8_t* __restrict__ scales,
                                                           const float* __restrict__ tensor_scale, int64_t ngroups,
                                                           uint4* __restrict__ out) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float st = FMT == FMT_NVFP4 ? *tensor_scale : 1.0f;
  const bool tiny = !(st >= 0x1p-90f);
  const int j = lane & 3;                           // code dword of the group: elements 8 j .. 8 j + 7
  for (int64_t g0 = ((int64_t)blockIdx.x * 4 + wave) * 64; g0 < ngroups; g0 += (int64_t)gridDim.x * 256) {
    uint32_t cw[4], sb[4];
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const int64_t g = g0 + 16 * q + (lane >> 2);
      const bool ok = g < ngroups;
      cw[q] = ok ? codes[4 * g + j] : 0u;
      sb[q] = ok ? (FMT == FMT_NVFP4 ? scales[2 * g + (j >> 1)] : scales[g]) : 0u;
    }
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const int64_t g = g0 + 16 * q + (lane >> 2);
      uint32_t o[4];
      if (FMT == FMT_NVFP4) {
        const float d = e4m3_to_f32(sb[q]);
        float f0, f1;
        nvfp4_pair(fp4x2_to_f32x2<0>(cw[q], 1.0f), d, st, tiny, f0, f1, o[0], true);
        nvfp4_pair(fp4x2_to_f32x2<1>(cw[q], 1.0f), d, st, tiny, f0, f1, o[1], true);
        nvfp4_pair(fp4x2_to_f32x2<2>(cw[q], 1.0f), d, st, tiny, f0, f1, o[2], true);
        nvfp4_pair(fp4x2_to_f32x2<3>(cw[q], 1.0f), d, st, tiny, f0, f1, o[3], true);
      } else if (sb[q] < 0xFDu) {
        const float sc = e8m0_scale_operand(sb[q]);
        o[0] = fp4x2_to_bf16x2_scaled<0>(cw[q], sc);
        o[1] = fp4x2_to_bf16x2_scaled<1>(cw[q], sc);
        o[2] = fp4x2_to_bf16x2_scaled<2>(cw[q], sc);
        o[3] = fp4x2_to_bf16x2_scaled<3>(cw[q], sc);
      } else {
        float v[8];
        mx_plain8(cw[q], sb[q], v);
        // values are exact in bf16 (<= 2 significant bits) or +-inf / NaN
#pragma unroll
        for (int e = 0; e < 4; e++) o[e] = f32_to_bf16_rne(v[2 * e]) | (f32_to_bf16_rne(v[2 * e + 1]) << 16);
      }
      if (g < ngroups) out[4 * g + j] = make_uint4(o[0], o[1], o[2], o[3]);
    }
  }
}

hipError_t launch_dequantize(int fmt, const uint8_t* codes, const uint8_t* scales, const float* tensor_scale,
                             int64_t n, int64_t k, void* out, bool out_fp32, hipStream_t stream) {
  const int64_t ngroups = n * k / 32;
  if (ngroups == 0) return hipSuccess;
  int64_t g = (ngroups + 255) / 256;
  const int grid = (int)(g > 16384 ? 16384 : g);
  const uint4* c = reinterpret_cast<const uint4*>(codes);
  if (!out_fp32) {
    int64_t gb = (ngroups + 255) / 256;
    const int gridb = (int)(gb > 16384 ? 16384 : gb);
    const uint32_t* cw = reinterpret_cast<const uint32_t*>(codes);
    uint4* o = reinterpret_cast<uint4*>(out);
    if (fmt == FMT_NVFP4)
      hipLaunchKernelGGL(dequant_bf16_kernel<FMT_NVFP4>, dim3(gridb), dim3(256), 0, stream, cw, scales, tensor_scale,
                         ngroups, o);
    else
      hipLaunchKernelGGL(dequant_bf16_kernel<FMT_MXFP4>, dim3(gridb), dim3(256), 0, stream, cw, scales, tensor_scale,
                         ngroups, o);
    return hipGetLastError();
  }
  if (fmt == FMT_NVFP4) {
    if (out_fp32)
      hipLaunchKernelGGL(nvfp4_dequant_kernel<true>, dim3(grid), dim3(256), 0, stream, c, scales, tensor_scale, ngroups, out);
    else
      hipLaunchKernelGGL(nvfp4_dequant_kernel<false>, dim3(grid), dim3(256), 0, stream, c, scales, tensor_scale, ngroups, out);
  } else {
    if (out_fp32)
      hipLaunchKernelGGL(mxfp4_dequant_kernel<true>, dim3(grid), dim3(256), 0, stream, c, scales, ngroups, out);
    else
      hipLaunchKernelGGL(mxfp4_dequant_kernel<false>, dim3(grid), dim3(256), 0, stream, c, scales, ngroups, out);
  }
  return hipGetLastError();
}

}  // namespace fp4w
