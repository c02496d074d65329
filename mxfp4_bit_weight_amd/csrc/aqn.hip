// aqn.hip -- the noisy RMSNorm ahead of the projections (adaptive noise for
// exploration, Telegram post, "Metod"): per row of x (m, k),
//   y[k] = bf16( x[k] * rsqrt(mean_k x^2 + eps) * gamma[k] * (1 + sigma * noise[k]) )
// The noise sits in the norm's per-channel gain, so the projection that follows
// sees its weight columns scaled by (1 + sigma * noise[k]) -- the multiplicative
// weight noise the post describes -- while only the 4-bit weights stay resident.
// noise (k values, drawn by the caller per step) is an input; sigma follows the
// exponential schedule of fp4w_aqn_sigma.
//
// One workgroup of 256 threads per row: a first pass sums x^2 (fp32, 16-byte
// loads, wave sums then one add over the 4 waves in LDS), a second pass re-reads
// x (cache-resident) with gamma and noise and writes y in 16-byte stores.
#include <cmath>

#include "fp4w_device.hpp"
#include "fp4w_internal.hpp"

namespace fp4w {

__global__ __launch_bounds__(256) void aqn_rmsnorm_kernel(const uint16_t* __restrict__ x, int64_t K,
                                                          const uint16_t* __restrict__ gamma,
                                                          const float* __restrict__ noise, float sigma, float eps,
                                                          uint16_t* __restrict__ y) {
  __shared__ float part[4];
  const int64_t row = blockIdx.x;
  const uint16_t* xr = x + row * K;
  const int tid = threadIdx.x;
  float ss = 0.f;
  for (int64_t k = 8 * (int64_t)tid; k < K; k += 8 * 256) {
    const u32x4_t v = load16(xr + k);
#pragma unroll
    for (int d = 0; d < 4; d++) {
      const float a = bf16lo_f32(v[d]), b = bf16hi_f32(v[d]);
      ss = fmaf(a, a, ss);
      ss = fmaf(b, b, ss);
    }
  }
  ss = wave_sum(ss);
  if ((tid & 63) == 0) part[tid >> 6] = ss;
  __syncthreads();
  const float tot = (part[0] + part[1]) + (part[2] + part[3]);
  const float r = 1.0f / sqrtf(tot / (float)K + eps);
  for (int64_t k = 8 * (int64_t)tid; k < K; k += 8 * 256) {
    const u32x4_t v = load16(xr + k), g = load16(gamma + k);
    const u32x4_t n0 = load16(noise + k), n1 = load16(noise + k + 4);
    u32x4_t o;
#pragma unroll
    for (int d = 0; d < 4; d++) {
      const float na = __uint_as_float(d < 2 ? n0[2 * d] : n1[2 * d - 4]);
      const float nb = __uint_as_float(d < 2 ? n0[2 * d + 1] : n1[2 * d - 3]);
      const float a = bf16lo_f32(v[d]) * r * bf16lo_f32(g[d]) * fmaf(sigma, na, 1.0f);
      const float b = bf16hi_f32(v[d]) * r * bf16hi_f32(g[d]) * fmaf(sigma, nb, 1.0f);
      o[d] = f32_to_bf16_rne(a) | (f32_to_bf16_rne(b) << 16);
    }
    *reinterpret_cast<u32x4_t*>(y + row * K + k) = o;
  }
}

hipError_t launch_aqn_rmsnorm(const void* x, int64_t m, int64_t k, const void* gamma, const float* noise,
                              float sigma, float eps, void* y, hipStream_t stream) {
  if (m == 0 || k == 0) return hipSuccess;
  hipLaunchKernelGGL(aqn_rmsnorm_kernel, dim3((unsigned)m), dim3(256), 0, stream,
                     reinterpret_cast<const uint16_t*>(x), k, reinterpret_cast<const uint16_t*>(gamma), noise, sigma,
                     eps, reinterpret_cast<uint16_t*>(y));
  return hipGetLastError();
}

}  // namespace fp4w
