// merge.hip -- scale-only merge on gfx950.
//
// Scale-QLoRA keeps the code plane frozen and trains corrections of the block
// scales; the forward rounds scales to the format's grid, and the merge writes
// the trained scale bytes and copies the codes verbatim, so the merged weights
// are bitwise what training saw (rit.work, "Scale-QLoRA: merge native 4-bit
// models", merge paragraphs).  Per block: v = dec(S) + delta exactly, v <= 0 ->
// code 0, else the nearest value of the scale grid (E4M3, or E8M0 nearest in the
// linear domain), ties to the even code, saturating at the top.
//
// Exactness: (hi, lo) = TwoSum(dec(S), delta) in binary64 is the exact sum.  A
// candidate code comes from hi; it can only be off by one where hi sits exactly
// on a grid midpoint, and comparing (hi, lo) with the two neighbouring
// midpoints (exact binary64 values) settles it.
#include "fp4w_device.hpp"
#include "fp4w_internal.hpp"

namespace fp4w {

__device__ __forceinline__ int cmp_pair(double hi, double lo, double g) {
  if (hi != g) return hi > g ? 1 : -1;
  return lo > 0.0 ? 1 : (lo < 0.0 ? -1 : 0);
}

__device__ __forceinline__ double grid_value(int fmt, int c) {
  if (fmt == FMT_NVFP4) return (double)e4m3_to_f32((uint32_t)c);
  return __builtin_ldexp(1.0, c - 127);
}

// Nearest power of two to v > 0 in the linear domain (ties to the even code),
// as an E8M0 code clamped to [0, 254].
__device__ __forceinline__ int e8m0_candidate(double v) {
  if (!(v < 0x1p127)) return 254;
  if (v < 0x1p-127) return 0;
  int ex;
  double f = __builtin_frexp(v, &ex);          // v = f * 2^ex, f in [0.5, 1)
  int e = ex - 1;                              // v in [2^e, 2^(e+1))
  double m = 2.0 * f;                          // [1, 2)
  if (m > 1.5 || (m == 1.5 && ((e + 1 + 127) & 1) == 0)) e += 1;
  int c = e + 127;
  return c < 0 ? 0 : (c > 254 ? 254 : c);
}

__global__ __launch_bounds__(256) void merge_scales_kernel(int fmt, const uint8_t* __restrict__ s_in,
                                                           const float* __restrict__ deltas, int64_t nb,
                                                           uint8_t* __restrict__ s_out) {
  const int top = (fmt == FMT_NVFP4) ? 0x7E : 0xFE;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < nb; i += (int64_t)gridDim.x * 256) {
    const uint32_t code = s_in[i];
    const float delta = deltas[i];
    const double base = (fmt == FMT_NVFP4) ? (double)e4m3_to_f32(code) : (double)e8m0_to_f32(code);
    int out;
    if (base != base || delta != delta) {
      out = (fmt == FMT_NVFP4) ? 0x7F : 0xFF;
    } else {
      const double b = (double)delta;
      const double hi = base + b;                  // TwoSum (Knuth)
      const double bb = hi - base;
      const double lo = (base - (hi - bb)) + (b - bb);
      if (hi < 0.0 || (hi == 0.0 && lo <= 0.0)) {
        out = 0;
      } else if (hi > 1.0e300) {
        out = top;
      } else {
        int c = (fmt == FMT_NVFP4) ? (int)e4m3_rne_sat_from_f64(hi) : e8m0_candidate(hi);
        if (c > 0) {                              // midpoint with the code below
          double mid = 0.5 * (grid_value(fmt, c - 1) + grid_value(fmt, c));
          int s = cmp_pair(hi, lo, mid);
          if (s < 0 || (s == 0 && ((c - 1) & 1) == 0)) c -= 1;
        }
        if (c < top) {                            // midpoint with the code above
          double mid = 0.5 * (grid_value(fmt, c) + grid_value(fmt, c + 1));
          int s = cmp_pair(hi, lo, mid);
          if (s > 0 || (s == 0 && ((c + 1) & 1) == 0)) c += 1;
        }
        out = c;
      }
    }
    s_out[i] = (uint8_t)out;
  }
}

// Byte-for-byte copy of the code plane (16-byte body, byte tail).
__global__ __launch_bounds__(256) void copy_bytes_kernel(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                                         int64_t nbytes) {
  const int64_t n16 = nbytes / 16;
  const uint4* s = reinterpret_cast<const uint4*>(src);
  uint4* d = reinterpret_cast<uint4*>(dst);
  const int64_t stride = (int64_t)gridDim.x * 256;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (int64_t i = t; i < n16; i += stride) d[i] = s[i];
  for (int64_t i = n16 * 16 + t; i < nbytes; i += stride) dst[i] = src[i];
}

hipError_t launch_merge_scales(int fmt, const uint8_t* scales_in, const float* deltas, int64_t num_blocks,
                               uint8_t* scales_out, const uint8_t* codes_in, uint8_t* codes_out,
                               int64_t code_bytes, hipStream_t stream) {
  if (num_blocks > 0) {
    int64_t g = (num_blocks + 255) / 256;
    hipLaunchKernelGGL(merge_scales_kernel, dim3((int)(g > 8192 ? 8192 : g)), dim3(256), 0, stream, fmt, scales_in,
                       deltas, num_blocks, scales_out);
  }
  if (codes_in && codes_out && codes_in != codes_out && code_bytes > 0) {
    int64_t g = (code_bytes / 16 + 255) / 256;
    if (g < 1) g = 1;
    hipLaunchKernelGGL(copy_bytes_kernel, dim3((int)(g > 8192 ? 8192 : g)), dim3(256), 0, stream, codes_in,
                       codes_out, code_bytes);
  }
  return hipGetLastError();
}

}  // namespace fp4w
