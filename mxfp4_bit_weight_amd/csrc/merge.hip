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
// Exactness: (hi, lo) = TwoSum(dec(S), delta) is the exact sum.  A candidate
// code comes from hi; it can only be off by one where hi sits exactly on a grid
// midpoint, and comparing (hi, lo) with the neighbouring midpoints settles it.
// Almost every block is decided in binary32 without branches (merge_fast); the
// few out of its range go through binary64 (merge_exact).
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

// The exact merge of one block in binary64 (TwoSum, then the grid's neighbouring
// midpoints compared with (hi, lo)).
__device__ uint32_t merge_exact(int fmt, uint32_t code, float delta) {
  const int top = (fmt == FMT_NVFP4) ? 0x7E : 0xFE;
  const double base = (fmt == FMT_NVFP4) ? (double)e4m3_to_f32(code) : (double)e8m0_to_f32(code);
  if (base != base || delta != delta) return (fmt == FMT_NVFP4) ? 0x7Fu : 0xFFu;
  const double b = (double)delta;
  const double hi = base + b;                      // TwoSum (Knuth)
  const double bb = hi - base;
  const double lo = (base - (hi - bb)) + (b - bb);
  if (hi < 0.0 || (hi == 0.0 && lo <= 0.0)) return 0u;
  if (hi > 1.0e300) return (uint32_t)top;
  int c = (fmt == FMT_NVFP4) ? (int)e4m3_rne_sat_from_f64(hi) : e8m0_candidate(hi);
  if (c > 0) {                                     // midpoint with the code below
    double mid = 0.5 * (grid_value(fmt, c - 1) + grid_value(fmt, c));
    int sg = cmp_pair(hi, lo, mid);
    if (sg < 0 || (sg == 0 && ((c - 1) & 1) == 0)) c -= 1;
  }
  if (c < top) {                                   // midpoint with the code above
    double mid = 0.5 * (grid_value(fmt, c) + grid_value(fmt, c + 1));
    int sg = cmp_pair(hi, lo, mid);
    if (sg > 0 || (sg == 0 && ((c + 1) & 1) == 0)) c += 1;
  }
  return (uint32_t)c;
}

// The common case in binary32, without branches.  (hi, lo) = TwoSum(dec(S),
// delta) in binary32 is the exact sum when nothing overflows or underflows
// (|delta| in [2^-60, 2^60] or 0, dec(S) and the sum normal numbers away from
// the ends); every grid value and midpoint is a binary32 number, so hi lies on
// the same side of each midpoint as the exact sum unless hi is the midpoint,
// where the sign of lo decides (0: ties to the even code; E8M0 here, E4M3 on the
// exact path).  `slow` marks the blocks outside that range, which merge_exact
// decides.
template <int FMT>
__device__ __forceinline__ uint32_t merge_fast(uint32_t code, float delta, bool& slow) {
  const float base = (FMT == FMT_NVFP4) ? e4m3_to_f32(code) : e8m0_to_f32(code);
  const bool nan_in = base != base || delta != delta;
  const float ad = __builtin_fabsf(delta);
  const bool ok_d = ad == 0.0f || (ad >= 0x1p-60f && ad <= 0x1p60f);
  // an E4M3 base is 0 or within [2^-9, 448] in magnitude: always in range
  const bool ok_b = FMT == FMT_NVFP4 || base == 0.0f || (base >= 0x1p-100f && base < 0x1p100f);
  const float hi = base + delta;
  const float bb = hi - base;
  const float lo = (base - (hi - bb)) + (delta - bb);
  const bool nonpos = hi <= 0.0f;                  // hi == 0 only for an exact zero sum
  const uint32_t bh = __float_as_uint(hi);
  const bool lo_up = lo > 0.0f, lo_zero = lo == 0.0f;
  uint32_t c;
  bool in_range;
  if (FMT == FMT_NVFP4) {
    // hi to the E4M3 grid, nearest with ties to even: v_cvt_pk_fp8_f32 (the same
    // code as a bit-level rounding for every fp32 in [0, 448)).  That is the code of
    // the exact sum unless hi sits exactly on a midpoint (subnormal step 2^-9: hi 2^9
    // has fraction 1/2; normal: the 20 bits below E4M3's 3 are 1000...0) and lo is
    // not zero; those take the exact path.
    const uint32_t hw = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(hi, hi, 0, false) & 0xFFu;
    const bool sat = hi >= 448.0f;
    c = sat ? 0x7Eu : hw;
    const bool mid = hi < 0x1p-6f ? __builtin_amdgcn_fractf(hi * 512.0f) == 0.5f : (bh & 0xFFFFFu) == 0x80000u;
    const bool tie = !lo_zero && mid;
    in_range = sat || (hi >= 0x1p-60f && !tie);
  } else {
    const uint32_t mant = bh & 0x7FFFFFu;          // 1.5 * 2^e is mantissa 0x400000
    const uint32_t low = (bh >> 23) & 0xFFu;       // e + 127
    const bool up = mant > 0x400000u || (mant == 0x400000u && (lo_up || (lo_zero && (low & 1u))));
    c = low + (up ? 1u : 0u);
    in_range = hi >= 0x1p-100f && hi < 0x1p100f;
  }
  c = nonpos ? 0u : c;
  c = nan_in ? ((FMT == FMT_NVFP4) ? 0x7Fu : 0xFFu) : c;
  slow = !nan_in && (!ok_d || !ok_b || (!nonpos && !in_range));
  return c;
}

// A wave takes 256 MQ consecutive blocks: in round q < MQ lane l merges blocks
// 256 q + 4 l .. + 3 from one 4-byte scale load and one 16-byte delta load, so
// every load and store instruction moves one contiguous run (256 B of scales,
// 1 KB of deltas), and all rounds' loads are in flight before the first merge.
// The blocks the binary32 path cannot decide are redone after it.  VEC needs
// scales 4-byte and deltas 16-byte aligned; the blocks past the last whole chunk
// (and every block without VEC) go one per thread.
constexpr int MQ = 1;

template <int FMT, bool VEC>
__global__ __launch_bounds__(256) void merge_scales_kernel(const uint8_t* __restrict__ s_in,
                                                           const float* __restrict__ deltas, int64_t nb,
                                                           uint8_t* __restrict__ s_out) {
  int64_t done = 0;
  if (VEC) {
    const int64_t chunks = nb / (256 * MQ);
    const int lane = threadIdx.x & 63;
    const int64_t nwaves = (int64_t)gridDim.x * 4;
    for (int64_t ch = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 6; ch < chunks; ch += nwaves) {
      const int64_t b0 = ch * (256 * MQ) + 4 * lane;
      uint32_t sc[MQ];
      float4 dv[MQ];
#pragma unroll
      for (int q = 0; q < MQ; q++) {
        sc[q] = *reinterpret_cast<const uint32_t*>(s_in + b0 + 256 * q);
        dv[q] = *reinterpret_cast<const float4*>(deltas + b0 + 256 * q);
      }
#pragma unroll
      for (int q = 0; q < MQ; q++) {
        const float d4[4] = {dv[q].x, dv[q].y, dv[q].z, dv[q].w};
        uint32_t o = 0, redo = 0;
#pragma unroll
        for (int j = 0; j < 4; j++) {
          bool slow;
          o |= merge_fast<FMT>((sc[q] >> (8 * j)) & 0xFFu, d4[j], slow) << (8 * j);
          redo |= slow ? (1u << j) : 0u;
        }
        if (__builtin_expect(redo != 0u, 0)) {
          for (int j = 0; j < 4; j++)
            if ((redo >> j) & 1u)
              o = (o & ~(0xFFu << (8 * j))) | (merge_exact(FMT, (sc[q] >> (8 * j)) & 0xFFu, d4[j]) << (8 * j));
        }
        *reinterpret_cast<uint32_t*>(s_out + b0 + 256 * q) = o;
      }
    }
    done = chunks * (256 * MQ);
  }
  for (int64_t i = done + (int64_t)blockIdx.x * 256 + threadIdx.x; i < nb; i += (int64_t)gridDim.x * 256) {
    bool slow;
    uint32_t o = merge_fast<FMT>(s_in[i], deltas[i], slow);
    if (slow) o = merge_exact(FMT, s_in[i], deltas[i]);
    s_out[i] = (uint8_t)o;
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
    const bool vec = (reinterpret_cast<uintptr_t>(scales_in) & 3u) == 0 &&
                     (reinterpret_cast<uintptr_t>(scales_out) & 3u) == 0 &&
                     (reinterpret_cast<uintptr_t>(deltas) & 15u) == 0 && num_blocks >= 1024 * MQ;
    const int64_t gv = num_blocks / (1024 * MQ);              // one chunk per wave
    const int64_t gs = (num_blocks + 255) / 256;
    const dim3 grid((unsigned)((vec ? gv : gs) > 8192 ? 8192 : (vec ? gv : gs)));
#define FP4W_MERGE(F, V)                                                                             \
  hipLaunchKernelGGL((merge_scales_kernel<F, V>), grid, dim3(256), 0, stream, scales_in, deltas, num_blocks, \
                     scales_out)
    if (fmt == FMT_NVFP4) {
      if (vec) FP4W_MERGE(FMT_NVFP4, true); else FP4W_MERGE(FMT_NVFP4, false);
    } else {
      if (vec) FP4W_MERGE(FMT_MXFP4, true); else FP4W_MERGE(FMT_MXFP4, false);
    }
#undef FP4W_MERGE
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
