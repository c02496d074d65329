// quantize.hip -- bf16 weights -> E2M1 codes + block scales on gfx950.
//
// NVFP4 ("max" calibration: scales recomputed from the current tensor each call,
// Nemotron 3.5 Lightning NVFP4 via QAD, section 03):
//   1. zero the tensor-scale word          (1 thread)
//   2. amax: integer atomicMax of |w| bits  (order-independent, so deterministic)
//   3. encode: one thread per 16-element block reads the amax, derives
//      s_t = fl32(A / 2688), the E4M3 block scale and 16 codes
//   4. finalize: overwrite the word with s_t (1 thread)
// MXFP4: one pass, one thread per 32-element block.
// Frozen scales (same page, frozen-scale QAD): only the codes are recomputed.
// Fused fake-quant (launch_fake_quant): the same passes, the encode writing the
// values decoded from its codes (bf16, as dequantize rounds them) instead of the
// codes -- the quantize-dequantize a training forward inserts (QATFactory page,
// section on how training repeats the engine's arithmetic).
//
// Exactness of the NVFP4 element codes: q = |w| / (dec(sb) s_t) is evaluated in
// binary32 with a relative error below 4 * 2^-24; the code is converted from the
// bracket q(1 - 2^-21) and q(1 + 2^-21).  Rounding to the E2M1 grid is monotone,
// so when both ends give the same code it is the code of the exact quotient.
// Otherwise (a midpoint lies inside the bracket, about 3e-6 of elements) the
// lane recomputes its codes with exact fma sign tests.
#include "codec.hpp"
#include "fp4w_device.hpp"
#include "fp4w_internal.hpp"

namespace fp4w {

__global__ void nvfp4_amax_zero_kernel(uint32_t* word) { *word = 0u; }

// |w| of a bf16 is its bit pattern without the sign; as unsigned integers these
// order like the values (NaN patterns above +inf above every finite value).
// A workgroup reads one contiguous chunk with AMAX_UNROLL loads in flight per
// thread, reduces across its waves in LDS and offers its maximum with a single
// atomic, skipped when the word already holds as much (atomics on one address
// are serialized, so their number, not the reads, would otherwise set the time).
constexpr int AMAX_THREADS = 256;
constexpr int AMAX_UNROLL = 8;

__global__ __launch_bounds__(AMAX_THREADS) void nvfp4_amax_kernel(const uint4* __restrict__ w, int64_t n16,
                                                                  uint32_t* __restrict__ word) {
  __shared__ uint32_t wmax[AMAX_THREADS / 64];
  const int64_t chunk = (n16 + gridDim.x - 1) / gridDim.x;
  const int64_t i0 = (int64_t)blockIdx.x * chunk;
  const int64_t i1 = i0 + chunk < n16 ? i0 + chunk : n16;
  uint32_t m = 0;
  for (int64_t i = i0 + threadIdx.x; i < i1; i += (int64_t)AMAX_THREADS * AMAX_UNROLL) {
    uint4 v[AMAX_UNROLL];
#pragma unroll
    for (int u = 0; u < AMAX_UNROLL; u++) {
      const int64_t j = i + (int64_t)u * AMAX_THREADS;
      v[u] = j < i1 ? w[j] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < AMAX_UNROLL; u++) {
      const uint32_t a[4] = {v[u].x & 0x7FFF7FFFu, v[u].y & 0x7FFF7FFFu, v[u].z & 0x7FFF7FFFu, v[u].w & 0x7FFF7FFFu};
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const uint32_t lo = a[q] & 0xFFFFu, hi = a[q] >> 16;
        m = lo > m ? lo : m;
        m = hi > m ? hi : m;
      }
    }
  }
  m = wave_max_u32(m);
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
#pragma unroll
    for (int q = 1; q < AMAX_THREADS / 64; q++) m = wmax[q] > m ? wmax[q] : m;
    const uint32_t cur = __hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (m > cur) atomicMax(word, m);
  }
}

__device__ __forceinline__ float tensor_scale_from_amax_word(uint32_t word) {
  float A = __uint_as_float(word << 16);     // the bf16 amax, exact in fp32
  return A / 2688.0f;                        // correctly rounded binary32 division
}

__global__ void nvfp4_finalize_kernel(uint32_t* word) {
  float st = tensor_scale_from_amax_word(*word);
  *reinterpret_cast<float*>(word) = st;
}

// Exact codes of 8 elements (one packed dword) for block scale d and tensor scale st.
__device__ __noinline__ uint32_t nvfp4_codes_exact(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3,
                                                   float d, float st) {
  uint32_t words[4] = {w0, w1, w2, w3};
  uint32_t out = 0;
#pragma unroll
  for (int j = 0; j < 4; j++) {
#pragma unroll
    for (int h = 0; h < 2; h++) {
      uint32_t bits = h ? (words[j] >> 16) : (words[j] & 0xFFFFu);
      float a = __uint_as_float((bits & 0x7FFFu) << 16);
      uint32_t code = e2m1_code_exact(a, d, st) | ((bits >> 12) & 0x8u);
      out |= code << (8 * j + 4 * h);
    }
  }
  return out;
}

// 8 codes from 8 bf16 (4 dwords) with the bracket test; sets `slow` when the
// bracket straddles a midpoint.
__device__ __forceinline__ uint32_t nvfp4_codes_fast(const uint32_t* wd, float inv_lo, float inv_hi,
                                                     bool& slow) {
  uint32_t c_lo = 0, c_hi = 0;
  c_lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c_lo, bf16lo_f32(wd[0]) * inv_lo, bf16hi_f32(wd[0]) * inv_lo, 1.0f, 0);
  c_hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c_hi, bf16lo_f32(wd[0]) * inv_hi, bf16hi_f32(wd[0]) * inv_hi, 1.0f, 0);
  c_lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c_lo, bf16lo_f32(wd[1]) * inv_lo, bf16hi_f32(wd[1]) * inv_lo, 1.0f, 1);
  c_hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c_hi, bf16lo_f32(wd[1]) * inv_hi, bf16hi_f32(wd[1]) * inv_hi, 1.0f, 1);
  c_lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c_lo, bf16lo_f32(wd[2]) * inv_lo, bf16hi_f32(wd[2]) * inv_lo, 1.0f, 2);
  c_hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c_hi, bf16lo_f32(wd[2]) * inv_hi, bf16hi_f32(wd[2]) * inv_hi, 1.0f, 2);
  c_lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c_lo, bf16lo_f32(wd[3]) * inv_lo, bf16hi_f32(wd[3]) * inv_lo, 1.0f, 3);
  c_hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c_hi, bf16lo_f32(wd[3]) * inv_hi, bf16hi_f32(wd[3]) * inv_hi, 1.0f, 3);
  slow = slow || (c_lo != c_hi);
  return c_lo;
}

// Signed-zero codes of 8 bf16 (a block whose scale decodes to 0).
__device__ __forceinline__ uint32_t sign_codes(const uint32_t* wd) {
  uint32_t out = 0;
#pragma unroll
  for (int j = 0; j < 4; j++) {
    out |= ((wd[j] >> 12) & 0x8u) << (8 * j);          // element 2j   : bit 15 -> bit 3
    out |= ((wd[j] >> 28) & 0x8u) << (8 * j + 4);      // element 2j+1 : bit 31 -> bit 3
  }
  return out;
}

// FQ: fused fake-quant -- instead of the codes, write the block's 16 values
// decoded from them as dequantize does (codec.hpp), 32 bytes of bf16 (fq).
template <bool FROZEN, bool FQ = false>
__global__ __launch_bounds__(256) void nvfp4_encode_kernel(const uint4* __restrict__ w, int64_t nblocks,
                                                           const uint32_t* __restrict__ ts_word,
                                                           uint8_t* __restrict__ scales,
                                                           uint2* __restrict__ codes, uint4* __restrict__ fq = nullptr) {
  const uint32_t tw = *ts_word;
  const float st = FROZEN ? __uint_as_float(tw) : tensor_scale_from_amax_word(tw);
  const bool st_fast = st >= 0x1p-64f && st <= 0x1p120f;
  const bool tiny = !(st >= 0x1p-90f);
  for (int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x; b < nblocks; b += (int64_t)gridDim.x * 256) {
    uint4 v0 = w[2 * b];
    uint4 v1 = w[2 * b + 1];
    uint32_t wd[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    uint32_t sb;
    if (FROZEN) {
      sb = scales[b];
    } else {
      uint32_t m = 0;
#pragma unroll
      for (int j = 0; j < 8; j++) {
        uint32_t a = wd[j] & 0x7FFF7FFFu;
        uint32_t lo = a & 0xFFFFu, hi = a >> 16;
        m = lo > m ? lo : m;
        m = hi > m ? hi : m;
      }
      sb = nvfp4_block_scale(__uint_as_float(m << 16), st);
      scales[b] = (uint8_t)sb;
    }
    const float d = e4m3_to_f32(sb);
    uint2 out;
    if (!(d > 0.0f) || !(st > 0.0f)) {
      // scale decodes to 0 (or is not a valid positive scale): signed zeros
      out.x = sign_codes(wd);
      out.y = sign_codes(wd + 4);
    } else {
      bool slow = !st_fast;
      if (st_fast) {
        const float inv = 1.0f / (d * st);
        const float inv_lo = inv * (1.0f - 0x1p-21f);
        const float inv_hi = inv * (1.0f + 0x1p-21f);
        out.x = nvfp4_codes_fast(wd, inv_lo, inv_hi, slow);
        out.y = nvfp4_codes_fast(wd + 4, inv_lo, inv_hi, slow);
      }
      if (slow) {
        out.x = nvfp4_codes_exact(wd[0], wd[1], wd[2], wd[3], d, st);
        out.y = nvfp4_codes_exact(wd[4], wd[5], wd[6], wd[7], d, st);
      }
    }
    if (!FQ) {
      codes[b] = out;
    } else {
      const uint32_t cw[2] = {out.x, out.y};
      uint32_t o[8];
      float f0, f1;
#pragma unroll
      for (int j = 0; j < 2; j++) {
        nvfp4_pair(fp4x2_to_f32x2<0>(cw[j], 1.0f), d, st, tiny, f0, f1, o[4 * j + 0], true);
        nvfp4_pair(fp4x2_to_f32x2<1>(cw[j], 1.0f), d, st, tiny, f0, f1, o[4 * j + 1], true);
        nvfp4_pair(fp4x2_to_f32x2<2>(cw[j], 1.0f), d, st, tiny, f0, f1, o[4 * j + 2], true);
        nvfp4_pair(fp4x2_to_f32x2<3>(cw[j], 1.0f), d, st, tiny, f0, f1, o[4 * j + 3], true);
      }
      fq[2 * b] = make_uint4(o[0], o[1], o[2], o[3]);
      fq[2 * b + 1] = make_uint4(o[4], o[5], o[6], o[7]);
    }
  }
}

// MXFP4: per 32-element block, e = clamp(floor(log2 a_b) - 2, -127, 127) read off
// the bf16 exponent field E (floor(log2) = E - 127 for normal values, and every
// subnormal or zero block clamps to -127), scale byte e + 127 = max(E - 2, 0);
// a block holding inf/NaN (E = 255) gets the NaN scale 0xFF.  The codes come from
// the scaled conversion, which divides by the power of two exactly and rounds to
// nearest even with saturation.
template <bool FROZEN, bool FQ = false>
__global__ __launch_bounds__(256) void mxfp4_encode_kernel(const uint4* __restrict__ w, int64_t nblocks,
                                                           uint8_t* __restrict__ scales,
                                                           uint4* __restrict__ codes, uint4* __restrict__ fq = nullptr) {
  for (int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x; b < nblocks; b += (int64_t)gridDim.x * 256) {
    uint32_t wd[16];
#pragma unroll
    for (int q = 0; q < 4; q++) {
      uint4 v = w[4 * b + q];
      wd[4 * q + 0] = v.x; wd[4 * q + 1] = v.y; wd[4 * q + 2] = v.z; wd[4 * q + 3] = v.w;
    }
    uint32_t sc;
    if (FROZEN) {
      sc = scales[b];
    } else {
      uint32_t m = 0;
#pragma unroll
      for (int j = 0; j < 16; j++) {
        uint32_t a = wd[j] & 0x7FFF7FFFu;
        uint32_t lo = a & 0xFFFFu, hi = a >> 16;
        m = lo > m ? lo : m;
        m = hi > m ? hi : m;
      }
      uint32_t E = (m >> 7) & 0xFFu;
      sc = (E == 0xFFu) ? 0xFFu : (E > 2u ? E - 2u : 0u);
      scales[b] = (uint8_t)sc;
    }
    const float s = e8m0_scale_operand(sc);
    uint32_t c[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int q = 0; q < 4; q++) {
      c[q] = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(c[q], as_bf16x2(wd[4 * q + 0]), s, 0);
      c[q] = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(c[q], as_bf16x2(wd[4 * q + 1]), s, 1);
      c[q] = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(c[q], as_bf16x2(wd[4 * q + 2]), s, 2);
      c[q] = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(c[q], as_bf16x2(wd[4 * q + 3]), s, 3);
    }
    if (!FQ) {
      codes[b] = make_uint4(c[0], c[1], c[2], c[3]);
    } else {
      // the 32 values decoded from the codes as dequantize does (codec.hpp)
      uint32_t o[16];
      if (sc < 0xFDu) {
#pragma unroll
        for (int j = 0; j < 4; j++) {
          o[4 * j + 0] = fp4x2_to_bf16x2_scaled<0>(c[j], s);
          o[4 * j + 1] = fp4x2_to_bf16x2_scaled<1>(c[j], s);
          o[4 * j + 2] = fp4x2_to_bf16x2_scaled<2>(c[j], s);
          o[4 * j + 3] = fp4x2_to_bf16x2_scaled<3>(c[j], s);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; j++) {
          float v[8];
          mx_plain8(c[j], sc, v);
#pragma unroll
          for (int e = 0; e < 4; e++)
            o[4 * j + e] = f32_to_bf16_rne(v[2 * e]) | (f32_to_bf16_rne(v[2 * e + 1]) << 16);
        }
      }
#pragma unroll
      for (int q = 0; q < 4; q++) fq[4 * b + q] = make_uint4(o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]);
    }
  }
}

static int grid_for(int64_t items, int per_block = 256, int max_blocks = 8192) {
  int64_t g = (items + per_block - 1) / per_block;
  if (g < 1) g = 1;
  if (g > max_blocks) g = max_blocks;
  return (int)g;
}

hipError_t launch_quantize(int fmt, const void* w, int64_t n, int64_t k, uint8_t* codes, uint8_t* scales,
                           float* tensor_scale, bool frozen, hipStream_t stream) {
  const int64_t count = n * k;
  if (count == 0) return hipSuccess;
  if (fmt == FMT_NVFP4) {
    const int64_t nblocks = count / 16;
    uint32_t* word = reinterpret_cast<uint32_t*>(tensor_scale);
    if (!frozen) {
      hipLaunchKernelGGL(nvfp4_amax_zero_kernel, dim3(1), dim3(1), 0, stream, word);
      // about 4 workgroups per CU, each at least 32 KiB of the tensor
      hipLaunchKernelGGL(nvfp4_amax_kernel, dim3(grid_for(count / 8, AMAX_THREADS * AMAX_UNROLL, 1024)),
                         dim3(AMAX_THREADS), 0, stream, reinterpret_cast<const uint4*>(w), count / 8, word);
      hipLaunchKernelGGL(nvfp4_encode_kernel<false>, dim3(grid_for(nblocks, 256, 16384)), dim3(256), 0, stream,
                         reinterpret_cast<const uint4*>(w), nblocks, word, scales,
                         reinterpret_cast<uint2*>(codes));
      hipLaunchKernelGGL(nvfp4_finalize_kernel, dim3(1), dim3(1), 0, stream, word);
    } else {
      hipLaunchKernelGGL(nvfp4_encode_kernel<true>, dim3(grid_for(nblocks, 256, 16384)), dim3(256), 0, stream,
                         reinterpret_cast<const uint4*>(w), nblocks, word, scales,
                         reinterpret_cast<uint2*>(codes));
    }
  } else {
    const int64_t nblocks = count / 32;
    if (!frozen)
      hipLaunchKernelGGL(mxfp4_encode_kernel<false>, dim3(grid_for(nblocks, 256, 16384)), dim3(256), 0, stream,
                         reinterpret_cast<const uint4*>(w), nblocks, scales, reinterpret_cast<uint4*>(codes));
    else
      hipLaunchKernelGGL(mxfp4_encode_kernel<true>, dim3(grid_for(nblocks, 256, 16384)), dim3(256), 0, stream,
                         reinterpret_cast<const uint4*>(w), nblocks, scales, reinterpret_cast<uint4*>(codes));
  }
  return hipGetLastError();
}

hipError_t launch_fake_quant(int fmt, const void* w, int64_t n, int64_t k, void* out, uint8_t* scales,
                             float* tensor_scale, bool frozen, hipStream_t stream) {
  const int64_t count = n * k;
  if (count == 0) return hipSuccess;
  const uint4* wv = reinterpret_cast<const uint4*>(w);
  uint4* fq = reinterpret_cast<uint4*>(out);
  if (fmt == FMT_NVFP4) {
    const int64_t nblocks = count / 16;
    uint32_t* word = reinterpret_cast<uint32_t*>(tensor_scale);
    if (!frozen) {
      hipLaunchKernelGGL(nvfp4_amax_zero_kernel, dim3(1), dim3(1), 0, stream, word);
      hipLaunchKernelGGL(nvfp4_amax_kernel, dim3(grid_for(count / 8, AMAX_THREADS * AMAX_UNROLL, 1024)),
                         dim3(AMAX_THREADS), 0, stream, wv, count / 8, word);
      hipLaunchKernelGGL((nvfp4_encode_kernel<false, true>), dim3(grid_for(nblocks, 256, 16384)), dim3(256), 0,
                         stream, wv, nblocks, word, scales, nullptr, fq);
      hipLaunchKernelGGL(nvfp4_finalize_kernel, dim3(1), dim3(1), 0, stream, word);
    } else {
      hipLaunchKernelGGL((nvfp4_encode_kernel<true, true>), dim3(grid_for(nblocks, 256, 16384)), dim3(256), 0,
                         stream, wv, nblocks, word, scales, nullptr, fq);
    }
  } else {
    const int64_t nblocks = count / 32;
    if (!frozen)
      hipLaunchKernelGGL((mxfp4_encode_kernel<false, true>), dim3(grid_for(nblocks, 256, 16384)), dim3(256), 0,
                         stream, wv, nblocks, scales, nullptr, fq);
    else
      hipLaunchKernelGGL((mxfp4_encode_kernel<true, true>), dim3(grid_for(nblocks, 256, 16384)), dim3(256), 0,
                         stream, wv, nblocks, scales, nullptr, fq);
  }
  return hipGetLastError();
}

}  // namespace fp4w
