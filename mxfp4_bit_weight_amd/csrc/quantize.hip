// quantize.hip -- bf16 weights -> E2M1 codes + block scales on gfx950.
//
// NVFP4 ("max" calibration: scales recomputed from the current tensor each call,
// Nemotron 3.5 Lightning NVFP4 via QAD, section 03), two launches:
//   1. amax: each of G <= 512 workgroups writes the max of the |w| bits of its
//      chunk to its entry of a partial-max slot the library holds
//   2. encode: every workgroup first takes the max of the G entries (an integer
//      max: order-independent, so deterministic), derives s_t = fl32(A / 2688)
//      (workgroup 0 also writes it to the tensor-scale word), then each thread
//      takes ENC_U 16-element blocks: the E4M3 block scale and 16 codes each
// No atomics and no clearing: every entry a call reads was written by that
// call's amax launch, earlier on the same stream.  The slots are a device array
// (nothing is allocated per call), one per stream that has called (up to
// kAmaxSlots streams per device; more share slots).
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
// Otherwise (a midpoint lies inside the bracket) the one midpoint between the two
// codes is tested exactly with an fma sign (nvfp4_resolve).
#include <mutex>
#include <unordered_map>

#include "codec.hpp"
#include "fp4w_device.hpp"
#include "fp4w_internal.hpp"

namespace fp4w {

// Partial maxima of the NVFP4 amax: slot [stream][group], as |w| bf16 bits.
constexpr int kAmaxSlots = 64;
constexpr int kAmaxMaxGroups = 512;
__device__ __align__(256) uint32_t g_amax_part[kAmaxSlots][kAmaxMaxGroups];

__device__ __forceinline__ float tensor_scale_from_amax_word(uint32_t word) {
  float A = __uint_as_float(word << 16);     // the bf16 amax, exact in fp32
  return A / 2688.0f;                        // correctly rounded binary32 division
}

// |w| of a bf16 is its bit pattern without the sign; as unsigned integers these
// order like the values (NaN patterns above +inf above every finite value).
// A workgroup reads one contiguous chunk with AMAX_UNROLL loads in flight per
// thread, reduces across its waves in LDS and stores its maximum in its entry.
constexpr int AMAX_THREADS = 256;
constexpr int AMAX_UNROLL = 8;

__device__ __forceinline__ uint32_t amax_of(const uint4* v, uint32_t m) {
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
  return m;
}

// Two batches of AMAX_UNROLL loads alternate: the next batch is in flight while
// the current one is reduced, so a workgroup streams its chunk without a gap.
__global__ __launch_bounds__(AMAX_THREADS) void nvfp4_amax_kernel(const uint4* __restrict__ w, int64_t n16,
                                                                  int slot) {
  __shared__ uint32_t wmax[AMAX_THREADS / 64];
  const int64_t chunk = (n16 + gridDim.x - 1) / gridDim.x;
  const int64_t i0 = (int64_t)blockIdx.x * chunk;
  const int64_t i1 = i0 + chunk < n16 ? i0 + chunk : n16;
  constexpr int64_t STEP = (int64_t)AMAX_THREADS * AMAX_UNROLL;
  auto load = [&](uint4* v, int64_t i) {
#pragma unroll
    for (int u = 0; u < AMAX_UNROLL; u++) {
      const int64_t j = i + (int64_t)u * AMAX_THREADS;
      v[u] = j < i1 ? w[j] : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  uint32_t m = 0;
  uint4 va[AMAX_UNROLL], vb[AMAX_UNROLL];
  int64_t i = i0 + threadIdx.x;
  if (i0 < i1) load(va, i);
  for (; i0 < i1 && i < i1 + (int64_t)threadIdx.x; i += 2 * STEP) {
    const bool more_b = i + STEP - threadIdx.x < i1;
    if (more_b) load(vb, i + STEP);
    m = amax_of(va, m);
    if (!more_b) break;
    const bool more_a = i + 2 * STEP - threadIdx.x < i1;
    if (more_a) load(va, i + 2 * STEP);
    m = amax_of(vb, m);
    if (!more_a) break;
  }
  m = wave_max_u32(m);
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
#pragma unroll
    for (int q = 1; q < AMAX_THREADS / 64; q++) m = wmax[q] > m ? wmax[q] : m;
    g_amax_part[slot][blockIdx.x] = m;
  }
}

// s_t from the `groups` partial maxima of the slot (all threads of a 256-thread
// workgroup; the same value in every workgroup).
__device__ __forceinline__ float nvfp4_tensor_scale_of_slot(int slot, int groups) {
  __shared__ uint32_t red[4];
  uint32_t m = 0;
  for (int i = threadIdx.x; i < groups; i += 256) {
    const uint32_t v = g_amax_part[slot][i];
    m = v > m ? v : m;
  }
  m = wave_max_u32(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 4; q++) m = red[q] > m ? red[q] : m;
  return tensor_scale_from_amax_word(m);
}

typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));

// max |w| of a 16-element block (8 bf16 pairs) as an fp32 value: the sign bits
// cleared, then a packed 16-bit max tree (bit patterns order like magnitudes).
__device__ __forceinline__ float block_amax16(const uint32_t* wd) {
  u16x2_t m[4];
#pragma unroll
  for (int j = 0; j < 4; j++)
    m[j] = __builtin_elementwise_max(__builtin_bit_cast(u16x2_t, wd[2 * j] & 0x7FFF7FFFu),
                                     __builtin_bit_cast(u16x2_t, wd[2 * j + 1] & 0x7FFF7FFFu));
  const u16x2_t r = __builtin_elementwise_max(__builtin_elementwise_max(m[0], m[1]),
                                              __builtin_elementwise_max(m[2], m[3]));
  const uint32_t top = r.x > r.y ? r.x : r.y;
  return __uint_as_float(top << 16);
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

// 8 codes from 8 bf16 (4 dwords) at the two ends of the bracket.
__device__ __forceinline__ void nvfp4_codes_bracket(const uint32_t* wd, float inv_lo, float inv_hi, uint32_t& c_lo,
                                                    uint32_t& c_hi) {
  c_lo = 0u;
  c_hi = 0u;
  c_lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c_lo, bf16lo_f32(wd[0]) * inv_lo, bf16hi_f32(wd[0]) * inv_lo, 1.0f, 0);
  c_hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c_hi, bf16lo_f32(wd[0]) * inv_hi, bf16hi_f32(wd[0]) * inv_hi, 1.0f, 0);
  c_lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c_lo, bf16lo_f32(wd[1]) * inv_lo, bf16hi_f32(wd[1]) * inv_lo, 1.0f, 1);
  c_hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c_hi, bf16lo_f32(wd[1]) * inv_hi, bf16hi_f32(wd[1]) * inv_hi, 1.0f, 1);
  c_lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c_lo, bf16lo_f32(wd[2]) * inv_lo, bf16hi_f32(wd[2]) * inv_lo, 1.0f, 2);
  c_hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c_hi, bf16lo_f32(wd[2]) * inv_hi, bf16hi_f32(wd[2]) * inv_hi, 1.0f, 2);
  c_lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c_lo, bf16lo_f32(wd[3]) * inv_lo, bf16hi_f32(wd[3]) * inv_lo, 1.0f, 3);
  c_hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c_hi, bf16lo_f32(wd[3]) * inv_hi, bf16hi_f32(wd[3]) * inv_hi, 1.0f, 3);
}

// Codes of the elements whose bracket ends straddle a grid midpoint (their
// nibbles differ, by one step of magnitude): the sign of fma(mu d, s_t, -|w|)
// with mu the midpoint between the two decides exactly (mu d has at most 7
// significant bits, so it is exact, and the fma rounds once): above -> the upper
// code, on it -> the even one.  Such near-ties are not rare: 2688 = 2^7 * 3 * 7,
// so for many tensor maxima s_t sits within its rounding of a value that puts
// the midpoints 1.75 and 3.5 exactly on bf16 weights (about 1e-3 of elements).
template <int SEL>
__device__ __forceinline__ uint32_t nvfp4_resolve_pair(uint32_t out, uint32_t c_lo, uint32_t c_hi, uint32_t wdj,
                                                       float hd, float st) {
  const f32x2_t glo = fp4x2_to_f32x2<SEL>(c_lo, 1.0f), ghi = fp4x2_to_f32x2<SEL>(c_hi, 1.0f);
  const float a[2] = {__builtin_fabsf(bf16lo_f32(wdj)), __builtin_fabsf(bf16hi_f32(wdj))};
  const float gl[2] = {__builtin_fabsf(glo.x), __builtin_fabsf(glo.y)};
  const float gh[2] = {__builtin_fabsf(ghi.x), __builtin_fabsf(ghi.y)};
#pragma unroll
  for (int h = 0; h < 2; h++) {
    const int sh = 8 * SEL + 4 * h;
    const float r = __builtin_fmaf((gl[h] + gh[h]) * hd, st, -a[h]);     // sign(mu d s_t - |w|)
    const uint32_t mag = (c_lo >> sh) & 7u;
    const bool up = r < 0.0f || (r == 0.0f && (mag & 1u) != 0u);          // tie: the even code
    const bool differ = ((c_lo ^ c_hi) >> sh) & 0xFu;
    out += (differ && up) ? (1u << sh) : 0u;
  }
  return out;
}

__device__ __forceinline__ uint32_t nvfp4_resolve(uint32_t c_lo, uint32_t c_hi, const uint32_t* wd, float d,
                                                  float st) {
  const float hd = 0.5f * d;                                              // exact
  uint32_t out = c_lo;
  out = nvfp4_resolve_pair<0>(out, c_lo, c_hi, wd[0], hd, st);
  out = nvfp4_resolve_pair<1>(out, c_lo, c_hi, wd[1], hd, st);
  out = nvfp4_resolve_pair<2>(out, c_lo, c_hi, wd[2], hd, st);
  out = nvfp4_resolve_pair<3>(out, c_lo, c_hi, wd[3], hd, st);
  return out;
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
// Each thread takes ENC_U blocks per round, all loads issued first (a block per
// thread left too few bytes in flight to cover the memory latency).  The round
// is straight-line binary32 work: the block scale from a_b * (1 / (6 s_t)) with
// the near-midpoint test of nvfp4_block_scale_fast, 1 / (dec(sb) s_t) from
// v_rcp_f32 (1 ulp; the element quotients stay within 4 * 2^-24), the codes from
// the bracket.  Blocks that need the exact paths (a scale or code near a
// midpoint, or s_t outside [2^-64, 2^120]) are marked and redone after the
// round, so the common path has no branches.
constexpr int ENC_U = 2;

// RNE_sat(q) on the E4M3 grid for the binary32 q ~ a_b / (6 s_t) (relative error
// at most 2^-22, under 4 units of q's last place), or `near` where q lies
// within 8 units of a grid midpoint (the exact path decides).
__device__ __forceinline__ uint32_t e4m3_code_of_q(float q, bool& near) {
  const float t = q * 512.0f;                                   // subnormal step 2^-9
  const float f = t - __builtin_floorf(t);
  const uint32_t c_sub = (uint32_t)__builtin_rintf(t);
  const bool near_sub = __builtin_fabsf(f - 0.5f) < 0x1p-18f;
  uint32_t bq = __float_as_uint(q);
  const bool near_norm = ((bq & 0xFFFFFu) - 0x7FFF8u) <= 16u;
  bq += 0x7FFFFu + ((bq >> 20) & 1u);                           // round at bit 20, ties to even
  uint32_t c_norm = ((((bq >> 23) & 0xFFu) - 120u) << 3) | ((bq >> 20) & 7u);   // (e + 7) << 3 | m
  c_norm = c_norm > 0x7Eu ? 0x7Eu : c_norm;
  const bool sub = q < 0x1p-6f;
  const bool sat = !(q < 448.0f);
  near = !sat && (sub ? near_sub : near_norm);
  return sat ? 0x7Eu : (sub ? c_sub : c_norm);
}

template <bool FROZEN, bool FQ = false>
__global__ __launch_bounds__(256) void nvfp4_encode_kernel(const uint4* __restrict__ w, int64_t nblocks,
                                                           uint32_t* __restrict__ ts_word, int slot, int groups,
                                                           uint8_t* __restrict__ scales,
                                                           uint2* __restrict__ codes, uint4* __restrict__ fq = nullptr) {
  float st;
  if (FROZEN) {
    st = __uint_as_float(*ts_word);
  } else {
    st = nvfp4_tensor_scale_of_slot(slot, groups);
    if (blockIdx.x == 0 && threadIdx.x == 0) *reinterpret_cast<float*>(ts_word) = st;
  }
  const bool st_fast = st >= 0x1p-64f && st <= 0x1p120f;
  const bool tiny = !(st >= 0x1p-90f);
  const float r6 = __builtin_amdgcn_rcpf(6.0f * st);            // 1 / (6 s_t), within 2^-22
  for (int64_t r0 = (int64_t)blockIdx.x * 256 * ENC_U; r0 < nblocks; r0 += (int64_t)gridDim.x * 256 * ENC_U) {
    uint4 vv[ENC_U][2];
    uint32_t sbv[ENC_U];
#pragma unroll
    for (int u = 0; u < ENC_U; u++) {
      const int64_t b = r0 + u * 256 + threadIdx.x;
      const int64_t bl = b < nblocks ? b : 0;
      vv[u][0] = w[2 * bl];
      vv[u][1] = w[2 * bl + 1];
      if (FROZEN) sbv[u] = scales[bl];
    }
    uint2 outv[ENC_U];
    uint32_t redo = 0;                                           // bit u: block u takes the exact paths
#pragma unroll
    for (int u = 0; u < ENC_U; u++) {
      const uint32_t wd[8] = {vv[u][0].x, vv[u][0].y, vv[u][0].z, vv[u][0].w,
                              vv[u][1].x, vv[u][1].y, vv[u][1].z, vv[u][1].w};
      bool near = false;
      if (!FROZEN) sbv[u] = e4m3_code_of_q(block_amax16(wd) * r6, near);
      const float d = e4m3_to_f32(sbv[u]);
      const float inv = __builtin_amdgcn_rcpf(d * st);
      const float inv_lo = inv * (1.0f - 0x1p-21f), inv_hi = inv * (1.0f + 0x1p-21f);
      uint32_t lo0, hi0, lo1, hi1;
      nvfp4_codes_bracket(wd, inv_lo, inv_hi, lo0, hi0);
      nvfp4_codes_bracket(wd + 4, inv_lo, inv_hi, lo1, hi1);
      uint2 out = make_uint2(lo0, lo1);
      if (lo0 != hi0) out.x = nvfp4_resolve(lo0, hi0, wd, d, st);
      if (lo1 != hi1) out.y = nvfp4_resolve(lo1, hi1, wd + 4, d, st);
      const bool zero = !(d > 0.0f) || !(st > 0.0f);           // scale decodes to 0: signed zeros
      if (zero) out = make_uint2(sign_codes(wd), sign_codes(wd + 4));
      if (!st_fast || near) redo |= 1u << u;
      outv[u] = out;
    }
    if (__builtin_expect(redo != 0u, 0)) {
      // rare: the block's 32 bytes are loaded again rather than kept in registers
      for (int u = 0; u < ENC_U; u++) {
        if (!((redo >> u) & 1u)) continue;
        const int64_t b = r0 + u * 256 + threadIdx.x;
        const int64_t bl = b < nblocks ? b : 0;
        const uint4 v0 = w[2 * bl], v1 = w[2 * bl + 1];
        const uint32_t wd[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
        if (!FROZEN) sbv[u] = nvfp4_block_scale(block_amax16(wd), st);
        const float d = e4m3_to_f32(sbv[u]);
        if (!(d > 0.0f) || !(st > 0.0f))
          outv[u] = make_uint2(sign_codes(wd), sign_codes(wd + 4));
        else
          outv[u] = make_uint2(nvfp4_codes_exact(wd[0], wd[1], wd[2], wd[3], d, st),
                               nvfp4_codes_exact(wd[4], wd[5], wd[6], wd[7], d, st));
      }
    }
#pragma unroll
    for (int u = 0; u < ENC_U; u++) {
      const int64_t b = r0 + u * 256 + threadIdx.x;
      if (b >= nblocks) break;
      if (!FROZEN) scales[b] = (uint8_t)sbv[u];
      if (!FQ) {
        codes[b] = outv[u];
      } else {
        const float d = e4m3_to_f32(sbv[u]);
        const uint32_t cw[2] = {outv[u].x, outv[u].y};
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
}

// MXFP4: per 32-element block, e = clamp(floor(log2 a_b) - 2, -127, 127) read off
// the bf16 exponent field E (floor(log2) = E - 127 for normal values, and every
// subnormal or zero block clamps to -127), scale byte e + 127 = max(E - 2, 0);
// a block holding inf/NaN (E = 255) gets the NaN scale 0xFF.  The codes come from
// the scaled conversion, which divides by the power of two exactly and rounds to
// nearest even with saturation.
template <bool FROZEN>
__global__ __launch_bounds__(256) void mxfp4_encode_kernel(const uint4* __restrict__ w, int64_t nblocks,
                                                           uint8_t* __restrict__ scales,
                                                           uint4* __restrict__ codes) {
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
    codes[b] = make_uint4(c[0], c[1], c[2], c[3]);
  }
}

// MXFP4 fake-quant, whose bf16 output is as wide as its input: a wave takes 64
// blocks (4 KB of w) a round; load q of lane l is the 16 bytes at 1024 q + 16 l,
// quarter l % 4 of block 16 q + l / 4 (8 elements, one code dword), and its
// output goes to the same 16 bytes of the output, so every load and store of
// the wave moves one contiguous piece (one block per thread wrote 64 bytes a
// lane, each store instruction touching 64 separate half-lines).  The four
// lanes of a block reduce its maximum together.
template <bool FROZEN>
__global__ __launch_bounds__(256) void mxfp4_fake_quant_kernel(const uint4* __restrict__ w, int64_t nblocks,
                                                               uint8_t* __restrict__ scales,
                                                               uint4* __restrict__ fq) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, j = lane & 3;
  for (int64_t b0 = ((int64_t)blockIdx.x * 4 + wave) * 64; b0 < nblocks; b0 += (int64_t)gridDim.x * 256) {
    uint4 v[4];
    uint32_t scq[4];
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const int64_t bq = b0 + 16 * q + (lane >> 2);
      const bool ok = bq < nblocks;
      v[q] = ok ? w[4 * bq + j] : make_uint4(0u, 0u, 0u, 0u);
      if (FROZEN) scq[q] = ok ? scales[bq] : 0u;
    }
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const int64_t bq = b0 + 16 * q + (lane >> 2);
      const uint32_t wd[4] = {v[q].x, v[q].y, v[q].z, v[q].w};
      uint32_t sc;
      if (FROZEN) {
        sc = scq[q];
      } else {
        const u16x2_t m2 = __builtin_elementwise_max(
            __builtin_elementwise_max(__builtin_bit_cast(u16x2_t, wd[0] & 0x7FFF7FFFu),
                                      __builtin_bit_cast(u16x2_t, wd[1] & 0x7FFF7FFFu)),
            __builtin_elementwise_max(__builtin_bit_cast(u16x2_t, wd[2] & 0x7FFF7FFFu),
                                      __builtin_bit_cast(u16x2_t, wd[3] & 0x7FFF7FFFu)));
        uint32_t m = m2.x > m2.y ? (uint32_t)m2.x : (uint32_t)m2.y;
        uint32_t o = (uint32_t)__shfl_xor((int)m, 1, 64);
        m = o > m ? o : m;
        o = (uint32_t)__shfl_xor((int)m, 2, 64);
        m = o > m ? o : m;
        const uint32_t E = (m >> 7) & 0xFFu;
        sc = (E == 0xFFu) ? 0xFFu : (E > 2u ? E - 2u : 0u);
      }
      const float s = e8m0_scale_operand(sc);
      uint32_t c = 0u;
      c = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(c, as_bf16x2(wd[0]), s, 0);
      c = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(c, as_bf16x2(wd[1]), s, 1);
      c = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(c, as_bf16x2(wd[2]), s, 2);
      c = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(c, as_bf16x2(wd[3]), s, 3);
      if (bq >= nblocks) continue;
      if (!FROZEN && j == 0) scales[bq] = (uint8_t)sc;
      {
        // the 8 values decoded from the codes as dequantize does (codec.hpp)
        uint32_t o[4];
        if (sc < 0xFDu) {
          o[0] = fp4x2_to_bf16x2_scaled<0>(c, s);
          o[1] = fp4x2_to_bf16x2_scaled<1>(c, s);
          o[2] = fp4x2_to_bf16x2_scaled<2>(c, s);
          o[3] = fp4x2_to_bf16x2_scaled<3>(c, s);
        } else {
          float vv[8];
          mx_plain8(c, sc, vv);
#pragma unroll
          for (int e = 0; e < 4; e++) o[e] = f32_to_bf16_rne(vv[2 * e]) | (f32_to_bf16_rne(vv[2 * e + 1]) << 16);
        }
        fq[4 * bq + j] = make_uint4(o[0], o[1], o[2], o[3]);
      }
    }
  }
}

// The partial-max slot of the calling stream on the current device.
namespace {
constexpr int kMaxDevices = 64;
std::mutex g_slot_mu;
std::unordered_map<hipStream_t, int> g_slot_of[kMaxDevices];
int g_slot_next[kMaxDevices];
}  // namespace

static hipError_t amax_slot(hipStream_t stream, int* slot) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_slot_mu);
  auto& map = g_slot_of[dev];
  auto it = map.find(stream);
  if (it != map.end()) {
    *slot = it->second;
    return hipSuccess;
  }
  if (map.size() >= 4096) map.clear();            // stale handles of destroyed streams
  const int s = g_slot_next[dev]++ % kAmaxSlots;
  map[stream] = s;
  *slot = s;
  return hipSuccess;
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
      int slot = 0;
      hipError_t e = amax_slot(stream, &slot);
      if (e != hipSuccess) return e;
      // up to 2 workgroups per CU, each at least 32 KiB of the tensor
      const int groups = grid_for(count / 8, AMAX_THREADS * AMAX_UNROLL, kAmaxMaxGroups);
      hipLaunchKernelGGL(nvfp4_amax_kernel, dim3(groups), dim3(AMAX_THREADS), 0, stream,
                         reinterpret_cast<const uint4*>(w), count / 8, slot);
      hipLaunchKernelGGL(nvfp4_encode_kernel<false>, dim3(grid_for(nblocks, 256 * ENC_U, 8192)), dim3(256), 0,
                         stream, reinterpret_cast<const uint4*>(w), nblocks, word, slot, groups, scales,
                         reinterpret_cast<uint2*>(codes));
    } else {
      hipLaunchKernelGGL(nvfp4_encode_kernel<true>, dim3(grid_for(nblocks, 256 * ENC_U, 8192)), dim3(256), 0,
                         stream, reinterpret_cast<const uint4*>(w), nblocks, word, 0, 0, scales,
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
      int slot = 0;
      hipError_t e = amax_slot(stream, &slot);
      if (e != hipSuccess) return e;
      const int groups = grid_for(count / 8, AMAX_THREADS * AMAX_UNROLL, kAmaxMaxGroups);
      hipLaunchKernelGGL(nvfp4_amax_kernel, dim3(groups), dim3(AMAX_THREADS), 0, stream, wv, count / 8, slot);
      hipLaunchKernelGGL((nvfp4_encode_kernel<false, true>), dim3(grid_for(nblocks, 256 * ENC_U, 8192)), dim3(256),
                         0, stream, wv, nblocks, word, slot, groups, scales, nullptr, fq);
    } else {
      hipLaunchKernelGGL((nvfp4_encode_kernel<true, true>), dim3(grid_for(nblocks, 256 * ENC_U, 8192)), dim3(256),
                         0, stream, wv, nblocks, word, 0, 0, scales, nullptr, fq);
    }
  } else {
    const int64_t nblocks = count / 32;
    if (!frozen)
      hipLaunchKernelGGL(mxfp4_fake_quant_kernel<false>, dim3(grid_for(nblocks, 256, 16384)), dim3(256), 0, stream,
                         wv, nblocks, scales, fq);
    else
      hipLaunchKernelGGL(mxfp4_fake_quant_kernel<true>, dim3(grid_for(nblocks, 256, 16384)), dim3(256), 0, stream,
                         wv, nblocks, scales, fq);
  }
  return hipGetLastError();
}

}  // namespace fp4w
