// decode_xs.hip -- the decode-shaped W4A16 product for 1 <= m <= 16 rows of x,
// with x held in registers while the weight codes stream past it.
//
// Each decode step streams every weight code once, so the product is bound by
// memory traffic (tggo.me/sberlogasci/42740, section "Eksperimenty").  The
// arithmetic is 16-bit activations times decoded 4-bit weights with fp32
// accumulation (QATFactory page, section on how training repeats the engine's
// arithmetic).  Here every weight is decoded exactly to a 16-bit float in
// registers and fed to a 16x16x32 MFMA whose 16 rows are the rows of x, so the
// matrix core work does not grow with m up to 16:
//
//   NVFP4: e2m1 * e4m3 has at most 6 significant bits and lies in [2^-10, 2688],
//          so it is an exact fp16 value: v_cvt_scalef32_pk_f16_fp4 (two codes)
//          and one v_pk_mul_f16 by the block scale (two weights), then
//          v_mfma_f32_16x16x32_f16.  x is brought to fp16 by a power of two
//          per (row, wave): x~ = x * 2^-E with E = floor(log2 max|x|) - 14 over
//          the wave's K range, exact for every element within 2^28 of that
//          maximum (smaller ones round in fp16's subnormal range, an error below
//          2^-38 of the maximum).  The fp32 partial is multiplied back by 2^E.
//   MXFP4: the E8M0 scale is a power of two and rides in the conversion
//          (v_cvt_scalef32_pk_bf16_fp4): e2m1 * 2^e exactly in bf16, x as it is,
//          v_mfma_f32_16x16x32_bf16.  A block whose scale is 0xFF (NaN) turns
//          its whole column NaN.  Like the bf16 output of dequantize, products
//          whose decoded weight exceeds bf16's range (scale codes 253, 254 with
//          large codes) become infinite.
//
// A row of x holding an Inf or NaN turns its whole output row NaN.
//
// Work split.  K is cut into 32-wide groups.  A workgroup of nw waves owns one
// span of K (S spans in all) and every G-th 16-row weight tile from its run
// index on (G runs).  Wave w of the span takes groups qw0 + 4u + g (u < CPW) for
// lane group g = lane / 16, so each code load moves 64 contiguous bytes of
// each of the tile's 16 rows.  The wave loads its part of x once (lane (r, g)
// holds row r of those groups: the MFMA's A operand) and then streams the
// tiles, P tiles of code and scale loads in flight.  MFMA (u, sub) takes the
// dword sub of the lane's 16 code bytes: weight row n = lane % 16 and k =
// 32 q(u) + 8 sub + 0..7 on both operands.  Partials are added in LDS in wave
// order; with S > 1 spans the last workgroup of a run to arrive adds the spans'
// partials in span order, so results never depend on scheduling.
#include "fp4w_device.hpp"
#include "fp4w_internal.hpp"
#include "gemm_common.hpp"
#include "lora_handover.hpp"
#include "sync.hpp"

namespace fp4w {

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));

constexpr int XS_ROWS = 16;          // weight rows per tile (MFMA columns)
constexpr int XS_MAX_M = 16;         // rows of x (MFMA rows)
constexpr int XS_MAX_R = 64;         // LoRA rank
constexpr int XS_MAX_WAVES = 16;
constexpr int XS_CPW = 2;            // 32-wide K groups per lane
constexpr int XS_SC_UNITS = 4;       // staged scale units per thread at most
constexpr int XS_RING = 2;           // tiles of code loads in flight per wave

// LDS of one workgroup (byte offsets):
//   red   [nw][tg][m][16] fp32   wave partials of each tile
//   tred  [nw][m][r] fp32        LoRA: wave partials of one K chunk of t = x A^T
//   lb    [tg * 16][r] bf16      the LoRA B rows of the tiles
//   lt    [m][r] fp32            t over the span
//   ssc   [tg * 16][span_bytes]   block-scale bytes of the tiles' rows over the span
//                                 (staged mode; span_bytes = scale bytes of qspan groups)
//   gain  [nw][256] fp32          noisy RMSNorm: gamma (1 + sigma noise) over each wave's K groups
//   ss    [16][nw4] fp32          noisy RMSNorm: each wave's sums of x^2 of the rows
//                                 (nw4 = nw rounded up to 4; the slots past nw hold 0)
// (every region starts 16-byte aligned)
struct XsLayout {
  int red_off, tred_off, lb_off, lt_off, ssc_off, gain_off, ss_off, bytes;
};
__host__ __device__ inline XsLayout xs_layout(int m, int nw, int tg, int r, int span_bytes, bool aqn = false) {
  XsLayout L;
  int off = 0;
  L.red_off = off;  off += nw * tg * m * XS_ROWS * 4;
  L.tred_off = off; off += (nw * m * r * 4 + 15) & ~15;
  L.lb_off = off;   off += (tg * XS_ROWS * r * 2 + 15) & ~15;
  L.lt_off = off;   off += (m * r * 4 + 15) & ~15;
  L.ssc_off = off;  off += tg * XS_ROWS * span_bytes;
  L.gain_off = off; off += aqn ? nw * 128 * XS_CPW * 4 : 0;
  L.ss_off = off;   off += aqn ? XS_ROWS * ((nw + 3) & ~3) * 4 : 0;
  L.bytes = off;
  return L;
}

// The noisy RMSNorm ahead of the product (one span of K only): row m of x enters
// as bf16(x gamma (1 + sigma noise)), and the row's sums are multiplied by
// 1 / sqrt(mean_k x^2 + eps) at the end.
struct XsAqn {
  const uint16_t* gamma;    // (K) bf16
  const float* noise;       // (K) fp32
  float sigma, eps;
};

__device__ __forceinline__ f16x8_t bits_as_f16x8(u32x4_t v) { return __builtin_bit_cast(f16x8_t, v); }
__device__ __forceinline__ bf16x8_t bits_as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

// 8 E2M1 codes (one dword, low nibble first) times the E4M3 block scale held in
// both halves of s2, as 8 exact fp16 values.
__device__ __forceinline__ f16x8_t codes8_to_f16(uint32_t dw, f16x2_t s2) {
  const f16x2_t v0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(dw, 1.0f, 0) * s2;
  const f16x2_t v1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(dw, 1.0f, 1) * s2;
  const f16x2_t v2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(dw, 1.0f, 2) * s2;
  const f16x2_t v3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(dw, 1.0f, 3) * s2;
  return f16x8_t{v0.x, v0.y, v1.x, v1.y, v2.x, v2.y, v3.x, v3.y};
}

// 8 E2M1 codes times the power of two in `pow2`'s exponent field, as 8 exact bf16.
__device__ __forceinline__ bf16x8_t codes8_to_bf16_pow2(uint32_t dw, float pow2) {
  u32x4_t r;
  r.x = fp4x2_to_bf16x2_scaled<0>(dw, pow2);
  r.y = fp4x2_to_bf16x2_scaled<1>(dw, pow2);
  r.z = fp4x2_to_bf16x2_scaled<2>(dw, pow2);
  r.w = fp4x2_to_bf16x2_scaled<3>(dw, pow2);
  return bits_as_bf16x8(r);
}

// The product of one workgroup: span s of K, tile run gi, M <= 16 rows of x.
// SC: 1 = the block scales of the tiles are staged in LDS by the whole workgroup with
// 16-byte loads (each scale line is fetched once); 0 = every lane loads its own
// bytes (any alignment).  xrow: nullptr = row m of x is x[m]; otherwise row m is
// x[xrow[m]] of xrows rows, and a row index outside [0, xrows) makes the output
// row NaN (the routed rows of an expert).
// LORA: t = x A^T comes from the launch's chunk workgroups (lora_handover.hpp):
// wave 0 waits for it in the epilogue, reader `rd` of `nread`, and span 0 adds
// t B^T to its outputs.
// AQN (S = 1 only): the noisy RMSNorm of `aq` is applied to x on the way in, its
// row factor to the sums on the way out (t then comes from gained x as well).
template <int FMT, int TG, int SC, bool LORA, bool AQN>
__device__ __forceinline__ void xs_body(
    uint8_t* __restrict__ lds, int* flag, int* have_t, const uint16_t* __restrict__ x,
    const int32_t* __restrict__ xrow, int64_t xrows, int M, int64_t K, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ scales, const float* __restrict__ tensor_scale, int64_t N,
    const uint16_t* __restrict__ lora_a, const uint16_t* __restrict__ lora_b, int r, int lparts, int lsw,
    uint32_t* __restrict__ lsync, uint64_t wait_ticks, uint16_t* __restrict__ y, float* __restrict__ part,
    uint32_t* __restrict__ cnt, int S, int qspan, int ntiles, int G, int tg, int lb16, int s, int gi, int rd,
    int nread, XsAqn aq) {
  constexpr int CPW = XS_CPW;
  const int nt = (int)blockDim.x;
  const int nw = nt >> 6;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);      // uniform: buffer descriptors stay scalar
  // tiles gi, gi + G, gi + 2 G, ...: at each step the G runs read one contiguous
  // stretch of the weight matrix
  const int ntg = (ntiles - gi + G - 1) / G;                         // 1 .. tg <= TG
  auto tile_of = [&](int ti) -> int64_t { return (int64_t)gi + (int64_t)ti * G; };
  const int nq = (int)(K >> 5);
  const int qs1 = min((s + 1) * qspan, nq);
  const int qw0 = s * qspan + wave * 4 * CPW;
  const int n = lane & 15, g = lane >> 4;
  const int rr = LORA ? r : 0;                     // LoRA rank (0: none)
  constexpr uint32_t SB = FMT == FMT_NVFP4 ? 2u : 1u;              // scale bytes per 32-wide group
  const int span_bytes = SC ? (int)SB * qspan : 0;
  const XsLayout L = xs_layout(M, nw, tg, rr, span_bytes, AQN);

  // lane (n, g) takes the 32-wide K groups q(u) = qw0 + 4 u + g of the span
  bool qok[CPW];
  uint32_t qv[CPW];
#pragma unroll
  for (int u = 0; u < CPW; u++) {
    qv[u] = (uint32_t)(qw0 + 4 * u + g);
    qok[u] = qw0 + 4 * u + g < qs1;
  }

  // ---- 1. x and the LoRA A rows (loads return in order: these first) ------------
  // Every load below is issued unconditionally (a lane or tile with nothing to
  // read gets an offset past its buffer), so the compiler's wait counts stay
  // exact and no wait drains loads that are not needed yet.
  const __amdgpu_buffer_rsrc_t xrs = make_rsrc(x, (uint32_t)(xrows * K * 2));
  int64_t xr = n;                                // the row of x lane row n reads
  if (xrow) xr = n < M ? (int64_t)xrow[n] : -1;
  const bool xr_ok = n < M && xr >= 0 && xr < xrows;
  u32x4_t xa[CPW][4];
#pragma unroll
  for (int u = 0; u < CPW; u++) {
    const bool ok = xr_ok & qok[u];
    const uint32_t base = (uint32_t)((xr_ok ? xr : 0) * K + 32 * (int64_t)qv[u]) * 2u;
#pragma unroll
    for (int sub = 0; sub < 4; sub++) xa[u][sub] = buffer_load16(xrs, ok ? base + 16u * sub : kBufferOob);
  }
  // first 16-byte unit of the LoRA B rows of the tiles (B 16-byte aligned, r % 8 == 0)
  // (unit e: tile e / (2 r), 16-byte unit e % (2 r) of its 16 rows; rows >= N not read)
  const int lb_elems = ntg * XS_ROWS * rr;
  const int lb_units = lb_elems / 8;
  const int lb_tile_units = 2 * rr;
  auto lb_off = [&](int e) -> int64_t {         // element offset of unit e in B, -1: past N
    const int ti = e / (lb_tile_units > 0 ? lb_tile_units : 1), w = e - ti * lb_tile_units;
    const int64_t el = tile_of(ti) * XS_ROWS * rr + 8 * w;
    return el < N * rr ? el : -1;
  };
  const __amdgpu_buffer_rsrc_t brs = make_rsrc(lora_b, (uint32_t)(N * (int64_t)rr * 2));
  int64_t lb0 = -1;
  if (lb16 && tid < lb_units) lb0 = lb_off(tid);
  const u32x4_t lbv = buffer_load16(brs, lb0 >= 0 ? (uint32_t)(lb0 * 2) : kBufferOob);
  // AQN: gamma and noise of the wave's K groups, 8 elements per lane j < GU
  // (group qw0 + j / 4, elements 8 (j % 4) .. + 7; groups past the span read
  // zeros, so their gain is 0)
  constexpr int GU = 16 * CPW;
  u32x4_t gmv = {0u, 0u, 0u, 0u}, nz0 = gmv, nz1 = gmv;
  if (AQN) {
    const __amdgpu_buffer_rsrc_t grs = make_rsrc(aq.gamma, (uint32_t)(K * 2));
    const __amdgpu_buffer_rsrc_t nrs = make_rsrc(aq.noise, (uint32_t)(K * 4));
    const int qj = qw0 + (lane >> 2);
    const uint32_t k8 = (uint32_t)(32 * qj + 8 * (lane & 3));
    const bool ok = lane < GU && qj < qs1;
    gmv = buffer_load16(grs, ok ? 2u * k8 : kBufferOob);
    nz0 = buffer_load16(nrs, ok ? 4u * k8 : kBufferOob);
    nz1 = buffer_load16(nrs, ok ? 4u * k8 + 16u : kBufferOob);
  }
  __builtin_amdgcn_sched_barrier(0);

  // ---- 2. code and scale loads of a tile (tiles past the run read nothing) -------------
  const uint32_t kb = (uint32_t)(K >> 1);                          // code bytes per row
  const __amdgpu_buffer_rsrc_t crs = make_rsrc(codes, (uint32_t)(N * (int64_t)kb));
  const uint32_t sbr = (uint32_t)(K >> 5) * SB;                     // scale bytes per row
  const __amdgpu_buffer_rsrc_t srs = make_rsrc(scales, (uint32_t)(N * (int64_t)sbr));
  // code loads: a ring of RP tiles per wave, refilled as each tile is consumed, so
  // the stream and the decode work overlap
  constexpr int RP = TG < XS_RING ? TG : XS_RING;
  u32x4_t cr[RP][CPW];
  uint32_t sr[TG][CPW];
  auto load_tile = [&](int ti) {                 // tiles past the run read nothing
    const int64_t row = tile_of(ti) * XS_ROWS + n;
    const bool rok = (ti < ntg) & (row < N);
    const uint32_t cb = (uint32_t)row * kb, sbase = (uint32_t)row * sbr;
#pragma unroll
    for (int u = 0; u < CPW; u++) {
      const bool ok = rok & qok[u];
      cr[ti % RP][u] = buffer_load16(crs, ok ? cb + 16u * qv[u] : kBufferOob);
      // NVFP4: the two scale bytes of group q (2-byte aligned: K % 32 == 0, scales 2-byte aligned)
      if (!SC)
        sr[ti][u] = FMT == FMT_NVFP4
                        ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(srs, ok ? sbase + 2u * qv[u] : kBufferOob, 0, 0)
                        : (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(srs, ok ? sbase + qv[u] : kBufferOob, 0, 0);
    }
  };
  // staged scales: 16-byte units (tile ti, row r, chunk c) of the rows' span bytes,
  // at most XS_SC_UNITS per thread (the host checks); units past the span's groups
  // or rows past N read zeros and are never used
  const int upr = span_bytes / 16;
  const int sc_units = ntg * XS_ROWS * upr;
  const uint32_t span_b0 = SB * (uint32_t)(s * qspan);
  const uint32_t span_blen = SB * (uint32_t)(qs1 - s * qspan);
  u32x4_t scv[XS_SC_UNITS];

  // ---- 5. the tiles' loads, then stream ----------------------------------------------
  // Issued once every wave of the workgroup has issued its x loads (requests
  // already in flight delay a later x load by most of the stream: they are not
  // served first), before x has arrived: x returns first, and the first tiles'
  // latency overlaps the conversion of x.
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  if (SC) {
#pragma unroll
    for (int c = 0; c < XS_SC_UNITS; c++) {
      const int e = tid + c * nt;
      const int ti = e / (XS_ROWS * upr), rem = e - ti * XS_ROWS * upr;
      const int r0 = rem / upr, ch = rem - r0 * upr;
      const int64_t row = tile_of(ti) * XS_ROWS + r0;
      const bool ok = (e < sc_units) & (row < N) & (16u * (uint32_t)ch < span_blen);
      scv[c] = buffer_load16(srs, ok ? (uint32_t)row * sbr + span_b0 + 16u * (uint32_t)ch : kBufferOob);
    }
  }
#pragma unroll
  for (int ti = 0; ti < RP; ti++) load_tile(ti);
  __builtin_amdgcn_sched_barrier(0);

  // ---- 4. x to the operand format -------------------------------------------------
  if (AQN) {
    // the gain g = gamma (1 + sigma noise) of the wave's K groups into its LDS
    // slice, then every lane forms bf16(x g) of its elements and its rows' sums
    // of x^2 (no other wave reads the slice: no workgroup barrier)
    float* gl = reinterpret_cast<float*>(lds + L.gain_off) + wave * (8 * GU);
    if (lane < GU) {
      f32x4_t g0, g1;
#pragma unroll
      for (int d = 0; d < 4; d++) {
        const uint32_t gb = gmv[d >> 1];
        const float gm = (d & 1) ? bf16hi_f32(gb) : bf16lo_f32(gb);
        g0[d] = gm * __builtin_fmaf(aq.sigma, __uint_as_float(nz0[d]), 1.0f);
        const uint32_t gb1 = gmv[2 + (d >> 1)];
        const float gm1 = (d & 1) ? bf16hi_f32(gb1) : bf16lo_f32(gb1);
        g1[d] = gm1 * __builtin_fmaf(aq.sigma, __uint_as_float(nz1[d]), 1.0f);
      }
      *reinterpret_cast<f32x4_t*>(gl + 8 * lane) = g0;
      *reinterpret_cast<f32x4_t*>(gl + 8 * lane + 4) = g1;
    }
    // the rows' sums of x^2 (x as it came in) while the writes land
    float ss = 0.f;
#pragma unroll
    for (int u = 0; u < CPW; u++)
#pragma unroll
      for (int sub = 0; sub < 4; sub++)
#pragma unroll
        for (int d = 0; d < 4; d++) ss = bf16x2_sumsq(xa[u][sub][d], ss);
    __builtin_amdgcn_s_waitcnt(0xC07F);         // lgkmcnt(0): the slice is written; loads stay in flight
    __builtin_amdgcn_wave_barrier();
    asm volatile("" ::: "memory");
    // unit i = (u, sub) of the lane: k = 32 (qw0 + 4 u + g) + 8 sub; its gain sits
    // at 32 (4 u + g) + 8 sub of the slice (groups past the span were staged as
    // 0, and their x is 0: no select).  The next unit's gain is read while this
    // one is formed.
    constexpr int NU = 4 * CPW;
    auto gain_at = [&](int i, f32x4_t& ga, f32x4_t& gb) {
      int kl = 32 * (4 * (i >> 2) + g) + 8 * (i & 3);
      asm volatile("" : "+v"(kl));               // read here, not hoisted
      ga = *reinterpret_cast<const f32x4_t*>(gl + kl);
      gb = *reinterpret_cast<const f32x4_t*>(gl + kl + 4);
    };
    f32x4_t ga_n, gb_n;
    gain_at(0, ga_n, gb_n);
#pragma unroll
    for (int i = 0; i < NU; i++) {
      const f32x4_t ga = ga_n, gb = gb_n;
      if (i + 1 < NU) gain_at(i + 1, ga_n, gb_n);
      const int u = i >> 2, sub = i & 3;
#pragma unroll
      for (int d = 0; d < 4; d++) {
        const uint32_t w = xa[u][sub][d];
        const float g0 = d < 2 ? ga[2 * d] : gb[2 * d - 4];
        const float g1 = d < 2 ? ga[2 * d + 1] : gb[2 * d - 3];
        xa[u][sub][d] = f32x2_to_bf16x2_rne(bf16lo_f32(w) * g0, bf16hi_f32(w) * g1);
        asm volatile("" : "+v"(xa[u][sub][d]));   // formed here, one unit at a time
      }
    }
    ss += __shfl_xor(ss, 16, 64);
    ss += __shfl_xor(ss, 32, 64);
    const int nw4 = (nw + 3) & ~3;
    float* ssw = reinterpret_cast<float*>(lds + L.ss_off);
    if (g == 0) ssw[n * nw4 + wave] = ss;
    if (wave == 0 && lane < XS_ROWS * (nw4 - nw))     // the slots past the last wave
      ssw[(lane / (nw4 - nw)) * nw4 + nw + lane % (nw4 - nw)] = 0.f;
  }
  // Largest |x| of each row over this wave's K groups, as the 15 magnitude bits
  // of bf16 (integer order = magnitude order, Inf and NaN on top); lanes r,
  // r + 16, r + 32, r + 48 hold row r.  Both halves at once (v_pk_max_u16).
  u16x2_t mxp = {0, 0};
#pragma unroll
  for (int u = 0; u < CPW; u++)
#pragma unroll
    for (int sub = 0; sub < 4; sub++)
#pragma unroll
      for (int d = 0; d < 4; d++)
        mxp = __builtin_elementwise_max(mxp, __builtin_bit_cast(u16x2_t, xa[u][sub][d] & 0x7FFF7FFFu));
  uint32_t mx = mxp[0] > mxp[1] ? (uint32_t)mxp[0] : (uint32_t)mxp[1];
  if (xrow && n < M && !xr_ok) mx = 0x7F80u;     // a routed row without a valid token: NaN outputs
  {
    uint32_t o = (uint32_t)__shfl_xor((int)mx, 16, 64);
    mx = o > mx ? o : mx;
    o = (uint32_t)__shfl_xor((int)mx, 32, 64);
    mx = o > mx ? o : mx;
  }
  const int fin = mx < 0x7F80u ? 1 : 0;
  const int ex = (int)(mx >> 7) - 141;         // floor(log2 max) - 14 (zero and subnormal rows: -141)
  if (FMT == FMT_NVFP4) {
#pragma unroll
    for (int u = 0; u < CPW; u++)
#pragma unroll
      for (int sub = 0; sub < 4; sub++)
#pragma unroll
        for (int d = 0; d < 4; d++) {
          const uint32_t w = xa[u][sub][d];
          const float lo = __builtin_ldexpf(bf16lo_f32(w), -ex), hi = __builtin_ldexpf(bf16hi_f32(w), -ex);
          xa[u][sub][d] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
        }
  }
  // the scale and finiteness of output rows 4 g + i (D layout: lane (n, g))
  int er[4], fr[4];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    er[i] = __shfl(ex, 4 * g + i, 64);
    fr[i] = __shfl(fin, 4 * g + i, 64);
  }

  if (SC) {
    u32x4_t* ssc = reinterpret_cast<u32x4_t*>(lds + L.ssc_off);
#pragma unroll
    for (int c = 0; c < XS_SC_UNITS; c++) {
      const int e = tid + c * nt;
      if (e < sc_units) ssc[e] = scv[c];        // unit e sits at 16 e: [tile][row][chunk]
    }
    // LDS writes complete, then the workgroup meets; the tile loads stay in flight
    __builtin_amdgcn_s_waitcnt(0xC07F);         // lgkmcnt(0) only
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    const uint8_t* sl = lds + L.ssc_off;
#pragma unroll
    for (int ti = 0; ti < TG; ti++)
#pragma unroll
      for (int u = 0; u < CPW; u++) {
        const bool use = (ti < ntg) & qok[u];
        const int bo = use ? (ti * XS_ROWS + n) * span_bytes + (int)SB * ((int)qv[u] - s * qspan) : 0;
        const uint32_t v = FMT == FMT_NVFP4 ? (uint32_t)*reinterpret_cast<const uint16_t*>(sl + bo)
                                            : (uint32_t)sl[bo];
        sr[ti][u] = use ? v : 0u;
      }
  }
  const int per_tile = M * XS_ROWS;
  float* red = reinterpret_cast<float*>(lds + L.red_off);
#pragma unroll
  for (int ti = 0; ti < TG; ti++) {
    if (ti < ntg) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
      bool nan_scale = false;                   // MXFP4: a NaN block scale in this lane
#pragma unroll
      for (int u = 0; u < CPW; u++) {
        const u32x4_t c = cr[ti % RP][u];
        if (FMT == FMT_NVFP4) {
          const f16x2_t s2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sr[ti][u], 1.0f, false);
          const f16x2_t sa = {s2.x, s2.x}, sb = {s2.y, s2.y};
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(bits_as_f16x8(xa[u][0]), codes8_to_f16(c.x, sa), acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(bits_as_f16x8(xa[u][1]), codes8_to_f16(c.y, sa), acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(bits_as_f16x8(xa[u][2]), codes8_to_f16(c.z, sb), acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(bits_as_f16x8(xa[u][3]), codes8_to_f16(c.w, sb), acc, 0, 0, 0);
        } else {
          const uint32_t sc = sr[ti][u];
          nan_scale = nan_scale || sc == 0xFFu;
          const float ps = e8m0_scale_operand(sc);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bits_as_bf16x8(xa[u][0]), codes8_to_bf16_pow2(c.x, ps), acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bits_as_bf16x8(xa[u][1]), codes8_to_bf16_pow2(c.y, ps), acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bits_as_bf16x8(xa[u][2]), codes8_to_bf16_pow2(c.z, ps), acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bits_as_bf16x8(xa[u][3]), codes8_to_bf16_pow2(c.w, ps), acc, 0, 0, 0);
        }
      }
      int col_nan = 0;
      if (FMT == FMT_MXFP4) {                   // a NaN scale poisons every row of its column
        col_nan = nan_scale ? 1 : 0;
        col_nan |= __shfl_xor(col_nan, 16, 64);
        col_nan |= __shfl_xor(col_nan, 32, 64);
      }
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int row = 4 * g + i;
        float v = acc[i];
        if (FMT == FMT_NVFP4) v = __builtin_ldexpf(v, er[i]);
        if (fr[i] == 0 || col_nan) v = __builtin_nanf("");
        if (row < M) red[(wave * tg + ti) * per_tile + row * XS_ROWS + n] = v;
      }
    }
    if (ti + RP < TG) load_tile(ti + RP);
  }

  // ---- 6. LoRA B rows and t to LDS ---------------------------------------------------------
  float* lt = reinterpret_cast<float*>(lds + L.lt_off);
  uint32_t arr_old = 0;                          // wave 0 of span 0: the arrival's group count
  if (rr > 0) {
    if (lb16) {
      u32x4_t* lb = reinterpret_cast<u32x4_t*>(lds + L.lb_off);
      if (tid < lb_units) lb[tid] = lbv;
      for (int e = tid + nt; e < lb_units; e += nt) {
        const int64_t o = lb_off(e);
        lb[e] = o >= 0 ? load16(lora_b + o) : (u32x4_t){0u, 0u, 0u, 0u};
      }
    } else {                                     // B not 16-byte aligned or r % 8 != 0: element by element
      uint16_t* lbe = reinterpret_cast<uint16_t*>(lds + L.lb_off);
      const int tile_elems = XS_ROWS * rr;
      for (int e = tid; e < lb_elems; e += nt) {
        const int ti = e / tile_elems;
        const int64_t el = tile_of(ti) * tile_elems + (e - ti * tile_elems);
        lbe[e] = el < N * rr ? lora_b[el] : (uint16_t)0;
      }
    }
    // t: the chunk words of the launch (bounded wait), read by wave 0 of the
    // span-0 workgroups while the other waves stage B
    if (wave == 0) {
      const int ok = s == 0 ? lora_poll(lsync, lparts, M * rr, lt, wait_ticks, lane) : 1;
      if (lane == 0) *have_t = ok;
      if (s == 0) arr_old = lsync_reader_issue(lsync, rd, lane);    // the words are read: arrive
    }
  }
  __syncthreads();
  if (LORA && __builtin_expect(!*have_t, 0))      // the wait ran out (span 0): the chunks formed here
    lora_form_all(reinterpret_cast<float*>(lds + L.tred_off), lt, x, M, K, lora_a, rr, nw, lsw, lparts,
                  AQN ? XGain{aq.gamma, aq.noise, aq.sigma} : XGain{nullptr, nullptr, 0.f});

  // ---- 7. tile sums in wave order (+ the span's LoRA term); spans in span order --------
  const float st = (FMT == FMT_NVFP4) ? *tensor_scale : 1.0f;
  const uint16_t* lbs = reinterpret_cast<const uint16_t*>(lds + L.lb_off);
  const int nout = ntg * per_tile;
  auto out_index = [&](int e, int& m, int64_t& row) {
    const int ti = e / per_tile, rem = e - ti * per_tile;
    m = rem / XS_ROWS;
    row = tile_of(ti) * XS_ROWS + (rem - m * XS_ROWS);
  };
  for (int e = tid; e < nout; e += nt) {
    const int ti = e / per_tile, rem = e - ti * per_tile;
    float o = 0.f;
    for (int w = 0; w < nw; w++) o += red[(w * tg + ti) * per_tile + rem];
    float v = st * o;
    if (rr > 0 && s == 0) {                      // t B^T once per output: span 0
      const int m = rem / XS_ROWS, nn = rem - m * XS_ROWS;
      const uint16_t* b = lbs + (ti * XS_ROWS + nn) * rr;
      float l = 0.f;
      for (int j = 0; j < rr; j++) l = __builtin_fmaf(lt[m * rr + j], __uint_as_float((uint32_t)b[j] << 16), l);
      v += l;
    }
    if (AQN) {                                   // the row factor of the norm, waves in order
      const int m = rem / XS_ROWS, nw4 = (nw + 3) & ~3;
      const f32x4_t* ssv = reinterpret_cast<const f32x4_t*>(lds + L.ss_off) + m * (nw4 / 4);
      float ss = 0.f;
      for (int w4 = 0; w4 < nw4 / 4; w4++) {
        const f32x4_t v = ssv[w4];
        ss += v[0];
        ss += v[1];
        ss += v[2];
        ss += v[3];
      }
      v *= 1.0f / __builtin_sqrtf(ss / (float)K + aq.eps);
    }
    if (S > 1) {
      store_agent(&part[((int64_t)s * ntiles + tile_of(ti)) * per_tile + rem], v);
    } else {
      int m;
      int64_t row;
      out_index(e, m, row);
      if (row < N) y[(int64_t)m * N + row] = (uint16_t)f32_to_bf16_rne(v);
    }
  }
  // the arrival issued after the poll, completed before the workgroup can exit
  if (LORA && s == 0 && wave == 0) lsync_reader_complete(lsync, arr_old, rd, nread, lparts, lparts * M * rr, lane);
  if (S > 1) {
    if (!arrive_last(&cnt[gi], (uint32_t)S, flag)) return;
    for (int e = tid; e < nout; e += nt) {
      float v = 0.f;
      const int ti = e / per_tile, rem = e - ti * per_tile;
      for (int q = 0; q < S; q++) v += load_agent(&part[((int64_t)q * ntiles + tile_of(ti)) * per_tile + rem]);
      int m;
      int64_t row;
      out_index(e, m, row);
      if (row < N) y[(int64_t)m * N + row] = (uint16_t)f32_to_bf16_rne(v);
    }
  }
}

// Dense: LORA workgroups below lparts form the chunks of t (and stream no codes);
// workgroup lparts + bid takes span bid % S of tile run bid / S.
template <int FMT, int TG, int SC, bool LORA, bool AQN>
__global__ __launch_bounds__(64 * XS_MAX_WAVES) void decode_xs_kernel(
    const uint16_t* __restrict__ x, int M, int64_t K, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ scales, const float* __restrict__ tensor_scale, int64_t N,
    const uint16_t* __restrict__ lora_a, const uint16_t* __restrict__ lora_b, int r, int lparts, int lsw,
    uint32_t* __restrict__ lsync, uint64_t wait_ticks, uint16_t* __restrict__ y, float* __restrict__ part,
    uint32_t* __restrict__ cnt, int S, int qspan, int ntiles, int G, int tg, int lb16, XsAqn aq) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  __shared__ int flag, have_t;
  if (LORA && (int)blockIdx.x < lparts) {
    const XsLayout L = xs_layout(M, (int)blockDim.x >> 6, tg, r, 0);
    lora_chunk_publish(reinterpret_cast<float*>(lds + L.tred_off), x, M, K, lora_a, r, (int)blockIdx.x,
                       (int)blockDim.x >> 6, lsw, lsync, G, lparts,
                       AQN ? XGain{aq.gamma, aq.noise, aq.sigma} : XGain{nullptr, nullptr, 0.f});
    return;
  }
  const int bid = (int)blockIdx.x - (LORA ? lparts : 0);
  const int s = bid % S, gi = bid / S;
  xs_body<FMT, TG, SC, LORA, AQN>(lds, &flag, &have_t, x, nullptr, M, M, K, codes, scales, tensor_scale, N, lora_a,
                                  lora_b, r, lparts, lsw, lsync, wait_ticks, y, part, cnt, S, qspan, ntiles, G, tg,
                                  lb16, s, gi, gi, G, aq);
}

// ---------------------------------------------------------------------------------
// Grouped (mixture of experts): workgroup (expert e, tile run gi) takes the
// expert's routed rows [offsets[e], offsets[e+1]) 16 at a time, each chunk
// against the run's tiles of W_e, K in one span.  The routing stays on the
// device: an expert with no rows returns at once.
// ---------------------------------------------------------------------------------
template <int FMT, int TG, int SC>
__global__ __launch_bounds__(64 * XS_MAX_WAVES) void grouped_xs_kernel(
    const uint16_t* __restrict__ x, int64_t num_tokens, const int32_t* __restrict__ row_index,
    const int32_t* __restrict__ offsets, int64_t total_rows, int64_t N, int64_t K,
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales, const float* __restrict__ tscales,
    uint16_t* __restrict__ y, int qspan, int ntiles, int G, int tg) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  __shared__ int flag, have_t;
  const int64_t e = blockIdx.x / (unsigned)G;
  const int gi = (int)(blockIdx.x % (unsigned)G);
  int64_t q0 = offsets[e], q1 = offsets[e + 1];
  q0 = q0 < 0 ? 0 : (q0 > total_rows ? total_rows : q0);
  q1 = q1 > total_rows ? total_rows : q1;
  constexpr int64_t BLK = FMT == FMT_NVFP4 ? 16 : 32;
  const uint8_t* ce = codes + e * N * (K / 2);
  const uint8_t* se = scales + e * N * (K / BLK);
  const float* te = FMT == FMT_NVFP4 ? tscales + e : nullptr;
  for (; q0 < q1; q0 += XS_MAX_M) {
    const int mc = (int)(q1 - q0 < XS_MAX_M ? q1 - q0 : XS_MAX_M);
    xs_body<FMT, TG, SC, false, false>(lds, &flag, &have_t, x, row_index + q0, num_tokens, mc, K, ce, se, te, N,
                                       nullptr, nullptr, 0, 0, 0, nullptr, 0, y + q0 * N, nullptr, nullptr, 1, qspan,
                                       ntiles, G, tg, 0, 0, gi, 0, 0, XsAqn{nullptr, nullptr, 0.f, 0.f});
    __syncthreads();                             // LDS is reused by the next chunk
  }
}

// ---------------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------------
bool decode_xs_supports(int64_t m, int64_t n, int64_t k, int r) {
  return m >= 1 && m <= XS_MAX_M && k % 32 == 0 && r <= XS_MAX_R &&
         n * (k / 2) < ((int64_t)1 << 31) && m * k * 2 < ((int64_t)1 << 31) && (int64_t)r * k * 2 < ((int64_t)1 << 31);
}

// Spans: the fewest with at most XS_MAX_WAVES waves each; waves: just enough for
// the span.  The tile runs (G) are chosen at launch from the device's CU count.
XsConfig plan_decode_xs(int64_t m, int64_t n, int64_t k, int r) {
  (void)m; (void)r;
  XsConfig c{};
  const int64_t nq = k / 32;
  const int64_t per_wave = 4 * XS_CPW;
  int64_t S = (nq + per_wave * XS_MAX_WAVES - 1) / (per_wave * XS_MAX_WAVES);
  if (S < 1) S = 1;
  // spans of a multiple of 16 groups: their scale bytes start 16-byte aligned;
  // a single span is K itself (no wave left without groups)
  int64_t qspan = (nq + S - 1) / S;
  qspan = (qspan + 15) & ~(int64_t)15;
  S = (nq + qspan - 1) / qspan;
  if (S == 1) qspan = nq > 0 ? nq : 1;
  c.splits = (int)S;
  c.qspan = (int)qspan;
  c.nw = (int)((qspan + per_wave - 1) / per_wave);
  if (c.nw < 1) c.nw = 1;
  c.ntiles = (int)((n + XS_ROWS - 1) / XS_ROWS);
  return c;
}

// Workgroups per CU the tile runs aim for (all resident at once).
constexpr int kXsGroupsPerCu = 1;
constexpr int kXsMaxTilesPerGroup = 6;
constexpr int kXsMaxLds = 160 * 1024 - 64;      // dynamic LDS bytes a workgroup may take

struct XsLaunch {
  const uint16_t* x;
  int m;
  int64_t k;
  const uint8_t* codes;
  const uint8_t* scales;
  const float* ts;
  int64_t n;
  const uint16_t* la;
  const uint16_t* lb;
  int r, lparts, lsw;
  uint32_t* lsync;
  uint16_t* y;
  float* part;
  uint32_t* cnt;
  int G, tg, lb16;
  XsAqn aq;
};

template <int FMT, int TG, int SC, bool LORA, bool AQN>
static hipError_t launch_xs_tg(dim3 grid, dim3 block, size_t lds, hipStream_t stream, const XsLaunch& a,
                               const XsConfig& c) {
  static std::atomic<uint64_t> lds_done{0};
  {
    hipError_t e = set_max_lds_once(reinterpret_cast<const void*>(&decode_xs_kernel<FMT, TG, SC, LORA, AQN>), kXsMaxLds,
                                    lds_done);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((decode_xs_kernel<FMT, TG, SC, LORA, AQN>), grid, block, lds, stream, a.x, a.m, a.k, a.codes,
                     a.scales, a.ts, a.n, a.la, a.lb, a.r, a.lparts, a.lsw, a.lsync,
                     (uint64_t)(LORA ? lora_wait_ticks() : 0), a.y, a.part, a.cnt, c.splits, c.qspan, c.ntiles, a.G,
                     a.tg, a.lb16, a.aq);
  return hipGetLastError();
}

template <int FMT, bool LORA, bool AQN>
static hipError_t launch_xs_fmt(dim3 grid, dim3 block, size_t lds, hipStream_t stream, const XsLaunch& a,
                                const XsConfig& c, int sc) {
  // the run's tile count exactly where it is 3 or 5: tiles past the run still
  // cost their (empty) loads, 0.15-0.25 us at m = 8 on the Qwen-2.5-7B shapes
#define FP4W_XS(TGv, SCv) launch_xs_tg<FMT, TGv, SCv, LORA, AQN>(grid, block, lds, stream, a, c)
  const int tg = a.tg;
  if (sc) {
    if (tg <= 1) return FP4W_XS(1, 1);
    if (tg <= 2) return FP4W_XS(2, 1);
    if (tg <= 3) return FP4W_XS(3, 1);
    if (tg <= 4) return FP4W_XS(4, 1);
    if (tg <= 5) return FP4W_XS(5, 1);
    return FP4W_XS(6, 1);
  }
  if (tg <= 1) return FP4W_XS(1, 0);
  if (tg <= 2) return FP4W_XS(2, 0);
  if (tg <= 3) return FP4W_XS(3, 0);
  if (tg <= 4) return FP4W_XS(4, 0);
  if (tg <= 5) return FP4W_XS(5, 0);
  return FP4W_XS(6, 0);
#undef FP4W_XS
}

static int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    cached[dev] = cus;
  }
  return cached[dev];
}

// The launch shape of one call: LoRA chunks, tile runs, staged scales and LDS.
struct XsGeometry {
  int lsw, lparts;
  int64_t G, tg;
  int sc;
  size_t lds;
  bool ok;
};
static XsGeometry xs_geometry(int fmt, const XsConfig& c, int64_t m, int64_t k, int rr, const uint8_t* scales,
                              bool aqn) {
  XsGeometry q{};
  // chunk workgroups of the LoRA down-projection go first in the grid
  q.lsw = rr > 0 ? lora_chunk_steps(c.nw, k, (int)m * rr) : kLoraStepsPerLoad;
  // long K: chunks of twice the steps (half as many chunk workgroups, half the
  // words to poll; MI355X, m = 8, LoRA r = 16, 3584 x 18944: 19.23 -> 18.71 us
  // NVFP4, 18.51 -> 17.69 us MXFP4; no change below K = 8192)
  if (rr > 0 && k >= 8192 && q.lsw < 2 * kLoraStepsPerLoad) q.lsw = 2 * kLoraStepsPerLoad;
  q.lparts = rr > 0 ? lora_chunk_count(c.nw, k, q.lsw) : 0;
  // tile runs: about kXsGroupsPerCu workgroups per CU over all spans, the chunk
  // workgroups included (one more workgroup than the chip holds at once would
  // start after the first ones finish, adding a whole workgroup's time), at most
  // kXsMaxTilesPerGroup tiles each, never more runs than tiles
  int64_t G = ((int64_t)device_cu_count() * kXsGroupsPerCu - q.lparts) / c.splits;
  if (G > c.ntiles) G = c.ntiles;
  if (G > kTileSlots) G = kTileSlots;
  if (G < 1) G = 1;
  int64_t tg = (c.ntiles + G - 1) / G;
  if (tg > kXsMaxTilesPerGroup) {
    tg = kXsMaxTilesPerGroup;
    G = (c.ntiles + tg - 1) / tg;
  }
  q.G = G;
  q.tg = tg;
  q.ok = !(c.splits > 1 && G > kTileSlots);        // arrival counters must fit
  // staged scales: 16-byte aligned rows and spans, few enough units per thread
  const int sb = fmt == FMT_NVFP4 ? 2 : 1;
  const int64_t span_bytes = (int64_t)sb * c.qspan;
  q.sc = (reinterpret_cast<uintptr_t>(scales) & 15u) == 0 && ((k / 32) * sb) % 16 == 0 && span_bytes % 16 == 0 &&
                 tg * XS_ROWS * (span_bytes / 16) <= (int64_t)XS_SC_UNITS * 64 * c.nw
             ? 1
             : 0;
  q.lds = (size_t)xs_layout((int)m, c.nw, (int)tg, rr, q.sc ? (int)span_bytes : 0, aqn).bytes;
  if (q.lds > (size_t)kXsMaxLds && q.sc) {
    q.sc = 0;
    q.lds = (size_t)xs_layout((int)m, c.nw, (int)tg, rr, 0, aqn).bytes;
  }
  if (q.lds > (size_t)kXsMaxLds) q.ok = false;
  return q;
}

bool decode_xs_fuses_aqn(int fmt, const XsConfig& c, int64_t m, int64_t k, int r, const uint8_t* scales) {
  if (c.splits != 1 || m < 1 || m > XS_MAX_M || k <= 0) return false;
  return xs_geometry(fmt, c, m, k, r, scales, true).ok;
}

hipError_t launch_decode_xs(int fmt, const XsConfig& c, const void* x, int64_t m, int64_t k, const uint8_t* codes,
                            const uint8_t* scales, const float* ts, int64_t n, const void* la, const void* lb, int r,
                            uint32_t* lsync, void* y, float* part, uint32_t* cnt, hipStream_t stream,
                            const void* aqn_gamma, const float* aqn_noise, float aqn_sigma, float aqn_eps) {
  const int rr = la && lb && k > 0 ? r : 0;      // k = 0: t = x A^T is zero
  if (rr > XS_MAX_R || m * rr > 1024) return hipErrorInvalidValue;
  const bool aqn = aqn_gamma != nullptr;
  if (aqn && (c.splits != 1 || !aqn_noise)) return hipErrorInvalidValue;
  const XsGeometry q = xs_geometry(fmt, c, m, k, rr, scales, aqn);
  if (!q.ok) return hipErrorInvalidValue;
  XsLaunch a{};
  a.x = reinterpret_cast<const uint16_t*>(x);
  a.m = (int)m;
  a.k = k;
  a.codes = codes;
  a.scales = scales;
  a.ts = ts;
  a.n = n;
  a.la = rr > 0 ? reinterpret_cast<const uint16_t*>(la) : nullptr;
  a.lb = reinterpret_cast<const uint16_t*>(lb);
  a.r = rr;
  a.lsw = q.lsw;
  a.lparts = q.lparts;
  a.lsync = lsync;
  a.y = reinterpret_cast<uint16_t*>(y);
  a.part = part;
  a.cnt = cnt;
  a.G = (int)q.G;
  a.tg = (int)q.tg;
  a.lb16 = (reinterpret_cast<uintptr_t>(lb) & 15u) == 0 && rr % 8 == 0 ? 1 : 0;
  a.aq = XsAqn{reinterpret_cast<const uint16_t*>(aqn_gamma), aqn_noise, aqn_sigma, aqn_eps};
  const dim3 grid((unsigned)(a.lparts + q.G * c.splits)), block((unsigned)(64 * c.nw));
  const size_t lds = q.lds;
  const int sc = q.sc;
  if (fmt == FMT_NVFP4) {
    if (aqn)
      return rr > 0 ? launch_xs_fmt<FMT_NVFP4, true, true>(grid, block, lds, stream, a, c, sc)
                    : launch_xs_fmt<FMT_NVFP4, false, true>(grid, block, lds, stream, a, c, sc);
    return rr > 0 ? launch_xs_fmt<FMT_NVFP4, true, false>(grid, block, lds, stream, a, c, sc)
                  : launch_xs_fmt<FMT_NVFP4, false, false>(grid, block, lds, stream, a, c, sc);
  }
  if (aqn)
    return rr > 0 ? launch_xs_fmt<FMT_MXFP4, true, true>(grid, block, lds, stream, a, c, sc)
                  : launch_xs_fmt<FMT_MXFP4, false, true>(grid, block, lds, stream, a, c, sc);
  return rr > 0 ? launch_xs_fmt<FMT_MXFP4, true, false>(grid, block, lds, stream, a, c, sc)
                : launch_xs_fmt<FMT_MXFP4, false, false>(grid, block, lds, stream, a, c, sc);
}

// ---- grouped ------------------------------------------------------------------------
bool grouped_xs_supports(int64_t num_tokens, int64_t n, int64_t k) {
  const int64_t nq = k / 32;
  return k % 32 == 0 && nq > 0 && nq <= (int64_t)4 * XS_CPW * XS_MAX_WAVES &&     // K in one span
         n * (k / 2) < ((int64_t)1 << 31) && num_tokens * k * 2 < ((int64_t)1 << 31);
}

template <int FMT, int TG, int SC>
static hipError_t launch_gxs_tg(dim3 grid, dim3 block, size_t lds, hipStream_t stream, const uint16_t* x,
                                int64_t num_tokens, const int32_t* row_index, const int32_t* offsets,
                                int64_t total_rows, int64_t n, int64_t k, const uint8_t* codes, const uint8_t* scales,
                                const float* ts, uint16_t* y, int qspan, int ntiles, int G, int tg) {
  static std::atomic<uint64_t> lds_done{0};
  {
    hipError_t e = set_max_lds_once(reinterpret_cast<const void*>(&grouped_xs_kernel<FMT, TG, SC>), kXsMaxLds, lds_done);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((grouped_xs_kernel<FMT, TG, SC>), grid, block, lds, stream, x, num_tokens, row_index, offsets,
                     total_rows, n, k, codes, scales, ts, y, qspan, ntiles, G, tg);
  return hipGetLastError();
}

template <int FMT>
static hipError_t launch_gxs_fmt(int tg, int sc, dim3 grid, dim3 block, size_t lds, hipStream_t stream,
                                 const uint16_t* x, int64_t num_tokens, const int32_t* row_index,
                                 const int32_t* offsets, int64_t total_rows, int64_t n, int64_t k,
                                 const uint8_t* codes, const uint8_t* scales, const float* ts, uint16_t* y, int qspan,
                                 int ntiles, int G) {
#define FP4W_GXS(TGv, SCv)                                                                                    \
  launch_gxs_tg<FMT, TGv, SCv>(grid, block, lds, stream, x, num_tokens, row_index, offsets, total_rows, n, k, \
                               codes, scales, ts, y, qspan, ntiles, G, tg)
  if (sc) {
    if (tg <= 1) return FP4W_GXS(1, 1);
    if (tg <= 2) return FP4W_GXS(2, 1);
    if (tg <= 3) return FP4W_GXS(3, 1);
    if (tg <= 4) return FP4W_GXS(4, 1);
    if (tg <= 5) return FP4W_GXS(5, 1);
    return FP4W_GXS(6, 1);
  }
  if (tg <= 1) return FP4W_GXS(1, 0);
  if (tg <= 2) return FP4W_GXS(2, 0);
  if (tg <= 3) return FP4W_GXS(3, 0);
  if (tg <= 4) return FP4W_GXS(4, 0);
  if (tg <= 5) return FP4W_GXS(5, 0);
  return FP4W_GXS(6, 0);
#undef FP4W_GXS
}

hipError_t launch_grouped_xs(int fmt, const void* x, int64_t num_tokens, const int32_t* row_index,
                             const int32_t* expert_offsets, int64_t num_experts, int64_t total_rows, int64_t n,
                             int64_t k, const uint8_t* codes, const uint8_t* scales, const float* tensor_scales,
                             void* y, hipStream_t stream) {
  const XsConfig c = plan_decode_xs(XS_MAX_M, n, k, 0);
  if (c.splits != 1) return hipErrorInvalidValue;
  // runs of at most kXsMaxTilesPerGroup tiles per expert
  const int64_t tg = c.ntiles < kXsMaxTilesPerGroup ? c.ntiles : kXsMaxTilesPerGroup;
  const int64_t G = (c.ntiles + tg - 1) / tg;
  if (num_experts * G > 0x7FFFFFFF) return hipErrorInvalidValue;
  const int sb = fmt == FMT_NVFP4 ? 2 : 1;
  const int64_t span_bytes = (int64_t)sb * c.qspan;
  int sc = (reinterpret_cast<uintptr_t>(scales) & 15u) == 0 && ((k / 32) * sb) % 16 == 0 && span_bytes % 16 == 0 &&
           tg * XS_ROWS * (span_bytes / 16) <= (int64_t)XS_SC_UNITS * 64 * c.nw ? 1 : 0;
  size_t lds = (size_t)xs_layout(XS_MAX_M, c.nw, (int)tg, 0, sc ? (int)span_bytes : 0).bytes;
  if (lds > (size_t)kXsMaxLds && sc) {
    sc = 0;
    lds = (size_t)xs_layout(XS_MAX_M, c.nw, (int)tg, 0, 0).bytes;
  }
  if (lds > (size_t)kXsMaxLds) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(num_experts * G)), block((unsigned)(64 * c.nw));
  const uint16_t* xx = reinterpret_cast<const uint16_t*>(x);
  uint16_t* yy = reinterpret_cast<uint16_t*>(y);
  if (fmt == FMT_NVFP4)
    return launch_gxs_fmt<FMT_NVFP4>((int)tg, sc, grid, block, lds, stream, xx, num_tokens, row_index, expert_offsets,
                                     total_rows, n, k, codes, scales, tensor_scales, yy, c.qspan, c.ntiles, (int)G);
  return launch_gxs_fmt<FMT_MXFP4>((int)tg, sc, grid, block, lds, stream, xx, num_tokens, row_index, expert_offsets,
                                   total_rows, n, k, codes, scales, tensor_scales, yy, c.qspan, c.ntiles, (int)G);
}

}  // namespace fp4w
