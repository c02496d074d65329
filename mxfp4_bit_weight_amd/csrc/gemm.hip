// gemm.hip -- the prefill-shaped linear (m > 16): y = s_t x deq(W)^T + (x A^T) B^T
// as a bf16 MFMA GEMM whose weight operand is decoded in registers.
//
// The pages: weight-only FP4 with a LoRA adapter in parallel to the frozen base
// (tggo.me/sberlogasci/42740, section "Metod"); the product runs on 16-bit
// values (QATFactory page, section on how training repeats the engine's
// arithmetic), which is why W is decoded to bf16 here, not x squeezed to FP8.
//
// Workgroup: a 256 x 256 tile of y, 4 waves (one per SIMD), each a 128 x 128
// wave tile: 4 x 4 products of v_mfma_f32_32x32x16_bf16, 256 accumulator
// registers.  Per K tile of 64:
//   - x (256 rows x 64) is staged in LDS, double-buffered;
//   - the weight codes and scales stay packed: they are staged in LDS 4 K tiles
//     (256 k) at a time, with loads of whole 128-byte lines, and each wave reads
//     the codes of its columns from there and decodes them to exact bf16 just
//     before the MFMAs that take them (e2m1 * dec(scale) has at most 6
//     significant bits).  Lane half hh of a wave owns k = 32 hh .. 32 hh + 31
//     of each of its 4 columns in a K tile; step s of the tile contracts
//     k = 32 hh + 8 s + e in lane half hh, the x fragment read from the same k.
// LDS rows of x and of codes are 128 bytes, unpadded, their 8 chunks of 16
// bytes XOR-swizzled so that tile stores (one row, 8 chunks) and fragment reads
// (32 rows, one chunk) spread over all bank groups.
// W is product A of the MFMA and x product B; the y block goes out through LDS
// in whole 128-byte lines.
// Loads go through buffer descriptors (chunks outside the matrices read zeros,
// no select after the load): x and the codes must each lie below 2 GiB, K must
// be a multiple of 256 and the scales 16-byte aligned.
#include "fp4w_device.hpp"
#include "fp4w_internal.hpp"

namespace fp4w {

constexpr int W4_BM = 256, W4_BN = 256, W4_BK = 64, W4_THREADS = 256;
constexpr int W4_SK = 4;                               // K tiles per weight stage (256 k)
constexpr int W4_GM = 4;                               // rows of tiles a group of the tile order spans
constexpr int W4_XB = W4_BM * 128;                     // bytes per x buffer (256 rows x 64 bf16)
constexpr int W4_CB = W4_BN * 128;                     // bytes per code stage (256 rows x 256 codes)
constexpr int W4_SB = W4_BN * 16;                      // bytes per scale stage (NVFP4: 16 per row, MXFP4: 8)
constexpr int W4_LDS = 2 * (W4_XB + W4_CB + W4_SB);    // x buffers, code stages, scale stages
static_assert(4 * 128 * 272 <= W4_LDS, "the epilogue's 4 blocks of y (128 rows of 272 bytes) fit the LDS");

// Position of chunk c of LDS row m: c ^ swz(m), swz(m) = (m ^ (m >> 3 & 1)) & 7.
// Rows m..m+7 (m a multiple of 8) get 8 distinct swizzles, and over 16 rows each
// parity class gets 8 distinct ones: a b128 access of 16 rows at one chunk, or
// of one row's 8 chunks, is conflict-free for 128- and 256-byte bank widths.
__device__ __forceinline__ int w4_swz(int m) { return (m ^ ((m >> 3) & 1)) & 7; }

// The accumulators live in AGPRs (v_mfma's AGPR form); the epilogue moves them
// through these explicit copies, because a plain VALU use of an accumulator
// made the register allocator keep some of them in VGPRs and shuffle them
// through the loop.
__device__ __forceinline__ float acc_read(float a) {
  float v;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(a));
  return v;
}
__device__ __forceinline__ float acc_write(float v) {
  float a;
  asm volatile("v_accvgpr_write_b32 %0, %1" : "=a"(a) : "v"(v));
  return a;
}

typedef __attribute__((ext_vector_type(16))) float f32x16_t;

struct W4Frag {
  u32x4_t c[4];        // codes of column j: k = 32 hh + 8 s .. + 7 in c[j][s]
  uint32_t s[4];       // scale byte(s) of column j (NVFP4: two, for k = 32 hh and 32 hh + 16)
};

template <int FMT>
__global__ __launch_bounds__(W4_THREADS, 1) void gemm_w4_kernel(
    const uint16_t* __restrict__ x, int M, int K, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ scales, const float* __restrict__ tensor_scale, int N,
    const float* __restrict__ t, const uint16_t* __restrict__ lora_b, int r, uint16_t* __restrict__ y, int flags) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint8_t* const xb0 = smem;
  uint8_t* const xb1 = smem + W4_XB;
  uint8_t* const cb0 = smem + 2 * W4_XB;
  uint8_t* const sb0 = smem + 2 * W4_XB + 2 * W4_CB;
  constexpr int BLK = (FMT == FMT_NVFP4) ? 16 : 32;
  // Tile order: workgroups go to the 8 XCDs in turn (workgroup b to XCD b % 8),
  // each XCD with its own L2.  XCD x takes a contiguous range of the tiles, and
  // within it the tiles run W4_GM rows of tiles at a time, column by column, so
  // the workgroups an XCD runs together share x rows and weight columns.
  const int tiles_n = (N + W4_BN - 1) / W4_BN, tiles_m = (M + W4_BM - 1) / W4_BM;
  const int ntiles = tiles_n * tiles_m;
  const int xcd = blockIdx.x % 8, per = ntiles / 8, extra = ntiles % 8;
  const int g = xcd * per + (xcd < extra ? xcd : extra) + (int)blockIdx.x / 8;
  const int grp = g / (W4_GM * tiles_n), rem = g - grp * (W4_GM * tiles_n);
  const int gm = min(W4_GM, tiles_m - grp * W4_GM);
  const int tm = grp * W4_GM + rem % gm, tn = rem / gm;
  const int m0 = tm * W4_BM, n0 = tn * W4_BN;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, hh = lane >> 5;

  const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, (uint32_t)M * (uint32_t)K * 2u);
  const __amdgpu_buffer_rsrc_t cr = make_rsrc(codes, (uint32_t)N * (uint32_t)(K / 2));
  const __amdgpu_buffer_rsrc_t sr = make_rsrc(scales, (uint32_t)N * (uint32_t)(K / BLK));

  // Staging: thread tid moves chunk tid & 7 of rows tid / 8 + 32 s, s < 8, of
  // an x tile and of a code stage.  K is a multiple of 256, so within the K
  // range a chunk is outside its matrix only when its row is (past the buffer's
  // end: zeros).
  const int srow = tid >> 3, sc = tid & 7;
  const int sst = srow * 128 + 16 * (sc ^ w4_swz(srow));            // + 32 s rows: same swizzle
  const uint32_t xbase = ((uint32_t)(m0 + srow) * (uint32_t)K + 8u * (uint32_t)sc) * 2u;
  const uint32_t xstep = 32u * (uint32_t)K * 2u;
  u32x4_t xv[8];
  auto load_x = [&](int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < 8; q++) xv[q] = buffer_load16(xr, xbase + ((uint32_t)q * xstep + (uint32_t)k0 * 2u));
  };
  auto store_x = [&](uint8_t* buf) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < 8; q++) *reinterpret_cast<u32x4_t*>(buf + sst + 32 * q * 128) = xv[q];
  };
  // a code stage: 256 rows x 128 bytes (k0 .. k0 + 255); its scales: row tid,
  // 16 bytes (NVFP4) or 8 (MXFP4)
  const uint32_t cbase = (uint32_t)(n0 + srow) * (uint32_t)(K / 2) + 16u * (uint32_t)sc;
  const uint32_t cstep = 32u * (uint32_t)(K / 2);
  const uint32_t sbase = (uint32_t)(n0 + tid) * (uint32_t)(K / BLK);
  u32x4_t cv[8];
  u32x4_t sv;
  auto load_w = [&](int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < 8; q++) cv[q] = buffer_load16(cr, cbase + ((uint32_t)q * cstep + (uint32_t)(k0 / 2)));
    if (FMT == FMT_NVFP4) {
      sv = buffer_load16(sr, sbase + (uint32_t)(k0 / 16));
    } else {
      const auto v = __builtin_amdgcn_raw_buffer_load_b64(sr, sbase + (uint32_t)(k0 / 32), 0, 0);
      sv = u32x4_t{v[0], v[1], 0u, 0u};
    }
  };
  auto store_w = [&](uint8_t* cbuf, uint8_t* sbuf) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < 8; q++) *reinterpret_cast<u32x4_t*>(cbuf + sst + 32 * q * 128) = cv[q];
    if (FMT == FMT_NVFP4) *reinterpret_cast<u32x4_t*>(sbuf + 16 * tid) = sv;
    else *reinterpret_cast<uint2*>(sbuf + 16 * tid) = make_uint2(sv[0], sv[1]);
  };

  // fragments: x row 128 wm + 32 i + l32 and W row 128 wn + 32 j + l32, chunk
  // 4 hh + s of an x tile, chunk 2 q + hh of a code stage (K tile q of it)
  const int arow = 128 * wm + l32, wrow = 128 * wn + l32;
  int aoff[4];
#pragma unroll
  for (int s = 0; s < 4; s++) aoff[s] = arow * 128 + 16 * ((4 * hh + s) ^ w4_swz(arow));
  auto read_a = [&](bf16x8_t* a, const uint8_t* buf, int s) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; i++) a[i] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(buf + aoff[s] + 32 * i * 128));
  };
  auto read_w = [&](W4Frag& f, const uint8_t* cbuf, const uint8_t* sbuf, int q) __attribute__((always_inline)) {
    const int coff = wrow * 128 + 16 * ((2 * q + hh) ^ w4_swz(wrow));
#pragma unroll
    for (int j = 0; j < 4; j++) {
      f.c[j] = *reinterpret_cast<const u32x4_t*>(cbuf + coff + 32 * j * 128);
      if (FMT == FMT_NVFP4) f.s[j] = *reinterpret_cast<const uint16_t*>(sbuf + (wrow + 32 * j) * 16 + 4 * q + 2 * hh);
      else f.s[j] = sbuf[(wrow + 32 * j) * 16 + 2 * q + hh];
    }
  };
  // column j's fragment for step s: 8 exact bf16 values
  auto wfrag = [&](const W4Frag& f, int j, int s) __attribute__((always_inline)) -> bf16x8_t {
    const uint32_t dw = f.c[j][s];
    u32x4_t o;
    if (FMT == FMT_MXFP4) {
      const float sc = e8m0_scale_operand(f.s[j]);
      o.x = fp4x2_to_bf16x2_scaled<0>(dw, sc);
      o.y = fp4x2_to_bf16x2_scaled<1>(dw, sc);
      o.z = fp4x2_to_bf16x2_scaled<2>(dw, sc);
      o.w = fp4x2_to_bf16x2_scaled<3>(dw, sc);
    } else {
      const float d = e4m3_to_f32(s < 2 ? (f.s[j] & 0xFFu) : (f.s[j] >> 8));
      const f32x2_t a0 = fp4x2_to_f32x2<0>(dw, 1.0f), a1 = fp4x2_to_f32x2<1>(dw, 1.0f);
      const f32x2_t a2 = fp4x2_to_f32x2<2>(dw, 1.0f), a3 = fp4x2_to_f32x2<3>(dw, 1.0f);
      o.x = (__float_as_uint(a0.x * d) >> 16) | (__float_as_uint(a0.y * d) & 0xFFFF0000u);
      o.y = (__float_as_uint(a1.x * d) >> 16) | (__float_as_uint(a1.y * d) & 0xFFFF0000u);
      o.z = (__float_as_uint(a2.x * d) >> 16) | (__float_as_uint(a2.y * d) & 0xFFFF0000u);
      o.w = (__float_as_uint(a3.x * d) >> 16) | (__float_as_uint(a3.y * d) & 0xFFFF0000u);
    }
    return as_bf16x8(o);
  };

  f32x16_t acc[4][4];                             // [j: 32 columns of W][i: 32 rows of x]
#pragma unroll
  for (int j = 0; j < 4; j++)
#pragma unroll
    for (int i = 0; i < 4; i++) acc[j][i] = f32x16_t{};

  // 16 MFMAs of step s (x fragments a), the W fragments decoded on the way
  auto mfma_step = [&](const bf16x8_t* a, const W4Frag& f, int s) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const bf16x8_t b = wfrag(f, j, s);
#pragma unroll
      for (int i = 0; i < 4; i++) acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a[i], acc[j][i], 0, 0, 0);
    }
  };
  auto fence = [&]() __attribute__((always_inline)) { __builtin_amdgcn_sched_barrier(0); };

  const int nst = K / (W4_BK * W4_SK);
  bf16x8_t a0[4], a1[4], a2[4], a3[4];
  W4Frag f0, f1;
  // K tile q of weight stage S (LDS stage S & 1), x from buffer cur.  On entry
  // a0 and f hold its step-0 x fragments and its W fragments (reads issued).
  // Step 0 reads the next tile's W fragments into fn (the next stage's, for
  // q = 3: stored two tiles before).  During step 1 the x of the next tile
  // (loaded a tile ago) goes to buffer nxt and the x of the tile after it is
  // loaded; q = 0 also loads stage S + 1, which q = 2 stores to the other
  // stage.  The barrier comes before step 3, whose MFMAs cover the reads of the
  // next tile's step-0 x fragments.
  auto tile = [&](int S, int q, const uint8_t* cur, uint8_t* nxt, W4Frag& f, W4Frag& fn)
                  __attribute__((always_inline)) {
    const int kt = S * W4_SK + q;
    uint8_t* const cbuf = cb0 + (S & 1) * W4_CB;
    uint8_t* const sbuf = sb0 + (S & 1) * W4_SB;
    uint8_t* const cnext = cb0 + ((S + 1) & 1) * W4_CB;
    uint8_t* const snext = sb0 + ((S + 1) & 1) * W4_SB;
    read_a(a1, cur, 1);
    if (q < 3) read_w(fn, cbuf, sbuf, q + 1);
    else read_w(fn, cnext, snext, 0);
    mfma_step(a0, f, 0);
    fence();
    read_a(a2, cur, 2);
    store_x(nxt);
    load_x((kt + 2) * W4_BK);
    if (q == 0) load_w((S + 1) * W4_SK * W4_BK);
    mfma_step(a1, f, 1);
    fence();
    read_a(a3, cur, 3);
    if (q == 2) store_w(cnext, snext);
    mfma_step(a2, f, 2);
    fence();
    __builtin_amdgcn_s_waitcnt(0xC07F);           // lgkmcnt(0): this wave's LDS stores (and reads) done
    __builtin_amdgcn_s_barrier();
    fence();
    read_a(a0, nxt, 0);
    mfma_step(a3, f, 3);
    fence();
  };

  load_x(0);
  load_w(0);
  store_x(xb0);
  store_w(cb0, sb0);
  load_x(W4_BK);
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  fence();
  read_a(a0, xb0, 0);
  read_w(f0, cb0, sb0, 0);
  // The prologue's loads land before the loop (the empty asm takes their
  // registers), so the compiler's wait counts at the loop's head follow the
  // loop's own order of loads.  Otherwise the compiler sank the prologue's loads
  // to the loop's entry and the merged counts made tiles wait for loads issued
  // just before them.
#pragma unroll
  for (int q = 0; q < 8; q++) asm volatile("" ::"v"(xv[q]));
  fence();
  // Loads past K (the last stage's x tiles and weight stage) read the next
  // rows' data or zeros past the buffers and feed nothing.  (No exit inside
  // the loop body: a second loop exit made the compiler copy the accumulators.)
  for (int S = 0; S < nst; S++) {
    tile(S, 0, xb0, xb1, f0, f1);
    tile(S, 1, xb1, xb0, f1, f0);
    tile(S, 2, xb0, xb1, f0, f1);
    tile(S, 3, xb1, xb0, f1, f0);
  }

  // epilogue: y = s_t acc + LoRA, the LoRA as MFMA steps over K' = [t_hi | t_lo]
  // (t split into two bf16 parts, 8 ranks a step) against [B | B]; s_t is
  // applied before the first LoRA step, or at the store without LoRA.
  // flags & 2: r a multiple of 8 and B 16-byte aligned, so a lane's 8 ranks of
  // B and of t are 16-byte loads.
  const float st = (FMT == FMT_NVFP4) ? *tensor_scale : 1.0f;
  const bool has_t = t != nullptr && r > 0;
  const __amdgpu_buffer_rsrc_t br = make_rsrc(lora_b, has_t ? (uint32_t)N * (uint32_t)r * 2u : 0u);
  const __amdgpu_buffer_rsrc_t tr = make_rsrc(t, has_t ? (uint32_t)M * (uint32_t)r * 4u : 0u);
  auto pack8 = [](const uint32_t* h) __attribute__((always_inline)) {
    return as_bf16x8(u32x4_t{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)});
  };
  auto lora_step = [&](int jb, bool scale_first) __attribute__((always_inline)) {
    // lane half hh covers K' entries 8 hh .. 8 hh + 7: part hh of ranks jb + e
    bf16x8_t lb[4], tf[4];
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int n = n0 + 128 * wn + 32 * j + l32;
      if (flags & 2) {
        lb[j] = as_bf16x8(buffer_load16(br, ((uint32_t)n * (uint32_t)r + (uint32_t)jb) * 2u));
      } else {
        uint32_t h[8];
#pragma unroll
        for (int e = 0; e < 8; e++) h[e] = (n < N && jb + e < r) ? lora_b[(int64_t)n * r + jb + e] : 0u;
        lb[j] = pack8(h);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int mr = m0 + 128 * wm + 32 * i + l32;
      float tv[8];
      if (flags & 2) {
        const uint32_t o = ((uint32_t)mr * (uint32_t)r + (uint32_t)jb) * 4u;
        const u32x4_t v0 = buffer_load16(tr, o), v1 = buffer_load16(tr, o + 16u);
#pragma unroll
        for (int e = 0; e < 4; e++) { tv[e] = __uint_as_float(v0[e]); tv[4 + e] = __uint_as_float(v1[e]); }
      } else {
#pragma unroll
        for (int e = 0; e < 8; e++) tv[e] = (mr < M && jb + e < r) ? t[(int64_t)mr * r + jb + e] : 0.f;
      }
      uint32_t h[8];
#pragma unroll
      for (int e = 0; e < 8; e++) {
        const uint32_t hi = f32_to_bf16_rne(tv[e]);
        h[e] = hh ? f32_to_bf16_rne(tv[e] - __uint_as_float(hi << 16)) : hi;
      }
      tf[i] = pack8(h);
    }
#pragma unroll
    for (int j = 0; j < 4; j++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        if (scale_first) {
#pragma unroll
          for (int e = 0; e < 16; e++) acc[j][i][e] = acc_write(acc_read(acc[j][i][e]) * st);
        }
        acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lb[j], tf[i], acc[j][i], 0, 0, 0);
      }
  };
  if (has_t) {
    lora_step(0, FMT == FMT_NVFP4);
    for (int jb = 8; jb < r; jb += 8) lora_step(jb, false);
  }

  // store: result e of lane (l32, hh) in product (j, i) is y[m][n], m = row l32
  // of x block i, n = 8 (e / 4) + 4 hh + e % 4 of W block j.  Each wave puts
  // its 128 x 128 bf16 block in LDS (rows of 272 bytes), then writes it out
  // row-contiguously, 16 bytes a lane (whole 128-byte lines); flags & 1: y
  // 16-byte aligned and n a multiple of 8.
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();                   // every wave is done with the loop's LDS
  uint8_t* const ys = smem + wave * (128 * 272);
#pragma unroll
  for (int i = 0; i < 4; i++) {
#pragma unroll
    for (int j = 0; j < 4; j++) {
#pragma unroll
      for (int q = 0; q < 4; q++) {
        uint32_t o[4];
#pragma unroll
        for (int e = 0; e < 4; e++) {
          const float v = acc_read(acc[j][i][4 * q + e]);
          o[e] = f32_to_bf16_rne((FMT == FMT_NVFP4 && !has_t) ? v * st : v);
        }
        *reinterpret_cast<uint2*>(ys + (32 * i + l32) * 272 + (32 * j + 8 * q + 4 * hh) * 2) =
            make_uint2(o[0] | (o[1] << 16), o[2] | (o[3] << 16));
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);             // the wave reads back only what it wrote
  const int rr = lane >> 4, cc = lane & 15;
#pragma unroll 4
  for (int it = 0; it < 32; it++) {
    const int row = 4 * it + rr;
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(ys + row * 272 + cc * 16);
    const int mr = m0 + 128 * wm + row, n = n0 + 128 * wn + 8 * cc;
    if (mr >= M) continue;
    uint16_t* dst = y + (int64_t)mr * N + n;
    if ((flags & 1) && n + 7 < N) {
      *reinterpret_cast<u32x4_t*>(dst) = v;
    } else {
#pragma unroll
      for (int e = 0; e < 8; e++)
        if (n + e < N) dst[e] = (uint16_t)(v[e >> 1] >> (16 * (e & 1)));
    }
  }
}

bool gemm_w4_supports(int64_t m, int64_t n, int64_t k, const void* scales) {
  return k % (W4_BK * W4_SK) == 0 && (reinterpret_cast<uintptr_t>(scales) & 15u) == 0 &&
         m * k * 2 < ((int64_t)1 << 31) && n * (k / 2) < ((int64_t)1 << 31);
}

template <int FMT>
static hipError_t launch_w4(const uint16_t* x, int64_t m, int64_t k, const uint8_t* codes, const uint8_t* scales,
                            const float* tensor_scale, int64_t n, const float* t, const uint16_t* lora_b, int r,
                            uint16_t* y, hipStream_t stream) {
  const int64_t tiles = ((m + W4_BM - 1) / W4_BM) * ((n + W4_BN - 1) / W4_BN);
  static bool lds_set = false;
  if (!lds_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_w4_kernel<FMT>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, W4_LDS);
    if (e != hipSuccess) return e;
    lds_set = true;
  }
  // flags: 1 = 16-byte stores of y (y 16-byte aligned, n a multiple of 8);
  // 2 = 16-byte loads of B and t (r a multiple of 8, B 16-byte aligned)
  const int flags = ((n % 8 == 0 && (reinterpret_cast<uintptr_t>(y) & 15u) == 0) ? 1 : 0) |
                    ((t && r > 0 && r % 8 == 0 && (reinterpret_cast<uintptr_t>(lora_b) & 15u) == 0) ? 2 : 0);
  hipLaunchKernelGGL((gemm_w4_kernel<FMT>), dim3((unsigned)tiles), dim3(W4_THREADS), W4_LDS, stream, x, (int)m,
                     (int)k, codes, scales, tensor_scale, (int)n, t, lora_b, r, y, flags);
  return hipGetLastError();
}

hipError_t launch_gemm_w4(int fmt, const void* x, int64_t m, int64_t k, const uint8_t* codes, const uint8_t* scales,
                          const float* tensor_scale, int64_t n, const float* t, const void* lora_b, int r, void* y,
                          hipStream_t stream) {
  const uint16_t* xx = reinterpret_cast<const uint16_t*>(x);
  const uint16_t* bb = reinterpret_cast<const uint16_t*>(lora_b);
  uint16_t* yy = reinterpret_cast<uint16_t*>(y);
  return fmt == FMT_NVFP4 ? launch_w4<FMT_NVFP4>(xx, m, k, codes, scales, tensor_scale, n, t, bb, r, yy, stream)
                          : launch_w4<FMT_MXFP4>(xx, m, k, codes, scales, tensor_scale, n, t, bb, r, yy, stream);
}

}  // namespace fp4w
