// gemm.hip -- the prefill-shaped linear (m > 16): y = s_t x deq(W)^T + (x A^T) B^T
// as a bf16 MFMA GEMM whose weight operand is decoded in registers.
//
// The pages: weight-only FP4 with a LoRA adapter in parallel to the frozen base
// (tggo.me/sberlogasci/42740, section "Metod"); the product runs on 16-bit
// values (QATFactory page, section on how training repeats the engine's
// arithmetic), which is why W is decoded to bf16 here, not x squeezed to FP8.
//
// One workgroup per CU, looping over 256 x 256 tiles of y; 4 waves (one per
// SIMD), each a 128 x 128 wave tile: 4 x 4 products of v_mfma_f32_32x32x16_bf16,
// 256 accumulator registers.  Operands reach LDS by DMA (buffer loads that write
// LDS directly, 16 bytes a lane, lane-contiguous), with no register staging and
// no LDS store instructions:
//   - x: one 256 x 64 bf16 tile per K tile, three buffers, loaded two K tiles
//     ahead;
//   - W: codes and scales stay packed, one stage per 2 K tiles (256 rows x 64
//     code bytes and their scale bytes), three stages, loaded two stages ahead.
//     Each wave reads the codes of its columns and decodes them to exact bf16
//     just before the MFMAs that take them (e2m1 * dec(scale) has at most 6
//     significant bits).  Lane half hh of a wave owns k = 32 hh .. 32 hh + 31
//     of each of its 4 columns in a K tile; step s of the tile contracts
//     k = 32 hh + 8 s + e in lane half hh, the x fragment read from the same k.
// LDS rows are unpadded, their 16-byte chunks XOR-swizzled (the DMA lanes load
// the chunk that belongs at their position) so that fragment reads of 32 rows
// at one chunk spread over all bank groups.  One barrier per K tile; before it
// each wave waits for its own DMA of the next K tile (a fixed count of later
// loads may stay in flight).
// W is product A of the MFMA and x product B; the y block goes out through LDS
// in whole 128-byte lines.
// Loads and stores go through buffer descriptors (out of range: zeros read,
// stores dropped): x, the codes and y must each lie below 2 GiB, 2 GiB and
// 4 GiB, K must be a multiple of 128 and the scales 16-byte aligned.
#include "fp4w_device.hpp"
#include "fp4w_internal.hpp"
#include "gemm_common.hpp"

namespace fp4w {

constexpr int W4_BM = 256, W4_BN = 256, W4_BK = 64, W4_THREADS = 256;
constexpr int W4_SK = 2;                               // K tiles per weight stage (128 k)
constexpr int W4_GM = 4;                               // rows of tiles a group of the tile order spans
#ifndef W4_WL_NVFP4
#define W4_WL_NVFP4 1                                  // wave layout per format (see gemm_w4_kernel)
#endif
#ifndef W4_WL_MXFP4
#define W4_WL_MXFP4 0
#endif
constexpr int W4_XB = W4_BM * 128;                     // bytes per x buffer (256 rows x 64 bf16)
constexpr int W4_CB = W4_BN * 64;                      // code bytes per weight stage (256 rows x 128 codes)
constexpr int W4_WB = W4_CB + W4_BN * 8;               // bytes per weight stage (codes, then 8 scale bytes a row)
// LDS: [x0][x1][w0][w1][x2][w2]; the last x buffer and weight stage are
// contiguous and hold the epilogue's y staging (the next tile's first DMA goes
// to x0, x1, w0, w1 meanwhile)
constexpr int W4_X0 = 0, W4_X1 = W4_XB, W4_W0 = 2 * W4_XB, W4_W1 = W4_W0 + W4_WB;
constexpr int W4_X2 = W4_W1 + W4_WB, W4_W2 = W4_X2 + W4_XB;
constexpr int W4_LDS = W4_W2 + W4_WB;                  // 153600 bytes
constexpr int W4_YROW = 272;                           // bytes per staged y row (256 + 16 of padding)
static_assert(4 * 32 * W4_YROW <= W4_XB + W4_WB && 4 * 64 * 144 <= W4_XB + W4_WB,
              "a pass of the y staging (either wave layout) fits the last x buffer and stage");
static_assert(W4_LDS <= 160 * 1024, "LDS of one CU");


template <int TJ>
struct W4Frag {
  u32x4_t c[TJ];       // codes of column block j: k = 32 hh + 8 s .. + 7 in c[j][s]
  uint32_t s[TJ];      // scale byte(s) of column block j (NVFP4: two, for k = 32 hh and 32 hh + 16)
};

// WL: the 4 waves' layout over the 256 x 256 tile: 0 = 2 x 2 waves of 128 x 128
// (4 x 4 products each), 1 = 1 x 4 waves of 256 rows x 64 columns (8 x 2
// products each: a weight column is decoded by one wave instead of two, and
// each x fragment read by four waves instead of two).
template <int FMT, int WL>
__global__ __launch_bounds__(W4_THREADS, 1) void gemm_w4_kernel(
    const uint16_t* __restrict__ x, int M, int K, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ scales, const float* __restrict__ tensor_scale, int N,
    const float* __restrict__ t, const uint16_t* __restrict__ lora_b, int r, uint16_t* __restrict__ y, int flags) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  constexpr int BLK = (FMT == FMT_NVFP4) ? 16 : 32;
  constexpr int NSC = (FMT == FMT_NVFP4) ? 2 : 1;        // scale DMAs per wave and stage
  // Tile order: workgroups go to the 8 XCDs in turn (workgroup b to XCD b % 8),
  // each XCD with its own L2.  XCD x owns a contiguous range of the tiles, and
  // within it the tiles run W4_GM rows of tiles at a time, column by column;
  // the XCD's workgroups (one per CU) take its tiles in turn, so the ones it
  // runs together share x rows and weight columns.
  const int tiles_n = (N + W4_BN - 1) / W4_BN, tiles_m = (M + W4_BM - 1) / W4_BM;
  const int ntiles = tiles_n * tiles_m;
  // XCD x runs nwg of the grid's workgroups and owns that share of the tiles
  const int grid = (int)gridDim.x, xcd = blockIdx.x % 8, gq = grid / 8, gr = grid % 8;
  const int nwg = gq + (xcd < gr ? 1 : 0), cum = xcd * gq + (xcd < gr ? xcd : gr);
  const int xstart = (int)((int64_t)ntiles * cum / grid);
  const int xcount = (int)((int64_t)ntiles * (cum + nwg) / grid) - xstart;
  int local = (int)blockIdx.x / 8;
  if (local >= xcount) return;
  auto origin = [&](int lc, int& om0, int& on0) __attribute__((always_inline)) {
    const int g = xstart + lc;
    const int grp = g / (W4_GM * tiles_n), rem = g - grp * (W4_GM * tiles_n);
    const int gm = min(W4_GM, tiles_m - grp * W4_GM);
    om0 = (grp * W4_GM + rem % gm) * W4_BM;
    on0 = (rem / gm) * W4_BN;
  };
  int m0, n0;
  origin(local, m0, n0);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  constexpr int TI = WL ? 8 : 4, TJ = WL ? 2 : 4;   // x blocks (32 rows) and W blocks (32 columns) of a wave
  const int xrow0 = WL ? 0 : 128 * (wave >> 1);      // the wave's first x row and W column in the tile
  const int wcol0 = WL ? 64 * wave : 128 * (wave & 1);
  const int l32 = lane & 31, hh = lane >> 5;

  const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, (uint32_t)M * (uint32_t)K * 2u);
  const __amdgpu_buffer_rsrc_t cr = make_rsrc(codes, (uint32_t)N * (uint32_t)(K / 2));
  const __amdgpu_buffer_rsrc_t sr = make_rsrc(scales, (uint32_t)N * (uint32_t)(K / BLK));

  // DMA lanes.  x: instruction q (of 8) of wave w fills LDS rows 32 q + 8 w ..
  // + 7 (1 KB); lane l takes row 32 q + 8 w + l / 8, position l % 8, so it loads
  // that row's chunk (l % 8) ^ swz(row).  Codes: instruction i (of 4) fills rows
  // 64 i + 16 w .. + 15 (64 bytes each); lane l takes row + l / 4, position
  // l % 4, chunk (l % 4) ^ swzw(row).  Scales (4-byte DMA, 256 bytes an
  // instruction): NVFP4 rows 128 i + 32 w + l / 2, word l % 2 (8 bytes a row);
  // MXFP4 rows 64 w + l, one word.  K is a multiple of 128, so within the K
  // range a chunk lies outside its matrix only when its row does (past the
  // buffer's end: zeros).
  const int xrow = 8 * wave + (lane >> 3);
  const uint32_t xlane = (uint32_t)(8 * ((lane & 7) ^ w4_swz(xrow))) * 2u;
  const int crow = 16 * wave + (lane >> 2);
  const uint32_t clane = 16u * (uint32_t)((lane & 3) ^ w4_swzw(crow));
  const int srow = (FMT == FMT_NVFP4) ? 32 * wave + (lane >> 1) : 64 * wave + lane;
  const uint32_t slane = (FMT == FMT_NVFP4) ? 4u * (uint32_t)(lane & 1) : 0u;
  uint32_t xbase, cbase, sbase;
  auto set_bases = [&](int om0, int on0) __attribute__((always_inline)) {
    xbase = (uint32_t)(om0 + xrow) * (uint32_t)K * 2u + xlane;
    cbase = (uint32_t)(on0 + crow) * (uint32_t)(K / 2) + clane;
    sbase = (uint32_t)(on0 + srow) * (uint32_t)(K / BLK) + slane;
  };
  set_bases(m0, n0);
  auto dma_xh = [&](uint8_t* buf, int k0, int h) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 4 * h; q < 4 * h + 4; q++)
      dma16(xr, buf + (32 * q + 8 * wave) * 128, xbase + (uint32_t)q * 32u * (uint32_t)K * 2u + (uint32_t)k0 * 2u);
  };
  auto dma_x = [&](uint8_t* buf, int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < 8; q++)
      dma16(xr, buf + (32 * q + 8 * wave) * 128, xbase + (uint32_t)q * 32u * (uint32_t)K * 2u + (uint32_t)k0 * 2u);
  };
  auto dma_w = [&](uint8_t* buf, int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; i++)
      dma16(cr, buf + (64 * i + 16 * wave) * 64, cbase + (uint32_t)i * 64u * (uint32_t)(K / 2) + (uint32_t)(k0 / 2));
    if (FMT == FMT_NVFP4) {
#pragma unroll
      for (int i = 0; i < 2; i++)
        dma4(sr, buf + W4_CB + (128 * i + 32 * wave) * 8, sbase + (uint32_t)i * 128u * (uint32_t)(K / 16) + (uint32_t)(k0 / 16));
    } else {
      dma4(sr, buf + W4_CB + (64 * wave) * 4, sbase + (uint32_t)(k0 / 32));
    }
  };

  // fragments: x row xrow0 + 32 i + l32, chunk 4 hh + s of an x tile; W row
  // wcol0 + 32 j + l32, chunk 2 q + hh of a weight stage (its K tile q)
  const int arow = xrow0 + l32, wrow = wcol0 + l32;
  int aoff[4];
#pragma unroll
  for (int s = 0; s < 4; s++) aoff[s] = arow * 128 + 16 * ((4 * hh + s) ^ w4_swz(arow));
  int woff[2];
#pragma unroll
  for (int q = 0; q < 2; q++) woff[q] = wrow * 64 + 16 * ((2 * q + hh) ^ w4_swzw(wrow));
  auto read_a = [&](bf16x8_t* a, const uint8_t* buf, int s) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < TI; i++) a[i] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(buf + aoff[s] + 32 * i * 128));
  };
  auto read_w = [&](W4Frag<TJ>& f, const uint8_t* wbuf, int q) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < TJ; j++) {
      f.c[j] = *reinterpret_cast<const u32x4_t*>(wbuf + woff[q] + 32 * j * 64);
      if (FMT == FMT_NVFP4) f.s[j] = *reinterpret_cast<const uint16_t*>(wbuf + W4_CB + (wrow + 32 * j) * 8 + 4 * q + 2 * hh);
      else f.s[j] = wbuf[W4_CB + (wrow + 32 * j) * 4 + 2 * q + hh];
    }
  };
  // column j's fragment for step s: 8 exact bf16 values
  auto wfrag = [&](const W4Frag<TJ>& f, int j, int s) __attribute__((always_inline)) -> bf16x8_t {
    const uint32_t dw = f.c[j][s];
    u32x4_t o;
    if (FMT == FMT_MXFP4) {
      const float sc = e8m0_scale_operand(f.s[j]);
      o.x = fp4x2_to_bf16x2_scaled<0>(dw, sc);
      o.y = fp4x2_to_bf16x2_scaled<1>(dw, sc);
      o.z = fp4x2_to_bf16x2_scaled<2>(dw, sc);
      o.w = fp4x2_to_bf16x2_scaled<3>(dw, sc);
    } else {
      // the products are exact in bf16, so the packing conversion (RNE) keeps them
      const float d = e4m3_to_f32(s < 2 ? (f.s[j] & 0xFFu) : (f.s[j] >> 8));
      o.x = __builtin_bit_cast(uint32_t, __builtin_convertvector(fp4x2_to_f32x2<0>(dw, 1.0f) * d, bf16x2_t));
      o.y = __builtin_bit_cast(uint32_t, __builtin_convertvector(fp4x2_to_f32x2<1>(dw, 1.0f) * d, bf16x2_t));
      o.z = __builtin_bit_cast(uint32_t, __builtin_convertvector(fp4x2_to_f32x2<2>(dw, 1.0f) * d, bf16x2_t));
      o.w = __builtin_bit_cast(uint32_t, __builtin_convertvector(fp4x2_to_f32x2<3>(dw, 1.0f) * d, bf16x2_t));
    }
    return as_bf16x8(o);
  };

  f32x16_t acc[TJ][TI];                           // [j: 32 columns of W][i: 32 rows of x]
  // 16 MFMAs of step s (x fragments a), the W fragments decoded on the way
  auto mfma_step = [&](const bf16x8_t* a, const W4Frag<TJ>& f, int s) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < TJ; j++) {
      const bf16x8_t b = wfrag(f, j, s);
#pragma unroll
      for (int i = 0; i < TI; i++) acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a[i], acc[j][i], 0, 0, 0);
    }
  };
  auto fence = [&]() __attribute__((always_inline)) { __builtin_amdgcn_sched_barrier(0); };
  auto xbuf = [&](int i) __attribute__((always_inline)) -> uint8_t* {
    return smem + (i == 0 ? W4_X0 : i == 1 ? W4_X1 : W4_X2);
  };
  auto wbuf = [&](int i) __attribute__((always_inline)) -> uint8_t* {
    return smem + (i == 0 ? W4_W0 : i == 1 ? W4_W1 : W4_W2);
  };

  const int nk = K / W4_BK;
  bf16x8_t a0[TI], a1[TI], a2[TI], a3[TI];
  W4Frag<TJ> f0, f1;
  // K tile kt = 2 S + q (x buffer kt % 3, weight stage S % 3).  On entry a0 and
  // f hold its step-0 x fragments and its W fragments (reads issued).  Step 0
  // reads the next tile's W fragments into fn.  The DMA of x tile kt + 2 (into
  // the buffer tile kt - 1 used) goes out in halves in steps 0 and 1, and for
  // q = 0 the DMA of weight stage S + 2 (into the stage S - 1 used) in step 2:
  // spread over the MFMA steps rather than in one burst, whose LDS writes held
  // up the steps' fragment reads.  Before the barrier each wave waits for its
  // DMA of x tile kt + 1 (and so of weight stage S + 1): the loads issued after
  // it, 8 of x and 4 + NSC of W, may stay in flight.  The barrier comes before
  // step 3, whose MFMAs cover the reads of the next tile's step-0 x fragments.
  auto tile = [&](int kt, int q, W4Frag<TJ>& f, W4Frag<TJ>& fn) __attribute__((always_inline)) {
    const int S = kt >> 1;
    const uint8_t* cur = xbuf(kt % 3);
    read_a(a1, cur, 1);
    if (q == 0) read_w(fn, wbuf(S % 3), 1);
    else read_w(fn, wbuf((S + 1) % 3), 0);
    dma_xh(xbuf((kt + 2) % 3), (kt + 2) * W4_BK, 0);
    mfma_step(a0, f, 0);
    fence();
    read_a(a2, cur, 2);
    dma_xh(xbuf((kt + 2) % 3), (kt + 2) * W4_BK, 1);
    mfma_step(a1, f, 1);
    fence();
    read_a(a3, cur, 3);
    if (q == 0) dma_w(wbuf((S + 2) % 3), (S + 2) * W4_SK * W4_BK);
    mfma_step(a2, f, 2);
    fence();
    wait_vm_lgkm0<12 + NSC>();
    __builtin_amdgcn_s_barrier();
    fence();
    read_a(a0, xbuf((kt + 1) % 3), 0);
    mfma_step(a3, f, 3);
    fence();
  };

  // the first tile's first two x tiles and weight stages
  dma_x(xbuf(0), 0);
  dma_x(xbuf(1), W4_BK);
  dma_w(wbuf(0), 0);
  dma_w(wbuf(1), W4_SK * W4_BK);
  const float st = (FMT == FMT_NVFP4) ? *tensor_scale : 1.0f;
  const bool has_t = t != nullptr && r > 0;
  wait_vm_lgkm0<0>();
  __builtin_amdgcn_s_barrier();
  fence();
  for (;;) {
    read_a(a0, xbuf(0), 0);
    read_w(f0, wbuf(0), 0);
#pragma unroll
    for (int j = 0; j < TJ; j++)
#pragma unroll
      for (int i = 0; i < TI; i++) acc[j][i] = f32x16_t{};
    fence();
    // DMAs past K (the last tiles' x and weight stages) read the next rows'
    // data or zeros past the buffers and feed nothing.  (No exit inside the
    // loop body: a second loop exit made the compiler copy the accumulators.)
    for (int kt = 0; kt < nk; kt += 2) {
      tile(kt, 0, f0, f1);
      tile(kt + 1, 1, f1, f0);
    }
    // every wave is past the loop's last LDS reads
    wait_vm_lgkm0<0>();
    __builtin_amdgcn_s_barrier();
    fence();
    const int em0 = m0, en0 = n0;

    // epilogue: y = s_t acc + LoRA, the LoRA as MFMA steps over K' = [t_hi | t_lo]
    // (t split into two bf16 parts, 8 ranks a step) against [B | B]; s_t is
    // applied before the first LoRA step, or at the store without LoRA.
    // flags & 2: r a multiple of 8 and B 16-byte aligned, so a lane's 8 ranks of
    // B and of t are 16-byte loads.
    const __amdgpu_buffer_rsrc_t br = make_rsrc(lora_b, has_t ? (uint32_t)N * (uint32_t)r * 2u : 0u);
    const __amdgpu_buffer_rsrc_t tr = make_rsrc(t, has_t ? (uint32_t)M * (uint32_t)r * 4u : 0u);
    auto pack8 = [](const uint32_t* h) __attribute__((always_inline)) {
      return as_bf16x8(u32x4_t{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)});
    };
    auto lora_step = [&](int jb, bool scale_first) __attribute__((always_inline)) {
      // lane half hh covers K' entries 8 hh .. 8 hh + 7: part hh of ranks jb + e
      bf16x8_t lb[TJ], tf[TI];
#pragma unroll
      for (int j = 0; j < TJ; j++) {
        const int n = en0 + wcol0 + 32 * j + l32;
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
      for (int i = 0; i < TI; i++) {
        const int mr = em0 + xrow0 + 32 * i + l32;
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
      for (int j = 0; j < TJ; j++)
#pragma unroll
        for (int i = 0; i < TI; i++) {
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
    // the next tile's first x tiles and weight stages go by DMA into x0, x1,
    // w0, w1 while this tile's y goes out through the x2 / w2 region
    const int nlocal = local + nwg;
    const bool more = nlocal < xcount;
    if (more) {
      origin(nlocal, m0, n0);
      set_bases(m0, n0);
      dma_x(xbuf(0), 0);
      dma_x(xbuf(1), W4_BK);
      dma_w(wbuf(0), 0);
      dma_w(wbuf(1), W4_SK * W4_BK);
    }
    asm volatile("" ::: "memory");                // the stores below stay after these DMAs
    fence();

    // store: result e of lane (l32, hh) in product (j, i) is y[m][n], m = row l32
    // of x block i, n = 8 (e / 4) + 4 hh + e % 4 of W block j.  In 4 passes (TI / 4
    // x blocks each), every wave stages its RP x 32 TJ bf16 block in LDS (rows of
    // 64 TJ + 16 bytes), then writes it out row-contiguously, 16 bytes a lane
    // (whole 128-byte lines), through a buffer descriptor (rows and columns past
    // y are dropped): 8 stores a pass.  flags & 1: y 16-byte aligned and n a
    // multiple of 8, else 2-byte stores.
    constexpr int IB = TI / 4, RP = 32 * IB, YR = 64 * TJ + 16, LPR = 4 * TJ;   // blocks, rows a pass; row bytes; lanes a row
    const __amdgpu_buffer_rsrc_t yr = make_rsrc(y, (uint32_t)M * (uint32_t)N * 2u);
    uint8_t* const ys = smem + W4_X2 + wave * (RP * YR);
    const int rr = lane / LPR, cc = lane % LPR;
#pragma unroll
    for (int pass = 0; pass < 4; pass++) {
#pragma unroll
      for (int ii = 0; ii < IB; ii++) {
        const int i = pass * IB + ii;
#pragma unroll
        for (int j = 0; j < TJ; j++) {
#pragma unroll
          for (int qq = 0; qq < 4; qq++) {
            uint32_t o[4];
#pragma unroll
            for (int e = 0; e < 4; e++) {
              const float v = acc_read(acc[j][i][4 * qq + e]);
              o[e] = f32_to_bf16_rne((FMT == FMT_NVFP4 && !has_t) ? v * st : v);
            }
            *reinterpret_cast<uint2*>(ys + (32 * ii + l32) * YR + (32 * j + 8 * qq + 4 * hh) * 2) =
                make_uint2(o[0] | (o[1] << 16), o[2] | (o[3] << 16));
          }
        }
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);         // lgkmcnt(0): the wave reads back only what it wrote
#pragma unroll
      for (int it = 0; it < 8; it++) {
        const int row = it * (64 / LPR) + rr;
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(ys + row * YR + cc * 16);
        const int mr = em0 + xrow0 + RP * pass + row, n = en0 + wcol0 + 8 * cc;
        const bool in = mr < M && n < N;
        if (flags & 1) {
          const uint32_t yo = in ? ((uint32_t)mr * (uint32_t)N + (uint32_t)n) * 2u : kBufferOob;
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned, v), yr, yo, 0, 0);
        } else {
#pragma unroll
          for (int e = 0; e < 8; e++) {
            const uint32_t yo = (mr < M && n + e < N) ? ((uint32_t)mr * (uint32_t)N + (uint32_t)(n + e)) * 2u : kBufferOob;
            __builtin_amdgcn_raw_buffer_store_b16((unsigned short)(v[e >> 1] >> (16 * (e & 1))), yr, yo, 0, 0);
          }
        }
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);         // this pass's LDS reads done before the next pass writes
    }
    if (!more) break;
    // the next tile's DMA was issued before this tile's 32 vector stores of y
    // (or 256 element stores), which may stay in flight
    if (flags & 1) wait_vm_lgkm0<32>();
    else wait_vm_lgkm0<0>();
    __builtin_amdgcn_s_barrier();
    fence();
    local = nlocal;
  }
}

bool gemm_w4_supports(int64_t m, int64_t n, int64_t k, const void* scales) {
  return k % (W4_BK * W4_SK) == 0 && (reinterpret_cast<uintptr_t>(scales) & 15u) == 0 &&
         m * k * 2 < ((int64_t)1 << 31) && n * (k / 2) < ((int64_t)1 << 31) && m * n * 2 < ((int64_t)1 << 32);
}

template <int FMT, int WL>
static hipError_t launch_w4(const uint16_t* x, int64_t m, int64_t k, const uint8_t* codes, const uint8_t* scales,
                            const float* tensor_scale, int64_t n, const float* t, const uint16_t* lora_b, int r,
                            uint16_t* y, hipStream_t stream) {
  const int64_t tiles = ((m + W4_BM - 1) / W4_BM) * ((n + W4_BN - 1) / W4_BN);
  static std::atomic<uint64_t> lds_done{0};
  {
    hipError_t e = set_max_lds_once(reinterpret_cast<const void*>(&gemm_w4_kernel<FMT, WL>), W4_LDS, lds_done);
    if (e != hipSuccess) return e;
  }
  // flags: 1 = 16-byte stores of y (y 16-byte aligned, n a multiple of 8);
  // 2 = 16-byte loads of B and t (r a multiple of 8, B 16-byte aligned)
  const int flags = ((n % 8 == 0 && (reinterpret_cast<uintptr_t>(y) & 15u) == 0) ? 1 : 0) |
                    ((t && r > 0 && r % 8 == 0 && (reinterpret_cast<uintptr_t>(lora_b) & 15u) == 0) ? 2 : 0);
  // one workgroup per CU (the LDS holds one), each looping over its XCD's tiles
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const int64_t grid = tiles < cus ? tiles : (cus > 0 ? cus : 1);
  hipLaunchKernelGGL((gemm_w4_kernel<FMT, WL>), dim3((unsigned)grid), dim3(W4_THREADS), W4_LDS, stream, x, (int)m,
                     (int)k, codes, scales, tensor_scale, (int)n, t, lora_b, r, y, flags);
  return hipGetLastError();
}

hipError_t launch_gemm_w4(int fmt, const void* x, int64_t m, int64_t k, const uint8_t* codes, const uint8_t* scales,
                          const float* tensor_scale, int64_t n, const float* t, const void* lora_b, int r, void* y,
                          hipStream_t stream) {
  const uint16_t* xx = reinterpret_cast<const uint16_t*>(x);
  const uint16_t* bb = reinterpret_cast<const uint16_t*>(lora_b);
  uint16_t* yy = reinterpret_cast<uint16_t*>(y);
  return fmt == FMT_NVFP4 ? launch_w4<FMT_NVFP4, W4_WL_NVFP4>(xx, m, k, codes, scales, tensor_scale, n, t, bb, r, yy, stream)
                          : launch_w4<FMT_MXFP4, W4_WL_MXFP4>(xx, m, k, codes, scales, tensor_scale, n, t, bb, r, yy, stream);
}

}  // namespace fp4w
