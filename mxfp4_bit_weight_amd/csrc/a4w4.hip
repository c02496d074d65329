// a4w4.hip -- the W4A4 MXFP4 product y = deq(x) deq(W)^T: x (m, k) and W (n, k)
// both MXFP4 (E2M1 codes, an E8M0 scale per 32 consecutive k), fed to gfx950's
// block-scaled matrix core exactly as stored.
//
// W4A4 (4-bit weights and 4-bit activations) is the MXFP4 mode that survived
// deployment best when training quantized both (QATFactory page, section on the
// different strategies NVFP4 and MXFP4 need), and the compute-bound case the
// Telegram post leaves open ("Vyvody").  gfx950's
// v_mfma_scale_f32_32x32x64_f8f6f4 multiplies E2M1 operands under E8M0 block
// scales natively, so no operand is decoded: every product is exact in the
// instruction, accumulated in fp32.
//
// Instruction layout (measured on the device, E2M1 x E2M1):
//   A: lane (r = l % 32, h = l / 32) holds 32 codes of row r (16 bytes), the
//      k-slots of half h; B: lane (c, h) the same for column c -- A and B slots
//      pair one to one, so loading both as 16 contiguous code bytes (32
//      consecutive k, one MXFP4 block) pairs equal k;
//   scales: E8M0 byte `opsel` of lane 32 h + r's scale register, for row
//      (column) r and half h;
//   D: lane (c, h), register e: row 8 (e / 4) + 4 h + e % 4, column c.
// W is operand A (rows n), x operand B (columns m), so a lane's results are runs
// of 4 consecutive outputs of one row of y.
//
// One workgroup per CU, looping over 256 x 256 tiles of y (tile order as in
// gemm.hip); 4 waves in 2 x 2, each 128 x 128 = 4 x 4 products, 256 fp32
// accumulators in AGPRs.  Per K tile of 256 (four MFMA steps of 64): the codes
// of x and of W (256 rows x 128 bytes each, one cache line a row) reach LDS by
// DMA, two buffer sets, one K tile ahead; the scale bytes of 512 k per row
// (16 bytes) every second K tile into one of two scale buffers.  Each step's
// fragment reads are issued ahead of its MFMAs; one barrier per K tile, after
// each wave's wait for its own DMA of the next tile.  K a multiple of 128 (a
// 128-k tail runs two steps of a last K tile).
#include "fp4w_device.hpp"
#include "fp4w_internal.hpp"
#include "gemm_common.hpp"

namespace fp4w {

constexpr int A4_BM = 256, A4_BN = 256, A4_BK = 256, A4_THREADS = 256, A4_GM = 4;
constexpr int A4_CB = 256 * 128;                      // code bytes of one operand's K tile (256 rows x 128 B)
constexpr int A4_SET = 2 * A4_CB;                     // one buffer set: x codes, then W codes
constexpr int A4_SC = 2 * A4_SET;                     // scale buffers: [2][x, W][256 rows][16 B]
constexpr int A4_SCB = 256 * 16;                      // scale bytes of one operand's 512-k chunk
constexpr int A4_LDS = A4_SC + 4 * A4_SCB;            // 147456 bytes
constexpr int A4_YROW = 272;                          // bytes per staged y row (128 bf16 + 16)
static_assert(4 * 32 * A4_YROW <= A4_SET, "the y staging of one pass fits buffer set 1");

// position of 16-byte chunk c of code row r in LDS: c ^ swz(r); 8 (16) consecutive
// rows read at one chunk hit 8 (16) distinct 16-byte bank groups
__device__ __forceinline__ int a4_swz(int r) { return (r & 7) ^ ((r >> 3) & 3); }

__global__ __launch_bounds__(A4_THREADS, 1) void gemm_a4w4_kernel(
    const uint8_t* __restrict__ xc, const uint8_t* __restrict__ xs, int M, int K,
    const uint8_t* __restrict__ wc, const uint8_t* __restrict__ ws, int N, uint16_t* __restrict__ y, int flags) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  // tile order: XCD x owns a contiguous share of the tiles, A4_GM rows of tiles
  // at a time, its workgroups (one per CU) taking them in turn
  const int tiles_n = (N + A4_BN - 1) / A4_BN, tiles_m = (M + A4_BM - 1) / A4_BM;
  const int ntiles = tiles_n * tiles_m;
  const int grid = (int)gridDim.x, xcd = blockIdx.x % 8, gq = grid / 8, gr = grid % 8;
  const int nwg = gq + (xcd < gr ? 1 : 0), cum = xcd * gq + (xcd < gr ? xcd : gr);
  const int xstart = (int)((int64_t)ntiles * cum / grid);
  const int xcount = (int)((int64_t)ntiles * (cum + nwg) / grid) - xstart;
  int local = (int)blockIdx.x / 8;
  if (local >= xcount) return;
  auto origin = [&](int lc, int& om0, int& on0) __attribute__((always_inline)) {
    const int g = xstart + lc;
    const int grp = g / (A4_GM * tiles_n), rem = g - grp * (A4_GM * tiles_n);
    const int gm = min(A4_GM, tiles_m - grp * A4_GM);
    om0 = (grp * A4_GM + rem % gm) * A4_BM;
    on0 = (rem / gm) * A4_BN;
  };
  int m0, n0;
  origin(local, m0, n0);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int xrow0 = 128 * (wave >> 1), wcol0 = 128 * (wave & 1);
  const int l32 = lane & 31, hh = lane >> 5;
  const int nkf = K / A4_BK, nk = (K + A4_BK - 1) / A4_BK;   // full K tiles; with a 128-k tail

  const __amdgpu_buffer_rsrc_t xcr = make_rsrc(xc, (uint32_t)M * (uint32_t)(K / 2));
  const __amdgpu_buffer_rsrc_t xsr = make_rsrc(xs, (uint32_t)M * (uint32_t)(K / 32));
  const __amdgpu_buffer_rsrc_t wcr = make_rsrc(wc, (uint32_t)N * (uint32_t)(K / 2));
  const __amdgpu_buffer_rsrc_t wsr = make_rsrc(ws, (uint32_t)N * (uint32_t)(K / 32));

  // DMA lanes.  Codes: instruction i (of 8) of wave w fills rows 32 i + 8 w ..
  // + 7 of a 256 x 128-byte tile; lane l takes row + l / 8, position l % 8, so it
  // loads that row's chunk (l % 8) ^ swz(row).  Scales, every second K tile: the
  // 16 bytes of 512 k of each row, 4 lanes a row (4-byte DMA): instruction i (of
  // 4) of wave w fills rows 64 w + 16 i .. + 15.  Rows past the matrix read zeros
  // (past the buffer's end); bytes past a row's end feed nothing.
  const int crow = 8 * wave + (lane >> 3);
  const uint32_t clane = 16u * (uint32_t)((lane & 7) ^ a4_swz(crow));
  const int srow = 64 * wave + (lane >> 2);
  const uint32_t slane = 4u * (uint32_t)(lane & 3);
  uint32_t xcb, wcb, xsb, wsb;
  auto set_bases = [&](int om0, int on0) __attribute__((always_inline)) {
    xcb = (uint32_t)(om0 + crow) * (uint32_t)(K / 2) + clane;
    wcb = (uint32_t)(on0 + crow) * (uint32_t)(K / 2) + clane;
    xsb = (uint32_t)(om0 + srow) * (uint32_t)(K / 32) + slane;
    wsb = (uint32_t)(on0 + srow) * (uint32_t)(K / 32) + slane;
  };
  set_bases(m0, n0);
  auto setp = [&](int i) __attribute__((always_inline)) -> uint8_t* { return smem + i * A4_SET; };
  auto scp = [&](int b) __attribute__((always_inline)) -> uint8_t* { return smem + A4_SC + b * 2 * A4_SCB; };
  // live == false: the DMAs still run (no branch around them in the K loop)
  // but read past the buffers, so they fetch nothing and write zeros
  auto dma_codes = [&](uint8_t* set, int k0, bool live) __attribute__((always_inline)) {   // 16 DMAs a wave
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const uint32_t ro = (uint32_t)i * 32u * (uint32_t)(K / 2) + (uint32_t)(k0 / 2);
      dma16(xcr, set + (32 * i + 8 * wave) * 128, live ? xcb + ro : kBufferOob);
      dma16(wcr, set + A4_CB + (32 * i + 8 * wave) * 128, live ? wcb + ro : kBufferOob);
    }
  };
  auto dma_scales = [&](uint8_t* sb, int k0, bool live) __attribute__((always_inline)) {   // 8 DMAs a wave
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const uint32_t ro = (uint32_t)i * 16u * (uint32_t)(K / 32) + (uint32_t)(k0 / 32);
      dma4(xsr, sb + (64 * wave + 16 * i) * 16, live ? xsb + ro : kBufferOob);
      dma4(wsr, sb + A4_SCB + (64 * wave + 16 * i) * 16, live ? wsb + ro : kBufferOob);
    }
  };

  // fragments of step s (k 64 s .. 64 s + 63 of the K tile): chunk 2 s + hh of
  // rows xrow0 / wcol0 + 32 i + l32 (swz does not depend on the 32 i)
  const int arow = xrow0 + l32, brow = wcol0 + l32;
  typedef __attribute__((ext_vector_type(8))) int i32x8_t;
  struct Frag {
    i32x8_t x[4], w[4];
  };
  auto read_frag = [&](Frag& f, const uint8_t* set, int s) __attribute__((always_inline)) {
    const int xo = arow * 128 + 16 * ((2 * s + hh) ^ a4_swz(arow));
    const int wo = A4_CB + brow * 128 + 16 * ((2 * s + hh) ^ a4_swz(brow));
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(set + xo + 32 * i * 128);
      f.x[i] = i32x8_t{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
      const u32x4_t u = *reinterpret_cast<const u32x4_t*>(set + wo + 32 * i * 128);
      f.w[i] = i32x8_t{(int)u.x, (int)u.y, (int)u.z, (int)u.w, 0, 0, 0, 0};
    }
  };
  // the 8 scale bytes of K tile kt for each fragment row, as two words shifted
  // so that the block of step s and half hh sits in byte 2 (s % 2) of word s / 2
  uint32_t xsc[4][2], wsc[4][2];
  uint2 xsr_[4], wsr_[4];
  auto read_scales_raw = [&](int kt) __attribute__((always_inline)) {
    const uint8_t* sb = scp((kt >> 1) & 1) + 8 * (kt & 1);
#pragma unroll
    for (int i = 0; i < 4; i++) {
      xsr_[i] = *reinterpret_cast<const uint2*>(sb + (arow + 32 * i) * 16);
      wsr_[i] = *reinterpret_cast<const uint2*>(sb + A4_SCB + (brow + 32 * i) * 16);
    }
  };
  auto shift_scales = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; i++) {
      xsc[i][0] = xsr_[i].x >> (8 * hh);
      xsc[i][1] = xsr_[i].y >> (8 * hh);
      wsc[i][0] = wsr_[i].x >> (8 * hh);
      wsc[i][1] = wsr_[i].y >> (8 * hh);
    }
  };

  f32x16_t acc[4][4];                             // [j: 32 rows of W][i: 32 rows of x]
  auto mfma_step = [&](const Frag& f, int s) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 4; j++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        if ((s & 1) == 0)
          acc[j][i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.w[j], f.x[i], acc[j][i], 4, 4, 0,
                                                                       (int)wsc[j][s >> 1], 0, (int)xsc[i][s >> 1]);
        else
          acc[j][i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.w[j], f.x[i], acc[j][i], 4, 4, 2,
                                                                       (int)wsc[j][s >> 1], 2, (int)xsc[i][s >> 1]);
      }
  };
  auto fence = [&]() __attribute__((always_inline)) { __builtin_amdgcn_sched_barrier(0); };

  Frag f0, f1;
  // one full K tile (buffer set kt % 2): on entry f0 and the scale words hold
  // its step-0 fragments and its scales (reads issued).  Step 0 issues the DMA
  // of tile kt + 1 into the other set (every wave finished reading it before
  // the previous barrier); each wave waits for its own DMA before the barrier
  // ahead of step 3, which reads the next tile's step-0 fragments and scales.
  auto tile = [&](int kt) __attribute__((always_inline)) {
    const uint8_t* cur = setp(kt & 1);
    read_frag(f1, cur, 1);
    fence();                                      // each step's reads go out ahead of its MFMAs
    // the next K tile's codes; on odd kt the scales of the next 512 k into the
    // scale buffer not in use (on even kt that buffer, idle, takes zeros)
    dma_codes(setp((kt + 1) & 1), (kt + 1) * A4_BK, kt + 1 < nk);
    dma_scales(scp(((kt >> 1) + 1) & 1), (kt + 1) * A4_BK, (kt & 1) && kt + 1 < nk);
    mfma_step(f0, 0);
    fence();
    read_frag(f0, cur, 2);
    fence();
    mfma_step(f1, 1);
    fence();
    read_frag(f1, cur, 3);
    fence();
    mfma_step(f0, 2);
    fence();
    wait_vm_lgkm0<0>();
    __builtin_amdgcn_s_barrier();
    fence();
    read_frag(f0, setp((kt + 1) & 1), 0);
    read_scales_raw(kt + 1);
    fence();
    mfma_step(f1, 3);
    fence();
    shift_scales();
  };

  dma_codes(setp(0), 0, true);
  dma_scales(scp(0), 0, true);
  wait_vm_lgkm0<0>();
  __builtin_amdgcn_s_barrier();
  fence();
  for (;;) {
    read_frag(f0, setp(0), 0);
    read_scales_raw(0);
    shift_scales();
#pragma unroll
    for (int j = 0; j < 4; j++)
#pragma unroll
      for (int i = 0; i < 4; i++) acc[j][i] = f32x16_t{};
    fence();
    for (int kt = 0; kt < nkf; kt++) tile(kt);
    if (nk > nkf) {                               // the last 128 k: steps 0 and 1 of tile nkf
      read_frag(f1, setp(nkf & 1), 1);
      fence();
      mfma_step(f0, 0);
      fence();
      mfma_step(f1, 1);
      fence();
    }
    wait_vm_lgkm0<0>();                           // every wave is past the loop's last LDS reads
    __builtin_amdgcn_s_barrier();
    fence();
    const int em0 = m0, en0 = n0;
    const int nlocal = local + nwg;
    const bool more = nlocal < xcount;
    if (more) {                                   // the next tile's first K tile, into set 0
      origin(nlocal, m0, n0);
      set_bases(m0, n0);
      dma_codes(setp(0), 0, true);
      dma_scales(scp(0), 0, true);
    }
    asm volatile("" ::: "memory");                // the stores below stay after these DMAs
    fence();

    // store (as in gemm.hip): 4 passes of one x block each through set 1, 32 rows
    // x 128 bf16 a wave, 8 stores of 16 bytes a lane and pass (rows and columns
    // past y dropped); flags & 1: y 16-byte aligned and n a multiple of 8, else
    // 2-byte stores
    const __amdgpu_buffer_rsrc_t yr = make_rsrc(y, (uint32_t)M * (uint32_t)N * 2u);
    uint8_t* const ysg = setp(1) + wave * (32 * A4_YROW);
    const int rr = lane >> 4, cc = lane & 15;
#pragma unroll
    for (int i = 0; i < 4; i++) {
#pragma unroll
      for (int j = 0; j < 4; j++) {
#pragma unroll
        for (int qq = 0; qq < 4; qq++) {
          uint32_t o[4];
#pragma unroll
          for (int e = 0; e < 4; e++) o[e] = f32_to_bf16_rne(acc_read(acc[j][i][4 * qq + e]));
          *reinterpret_cast<uint2*>(ysg + l32 * A4_YROW + (32 * j + 8 * qq + 4 * hh) * 2) =
              make_uint2(o[0] | (o[1] << 16), o[2] | (o[3] << 16));
        }
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);         // lgkmcnt(0): the wave reads back only what it wrote
#pragma unroll
      for (int it = 0; it < 8; it++) {
        const int row = 4 * it + rr;
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(ysg + row * A4_YROW + cc * 16);
        const int mr = em0 + xrow0 + 32 * i + row, n = en0 + wcol0 + 8 * cc;
        if (flags & 1) {
          const uint32_t yo = (mr < M && n < N) ? ((uint32_t)mr * (uint32_t)N + (uint32_t)n) * 2u : kBufferOob;
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
    // the next tile's 24 DMAs were issued before this tile's 32 vector stores of
    // y (or 256 element stores), which may stay in flight
    if (flags & 1) wait_vm_lgkm0<32>();
    else wait_vm_lgkm0<0>();
    __builtin_amdgcn_s_barrier();
    fence();
    local = nlocal;
  }
}

// The DMA offsets reach (rows + 255) * k/2 + k/2 + 64 bytes into a code plane
// (the last tile's rows, a 128-k tail loaded as a full K tile), all 32-bit.
bool gemm_a4w4_supports(int64_t m, int64_t n, int64_t k) {
  const int64_t lim = (int64_t)1 << 31;
  return k > 0 && k % 128 == 0 && k < lim && (m + 2 * A4_BM) * (k / 2) < lim && (n + 2 * A4_BN) * (k / 2) < lim &&
         m * n * 2 < ((int64_t)1 << 32);
}

hipError_t launch_gemm_a4w4(const uint8_t* xc, const uint8_t* xs, int64_t m, int64_t k, const uint8_t* wc,
                            const uint8_t* ws, int64_t n, void* y, hipStream_t stream) {
  if (m == 0 || n == 0) return hipSuccess;
  const int64_t tiles = ((m + A4_BM - 1) / A4_BM) * ((n + A4_BN - 1) / A4_BN);
  static std::atomic<uint64_t> lds_done{0};
  {
    hipError_t e = set_max_lds_once(reinterpret_cast<const void*>(&gemm_a4w4_kernel), A4_LDS, lds_done);
    if (e != hipSuccess) return e;
  }
  const int flags = (n % 8 == 0 && (reinterpret_cast<uintptr_t>(y) & 15u) == 0) ? 1 : 0;
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const int64_t grid = tiles < cus ? tiles : (cus > 0 ? cus : 1);
  hipLaunchKernelGGL(gemm_a4w4_kernel, dim3((unsigned)grid), dim3(A4_THREADS), A4_LDS, stream, xc, xs, (int)m,
                     (int)k, wc, ws, (int)n, reinterpret_cast<uint16_t*>(y), flags);
  return hipGetLastError();
}

}  // namespace fp4w
