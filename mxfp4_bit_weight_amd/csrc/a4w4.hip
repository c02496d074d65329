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
// accumulators in AGPRs.  Per K tile of 128 (two MFMA steps of 64): the codes of
// x and of W (256 rows x 64 bytes each) and their scale bytes (4 a row) reach
// LDS by DMA, three buffer sets, two K tiles ahead; code rows are swizzled as
// in gemm.hip.  Step 0 reads step 1's fragments and issues the DMA of tile
// kt + 2; the barrier (after each wave's wait for its DMA of tile kt + 1) sits
// before step 1, whose MFMAs cover the reads of the next tile's step-0
// fragments.
#include "fp4w_device.hpp"
#include "fp4w_internal.hpp"
#include "gemm_common.hpp"

namespace fp4w {

constexpr int A4_BM = 256, A4_BN = 256, A4_BK = 128, A4_THREADS = 256, A4_GM = 4;
constexpr int A4_CB = 256 * 64;                       // code bytes of one operand's tile
constexpr int A4_SB = 256 * 4;                        // scale bytes of one operand's tile
constexpr int A4_XC = 0, A4_WC = A4_CB, A4_XS = 2 * A4_CB, A4_WS = 2 * A4_CB + A4_SB;   // offsets in a set
constexpr int A4_SET = 2 * (A4_CB + A4_SB);           // 34816 bytes per buffer set
constexpr int A4_LDS = 3 * A4_SET;
constexpr int A4_YROW = 272;                          // bytes per staged y row (128 bf16 + 16)
static_assert(4 * 32 * A4_YROW <= A4_SET, "the y staging of one pass fits buffer set 2");

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

  const __amdgpu_buffer_rsrc_t xcr = make_rsrc(xc, (uint32_t)M * (uint32_t)(K / 2));
  const __amdgpu_buffer_rsrc_t xsr = make_rsrc(xs, (uint32_t)M * (uint32_t)(K / 32));
  const __amdgpu_buffer_rsrc_t wcr = make_rsrc(wc, (uint32_t)N * (uint32_t)(K / 2));
  const __amdgpu_buffer_rsrc_t wsr = make_rsrc(ws, (uint32_t)N * (uint32_t)(K / 32));

  // DMA lanes.  Codes: instruction i (of 4) of wave w fills rows 64 i + 16 w ..
  // + 15 of a 256 x 64-byte tile; lane l takes row + l / 4, position l % 4, so
  // it loads that row's chunk (l % 4) ^ swzw(row).  Scales (4-byte DMA): wave w
  // fills rows 64 w + l, the 4 scale bytes of the tile's 128 k.  Rows past the
  // matrix read zeros (past the buffer's end).
  const int crow = 16 * wave + (lane >> 2);
  const uint32_t clane = 16u * (uint32_t)((lane & 3) ^ w4_swzw(crow));
  const int srow = 64 * wave + lane;
  uint32_t xcb, wcb, xsb, wsb;
  auto set_bases = [&](int om0, int on0) __attribute__((always_inline)) {
    xcb = (uint32_t)(om0 + crow) * (uint32_t)(K / 2) + clane;
    wcb = (uint32_t)(on0 + crow) * (uint32_t)(K / 2) + clane;
    xsb = (uint32_t)(om0 + srow) * (uint32_t)(K / 32);
    wsb = (uint32_t)(on0 + srow) * (uint32_t)(K / 32);
  };
  set_bases(m0, n0);
  auto setp = [&](int i) __attribute__((always_inline)) -> uint8_t* { return smem + i * A4_SET; };
  // 10 DMAs a wave: 4 + 4 of codes, 1 + 1 of scales
  auto dma_tile = [&](uint8_t* set, int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const uint32_t ro = (uint32_t)i * 64u * (uint32_t)(K / 2) + (uint32_t)(k0 / 2);
      dma16(xcr, set + A4_XC + (64 * i + 16 * wave) * 64, xcb + ro);
      dma16(wcr, set + A4_WC + (64 * i + 16 * wave) * 64, wcb + ro);
    }
    dma4(xsr, set + A4_XS + 64 * wave * 4, xsb + (uint32_t)(k0 / 32));
    dma4(wsr, set + A4_WS + 64 * wave * 4, wsb + (uint32_t)(k0 / 32));
  };

  // fragments of step s (k 64 s .. 64 s + 63 of the tile): chunk 2 s + hh of
  // rows xrow0 / wcol0 + 32 i + l32; the rows' 4 scale bytes once a tile, shifted
  // so that the block of step s and half hh sits in byte 2 s (the MFMA's opsel)
  const int arow = xrow0 + l32, brow = wcol0 + l32;
  int xoff[2], woff[2];
#pragma unroll
  for (int s = 0; s < 2; s++) {
    xoff[s] = arow * 64 + 16 * ((2 * s + hh) ^ w4_swzw(arow));
    woff[s] = brow * 64 + 16 * ((2 * s + hh) ^ w4_swzw(brow));
  }
  typedef __attribute__((ext_vector_type(8))) int i32x8_t;
  struct Frag {
    i32x8_t x[4], w[4];
  };
  auto read_frag = [&](Frag& f, const uint8_t* set, int s) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(set + A4_XC + xoff[s] + 32 * i * 64);
      f.x[i] = i32x8_t{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
      const u32x4_t u = *reinterpret_cast<const u32x4_t*>(set + A4_WC + woff[s] + 32 * i * 64);
      f.w[i] = i32x8_t{(int)u.x, (int)u.y, (int)u.z, (int)u.w, 0, 0, 0, 0};
    }
  };
  uint32_t xsc[4], wsc[4];
  auto read_scales = [&](const uint8_t* set) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; i++) {
      xsc[i] = *reinterpret_cast<const uint32_t*>(set + A4_XS + (arow + 32 * i) * 4) >> (8 * hh);
      wsc[i] = *reinterpret_cast<const uint32_t*>(set + A4_WS + (brow + 32 * i) * 4) >> (8 * hh);
    }
  };

  f32x16_t acc[4][4];                             // [j: 32 rows of W][i: 32 rows of x]
  auto mfma_step = [&](const Frag& f, int s) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 4; j++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        if (s == 0)
          acc[j][i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.w[j], f.x[i], acc[j][i], 4, 4, 0,
                                                                       (int)wsc[j], 0, (int)xsc[i]);
        else
          acc[j][i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.w[j], f.x[i], acc[j][i], 4, 4, 2,
                                                                       (int)wsc[j], 2, (int)xsc[i]);
      }
  };
  auto fence = [&]() __attribute__((always_inline)) { __builtin_amdgcn_sched_barrier(0); };

  const int nk = K / A4_BK;
  Frag f0, f1;
  uint32_t xsn[4], wsn[4];
  // one K tile (buffer set kt % 3): on entry f0 and xsc / wsc hold its step-0
  // fragments and its scale words (reads issued)
  auto tile = [&](int kt) __attribute__((always_inline)) {
    const uint8_t* cur = setp(kt % 3);
    read_frag(f1, cur, 1);
    dma_tile(setp((kt + 2) % 3), (kt + 2) * A4_BK);
    mfma_step(f0, 0);
    fence();
    wait_vm_lgkm0<10>();                          // this wave's DMA of tile kt + 1 is done
    __builtin_amdgcn_s_barrier();
    fence();
    const uint8_t* nxt = setp((kt + 1) % 3);
    read_frag(f0, nxt, 0);
#pragma unroll
    for (int i = 0; i < 4; i++) {
      xsn[i] = *reinterpret_cast<const uint32_t*>(nxt + A4_XS + (arow + 32 * i) * 4) >> (8 * hh);
      wsn[i] = *reinterpret_cast<const uint32_t*>(nxt + A4_WS + (brow + 32 * i) * 4) >> (8 * hh);
    }
    mfma_step(f1, 1);
    fence();
#pragma unroll
    for (int i = 0; i < 4; i++) { xsc[i] = xsn[i]; wsc[i] = wsn[i]; }
  };

  dma_tile(setp(0), 0);
  dma_tile(setp(1), A4_BK);
  wait_vm_lgkm0<0>();
  __builtin_amdgcn_s_barrier();
  fence();
  for (;;) {
    read_frag(f0, setp(0), 0);
    read_scales(setp(0));
#pragma unroll
    for (int j = 0; j < 4; j++)
#pragma unroll
      for (int i = 0; i < 4; i++) acc[j][i] = f32x16_t{};
    fence();
    // DMAs past K (the last two tiles' successors) read the next rows' data or
    // zeros past the buffers and feed nothing
    for (int kt = 0; kt < nk; kt++) tile(kt);
    wait_vm_lgkm0<0>();                           // every wave is past the loop's last LDS reads
    __builtin_amdgcn_s_barrier();
    fence();
    const int em0 = m0, en0 = n0;
    const int nlocal = local + nwg;
    const bool more = nlocal < xcount;
    if (more) {                                   // the next tile's first two K tiles, into sets 0 and 1
      origin(nlocal, m0, n0);
      set_bases(m0, n0);
      dma_tile(setp(0), 0);
      dma_tile(setp(1), A4_BK);
    }
    asm volatile("" ::: "memory");                // the stores below stay after these DMAs
    fence();

    // store (as in gemm.hip): 4 passes of one x block each through set 2, 32 rows
    // x 128 bf16 a wave, 8 stores of 16 bytes a lane and pass (rows and columns
    // past y dropped); flags & 1: y 16-byte aligned and n a multiple of 8, else
    // 2-byte stores
    const __amdgpu_buffer_rsrc_t yr = make_rsrc(y, (uint32_t)M * (uint32_t)N * 2u);
    uint8_t* const ysg = smem + 2 * A4_SET + wave * (32 * A4_YROW);
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
    // the next tile's DMA was issued before this tile's 32 vector stores of y
    // (or 256 element stores), which may stay in flight
    if (flags & 1) wait_vm_lgkm0<32>();
    else wait_vm_lgkm0<0>();
    __builtin_amdgcn_s_barrier();
    fence();
    local = nlocal;
  }
}

// The DMA offsets reach (rows + 255) * k/2 + k/2 + 112 bytes into a code plane
// (the last tile's rows and the two K tiles past the end), all 32-bit.
bool gemm_a4w4_supports(int64_t m, int64_t n, int64_t k) {
  const int64_t lim = (int64_t)1 << 31;
  return k > 0 && k % A4_BK == 0 && k < lim && (m + 2 * A4_BM) * (k / 2) < lim && (n + 2 * A4_BN) * (k / 2) < lim &&
         m * n * 2 < ((int64_t)1 << 32);
}

hipError_t launch_gemm_a4w4(const uint8_t* xc, const uint8_t* xs, int64_t m, int64_t k, const uint8_t* wc,
                            const uint8_t* ws, int64_t n, void* y, hipStream_t stream) {
  if (m == 0 || n == 0) return hipSuccess;
  const int64_t tiles = ((m + A4_BM - 1) / A4_BM) * ((n + A4_BN - 1) / A4_BN);
  static bool lds_set = false;
  if (!lds_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_a4w4_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, A4_LDS);
    if (e != hipSuccess) return e;
    lds_set = true;
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
