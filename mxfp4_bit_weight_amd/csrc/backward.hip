// backward.hip -- the input gradient through the frozen 4-bit base,
// dX (m, k) = dY (m, n) deq(W) (n, k), fp32 accumulation, bf16 out.
//
// QLoRA-style training keeps the quantized base frozen and back-propagates
// through it into the adapter and the layers below (Telegram post, "Metod";
// the same post trains at batch 8 x 2k, "Eksperimenty").  The forward contracts
// over k, along which the blocks run; here the contraction runs over n, across
// code rows, so a weight tile is decoded once per workgroup into LDS transposed
// ([k][n], n contiguous) and fed to the bf16 matrix core from there.  The decode
// is exact: e2m1 times an E4M3 scale has at most 6 significant bits, e2m1 times
// an E8M0 power of two is a bf16 value (or inf past bf16's range, scale codes 253
// and 254, as dequantizing to bf16 gives); the NVFP4 tensor scale multiplies the
// fp32 sums once.
//
// Workgroup: 128 rows of dX x 128 columns (k), 4 waves in 2 x 2, each 64 x 64 =
// 2 x 2 v_mfma_f32_32x32x16_bf16 tiles, W as operand A (rows k) and dY as operand
// B (columns m), so a lane's results are runs of 4 consecutive k of one row of
// dX.  The n loop takes chunks of 64: the next chunk's dY (128 x 64 bf16) and
// codes (64 x 64 bytes) are loaded into registers while the current chunk's
// MFMAs run, then written (dY as is, W decoded) into the other of two LDS
// buffers; one barrier per chunk.  Needs n % 8 == 0 and k % 32 == 0.
#include "fp4w_device.hpp"
#include "fp4w_internal.hpp"

namespace fp4w {

constexpr int BW_BM = 128, BW_BK = 128, BW_NC = 64, BW_THREADS = 256;
constexpr int BW_STRIDE = 144;                 // bytes per LDS row: 64 bf16 + 16 (16 consecutive rows: distinct banks)
constexpr int BW_TILE = 128 * BW_STRIDE;       // one operand tile (128 rows)
constexpr int BW_LDS = 2 * 2 * BW_TILE;        // two buffers of [dY tile][W^T tile]

typedef __attribute__((ext_vector_type(16))) float bw_f32x16_t;

template <int SEL>
__device__ __forceinline__ void bw_decode_byte(uint32_t c0, uint32_t c1, float s0, float s1, uint8_t* bt, int kl,
                                               int wp) {
  // byte SEL of rows 2 wp (c0) and 2 wp + 1 (c1): k = kl, kl + 1 -> two dwords
  // (bf16 of row 2 wp low, row 2 wp + 1 high) at W^T rows kl and kl + 1
  const f32x2_t a = fp4x2_to_f32x2<SEL>(c0, 1.0f) * s0;
  const f32x2_t b = fp4x2_to_f32x2<SEL>(c1, 1.0f) * s1;
  // the products are bf16 values (or inf / NaN), so dropping the low half is exact
  *reinterpret_cast<uint32_t*>(bt + kl * BW_STRIDE + 4 * wp) =
      (__float_as_uint(b.x) & 0xFFFF0000u) | (__float_as_uint(a.x) >> 16);
  *reinterpret_cast<uint32_t*>(bt + (kl + 1) * BW_STRIDE + 4 * wp) =
      (__float_as_uint(b.y) & 0xFFFF0000u) | (__float_as_uint(a.y) >> 16);
}

template <int FMT>
__global__ __launch_bounds__(BW_THREADS, 2) void backward_dx_kernel(
    const uint16_t* __restrict__ dy, int M, int N, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ scales, const float* __restrict__ tensor_scale, int K, uint16_t* __restrict__ dx,
    const float* __restrict__ lu, const uint16_t* __restrict__ la, int lr) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[BW_LDS];
  constexpr int BLK = FMT == FMT_NVFP4 ? 16 : 32;
  const int k0 = blockIdx.x * BW_BK, m0 = blockIdx.y * BW_BM;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wk = wave & 1;
  const int l32 = lane & 31, hh = lane >> 5;
  const int64_t kb = K / 2, ks = K / BLK;        // code bytes and scale bytes per row of W

  // loaders: dY row ar, n 32 ac .. + 31 (four 16-byte loads); W rows 2 wp and
  // 2 wp + 1 of the chunk, k = 16 wc .. + 15 (8 code bytes and one scale byte
  // each: 16 k lie inside one block of either format)
  const int ar = tid >> 1, ac = tid & 1;
  const int wp = tid & 31, wc = tid >> 5;
  u32x4_t ya[4];
  uint2 cw0, cw1;
  uint32_t sb0, sb1;
  auto gload = [&](int n0) __attribute__((always_inline)) {
    const int m = m0 + ar;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int n = n0 + 32 * ac + 8 * i;
      ya[i] = (m < M && n < N) ? load16(dy + (int64_t)m * N + n) : u32x4_t{0u, 0u, 0u, 0u};
    }
    const int n = n0 + 2 * wp, kk = k0 + 16 * wc;
    cw0 = cw1 = make_uint2(0u, 0u);
    sb0 = sb1 = 0u;                               // rows past W decode to zero (scale 0, code 0)
    if (kk < K) {
      if (n < N) {
        cw0 = *reinterpret_cast<const uint2*>(codes + (int64_t)n * kb + kk / 2);
        sb0 = scales[(int64_t)n * ks + kk / BLK];
      }
      if (n + 1 < N) {
        cw1 = *reinterpret_cast<const uint2*>(codes + (int64_t)(n + 1) * kb + kk / 2);
        sb1 = scales[(int64_t)(n + 1) * ks + kk / BLK];
      }
    }
  };
  auto lstore = [&](int buf) __attribute__((always_inline)) {
    uint8_t* ay = smem + buf * 2 * BW_TILE;
    uint8_t* bt = ay + BW_TILE;
#pragma unroll
    for (int i = 0; i < 4; i++) *reinterpret_cast<u32x4_t*>(ay + ar * BW_STRIDE + 64 * ac + 16 * i) = ya[i];
    const float s0 = FMT == FMT_NVFP4 ? e4m3_to_f32(sb0) : e8m0_to_f32(sb0);
    const float s1 = FMT == FMT_NVFP4 ? e4m3_to_f32(sb1) : e8m0_to_f32(sb1);
    const int kl = 16 * wc;
    bw_decode_byte<0>(cw0.x, cw1.x, s0, s1, bt, kl + 0, wp);
    bw_decode_byte<1>(cw0.x, cw1.x, s0, s1, bt, kl + 2, wp);
    bw_decode_byte<2>(cw0.x, cw1.x, s0, s1, bt, kl + 4, wp);
    bw_decode_byte<3>(cw0.x, cw1.x, s0, s1, bt, kl + 6, wp);
    bw_decode_byte<0>(cw0.y, cw1.y, s0, s1, bt, kl + 8, wp);
    bw_decode_byte<1>(cw0.y, cw1.y, s0, s1, bt, kl + 10, wp);
    bw_decode_byte<2>(cw0.y, cw1.y, s0, s1, bt, kl + 12, wp);
    bw_decode_byte<3>(cw0.y, cw1.y, s0, s1, bt, kl + 14, wp);
  };

  bw_f32x16_t acc[2][2];                          // [jk: 32 k][im: 32 m]
#pragma unroll
  for (int j = 0; j < 2; j++)
#pragma unroll
    for (int i = 0; i < 2; i++) acc[j][i] = bw_f32x16_t{};
  // fragments: lane (r, hh) reads row r of a tile, n 16 s + 8 hh .. + 7
  const int aoff = (64 * wk + l32) * BW_STRIDE + 16 * hh;   // W^T rows (k)
  const int boff = (64 * wm + l32) * BW_STRIDE + 16 * hh;   // dY rows (m)
  auto compute = [&](int buf) __attribute__((always_inline)) {
    const uint8_t* ay = smem + buf * 2 * BW_TILE;
    const uint8_t* bt = ay + BW_TILE;
#pragma unroll
    for (int s = 0; s < 4; s++) {
      bf16x8_t wf[2], yf[2];
#pragma unroll
      for (int j = 0; j < 2; j++) {
        wf[j] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(bt + aoff + 32 * j * BW_STRIDE + 32 * s));
        yf[j] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(ay + boff + 32 * j * BW_STRIDE + 32 * s));
      }
#pragma unroll
      for (int j = 0; j < 2; j++)
#pragma unroll
        for (int i = 0; i < 2; i++) acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[j], yf[i], acc[j][i], 0, 0, 0);
    }
  };

  const int nch = (N + BW_NC - 1) / BW_NC;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int c = 0; c < nch; c++) {
    const bool more = c + 1 < nch;
    if (more) gload((c + 1) * BW_NC);             // in flight during this chunk's MFMAs
    compute(c & 1);
    if (more) lstore((c + 1) & 1);                // that buffer's last reads were before the previous barrier
    __syncthreads();
  }

  // dX = s_t * acc (+ u A), rounded once to bf16: lane (l32, hh), register 4 qq + e
  // of tile (jk, im) is k = 32 jk + 8 qq + 4 hh + e, m = 32 im + l32 of the wave's block
  const float st = FMT == FMT_NVFP4 ? *tensor_scale : 1.0f;
#pragma unroll
  for (int j = 0; j < 2; j++)
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
      for (int q = 0; q < 16; q++) acc[j][i][q] *= st;
  if (lr > 0) {
    // the LoRA term u A (u = dY B, fp32 (M, lr); A (lr, K) bf16) on the same
    // matrix core: A^T of the block's 128 k staged in LDS ([k][j], 16-byte rows of
    // 8 j), u split into two bf16 parts (hi + lo, 2^-16 relative) in registers
    const int RB = (lr + 15) / 16;
    constexpr int AS = 72;                          // bf16 per staged row: 64 j + 8 (bank spread)
    uint16_t* at = reinterpret_cast<uint16_t*>(smem);
    for (int e = tid; e < BW_BK * 16 * RB; e += BW_THREADS) {
      const int jj = e / BW_BK, kk = e - jj * BW_BK;   // consecutive threads: consecutive k of one row of A
      const int k = k0 + kk;
      at[kk * AS + jj] = (jj < lr && k < K) ? la[(int64_t)jj * K + k] : (uint16_t)0;
    }
    __syncthreads();
    for (int b = 0; b < RB; b++) {
      bf16x8_t af[2], uh[2], ul[2];
#pragma unroll
      for (int j = 0; j < 2; j++)
        af[j] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(at + (64 * wk + 32 * j + l32) * AS + 16 * b + 8 * hh));
#pragma unroll
      for (int i = 0; i < 2; i++) {
        const int m = m0 + 64 * wm + 32 * i + l32;
        uint32_t h[4], l[4];
#pragma unroll
        for (int e = 0; e < 4; e++) {
          float v[2];
#pragma unroll
          for (int d = 0; d < 2; d++) {
            const int jj = 16 * b + 8 * hh + 2 * e + d;
            v[d] = (m < M && jj < lr) ? lu[(int64_t)m * lr + jj] : 0.f;
          }
          const uint32_t h0 = f32_to_bf16_rne(v[0]), h1 = f32_to_bf16_rne(v[1]);
          h[e] = h0 | (h1 << 16);
          l[e] = f32_to_bf16_rne(v[0] - __uint_as_float(h0 << 16)) |
                 (f32_to_bf16_rne(v[1] - __uint_as_float(h1 << 16)) << 16);
        }
        uh[i] = as_bf16x8((u32x4_t){h[0], h[1], h[2], h[3]});
        ul[i] = as_bf16x8((u32x4_t){l[0], l[1], l[2], l[3]});
      }
#pragma unroll
      for (int j = 0; j < 2; j++)
#pragma unroll
        for (int i = 0; i < 2; i++) {
          acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[j], uh[i], acc[j][i], 0, 0, 0);
          acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[j], ul[i], acc[j][i], 0, 0, 0);
        }
    }
  }
#pragma unroll
  for (int j = 0; j < 2; j++)
#pragma unroll
    for (int i = 0; i < 2; i++) {
      const int m = m0 + 64 * wm + 32 * i + l32;
#pragma unroll
      for (int qq = 0; qq < 4; qq++) {
        const int k = k0 + 64 * wk + 32 * j + 8 * qq + 4 * hh;
        if (m < M && k < K) {
          uint32_t o[4];
#pragma unroll
          for (int e = 0; e < 4; e++) o[e] = f32_to_bf16_rne(acc[j][i][4 * qq + e]);
          *reinterpret_cast<uint2*>(dx + (int64_t)m * K + k) = make_uint2(o[0] | (o[1] << 16), o[2] | (o[3] << 16));
        }
      }
    }
}

hipError_t launch_backward_dx(int fmt, const void* dy, int64_t m, int64_t n, const uint8_t* codes,
                              const uint8_t* scales, const float* tensor_scale, int64_t k, void* dx, const float* lu,
                              const void* la, int lr, hipStream_t stream) {
  if (m == 0 || k == 0) return hipSuccess;
  const dim3 grid((unsigned)((k + BW_BK - 1) / BW_BK), (unsigned)((m + BW_BM - 1) / BW_BM));
  const uint16_t* y = reinterpret_cast<const uint16_t*>(dy);
  uint16_t* o = reinterpret_cast<uint16_t*>(dx);
  if (fmt == FMT_NVFP4)
    hipLaunchKernelGGL(backward_dx_kernel<FMT_NVFP4>, grid, dim3(BW_THREADS), 0, stream, y, (int)m, (int)n, codes,
                       scales, tensor_scale, (int)k, o, lu, reinterpret_cast<const uint16_t*>(la), lr);
  else
    hipLaunchKernelGGL(backward_dx_kernel<FMT_MXFP4>, grid, dim3(BW_THREADS), 0, stream, y, (int)m, (int)n, codes,
                       scales, tensor_scale, (int)k, o, lu, reinterpret_cast<const uint16_t*>(la), lr);
  return hipGetLastError();
}

}  // namespace fp4w
