// delta_grad.hip -- the Scale-QLoRA training gradient of the block-scale deltas:
//   g[n, b] = s_t * sum_{k in block b} e2m1(q[n, k]) * G[n, k],  G = dY^T X,
// for a frozen quantized W (n, k), the layer's input X (m, k) and its output
// gradient dY (m, n); fp32 out (n, k / blk).
//
// Scale-QLoRA trains a correction per block scale in the decoded scale domain,
// rounded to the format's scale grid in every forward (Scale-QLoRA page, merge
// paragraphs); the rounding is passed straight through, so the gradient of a
// block's delta is the sum over its k of dL/dW[n, k] = G[n, k] times the
// block's codes decoded without their scale (times the NVFP4 tensor scale).
// G never reaches HBM: each workgroup forms a 128 x 128 tile of it on the bf16
// matrix core, contracting over the m rows, and reduces it against the codes in
// its epilogue.
//
// Both operands contract over their row index m, so each m chunk (64 rows) of
// X (128 columns k) and of dY (128 columns n) is written to LDS transposed
// ([k][m] and [n][m], m contiguous, rows padded to 144 bytes), two rows of m
// per 32-bit store.  4 waves in 2 x 2, each 64 (k) x 64 (n) = 2 x 2
// v_mfma_f32_32x32x16_bf16 tiles with X^T as operand A (rows k) and dY^T as
// operand B (columns n): a lane holds 16 k of one n, those of one NVFP4 block
// (rows 0-15 or 16-31 of a tile) split over the lane and the lane 32 away.
// The next chunk is loaded into registers while the current one's MFMAs run;
// one barrier per chunk.  Needs n % 8 == 0, k % 32 == 0.
#include "fp4w_device.hpp"
#include "fp4w_internal.hpp"

namespace fp4w {

constexpr int DG_BN = 128, DG_BK = 128, DG_MC = 64, DG_THREADS = 256;
constexpr int DG_STRIDE = 144;                 // bytes per LDS row: 64 bf16 of m + 16
constexpr int DG_TILE = 128 * DG_STRIDE;
constexpr int DG_BUF = 2 * DG_TILE;            // [X^T tile][dY^T tile]
constexpr int DG_LDS = 2 * DG_BUF;             // 73728 bytes

typedef __attribute__((ext_vector_type(16))) float dg_f32x16_t;

template <int FMT>
__global__ __launch_bounds__(DG_THREADS, 2) void delta_grad_kernel(
    const uint16_t* __restrict__ dy, const uint16_t* __restrict__ x, int M, int N, int K,
    const uint8_t* __restrict__ codes, const float* __restrict__ tensor_scale, float* __restrict__ g) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[DG_LDS];
  constexpr int BLK = FMT == FMT_NVFP4 ? 16 : 32;
  const int k0 = blockIdx.x * DG_BK, n0 = blockIdx.y * DG_BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wk = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, hh = lane >> 5;

  // loaders: rows 2 p and 2 p + 1 of the m chunk, columns 16 q .. 16 q + 15 of
  // the tile, for X and for dY (two 16-byte loads per row and operand)
  const int p = tid & 31, q = tid >> 5;
  u32x4_t xr[2][2], yr[2][2];                     // [row][half]
  auto gload = [&](int mc) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < 2; r++) {
      const int m = mc + 2 * p + r;
#pragma unroll
      for (int h = 0; h < 2; h++) {
        const int kk = k0 + 16 * q + 8 * h, nn = n0 + 16 * q + 8 * h;
        xr[r][h] = (m < M && kk < K) ? load16(x + (int64_t)m * K + kk) : u32x4_t{0u, 0u, 0u, 0u};
        yr[r][h] = (m < M && nn < N) ? load16(dy + (int64_t)m * N + nn) : u32x4_t{0u, 0u, 0u, 0u};
      }
    }
  };
  // column c of the tile, rows 2 p and 2 p + 1: one dword (row 2 p in the low half)
  auto lstore = [&](int buf) __attribute__((always_inline)) {
    uint8_t* xt = smem + buf * DG_BUF;
    uint8_t* yt = xt + DG_TILE;
#pragma unroll
    for (int h = 0; h < 2; h++)
#pragma unroll
      for (int d = 0; d < 4; d++) {
        const int c = 16 * q + 8 * h + 2 * d;
        const uint32_t x0 = xr[0][h][d], x1 = xr[1][h][d], y0 = yr[0][h][d], y1 = yr[1][h][d];
        *reinterpret_cast<uint32_t*>(xt + c * DG_STRIDE + 4 * p) = (x0 & 0xFFFFu) | (x1 << 16);
        *reinterpret_cast<uint32_t*>(xt + (c + 1) * DG_STRIDE + 4 * p) = (x0 >> 16) | (x1 & 0xFFFF0000u);
        *reinterpret_cast<uint32_t*>(yt + c * DG_STRIDE + 4 * p) = (y0 & 0xFFFFu) | (y1 << 16);
        *reinterpret_cast<uint32_t*>(yt + (c + 1) * DG_STRIDE + 4 * p) = (y0 >> 16) | (y1 & 0xFFFF0000u);
      }
  };

  dg_f32x16_t acc[2][2];                          // [jk: 32 k][in: 32 n]
#pragma unroll
  for (int j = 0; j < 2; j++)
#pragma unroll
    for (int i = 0; i < 2; i++) acc[j][i] = dg_f32x16_t{};
  const int aoff = (64 * wk + l32) * DG_STRIDE + 16 * hh;   // X^T rows (k)
  const int boff = (64 * wn + l32) * DG_STRIDE + 16 * hh;   // dY^T rows (n)
  auto compute = [&](int buf) __attribute__((always_inline)) {
    const uint8_t* xt = smem + buf * DG_BUF;
    const uint8_t* yt = xt + DG_TILE;
#pragma unroll
    for (int s = 0; s < 4; s++) {
      bf16x8_t af[2], bf[2];
#pragma unroll
      for (int j = 0; j < 2; j++) {
        af[j] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(xt + aoff + 32 * j * DG_STRIDE + 32 * s));
        bf[j] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(yt + boff + 32 * j * DG_STRIDE + 32 * s));
      }
#pragma unroll
      for (int j = 0; j < 2; j++)
#pragma unroll
        for (int i = 0; i < 2; i++) acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[j], bf[i], acc[j][i], 0, 0, 0);
    }
  };

  const int nch = (M + DG_MC - 1) / DG_MC;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int c = 0; c < nch; c++) {
    const bool more = c + 1 < nch;
    if (more) gload((c + 1) * DG_MC);
    compute(c & 1);
    if (more) lstore((c + 1) & 1);
    __syncthreads();
  }

  // epilogue: tile (jk, in) holds G[n, k] for n = n-base + l32, k = k-base +
  // 8 (e / 4) + 4 hh + e % 4 (register e).  Times e2m1(q[n, k]), summed per block:
  // NVFP4 blocks are rows 0-15 (e < 8) and 16-31 (e >= 8), MXFP4 the whole tile;
  // the lane 32 away holds the other half of each block's k.
  const float st = FMT == FMT_NVFP4 ? *tensor_scale : 1.0f;
  const int64_t kb = K / 2, gs = K / BLK;
#pragma unroll
  for (int j = 0; j < 2; j++)
#pragma unroll
    for (int i = 0; i < 2; i++) {
      const int n = n0 + 64 * wn + 32 * i + l32;
      const int kt = k0 + 64 * wk + 32 * j;       // first k of this 32 x 32 tile
      u32x4_t cw = {0u, 0u, 0u, 0u};
      if (n < N && kt < K) cw = load16(codes + (int64_t)n * kb + kt / 2);
      float part[2] = {0.f, 0.f};
#pragma unroll
      for (int e = 0; e < 16; e++) {
        const int kr = 8 * (e / 4) + 4 * hh + (e % 4);   // k within the tile: nibble kr of cw
        const uint32_t nib = (cw[kr >> 3] >> (4 * (kr & 7))) & 0xFu;
        // e2m1 decoded from its bits: sign, exponent (bias 1), mantissa
        const uint32_t ex = (nib >> 1) & 3u, mt = nib & 1u;
        float v = ex == 0 ? 0.5f * (float)mt : (float)(2u + mt) * (float)(1u << ex) * 0.25f;
        v = (nib & 8u) ? -v : v;
        part[e >> 3] += v * acc[j][i][e];
      }
      // the other half of each block: lane +- 32
      part[0] += __shfl_xor(part[0], 32);
      part[1] += __shfl_xor(part[1], 32);
      if (n < N && kt < K) {
        if (FMT == FMT_NVFP4) {
          if (hh == 0) g[(int64_t)n * gs + kt / 16 + 0] = st * part[0];
          else g[(int64_t)n * gs + kt / 16 + 1] = st * part[1];
        } else if (hh == 0) {
          g[(int64_t)n * gs + kt / 32] = part[0] + part[1];
        }
      }
    }
}

hipError_t launch_delta_grad(int fmt, const void* dy, const void* x, int64_t m, int64_t n, int64_t k,
                             const uint8_t* codes, const float* tensor_scale, float* grad, hipStream_t stream) {
  if (n == 0 || k == 0) return hipSuccess;
  const dim3 grid((unsigned)((k + DG_BK - 1) / DG_BK), (unsigned)((n + DG_BN - 1) / DG_BN));
  const uint16_t* yy = reinterpret_cast<const uint16_t*>(dy);
  const uint16_t* xx = reinterpret_cast<const uint16_t*>(x);
  if (fmt == FMT_NVFP4)
    hipLaunchKernelGGL(delta_grad_kernel<FMT_NVFP4>, grid, dim3(DG_THREADS), 0, stream, yy, xx, (int)m, (int)n,
                       (int)k, codes, tensor_scale, grad);
  else
    hipLaunchKernelGGL(delta_grad_kernel<FMT_MXFP4>, grid, dim3(DG_THREADS), 0, stream, yy, xx, (int)m, (int)n,
                       (int)k, codes, tensor_scale, grad);
  return hipGetLastError();
}

}  // namespace fp4w
