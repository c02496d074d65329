// lora_grad.hip -- gradients of the LoRA branch of the linear.
//
// The pages train a LoRA adapter in parallel to the frozen 4-bit base (Telegram
// post tggo.me/sberlogasci/42740, section "Metod"; batch 8 x 2k in
// "Eksperimenty"): y = x deq(W)^T + (x A^T) B^T with A (r, k) and B (n, r).
// From the output gradient dY (m, n) and the input x (m, k):
//     t  = x A^T   (m, r)      u  = dY B    (m, r)
//     dB = dY^T t  (n, r)      dA = u^T x   (r, k)
// and u A joins the input gradient inside the backward through the base
// (backward.hip).  None of these has a 4-bit operand; they are bf16 products
// on the matrix core with fp32 accumulation:
//  - t and u contract over the contiguous dimension of x / dY ("row" products,
//    lg_row_kernel): each wave takes 16 rows, v_mfma_f32_16x16x32_bf16 with the
//    rows as A and A / B^T (rows of r) as B; the contracted dimension is split
//    over workgroups and the partials added in a fixed order (lg_reduce_kernel);
//  - dB and dA contract over m, the strided dimension ("column" products,
//    lg_col_kernel): a 32 x 64 tile of dY / x is written to LDS transposed, so a
//    lane reads 8 consecutive m of one column; t and u enter as two bf16 parts
//    (hi + lo, 2^-16 relative), written transposed by the reduction before.
// Every sum runs in a fixed order, so results do not depend on scheduling.
#include "fp4w_device.hpp"
#include "fp4w_internal.hpp"

namespace fp4w {

constexpr int LG_MAX_RB = 4;          // r <= 64: four column blocks of 16
constexpr int LG_ROW_U = 4;           // 32-wide steps whose loads are issued together
constexpr int LG_CT = 64;             // columns per workgroup of the column product
constexpr int LG_CM = 32;             // m per step of the column product
constexpr int LG_TS = LG_CM + 8;      // LDS row stride (bf16) of the transposed tile

// B (n, r) -> B^T (r, n) bf16 (B need only be 2-byte aligned).
__global__ void lg_transpose_kernel(const uint16_t* __restrict__ b, int64_t n, int r, uint16_t* __restrict__ bt) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= n * r) return;
  const int64_t row = e / r;
  const int j = (int)(e - row * r);
  bt[(int64_t)j * n + row] = b[e];
}

// out[s][m][j] = sum over c in split s of Y[m][c] V[j][c]; Y (M, C), V (r, C) bf16,
// rows 16-byte aligned, C % 8 == 0.  Grid (ceil(M / 64), S); 4 waves of 16 rows.
__global__ __launch_bounds__(256) void lg_row_kernel(const uint16_t* __restrict__ y, int64_t M, int64_t C,
                                                     const uint16_t* __restrict__ v, int r, int64_t cs,
                                                     float* __restrict__ out) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, li = lane & 15, g = lane >> 4;
  const int64_t m = (int64_t)blockIdx.x * 64 + 16 * wave + li;
  const int s = blockIdx.y;
  const int64_t c0 = (int64_t)s * cs, c1 = c0 + cs < C ? c0 + cs : C;
  const int RB = (r + 15) / 16;
  f32x4_t acc[LG_MAX_RB];
#pragma unroll
  for (int b = 0; b < LG_MAX_RB; b++) acc[b] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  for (int64_t c = c0; c < c1; c += 32 * LG_ROW_U) {
    u32x4_t ya[LG_ROW_U], va[LG_ROW_U][LG_MAX_RB];
#pragma unroll
    for (int u = 0; u < LG_ROW_U; u++) {
      const int64_t cc = c + 32 * u + 8 * g;
      const bool cok = cc + 8 <= c1;
      ya[u] = (cok && m < M) ? load16(y + m * C + cc) : (u32x4_t){0u, 0u, 0u, 0u};
#pragma unroll
      for (int b = 0; b < LG_MAX_RB; b++) {
        const int j = 16 * b + li;
        va[u][b] = (b < RB && cok && j < r) ? load16(v + (int64_t)j * C + cc) : (u32x4_t){0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int u = 0; u < LG_ROW_U; u++)
#pragma unroll
      for (int b = 0; b < LG_MAX_RB; b++)
        if (b < RB) acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ya[u]), as_bf16x8(va[u][b]), acc[b], 0, 0, 0);
  }
  // lane (j = li, g) holds rows 4 g + i of the wave's 16
#pragma unroll
  for (int b = 0; b < LG_MAX_RB; b++) {
    if (b >= RB) break;
    const int j = 16 * b + li;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int64_t mm = (int64_t)blockIdx.x * 64 + 16 * wave + 4 * g + i;
      if (mm < M && j < r) out[((int64_t)s * M + mm) * r + j] = acc[b][i];
    }
  }
}

// out[s][c][j] = sum over m in split s of Y[m][c] (vh[j][m] + vl[j][m]); Y (M, C)
// bf16 rows 16-byte aligned, C % 8 == 0; vh, vl (r, Mp) bf16, Mp a multiple of 32,
// zero past M.  Grid (ceil(C / 64), S), 4 waves of 16 columns; a 32 x 64 tile of Y
// per step, loaded into registers one step ahead and stored transposed into the
// other of two LDS buffers.
__global__ __launch_bounds__(256) void lg_col_kernel(const uint16_t* __restrict__ y, int64_t M, int64_t C,
                                                     const uint16_t* __restrict__ vh, const uint16_t* __restrict__ vl,
                                                     int64_t Mp, int r, int64_t ms, float* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[2][LG_CT * LG_TS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, li = lane & 15, g = lane >> 4;
  const int64_t cb = (int64_t)blockIdx.x * LG_CT;
  const int s = blockIdx.y;
  const int64_t m0 = (int64_t)s * ms, m1 = m0 + ms < M ? m0 + ms : M;
  const int RB = (r + 15) / 16;
  // loader: row ml = tid / 8 of the step, columns 8 (tid % 8) .. + 7
  const int ml = tid >> 3, cl = 8 * (tid & 7);
  const bool cok = cb + cl + 8 <= C;
  auto gload = [&](int64_t ms0) -> u32x4_t {
    const int64_t mm = ms0 + ml;
    return (cok && mm < m1) ? load16(y + mm * C + cb + cl) : (u32x4_t){0u, 0u, 0u, 0u};
  };
  auto lstore = [&](int buf, u32x4_t v) {
    uint16_t* t = tile[buf];
#pragma unroll
    for (int e = 0; e < 4; e++) {
      t[(cl + 2 * e) * LG_TS + ml] = (uint16_t)(v[e] & 0xFFFFu);
      t[(cl + 2 * e + 1) * LG_TS + ml] = (uint16_t)(v[e] >> 16);
    }
  };
  f32x4_t acc[LG_MAX_RB];
#pragma unroll
  for (int b = 0; b < LG_MAX_RB; b++) acc[b] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  const int nst = (int)((m1 - m0 + LG_CM - 1) / LG_CM);
  if (nst > 0) lstore(0, gload(m0));
  __syncthreads();
  for (int st = 0; st < nst; st++) {
    const int64_t msn = m0 + (int64_t)(st + 1) * LG_CM;
    const u32x4_t next = st + 1 < nst ? gload(msn) : (u32x4_t){0u, 0u, 0u, 0u};
    const int64_t mcur = m0 + (int64_t)st * LG_CM + 8 * g;     // this lane's first m of the step
    const u32x4_t a = *reinterpret_cast<const u32x4_t*>(tile[st & 1] + (16 * wave + li) * LG_TS + 8 * g);
#pragma unroll
    for (int b = 0; b < LG_MAX_RB; b++) {
      if (b < RB) {
        const int j = 16 * b + li;
        const bool ok = j < r;
        const u32x4_t bh = ok ? load16(vh + (int64_t)j * Mp + mcur) : (u32x4_t){0u, 0u, 0u, 0u};
        const u32x4_t bl = ok ? load16(vl + (int64_t)j * Mp + mcur) : (u32x4_t){0u, 0u, 0u, 0u};
        acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(bh), acc[b], 0, 0, 0);
        acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(bl), acc[b], 0, 0, 0);
      }
    }
    if (st + 1 < nst) lstore((st + 1) & 1, next);     // that buffer's last reads were before the last barrier
    __syncthreads();
  }
  // lane (j = li, g) holds columns 16 wave + 4 g + i
#pragma unroll
  for (int b = 0; b < LG_MAX_RB; b++) {
    if (b >= RB) break;
    const int j = 16 * b + li;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int64_t c = cb + 16 * wave + 4 * g + i;
      if (c < C && j < r) out[((int64_t)s * C + c) * r + j] = acc[b][i];
    }
  }
}

// The partials [S][R][r] added in split order, written as:
//   mode 0: (hi, lo) bf16 parts transposed, (r, Mp), zeros for rows R .. Mp - 1
//   mode 1: as mode 0, and fp32 (R, r) into o32 (when given)
//   mode 2: fp32 (R, r) into o32
//   mode 3: fp32 transposed (r, R) into o32
__global__ void lg_reduce_kernel(const float* __restrict__ part, int S, int64_t R, int r, int mode,
                                 float* __restrict__ o32, uint16_t* __restrict__ hi, uint16_t* __restrict__ lo,
                                 int64_t Rp) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t rows = mode <= 1 ? Rp : R;
  if (e >= rows * r) return;
  const int64_t row = e / r;
  const int j = (int)(e - row * r);
  float v = 0.f;
  if (row < R)
    for (int q = 0; q < S; q++) v += part[((int64_t)q * R + row) * r + j];
  if (mode <= 1) {
    const uint32_t h = f32_to_bf16_rne(v);
    const float rem = v - __uint_as_float(h << 16);
    hi[(int64_t)j * Rp + row] = (uint16_t)h;
    lo[(int64_t)j * Rp + row] = (uint16_t)f32_to_bf16_rne(rem);
    if (mode == 1 && o32 && row < R) o32[e] = v;
  } else if (mode == 2) {
    o32[e] = v;
  } else {
    o32[(int64_t)j * R + row] = v;
  }
}

// ---------------------------------------------------------------------------------
// Host side: workspace layout and launches.
// ---------------------------------------------------------------------------------
static size_t lg_align(size_t v) { return (v + 255) & ~(size_t)255; }

struct LgPlan {
  int64_t Mp;
  int st_, su, sb, sa;            // splits of the four products
  int64_t cst, csu, msb, msa;     // their sizes along the contracted dimension
  size_t o_bt, o_tp, o_th, o_tl, o_up, o_uh, o_ul, o_bp, o_ap, bytes;
};

static int64_t lg_round(int64_t v, int64_t q) { return (v + q - 1) / q * q; }

// splits so that a product has about 1024 workgroups, each split a multiple of q
static void lg_split(int64_t blocks, int64_t len, int64_t q, int& S, int64_t& sz) {
  int64_t s = (1024 + blocks - 1) / (blocks > 0 ? blocks : 1);
  if (s < 1) s = 1;
  const int64_t maxs = (len + 4 * q - 1) / (4 * q);             // at least 4 q per split
  if (s > maxs) s = maxs > 0 ? maxs : 1;
  sz = lg_round((len + s - 1) / s, q);
  if (sz < q) sz = q;
  S = (int)((len + sz - 1) / sz);
  if (S < 1) S = 1;
}

static LgPlan lg_plan(int64_t m, int64_t n, int64_t k, int r) {
  LgPlan p{};
  p.Mp = lg_round(m > 0 ? m : 1, 32);
  const int64_t mb = (m + 63) / 64;
  lg_split(mb, k, 32 * LG_ROW_U, p.st_, p.cst);
  lg_split(mb, n, 32 * LG_ROW_U, p.su, p.csu);
  lg_split((n + LG_CT - 1) / LG_CT, m, LG_CM, p.sb, p.msb);
  lg_split((k + LG_CT - 1) / LG_CT, m, LG_CM, p.sa, p.msa);
  size_t off = 0;
  p.o_bt = off; off += lg_align((size_t)r * n * 2);
  p.o_tp = off; off += lg_align((size_t)p.st_ * m * r * 4);
  p.o_th = off; off += lg_align((size_t)r * p.Mp * 2);
  p.o_tl = off; off += lg_align((size_t)r * p.Mp * 2);
  p.o_up = off; off += lg_align((size_t)p.su * m * r * 4);
  p.o_uh = off; off += lg_align((size_t)r * p.Mp * 2);
  p.o_ul = off; off += lg_align((size_t)r * p.Mp * 2);
  p.o_bp = off; off += lg_align((size_t)p.sb * n * r * 4);
  p.o_ap = off; off += lg_align((size_t)p.sa * k * r * 4);
  p.bytes = off;
  return p;
}

size_t lora_backward_workspace_bytes(int64_t m, int64_t n, int64_t k, int r) { return lg_plan(m, n, k, r).bytes; }

static hipError_t lg_reduce(const float* part, int S, int64_t R, int r, int mode, float* o32, uint16_t* hi,
                            uint16_t* lo, int64_t Rp, hipStream_t stream) {
  const int64_t rows = mode <= 1 ? Rp : R;
  const int64_t total = rows * r;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(lg_reduce_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, part, S, R, r,
                     mode, o32, hi, lo, Rp);
  return hipGetLastError();
}

hipError_t launch_lora_backward(const void* dy, int64_t m, int64_t n, const void* x, int64_t k, const void* la,
                                const void* lb, int r, float* u_out, float* grad_a, float* grad_b, void* workspace,
                                hipStream_t stream) {
  const LgPlan p = lg_plan(m, n, k, r);
  uint8_t* ws = reinterpret_cast<uint8_t*>(workspace);
  uint16_t* bt = reinterpret_cast<uint16_t*>(ws + p.o_bt);
  float* tp = reinterpret_cast<float*>(ws + p.o_tp);
  uint16_t* th = reinterpret_cast<uint16_t*>(ws + p.o_th);
  uint16_t* tl = reinterpret_cast<uint16_t*>(ws + p.o_tl);
  float* up = reinterpret_cast<float*>(ws + p.o_up);
  uint16_t* uh = reinterpret_cast<uint16_t*>(ws + p.o_uh);
  uint16_t* ul = reinterpret_cast<uint16_t*>(ws + p.o_ul);
  float* bp = reinterpret_cast<float*>(ws + p.o_bp);
  float* ap = reinterpret_cast<float*>(ws + p.o_ap);
  const uint16_t* yy = reinterpret_cast<const uint16_t*>(dy);
  const uint16_t* xx = reinterpret_cast<const uint16_t*>(x);
  const uint16_t* aa = reinterpret_cast<const uint16_t*>(la);
  const uint16_t* bb = reinterpret_cast<const uint16_t*>(lb);
  const unsigned mb = (unsigned)((m + 63) / 64);
  const bool rows = m > 0;                          // m == 0: every gradient is zero (the reductions write it)
  hipError_t e;
  // B^T
  if (n > 0) {
    hipLaunchKernelGGL(lg_transpose_kernel, dim3((unsigned)((n * r + 255) / 256)), dim3(256), 0, stream, bb, n, r, bt);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // t = x A^T -> (hi, lo)^T
  if (k > 0 && rows) {
    hipLaunchKernelGGL(lg_row_kernel, dim3(mb, (unsigned)p.st_), dim3(256), 0, stream, xx, m, k, aa, r, p.cst, tp);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if ((e = lg_reduce(tp, k > 0 && rows ? p.st_ : 0, m, r, 0, nullptr, th, tl, p.Mp, stream)) != hipSuccess) return e;
  // u = dY B -> fp32 (m, r) and (hi, lo)^T
  if (n > 0 && rows) {
    hipLaunchKernelGGL(lg_row_kernel, dim3(mb, (unsigned)p.su), dim3(256), 0, stream, yy, m, n, bt, r, p.csu, up);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if ((e = lg_reduce(up, n > 0 && rows ? p.su : 0, m, r, 1, u_out, uh, ul, p.Mp, stream)) != hipSuccess) return e;
  // dB = dY^T t
  if (grad_b && n > 0) {
    if (rows) {
      hipLaunchKernelGGL(lg_col_kernel, dim3((unsigned)((n + LG_CT - 1) / LG_CT), (unsigned)p.sb), dim3(256), 0,
                         stream, yy, m, n, th, tl, p.Mp, r, p.msb, bp);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if ((e = lg_reduce(bp, rows ? p.sb : 0, n, r, 2, grad_b, nullptr, nullptr, 0, stream)) != hipSuccess) return e;
  }
  // dA = u^T x, written (r, k)
  if (grad_a && k > 0) {
    if (rows) {
      hipLaunchKernelGGL(lg_col_kernel, dim3((unsigned)((k + LG_CT - 1) / LG_CT), (unsigned)p.sa), dim3(256), 0,
                         stream, xx, m, k, uh, ul, p.Mp, r, p.msa, ap);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if ((e = lg_reduce(ap, rows ? p.sa : 0, k, r, 3, grad_a, nullptr, nullptr, 0, stream)) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace fp4w
