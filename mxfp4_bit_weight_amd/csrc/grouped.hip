// grouped.hip -- the W4A16 product over the experts of a mixture of experts.
//
// QATFactory supports dense and mixture-of-experts models, and the Nemotron
// base model the QAD page starts from is a 30B-A3B MoE (QATFactory page, section
// on how training repeats the engine's arithmetic; Nemotron 3.5 Lightning page,
// section 02).  Routed rows are sorted by expert; expert e owns rows
// [offsets[e], offsets[e+1]) and row q reads token x[row_index[q]].
//
// K up to 4096 (every shape of the pages' MoE model) runs on the x-in-registers
// kernel of decode_xs.hip, a workgroup per (expert, run of weight tiles).
// Otherwise one workgroup per (expert, 16-row weight tile) runs the decode tile
// of skinny.hpp over the whole K for each chunk of up to 16 of its routed rows.
// The routing never leaves the device: a workgroup whose expert received no
// rows exits at once, and the number of m-groups is chosen per chunk (uniform
// branch).  Rows with a token index outside [0, num_tokens) are written as NaN.
#include "fp4w_device.hpp"
#include "fp4w_internal.hpp"
#include "skinny.hpp"

namespace fp4w {

template <int FMT, int MG>
__device__ __forceinline__ void grouped_chunk(const uint16_t* __restrict__ x, int64_t K, const uint8_t* codes_row,
                                              const uint8_t* scales_row, const int32_t* __restrict__ row_index,
                                              int64_t q0, int mc, int64_t num_tokens, int nsteps, float* red,
                                              float* fin) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4;
  const uint16_t* xrow[MG];
#pragma unroll
  for (int mg = 0; mg < MG; mg++) {
    const int m = a_operand_row<FMT>(lane, mg);
    xrow[mg] = nullptr;
    if (m >= 0 && m < mc) {
      const int64_t tok = row_index[q0 + m];
      if (tok >= 0 && tok < num_tokens) xrow[mg] = x + tok * K;
    }
  }
  SkinnyTileResult res;
  skinny_tile<FMT, MG, (MG == 1 ? 4 : (MG == 2 ? 2 : 1))>(codes_row, scales_row, xrow, K, 0, nsteps, wave, g, res);
  skinny_reduce<FMT, MG>(res, red, fin, mc);
}

template <int FMT>
__global__ __launch_bounds__(SK_THREADS) void grouped_skinny_kernel(
    const uint16_t* __restrict__ x, int64_t num_tokens, const int32_t* __restrict__ row_index,
    const int32_t* __restrict__ offsets, int64_t num_experts, int64_t total_rows, int64_t N, int64_t K,
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales, const float* __restrict__ tscales,
    uint16_t* __restrict__ y) {
  __shared__ float red[SK_WAVES * 16 * 64];
  __shared__ float fin[16 * 16];
  const int64_t tiles = (N + SK_TILE_N - 1) / SK_TILE_N;
  const int64_t e = blockIdx.x / tiles, tile = blockIdx.x % tiles;
  int64_t q_begin = offsets[e], q_end = offsets[e + 1];
  if (q_begin < 0) q_begin = 0;
  if (q_end > total_rows) q_end = total_rows;
  if (q_end <= q_begin) return;                        // expert received no rows
  const int lane = threadIdx.x & 63;
  const int64_t blk = (FMT == FMT_NVFP4) ? 16 : 32;
  const int64_t row = tile * SK_TILE_N + (lane & 15);
  const uint8_t* codes_e = codes + e * N * (K / 2);
  const uint8_t* scales_e = scales + e * N * (K / blk);
  const uint8_t* codes_row = row < N ? codes_e + row * (K / 2) : nullptr;
  const uint8_t* scales_row = row < N ? scales_e + row * (K / blk) : nullptr;
  const int nsteps = (int)((K + SK_STEP_K - 1) / SK_STEP_K);
  const float st = (FMT == FMT_NVFP4) ? tscales[e] : 1.0f;
  for (int64_t q0 = q_begin; q0 < q_end; q0 += 16) {
    const int mc = (int)(q_end - q0 < 16 ? q_end - q0 : 16);
    if (FMT == FMT_MXFP4) {
      grouped_chunk<FMT, 1>(x, K, codes_row, scales_row, row_index, q0, mc, num_tokens, nsteps, red, fin);
    } else {
      switch ((mc + 3) / 4) {
        case 1: grouped_chunk<FMT, 1>(x, K, codes_row, scales_row, row_index, q0, mc, num_tokens, nsteps, red, fin); break;
        case 2: grouped_chunk<FMT, 2>(x, K, codes_row, scales_row, row_index, q0, mc, num_tokens, nsteps, red, fin); break;
        case 3: grouped_chunk<FMT, 3>(x, K, codes_row, scales_row, row_index, q0, mc, num_tokens, nsteps, red, fin); break;
        default: grouped_chunk<FMT, 4>(x, K, codes_row, scales_row, row_index, q0, mc, num_tokens, nsteps, red, fin); break;
      }
    }
    const int tid = threadIdx.x, m = tid >> 4, nn = tid & 15;
    const int64_t orow = tile * SK_TILE_N + nn;
    if (m < mc && orow < N) {
      const int64_t tok = row_index[q0 + m];
      const bool ok = tok >= 0 && tok < num_tokens;
      const uint32_t o = ok ? f32_to_bf16_rne(st * fin[m * 16 + nn]) : 0x7FC0u;
      y[(q0 + m) * N + orow] = (uint16_t)o;
    }
    __syncthreads();                                   // fin / red are reused by the next chunk
  }
}

hipError_t launch_grouped_linear(int fmt, const void* x, int64_t num_tokens, const int32_t* row_index,
                                 const int32_t* expert_offsets, int64_t num_experts, int64_t total_rows,
                                 int64_t n, int64_t k, const uint8_t* codes, const uint8_t* scales,
                                 const float* tensor_scales, void* y, hipStream_t stream) {
  if (num_experts == 0 || total_rows == 0 || n == 0) return hipSuccess;
  if (grouped_xs_supports(num_tokens, n, k))
    return launch_grouped_xs(fmt, x, num_tokens, row_index, expert_offsets, num_experts, total_rows, n, k, codes,
                             scales, tensor_scales, y, stream);
  const int64_t tiles = (n + SK_TILE_N - 1) / SK_TILE_N;
  const dim3 grid((unsigned)(num_experts * tiles)), block(SK_THREADS);
  const uint16_t* xx = reinterpret_cast<const uint16_t*>(x);
  uint16_t* yy = reinterpret_cast<uint16_t*>(y);
  if (fmt == FMT_NVFP4)
    hipLaunchKernelGGL(grouped_skinny_kernel<FMT_NVFP4>, grid, block, 0, stream, xx, num_tokens, row_index,
                       expert_offsets, num_experts, total_rows, n, k, codes, scales, tensor_scales, yy);
  else
    hipLaunchKernelGGL(grouped_skinny_kernel<FMT_MXFP4>, grid, block, 0, stream, xx, num_tokens, row_index,
                       expert_offsets, num_experts, total_rows, n, k, codes, scales, tensor_scales, yy);
  return hipGetLastError();
}

}  // namespace fp4w
