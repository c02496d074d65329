// linear.hip -- y = x deq(W)^T + (x A^T) B^T on gfx950 (W4A16 with a parallel LoRA).
//
// The pages: weight-only NVFP4 with a LoRA adapter in parallel to the frozen
// base, as in QLoRA (tggo.me/sberlogasci/42740, section "Metod"); rollouts are
// memory-bound (same post, "Eksperimenty"); the product runs on 16-bit values
// (QATFactory page, section on how training repeats the engine's arithmetic).
//
// Launches per call (plan_linear picks the path):
//   m <= 2 (m <= 4 on small matrices): decode_f8f4_kernel (decode.hip; forms
//                t = x A^T itself)
//   other m <= 16: decode_xs_kernel (decode_xs.hip; forms t itself)
//   m > 16:      lora_down_kernel, then gemm_w4_kernel (gemm.hip: bf16 MFMA GEMM
//                with W decoded in registers; K a multiple of 128, x and the
//                codes below 2 GiB, scales 16-byte aligned) or else
//                linear_gemm_kernel (each weight tile dequantized once into LDS)
//   shapes the decode kernels do not take: lora_down_kernel, then
//                linear_decode_kernel (skinny.hpp)
// lora_down_kernel: t = x A^T (fp32, M x r), split over K, ordered sum.
// Split-K partial sums are combined by the last workgroup to arrive, in a fixed
// order, so results do not depend on scheduling.  Its arrival counters live in
// the caller's workspace and are returned to zero by that last workgroup.
#include "fp4w_device.hpp"
#include "fp4w_internal.hpp"
#include "gemm_common.hpp"
#include "skinny.hpp"
#include "sync.hpp"

namespace fp4w {

// ---------------------------------------------------------------------------------
// LoRA down-projection t = x A^T.  Workgroup (m-tile of 16 rows, K slice p);
// its 4 waves interleave 32-wide K steps; v_mfma_f32_16x16x32_bf16 with x as A
// (rows m) and the LoRA A rows as B (columns j), RB = ceil(r/16) column tiles.
// ---------------------------------------------------------------------------------
constexpr int LD_MAX_RB = 4;

__global__ __launch_bounds__(256) void lora_down_kernel(const uint16_t* __restrict__ x, int64_t M, int64_t K,
                                                        const uint16_t* __restrict__ a, int r, int P,
                                                        int steps_per_part, float* __restrict__ tp,
                                                        float* __restrict__ t, uint32_t* __restrict__ cnt) {
  __shared__ float red[4 * LD_MAX_RB * 4 * 64];
  __shared__ int flag;
  const int mt = blockIdx.x / P, p = blockIdx.x % P;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, li = lane & 15, g = lane >> 4;
  const int RB = (r + 15) / 16;
  const int64_t m = (int64_t)mt * 16 + li;
  const int nsteps = (int)((K + 31) / 32);
  const int s0 = p * steps_per_part, s1 = min(nsteps, s0 + steps_per_part);
  f32x4_t acc[LD_MAX_RB];
#pragma unroll
  for (int b = 0; b < LD_MAX_RB; b++) acc[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int step = s0 + wave; step < s1; step += 4) {
    const int64_t k = (int64_t)step * 32 + 8 * g;
    u32x4_t xa = {0u, 0u, 0u, 0u};
    if (m < M && k < K) xa = load16(x + m * K + k);
#pragma unroll
    for (int b = 0; b < LD_MAX_RB; b++) {
      if (b < RB) {
        const int j = b * 16 + li;
        u32x4_t av = {0u, 0u, 0u, 0u};
        if (j < r && k < K) av = load16(a + (int64_t)j * K + k);
        acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xa), as_bf16x8(av), acc[b], 0, 0, 0);
      }
    }
  }
  // reduce the 4 waves: D row = 4 g + i (m), column li (j within the tile)
#pragma unroll
  for (int b = 0; b < LD_MAX_RB; b++)
#pragma unroll
    for (int i = 0; i < 4; i++) red[((wave * LD_MAX_RB + b) * 4 + i) * 64 + lane] = acc[b][i];
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int b = 0; b < LD_MAX_RB; b++) {
      if (b < RB) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
          float s = 0.f;
#pragma unroll
          for (int w = 0; w < 4; w++) s += red[((w * LD_MAX_RB + b) * 4 + i) * 64 + lane];
          const int64_t mm = (int64_t)mt * 16 + 4 * g + i;
          const int j = b * 16 + li;
          if (mm < M && j < r) {
            if (P == 1) t[mm * r + j] = s;
            else store_agent(&tp[((int64_t)p * M + mm) * r + j], s);
          }
        }
      }
    }
  }
  if (P == 1) return;
  if (!arrive_last(&cnt[mt], (uint32_t)P, &flag)) return;
  for (int e = threadIdx.x; e < 16 * r; e += 256) {
    const int64_t mm = (int64_t)mt * 16 + e / r;
    const int j = e % r;
    if (mm >= M) continue;
    float s = 0.f;
    for (int q = 0; q < P; q++) s += load_agent(&tp[((int64_t)q * M + mm) * r + j]);
    t[mm * r + j] = s;
  }
}


// ---------------------------------------------------------------------------------
// Decode-shaped linear (m <= 16).
// ---------------------------------------------------------------------------------
__device__ __forceinline__ float lora_term(const float* __restrict__ t, const uint16_t* __restrict__ lb, int r,
                                           int64_t m, int64_t row) {
  float s = 0.f;
  for (int j = 0; j < r; j++) s = __builtin_fmaf(t[m * r + j], __uint_as_float((uint32_t)lb[row * r + j] << 16), s);
  return s;
}

// One wave per (16-row weight tile, K split).  WPW waves per workgroup share the
// split: its x rows and the scale bytes of the workgroup's tile rows are staged
// in LDS.  The staging loads are issued first, then each wave's ring prologue,
// so the memory latencies overlap; the LDS writes follow.  With one split the
// wave writes y; with several, the last wave of a tile to arrive adds the
// partials in split order and writes y.
//   scales16: scale rows of every split start 16-byte aligned (16-byte staging)
constexpr int DECODE_STAGE_CHUNK = 8;     // 16-byte staging units per thread issued before the ring

template <int FMT, int MG, int DEPTH, int WPW>
__global__ __launch_bounds__(64 * WPW) void linear_decode_kernel(
    const uint16_t* __restrict__ x, int M, int64_t K, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ scales, const float* __restrict__ tensor_scale, int64_t N,
    const float* __restrict__ t, const uint16_t* __restrict__ lora_b, int r, uint16_t* __restrict__ y,
    float* __restrict__ part, uint32_t* __restrict__ cnt, int S, int steps_per_split, int nsteps_total,
    int ntiles, int scales16) {
  extern __shared__ __attribute__((aligned(16))) uint16_t xs[];     // see DecodeLds
  constexpr int NT = 64 * WPW;
  constexpr int BLK = DecodeLds<FMT>::BLK;
  const int s = blockIdx.x % S, tg = blockIdx.x / S;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int kslice = steps_per_split * SK_STEP_K;
  const int step0 = s * steps_per_split;
  const int nsteps = min(steps_per_split, nsteps_total - step0);
  const int64_t k0 = (int64_t)step0 * SK_STEP_K;
  const int srow = DecodeLds<FMT>::srow_bytes(kslice);
  uint8_t* lds_s = reinterpret_cast<uint8_t*>(xs + DECODE_XS_ZERO + M * kslice);
  const int64_t krem = K - k0;
  const int svalid = krem <= 0 ? 0 : (int)((krem < kslice ? krem : kslice) / BLK);   // scale bytes per row here
  const int64_t srow_g = K / BLK;                                                       // global scale row length
  const int64_t row_base = (int64_t)tg * WPW * SK_TILE_N;

  // staging units of 16 bytes: x first, then (if aligned) whole 16-byte scale units
  const int ux = M * kslice / 8;
  const int us_row = svalid / 16;                     // full 16-byte units per scale row
  const int us = scales16 ? WPW * SK_TILE_N * us_row : 0;
  const int utotal = ux + us;
  auto unit_src = [&](int u, bool& ok) -> const void* {
    if (u < ux) {
      const int m = (8 * u) / kslice, kk = 8 * u - m * kslice;
      ok = k0 + kk < K;
      return x + (int64_t)m * K + (ok ? k0 + kk : 0);
    }
    const int v = u - ux, rw = v / (us_row > 0 ? us_row : 1), q = v - rw * us_row;
    int64_t grow = row_base + rw;
    ok = grow < N;
    grow = grow < N ? grow : N - 1;
    return scales + grow * srow_g + k0 / BLK + 16 * q;
  };
  auto unit_dst = [&](int u) -> u32x4_t* {
    if (u < ux) return reinterpret_cast<u32x4_t*>(xs + DECODE_XS_ZERO + 8 * u);
    const int v = u - ux, rw = v / (us_row > 0 ? us_row : 1), q = v - rw * us_row;
    return reinterpret_cast<u32x4_t*>(lds_s + rw * srow + 16 * q);
  };
  u32x4_t stage[DECODE_STAGE_CHUNK];
  bool stage_ok[DECODE_STAGE_CHUNK];
#pragma unroll
  for (int c = 0; c < DECODE_STAGE_CHUNK; c++) {
    const int u = tid + c * NT;
    bool ok = false;
    const void* src = unit_src(u < utotal ? u : 0, ok);
    stage[c] = load16(src);
    stage_ok[c] = ok && u < utotal;
  }

  const int tile_raw = tg * WPW + wave;
  const bool has_tile = tile_raw < ntiles;
  const int tile = has_tile ? tile_raw : ntiles - 1;
  const int g = lane >> 4, n = lane & 15;
  const int64_t row = (int64_t)tile * SK_TILE_N + n;
  const int64_t rrow = row < N ? row : N - 1;          // rows past N read row N - 1 (never stored)
  DecodeRing<FMT, MG, DEPTH> ring;
  ring.prologue(codes + rrow * (K / 2), k0, K, nsteps, lane);

  if (tid < DECODE_XS_ZERO / 8) *reinterpret_cast<u32x4_t*>(xs + 8 * tid) = (u32x4_t){0u, 0u, 0u, 0u};
#pragma unroll
  for (int c = 0; c < DECODE_STAGE_CHUNK; c++) {
    const int u = tid + c * NT;
    if (u < utotal) *unit_dst(u) = stage_ok[c] ? stage[c] : (u32x4_t){0u, 0u, 0u, 0u};
  }
  for (int u = tid + DECODE_STAGE_CHUNK * NT; u < utotal; u += NT) {
    bool ok;
    const void* src = unit_src(u, ok);
    const u32x4_t v = load16(src);
    *unit_dst(u) = ok ? v : (u32x4_t){0u, 0u, 0u, 0u};
  }
  // remaining scale bytes (unaligned rows, a partial last unit, padding): byte by byte
  {
    const int first = scales16 ? 16 * us_row : 0;
    const int per_row = srow - first;
    for (int idx = tid; idx < WPW * SK_TILE_N * per_row; idx += NT) {
      const int rw = idx / per_row, b = first + (idx - rw * per_row);
      const int64_t grow = row_base + rw;
      uint8_t val = 0;
      if (b < svalid && grow < N) val = scales[grow * srow_g + k0 / BLK + b];
      lds_s[rw * srow + b] = val;
    }
  }
  __syncthreads();
  if (!has_tile) return;
  float v[MG][4];
  ring.run(xs, kslice, lds_s + (wave * SK_TILE_N + n) * srow, M, lane, v);

  // the (m, n) outputs this lane owns (see DecodeRing)
  const float st = (FMT == FMT_NVFP4) ? *tensor_scale : 1.0f;
  auto owns = [&](int mg, int e, int& m) -> bool {
    m = (FMT == FMT_NVFP4) ? 4 * mg + e : 4 * g + e;
    const bool lane_ok = (FMT == FMT_NVFP4) ? (g == 0) : (mg == 0);
    return lane_ok && m < M && row < N;
  };
  if (S > 1) {
#pragma unroll
    for (int mg = 0; mg < MG; mg++)
#pragma unroll
      for (int e = 0; e < 4; e++) {
        int m;
        if (owns(mg, e, m)) store_agent(&part[((int64_t)s * N + row) * M + m], v[mg][e]);
      }
    if (!wave_arrive_last(&cnt[tile], (uint32_t)S, lane)) return;
#pragma unroll
    for (int mg = 0; mg < MG; mg++)
#pragma unroll
      for (int e = 0; e < 4; e++) {
        int m;
        if (owns(mg, e, m)) {
          float sum = 0.f;
          for (int q = 0; q < S; q++) sum += load_agent(&part[((int64_t)q * N + row) * M + m]);
          v[mg][e] = sum;
        }
      }
  }
#pragma unroll
  for (int mg = 0; mg < MG; mg++)
#pragma unroll
    for (int e = 0; e < 4; e++) {
      int m;
      if (owns(mg, e, m)) {
        float o = st * v[mg][e];
        if (t) o += lora_term(t, lora_b, r, m, row);
        y[(int64_t)m * N + row] = (uint16_t)f32_to_bf16_rne(o);
      }
    }
}

// ---------------------------------------------------------------------------------
// GEMM (m > 16): 256 x 256 output tile per workgroup, K tile 64, 8 waves in a
// 4 x 2 grid of 64 x 128, v_mfma_f32_16x16x32_bf16; two waves per SIMD, so one
// wave's LDS reads, loads and dequantization run under the other's MFMAs.  Each
// K tile of x is copied to LDS, each K tile of W is loaded as codes and
// dequantized once into LDS as exact bf16 (e2m1 * dec(sb) has at most 6
// significant bits; the tensor scale is applied at the end).  The next tile's
// global loads (buffer loads: chunks outside the matrices read zeros) are in
// flight while the current one is used.
// ---------------------------------------------------------------------------------
constexpr int G_BM = 256, G_BN = 256, G_BK = 64;
constexpr int G_LDA = G_BK + 8;   // bf16 elements per LDS row (16 bytes of padding)
constexpr int G_THREADS = 512;

template <int FMT>
struct GemmStage {
  u32x4_t xv[4];     // 4 x 16 bytes of x
  u32x4_t cv;        // 16 bytes of codes (32 codes of one row)
  uint32_t sv;       // their scale bytes (NVFP4: two, MXFP4: one)
};

// BUF: buffer loads through descriptors over x, the codes and the scales; a
// chunk outside the matrices gets an offset past its buffer and reads zeros
// without touching memory, so no select on the loaded data follows the load
// (such a select would make the wave wait for the data at once, not when the
// stage is stored a K tile later).  Needs x and the codes below 2 GiB.
// Otherwise plain loads of a clamped address, zeroed after the load.
template <int FMT, bool BUF>
__device__ __forceinline__ void gemm_load(GemmStage<FMT>& st, const uint16_t* __restrict__ x, int64_t M,
                                          int64_t K, const uint8_t* __restrict__ codes,
                                          const uint8_t* __restrict__ scales, int64_t N, int64_t m0, int64_t n0,
                                          int64_t k0, __amdgpu_buffer_rsrc_t xr, __amdgpu_buffer_rsrc_t cr,
                                          __amdgpu_buffer_rsrc_t sr) {
  const int tid = threadIdx.x;
  // x: 256 rows x 64 bf16 = 2048 chunks of 16 B; thread handles rows tid/8 + 64 i, chunk tid % 8
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int64_t mr = m0 + (tid >> 3) + 64 * i;
    const int64_t k = k0 + 8 * (tid & 7);
    const bool ok = mr < M && k < K;
    if (BUF) {                                   // 32-bit offsets: x below 2 GiB
      const uint32_t xo = ((uint32_t)mr * (uint32_t)K + (uint32_t)k) * 2u;
      st.xv[i] = buffer_load16(xr, ok ? xo : kBufferOob);
    } else {
      st.xv[i] = load16(x + (ok ? mr * K + k : 0));
      if (!ok) st.xv[i] = (u32x4_t){0u, 0u, 0u, 0u};
    }
  }
  // W: 256 rows x 64 codes = 512 chunks of 32 codes; thread handles row tid/2, half tid % 2
  const int64_t blk = (FMT == FMT_NVFP4) ? 16 : 32;
  const int64_t nr = n0 + (tid >> 1);
  const int64_t k = k0 + 32 * (tid & 1);
  const bool ok = nr < N && k < K;
  if (BUF) {                                     // 32-bit offsets: the codes below 2 GiB
    const uint32_t co = (uint32_t)nr * (uint32_t)(K >> 1) + ((uint32_t)k >> 1);
    st.cv = buffer_load16(cr, ok ? co : kBufferOob);
    const uint32_t so0 = (uint32_t)nr * (uint32_t)(K / blk) + (uint32_t)k / (uint32_t)blk;
    const uint32_t so = ok ? so0 : kBufferOob;
    if (FMT == FMT_NVFP4) st.sv = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(sr, so, 0, 0);
    else st.sv = (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(sr, so, 0, 0);
  } else {
    const int64_t nrc = ok ? nr : 0, kc = ok ? k : 0;
    st.cv = load16(codes + nrc * (K / 2) + kc / 2);
    if (FMT == FMT_NVFP4) st.sv = *reinterpret_cast<const uint16_t*>(scales + nrc * (K / blk) + kc / blk);
    else st.sv = scales[nrc * (K / blk) + kc / blk];
    if (!ok) { st.cv = (u32x4_t){0u, 0u, 0u, 0u}; st.sv = 0u; }
  }
}

template <int FMT>
__device__ __forceinline__ void gemm_store_lds(const GemmStage<FMT>& st, uint16_t* sa, uint16_t* sb) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int rr = (tid >> 3) + 64 * i, c = 8 * (tid & 7);
    *reinterpret_cast<u32x4_t*>(sa + rr * G_LDA + c) = st.xv[i];
  }
  const int rr = tid >> 1, c = 32 * (tid & 1);
  uint16_t* const dst = sb + rr * G_LDA + c;
  if (FMT == FMT_NVFP4) {
    const float d0 = e4m3_to_f32(st.sv & 0xFFu), d1 = e4m3_to_f32((st.sv >> 8) & 0xFFu);
    // one 16-byte piece at a time (few live registers: two stages of loads are in flight)
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const float d = q < 2 ? d0 : d1;
      const uint32_t dw = st.cv[q];
      const f32x2_t a0 = fp4x2_to_f32x2<0>(dw, 1.0f), a1 = fp4x2_to_f32x2<1>(dw, 1.0f);
      const f32x2_t a2 = fp4x2_to_f32x2<2>(dw, 1.0f), a3 = fp4x2_to_f32x2<3>(dw, 1.0f);
      // e2m1 * dec(sb) has at most 6 significant bits: exact in fp32 and in bf16
      u32x4_t o;
      o.x = (__float_as_uint(a0.x * d) >> 16) | (__float_as_uint(a0.y * d) & 0xFFFF0000u);
      o.y = (__float_as_uint(a1.x * d) >> 16) | (__float_as_uint(a1.y * d) & 0xFFFF0000u);
      o.z = (__float_as_uint(a2.x * d) >> 16) | (__float_as_uint(a2.y * d) & 0xFFFF0000u);
      o.w = (__float_as_uint(a3.x * d) >> 16) | (__float_as_uint(a3.y * d) & 0xFFFF0000u);
      *reinterpret_cast<u32x4_t*>(dst + 8 * q) = o;
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
    const float sc = e8m0_scale_operand(st.sv);
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const uint32_t dw = st.cv[q];
      u32x4_t o;
      o.x = fp4x2_to_bf16x2_scaled<0>(dw, sc);
      o.y = fp4x2_to_bf16x2_scaled<1>(dw, sc);
      o.z = fp4x2_to_bf16x2_scaled<2>(dw, sc);
      o.w = fp4x2_to_bf16x2_scaled<3>(dw, sc);
      *reinterpret_cast<u32x4_t*>(dst + 8 * q) = o;
    }
  }
}

template <int FMT, bool BUF>
__global__ __launch_bounds__(G_THREADS, 2) void linear_gemm_kernel(
    const uint16_t* __restrict__ x, int64_t M, int64_t K, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ scales, const float* __restrict__ tensor_scale, int64_t N,
    const float* __restrict__ t, const uint16_t* __restrict__ lora_b, int r, uint16_t* __restrict__ y) {
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  // LDS: [A stage 0][A stage 1][B stage 0][B stage 1]
  uint16_t* const sA0 = smem;
  uint16_t* const sB0 = smem + 2 * G_BM * G_LDA;
  const int tiles_n = (int)((N + G_BN - 1) / G_BN);
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
  const int64_t m0 = (int64_t)tm * G_BM, n0 = (int64_t)tn * G_BN;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, wm = wave >> 1, wn = wave & 1;
  const int li = lane & 15, g = lane >> 4;
  constexpr int TI = 4, TJ = 8;                  // 16 x 16 sub-tiles of the wave's 64 x 128

  f32x4_t acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; i++)
#pragma unroll
    for (int j = 0; j < TJ; j++) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nk = (int)((K + G_BK - 1) / G_BK);
  const int64_t blk = (FMT == FMT_NVFP4) ? 16 : 32;
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, BUF ? (uint32_t)(M * K * 2) : 0u);
  const __amdgpu_buffer_rsrc_t cr = make_rsrc(codes, BUF ? (uint32_t)(N * (K / 2)) : 0u);
  const __amdgpu_buffer_rsrc_t sr = make_rsrc(scales, BUF ? (uint32_t)(N * (K / blk)) : 0u);
  // The barrier waits for LDS work only; the global loads of the next tile stay
  // in flight across it.
  auto lds_barrier = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0xC07F);          // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };
  auto mfma_tile = [&](int cur) __attribute__((always_inline)) {
    const uint16_t* a = sA0 + cur * (G_BM * G_LDA);
    const uint16_t* b = sB0 + cur * (G_BN * G_LDA);
#pragma unroll
    for (int kk = 0; kk < G_BK / 32; kk++) {
      bf16x8_t af[TI], bfr[TJ];
#pragma unroll
      for (int i = 0; i < TI; i++)
        af[i] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(a + (wm * 64 + i * 16 + li) * G_LDA + kk * 32 + 8 * g));
#pragma unroll
      for (int j = 0; j < TJ; j++)
        bfr[j] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(b + (wn * 128 + j * 16 + li) * G_LDA + kk * 32 + 8 * g));
#pragma unroll
      for (int i = 0; i < TI; i++)
#pragma unroll
        for (int j = 0; j < TJ; j++) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  };
  // One register stage holds the next K tile.  During the second half of a
  // tile's MFMAs the stage is dequantized and stored into the other LDS buffer,
  // one piece after each MFMA, then refilled with the tile after that, so its
  // loads run under the next tile's MFMAs and the barrier finds the stores done.
  GemmStage<FMT> sg;
  gemm_load<FMT, BUF>(sg, x, M, K, codes, scales, N, m0, n0, 0, xr, cr, sr);
  gemm_store_lds<FMT>(sg, sA0, sB0);
  gemm_load<FMT, BUF>(sg, x, M, K, codes, scales, N, m0, n0, (int64_t)G_BK, xr, cr, sr);
  lds_barrier();
  const int srow = threadIdx.x >> 1, scol = 32 * (threadIdx.x & 1);
  auto step = [&](int cur, int64_t kload) __attribute__((always_inline)) {
    const uint16_t* a = sA0 + cur * (G_BM * G_LDA);
    const uint16_t* b = sB0 + cur * (G_BN * G_LDA);
    uint16_t* wa = sA0 + (cur ^ 1) * (G_BM * G_LDA);
    uint16_t* wb = sB0 + (cur ^ 1) * (G_BN * G_LDA) + srow * G_LDA + scol;
    u32x4_t o = {0u, 0u, 0u, 0u};
    float d0 = 0.f, d1 = 0.f;
#pragma unroll
    for (int kk = 0; kk < G_BK / 32; kk++) {
      bf16x8_t af[TI], bfr[TJ];
#pragma unroll
      for (int i = 0; i < TI; i++)
        af[i] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(a + (wm * 64 + i * 16 + li) * G_LDA + kk * 32 + 8 * g));
#pragma unroll
      for (int j = 0; j < TJ; j++)
        bfr[j] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(b + (wn * 128 + j * 16 + li) * G_LDA + kk * 32 + 8 * g));
      if (kk == 1) {
        if (FMT == FMT_NVFP4) { d0 = e4m3_to_f32(sg.sv & 0xFFu); d1 = e4m3_to_f32((sg.sv >> 8) & 0xFFu); }
        else d0 = e8m0_scale_operand(sg.sv);
      }
#pragma unroll
      for (int i = 0; i < TI; i++)
#pragma unroll
        for (int j = 0; j < TJ; j++) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
          const int slot = i * TJ + j;
          if (kk == 1) {
            if (slot < 4) {
              const int rr = (threadIdx.x >> 3) + 64 * slot, c = 8 * (threadIdx.x & 7);
              *reinterpret_cast<u32x4_t*>(wa + rr * G_LDA + c) = sg.xv[slot];
            } else if (slot < 20) {
              const int di = slot - 4, q = di >> 2, h = di & 3;
              const uint32_t dw = sg.cv[q];
              uint32_t v;
              if (FMT == FMT_NVFP4) {
                const float d = q < 2 ? d0 : d1;
                const f32x2_t f = h == 0 ? fp4x2_to_f32x2<0>(dw, 1.0f) : h == 1 ? fp4x2_to_f32x2<1>(dw, 1.0f)
                                : h == 2 ? fp4x2_to_f32x2<2>(dw, 1.0f) : fp4x2_to_f32x2<3>(dw, 1.0f);
                v = (__float_as_uint(f.x * d) >> 16) | (__float_as_uint(f.y * d) & 0xFFFF0000u);
              } else {
                v = h == 0 ? fp4x2_to_bf16x2_scaled<0>(dw, d0) : h == 1 ? fp4x2_to_bf16x2_scaled<1>(dw, d0)
                  : h == 2 ? fp4x2_to_bf16x2_scaled<2>(dw, d0) : fp4x2_to_bf16x2_scaled<3>(dw, d0);
              }
              o[h] = v;
              if (h == 3) *reinterpret_cast<u32x4_t*>(wb + 8 * q) = o;
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
    }
    gemm_load<FMT, BUF>(sg, x, M, K, codes, scales, N, m0, n0, kload, xr, cr, sr);
  };
  // every step stores and loads: loads past K read zeros, and the last steps'
  // stores go to a buffer no later step reads
  for (int kt = 0; kt < nk; kt += 2) {
    step(0, (int64_t)(kt + 2) * G_BK);
    lds_barrier();
    if (kt + 1 >= nk) break;
    step(1, (int64_t)(kt + 3) * G_BK);
    lds_barrier();
  }

  // epilogue: y = s_t * acc + LoRA, with the LoRA as extra MFMA steps over
  // K' = [t_hi | t_lo] (t split into two bf16 parts) against [B | B].
  // (s_t is applied in the first LoRA step, or at the store without LoRA: a
  // separate pass over the accumulators costs registers two load stages need)
  const float st = (FMT == FMT_NVFP4) ? *tensor_scale : 1.0f;
  if (t) {
    const int rpad = ((r + 15) / 16) * 16;
    for (int jb = 0; jb < rpad; jb += 16) {
      // K' slice: 32 entries = t_hi[jb..jb+16) then t_lo[jb..jb+16); lane group g
      // covers entries 8g..8g+7 -> part (g >> 1) of LoRA index jb + 8 (g & 1) + e
      const int jj = jb + 8 * (g & 1);
      const bool lo_part = (g >> 1) != 0;
      bf16x8_t tf[TI], bfv[TJ];
#pragma unroll
      for (int i = 0; i < TI; i++) {
        const int64_t mr = m0 + wm * 64 + i * 16 + li;
        u32x4_t v = {0u, 0u, 0u, 0u};
        if (mr < M) {
          uint32_t h[8];
#pragma unroll
          for (int e = 0; e < 8; e++) {
            const int j = jj + e;
            const float tv = j < r ? t[mr * r + j] : 0.f;
            const uint32_t hi = f32_to_bf16_rne(tv);
            h[e] = lo_part ? f32_to_bf16_rne(tv - __uint_as_float(hi << 16)) : hi;
          }
          v.x = h[0] | (h[1] << 16); v.y = h[2] | (h[3] << 16);
          v.z = h[4] | (h[5] << 16); v.w = h[6] | (h[7] << 16);
        }
        tf[i] = as_bf16x8(v);
      }
#pragma unroll
      for (int j2 = 0; j2 < TJ; j2++) {
        const int64_t nr = n0 + wn * 128 + j2 * 16 + li;
        u32x4_t v = {0u, 0u, 0u, 0u};
        if (nr < N) {
          uint32_t h[8];
#pragma unroll
          for (int e = 0; e < 8; e++) {
            const int j = jj + e;
            h[e] = j < r ? lora_b[nr * r + j] : 0u;
          }
          v.x = h[0] | (h[1] << 16); v.y = h[2] | (h[3] << 16);
          v.z = h[4] | (h[5] << 16); v.w = h[6] | (h[7] << 16);
        }
        bfv[j2] = as_bf16x8(v);
      }
#pragma unroll
      for (int i = 0; i < TI; i++)
#pragma unroll
        for (int j2 = 0; j2 < TJ; j2++) {
          if (FMT == FMT_NVFP4 && jb == 0) {
#pragma unroll
            for (int e = 0; e < 4; e++) acc[i][j2][e] *= st;
          }
          acc[i][j2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(tf[i], bfv[j2], acc[i][j2], 0, 0, 0);
        }
    }
  }
  // store: lane holds rows 4 g + e, column li of each 16 x 16 sub-tile
#pragma unroll
  for (int i = 0; i < TI; i++)
#pragma unroll
    for (int j = 0; j < TJ; j++) {
      const int64_t nc = n0 + wn * 128 + j * 16 + li;
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const int64_t mr = m0 + wm * 64 + i * 16 + 4 * g + e;
        const float v = (FMT == FMT_NVFP4 && !t) ? acc[i][j][e] * st : acc[i][j][e];
        if (mr < M && nc < N) y[mr * N + nc] = (uint16_t)f32_to_bf16_rne(v);
      }
    }
}

// ---------------------------------------------------------------------------------
// Planning and launch.
// ---------------------------------------------------------------------------------
static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

static int lora_parts_for(int64_t m, int64_t k) {
  const int64_t steps = (k + 31) / 32;
  if ((m + 15) / 16 > kLoraSlots || m > 16) return 1;
  int64_t p = steps / 8;
  if (p < 1) p = 1;
  if (p > 64) p = 64;
  return (int)p;
}

// x rows of one split are staged in LDS: at most this many bytes per workgroup.
constexpr int64_t kDecodeLdsBytes = 32768;
// Aim for at least this many waves (one per tile and split) in the decode kernel.
constexpr int64_t kDecodeTargetWaves = 1024;

static int decode_splits_for(int64_t m, int64_t n, int64_t k) {
  const int64_t tiles = (n + SK_TILE_N - 1) / SK_TILE_N;
  const int64_t nsteps = (k + SK_STEP_K - 1) / SK_STEP_K;
  const int64_t max_steps = kDecodeLdsBytes / (2 * SK_STEP_K * (m > 0 ? m : 1) + 4 * SK_TILE_N * 8);  // LDS per split
  int64_t s_lds = (nsteps + max_steps - 1) / max_steps;
  int64_t s_par = (kDecodeTargetWaves + tiles - 1) / tiles;
  const int64_t max_par = nsteps / 2 > 0 ? nsteps / 2 : 1;            // keep >= 2 steps per wave
  if (s_par > max_par) s_par = max_par;
  int64_t s = s_lds > s_par ? s_lds : s_par;
  if (s > nsteps) s = nsteps;
  if (s < 1) s = 1;
  return (int)s;
}

// Decode-shaped calls (m <= 16) run on the block-scaled kernel when its cost per
// row of x is small against a launch (m <= 2, or m <= 4 on a matrix of at most
// 2^24 weights), else on the x-in-registers kernel.  Measured on MI355X for the
// Qwen-2.5-7B shapes in both formats, with and without LoRA: at m = 2 the
// block-scaled kernel is faster on every shape, at m = 4 only on 3584 x 3584,
// at m = 8 on none.
static bool decode_prefers_f8f4(int64_t m, int64_t n, int64_t k) {
  return m <= 2 || (m <= 4 && n * k <= ((int64_t)1 << 24));
}

LinearPlan plan_linear(int64_t m, int64_t n, int64_t k, int r) {
  LinearPlan p{};
  if (k == 0) {                                  // no products: y = 0, the counter area only
    p.path = 4;
    p.splits = 1;
    p.bytes = sizeof(uint32_t) * kCounterSlots;
    p.off_t = p.off_part = p.bytes;
    return p;
  }
  if (m > 16) p.path = 1;
  else if (m >= 2 && decode_xs_supports(m, n, k, r) && !decode_prefers_f8f4(m, n, k)) p.path = 3;
  else p.path = decode_f8f4_supports(FMT_NVFP4, m) ? 0 : 2;
  if (p.path == 3) {
    p.xs = plan_decode_xs(m, n, k, r);
    if (p.xs.splits > 1 && (p.xs.ntiles + 7) / 8 > kTileSlots) p.path = 1;     // counters would not fit
  }
  size_t part_floats = 0;
  if (p.path == 3) {
    p.splits = p.xs.splits;
    part_floats = (size_t)p.xs.splits * p.xs.ntiles * 16 * m;
  } else if (p.path == 0) {
    // one plan for both formats: the NVFP4 layout is never smaller
    p.dq = plan_decode_f8f4(FMT_NVFP4, m, n, k, r);
    p.splits = p.dq.splits;
    const int64_t tiles = (n + SK_TILE_N - 1) / SK_TILE_N;
    if (p.splits > 1 && tiles > kTileSlots) p.path = 1;                       // counters would not fit
    part_floats = (size_t)p.splits * tiles * SK_TILE_N * m;
  } else if (p.path == 2) {
    p.splits = decode_splits_for(m, n, k);
    if (p.splits > 1 && (n + SK_TILE_N - 1) / SK_TILE_N > kTileSlots) p.path = 1;
    part_floats = (size_t)p.splits * n * m;
  }
  if (p.path == 1) p.splits = 1;
  // LoRA down-projection: formed inside the decode kernels (paths 0 and 3, chunk
  // workgroups handing t over through the counter area); else by
  // lora_down_kernel (K slices, ordered sum) into t
  const bool lora_inside = p.path == 0 || p.path == 3;
  p.lora_parts = r <= 0 || lora_inside ? 0 : lora_parts_for(m, k);
  size_t off = 0;
  p.off_count = off;
  off += sizeof(uint32_t) * kCounterSlots;
  p.off_t = off;
  if (r > 0 && !lora_inside) {
    off += align256(sizeof(float) * (size_t)m * (size_t)r);                           // t
    if (p.lora_parts > 1) off += align256(sizeof(float) * (size_t)p.lora_parts * m * r);   // partials
  }
  p.off_part = off;
  if (p.splits > 1) off += align256(sizeof(float) * part_floats);
  p.bytes = off;
  return p;
}

// y = 0 for k == 0 (every output is an empty sum).
__global__ __launch_bounds__(256) void zero_bf16_kernel(uint16_t* __restrict__ y, int64_t elems) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < elems; i += (int64_t)gridDim.x * 256) y[i] = 0;
}

// Waves per workgroup of the decode kernel: 1 while the staged x slice is small
// (every wave independent), 4 when it is large enough that sharing it matters.
static int decode_wpw(int64_t m) { return m <= 4 ? 1 : 4; }

template <int FMT>
static hipError_t launch_decode(int mg, const void* x, int64_t m, int64_t k, const uint8_t* codes,
                                const uint8_t* scales, const float* ts, int64_t n, const float* t, const void* lb,
                                int r, void* y, float* part, uint32_t* cnt, int S, hipStream_t stream) {
  constexpr int BLK = DecodeLds<FMT>::BLK;
  const int ntiles = (int)((n + SK_TILE_N - 1) / SK_TILE_N);
  const int nsteps = (int)((k + SK_STEP_K - 1) / SK_STEP_K);
  // steps per split: a multiple of 4 when the split is real (16-byte aligned
  // scale slices for both formats); the split count can only shrink
  int sps = (nsteps + S - 1) / S;
  if (S > 1) {
    sps = (sps + 3) & ~3;
    S = (nsteps + sps - 1) / sps;
  }
  const int kslice = sps * SK_STEP_K;
  const int wpw = decode_wpw(m);
  const int groups = (ntiles + wpw - 1) / wpw;
  const size_t lds = DecodeLds<FMT>::bytes((int)m, kslice, wpw * SK_TILE_N);
  const int scales16 = ((reinterpret_cast<uintptr_t>(scales) & 15u) == 0 && (k / BLK) % 16 == 0 &&
                        (kslice / BLK) % 16 == 0) ? 1 : 0;
  const dim3 grid((unsigned)((int64_t)groups * S));
  const uint16_t* xx = reinterpret_cast<const uint16_t*>(x);
  const uint16_t* bb = reinterpret_cast<const uint16_t*>(lb);
  uint16_t* yy = reinterpret_cast<uint16_t*>(y);
#define FP4W_DECODE(MGv, WPWv)                                                                                   \
  hipLaunchKernelGGL((linear_decode_kernel<FMT, MGv, (MGv == 1 ? 8 : 4), WPWv>), grid, dim3(64 * WPWv), lds,     \
                     stream, xx, (int)m, k, codes, scales, ts, n, t, bb, r, yy, part, cnt, S, sps, nsteps, ntiles, \
                     scales16)
  if (FMT == FMT_MXFP4) {
    if (wpw == 1) FP4W_DECODE(1, 1); else FP4W_DECODE(1, 4);
  } else {
    switch (mg) {
      case 1: FP4W_DECODE(1, 1); break;
      case 2: FP4W_DECODE(2, 4); break;
      case 3: FP4W_DECODE(3, 4); break;
      default: FP4W_DECODE(4, 4); break;
    }
  }
#undef FP4W_DECODE
  return hipGetLastError();
}

hipError_t launch_linear(int fmt, const void* x, int64_t m, int64_t k, const uint8_t* codes,
                         const uint8_t* scales, const float* tensor_scale, int64_t n, const void* lora_a,
                         const void* lora_b, int r, void* y, void* workspace, const LinearPlan& plan,
                         hipStream_t stream) {
  if (m == 0 || n == 0) return hipSuccess;
  if (plan.path == 4) {
    const int64_t elems = m * n;
    const int64_t blocks = (elems + 255) / 256;
    hipLaunchKernelGGL(zero_bf16_kernel, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(256), 0, stream,
                       reinterpret_cast<uint16_t*>(y), elems);
    return hipGetLastError();
  }
  uint8_t* ws = reinterpret_cast<uint8_t*>(workspace);
  const bool has_lora = r > 0 && lora_a && lora_b;
  float* t = has_lora ? reinterpret_cast<float*>(ws + plan.off_t) : nullptr;
  float* tp = (has_lora && plan.lora_parts > 1)
                  ? reinterpret_cast<float*>(ws + plan.off_t + align256(sizeof(float) * (size_t)m * r))
                  : nullptr;
  float* part = reinterpret_cast<float*>(ws + plan.off_part);
  uint32_t* cnt_m = reinterpret_cast<uint32_t*>(ws + plan.off_count);
  uint32_t* cnt_n = cnt_m + kLoraSlots;
  // t = x A^T for the paths that do not form it inside their decode kernel
  if (has_lora && plan.path != 0 && plan.path != 3) {
    const int64_t nsteps = (k + 31) / 32;
    const int P = plan.lora_parts;
    const int spp = (int)((nsteps + P - 1) / P);
    const int64_t mtiles = (m + 15) / 16;
    hipLaunchKernelGGL(lora_down_kernel, dim3((unsigned)(mtiles * P)), dim3(256), 0, stream,
                       reinterpret_cast<const uint16_t*>(x), m, k, reinterpret_cast<const uint16_t*>(lora_a), r, P,
                       spp, tp, t, cnt_m);
  }
  if (plan.path == 0) {
    hipError_t e = launch_decode_f8f4(fmt, plan.dq, x, m, k, codes, scales, tensor_scale, n,
                                      has_lora ? lora_a : nullptr, has_lora ? lora_b : nullptr, r,
                                      cnt_m + kLsyncBase, y, part, cnt_n, stream);
    if (e != hipSuccess) return e;
  } else if (plan.path == 3) {
    hipError_t e = launch_decode_xs(fmt, plan.xs, x, m, k, codes, scales, tensor_scale, n,
                                    has_lora ? lora_a : nullptr, has_lora ? lora_b : nullptr, r, cnt_m + kLsyncBase,
                                    y, part, cnt_n, stream);
    if (e != hipSuccess) return e;
  } else if (plan.path == 2) {
    hipError_t e =
        fmt == FMT_NVFP4
            ? launch_decode<FMT_NVFP4>((int)((m + 3) / 4), x, m, k, codes, scales, tensor_scale, n, t, lora_b, r, y,
                                       part, cnt_n, plan.splits, stream)
            : launch_decode<FMT_MXFP4>(1, x, m, k, codes, scales, tensor_scale, n, t, lora_b, r, y, part, cnt_n,
                                       plan.splits, stream);
    if (e != hipSuccess) return e;
  } else if (gemm_w4_supports(m, n, k, scales)) {
    hipError_t e = launch_gemm_w4(fmt, x, m, k, codes, scales, tensor_scale, n, t, has_lora ? lora_b : nullptr,
                                  has_lora ? r : 0, y, stream);
    if (e != hipSuccess) return e;
  } else {
    const int64_t tiles = ((m + G_BM - 1) / G_BM) * ((n + G_BN - 1) / G_BN);
    const size_t lds = sizeof(uint16_t) * 2 * (G_BM + G_BN) * G_LDA;
    const uint16_t* xx = reinterpret_cast<const uint16_t*>(x);
    const uint16_t* bb = reinterpret_cast<const uint16_t*>(lora_b);
    uint16_t* yy = reinterpret_cast<uint16_t*>(y);
    const bool buf = m * k * 2 < ((int64_t)1 << 31) && n * (k / 2) < ((int64_t)1 << 31);
#define FP4W_GEMM(FMTv, BUFv)                                                                                \
  do {                                                                                                       \
    static std::atomic<uint64_t> lds_done{0};                                                                \
    {                                                                                                        \
      hipError_t e = set_max_lds_once(reinterpret_cast<const void*>(&linear_gemm_kernel<FMTv, BUFv>),        \
                                      (int)lds, lds_done);                                                   \
      if (e != hipSuccess) return e;                                                                         \
    }                                                                                                        \
    hipLaunchKernelGGL((linear_gemm_kernel<FMTv, BUFv>), dim3((unsigned)tiles), dim3(G_THREADS), lds, stream, \
                       xx, m, k, codes, scales, tensor_scale, n, t, bb, has_lora ? r : 0, yy);              \
  } while (0)
    if (fmt == FMT_NVFP4) {
      if (buf) FP4W_GEMM(FMT_NVFP4, true); else FP4W_GEMM(FMT_NVFP4, false);
    } else {
      if (buf) FP4W_GEMM(FMT_MXFP4, true); else FP4W_GEMM(FMT_MXFP4, false);
    }
#undef FP4W_GEMM
  }
  return hipGetLastError();
}

size_t linear_aqn_workspace_bytes(const LinearPlan& plan, int64_t m, int64_t k) {
  return align256(plan.bytes) + align256((size_t)m * (size_t)k * 2);
}

hipError_t launch_linear_aqn(int fmt, const void* x, int64_t m, int64_t k, const void* gamma, const float* noise,
                             float sigma, float eps, const uint8_t* codes, const uint8_t* scales,
                             const float* tensor_scale, int64_t n, const void* lora_a, const void* lora_b, int r,
                             void* y, void* workspace, const LinearPlan& plan, hipStream_t stream) {
  if (m == 0 || n == 0) return hipSuccess;
  const bool has_lora = r > 0 && lora_a && lora_b;
  uint8_t* ws = reinterpret_cast<uint8_t*>(workspace);
  if (plan.path == 0 && k > 0 && decode_f8f4_fuses_aqn(plan.dq, m)) {
    uint32_t* cnt_m = reinterpret_cast<uint32_t*>(ws + plan.off_count);
    hipError_t e = launch_decode_f8f4(fmt, plan.dq, x, m, k, codes, scales, tensor_scale, n,
                                      has_lora ? lora_a : nullptr, has_lora ? lora_b : nullptr, r,
                                      cnt_m + kLsyncBase, y, reinterpret_cast<float*>(ws + plan.off_part),
                                      cnt_m + kLoraSlots, stream, gamma, noise, sigma, eps);
    if (e != hipSuccess) return e;
    return hipGetLastError();
  }
  if (plan.path == 3 && k > 0 && decode_xs_fuses_aqn(fmt, plan.xs, m, k, has_lora ? r : 0, scales)) {
    uint32_t* cnt_m = reinterpret_cast<uint32_t*>(ws + plan.off_count);
    return launch_decode_xs(fmt, plan.xs, x, m, k, codes, scales, tensor_scale, n, has_lora ? lora_a : nullptr,
                            has_lora ? lora_b : nullptr, r, cnt_m + kLsyncBase, y,
                            reinterpret_cast<float*>(ws + plan.off_part), cnt_m + kLoraSlots, stream, gamma, noise,
                            sigma, eps);
  }
  // two launches: the norm into the workspace, then the linear on it
  void* xn = ws + align256(plan.bytes);
  if (k > 0) {
    hipError_t e = launch_aqn_rmsnorm(x, m, k, gamma, noise, sigma, eps, xn, stream);
    if (e != hipSuccess) return e;
  }
  return launch_linear(fmt, xn, m, k, codes, scales, tensor_scale, n, lora_a, lora_b, r, y, workspace, plan, stream);
}

}  // namespace fp4w
