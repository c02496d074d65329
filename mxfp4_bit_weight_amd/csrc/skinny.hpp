// skinny.hpp -- one 16-row tile of the decode-shaped W4A16 product on gfx950.
//
// The pages credit the RL speed-up to rollouts generated in the memory-bound
// regime with a Marlin-like W4A16 kernel (tggo.me/sberlogasci/42740, section
// "Eksperimenty").  That kernel was written for H100; this is a gfx950 design:
//
//  * A workgroup of 4 waves owns a tile of 16 weight rows and a range of K.
//    Each lane loads 16 bytes (32 codes) per 128-wide K step: lane l handles
//    weight row n = l % 16 and K group g = l / 16, so a wave reads 64 bytes
//    per row and the 4 waves interleave steps (256 contiguous bytes per row).
//  * The product runs on v_mfma_f32_16x16x32_bf16 with the weights as the B
//    operand (column n = lane % 16, K group = lane / 16).  A lane's 32 codes
//    feed four MFMAs, 8 codes each; the K order inside an MFMA is free, so x is
//    loaded to match.
//  * NVFP4 block scales are E4M3 and cannot ride on the conversion (which only
//    applies a power of two).  Instead the A operand is block-diagonal: A row
//    4*slot + m holds x row m only in K group `slot` (zeros elsewhere), so the
//    16 output rows keep the four lane groups' block sums apart.  Lane (g, n)
//    receives exactly the outputs of its own block, decodes its own scale and
//    applies it with one FMA per output.  Up to 4 rows of x per m-group; 4
//    m-groups cover 16 rows.
//  * MXFP4 scales are powers of two and go into the conversion itself (exact),
//    so the A operand is plain x (16 rows) and the MFMA accumulates directly.
//
// Every code, scale and x load is predicated on the row and the K range, so
// any N and any K that is a multiple of 32 is handled.
#pragma once
#include "fp4w_device.hpp"

namespace fp4w {

constexpr int SK_WAVES = 4;
constexpr int SK_THREADS = 64 * SK_WAVES;
constexpr int SK_TILE_N = 16;
constexpr int SK_STEP_K = 128;

// 8 codes (one dword) -> 8 bf16 B-operand values, scaled by the power of two `pow2`.
__device__ __forceinline__ bf16x8_t codes8_to_bf16(uint32_t dw, float pow2) {
  u32x4_t r;
  r.x = fp4x2_to_bf16x2_scaled<0>(dw, pow2);
  r.y = fp4x2_to_bf16x2_scaled<1>(dw, pow2);
  r.z = fp4x2_to_bf16x2_scaled<2>(dw, pow2);
  r.w = fp4x2_to_bf16x2_scaled<3>(dw, pow2);
  return as_bf16x8(r);
}

// Per-lane source rows of x for the A operand.  `xrow` points at the start of
// x row m for this lane (nullptr: a zero row).
struct SkinnyTileResult {
  // NVFP4: v[mg][i] is the (m = 4 mg + i, n = lane % 16) sum over this lane's K
  // group only (the caller adds the 4 groups).  MXFP4: v[0][i] is the
  // (m = 4 (lane / 16) + i, n = lane % 16) sum, complete over K groups.
  float v[4][4];
};

// Loads of one K step for one lane: 32 codes, their block scale bytes, and the
// A-operand x values of every m-group.
template <int FMT, int MG>
struct StepData {
  u32x4_t cw;
  uint32_t sc;            // NVFP4: two E4M3 bytes (low = first block); MXFP4: one E8M0 byte
  u32x4_t xa[MG][4];
};

template <int FMT, int MG>
__device__ __forceinline__ void skinny_load(StepData<FMT, MG>& d, const uint8_t* __restrict__ codes_row,
                                            const uint8_t* __restrict__ scales_row,
                                            const uint16_t* const* xrow, int64_t K, int step, int step_end,
                                            int g) {
  const int64_t kg = (int64_t)step * SK_STEP_K + 32 * g;     // this lane's first k
  const bool kin = step < step_end && kg < K;
  d.cw = (u32x4_t){0u, 0u, 0u, 0u};
  d.sc = 0;
  if (kin && codes_row) {
    d.cw = load16(codes_row + kg / 2);
    if (FMT == FMT_NVFP4) d.sc = *reinterpret_cast<const uint16_t*>(scales_row + kg / 16);
    else d.sc = scales_row[kg / 32];
  }
#pragma unroll
  for (int mg = 0; mg < MG; mg++) {
    const uint16_t* xr = xrow[mg];
#pragma unroll
    for (int s = 0; s < 4; s++) d.xa[mg][s] = (u32x4_t){0u, 0u, 0u, 0u};
    if (xr && kin) {
#pragma unroll
      for (int s = 0; s < 4; s++) d.xa[mg][s] = load16(xr + kg + 8 * s);
    }
  }
}

template <int FMT, int MG>
__device__ __forceinline__ void skinny_compute(const StepData<FMT, MG>& d, f32x4_t* acc, float (*nacc)[4]) {
  if (FMT == FMT_NVFP4) {
    const float d0 = e4m3_to_f32(d.sc & 0xFFu), d1 = e4m3_to_f32(d.sc >> 8);
    bf16x8_t b[4];
#pragma unroll
    for (int s = 0; s < 4; s++) b[s] = codes8_to_bf16(d.cw[s], 1.0f);
#pragma unroll
    for (int mg = 0; mg < MG; mg++) {
      const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
      f32x4_t p0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(d.xa[mg][0]), b[0], z, 0, 0, 0);
      p0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(d.xa[mg][1]), b[1], p0, 0, 0, 0);
      f32x4_t p1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(d.xa[mg][2]), b[2], z, 0, 0, 0);
      p1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(d.xa[mg][3]), b[3], p1, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; i++) nacc[mg][i] = __builtin_fmaf(d1, p1[i], __builtin_fmaf(d0, p0[i], nacc[mg][i]));
    }
  } else {
    const float s = e8m0_scale_operand(d.sc);
#pragma unroll
    for (int q = 0; q < 4; q++)
      acc[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(d.xa[0][q]), codes8_to_bf16(d.cw[q], s), acc[0], 0, 0, 0);
  }
}

// Computes the partial tile over K steps [step_begin, step_end) for this wave
// (steps step_begin + wave, + SK_WAVES, ...), issuing the loads of U steps
// before any of their arithmetic.
//   codes_row, scales_row : this lane's weight row (nullptr if the row is out of range)
//   xrow[mg]              : A-operand source row of this lane for m-group mg (or nullptr)
template <int FMT, int MG, int U>
__device__ __forceinline__ void skinny_tile(const uint8_t* __restrict__ codes_row,
                                            const uint8_t* __restrict__ scales_row,
                                            const uint16_t* const* xrow, int64_t K, int step_begin,
                                            int step_end, int wave, int g, SkinnyTileResult& res) {
  f32x4_t acc[MG];
  float nacc[MG][4];
#pragma unroll
  for (int mg = 0; mg < MG; mg++) {
    acc[mg] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; i++) nacc[mg][i] = 0.f;
  }
  for (int step0 = step_begin + wave; step0 < step_end; step0 += SK_WAVES * U) {
    StepData<FMT, MG> d[U];
#pragma unroll
    for (int u = 0; u < U; u++) skinny_load<FMT, MG>(d[u], codes_row, scales_row, xrow, K, step0 + u * SK_WAVES, step_end, g);
#pragma unroll
    for (int u = 0; u < U; u++) skinny_compute<FMT, MG>(d[u], acc, nacc);
  }
#pragma unroll
  for (int mg = 0; mg < 4; mg++)
#pragma unroll
    for (int i = 0; i < 4; i++) res.v[mg][i] = 0.f;
#pragma unroll
  for (int mg = 0; mg < MG; mg++)
#pragma unroll
    for (int i = 0; i < 4; i++) res.v[mg][i] = (FMT == FMT_NVFP4) ? nacc[mg][i] : acc[mg][i];
}

// A-operand source row for lane (i = lane % 16, g = lane / 16) and m-group mg.
// NVFP4 (block-diagonal): active only when i / 4 == g, for x row m = 4 mg + i % 4.
// MXFP4 (plain): x row m = i.
template <int FMT>
__device__ __forceinline__ int a_operand_row(int lane, int mg) {
  const int i = lane & 15, g = lane >> 4;
  if (FMT == FMT_NVFP4) return (i >> 2) == g ? 4 * mg + (i & 3) : -1;
  return mg == 0 ? i : -1;
}

// Reduce the 4 waves' partial tiles (and, for NVFP4, the 4 K groups) into
// out[m * 16 + n] for m < M.  `red` is LDS of SK_WAVES * 64 * 16 floats.
template <int FMT, int MG>
__device__ __forceinline__ void skinny_reduce(const SkinnyTileResult& res, float* red, float* out, int M) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int mg = 0; mg < MG; mg++)
#pragma unroll
    for (int i = 0; i < 4; i++) red[(wave * 16 + mg * 4 + i) * 64 + lane] = res.v[mg][i];
  __syncthreads();
  if (wave == 0) {
    float v[MG][4];
#pragma unroll
    for (int mg = 0; mg < MG; mg++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        float s = 0.f;
#pragma unroll
        for (int w = 0; w < SK_WAVES; w++) s += red[(w * 16 + mg * 4 + i) * 64 + lane];
        v[mg][i] = s;
      }
    const int n = lane & 15, g = lane >> 4;
    if (FMT == FMT_NVFP4) {
#pragma unroll
      for (int mg = 0; mg < MG; mg++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
          float s = v[mg][i];
          s += __shfl_xor(s, 16, 64);
          s += __shfl_xor(s, 32, 64);
          v[mg][i] = s;
        }
      if (g == 0) {
#pragma unroll
        for (int mg = 0; mg < MG; mg++)
#pragma unroll
          for (int i = 0; i < 4; i++) {
            int m = 4 * mg + i;
            if (m < M) out[m * 16 + n] = v[mg][i];
          }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; i++) {
        int m = 4 * g + i;
        if (m < M) out[m * 16 + n] = v[0][i];
      }
    }
  }
  __syncthreads();
}


// ---------------------------------------------------------------------------------
// Decode kernel building blocks.  One wave owns one 16-row weight tile over a
// K range (split).  Its workgroup first stages, in LDS, the split's x rows and
// the block-scale bytes of every tile row, then each wave streams its codes
// through a ring of DEPTH steps of loads in flight: step j is consumed while
// step j + DEPTH loads.  Per step a lane then issues one 16-byte global load;
// scales and x come from LDS (a separate counter, so they never wait behind the
// ring).  Every global load is unconditional (addresses clamped into the
// tensor) so the compiler can count outstanding loads instead of draining:
//   * a row past N reads row N - 1; it only feeds output column n, never stored;
//   * a K group past K or past the split reads the row start; it is consumed
//     with zero x and a zero scale, so it adds nothing;
//   * x lanes that carry no row read a 64-byte zero area at the start of LDS.
// LDS layout: [64 zero bytes][x: M rows x kslice bf16][scales: rows x srow bytes]
// ---------------------------------------------------------------------------------
constexpr int DECODE_XS_ZERO = 32;   // bf16 elements of zeros in front of the staged x rows

template <int FMT>
struct DecodeLds {
  static constexpr int BLK = FMT == FMT_NVFP4 ? 16 : 32;
  // bytes of one staged scale row for a split of `kslice` weights, padded to 16
  __host__ __device__ static int srow_bytes(int kslice) { return ((kslice / BLK) + 15) & ~15; }
  __host__ __device__ static size_t bytes(int M, int kslice, int rows) {
    return 2 * (size_t)DECODE_XS_ZERO + 2 * (size_t)M * kslice + (size_t)rows * srow_bytes(kslice);
  }
};

// `valid` false: this lane's K group is past K or past the split; it then reads
// zero x and a zero scale, so the step adds nothing (no branch, see above).
template <int FMT, int MG>
__device__ __forceinline__ void decode_step(u32x4_t cw, uint32_t sc, bool valid, const uint16_t* __restrict__ xs,
                                            int xs_stride, int kl, int lane, int M, f32x4_t* acc, float (*nacc)[4]) {
  const int i = lane & 15, g = lane >> 4;
  sc = valid ? sc : 0u;
  bf16x8_t b[4];
  if (FMT == FMT_NVFP4) {
#pragma unroll
    for (int s = 0; s < 4; s++) b[s] = codes8_to_bf16(cw[s], 1.0f);
    const float d0 = e4m3_to_f32(sc & 0xFFu), d1 = e4m3_to_f32(sc >> 8);
#pragma unroll
    for (int mg = 0; mg < MG; mg++) {
      // block-diagonal A: lane (i, g) carries x row 4 mg + (i & 3) only when i / 4 == g
      const int m = 4 * mg + (i & 3);
      const bool active = valid && (i >> 2) == g && m < M;
      const uint16_t* xr = active ? xs + DECODE_XS_ZERO + m * xs_stride + kl : xs;
      u32x4_t xa[4];
#pragma unroll
      for (int s = 0; s < 4; s++) xa[s] = *reinterpret_cast<const u32x4_t*>(xr + 8 * s);
      const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
      f32x4_t p0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xa[0]), b[0], z, 0, 0, 0);
      p0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xa[1]), b[1], p0, 0, 0, 0);
      f32x4_t p1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xa[2]), b[2], z, 0, 0, 0);
      p1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xa[3]), b[3], p1, 0, 0, 0);
#pragma unroll
      for (int e = 0; e < 4; e++) nacc[mg][e] = __builtin_fmaf(d1, p1[e], __builtin_fmaf(d0, p0[e], nacc[mg][e]));
    }
  } else {
    const float s = e8m0_scale_operand(sc);
#pragma unroll
    for (int q = 0; q < 4; q++) b[q] = codes8_to_bf16(cw[q], s);
    const uint16_t* xr = (valid && i < M) ? xs + DECODE_XS_ZERO + i * xs_stride + kl : xs;
    u32x4_t xa[4];
#pragma unroll
    for (int q = 0; q < 4; q++) xa[q] = *reinterpret_cast<const u32x4_t*>(xr + 8 * q);
#pragma unroll
    for (int q = 0; q < 4; q++) acc[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xa[q]), b[q], acc[0], 0, 0, 0);
  }
}

// The code ring of one wave.  After run(), v[mg][e] holds:
//   NVFP4 -> (m = 4 mg + e, n = lane % 16), complete after the K-group sum,
//            in lanes 0..15;
//   MXFP4 -> (m = 4 (lane / 16) + e, n = lane % 16).
// codes_row must point into the tensor (clamped by the caller).
template <int FMT, int MG, int DEPTH>
struct DecodeRing {
  u32x4_t ring[DEPTH];
  const uint8_t* codes_row;
  int64_t k0, K;
  int nsteps, g;

  __device__ __forceinline__ void load(int j, u32x4_t& c) const {
    const int64_t k = k0 + (int64_t)j * SK_STEP_K + 32 * g;
    c = load16(codes_row + ((j < nsteps && k < K) ? k : 0) / 2);     // clamped into the row
  }
  __device__ __forceinline__ void prologue(const uint8_t* cr, int64_t k0_, int64_t K_, int nsteps_, int lane) {
    codes_row = cr; k0 = k0_; K = K_; nsteps = nsteps_; g = lane >> 4;
#pragma unroll
    for (int u = 0; u < DEPTH; u++) load(u, ring[u]);
    __builtin_amdgcn_sched_barrier(0);
  }
  // srow: this lane's staged scale row in LDS.  The scheduling barriers keep
  // each refill where it is written: without them the scheduler sinks the loads
  // next to their uses and the ring collapses.
  __device__ __forceinline__ void run(const uint16_t* __restrict__ xs, int xs_stride, const uint8_t* __restrict__ srow,
                                      int M, int lane, float (*v)[4]) {
    f32x4_t acc[1] = {{0.f, 0.f, 0.f, 0.f}};
    float nacc[MG][4];
#pragma unroll
    for (int mg = 0; mg < MG; mg++)
#pragma unroll
      for (int e = 0; e < 4; e++) nacc[mg][e] = 0.f;
    for (int base = 0; base < nsteps; base += DEPTH) {
#pragma unroll
      for (int u = 0; u < DEPTH; u++) {
        const int j = base + u;
        const int kl = j * SK_STEP_K + 32 * g;                     // k within the split
        const bool valid = j < nsteps && k0 + kl < K;
        const int jc = j < nsteps ? j : 0;
        uint32_t sc;
        if (FMT == FMT_NVFP4) sc = *reinterpret_cast<const uint16_t*>(srow + (jc * SK_STEP_K + 32 * g) / 16);
        else sc = srow[(jc * SK_STEP_K + 32 * g) / 32];
        decode_step<FMT, MG>(ring[u], sc, valid, xs, xs_stride, kl, lane, M, acc, nacc);
        load(j + DEPTH, ring[u]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (FMT == FMT_NVFP4) {
#pragma unroll
      for (int mg = 0; mg < MG; mg++)
#pragma unroll
        for (int e = 0; e < 4; e++) {
          float s = nacc[mg][e];
          s += __shfl_xor(s, 16, 64);
          s += __shfl_xor(s, 32, 64);
          v[mg][e] = s;
        }
    } else {
#pragma unroll
      for (int e = 0; e < 4; e++) v[0][e] = acc[0][e];
    }
  }
};

}  // namespace fp4w
