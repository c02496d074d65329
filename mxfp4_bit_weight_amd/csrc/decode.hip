// decode.hip -- the decode-shaped W4A16 product (1 <= m <= 16 rows of x) on
// gfx950's block-scaled matrix core.
//
// The pages generate rollouts with a weight-only 4-bit model whose product is
// memory-bound (tggo.me/sberlogasci/42740, section "Eksperimenty"): each decode
// step streams every weight code once.  The kernel credited there was written
// for H100 and dequantizes codes to 16-bit values in registers; on gfx950 that
// conversion (one instruction per two codes) left the kernel issue-bound.  Here
// the E2M1 codes go to v_mfma_scale_f32_16x16x128_f8f6f4 exactly as they sit in
// memory, and x is brought to the instruction's form instead (xenc.hpp: two
// E4M3 terms with E8M0 block scales, exact for the elements that matter).
//
// Instruction layout (measured on the device):
//   B (E2M1): lane (n = l % 16, g = l / 16) holds k = 32 g .. 32 g + 31 of column n
//             in 16 bytes -- the 16 bytes of codes a lane loads per 128-wide step;
//   A (E4M3): lane (r = l % 16, g) holds, in 32 bytes, k = 16 g + i (bytes 0-15)
//             and k = 64 + 16 g + i (bytes 16-31) of row r;
//   scales:   E8M0, one per 32-wide K block b and row (A) or column (B), taken
//             from lane 16 b + row / column;
//   D:        lane (n, g) holds rows 4 g + i, column n.
//
// MXFP4 (scales are E8M0 per 32 weights): the weight's own block scales are the
//   B scales, so the product is exact in the instruction.  A rows 0-7 carry the
//   high terms of x rows m = 8 q .. 8 q + 7, rows 8-15 their low terms; one
//   instruction per step covers 8 rows of x.
// NVFP4 (E4M3 scale per 16 weights, not a power of two): A is block-diagonal.
//   Row s (s < 8) carries the high term of x row m only inside the s-th
//   16-wide block of the step, row 8 + s its low term; B scales are 1.  Output
//   row s then holds the block sums of block s apart, and lane (n, g) -- rows
//   4 g .. 4 g + 3, i.e. blocks 4 (g & 1) .. 4 (g & 1) + 3 -- multiplies them by
//   its own four E4M3 scales.  One instruction per step and row of x.
//
// Work split: a workgroup of NW waves owns one tile of 16 weight rows and one of
// S slices of K.  Its threads encode the slice of x into LDS and stage the tile
// rows' scale bytes (and LoRA operands); the NW waves then stream contiguous
// parts of the slice, all their code loads in flight at once (buffer loads: a
// step past the part or rows past N read zeros and cost no memory traffic).
// Wave partials are added in LDS in wave order; with several slices the last
// workgroup of a tile to arrive adds the slices' partials in slice order, so
// the result never depends on scheduling.
//
// LoRA (t = x A^T, then t B^T added to every output row): formed inside the
// same launch by the grid's first workgroups and handed over through the
// workspace (lora_handover.hpp).  In the workgroups that write outputs, the
// first wave done with its share of the codes polls for t while its sibling
// waves still stream.
#include "fp4w_device.hpp"
#include "fp4w_internal.hpp"
#include "lora_handover.hpp"
#include "sync.hpp"
#include "xenc.hpp"

#include <atomic>
#include <type_traits>

namespace fp4w {

typedef __attribute__((ext_vector_type(8))) int i32x8_t;

constexpr int DQ_STEP = 128;       // K per step: one block-scaled MFMA
constexpr int DQ_ROWS = 16;        // weight rows per tile
constexpr int DQ_MAX_R = 64;       // LoRA rank staged in LDS

// LDS layout of one workgroup (byte offsets):
//   zeros   128 (spw + 1)          A lanes that carry no x read here (spw: the longest part of a wave)
//   xh, xl  m rows x (kslice + 16) high / low E4M3 terms (rows padded against bank conflicts)
//   sc      m x 2 x nblkp          E8M0 codes of the terms, byte 4 j + b = block b of step j
//   ws      16 x srow              the tile rows' weight-scale bytes of the slice
//   lb      16 x r bf16            the tile rows of the LoRA B
//   lt      m x r fp32             t = x A^T
//   red     nw x m x 16 fp32       wave partials
//   lr      nw x m x r fp32        wave partials of a LoRA chunk
// Steps of a slice per wave: wave 0 takes `first`, the others `rest` each.  With
// LoRA and 4 waves, wave 0 (the one that fetches t and arrives when its part is
// done) takes kDqLoraLead steps fewer than an even share, so that its wait for t
// and its arrival overlap the other waves' streaming instead of trailing it
// (MI355X, m = 1: 18944 x 3584 12.2 -> 11.6 us; with 8 or 16 waves the waves end
// spread out anyway, and a short part was slower: 3584 x 18944 12.9 -> 13.6 us).
constexpr int kDqLoraLead = 3;
struct DqParts { int first, rest; };
__host__ __device__ inline DqParts dq_parts(int nss, int nw, bool lora) {
  const int even = (nss + nw - 1) / nw;
  if (!lora || nw != 4 || even <= kDqLoraLead) return DqParts{even, even};
  const int first = even - kDqLoraLead;
  return DqParts{first, (nss - first + nw - 2) / (nw - 1)};
}

struct DqLayout {
  int kslice, xrow, nblkp, srow, spw;
  int zero_off, xh_off, xl_off, sc_off, ws_off, lb_off, lt_off, red_off, lr_off, bytes;
};

__host__ __device__ inline DqLayout dq_layout(int fmt, int m, int kslice, int nw, int r) {
  DqLayout L;
  const int blk = fmt == FMT_NVFP4 ? 16 : 32;
  L.kslice = kslice;
  L.xrow = kslice + 16;
  L.nblkp = ((kslice / 32) + 3) & ~3;
  L.srow = ((kslice / blk) + 15) & ~15;
  L.spw = dq_parts(kslice / DQ_STEP, nw, r > 0).rest;     // the longest part
  int off = 0;
  L.zero_off = off; off += DQ_STEP * (L.spw + 1);
  L.xh_off = off;   off += m * L.xrow;
  L.xl_off = off;   off += m * L.xrow;
  L.sc_off = off;   off += 2 * m * L.nblkp;
  off = (off + 15) & ~15;
  L.ws_off = off;   off += DQ_ROWS * L.srow;
  L.lb_off = off;   off += (DQ_ROWS * r * 2 + 15) & ~15;
  L.lt_off = off;   off += m * r * 4;
  L.red_off = off;  off += nw * m * DQ_ROWS * 4;
  L.lr_off = off;   off += nw * m * r * 4;
  L.bytes = off;
  return L;
}

template <int FMT, int NQ, int NW, int DEPTH, bool LORA, bool AQN>
// The fused norm's gain staging takes ~20 more VGPRs: held to 5 waves per SIMD at
// ring depth 8 (else a few AGPRs push the LoRA variant to 4, and a 4-wave grid of
// 1191 groups no longer fits the chip in one round)
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(AQN && DEPTH <= 8 ? 5 : 1)))
void decode_f8f4_kernel(
    const uint16_t* __restrict__ x, int M, int64_t K, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ scales, const float* __restrict__ tensor_scale, int64_t N,
    const uint16_t* __restrict__ lora_a, const uint16_t* __restrict__ lora_b, int r,
    int lparts, int lsw, uint32_t* __restrict__ lsync, uint16_t* __restrict__ y, float* __restrict__ part,
    uint32_t* __restrict__ cnt, int S, int sps, int nsteps_total, int ntiles, int scales16,
    uint64_t wait_ticks, const uint16_t* __restrict__ gam, const float* __restrict__ noise, float sigma,
    float eps) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  __shared__ int flag;
  __shared__ float aqn_ss[AQN ? NW : 1][2];                       // AQN: per-wave sums of x^2, rows 0 and 1
  const XGain xg = AQN ? XGain{gam, noise, sigma} : XGain{nullptr, nullptr, 0.f};
  __shared__ int lfin, have_t;                                    // LoRA: waves done streaming; t published
  constexpr int NT = 64 * NW;
  constexpr int BLK = FMT == FMT_NVFP4 ? 16 : 32;
  // staging units per thread whose loads are issued before the ring (the rest,
  // if any, load after it): x units of 8 elements, 16-byte scale units
  constexpr int DQ_XPRE = NW >= 16 ? 3 : 2;
  constexpr int DQ_SPRE = NW >= 16 ? 2 : 1;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);      // uniform: keeps the buffer descriptor scalar
  const int rr = LORA ? r : 0;                                   // LORA: lora_a, lora_b given, r > 0
  const int mr = M * rr;
  const int words = lparts * mr;                                  // chunk words of the hand-over
  const DqLayout L = dq_layout(FMT, M, sps * DQ_STEP, NW, rr);
  const int bid = (int)blockIdx.x - lparts;                       // < 0: a LoRA chunk workgroup
  const int s = bid % S, tile = bid / S;
  const int nread = ntiles * S;                                   // LoRA: every tile workgroup reads t
  float* lr = reinterpret_cast<float*>(lds + L.lr_off);            // [wave][m][j]: a LoRA chunk
  if (LORA && bid < 0) {
    // ---- 0. a chunk workgroup: its partial of t, complemented, then its arrival --
    lora_chunk_publish(lr, x, M, K, lora_a, rr, (int)blockIdx.x, NW, lsw, lsync, nread, lparts, xg);
    return;
  }


  const int kslice = L.kslice;
  const int step0 = s * sps;
  const int nss = min(sps, nsteps_total - step0);          // steps in this slice
  const int64_t k0 = (int64_t)step0 * DQ_STEP;
  const int64_t row_base = (int64_t)tile * DQ_ROWS;

  // ---- 1. staging loads: x units, weight-scale units, LoRA operands ----------------
  const int xunits_row = kslice / 8;
  const int xunits = M * xunits_row;
  u32x4_t xv[DQ_XPRE];
#pragma unroll
  for (int c = 0; c < DQ_XPRE; c++) {
    const int u = tid + c * NT;
    const int m = u / xunits_row, kk = 8 * (u - m * xunits_row);
    const bool ok = u < xunits && k0 + kk < K;
    xv[c] = load16(x + (ok ? (int64_t)m * K + k0 + kk : 0));
    if (!ok) xv[c] = (u32x4_t){0u, 0u, 0u, 0u};
  }
  // AQN: the gain's gamma and noise at the same k (one K slice: k0 = 0)
  u32x4_t gv[DQ_XPRE], nv0[DQ_XPRE], nv1[DQ_XPRE];
  if (AQN) {
#pragma unroll
    for (int c = 0; c < DQ_XPRE; c++) {
      const int u = tid + c * NT;
      const int m = u / xunits_row, kk = 8 * (u - m * xunits_row);
      const int64_t ko = u < xunits && k0 + kk < K ? k0 + kk : 0;
      gv[c] = load16(gam + ko);
      nv0[c] = load16(noise + ko);
      nv1[c] = load16(noise + ko + 4);
    }
  }
  const int64_t krem = K - k0;
  const int svalid = (int)((krem < kslice ? krem : kslice) / BLK);   // scale bytes of a row in this slice
  const int64_t srow_g = K / BLK;
  const int us_row = scales16 ? svalid / 16 : 0;                     // whole 16-byte units per row
  const int us = DQ_ROWS * us_row;
  u32x4_t sv[DQ_SPRE];
#pragma unroll
  for (int c = 0; c < DQ_SPRE; c++) {
    const int u = tid + c * NT;
    const int rw = u / (us_row > 0 ? us_row : 1), q = u - rw * us_row;
    int64_t grow = row_base + rw;
    grow = grow < N ? grow : N - 1;
    sv[c] = load16(scales + (u < us ? grow * srow_g + k0 / BLK + 16 * q : 0));
  }
  // first LoRA B element of this thread; the rest load later
  uint32_t lbv = 0;
  if (rr > 0) {
    const int rw = tid / rr, j = tid - rw * rr;
    if (tid < DQ_ROWS * rr && row_base + rw < N) lbv = lora_b[(row_base + rw) * rr + j];
  }

  // ---- 2. the code ring: every load of this wave's part in flight ---------------
  const int n = lane & 15, g = lane >> 4;
  const DqParts pp = dq_parts(nss, NW, LORA);
  const int j0 = wave == 0 ? 0 : pp.first + (wave - 1) * pp.rest;
  const int j1 = min(j0 + (wave == 0 ? pp.first : pp.rest), nss);
  const int64_t tile_rows = min((int64_t)DQ_ROWS, N - row_base);
  const __amdgpu_buffer_rsrc_t crs = make_rsrc(codes + row_base * (K / 2), (uint32_t)(tile_rows * (K / 2)));
  const uint32_t lane_off = (uint32_t)(n * (K / 2) + (k0 + 32 * g) / 2);
  const int64_t lane_rem = krem - 32 * g;          // K left for this lane's group from the slice start
  const int lane_lim = (int)(lane_rem < (int64_t)kslice ? lane_rem : (int64_t)kslice);
  auto code_off = [&](int j) -> uint32_t {
    // steps past the part, and the K tail of the last step, read past the buffer
    const bool ok = (j < j1) & (j * DQ_STEP < lane_lim);
    return ok ? lane_off + (uint32_t)(j * (DQ_STEP / 2)) : kBufferOob;
  };
  u32x4_t ring[DEPTH];
#pragma unroll
  for (int u = 0; u < DEPTH; u++) ring[u] = buffer_load16(crs, code_off(j0 + u));
  __builtin_amdgcn_sched_barrier(0);

  // ---- 3. encode x into LDS; zeros; scale bytes; LoRA operands ------------------
  float ssq[2] = {0.f, 0.f};                         // AQN: this thread's sums of x^2, rows 0 and 1
  auto put_x = [&](int u, u32x4_t v) {
    const XEnc8 e = encode_x8(v);
    if (u < xunits) {
      const int m = u / xunits_row, c = u - m * xunits_row;
      uint8_t* ph = lds + L.xh_off + m * L.xrow + 8 * c;
      uint8_t* pl = lds + L.xl_off + m * L.xrow + 8 * c;
      *reinterpret_cast<uint2*>(ph) = make_uint2(e.h[0], e.h[1]);
      *reinterpret_cast<uint2*>(pl) = make_uint2(e.l[0], e.l[1]);
      if ((c & 3) == 0) {
        lds[L.sc_off + (2 * m) * L.nblkp + c / 4] = (uint8_t)e.sch;
        lds[L.sc_off + (2 * m + 1) * L.nblkp + c / 4] = (uint8_t)e.scl;
      }
    }
  };
  // quads of lanes hold one 32-element block: all four take the same branch
  // AQN: x enters as bf16(x g), g = gamma (1 + sigma noise); the row factor
  // 1 / sqrt(mean x^2 + eps) multiplies the fp32 sums at the end
  auto gain = [&](int u, u32x4_t v, u32x4_t g_, u32x4_t n0, u32x4_t n1) -> u32x4_t {
    if (!AQN) return v;
    const int m = u / xunits_row;
    float s2 = 0.f;
    const u32x4_t o = xgain_bf16(v, g_, n0, n1, sigma, &s2);
    if (u < xunits) {
      if (m == 0) ssq[0] += s2;
      else ssq[1] += s2;
    }
    return o;
  };
#pragma unroll
  for (int c = 0; c < DQ_XPRE; c++) {
    const int u = tid + c * NT;
    if (u - (u & 3) < xunits) put_x(u, AQN ? gain(u, xv[c], gv[c], nv0[c], nv1[c]) : xv[c]);
  }
  for (int u = tid + DQ_XPRE * NT; u - (u & 3) < xunits; u += NT) {
    const int m = u / xunits_row, kk = 8 * (u - m * xunits_row);
    const bool ok = u < xunits && k0 + kk < K;
    u32x4_t v = load16(x + (ok ? (int64_t)m * K + k0 + kk : 0));
    if (!ok) v = (u32x4_t){0u, 0u, 0u, 0u};
    if (AQN) {
      const int64_t ko = ok ? k0 + kk : 0;
      v = gain(u, v, load16(gam + ko), load16(noise + ko), load16(noise + ko + 4));
    }
    put_x(u, v);
  }
  if (AQN) {                                         // per-wave sums, in lane order
#pragma unroll
    for (int q = 0; q < 2; q++) {
      float v = ssq[q];
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
      if (lane == 0) aqn_ss[wave][q] = v;
    }
  }
  for (int u = tid; u < DQ_STEP * (L.spw + 1) / 16; u += NT)
    *reinterpret_cast<u32x4_t*>(lds + L.zero_off + 16 * u) = (u32x4_t){0u, 0u, 0u, 0u};
#pragma unroll
  for (int c = 0; c < DQ_SPRE; c++) {
    const int u = tid + c * NT;
    if (u < us) {
      const int rw = u / us_row, q = u - rw * us_row;
      const bool ok = row_base + rw < N;
      *reinterpret_cast<u32x4_t*>(lds + L.ws_off + rw * L.srow + 16 * q) = ok ? sv[c] : (u32x4_t){0u, 0u, 0u, 0u};
    }
  }
  for (int u = tid + DQ_SPRE * NT; u < us; u += NT) {
    const int rw = u / us_row, q = u - rw * us_row;
    int64_t grow = row_base + rw;
    const bool ok = grow < N;
    grow = ok ? grow : N - 1;
    const u32x4_t v = load16(scales + grow * srow_g + k0 / BLK + 16 * q);
    *reinterpret_cast<u32x4_t*>(lds + L.ws_off + rw * L.srow + 16 * q) = ok ? v : (u32x4_t){0u, 0u, 0u, 0u};
  }
  {   // remaining scale bytes (unaligned rows, a partial last unit, padding), byte by byte
    const int first = 16 * us_row;
    const int per_row = L.srow - first;
    for (int idx = tid; idx < DQ_ROWS * per_row; idx += NT) {
      const int rw = idx / per_row, b = first + (idx - rw * per_row);
      const int64_t grow = row_base + rw;
      uint8_t val = 0;
      if (b < svalid && grow < N) val = scales[grow * srow_g + k0 / BLK + b];
      lds[L.ws_off + rw * L.srow + b] = val;
    }
  }
  if (rr > 0) {
    uint16_t* lb = reinterpret_cast<uint16_t*>(lds + L.lb_off);
    if (tid == 0) lfin = 0;
    if (tid < DQ_ROWS * rr) lb[tid] = (uint16_t)lbv;
    for (int e = tid + NT; e < DQ_ROWS * rr; e += NT) {
      const int rw = e / rr, j = e - rw * rr;
      lb[e] = row_base + rw < N ? lora_b[(row_base + rw) * rr + j] : (uint16_t)0;
    }
  }
  __syncthreads();

  // ---- 4. stream the part --------------------------------------------------------
  const int ar = lane & 15, ag = lane >> 4;       // A-operand row and K group of this lane
  const int hl = ar >> 3;                          // 0: high terms, 1: low terms
  float v[NQ][4];
  if (FMT == FMT_NVFP4) {
    const int sb = ar & 7;                         // the 16-wide block row ar carries
    const bool lo_on = sb < 4 && ag == sb, hi_on = sb >= 4 && ag == sb - 4;
    int a_lo[NQ], a_hi[NQ], a_sc[NQ];
#pragma unroll
    for (int q = 0; q < NQ; q++) {
      const int data = (hl ? L.xl_off : L.xh_off) + q * L.xrow + 16 * sb + DQ_STEP * j0;
      a_lo[q] = lo_on ? data : L.zero_off;
      a_hi[q] = hi_on ? data : L.zero_off;
      a_sc[q] = L.sc_off + (2 * q + hl) * L.nblkp + 4 * j0 + ag;
    }
    const int w_sc = L.ws_off + n * L.srow + 8 * j0 + 4 * (g & 1);
    // The scale FMAs of a step run one step later, after the next MFMA has been
    // issued, so the MFMA latency is not waited out in every step.
    float acc[NQ][4];
    f32x4_t dprev[NQ];
    f32x2_t s01 = {0.f, 0.f}, s23 = {0.f, 0.f};
#pragma unroll
    for (int q = 0; q < NQ; q++) {
      dprev[q] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; i++) acc[q][i] = 0.f;
    }
    // A part that fits the ring was issued whole by the prologue: no refill loads
    // (a load past the part still costs an instruction in the unit's in-order
    // return queue).  The two cases are separate loops, so each gets exact wait counts.
    auto run = [&](auto refill) {
    for (int jb = 0; jb < j1 - j0; jb += DEPTH) {
#pragma unroll
      for (int u = 0; u < DEPTH; u++) {
        const int jr = jb + u;                     // step relative to j0
        if (jr < j1 - j0) {
          const u32x4_t cw = ring[u];
          const i32x8_t b = {(int)cw.x, (int)cw.y, (int)cw.z, (int)cw.w, 0, 0, 0, 0};
          const uint32_t w4 = *reinterpret_cast<const uint32_t*>(lds + w_sc + 8 * jr);
          f32x4_t dcur[NQ];
#pragma unroll
          for (int q = 0; q < NQ; q++) {
            const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(lds + a_lo[q] + DQ_STEP * jr);
            const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(lds + a_hi[q] + DQ_STEP * jr);
            const int sa = lds[a_sc[q] + 4 * jr];
            const i32x8_t a = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
            dcur[q] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, z, 0, 4, 0, sa, 0, 127);
          }
#pragma unroll
          for (int q = 0; q < NQ; q++) {
            acc[q][0] = __builtin_fmaf(s01.x, dprev[q][0], acc[q][0]);
            acc[q][1] = __builtin_fmaf(s01.y, dprev[q][1], acc[q][1]);
            acc[q][2] = __builtin_fmaf(s23.x, dprev[q][2], acc[q][2]);
            acc[q][3] = __builtin_fmaf(s23.y, dprev[q][3], acc[q][3]);
            dprev[q] = dcur[q];
          }
          s01 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w4, 1.0f, false);   // E4M3 -> fp32, exact
          s23 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w4, 1.0f, true);
        }
        if constexpr (decltype(refill)::value) {
          // 16-wave single-chain groups with LoRA skip the loads past their part
          // (a uniform branch: its wait counts turn conservative, which costs the
          // 4- and 8-wave groups more than the loads; 3584 x 18944, m = 1, LoRA
          // r = 16: 12.51 -> 11.63 us NVFP4, 12.13 -> 11.26 us MXFP4)
          if (!(NQ == 1 && NW == 16 && LORA) || jb + u + DEPTH < j1 - j0)
            ring[u] = buffer_load16(crs, code_off(j0 + jb + u + DEPTH));
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    };
    if (j1 - j0 > DEPTH) run(std::true_type{});
    else run(std::false_type{});
#pragma unroll
    for (int q = 0; q < NQ; q++) {
      acc[q][0] = __builtin_fmaf(s01.x, dprev[q][0], acc[q][0]);
      acc[q][1] = __builtin_fmaf(s01.y, dprev[q][1], acc[q][1]);
      acc[q][2] = __builtin_fmaf(s23.x, dprev[q][2], acc[q][2]);
      acc[q][3] = __builtin_fmaf(s23.y, dprev[q][3], acc[q][3]);
    }
    // lane (n, g): blocks 4 (g & 1) + i of the high (g < 2) or low (g >= 2) terms
#pragma unroll
    for (int q = 0; q < NQ; q++) {
      float sum = (acc[q][0] + acc[q][1]) + (acc[q][2] + acc[q][3]);
      sum += __shfl_xor(sum, 16, 64);
      sum += __shfl_xor(sum, 32, 64);
      v[q][0] = sum;                                // (m = q, n), in every lane
    }
  } else {
    int a_x[NQ], a_sc[NQ];
#pragma unroll
    for (int q = 0; q < NQ; q++) {
      const int m = 8 * q + (ar & 7);
      const bool on = m < M;
      a_x[q] = on ? (hl ? L.xl_off : L.xh_off) + m * L.xrow + 16 * ag + DQ_STEP * j0 : L.zero_off + 16 * ag;
      a_sc[q] = L.sc_off + (2 * (on ? m : M - 1) + hl) * L.nblkp + 4 * j0 + ag;
    }
    const int w_sc = L.ws_off + n * L.srow + 4 * j0 + g;
    f32x4_t acc[NQ];
#pragma unroll
    for (int q = 0; q < NQ; q++) acc[q] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
    // A part that fits the ring was issued whole by the prologue: no refill loads
    // (a load past the part still costs an instruction in the unit's in-order
    // return queue).  The two cases are separate loops, so each gets exact wait counts.
    auto run = [&](auto refill) {
    for (int jb = 0; jb < j1 - j0; jb += DEPTH) {
#pragma unroll
      for (int u = 0; u < DEPTH; u++) {
        const int jr = jb + u;
        if (jr < j1 - j0) {
          const u32x4_t cw = ring[u];
          const i32x8_t b = {(int)cw.x, (int)cw.y, (int)cw.z, (int)cw.w, 0, 0, 0, 0};
          const int sbw = lds[w_sc + 4 * jr];
#pragma unroll
          for (int q = 0; q < NQ; q++) {
            const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(lds + a_x[q] + DQ_STEP * jr);
            const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(lds + a_x[q] + DQ_STEP * jr + 64);
            const int sa = lds[a_sc[q] + 4 * jr];
            const i32x8_t a = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            acc[q] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc[q], 0, 4, 0, sa, 0, sbw);
          }
        }
        if constexpr (decltype(refill)::value) {
          // 16-wave single-chain groups with LoRA skip the loads past their part
          // (a uniform branch: its wait counts turn conservative, which costs the
          // 4- and 8-wave groups more than the loads; 3584 x 18944, m = 1, LoRA
          // r = 16: 12.51 -> 11.63 us NVFP4, 12.13 -> 11.26 us MXFP4)
          if (!(NQ == 1 && NW == 16 && LORA) || jb + u + DEPTH < j1 - j0)
            ring[u] = buffer_load16(crs, code_off(j0 + jb + u + DEPTH));
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    };
    if (j1 - j0 > DEPTH) run(std::true_type{});
    else run(std::false_type{});
    // lane (n, g): rows 4 g + i = high (g < 2) / low (g >= 2) terms of m = 8 q + 4 (g & 1) + i
#pragma unroll
    for (int q = 0; q < NQ; q++)
#pragma unroll
      for (int i = 0; i < 4; i++) v[q][i] = acc[q][i] + __shfl_xor(acc[q][i], 32, 64);
  }

  if (LORA) {
    // ---- 4b. the first wave done with its part fetches the chunk words of t
    //      (bounded wait) and adds them in chunk order while the others stream;
    //      then it arrives (its round trips overlap the others' streaming) ------
    int first = 0;
    if (lane == 0) first = atomicAdd(&lfin, 1) == 0;
    first = __shfl(first, 0, 64);
    if (first) {
      float* lt = reinterpret_cast<float*>(lds + L.lt_off);
      const int ok = lora_poll(lsync, lparts, mr, lt, wait_ticks, lane);
      if (lane == 0) have_t = ok;
      const uint32_t old = lsync_reader_issue(lsync, bid, lane);
      lsync_reader_complete(lsync, old, bid, nread, lparts, words, lane);
    }
  }

  // ---- 5. wave partials -> LDS, tile sums in wave order --------------------------
  float* red = reinterpret_cast<float*>(lds + L.red_off);      // [wave][m][16]
  if (FMT == FMT_NVFP4) {
    if (g == 0) {
#pragma unroll
      for (int q = 0; q < NQ; q++)
        if (q < M) red[(wave * M + q) * DQ_ROWS + n] = v[q][0];
    }
  } else if (g < 2) {
#pragma unroll
    for (int q = 0; q < NQ; q++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int m = 8 * q + 4 * g + i;
        if (m < M) red[(wave * M + m) * DQ_ROWS + n] = v[q][i];
      }
  }
  __syncthreads();
  const int nout = M * DQ_ROWS;                 // (m, n) outputs of the tile, <= 256 <= NT
  const int e = tid;
  float o = 0.f;
  if (e < nout) {
#pragma unroll
    for (int p = 0; p < NW; p++) o += red[p * nout + e];
  }
  if (S > 1) {
    if (e < nout) store_agent(&part[((int64_t)s * ntiles + tile) * nout + e], o);
    if (!arrive_last(&cnt[tile], (uint32_t)S, &flag)) return;
    if (e < nout) {
      float sum = 0.f;
      for (int q = 0; q < S; q++) sum += load_agent(&part[((int64_t)q * ntiles + tile) * nout + e]);
      o = sum;
    }
  }
  if (LORA && __builtin_expect(!have_t, 0)) {
    // ---- 6. the wait for t ran out: the chunks formed here, by the same steps in
    //      the same order -----------------------------------------------------------
    lora_form_all(lr, reinterpret_cast<float*>(lds + L.lt_off), x, M, K, lora_a, rr, NW, lsw, lparts, xg);
  }
  if (e < nout) {
    const int m = e / DQ_ROWS, nn = e - m * DQ_ROWS;
    const int64_t row = row_base + nn;
    if (row < N) {
      const float st = (FMT == FMT_NVFP4) ? *tensor_scale : 1.0f;
      float out = st * o;
      if (rr > 0) {
        const uint16_t* lb = reinterpret_cast<const uint16_t*>(lds + L.lb_off);
        const float* lt = reinterpret_cast<const float*>(lds + L.lt_off);
        float l = 0.f;
        for (int j = 0; j < rr; j++) l = __builtin_fmaf(lt[m * rr + j], __uint_as_float((uint32_t)lb[nn * rr + j] << 16), l);
        out += l;
      }
      if (AQN) {                                     // the row factor of the norm, waves in order
        float ss = 0.f;
        for (int w = 0; w < NW; w++) ss += aqn_ss[w][m];
        out *= 1.0f / __builtin_sqrtf(ss / (float)K + eps);
      }
      y[(int64_t)m * N + row] = (uint16_t)f32_to_bf16_rne(out);
    }
  }
}

// ---------------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------------
bool decode_f8f4_supports(int fmt, int64_t m) {
  return m >= 1 && (fmt == FMT_NVFP4 ? m <= 8 : m <= 16);
}

size_t decode_f8f4_lds_bytes(int fmt, int64_t m, int kslice, int nw, int r) {
  return (size_t)dq_layout(fmt, (int)m, kslice, nw, r).bytes;
}

// Waves per tile (the workgroup) and K slices.  Aim: every code load of the
// launch issued up front, by as few waves as can hold them (a ring of at most 16
// loads each); K slices (an arrival atomic and a second pass over the partials)
// only when the x slice does not fit the LDS budget or the waves are very few.
constexpr int64_t kDqTargetWaves = 768;

static int dq_budget(int nw) { return nw == 4 ? 40 * 1024 : 64 * 1024; }

DecodeConfig plan_decode_f8f4(int fmt, int64_t m, int64_t n, int64_t k, int r) {
  DecodeConfig c{};
  const int64_t ntiles = (n + DQ_ROWS - 1) / DQ_ROWS;
  const int64_t nsteps = (k + DQ_STEP - 1) / DQ_STEP;
  // the fewest waves per tile whose parts (of the whole K) are at most 16 steps
  // (measured on MI355X at m = 1: 3584 x 3584 takes 4.7 us with 4 waves against
  // 6.3 us with 16; 18944 x 3584 is best with 4, 3584 x 18944 with 16)
  c.nw = nsteps <= 4 * 16 ? 4 : nsteps <= 8 * 16 ? 8 : 16;
  // more waves when the tiles are few (3584 x 3584 at m = 2: 5.4 us with 8
  // waves, 6.4 with 4; at m = 1 without LoRA 4.56 -> 4.47 us).  Not at m = 1 with
  // LoRA: 8-wave chunk workgroups take twice the K each, and with A read cold
  // (its own A per weight, as in a model) t comes later: 6.28 -> 6.92 us.
  if (c.nw == 4 && ntiles * 4 < 1536 && (m >= 2 || r == 0)) c.nw = 8;
  if (m >= 2 && c.nw > 8) c.nw = 8;     // several MFMA chains per wave: 1024-thread groups would spill
  auto sps_for = [&](int64_t s) {
    int64_t sps = (nsteps + s - 1) / s;
    if (s > 1) sps = (sps + 3) & ~(int64_t)3;                         // 16-byte aligned scale slices
    return sps;
  };
  int64_t s = 1;
  // LDS: grow S until the slice fits
  while (s < nsteps && decode_f8f4_lds_bytes(fmt, m, (int)(sps_for(s) * DQ_STEP), c.nw, r) > (size_t)dq_budget(c.nw)) s++;
  // parallelism: more slices while the waves are few and each keeps >= 4 steps
  while (ntiles * c.nw * s < kDqTargetWaves && (sps_for(s + 1) + c.nw - 1) / c.nw >= 4) s++;
  c.sps = (int)sps_for(s);
  c.splits = (int)((nsteps + c.sps - 1) / c.sps);
  const int spw = dq_parts(c.sps, c.nw, r > 0).rest;    // the longest part of a wave
  // Ring of code loads per wave: a part of at most 8 steps is issued whole up
  // front (at most 4: a ring of 4, so no load past the part is issued); longer
  // parts go through a ring of 4 refilled as steps are consumed, which spreads a
  // workgroup's arrivals, and its decode, over the stream (MI355X, m = 1, no
  // LoRA, 3584 x 18944: 11.7 -> 10.8 us against a ring of 16 issued whole).
  // launch_decode_f8f4 takes the ring of 4 also with LoRA and for NVFP4 at m >= 2.
  c.depth = spw <= 4 || spw > 8 ? 4 : 8;
  return c;
}

static std::atomic<int64_t> g_lora_wait{100000};          // 1 ms
int64_t lora_wait_ticks() { return g_lora_wait.load(std::memory_order_relaxed); }
int64_t set_lora_wait_ticks(int64_t ticks) { return g_lora_wait.exchange(ticks, std::memory_order_relaxed); }


template <int FMT, int NQ, bool AQN>
static void launch_nq(const DecodeConfig& c, dim3 grid, size_t lds, hipStream_t stream, const uint16_t* x, int m,
                      int64_t k, const uint8_t* codes, const uint8_t* scales, const float* ts, int64_t n,
                      const uint16_t* la, const uint16_t* lb, int r, int lparts, int lsw, uint32_t* lsync, uint16_t* y,
                      float* part, uint32_t* cnt, int nsteps, int ntiles, int scales16, const uint16_t* gam,
                      const float* noise, float sigma, float eps) {
#define FP4W_DQ(W, D)                                                                                        \
  do {                                                                                                       \
    if (r > 0)                                                                                               \
      hipLaunchKernelGGL((decode_f8f4_kernel<FMT, NQ, W, D, true, AQN>), grid, dim3(64 * W), lds, stream, x, m, \
                         k, codes, scales, ts, n, la, lb, r, lparts, lsw, lsync, y, part, cnt, c.splits, c.sps,      \
                         nsteps, ntiles, scales16, (uint64_t)lora_wait_ticks(), gam, noise, sigma, eps);         \
    else                                                                                                     \
      hipLaunchKernelGGL((decode_f8f4_kernel<FMT, NQ, W, D, false, AQN>), grid, dim3(64 * W), lds, stream, x, m, \
                         k, codes, scales, ts, n, la, lb, r, lparts, lsw, lsync, y, part, cnt, c.splits, c.sps,      \
                         nsteps, ntiles, scales16, (uint64_t)0, gam, noise, sigma, eps);                        \
  } while (0)
  if (c.nw == 4) {
    if (c.depth <= 4) FP4W_DQ(4, 4); else FP4W_DQ(4, 8);
  } else if (c.nw == 8 || (FMT == FMT_NVFP4 && NQ > 1)) {
    if (c.depth <= 4) FP4W_DQ(8, 4); else FP4W_DQ(8, 8);
  } else if constexpr (!AQN && (FMT == FMT_MXFP4 || NQ == 1)) {
    if (c.depth <= 4) FP4W_DQ(16, 4); else FP4W_DQ(16, 8);
  }
#undef FP4W_DQ
}

// The fused norm: one K slice (the row's sum of squares in one workgroup), m <= 2
// (two per-thread sums), at most 8 waves (16-wave groups would spill the gain's
// prefetched gamma and noise).
bool decode_f8f4_fuses_aqn(const DecodeConfig& c, int64_t m) {
  return m >= 1 && m <= 2 && c.splits == 1 && c.nw <= 8;
}

hipError_t launch_decode_f8f4(int fmt, const DecodeConfig& c0, const void* x, int64_t m, int64_t k,
                              const uint8_t* codes, const uint8_t* scales, const float* ts, int64_t n,
                              const void* la, const void* lb, int r, uint32_t* lsync, void* y, float* part,
                              uint32_t* cnt, hipStream_t stream, const void* aqn_gamma, const float* aqn_noise,
                              float aqn_sigma, float aqn_eps) {
  DecodeConfig c = c0;
  const int nq = fmt == FMT_NVFP4 ? (int)m : (int)((m + 7) / 8);
  if (fmt == FMT_NVFP4 && nq > 1 && c.nw > 8) c.nw = 8;   // 16-wave groups only for one chain (else they spill)
  const int blk = fmt == FMT_NVFP4 ? 16 : 32;
  const int ntiles = (int)((n + DQ_ROWS - 1) / DQ_ROWS);
  const int nsteps = (int)((k + DQ_STEP - 1) / DQ_STEP);
  const int kslice = c.sps * DQ_STEP;
  const int rr = la && lb && k > 0 ? r : 0;        // k = 0: t = x A^T is zero
  // With LoRA (wave 0's part is cut short so its wait for t overlaps the others'
  // streaming) and for NVFP4's several MFMA chains per step, the ring of 4 also
  // wins where the parts fit a ring of 8 (MI355X, m = 1, with LoRA r = 16, NVFP4:
  // 18944 x 3584 11.45 -> 11.11 us, 3584 x 3584 6.41 -> 6.23 us; m = 2: 18944 x
  // 3584 15.91 -> 13.31 us; the same outputs bit for bit)
  if (rr > 0 || (fmt == FMT_NVFP4 && m >= 2)) c.depth = 4;
  const size_t lds = decode_f8f4_lds_bytes(fmt, m, kslice, c.nw, rr);
  if (lds > 64 * 1024 || rr > DQ_MAX_R || m * rr > 1024) return hipErrorInvalidValue;
  // chunk workgroups of the LoRA down-projection go first in the grid
  const int lsw = rr > 0 ? lora_chunk_steps(c.nw, k, (int)m * rr) : kLoraStepsPerLoad;
  const int lparts = rr > 0 ? lora_chunk_count(c.nw, k, lsw) : 0;
  const dim3 grid((unsigned)(lparts + (int64_t)ntiles * c.splits));
  const int scales16 = ((reinterpret_cast<uintptr_t>(scales) & 15u) == 0 && (k / blk) % 16 == 0 &&
                        (kslice / blk) % 16 == 0) ? 1 : 0;
  const uint16_t* xx = reinterpret_cast<const uint16_t*>(x);
  const uint16_t* aa = rr > 0 ? reinterpret_cast<const uint16_t*>(la) : nullptr;
  const uint16_t* bb = reinterpret_cast<const uint16_t*>(lb);
  uint16_t* yy = reinterpret_cast<uint16_t*>(y);
  const int mm = (int)m;
  const uint16_t* gam = reinterpret_cast<const uint16_t*>(aqn_gamma);
  if (gam) {                                       // the fused noisy RMSNorm: one K slice, m <= 2
    if (!decode_f8f4_fuses_aqn(c, m) || !aqn_noise) return hipErrorInvalidValue;
    if (fmt == FMT_NVFP4 && mm == 2)
      launch_nq<FMT_NVFP4, 2, true>(c, grid, lds, stream, xx, mm, k, codes, scales, ts, n, aa, bb, rr, lparts, lsw,
                                    lsync, yy, part, cnt, nsteps, ntiles, scales16, gam, aqn_noise, aqn_sigma, aqn_eps);
    else if (fmt == FMT_NVFP4)
      launch_nq<FMT_NVFP4, 1, true>(c, grid, lds, stream, xx, mm, k, codes, scales, ts, n, aa, bb, rr, lparts, lsw,
                                    lsync, yy, part, cnt, nsteps, ntiles, scales16, gam, aqn_noise, aqn_sigma, aqn_eps);
    else
      launch_nq<FMT_MXFP4, 1, true>(c, grid, lds, stream, xx, mm, k, codes, scales, ts, n, aa, bb, rr, lparts, lsw,
                                    lsync, yy, part, cnt, nsteps, ntiles, scales16, gam, aqn_noise, aqn_sigma, aqn_eps);
    return hipSuccess;
  }
  if (fmt == FMT_NVFP4) {
    switch (mm) {
#define FP4W_NQ(Q_)                                                                                        \
  case Q_:                                                                                                 \
    launch_nq<FMT_NVFP4, Q_, false>(c, grid, lds, stream, xx, mm, k, codes, scales, ts, n, aa, bb, rr, lparts, lsw, \
                                    lsync, yy, part, cnt, nsteps, ntiles, scales16, nullptr, nullptr, 0.f, 0.f);   \
    break;
      FP4W_NQ(1) FP4W_NQ(2) FP4W_NQ(3) FP4W_NQ(4) FP4W_NQ(5) FP4W_NQ(6) FP4W_NQ(7) FP4W_NQ(8)
#undef FP4W_NQ
      default: return hipErrorInvalidValue;
    }
  } else {
    if (mm <= 8)
      launch_nq<FMT_MXFP4, 1, false>(c, grid, lds, stream, xx, mm, k, codes, scales, ts, n, aa, bb, rr, lparts, lsw,
                                     lsync, yy, part, cnt, nsteps, ntiles, scales16, nullptr, nullptr, 0.f, 0.f);
    else
      launch_nq<FMT_MXFP4, 2, false>(c, grid, lds, stream, xx, mm, k, codes, scales, ts, n, aa, bb, rr, lparts, lsw,
                                     lsync, yy, part, cnt, nsteps, ntiles, scales16, nullptr, nullptr, 0.f, 0.f);
  }
  return hipSuccess;
}

}  // namespace fp4w
