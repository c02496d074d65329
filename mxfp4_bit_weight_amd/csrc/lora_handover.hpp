// lora_handover.hpp -- the LoRA down-projection t = x A^T formed inside a decode
// launch and handed from the workgroups that form it to the ones that write
// outputs.
//
// The pages put a LoRA adapter in parallel to the frozen 4-bit base (QLoRA-style;
// tggo.me/sberlogasci/42740, section "Metod"): y = x deq(W)^T + (x A^T) B^T.  A
// decode kernel needs t only when a tile's outputs are written, after its codes
// have streamed, so t is formed in the same launch instead of a launch of its own:
//
//  - the grid's first `lparts` workgroups ("chunk workgroups") stream no codes;
//    workgroup p forms the partial of K chunk p on v_mfma_f32_16x16x32_bf16, each
//    wave a run of `lsw` 32-wide steps (x rows as A, rows of the LoRA A as B),
//    the waves' results added in wave order in LDS, and stores it complemented in
//    the chunk words, so that a zero word reads as "not yet written";
//  - a workgroup that writes outputs polls the chunk words with a bounded wait and
//    adds them in chunk order; were the wait ever to run out, it forms the chunks
//    itself by the same steps in the same order, so the value does not depend on
//    timing.  The chunk workgroups wait on nothing, so the wait ends;
//  - the words return to zero before the kernel ends: readers arrive on 32
//    counters a cache line apart, each completed group and each chunk workgroup
//    (after its stores have landed) on one more, and the arrival that completes
//    it clears the words and itself.
// The words live in the workspace's zero-invariant counter area (kLsync*).
#pragma once
#include "fp4w_device.hpp"
#include "fp4w_internal.hpp"
#include "sync.hpp"

namespace fp4w {

constexpr int kLoraStepsPerLoad = 4;   // 32-wide K steps per round of loads of a chunk wave

__device__ __forceinline__ uint32_t lsync_load(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void lsync_store(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t lsync_add(uint32_t* p) {
  return __hip_atomic_fetch_add(p, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One wave: an arrival on the top counter, which expects one arrival per reader
// group and per chunk; the arrival that completes it clears the `words` chunk
// words and the counter.
__device__ __forceinline__ void lsync_top_arrive(uint32_t* ls, uint32_t expected, int words, int lane) {
  uint32_t old = 0;
  if (lane == 0) old = lsync_add(&ls[kLsyncTop]);
  old = (uint32_t)__shfl((int)old, 0, 64);
  if (old == expected - 1u) {
    for (int e = lane; e < words; e += 64) lsync_store(&ls[e], 0u);
    if (lane == 0) lsync_store(&ls[kLsyncTop], 0u);
  }
}

__device__ __forceinline__ uint32_t lsync_top_expected(int nread, int lparts) {
  return (uint32_t)((nread < kLsyncSubs ? nread : kLsyncSubs) + lparts);
}

// The arrival of reader workgroup `rd` of `nread`, in two parts so that the
// returning atomic's round trip overlaps the reader's remaining work.  Issue: one
// wave, once its loads of the chunk words have returned; returns the group
// count before it (in lane 0).  Complete: the same wave, later but before the
// workgroup can exit; the arrival that completes its group clears the group's
// counter and arrives on top.
__device__ __forceinline__ uint32_t lsync_reader_issue(uint32_t* ls, int rd, int lane) {
  uint32_t old = 0;
  if (lane == 0) old = lsync_add(&ls[kLsyncSub + 32 * (rd % kLsyncSubs)]);
  return old;
}
__device__ __forceinline__ void lsync_reader_complete(uint32_t* ls, uint32_t old, int rd, int nread, int lparts,
                                                      int words, int lane) {
  const int c = rd % kLsyncSubs;
  const uint32_t quota = (uint32_t)(nread / kLsyncSubs + (c < nread % kLsyncSubs ? 1 : 0));
  if (lane == 0 && old == quota - 1u) lsync_store(&ls[kLsyncSub + 32 * c], 0u);
  old = (uint32_t)__shfl((int)old, 0, 64);
  if (old == quota - 1u) lsync_top_arrive(ls, lsync_top_expected(nread, lparts), words, lane);
}

// With a gain (the fused noisy RMSNorm), x enters as bf16(x * g), g = gamma (1 + sigma
// noise), exactly as the workgroups that stream the codes form it (xgain_bf16).
struct XGain {
  const uint16_t* gamma;    // (K) bf16, or nullptr: no gain
  const float* noise;       // (K) fp32
  float sigma;
};

// bf16(x * gamma (1 + sigma noise)) of the 8 elements of v at k .. k + 7, with
// gamma's 8 bf16 in gv and noise's 8 fp32 in n0, n1; also adds x^2 to *ss.
__device__ __forceinline__ u32x4_t xgain_bf16(u32x4_t v, u32x4_t gv, u32x4_t n0, u32x4_t n1, float sigma,
                                             float* ss) {
  u32x4_t o;
#pragma unroll
  for (int d = 0; d < 4; d++) {
    const float x0 = bf16lo_f32(v[d]), x1 = bf16hi_f32(v[d]);
    const float nz0 = __uint_as_float(d < 2 ? n0[2 * d] : n1[2 * d - 4]);
    const float nz1 = __uint_as_float(d < 2 ? n0[2 * d + 1] : n1[2 * d - 3]);
    const float g0 = bf16lo_f32(gv[d]) * __builtin_fmaf(sigma, nz0, 1.0f);
    const float g1 = bf16hi_f32(gv[d]) * __builtin_fmaf(sigma, nz1, 1.0f);
    if (ss) *ss = bf16x2_sumsq(v[d], *ss);
    o[d] = f32x2_to_bf16x2_rne(x0 * g0, x1 * g1);
  }
  return o;
}

// Wave `wave` of `nw` forms its share of chunk p into lr[wave][m][j] (m < M rows of
// x (M, K) row-major, j < r rows of A (r, K)): 32-wide steps (p nw + wave) lsw ..
// + lsw - 1, column block b of 16 rows of A at a time; lane (j, g) of the MFMA
// result holds rows m = 4 g + i.
__device__ __forceinline__ void lora_chunk_to_lds(float* lr, const uint16_t* __restrict__ x, int M, int64_t K,
                                                  const uint16_t* __restrict__ lora_a, int r, int p, int nw,
                                                  int wave, int lane, int lsw, XGain xg = XGain{nullptr, nullptr, 0.f}) {
  const int li = lane & 15, lg = lane >> 4;
  const int64_t st0 = ((int64_t)p * nw + wave) * lsw;
  for (int b = 0; b < (r + 15) / 16; b++) {
    const int j = 16 * b + li;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    for (int i0 = 0; i0 < lsw; i0 += kLoraStepsPerLoad) {
      u32x4_t xa[kLoraStepsPerLoad], av[kLoraStepsPerLoad];
#pragma unroll
      for (int i = 0; i < kLoraStepsPerLoad; i++) {
        const int64_t kk = (st0 + i0 + i) * 32 + 8 * lg;
        const bool okx = li < M && kk < K, oka = j < r && kk < K;
        xa[i] = load16(x + (okx ? (int64_t)li * K + kk : 0));
        av[i] = load16(lora_a + (oka ? (int64_t)j * K + kk : 0));
        if (xg.gamma) {
          const u32x4_t gv = load16(xg.gamma + (okx ? kk : 0));
          const u32x4_t n0 = load16(xg.noise + (okx ? kk : 0)), n1 = load16(xg.noise + (okx ? kk + 4 : 0));
          xa[i] = xgain_bf16(xa[i], gv, n0, n1, xg.sigma, nullptr);
        }
        if (!okx) xa[i] = (u32x4_t){0u, 0u, 0u, 0u};
        if (!oka) av[i] = (u32x4_t){0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int i = 0; i < kLoraStepsPerLoad; i++)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xa[i]), as_bf16x8(av[i]), acc, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int m = 4 * lg + i;
      if (m < M && j < r) lr[(wave * M + m) * r + j] = acc[i];
    }
  }
}

// The chunk's value at e = m r + j: its waves added in wave order (after a barrier
// that follows lora_chunk_to_lds).
__device__ __forceinline__ float lora_chunk_value(const float* lr, int e, int nw, int mr) {
  float v = 0.f;
  for (int w = 0; w < nw; w++) v += lr[w * mr + e];
  return v;
}

// A chunk workgroup (all threads): forms chunk p, stores it, arrives.
__device__ __forceinline__ void lora_chunk_publish(float* lr, const uint16_t* __restrict__ x, int M, int64_t K,
                                                   const uint16_t* __restrict__ lora_a, int r, int p, int nw,
                                                   int lsw, uint32_t* lsync, int nread, int lparts,
                                                   XGain xg = XGain{nullptr, nullptr, 0.f}) {
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int mr = M * r;
  lora_chunk_to_lds(lr, x, M, K, lora_a, r, p, nw, wave, lane, lsw, xg);
  __syncthreads();
  if (wave == 0) {
    for (int e = lane; e < mr; e += 64) lsync_store(&lsync[p * mr + e], ~__float_as_uint(lora_chunk_value(lr, e, nw, mr)));
    wait_stores_complete();
    lsync_top_arrive(lsync, lsync_top_expected(nread, lparts), lparts * mr, lane);
  }
}

// One wave of a reader: t[e] for e < M r into lt (the chunk words added in chunk
// order), polling until every word is written or `wait_ticks` of the 100 MHz
// clock have passed.  Returns whether t is complete.
__device__ __forceinline__ int lora_poll(const uint32_t* lsync, int lparts, int mr, float* lt, uint64_t wait_ticks,
                                         int lane) {
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  int ok;
  for (;;) {
    int mine = 1;
    for (int q = lane; q < mr; q += 64) {
      float t = 0.f;
      for (int p0 = 0; p0 < lparts; p0 += 8) {
        uint32_t w[8];
#pragma unroll
        for (int i = 0; i < 8; i++) w[i] = p0 + i < lparts ? lsync_load(&lsync[(p0 + i) * mr + q]) : ~0u;
#pragma unroll
        for (int i = 0; i < 8; i++) {
          if (w[i] == 0u) mine = 0;
          if (p0 + i < lparts) t += __uint_as_float(~w[i]);
        }
      }
      lt[q] = t;
    }
    ok = __all(mine);
    if (ok || __builtin_amdgcn_s_memrealtime() - t0 >= wait_ticks) break;
    __builtin_amdgcn_s_sleep(8);
  }
  return ok;
}

// The whole workgroup, when the wait ran out: t into lt by the chunk workgroups'
// steps in their order (the same value bit for bit).
__device__ __forceinline__ void lora_form_all(float* lr, float* lt, const uint16_t* __restrict__ x, int M,
                                              int64_t K, const uint16_t* __restrict__ lora_a, int r, int nw, int lsw,
                                              int lparts, XGain xg = XGain{nullptr, nullptr, 0.f}) {
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int mr = M * r;
  if (wave == 0)
    for (int q = lane; q < mr; q += 64) lt[q] = 0.f;
  for (int p = 0; p < lparts; p++) {
    lora_chunk_to_lds(lr, x, M, K, lora_a, r, p, nw, wave, lane, lsw, xg);
    __syncthreads();
    if (wave == 0)
      for (int q = lane; q < mr; q += 64) lt[q] += lora_chunk_value(lr, q, nw, mr);
    __syncthreads();
  }
}

// Host: steps per chunk wave (a multiple of kLoraStepsPerLoad, more when the
// chunk words of mr = M r each would not fit the hand-over area) and the chunk
// count.
inline int lora_chunk_steps(int nw, int64_t k, int mr) {
  const int64_t nsteps = (k + 31) / 32;
  int64_t lsw = kLoraStepsPerLoad;
  while ((nsteps + lsw * nw - 1) / (lsw * nw) * mr > kLsyncWords) lsw += kLoraStepsPerLoad;
  return (int)lsw;
}
inline int lora_chunk_count(int nw, int64_t k, int lsw) {
  return (int)(((k + 31) / 32 + (int64_t)lsw * nw - 1) / ((int64_t)lsw * nw));
}

}  // namespace fp4w
