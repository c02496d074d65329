// sync.hpp -- ordered cross-workgroup sums on gfx950 without L2-wide fences.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4w {

// ---------------------------------------------------------------------------------
// Cross-workgroup partial sums.  Partials are stored and loaded as relaxed
// agent-scope atomics: on gfx950 these are emitted with the SC1 bit, which makes
// them coherent across the XCDs' separate L2s without an L2-wide writeback or
// invalidate (a __threadfence() costs both, on every workgroup).  The writer
// waits for its stores to complete (s_waitcnt) before it increments the arrival
// counter, and the reader issues its loads only after the increment returned,
// so the last arrival sees every partial.
// ---------------------------------------------------------------------------------
__device__ __forceinline__ void store_agent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_agent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wait_stores_complete() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Workgroup version: every thread calls it after storing its partials; returns
// true in all threads of the last workgroup to arrive (which resets the counter).
__device__ __forceinline__ bool arrive_last(uint32_t* cnt, uint32_t expected, int* flag_lds) {
  wait_stores_complete();
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t old = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    bool last = old == expected - 1u;
    if (last) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *flag_lds = last ? 1 : 0;
  }
  __syncthreads();
  return *flag_lds != 0;
}

// Wave version: every lane calls it after storing its partials.
__device__ __forceinline__ bool wave_arrive_last(uint32_t* cnt, uint32_t expected, int lane) {
  wait_stores_complete();
  uint32_t old = 0;
  if (lane == 0) {
    old = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old == expected - 1u) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  old = (uint32_t)__shfl((int)old, 0, 64);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  return old == expected - 1u;
}

}  // namespace fp4w
