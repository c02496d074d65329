// gemm_common.hpp -- pieces shared by the MFMA GEMM kernels (gemm.hip, a4w4.hip):
// LDS chunk swizzles, DMA into LDS, wait counts, accumulator copies, and the
// once-per-device dynamic LDS limit (also used by decode_xs.hip, linear.hip).
#pragma once

#include <atomic>
#include "fp4w_device.hpp"

namespace fp4w {

// Position of chunk c of LDS row m: c ^ swz(m), swz(m) = (m ^ (m >> 3 & 1)) & 7.
// Rows m..m+7 (m a multiple of 8) get 8 distinct swizzles, and over 16 rows each
// parity class gets 8 distinct ones: a b128 access of 16 rows at one chunk, or
// of one row's 8 chunks, is conflict-free for 128- and 256-byte bank widths.
__device__ __forceinline__ int w4_swz(int m) { return (m ^ ((m >> 3) & 1)) & 7; }

// The accumulators live in AGPRs (v_mfma's AGPR form); the epilogue moves them
// through these explicit copies, because a plain VALU use of an accumulator
// made the register allocator keep some of them in VGPRs and shuffle them
// through the loop.
__device__ __forceinline__ float acc_read(float a) {
  float v;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(a));
  return v;
}
__device__ __forceinline__ float acc_write(float v) {
  float a;
  asm volatile("v_accvgpr_write_b32 %0, %1" : "=a"(a) : "v"(v));
  return a;
}

// Position of chunk c (of 4) of a 64-byte code row r: c ^ swzw(r),
// swzw(r) = ((r >> 1) ^ (r >> 3)) & 3: reads of 8 or 16 consecutive rows at one
// chunk hit distinct 16-byte slots for 128- and 256-byte bank widths.
__device__ __forceinline__ int w4_swzw(int r) { return ((r >> 1) ^ (r >> 3)) & 3; }

// s_waitcnt vmcnt(n) lgkmcnt(0) (gfx9 encoding: vmcnt split over bits 3:0 and 15:14)
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4));
}

typedef __attribute__((address_space(3))) void lds_void;
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint8_t* lds, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, off, 0, 0, 0);
}
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, uint8_t* lds, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 4, off, 0, 0, 0);
}

typedef __attribute__((ext_vector_type(16))) float f32x16_t;

// Raise `fn`'s dynamic LDS limit to `bytes` once per device: the attribute is
// per device, so `done` keeps one bit per device id (ids past 63 set it on every
// call); safe to call from several host threads.
inline hipError_t set_max_lds_once(const void* fn, int bytes, std::atomic<uint64_t>& done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = (dev >= 0 && dev < 64) ? (uint64_t)1 << dev : 0;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_acq_rel);
  return e;
}

}  // namespace fp4w
