// membench.hip -- measurement references for the benchmark (libfp4w_membench.so),
// not part of the W4A16 path and not behind include/fp4w.h:
//  - fp4w_membench_read: a plain streaming read of `bytes` bytes (16-byte loads,
//    256-thread workgroups, a grid-stride loop), the ceiling a memory-bound
//    launch of that size can reach on this chip (launch ramp, first-load
//    latency and drain included);
//  - fp4w_membench_clock: the shader clock, from the cycle counter (s_memtime)
//    against the constant 100 MHz counter (s_memrealtime) over about 50 us.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                          uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) {
    const u32x4 v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  // the loaded bytes feed a store that almost never happens, so the loads stay
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

// One wave: spin until the 100 MHz counter has advanced `ticks` (or a hard cap
// of iterations has passed), then report both counters' advance.
__global__ __launch_bounds__(64) void clock_probe_kernel(int64_t ticks, uint64_t* __restrict__ out) {
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  const uint64_t c0 = __builtin_amdgcn_s_memtime();
  uint64_t r1 = r0, c1 = c0;
  for (int it = 0; it < (1 << 26); it++) {
    r1 = __builtin_amdgcn_s_memrealtime();
    c1 = __builtin_amdgcn_s_memtime();
    if ((int64_t)(r1 - r0) >= ticks) break;
  }
  if (threadIdx.x == 0) {
    out[0] = c1 - c0;
    out[1] = r1 - r0;
  }
}

}  // namespace

extern "C" {

// Reads bytes (a multiple of 16, src 16-byte aligned) with `blocks` workgroups of
// 256 threads; sink: one device word.  Returns 0, or -1 for bad arguments, -5 when
// the launch fails.
int fp4w_membench_read(const void* src, int64_t bytes, int blocks, uint32_t* sink, void* stream) {
  if (!src || !sink || bytes <= 0 || bytes % 16 != 0 || blocks <= 0 ||
      (reinterpret_cast<uintptr_t>(src) & 15u) != 0)
    return -1;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                     reinterpret_cast<const u32x4*>(src), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

// out: two device uint64 words (shader cycles, 100 MHz ticks); ticks in [1, 10^6].
int fp4w_membench_clock(int64_t ticks, uint64_t* out, void* stream) {
  if (!out || ticks < 1 || ticks > 1000000) return -1;
  hipLaunchKernelGGL(clock_probe_kernel, dim3(1), dim3(64), 0, reinterpret_cast<hipStream_t>(stream), ticks, out);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

}  // extern "C"
