// api.hip -- the C ABI of libfp4w.so (declared in include/fp4w.h): host-side
// argument validation, then the launchers.  Nothing here allocates, frees or
// synchronizes; every kernel goes on the caller's stream.
#include <hip/hip_runtime.h>

#include <cmath>
#include <mutex>

#include "../../include/fp4w.h"
#include "fp4w_internal.hpp"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned2(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 1u) == 0; }

bool valid_fmt(int fmt) { return fmt == FP4W_NVFP4 || fmt == FP4W_MXFP4; }

// Largest element count the kernels index with 64-bit offsets but whose grid
// strides stay well inside int64: 2^40 elements (a 2 TiB bf16 tensor).
constexpr int64_t kMaxElems = int64_t(1) << 40;

int check_nk(int64_t n, int64_t k) {
  if (n < 0 || k < 0) return FP4W_ERR_ARG;
  if (k % 32 != 0) return FP4W_ERR_SHAPE;
  if (n > 0 && k > 0 && n > kMaxElems / k) return FP4W_ERR_SHAPE;
  return FP4W_OK;
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

int hip_status(hipError_t e) { return e == hipSuccess ? FP4W_OK : FP4W_ERR_HIP; }

}  // namespace

extern "C" {

int fp4w_version(void) { return 10; }

const char* fp4w_status_string(int status) {
  switch (status) {
    case FP4W_OK: return "ok";
    case FP4W_ERR_ARG: return "invalid argument (null pointer or negative size)";
    case FP4W_ERR_SHAPE: return "invalid shape (k % 32 != 0, rank outside [0, 64] or too large)";
    case FP4W_ERR_ALIGN: return "pointer not 16-byte aligned";
    case FP4W_ERR_FORMAT: return "unknown format or flag";
    case FP4W_ERR_HIP: return "HIP kernel launch failed";
    case FP4W_ERR_WORKSPACE: return "workspace missing or too small";
    case FP4W_ERR_SCRATCH:
      return "the call needs more workspace than the no-allocation entry point's device array holds "
             "(FP4W_NOALLOC_SCRATCH_BYTES); use fp4w_linear with a workspace";
    default: return "unknown status";
  }
}

int fp4w_quantize(int fmt, const void* w_bf16, int64_t n, int64_t k, uint8_t* codes, uint8_t* scales,
                  float* tensor_scale, uint32_t flags, void* stream) {
  if (!valid_fmt(fmt) || (flags & ~FP4W_FROZEN_SCALES)) return FP4W_ERR_FORMAT;
  int st = check_nk(n, k);
  if (st) return st;
  if (n * k == 0) return FP4W_OK;
  if (!w_bf16 || !codes || !scales) return FP4W_ERR_ARG;
  if (fmt == FP4W_NVFP4 && !tensor_scale) return FP4W_ERR_ARG;
  if (!aligned16(w_bf16) || !aligned16(codes)) return FP4W_ERR_ALIGN;
  if (fmt == FP4W_NVFP4 && ((reinterpret_cast<uintptr_t>(tensor_scale) & 3u) != 0)) return FP4W_ERR_ALIGN;
  return hip_status(fp4w::launch_quantize(fmt, w_bf16, n, k, codes, scales, tensor_scale,
                                          (flags & FP4W_FROZEN_SCALES) != 0, as_stream(stream)));
}

int fp4w_fake_quant(int fmt, const void* w_bf16, int64_t n, int64_t k, void* out_bf16, uint8_t* scales,
                    float* tensor_scale, uint32_t flags, void* stream) {
  if (!valid_fmt(fmt) || (flags & ~FP4W_FROZEN_SCALES)) return FP4W_ERR_FORMAT;
  int st = check_nk(n, k);
  if (st) return st;
  if (n * k == 0) return FP4W_OK;
  if (!w_bf16 || !out_bf16 || !scales) return FP4W_ERR_ARG;
  if (fmt == FP4W_NVFP4 && !tensor_scale) return FP4W_ERR_ARG;
  if (!aligned16(w_bf16) || !aligned16(out_bf16)) return FP4W_ERR_ALIGN;
  if (fmt == FP4W_NVFP4 && ((reinterpret_cast<uintptr_t>(tensor_scale) & 3u) != 0)) return FP4W_ERR_ALIGN;
  return hip_status(fp4w::launch_fake_quant(fmt, w_bf16, n, k, out_bf16, scales, tensor_scale,
                                            (flags & FP4W_FROZEN_SCALES) != 0, as_stream(stream)));
}

int fp4w_dequantize(int fmt, const uint8_t* codes, const uint8_t* scales, const float* tensor_scale, int64_t n,
                    int64_t k, void* out, uint32_t flags, void* stream) {
  if (!valid_fmt(fmt) || (flags & ~FP4W_OUT_FP32)) return FP4W_ERR_FORMAT;
  int st = check_nk(n, k);
  if (st) return st;
  if (n * k == 0) return FP4W_OK;
  if (!codes || !scales || !out) return FP4W_ERR_ARG;
  if (fmt == FP4W_NVFP4 && !tensor_scale) return FP4W_ERR_ARG;
  if (!aligned16(codes) || !aligned16(out)) return FP4W_ERR_ALIGN;
  return hip_status(fp4w::launch_dequantize(fmt, codes, scales, tensor_scale, n, k, out,
                                            (flags & FP4W_OUT_FP32) != 0, as_stream(stream)));
}

size_t fp4w_linear_workspace_bytes(int64_t m, int64_t n, int64_t k, int r) {
  if (m < 0 || n < 0 || k < 0 || r < 0 || r > FP4W_MAX_LORA_RANK) return 0;
  return fp4w::plan_linear(m, n, k, r).bytes;
}

int64_t fp4w_debug_lora_wait(int64_t ticks) {
  return ticks < 0 ? fp4w::lora_wait_ticks() : fp4w::set_lora_wait_ticks(ticks);
}

}  // extern "C"

namespace {

// Host validation shared by fp4w_linear and fp4w_linear_noalloc: arguments,
// shapes and alignment, then the plan (kernel shape and workspace layout).
// FP4W_OK with *nothing = true when there is no work.
int linear_check(int fmt, const void* x_bf16, int64_t m, int64_t k, const uint8_t* codes, const uint8_t* scales,
                 const float* tensor_scale, int64_t n, const void* lora_a, const void* lora_b, int r, void* y_bf16,
                 bool* nothing, bool* lora, fp4w::LinearPlan* plan) {
  *nothing = false;
  if (!valid_fmt(fmt)) return FP4W_ERR_FORMAT;
  if (m < 0 || n < 0 || k < 0 || r < 0) return FP4W_ERR_ARG;
  int st = check_nk(n, k);
  if (st) return st;
  if (r > FP4W_MAX_LORA_RANK) return FP4W_ERR_SHAPE;
  if (m > 0 && k > 0 && m > kMaxElems / k) return FP4W_ERR_SHAPE;
  if (m == 0 || n == 0) {
    *nothing = true;
    return FP4W_OK;
  }
  if (!x_bf16 || !y_bf16 || (k > 0 && (!codes || !scales))) return FP4W_ERR_ARG;
  if (fmt == FP4W_NVFP4 && !tensor_scale) return FP4W_ERR_ARG;
  *lora = r > 0 && (lora_a || lora_b);
  if (*lora && (!lora_a || !lora_b)) return FP4W_ERR_ARG;
  if (!aligned16(x_bf16) || !aligned16(codes) || !aligned2(y_bf16)) return FP4W_ERR_ALIGN;
  if (fmt == FP4W_NVFP4 && !aligned2(scales)) return FP4W_ERR_ALIGN;
  if (*lora && (!aligned16(lora_a) || !aligned2(lora_b))) return FP4W_ERR_ALIGN;
  *plan = fp4w::plan_linear(m, n, k, *lora ? r : 0);
  return FP4W_OK;
}

}  // namespace

extern "C" {

int fp4w_linear(int fmt, const void* x_bf16, int64_t m, int64_t k, const uint8_t* codes, const uint8_t* scales,
                const float* tensor_scale, int64_t n, const void* lora_a, const void* lora_b, int r, void* y_bf16,
                void* workspace, size_t workspace_bytes, void* stream) {
  bool nothing = false, lora = false;
  fp4w::LinearPlan plan{};
  int st = linear_check(fmt, x_bf16, m, k, codes, scales, tensor_scale, n, lora_a, lora_b, r, y_bf16, &nothing,
                        &lora, &plan);
  if (st || nothing) return st;
  if (!workspace || workspace_bytes < plan.bytes) return FP4W_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return FP4W_ERR_ALIGN;
  return hip_status(fp4w::launch_linear(fmt, x_bf16, m, k, codes, scales, tensor_scale, n, lora ? lora_a : nullptr,
                                        lora ? lora_b : nullptr, lora ? r : 0, y_bf16, workspace, plan,
                                        as_stream(stream)));
}

size_t fp4w_linear_aqn_workspace_bytes(int64_t m, int64_t n, int64_t k, int r) {
  if (m < 0 || n < 0 || k < 0 || r < 0 || r > FP4W_MAX_LORA_RANK) return 0;
  if (m > 0 && k > 0 && m > kMaxElems / k) return 0;
  return fp4w::linear_aqn_workspace_bytes(fp4w::plan_linear(m, n, k, r), m, k);
}

int fp4w_linear_aqn(int fmt, const void* x_bf16, int64_t m, int64_t k, const void* gamma_bf16, const float* noise,
                    float sigma, float eps, const uint8_t* codes, const uint8_t* scales, const float* tensor_scale,
                    int64_t n, const void* lora_a, const void* lora_b, int r, void* y_bf16, void* workspace,
                    size_t workspace_bytes, void* stream) {
  bool nothing = false, lora = false;
  fp4w::LinearPlan plan{};
  int st = linear_check(fmt, x_bf16, m, k, codes, scales, tensor_scale, n, lora_a, lora_b, r, y_bf16, &nothing,
                        &lora, &plan);
  if (st || nothing) return st;
  if (k > 0 && (!gamma_bf16 || !noise)) return FP4W_ERR_ARG;
  if (k > 0 && (!aligned16(gamma_bf16) || !aligned16(noise))) return FP4W_ERR_ALIGN;
  if (!workspace || workspace_bytes < fp4w::linear_aqn_workspace_bytes(plan, m, k)) return FP4W_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return FP4W_ERR_ALIGN;
  return hip_status(fp4w::launch_linear_aqn(fmt, x_bf16, m, k, gamma_bf16, noise, sigma, eps, codes, scales,
                                            tensor_scale, n, lora ? lora_a : nullptr, lora ? lora_b : nullptr,
                                            lora ? r : 0, y_bf16, workspace, plan, as_stream(stream)));
}

int fp4w_linear_w4a4(int fmt, const uint8_t* x_codes, const uint8_t* x_scales, int64_t m, int64_t k,
                     const uint8_t* codes, const uint8_t* scales, int64_t n, void* y_bf16, void* stream) {
  if (fmt != FP4W_MXFP4) return FP4W_ERR_FORMAT;
  if (m < 0 || n < 0 || k < 0) return FP4W_ERR_ARG;
  if (m == 0 || n == 0) return FP4W_OK;
  if (k == 0 || !fp4w::gemm_a4w4_supports(m, n, k)) return FP4W_ERR_SHAPE;
  if (!x_codes || !x_scales || !codes || !scales || !y_bf16) return FP4W_ERR_ARG;
  if (!aligned16(x_codes) || !aligned16(codes) || !aligned2(y_bf16)) return FP4W_ERR_ALIGN;
  if (((reinterpret_cast<uintptr_t>(x_scales) | reinterpret_cast<uintptr_t>(scales)) & 3u) != 0)
    return FP4W_ERR_ALIGN;
  return hip_status(fp4w::launch_gemm_a4w4(x_codes, x_scales, m, k, codes, scales, n, y_bf16, as_stream(stream)));
}

int fp4w_linear_backward_dx(int fmt, const void* dy_bf16, int64_t m, int64_t n, const uint8_t* codes,
                            const uint8_t* scales, const float* tensor_scale, int64_t k, const float* lora_u,
                            const void* lora_a, int r, void* dx_bf16, void* stream) {
  if (!valid_fmt(fmt)) return FP4W_ERR_FORMAT;
  if (m < 0 || n < 0 || k < 0 || r < 0) return FP4W_ERR_ARG;
  int st = check_nk(n, k);
  if (st) return st;
  if (n % 8 != 0 || m > ((int64_t)65535 * 128) || n > 0x7FFFFFFF || k > 0x7FFFFFFF) return FP4W_ERR_SHAPE;
  if (r > FP4W_MAX_LORA_RANK) return FP4W_ERR_SHAPE;
  if (m > 0 && n > kMaxElems / (m > 0 ? m : 1)) return FP4W_ERR_SHAPE;
  if (m == 0 || k == 0) return FP4W_OK;
  if (!dx_bf16 || (n > 0 && (!dy_bf16 || !codes || !scales))) return FP4W_ERR_ARG;
  if (fmt == FP4W_NVFP4 && !tensor_scale) return FP4W_ERR_ARG;
  const bool lora = r > 0 && (lora_u || lora_a);
  if (lora && (!lora_u || !lora_a)) return FP4W_ERR_ARG;
  if (!aligned16(dy_bf16) || !aligned16(codes) || (reinterpret_cast<uintptr_t>(dx_bf16) & 7u) != 0)
    return FP4W_ERR_ALIGN;
  if (lora && (((reinterpret_cast<uintptr_t>(lora_u) & 3u) != 0) || !aligned2(lora_a))) return FP4W_ERR_ALIGN;
  return hip_status(fp4w::launch_backward_dx(fmt, dy_bf16, m, n, codes, scales, tensor_scale, k, dx_bf16,
                                             lora ? lora_u : nullptr, lora ? lora_a : nullptr, lora ? r : 0,
                                             as_stream(stream)));
}

size_t fp4w_lora_backward_workspace_bytes(int64_t m, int64_t n, int64_t k, int r) {
  if (m < 0 || n < 0 || k < 0 || r < 1 || r > FP4W_MAX_LORA_RANK) return 0;
  if ((m > 0 && (n > kMaxElems / m || k > kMaxElems / m))) return 0;
  return fp4w::lora_backward_workspace_bytes(m, n, k, r);
}

int fp4w_lora_backward(const void* dy_bf16, int64_t m, int64_t n, const void* x_bf16, int64_t k,
                       const void* lora_a, const void* lora_b, int r, float* u, float* grad_a, float* grad_b,
                       void* workspace, size_t workspace_bytes, void* stream) {
  if (m < 0 || n < 0 || k < 0 || r < 0) return FP4W_ERR_ARG;
  if (r < 1 || r > FP4W_MAX_LORA_RANK || k % 32 != 0 || n % 8 != 0) return FP4W_ERR_SHAPE;
  if (m > 0 && (n > kMaxElems / m || k > kMaxElems / m)) return FP4W_ERR_SHAPE;
  if (n > kMaxElems / r || k > kMaxElems / r) return FP4W_ERR_SHAPE;
  if ((m > 0 && ((n > 0 && !dy_bf16) || (k > 0 && !x_bf16))) || (k > 0 && !lora_a) || (n > 0 && !lora_b))
    return FP4W_ERR_ARG;
  if (!aligned16(dy_bf16) || !aligned16(x_bf16) || !aligned16(lora_a) || !aligned2(lora_b)) return FP4W_ERR_ALIGN;
  if (((reinterpret_cast<uintptr_t>(u) | reinterpret_cast<uintptr_t>(grad_a) | reinterpret_cast<uintptr_t>(grad_b)) &
       3u) != 0)
    return FP4W_ERR_ALIGN;
  const size_t need = fp4w::lora_backward_workspace_bytes(m, n, k, r);
  if (!workspace || workspace_bytes < need) return FP4W_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return FP4W_ERR_ALIGN;
  return hip_status(fp4w::launch_lora_backward(dy_bf16, m, n, x_bf16, k, lora_a, lora_b, r, u, grad_a, grad_b,
                                               workspace, as_stream(stream)));
}

int fp4w_scale_delta_grad(int fmt, const void* dy_bf16, const void* x_bf16, int64_t m, int64_t n, int64_t k,
                          const uint8_t* codes, const float* tensor_scale, float* grad, void* stream) {
  if (!valid_fmt(fmt)) return FP4W_ERR_FORMAT;
  if (m < 0 || n < 0 || k < 0) return FP4W_ERR_ARG;
  int st = check_nk(n, k);
  if (st) return st;
  if (n % 8 != 0 || n > (int64_t)65535 * 128 || m > 0x7FFFFFFF || k > 0x7FFFFFFF) return FP4W_ERR_SHAPE;
  if (m > 0 && (n > kMaxElems / m || k > kMaxElems / m)) return FP4W_ERR_SHAPE;
  if (n == 0 || k == 0) return FP4W_OK;
  if (!codes || !grad || (m > 0 && (!dy_bf16 || !x_bf16))) return FP4W_ERR_ARG;
  if (fmt == FP4W_NVFP4 && !tensor_scale) return FP4W_ERR_ARG;
  if (!aligned16(dy_bf16) || !aligned16(x_bf16) || !aligned16(codes) ||
      (reinterpret_cast<uintptr_t>(grad) & 3u) != 0)
    return FP4W_ERR_ALIGN;
  return hip_status(fp4w::launch_delta_grad(fmt, dy_bf16, x_bf16, m, n, k, codes, tensor_scale, grad,
                                            as_stream(stream)));
}

double fp4w_aqn_sigma(int64_t step, int64_t total_steps, double sigma_max, double sigma_min) {
  if (!(sigma_max > 0.0) || !(sigma_min > 0.0)) return 0.0;
  if (total_steps <= 0 || step >= total_steps) return sigma_min;
  if (step <= 0) return sigma_max;
  return sigma_max * std::pow(sigma_min / sigma_max, (double)step / (double)total_steps);
}

int fp4w_aqn_rmsnorm(const void* x_bf16, int64_t m, int64_t k, const void* gamma_bf16, const float* noise,
                     float sigma, float eps, void* y_bf16, void* stream) {
  if (m < 0 || k < 0) return FP4W_ERR_ARG;
  if (k % 8 != 0 || m > 0x7FFFFFFF || (m > 0 && k > kMaxElems / m)) return FP4W_ERR_SHAPE;
  if (m == 0 || k == 0) return FP4W_OK;
  if (!x_bf16 || !gamma_bf16 || !noise || !y_bf16) return FP4W_ERR_ARG;
  if (!aligned16(x_bf16) || !aligned16(gamma_bf16) || !aligned16(noise) || !aligned16(y_bf16)) return FP4W_ERR_ALIGN;
  return hip_status(fp4w::launch_aqn_rmsnorm(x_bf16, m, k, gamma_bf16, noise, sigma, eps, y_bf16, as_stream(stream)));
}

int fp4w_grouped_linear(int fmt, const void* x_bf16, int64_t num_tokens, const int32_t* row_index,
                        const int32_t* expert_offsets, int64_t num_experts, int64_t total_rows, int64_t n,
                        int64_t k, const uint8_t* codes, const uint8_t* scales, const float* tensor_scales,
                        void* y_bf16, void* stream) {
  if (!valid_fmt(fmt)) return FP4W_ERR_FORMAT;
  if (num_tokens < 0 || num_experts < 0 || total_rows < 0) return FP4W_ERR_ARG;
  int st = check_nk(n, k);
  if (st) return st;
  if (num_experts > 0 && n > 0 && k > 0 && num_experts > kMaxElems / (n * k)) return FP4W_ERR_SHAPE;
  if (num_experts == 0 || total_rows == 0 || n == 0) return FP4W_OK;
  if (!x_bf16 || !row_index || !expert_offsets || !y_bf16 || (k > 0 && (!codes || !scales))) return FP4W_ERR_ARG;
  if (fmt == FP4W_NVFP4 && !tensor_scales) return FP4W_ERR_ARG;
  if (!aligned16(x_bf16) || !aligned16(codes) || !aligned2(y_bf16)) return FP4W_ERR_ALIGN;
  if (fmt == FP4W_NVFP4 && !aligned2(scales)) return FP4W_ERR_ALIGN;
  if (num_experts * ((n + 15) / 16) > 0x7FFFFFFF) return FP4W_ERR_SHAPE;
  return hip_status(fp4w::launch_grouped_linear(fmt, x_bf16, num_tokens, row_index, expert_offsets, num_experts,
                                                total_rows, n, k, codes, scales, tensor_scales, y_bf16,
                                                as_stream(stream)));
}

int fp4w_merge_scales(int fmt, const uint8_t* scales_in, const float* deltas, int64_t num_blocks,
                      uint8_t* scales_out, const uint8_t* codes_in, uint8_t* codes_out, int64_t code_bytes,
                      void* stream) {
  if (!valid_fmt(fmt)) return FP4W_ERR_FORMAT;
  if (num_blocks < 0 || code_bytes < 0) return FP4W_ERR_ARG;
  if (num_blocks > 0 && (!scales_in || !deltas || !scales_out)) return FP4W_ERR_ARG;
  const bool copy = codes_in && codes_out && codes_in != codes_out && code_bytes > 0;
  if (copy && (!aligned16(codes_in) || !aligned16(codes_out))) return FP4W_ERR_ALIGN;
  if (num_blocks > kMaxElems || code_bytes > kMaxElems) return FP4W_ERR_SHAPE;
  if (num_blocks == 0 && !copy) return FP4W_OK;
  return hip_status(fp4w::launch_merge_scales(fmt, scales_in, deltas, num_blocks, scales_out, codes_in, codes_out,
                                              code_bytes, as_stream(stream)));
}

}  // extern "C"

// ---------------------------------------------------------------------------------
// fp4w_linear_noalloc: fp4w_linear with its workspace in a library-owned device
// array instead of a caller's buffer, for callers that cannot allocate.
//
// `scratch` is one array per device (each device that loads the library holds
// its own copy until the process ends).  In host code its name is only a
// host-side stand-in, so it is never passed to a kernel: at the first call on a
// device (with that device current) hipGetSymbolAddress gives that device's
// address, which is kept per device and used for every launch.  The first 28800
// bytes hold the linear's arrival counters and LoRA hand-over words, which must
// be zero before a call; every call returns them to zero, and the set-up clears
// them once with a fill kernel on the caller's stream.  All calls on one device
// share the array: calls that overlap in time on one device race.
// ---------------------------------------------------------------------------------
__device__ __align__(256) uint8_t scratch[FP4W_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

__global__ void zero_words_kernel(uint32_t* __restrict__ p, int words) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < words; i += gridDim.x * blockDim.x) p[i] = 0u;
}

// This device's address of `scratch`, set up on the first call on the device.
int device_scratch(hipStream_t stream, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FP4W_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return FP4W_ERR_HIP;
    const int words = fp4w::kCounterSlots;
    hipLaunchKernelGGL(zero_words_kernel, dim3((words + 255) / 256), dim3(256), 0, stream,
                       reinterpret_cast<uint32_t*>(p), words);
    if (hipGetLastError() != hipSuccess) return FP4W_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return FP4W_OK;
}

}  // namespace

extern "C" int fp4w_linear_noalloc(int fmt, const void* x_bf16, int64_t m, int64_t k, const uint8_t* codes,
                                   const uint8_t* scales, const float* tensor_scale, int64_t n, const void* lora_a,
                                   const void* lora_b, int r, void* y_bf16, void* stream) {
  bool nothing = false, lora = false;
  fp4w::LinearPlan plan{};
  int st = linear_check(fmt, x_bf16, m, k, codes, scales, tensor_scale, n, lora_a, lora_b, r, y_bf16, &nothing,
                        &lora, &plan);
  if (st || nothing) return st;
  if (plan.bytes > (size_t)FP4W_NOALLOC_SCRATCH_BYTES) return FP4W_ERR_SCRATCH;
  void* ws = nullptr;
  st = device_scratch(as_stream(stream), &ws);
  if (st) return st;
  return hip_status(fp4w::launch_linear(fmt, x_bf16, m, k, codes, scales, tensor_scale, n, lora ? lora_a : nullptr,
                                        lora ? lora_b : nullptr, lora ? r : 0, y_bf16, ws, plan,
                                        as_stream(stream)));
}
