// fp4w_internal.hpp -- launchers the C ABI (api.hip) calls; one per kernel family.
// Shapes and pointers are validated by the caller before any launcher runs.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fp4w {

hipError_t launch_quantize(int fmt, const void* w, int64_t n, int64_t k, uint8_t* codes, uint8_t* scales,
                           float* tensor_scale, bool frozen, hipStream_t stream);
hipError_t launch_fake_quant(int fmt, const void* w, int64_t n, int64_t k, void* out, uint8_t* scales,
                             float* tensor_scale, bool frozen, hipStream_t stream);

hipError_t launch_dequantize(int fmt, const uint8_t* codes, const uint8_t* scales, const float* tensor_scale,
                             int64_t n, int64_t k, void* out, bool out_fp32, hipStream_t stream);

hipError_t launch_merge_scales(int fmt, const uint8_t* scales_in, const float* deltas, int64_t num_blocks,
                               uint8_t* scales_out, const uint8_t* codes_in, uint8_t* codes_out,
                               int64_t code_bytes, hipStream_t stream);

// Linear (dense).  The plan fixes the kernel shape and the workspace layout:
//   [counters: kCounterSlots u32, fixed][t: m x r fp32][t partials][split-K partials]
// The counter area sits at a fixed offset for every shape and every word of it
// is zero between calls (a call returns what it used to zero), so whatever the
// previous call's shape, the next one finds it cleared.  Slots:
//   [0, kLoraSlots)            arrival counters of the LoRA down-projection's m-tiles
//   [kLoraSlots, kTileBase + kTileSlots)  the decode kernels' weight tiles
//   [kLsyncBase, kCounterSlots) the block-scaled decode kernel's LoRA hand-over:
//       the chunk partials of t (up to kLsyncWords, stored complemented so that
//       zero means "not yet written"), and arrival counters: one per 128-byte
//       line for the workgroups that read them (kLsyncSubs), one on top.
constexpr int kLoraSlots = 16;
constexpr int kTileBase = kLoraSlots;
constexpr int kTileSlots = 2048 - kLoraSlots;
constexpr int kLsyncBase = 2048;
constexpr int kLsyncWords = 4096;       // chunk partials: chunks x m x r
constexpr int kLsyncTop = kLsyncWords;  // completed reader groups, then producers
constexpr int kLsyncSub = kLsyncTop + 32;
constexpr int kLsyncSubs = 32;          // reader arrivals, group c at kLsyncSub + 32 c
constexpr int kLsyncSlots = kLsyncSub + 32 * kLsyncSubs;
constexpr int kCounterSlots = kLsyncBase + kLsyncSlots;

// Decode kernel on the block-scaled matrix core (decode.hip): a workgroup of
// `nw` waves per tile of 16 weight rows, `splits` slices of K of `sps`
// 128-wide steps, a ring of `depth` code loads per wave.
struct DecodeConfig {
  int nw;
  int splits;
  int sps;
  int depth;
};
bool decode_f8f4_supports(int fmt, int64_t m);
DecodeConfig plan_decode_f8f4(int fmt, int64_t m, int64_t n, int64_t k, int r);
size_t decode_f8f4_lds_bytes(int fmt, int64_t m, int kslice, int nw, int r);
// bound on the decode kernel's wait for the published t (ticks of the 100 MHz clock)
int64_t lora_wait_ticks();
int64_t set_lora_wait_ticks(int64_t ticks);      // returns the previous bound
// la / lb: LoRA A (r x k bf16) and B (n x r bf16), or nullptr (no LoRA); the
// kernel forms t = x A^T itself (K chunks in workgroups of their own, handed
// over through lsync: the kLsyncSlots words of the counter area from kLsyncBase)
// aqn_gamma non-null: the noisy RMSNorm fused into the x staging (one K slice, m <= 2;
// decode_f8f4_fuses_aqn): x enters as bf16(x gamma (1 + sigma noise)), the row factor
// 1 / sqrt(mean x^2 + eps) multiplies the fp32 sums.
bool decode_f8f4_fuses_aqn(const DecodeConfig& c, int64_t m);
hipError_t launch_decode_f8f4(int fmt, const DecodeConfig& c, const void* x, int64_t m, int64_t k,
                              const uint8_t* codes, const uint8_t* scales, const float* ts, int64_t n,
                              const void* la, const void* lb, int r, uint32_t* lsync, void* y, float* part,
                              uint32_t* cnt, hipStream_t stream, const void* aqn_gamma = nullptr,
                              const float* aqn_noise = nullptr, float aqn_sigma = 0.f, float aqn_eps = 0.f);

// Decode kernel with x held in registers (decode_xs.hip): K in `splits` spans of
// `qspan` 32-wide groups, `nw` waves per workgroup, weight tiles of 16 rows.
struct XsConfig {
  int nw;
  int splits;
  int qspan;
  int ntiles;
};
bool decode_xs_supports(int64_t m, int64_t n, int64_t k, int r);
XsConfig plan_decode_xs(int64_t m, int64_t n, int64_t k, int r);
// LoRA operands: la = A (r x k bf16) and lb = B (n x r bf16), or nullptr (no
// LoRA); the kernel forms t = x A^T itself (lora_handover.hpp, through lsync).
// aqn_gamma (bf16, K) and aqn_noise (fp32, K), or nullptr: the noisy RMSNorm of x
// fused ahead of the product (one K span only: decode_xs_fuses_aqn).
hipError_t launch_decode_xs(int fmt, const XsConfig& c, const void* x, int64_t m, int64_t k, const uint8_t* codes,
                            const uint8_t* scales, const float* ts, int64_t n, const void* la, const void* lb, int r,
                            uint32_t* lsync, void* y, float* part, uint32_t* cnt, hipStream_t stream,
                            const void* aqn_gamma = nullptr, const float* aqn_noise = nullptr, float aqn_sigma = 0.f,
                            float aqn_eps = 0.f);
bool decode_xs_fuses_aqn(int fmt, const XsConfig& c, int64_t m, int64_t k, int r, const uint8_t* scales);

struct LinearPlan {
  int path;            // 0 = decode on the block-scaled MFMA, 2 = decode on bf16 MFMA, 1 = GEMM,
                       // 3 = decode with x in registers, 4 = k == 0 (y is the empty sum: zeros)
  DecodeConfig dq;     // path 0
  XsConfig xs;         // path 3
  int splits;          // K splits of the decode kernel (1 = none)
  int lora_parts;      // K slices of the LoRA down-projection (0 = no LoRA)
  size_t off_t;        // workspace offset of t partials: [lora_parts][m][r] fp32
  size_t off_part;     // workspace offset of split-K partials (fp32)
  size_t off_count;    // workspace offset of per-row-tile arrival counters: [n/16] u32
  size_t bytes;        // total workspace bytes
};
LinearPlan plan_linear(int64_t m, int64_t n, int64_t k, int r);

hipError_t launch_linear(int fmt, const void* x, int64_t m, int64_t k, const uint8_t* codes,
                         const uint8_t* scales, const float* tensor_scale, int64_t n, const void* lora_a,
                         const void* lora_b, int r, void* y, void* workspace, const LinearPlan& plan,
                         hipStream_t stream);

// The linear of the noisy RMSNorm of x (aqn.hip's prologue): fused into the decode
// kernel where it takes one K slice at m <= 2, else the norm into the workspace
// after the linear's own bytes (m x k bf16 at align256(plan.bytes)), then the linear.
size_t linear_aqn_workspace_bytes(const LinearPlan& plan, int64_t m, int64_t k);
hipError_t launch_linear_aqn(int fmt, const void* x, int64_t m, int64_t k, const void* gamma, const float* noise,
                             float sigma, float eps, const uint8_t* codes, const uint8_t* scales,
                             const float* tensor_scale, int64_t n, const void* lora_a, const void* lora_b, int r,
                             void* y, void* workspace, const LinearPlan& plan, hipStream_t stream);

// The m > 16 GEMM with W decoded in registers (gemm.hip): K a multiple of 128,
// x and the codes below 2 GiB each, scales 16-byte aligned; t = x A^T (fp32,
// m x r) formed beforehand.
bool gemm_w4_supports(int64_t m, int64_t n, int64_t k, const void* scales);
hipError_t launch_gemm_w4(int fmt, const void* x, int64_t m, int64_t k, const uint8_t* codes, const uint8_t* scales,
                          const float* tensor_scale, int64_t n, const float* t, const void* lora_b, int r, void* y,
                          hipStream_t stream);

// The W4A4 MXFP4 GEMM on the block-scaled matrix core (a4w4.hip): K a multiple
// of 128, each operand's codes and y within the buffer-offset range.
bool gemm_a4w4_supports(int64_t m, int64_t n, int64_t k);
hipError_t launch_gemm_a4w4(const uint8_t* xc, const uint8_t* xs, int64_t m, int64_t k, const uint8_t* wc,
                            const uint8_t* ws, int64_t n, void* y, hipStream_t stream);

// dX = dY deq(W) (+ u A) through the frozen base (backward.hip): n % 8 == 0, k % 32 == 0;
// lu (m, lr) fp32 and la (lr, k) bf16, or lr == 0.
hipError_t launch_backward_dx(int fmt, const void* dy, int64_t m, int64_t n, const uint8_t* codes,
                              const uint8_t* scales, const float* tensor_scale, int64_t k, void* dx, const float* lu,
                              const void* la, int lr, hipStream_t stream);

// LoRA gradients (lora_grad.hip): u = dY B (m, r), dA = u^T x (r, k), dB = dY^T t
// (n, r) with t = x A^T, all fp32; n % 8 == 0, k % 32 == 0, 1 <= r <= 64.
size_t lora_backward_workspace_bytes(int64_t m, int64_t n, int64_t k, int r);
hipError_t launch_lora_backward(const void* dy, int64_t m, int64_t n, const void* x, int64_t k, const void* la,
                                const void* lb, int r, float* u_out, float* grad_a, float* grad_b, void* workspace,
                                hipStream_t stream);

// Scale-QLoRA delta gradient (delta_grad.hip): n % 8 == 0, k % 32 == 0.
hipError_t launch_delta_grad(int fmt, const void* dy, const void* x, int64_t m, int64_t n, int64_t k,
                             const uint8_t* codes, const float* tensor_scale, float* grad, hipStream_t stream);

// Noisy RMSNorm ahead of the projections (aqn.hip): k % 8 == 0.
hipError_t launch_aqn_rmsnorm(const void* x, int64_t m, int64_t k, const void* gamma, const float* noise,
                              float sigma, float eps, void* y, hipStream_t stream);

// Grouped linear on the x-in-registers kernel (decode_xs.hip): K in one span.
bool grouped_xs_supports(int64_t num_tokens, int64_t n, int64_t k);
hipError_t launch_grouped_xs(int fmt, const void* x, int64_t num_tokens, const int32_t* row_index,
                             const int32_t* expert_offsets, int64_t num_experts, int64_t total_rows, int64_t n,
                             int64_t k, const uint8_t* codes, const uint8_t* scales, const float* tensor_scales,
                             void* y, hipStream_t stream);

hipError_t launch_grouped_linear(int fmt, const void* x, int64_t num_tokens, const int32_t* row_index,
                                 const int32_t* expert_offsets, int64_t num_experts, int64_t total_rows,
                                 int64_t n, int64_t k, const uint8_t* codes, const uint8_t* scales,
                                 const float* tensor_scales, void* y, hipStream_t stream);

}  // namespace fp4w
