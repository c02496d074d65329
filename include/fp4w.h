/*
 * fp4w.h -- C ABI of libfp4w.so: block-scaled 4-bit weights (NVFP4, MXFP4) and
 * the dequant-fused weight-only (W4A16) linear on AMD Instinct MI355X (gfx950).
 *
 * Sources on the pages:
 *  - The weight format is a 4-bit E2M1 code plus a scale shared by its block, in
 *    NVFP4 and MXFP4 (rit.work, "Scale-QLoRA: merge native 4-bit models",
 *    paragraph on the formats).
 *  - Weight-only quantization with a LoRA adapter in parallel to the base, as in
 *    QLoRA; rollouts are memory-bound and served by a W4A16 kernel
 *    (tggo.me/sberlogasci/42740, sections "Metod" and "Eksperimenty").
 *  - Dynamic ("max") scales recomputed from the current tensors, or frozen
 *    calibrated scales with only the codes recomputed (aikraft.ru, "Nemotron 3.5
 *    Lightning: NVFP4 via QAD", section 03).
 *  - Scale-only merge: trained scale bytes are written on the format's scale grid
 *    and the codes are copied verbatim (Scale-QLoRA page, merge paragraph).
 * The bit layouts are the OCP ones (E2M1, E4M3 "FN", E8M0); block sizes, the
 * tensor scale and round-to-nearest-even on exact quotients are stated readings.
 *
 * Conventions for every call:
 *  - All tensor pointers are DEVICE pointers (hipMalloc'ed or equivalent) unless
 *    stated; the caller owns and allocates every buffer, including workspaces.
 *    The library never allocates, frees or synchronizes.
 *  - Every call enqueues its kernels on `stream` (a hipStream_t; NULL = the
 *    default stream) and returns after host-side validation.  A negative status
 *    means nothing was launched (FP4W_ERR_HIP: a launch itself failed).
 *  - Arrays are row-major.  W is (n, k); codes are (n, k/2) bytes with element k
 *    in the low nibble when k is even; NVFP4 block scales are (n, k/16) E4M3
 *    bytes plus one fp32 tensor scale; MXFP4 block scales are (n, k/32) E8M0
 *    bytes.  bf16 tensors are 2-byte bf16 values.
 *  - k must be a multiple of 32; `w`, `x`, `codes`, `out` and `lora_a` must be
 *    16-byte aligned, bf16 outputs and the NVFP4 scales of the linear calls
 *    2-byte aligned, the linear's workspace 256-byte aligned.  n and m may be 0 (nothing is launched).
 *  - Values the device computes from non-finite inputs are not reported through
 *    the status: NVFP4 gives a non-finite tensor scale, MXFP4 the NaN scale 0xFF.
 *  - Calls on different buffers are thread-safe.  Calls that share an output or
 *    a workspace and overlap in time race.
 */
#ifndef FP4W_H
#define FP4W_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* formats */
#define FP4W_NVFP4 0   /* 16-element blocks, E4M3 block scale, fp32 tensor scale */
#define FP4W_MXFP4 1   /* 32-element blocks, E8M0 block scale                     */

/* status codes */
#define FP4W_OK             0
#define FP4W_ERR_ARG       (-1)  /* null pointer where one is required, negative size */
#define FP4W_ERR_SHAPE     (-2)  /* k % 32 != 0, r outside [0, 64], too large        */
#define FP4W_ERR_ALIGN     (-3)  /* a pointer that must be 16-byte aligned is not    */
#define FP4W_ERR_FORMAT    (-4)  /* unknown format or flag                            */
#define FP4W_ERR_HIP       (-5)  /* a kernel launch failed                            */
#define FP4W_ERR_WORKSPACE (-6)  /* workspace missing or smaller than required       */
#define FP4W_ERR_SCRATCH   (-7)  /* fp4w_linear_noalloc: needs more than its device array */

/* flags */
#define FP4W_FROZEN_SCALES 0x1u  /* fp4w_quantize, fp4w_fake_quant: scales (and tensor scale) are inputs */
#define FP4W_OUT_FP32      0x2u  /* fp4w_dequantize: write fp32 instead of bf16         */

/* Largest LoRA rank the fused linear accepts. */
#define FP4W_MAX_LORA_RANK 64

/*
 * fp4w_quantize -- bf16 weights W (n, k) -> codes (n, k/2) and block scales.
 *
 * NVFP4, dynamic ("max") scales: A = max |w| over the whole tensor; the tensor
 *   scale s_t = fl32(A / 2688) (correctly rounded binary32 division, 2688 = 6*448)
 *   is written to *tensor_scale (device, one float); block scale
 *   sb = RNE_sat(a_b / (6 s_t)) on the E4M3
 *   grid (0 when s_t == 0); code = sign | RNE_sat(|w| / (dec(sb) s_t)) on the
 *   E2M1 grid, with the quotients taken exactly; a block whose scale decodes to 0
 *   gets signed-zero codes.
 * MXFP4: per 32-block e = clamp(floor(log2 a_b) - 2, -127, 127) (a_b == 0 gives
 *   -127), scale byte e + 127, code = sign | RNE_sat(|w| * 2^-e); tensor_scale is
 *   not used (may be NULL).
 * FP4W_FROZEN_SCALES: `scales` and (NVFP4) `*tensor_scale` are read, not written;
 *   only the codes are computed (frozen-scale training, Nemotron QAD page,
 *   section 03).  The given scales must be valid non-negative scale codes
 *   (E4M3 0x00..0x7E, E8M0 0x00..0xFE) and s_t finite and >= 0.
 * RNE_sat: round to nearest, ties to the even code, saturate at the grid top.
 * -0 encodes as 0x8.
 * Launches on `stream`: MXFP4 and frozen scales one; NVFP4 dynamic two (per-
 * workgroup maxima of |w|, then the encode, whose workgroups each reduce those
 * maxima to s_t; one of them writes *tensor_scale).  The maxima live in a slot of
 * a small device array the library holds, one slot per calling stream (64 per
 * device, 2 KiB each; a 65th stream shares a slot): calls on one stream are
 * ordered, and NVFP4 dynamic calls that overlap in time on up to 64 streams of
 * one device do not interfere.
 */
int fp4w_quantize(int fmt, const void *w_bf16, int64_t n, int64_t k,
                  uint8_t *codes, uint8_t *scales, float *tensor_scale,
                  uint32_t flags, void *stream);

/*
 * fp4w_dequantize -- codes + scales -> W (n, k): the exact value
 * e2m1(c) * dec(sb) * s_t (NVFP4) or e2m1(c) * 2^(sb-127) (MXFP4), rounded once
 * to nearest even to bf16 (default) or to fp32 (FP4W_OUT_FP32).  This is the
 * fake-quant forward the training pages insert (QATFactory page, section on how
 * training repeats the engine's arithmetic).  tensor_scale is a device pointer
 * (NVFP4) or ignored (MXFP4).
 */
int fp4w_dequantize(int fmt, const uint8_t *codes, const uint8_t *scales,
                    const float *tensor_scale, int64_t n, int64_t k,
                    void *out, uint32_t flags, void *stream);

/*
 * fp4w_fake_quant -- fused fake-quant forward of a bf16 tensor W (n, k): in one
 * pass per block, the codes fp4w_quantize computes, decoded as fp4w_dequantize
 * decodes them (bf16), written to out_bf16 (n, k); the codes themselves are not
 * stored.  Bit for bit, out = dequantize(quantize(W)).  The quantize-then-
 * dequantize a training forward inserts so that it sees the engine's values
 * (QATFactory page, section on how training repeats the engine's arithmetic);
 * its backward is the plain straight-through estimator (the gradient passes
 * unchanged; page on QAT at low bit widths), which needs no kernel.
 * scales (n, k/16 or k/32) and, for NVFP4, *tensor_scale are written as
 * fp4w_quantize writes them, or read with FP4W_FROZEN_SCALES (frozen-scale
 * training).  Also
 * fits activations (rows of x) for W4A4 training.  w_bf16 and out_bf16 must be
 * 16-byte aligned and must not overlap.
 */
int fp4w_fake_quant(int fmt, const void *w_bf16, int64_t n, int64_t k,
                    void *out_bf16, uint8_t *scales, float *tensor_scale,
                    uint32_t flags, void *stream);

/*
 * Workspace for fp4w_linear, in bytes, for x (m, k), W (n, k) and LoRA rank r
 * (0 when there is no LoRA); 0 for invalid arguments.  It holds the LoRA
 * intermediate t = x A^T (fp32) or its per-chunk partials, split-K partial sums
 * and, in its first 28800 bytes at fixed offsets, arrival counters and the words
 * through which one kernel's workgroups hand t to each other.  That area must be
 * zero before the first call: zero-fill a new workspace once; every call returns
 * it to zero when it completes, so one workspace serves calls of any shape in
 * stream order (calls that overlap on one workspace race).
 */
size_t fp4w_linear_workspace_bytes(int64_t m, int64_t n, int64_t k, int r);

/*
 * fp4w_linear -- y (m, n) bf16 = x (m, k) deq(W)^T + (x A^T) B^T, with fp32
 * accumulation: the W4A16 linear with a parallel LoRA branch (Telegram post,
 * "Metod"; QATFactory page: the product runs on 16-bit values).
 *   x_bf16     (m, k) bf16
 *   codes, scales, tensor_scale   a quantized W (n, k), as fp4w_quantize writes
 *   lora_a     (r, k) bf16 or NULL;  lora_b (n, r) bf16 or NULL;  r in [0, 64]
 *              (both NULL or r == 0: no LoRA; any LoRA scaling is folded into B)
 *   y_bf16     (m, n) bf16, rounded once from the fp32 result
 *   workspace  >= fp4w_linear_workspace_bytes(m, n, k, r) bytes, see above
 * Launches (all on `stream`):
 *  - m <= 2, and m <= 4 when n * k <= 2^24: one launch of the decode kernel
 *    on gfx950's block-scaled MFMA,
 *    which feeds the codes to the matrix core as stored and x as two E4M3 terms
 *    per element under an E8M0 scale per 32 elements.  That split is exact for
 *    every element within 2^13 of its block's largest magnitude; smaller ones
 *    are off by at most 2^-21 of that maximum.  With a LoRA, the kernel's first
 *    workgroups form t = x A^T on the bf16 matrix core, one K chunk each, and
 *    hand it to the workgroups that write the outputs (chunks added in a fixed
 *    order: the result does not depend on scheduling).
 *  - other m <= 16: one launch of a decode kernel holding x in registers (with
 *    a LoRA, t = x A^T is formed and handed over inside it as above): the weights are decoded exactly to fp16 (NVFP4, with x scaled to
 *    fp16 by a power of two per row and K range: exact for every element within
 *    2^28 of that range's largest magnitude) or bf16 (MXFP4) in registers and
 *    fed to the 16-bit MFMA.  MXFP4 weights whose decoded value exceeds bf16's
 *    range (scale codes 253, 254 only) give infinite products, as dequantizing
 *    to bf16 does.
 *    On both decode paths a non-finite x element makes every output of its row
 *    NaN, and a NaN block scale every output of its weight row.
 *  - m > 16: the LoRA down-projection, then the LDS-staged bf16 MFMA GEMM.
 *  - k == 0: y = 0 (every output is an empty sum; one fill launch, no operand
 *    is read).
 * The LoRA product is added in fp32 (GEMM: t split into two bf16 parts for the
 * matrix cores).
 */
int fp4w_linear(int fmt, const void *x_bf16, int64_t m, int64_t k,
                const uint8_t *codes, const uint8_t *scales, const float *tensor_scale,
                int64_t n, const void *lora_a, const void *lora_b, int r,
                void *y_bf16, void *workspace, size_t workspace_bytes, void *stream);

/*
 * fp4w_linear_noalloc -- fp4w_linear without a workspace argument, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).  Same arguments, kernels and
 * results as fp4w_linear (bit for bit); the workspace is a library-owned device
 * array of FP4W_NOALLOC_SCRATCH_BYTES bytes, one per device, set up at the first
 * call on a device and held until the process ends.  The call allocates and
 * frees nothing.  A call whose fp4w_linear_workspace_bytes exceeds that size
 * returns FP4W_ERR_SCRATCH and launches nothing (8 MiB covers every m <= 16 up
 * to about 1.1e9 weights, and m * r * 4 up to about 8 MB on the GEMM path).
 * Every call on one device shares the array, which keeps the last call's
 * contents (its counter area is zero between calls): calls that overlap in
 * time on one device race, so issue them in one stream order.
 */
#define FP4W_NOALLOC_SCRATCH_BYTES (8u << 20)
int fp4w_linear_noalloc(int fmt, const void *x_bf16, int64_t m, int64_t k,
                        const uint8_t *codes, const uint8_t *scales, const float *tensor_scale,
                        int64_t n, const void *lora_a, const void *lora_b, int r,
                        void *y_bf16, void *stream);

/*
 * fp4w_linear_w4a4 -- y (m, n) bf16 = deq(x) deq(W)^T with x and W both MXFP4
 * (W4A4: 4-bit weights and activations, the mode MXFP4 deploys best in when
 * training quantized both; QATFactory page, section on the strategies NVFP4 and
 * MXFP4 need), on gfx950's block-scaled matrix core: the E2M1 codes and E8M0
 * scales go to the instruction as stored, every product is exact and the sum is
 * accumulated in fp32, rounded once to bf16.
 *   fmt        FP4W_MXFP4 (NVFP4's E4M3 block scales have no native scaled
 *              product: FP4W_ERR_FORMAT)
 *   x_codes    (m, k/2), x_scales (m, k/32): x as fp4w_quantize writes it
 *   codes      (n, k/2), scales   (n, k/32): W as fp4w_quantize writes it
 *   y_bf16     (m, n) bf16
 * k must be a positive multiple of 128 and m * n * 2 below 2^32, each code
 * plane (plus 512 rows) below 2 GiB: else FP4W_ERR_SHAPE.  Codes 16-byte,
 * scales 4-byte, y 2-byte aligned (FP4W_ERR_ALIGN).  A NaN block scale (0xFF)
 * makes the products of its block NaN.  One launch on `stream`; no workspace.
 */
int fp4w_linear_w4a4(int fmt, const uint8_t *x_codes, const uint8_t *x_scales,
                     int64_t m, int64_t k, const uint8_t *codes, const uint8_t *scales,
                     int64_t n, void *y_bf16, void *stream);

/*
 * fp4w_linear_backward_dx -- the input gradient through the frozen 4-bit base
 * and, with a LoRA, through the adapter (training with the quantized base frozen
 * back-propagates through it; Telegram post, "Metod"):
 *   dx (m, k) bf16 = dy (m, n) deq(W) (n, k) + u A,   u = dy B (see fp4w_lora_backward)
 * fp32 accumulation, rounded once to bf16.  The weight is decoded exactly (as
 * fp4w_dequantize to bf16), the NVFP4 tensor scale multiplies its fp32 sums; u
 * enters the bf16 matrix core as two bf16 parts (hi + lo, 2^-16 relative).
 *   dy_bf16    (m, n) bf16, 16-byte aligned;  n % 8 == 0 (else FP4W_ERR_SHAPE)
 *   codes, scales, tensor_scale   a quantized W (n, k), as fp4w_quantize writes it
 *   lora_u     (m, r) fp32, 4-byte aligned, and lora_a (r, k) bf16, 2-byte aligned;
 *              or both NULL / r == 0 (no LoRA term); r <= 64
 *   dx_bf16    (m, k) bf16, 8-byte aligned
 * m at most 65535 * 128.  n == 0 writes u A (zeros without a LoRA); m == 0 or
 * k == 0 does nothing.  A NaN block scale makes the outputs of its block's k
 * columns NaN in every row.  One launch on `stream`; no workspace.
 */
int fp4w_linear_backward_dx(int fmt, const void *dy_bf16, int64_t m, int64_t n,
                            const uint8_t *codes, const uint8_t *scales,
                            const float *tensor_scale, int64_t k, const float *lora_u,
                            const void *lora_a, int r, void *dx_bf16, void *stream);

/*
 * fp4w_lora_backward -- the gradients of the LoRA branch y_lora = (x A^T) B^T of
 * fp4w_linear (the adapter trained in parallel to the frozen base; Telegram post,
 * "Metod"), from the output gradient dy and the input x:
 *   t = x A^T (m, r);   u = dy B (m, r);   dB = dy^T t (n, r);   dA = u^T x (r, k)
 * all accumulated in fp32 on the bf16 matrix core (t and u enter the products
 * over m as two bf16 parts, hi + lo); every sum in a fixed order.  u is what
 * fp4w_linear_backward_dx takes for the adapter's share of dx.
 *   dy_bf16 (m, n), x_bf16 (m, k): bf16, 16-byte aligned; n % 8 == 0, k % 32 == 0
 *   lora_a (r, k) bf16 16-byte aligned; lora_b (n, r) bf16 2-byte aligned; 1 <= r <= 64
 *   u (m, r), grad_a (r, k), grad_b (n, r): fp32 outputs, 4-byte aligned, each may
 *     be NULL (not written); m == 0 writes zero gradients
 *   workspace >= fp4w_lora_backward_workspace_bytes(m, n, k, r) bytes, 256-byte
 *     aligned, no initial contents required
 * Nine launches on `stream`.
 */
size_t fp4w_lora_backward_workspace_bytes(int64_t m, int64_t n, int64_t k, int r);
int fp4w_lora_backward(const void *dy_bf16, int64_t m, int64_t n, const void *x_bf16, int64_t k,
                       const void *lora_a, const void *lora_b, int r, float *u, float *grad_a,
                       float *grad_b, void *workspace, size_t workspace_bytes, void *stream);

/*
 * fp4w_scale_delta_grad -- the Scale-QLoRA training gradient of the block-scale
 * deltas (Scale-QLoRA page: block-scale corrections trained with the codes
 * frozen, rounded to the scale grid in every forward; the rounding is passed
 * straight through): for y = x deq(W)^T with W's block scales shifted by deltas
 * in the decoded scale domain (before any tensor scale, as fp4w_merge_scales
 * takes them),
 *   grad[n, b] = s_t * sum_{k in block b} e2m1(q[n, k]) * (dy^T x)[n, k]
 * with s_t the NVFP4 tensor scale (1 for MXFP4); dy^T x is accumulated in fp32
 * and never stored.
 *   dy_bf16  (m, n) bf16, the gradient of y;  x_bf16 (m, k) bf16, the input
 *   codes    (n, k/2) of W, as fp4w_quantize writes them; tensor_scale (NVFP4)
 *   grad     (n, k/16) fp32 (NVFP4) or (n, k/32) (MXFP4), fully written
 * n % 8 == 0 and k % 32 == 0 (else FP4W_ERR_SHAPE); dy, x and codes 16-byte
 * aligned, grad 4-byte aligned.  m == 0 writes zeros.  One launch on `stream`.
 */
int fp4w_scale_delta_grad(int fmt, const void *dy_bf16, const void *x_bf16,
                          int64_t m, int64_t n, int64_t k, const uint8_t *codes,
                          const float *tensor_scale, float *grad, void *stream);

/*
 * fp4w_aqn_rmsnorm -- the noisy RMSNorm ahead of the projections (adaptive
 * noise for exploration in the RL fine-tuning of the Telegram post, "Metod":
 * noise applied in the RMS norm before the projections, which is multiplicative
 * noise on their weights).  Per row of x (m, k):
 *   y[k] = bf16( x[k] / sqrt(mean(x^2) + eps) * gamma[k] * (1 + sigma * noise[k]) )
 * computed in fp32, rounded once (RNE).  The linear that consumes y sees its
 * weight columns scaled by (1 + sigma * noise[k]).
 *   x_bf16, y_bf16 (m, k) bf16 (may be the same buffer); gamma_bf16 (k) bf16;
 *   noise (k) fp32, drawn by the caller each step (standard normal);
 *   sigma from fp4w_aqn_sigma; eps the norm's epsilon
 * k % 8 == 0 (else FP4W_ERR_SHAPE); all pointers 16-byte aligned.
 */
int fp4w_aqn_rmsnorm(const void *x_bf16, int64_t m, int64_t k, const void *gamma_bf16,
                     const float *noise, float sigma, float eps, void *y_bf16, void *stream);

/*
 * fp4w_aqn_sigma -- the noise scale at `step` of `total_steps` on the
 * exponential schedule from sigma_max down to sigma_min (the post: 1e-2 to
 * 5e-4, exponential decay doing slightly better than other schedules):
 * sigma_max * (sigma_min / sigma_max)^(step / total_steps), clamped to the ends;
 * 0 for non-positive sigmas.  Host function.
 */
double fp4w_aqn_sigma(int64_t step, int64_t total_steps, double sigma_max, double sigma_min);

/*
 * Workspace for fp4w_linear_aqn, in bytes: fp4w_linear_workspace_bytes(m, n, k,
 * r) rounded up to 256, plus m * k * 2 (the normalized x where the norm runs as
 * a launch of its own) rounded up to 256; 0 for invalid arguments.  Its first
 * bytes are fp4w_linear's counter area, with the same zero-fill rule.
 */
size_t fp4w_linear_aqn_workspace_bytes(int64_t m, int64_t n, int64_t k, int r);

/*
 * fp4w_linear_aqn -- the linear of the noisy RMSNorm of x: y = fp4w_linear of
 * x~ (m, k), x~ = x / sqrt(mean(x^2) + eps) * gamma * (1 + sigma * noise) per row
 * (the norm of fp4w_aqn_rmsnorm, the projection that follows it; Telegram post,
 * "Metod": noise in the RMS norm before the projections).  Arguments are
 * fp4w_aqn_rmsnorm's (gamma_bf16, noise, sigma, eps) followed by fp4w_linear's;
 * gamma and noise 16-byte aligned, workspace 256-byte aligned and at least
 * fp4w_linear_aqn_workspace_bytes(m, n, k, r).
 * Where the linear runs as one decode launch whose workgroups each cover the
 * whole K (m <= 16 with no K split, as for k = 3584 at any n of the Qwen-2.5-7B
 * projections) the norm runs inside it: each workgroup forms
 * bf16(x * gamma * (1 + sigma * noise)) while
 * staging x, sums x^2 of its rows in fp32, and multiplies its fp32 outputs (with
 * the LoRA term) by 1 / sqrt(mean(x^2) + eps) before the one rounding to bf16.
 * Elsewhere fp4w_aqn_rmsnorm writes x~ into the workspace and fp4w_linear reads
 * it.  Both round x~ (or x~ without the row factor) to bf16 once: the outputs
 * are within the linear's bound of x~ plus 2^-8 of sum_k |x~_k w_k|.
 */
int fp4w_linear_aqn(int fmt, const void *x_bf16, int64_t m, int64_t k, const void *gamma_bf16,
                    const float *noise, float sigma, float eps, const uint8_t *codes,
                    const uint8_t *scales, const float *tensor_scale, int64_t n,
                    const void *lora_a, const void *lora_b, int r, void *y_bf16,
                    void *workspace, size_t workspace_bytes, void *stream);

/*
 * fp4w_grouped_linear -- the W4A16 linear over the experts of a mixture of
 * experts (QATFactory page: dense and MoE models; Nemotron page: 30B-A3B base).
 * For every expert e and every row q in [expert_offsets[e], expert_offsets[e+1]):
 *   y[q, :] = x[row_index[q], :] deq(W_e)^T
 *   x_bf16          (num_tokens, k) bf16
 *   row_index       (total_rows) int32, device; token of each routed row
 *   expert_offsets  (num_experts + 1) int32, device, non-decreasing, [0]=0,
 *                   [num_experts] = total_rows; the routing stays on the device
 *   codes           (num_experts, n, k/2);  scales (num_experts, n, k/blk)
 *   tensor_scales   (num_experts) fp32, device (NVFP4) or NULL (MXFP4)
 *   y_bf16          (total_rows, n) bf16
 * Device-side checks: offsets are clamped to [0, total_rows] (an expert whose
 * range is empty does nothing); a row whose row_index is outside
 * [0, num_tokens) is written as NaN; rows no expert covers are left unchanged.
 * There is no LoRA branch here.
 */
int fp4w_grouped_linear(int fmt, const void *x_bf16, int64_t num_tokens,
                        const int32_t *row_index, const int32_t *expert_offsets,
                        int64_t num_experts, int64_t total_rows, int64_t n, int64_t k,
                        const uint8_t *codes, const uint8_t *scales,
                        const float *tensor_scales, void *y_bf16, void *stream);

/*
 * fp4w_merge_scales -- scale-only merge (Scale-QLoRA page, merge paragraph):
 * per block, v = dec(scales_in[i]) + deltas[i] exactly (deltas are fp32, in the
 * decoded scale domain, before any tensor scale); v <= 0 gives code 0x00, else
 * the nearest value of the format's scale grid (E4M3 or E8M0, nearest in the
 * linear domain), ties to the even code, saturating at 448 (0x7E) or 2^127
 * (0xFE); a NaN scale or delta gives the NaN code.  scales_out may equal
 * scales_in.  When codes_out != codes_in and both are non-NULL, the code plane
 * (code_bytes bytes) is copied byte for byte; with codes_out == codes_in or NULL
 * nothing is copied.  The NVFP4 tensor scale is not touched.
 */
int fp4w_merge_scales(int fmt, const uint8_t *scales_in, const float *deltas,
                      int64_t num_blocks, uint8_t *scales_out,
                      const uint8_t *codes_in, uint8_t *codes_out, int64_t code_bytes,
                      void *stream);

/*
 * Test hook (not part of the method): the longest time, in ticks of the
 * device's 100 MHz clock, that a workgroup of the m == 1 decode kernel waits
 * for the t = x A^T that other workgroups publish before it forms t itself by
 * the same steps in the same order (the outputs are the same either way).
 * Default 100000 (1 ms); 0 makes most workgroups form t themselves.  Applies to
 * later launches of this process; ticks < 0 only queries.  Returns the value
 * in force before the call.
 */
int64_t fp4w_debug_lora_wait(int64_t ticks);

/* Human-readable name of a status code (static string). */
const char *fp4w_status_string(int status);

/* Library ABI version (increments on any signature change). */
int fp4w_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FP4W_H */
