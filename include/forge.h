/*
 * forge.h - C ABI of the MI355X (gfx950) fused weight-gradient + optimizer step.
 *
 * Method: FORGE, "Fused On-Register Gradient Elimination for Memory-Efficient
 * LLM Training" (explainer pages, technical summary). For a linear layer
 * Y = X W^T the weight gradient dW = dY^T X (summed over the T tokens) is
 * computed one weight tile at a time in FP32 accumulators; the element-wise
 * optimizer update is applied to the tile while it is still in registers and
 * only the updated weight tile and its moment tiles are written back, so the
 * gradient never reaches device memory (§2 Method, "Core mechanism", steps
 * 1-4). The input gradient dX = dY W must be computed from the old weights,
 * i.e. before the update (§5, limitations paragraph).
 *
 * Conventions for every entry point
 *   - All tensors are row-major and live in device memory owned by the caller;
 *     the library never allocates, frees or keeps a pointer after returning.
 *     (forge_linear_wgrad_unfused_noalloc uses static device memory of its own.)
 *   - W and the moments are [out, in]; X is [T, in]; dY is [T, out]; dX is [T, in].
 *   - `ld` is the row pitch in elements (ld >= cols). Data pointers must be
 *     16-byte aligned; cols and ld must be multiples of 8 (bf16) or 4 (fp32).
 *     A tensor with no elements may have a NULL data pointer. Every tensor must
 *     span less than 2^31 bytes (rows * ld * element size); larger ones are
 *     rejected with FORGE_ERR_UNSUPPORTED.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *     null stream). No entry point synchronises the host.
 *   - Arguments are validated on the host before anything is enqueued; on an
 *     error nothing is launched and a negative status is returned. No entry
 *     point keeps global mutable state and calls are thread-safe, except for
 *     forge_linear_wgrad_unfused_noalloc (its per-GPU scratch; see there).
 *   - Results are deterministic: fixed reduction order, no atomics.
 */
#ifndef FORGE_H
#define FORGE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void* forge_stream_t; /* hipStream_t */

/* Element types. */
typedef enum {
  FORGE_F32 = 0,  /* IEEE float32 */
  FORGE_BF16 = 1, /* bfloat16 */
  FORGE_I8 = 2,   /* int8 codes of a signed moment (block-64 absmax, scale/127) */
  FORGE_U8 = 3,   /* uint8 codes of sqrt(second moment) (block-64 absmax, scale/255) */
  FORGE_E4M3 = 4, /* OCP FP8 E4M3 input codes (value = decode(code) * scale[0]) */
  FORGE_E5M2 = 5, /* OCP FP8 E5M2 input codes (value = decode(code) * scale[0]) */
  FORGE_I8_DYN = 6, /* signed dynamic 8-bit codes of m (block-64 absmax; see forge_dyn_value) */
  FORGE_U8_DYN = 7  /* unsigned dynamic 8-bit codes of v (block-64 max; see forge_dyn_value) */
} forge_dtype;

/* The eight element-wise optimizers the pages list (§3 Contributions, generality). */
typedef enum {
  FORGE_ADAMW = 0,
  FORGE_SGD = 1,
  FORGE_SGD_MOMENTUM = 2,
  FORGE_LION = 3,
  FORGE_RMSPROP = 4,
  FORGE_ADAGRAD = 5,
  FORGE_NADAM = 6,
  FORGE_RADAM = 7
} forge_opt;

/* A 2-D row-major device tensor. `scale` is used only for
 *   - FORGE_I8 / FORGE_U8 moments: float32 block scales, [rows, cols/64] with row
 *     pitch cols/64, one per 64 consecutive elements of a row (§2 "Precision and
 *     fidelity": INT8 states with blocks of 64); the scale is absmax/127 (m) or
 *     max sqrt(v)/255 (v);
 *   - FORGE_I8_DYN / FORGE_U8_DYN moments: the same layout, the scale being the
 *     block's absmax of m (or max of v);
 *   - FORGE_E4M3 / FORGE_E5M2 inputs: one float32 in device memory, the tensor's
 *     dequantisation scale (element value = decoded code * scale[0]). */
typedef struct {
  void* data;
  int32_t dtype; /* forge_dtype */
  int32_t reserved;
  int64_t rows;
  int64_t cols;
  int64_t ld;
  float* scale;
} forge_tensor;

/* Optimizer hyper-parameters in double (torch.optim conventions; unused fields ignored).
 *   AdamW, Lion: decoupled decay theta *= (1 - lr*weight_decay).
 *   SGD, SGD-momentum, RMSprop, AdaGrad, NAdam, RAdam: coupled L2, g += weight_decay*theta.
 *   Lion: beta1 interpolates the sign argument, beta2 tracks the state.
 *   RMSprop: alpha is the smoothing constant. AdaGrad: lr_decay. NAdam: momentum_decay (>= 0).
 *   SGD-momentum: momentum, dampening, nesterov. */
typedef struct {
  double lr, beta1, beta2, eps, weight_decay;
  double momentum, dampening, alpha, lr_decay, momentum_decay;
  int32_t nesterov;
  int32_t stochastic_round; /* bf16 W only: 1 = stochastic rounding (default), 0 = nearest-even */
} forge_hyper;

/* Per-step scalars the kernels use, computed on the host in double precision
 * from (opt, hyper, step) and rounded once to float (bias corrections, NAdam
 * momentum products, RAdam rectification). Exposed for inspection and tests. */
typedef struct {
  float lr;           /* lr (AdaGrad: lr / (1 + (t-1) lr_decay)) */
  float decay;        /* 1 - lr*weight_decay (AdamW, Lion) */
  float wd;           /* weight_decay for coupled L2 */
  float b1, omb1;     /* beta1 and 1-beta1 (SGD-m: momentum-buffer coefficients) */
  float b2, omb2;     /* beta2 and 1-beta2 (RMSprop: alpha, 1-alpha) */
  float step_size;    /* AdamW: lr/bc1; RAdam: lr*r_t*sqrt(bc2)/bc1 or lr/bc1 */
  float inv_sqrt_bc2; /* 1/sqrt(1-beta2^t) */
  float eps;
  float c_g, c_m;     /* NAdam gradient / momentum coefficients; SGD-m: momentum */
  int32_t flag;       /* RAdam: 1 = rectified branch; SGD-m: nesterov */
  int32_t opt;
} forge_scalars;

/* Status codes. */
#define FORGE_OK 0
#define FORGE_ERR_NULL (-1)        /* a required pointer is NULL */
#define FORGE_ERR_SHAPE (-2)       /* dimensions inconsistent between tensors */
#define FORGE_ERR_DTYPE (-3)       /* unsupported dtype combination */
#define FORGE_ERR_ALIGN (-4)       /* pointer not 16-B aligned, or cols/ld not a multiple of 8 (bf16) / 4 (fp32) */
#define FORGE_ERR_UNSUPPORTED (-5) /* size outside what the kernels handle (e.g. INT8 needs in % 64 == 0) */
#define FORGE_ERR_HYPER (-6)       /* step < 1, unknown optimizer, non-finite or out-of-range hyper-parameter */
#define FORGE_ERR_HIP (-7)         /* kernel launch failed (HIP error) */
#define FORGE_ERR_ALIAS (-8)       /* output tensors overlap each other or an input */
#define FORGE_ERR_SCRATCH (-9)     /* forge_linear_wgrad_unfused_noalloc: out*in > 2^24 (its scratch) */

/*
 * Dynamic 8-bit moment code (FORGE_I8_DYN / FORGE_U8_DYN; §2 "Precision and
 * fidelity" compares the INT8 states' block of 64 with the 2048 of the standard
 * 8-bit optimizers, whose states use a dynamic-exponent code). The n magnitude bits
 * of a code (n = 7 signed, 8 unsigned) hold, from the top, E zeros, an indicator 1
 * and F = n - 1 - E fraction bits f; the magnitude is 10^-E (0.1 + 0.9 (f+1)/2^F),
 * computed as the double quotient (2^F + 9 (f+1)) / (2^F 10^(E+1)) rounded to float;
 * magnitude index 0 is 0. A signed code is sign << 7 | magnitude index. Stored
 * moment = code value * block scale; a new code is the nearest magnitude to
 * |x| / scale in float32 (ties to the larger; x = 0 or a zero block -> code 0).
 * Host-only helpers, no device work:
 *   forge_dyn_value:  float value of a code (is_signed: 1 for m codes, 0 for v codes;
 *                     code 0..255; NaN for other codes).
 *   forge_dyn_encode: the code the kernels store for the normalised value y.
 */
float forge_dyn_value(int32_t is_signed, int32_t code);
int32_t forge_dyn_encode(int32_t is_signed, float y);

/*
 * Fused weight-gradient + optimizer step (§2 Method, "Core mechanism"):
 *   dW = dY^T X (FP32 accumulation over T tokens, tile by tile, never stored),
 *   then the `opt` update of W, m, v in place, with step t = `step` (1-based).
 * X [T, in] and dY [T, out] are read only; W [out, in] is updated in place.
 * dtypes: X, dY, W all FORGE_F32, or all FORGE_BF16. m and v: FORGE_F32, or
 * FORGE_I8 (m) and FORGE_U8 (v) with block scales, or FORGE_I8_DYN (m) and
 * FORGE_U8_DYN (v) with block scales (both INT8 forms: bf16 W, in % 64 == 0, ld a
 * multiple of 16), or FORGE_BF16 (with bf16 W; ld a multiple of 8);
 * m and v must share one format.
 * Slots an optimizer does not use may be NULL and are never touched:
 *   SGD: none; SGD-momentum, Lion: m; RMSprop, AdaGrad: v; others: m and v.
 * bfloat16 W is written with stochastic rounding (hyper->stochastic_round)
 * driven by a counter hash: r16 = top 16 bits of the SplitMix64 output number
 * ((step << 32) | (o*in + i)) + 1 from state `seed`; bf16 = (bits(w32) + r16) >> 16
 * (NaN -> quiet NaN). bfloat16 m and v are rounded the same way from their float32
 * update (the weight update uses the unrounded moments), with other 16-bit fields
 * of the same SplitMix64 word: bits 32..47 for m, bits 16..31 for v (W: bits
 * 48..63); with stochastic_round = 0 all three round to nearest-even.
 * 1 <= step < 2^31.
 * T == 0 is allowed (zero gradient). Requires out*in < 2^32.
 * FP8 inputs (the pages' outlook, §5): X FORGE_E4M3 and dY FORGE_E4M3 or
 * FORGE_E5M2, each with its scale (see forge_tensor), with W FORGE_BF16 and m, v
 * in any of the moment formats above; cols and ld of X and dY must be multiples of
 * 16 (else FORGE_ERR_ALIGN). The gradient is (sum over tokens of the decoded code
 * products) * scale_X * scale_dY.
 * Must be enqueued after forge_linear_dgrad of the same layer (which reads the old W).
 */
int forge_linear_wgrad_step(const forge_tensor* X, const forge_tensor* dY, forge_tensor* W,
                            forge_tensor* m, forge_tensor* v, int32_t opt, const forge_hyper* hyper,
                            int64_t step, uint64_t seed, forge_stream_t stream);

/*
 * The fused step of several layers that read the same input X (the q, k, v projections
 * of an attention block, or gate and up of an MLP), in one launch whose grid holds all
 * their tiles; for a small layer (a few hundred output rows) that is the difference
 * between a few and all of the compute units being busy. Layer l has its own gradient
 * dY[l] [T, out_l], weights W[l] [out_l, in] and moments m[l], v[l] (arrays of
 * n_layers descriptors; m or v may be NULL when the optimizer keeps no such slot), and
 * its own seed seeds[l]; opt, hyper and step are common. Each layer is updated exactly
 * as forge_linear_wgrad_step would update it (same element indices and random streams),
 * except that the tile shape, and so the order of the FP32 summation over tokens, is
 * chosen for the group as a whole. bfloat16 W; X and dY bfloat16, or FP8 codes as in
 * forge_linear_wgrad_step (X E4M3 with its scale; every dY in one format, E4M3 or E5M2,
 * each with its own scale), else FORGE_ERR_DTYPE; fp32 layers: FORGE_ERR_UNSUPPORTED.
 * Every layer's moments in the same format (FORGE_ERR_DTYPE).
 * 1 <= n_layers <= FORGE_MAX_GROUP, else FORGE_ERR_SHAPE. Every argument check of
 * forge_linear_wgrad_step applies to each layer; in addition no layer's W, m, v or block
 * scales may overlap any other layer's tensors (FORGE_ERR_ALIAS). Nothing is enqueued
 * on an error. Must be enqueued after each layer's forge_linear_dgrad.
 * The operation is the pages' fused step (§2 Method, "Core mechanism") for each layer; sharing one
 * launch is this library's arrangement, not part of the method. The descriptor arrays
 * and seeds are host memory read during the call; the tensors' data is caller-owned
 * device memory, as for forge_linear_wgrad_step.
 */
#define FORGE_MAX_GROUP 4
int forge_linear_wgrad_step_group(const forge_tensor* X, int32_t n_layers, const forge_tensor* dY,
                                  forge_tensor* W, forge_tensor* m, forge_tensor* v, int32_t opt,
                                  const forge_hyper* hyper, int64_t step, const uint64_t* seeds,
                                  forge_stream_t stream);

/*
 * Input gradient dX = dY W (§5, limitations: read before the weight update).
 * dY [T, out], W [out, in], dX [T, in]; all FORGE_F32, or all FORGE_BF16
 * (bf16 output rounded to nearest-even from the FP32 accumulator). FP8 dY returns
 * FORGE_ERR_UNSUPPORTED.
 */
int forge_linear_dgrad(const forge_tensor* dY, const forge_tensor* W, forge_tensor* dX,
                       forge_stream_t stream);

/*
 * Unfused baseline, first half: the two-phase schedule the pages describe as
 * the standard one (§1, "the gradient floor"): the same GEMM, but dW [out, in]
 * is written to device memory as float32 (row pitch ld_dw >= in, multiple of 4).
 * X and dY as for forge_linear_wgrad_step, FP8 included.
 */
int forge_linear_wgrad(const forge_tensor* X, const forge_tensor* dY, float* dW, int64_t ld_dw,
                       forge_stream_t stream);

/*
 * Unfused baseline, second half: a separate element-wise optimizer pass that
 * reads the stored float32 dW back and updates W, m, v exactly as the fused
 * step does (same per-element arithmetic, same rounding and RNG).
 */
int forge_optimizer_step(const float* dW, int64_t ld_dw, forge_tensor* W, forge_tensor* m,
                         forge_tensor* v, int32_t opt, const forge_hyper* hyper, int64_t step,
                         uint64_t seed, forge_stream_t stream);

/*
 * The whole unfused baseline in one call (the two-phase schedule of §1: the gradient
 * is materialised in device memory, then a separate optimizer pass reads it back):
 * enqueues forge_linear_wgrad into the caller's float32 workspace dW_workspace [out,
 * ld_ws] (ld_ws >= in, a multiple of 4, 16-byte aligned), then forge_optimizer_step
 * from it. Arguments as for forge_linear_wgrad_step; every one of them, the workspace
 * included, is validated before anything is enqueued. The workspace may overlap no
 * other tensor (FORGE_ERR_ALIAS) and holds dW when the work completes.
 */
int forge_linear_wgrad_unfused(const forge_tensor* X, const forge_tensor* dY, forge_tensor* W,
                               forge_tensor* m, forge_tensor* v, int32_t opt, const forge_hyper* hyper,
                               int64_t step, uint64_t seed, float* dW_workspace, int64_t ld_ws,
                               forge_stream_t stream);

/*
 * forge_linear_wgrad_unfused without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc). The float32 dW lives in a scratch array the library holds in
 * static device memory: 2^24 elements (64 MiB) on each GPU it runs on, for the life of
 * the process. Layers with out*in > 2^24 return FORGE_ERR_SCRATCH (nothing enqueued).
 * No hipMalloc / hipFree or allocating library routine is called; the first call on a
 * device looks up that device's scratch address (hipGetSymbolAddress) and keeps it.
 * Arguments and errors as for forge_linear_wgrad_unfused; the current device must be
 * the one `stream` belongs to. Every call on a GPU shares that GPU's scratch, which keeps
 * the last call's dW: calls that overlap in time on one GPU (other streams, other host
 * threads) race on it and must be ordered by the caller.
 */
int forge_linear_wgrad_unfused_noalloc(const forge_tensor* X, const forge_tensor* dY, forge_tensor* W,
                                       forge_tensor* m, forge_tensor* v, int32_t opt, const forge_hyper* hyper,
                                       int64_t step, uint64_t seed, forge_stream_t stream);

/* Host-only helpers (no GPU work). */

/* Fills *out with the per-step scalars of (opt, hyper, step). Returns a status. */
int forge_step_scalars(int32_t opt, const forge_hyper* hyper, int64_t step, forge_scalars* out);

/* Defaults of the optimizer sweep for `opt` (lr, betas, eps, decay ...). Returns a status. */
int forge_default_hyper(int32_t opt, forge_hyper* out);

/* The stochastic-rounding random bits of element `idx` at `step` (same hash as the kernels). */
uint32_t forge_rand16(uint64_t seed, int64_t step, uint32_t idx);

/* Stochastic rounding of float32 x to bfloat16 bits with random bits r16 (same rule as the kernels). */
uint16_t forge_sr_bf16(float x, uint32_t r16);

/* Human-readable text of a status code (static storage). */
const char* forge_status_str(int status);

/* Library ABI version (major*100 + minor). */
int forge_version(void);

/*
 * MFMA-throughput microbenchmark (no part of the method; it measures the matrix
 * cores' achievable bf16 rate for the roofline of the kernels above). Enqueues
 * n_workgroups workgroups of 256 threads (4 waves); every wave issues 8 * iters
 * v_mfma_f32_32x32x16_bf16 back to back on four independent accumulator sets with
 * all elements of A equal to a and of B equal to b (as bfloat16), then writes the
 * sum of its thread's 64 accumulator values to out[workgroup * 256 + thread]
 * (out: device float array of n_workgroups * 256 elements, caller-owned), which is
 * 2048 * iters * bf16(a) * bf16(b) up to float32 summation (exact for a = 1,
 * b = 2^-10). Requires 1 <= n_workgroups <= 2^20 and 1 <= iters <= 2^24.
 * forge_mfma_peak_flops gives the floating-point operations of such a launch.
 */
int forge_mfma_peak(float* out, int32_t n_workgroups, int32_t iters, float a, float b, forge_stream_t stream);
double forge_mfma_peak_flops(int32_t n_workgroups, int32_t iters);

#ifdef __cplusplus
}
#endif

#endif /* FORGE_H */
