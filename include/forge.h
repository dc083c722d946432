/*
 * forge.h -- C ABI of the fused weight-gradient + optimizer-step library for
 * AMD Instinct MI355X (gfx950).
 *
 * Source of the method: the FORGE explainer pages (gist.science, "FORGE:
 * Fused On-Register Gradient Elimination for Memory-Efficient LLM Training").
 *   - Technical Summary section 1 "The Problem": the standard schedule writes
 *     the full weight gradient of a layer to HBM and the optimizer reads it
 *     back.
 *   - Technical Summary section 2 "Core Mechanism": for each 128 x 128 tile of
 *     W the kernel accumulates the products of the upstream gradient dY and the
 *     input X over all tokens in fp32 registers, applies the optimizer to the
 *     tile in registers, discards the gradient, and writes back only the
 *     updated weight tile and its moment tiles.
 *   - Technical Summary section 2 "Precision and Fidelity": the gradient stays
 *     fp32; the bf16 weight write-back is rounded stochastically; int8
 *     optimizer states use blocks of 64 elements.
 *   - Technical Summary section 3 "Key Contributions": eight element-wise
 *     optimizers (AdamW, NAdam, RAdam, Lion, RMSprop, AdaGrad, SGD,
 *     SGD-momentum).
 *   - Technical Summary section 4 "Composability": fp8 inputs.
 *   - Technical Summary section 5 "Significance and Claims" (limitations): the
 *     input gradient must be read before the weight update; weights with
 *     several gradient consumers in one step are excluded.
 *
 * Conventions for every entry point
 *   - Tensors are row-major and contiguous (row stride `ld` equal to `cols`);
 *     every data pointer is a device pointer to memory of the current HIP
 *     device, aligned to 16 bytes.  All buffers are owned by the caller; the
 *     library keeps no pointer to them after a call returns.  Its only global
 *     state is a per-device cache (whether the device passed the gfx950 check,
 *     its compute-unit count, the address of the counter array of
 *     forge_linear_backward_step_fused_noalloc), written once per device and
 *     never cleared, and that counter array itself (a static device array).
 *   - Shapes: X[T, K] layer input, dY[T, N] upstream gradient, W[N, K] weight
 *     (PyTorch nn.Linear layout), dW[N, K], dX[T, K].  N and K must be
 *     multiples of 128; T may be any value >= 0 (a ragged final token slab is
 *     handled; T = 0 means a zero gradient).
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *     asynchronously; arguments are validated synchronously first.  On any
 *     error nothing is launched and no buffer is touched.
 *   - No entry point allocates device memory.
 *   - Thread safety: entry points may be called from several threads; the
 *     text of the last error is kept per thread.
 */
#ifndef FORGE_H
#define FORGE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FORGE_VERSION 100 /* 1.0.0 */

typedef enum forge_status {
  FORGE_OK = 0,
  FORGE_ERR_ARG = 1,    /* null pointer, step < 1, unknown enum, state given/missing for the rule,
                           hyper-parameters giving a non-finite per-step scalar (see forge_hyper) */
  FORGE_ERR_SHAPE = 2,  /* shapes disagree, N or K not a multiple of 128, N*K >= 2^32, a tensor
                           of 2^48 bytes or more */
  FORGE_ERR_DTYPE = 3,  /* unsupported dtype or dtype combination */
  FORGE_ERR_LAYOUT = 4, /* pointer not 16-byte aligned, or row stride ld != cols */
  FORGE_ERR_ALIAS = 5,  /* an output buffer overlaps an input or another output */
  FORGE_ERR_DEVICE = 6, /* no device, or the current device is not gfx950 */
  FORGE_ERR_LAUNCH = 7  /* the HIP runtime refused the launch; see forge_last_error() */
} forge_status;

typedef enum forge_dtype {
  FORGE_F32 = 0,
  FORGE_BF16 = 1,
  FORGE_FP8_E4M3 = 2, /* OCP e4m3 bytes; `scale` -> one fp32 per-tensor scale (value = decode(code) * scale) */
  FORGE_I8_B64 = 3,   /* signed int8 moment, codes -127..127; `scale` -> rows*cols/64 fp32 block absmax */
  FORGE_U8_B64 = 4,   /* non-negative uint8 moment, codes 0..255; `scale` -> rows*cols/64 fp32 block absmax */
  FORGE_I8DYN_B64 = 5, /* signed moment in the dynamic 8-bit map (see below); `scale` as FORGE_I8_B64 */
  FORGE_U8DYN_B64 = 6  /* non-negative moment in the dynamic 8-bit map; `scale` as FORGE_U8_B64 */
} forge_dtype;

/* 8-bit moments (Technical Summary section 2 "Precision and Fidelity": int8 optimizer states in
 * blocks of 64).  A block is 64 consecutive elements of a row; its fp32 scale is the absmax of
 * the new values.  The linear map stores code = nearest-even of x * levels / scale (levels 127
 * signed, 255 unsigned).  The dynamic map (the dynamic tree code of common 8-bit optimizers,
 * offered for comparison) stores a sign bit (signed only), then in the 7 (signed) or 8
 * (unsigned) magnitude bits p a run of E zero bits, an indicator bit and F = bits - 1 - E
 * fraction bits f, for the magnitude scale * 10^-E * (0.1 + 0.9 (f + 1) / 2^F) (p = 0: zero),
 * nearest magnitude on encoding.  Both maps: a non-zero second moment never stores zero; a
 * block holding NaN or an infinity stores zero codes and a NaN scale.  m and v of one call
 * must use the same map. */

typedef enum forge_opt {
  FORGE_ADAMW = 0,        /* states m, v */
  FORGE_NADAM = 1,        /* states m, v */
  FORGE_RADAM = 2,        /* states m, v */
  FORGE_LION = 3,         /* state m */
  FORGE_RMSPROP = 4,      /* state v */
  FORGE_ADAGRAD = 5,      /* state v (sum of squared gradients) */
  FORGE_SGD = 6,          /* no state */
  FORGE_SGD_MOMENTUM = 7  /* state m (momentum buffer) */
} forge_opt;

/* A 2-D tensor descriptor.  `ld` is the row stride in elements; every entry point requires
 * ld == cols (contiguous rows) and returns FORGE_ERR_LAYOUT otherwise.  `scale` is a device
 * pointer (see forge_dtype) or NULL; the library cannot see its allocation size, so the
 * caller must provide the element count the dtype names. */
typedef struct forge_tensor {
  void* data;
  int32_t dtype; /* forge_dtype */
  int64_t rows;
  int64_t cols;
  int64_t ld;
  void* scale;
} forge_tensor;

/* Weight-decay modes. DEFAULT: decoupled for AdamW and Lion, coupled L2 for the others. */
#define FORGE_WD_DEFAULT 0
#define FORGE_WD_DECOUPLED 1
#define FORGE_WD_L2 2

/* Hyper-parameters.  Fields a rule does not use are ignored (never read).
 *   AdamW/NAdam/RAdam: lr, beta1, beta2, eps, weight_decay; NAdam also momentum_decay (psi).
 *   Lion: lr, beta1 (interpolation inside sign), beta2 (moment), weight_decay.
 *   RMSprop: lr, alpha, eps, weight_decay.   AdaGrad: lr, eps, weight_decay.
 *   SGD: lr, weight_decay.   SGD-momentum: lr, momentum, weight_decay.
 * AdamW, NAdam and RAdam need 0 <= beta1, beta2 < 1, and NAdam a finite momentum_decay >= 0;
 * every per-step scalar derived from the fields (forge_step_scalars) must be finite in fp32.
 * Anything else: FORGE_ERR_ARG. */
typedef struct forge_hyper {
  float lr, beta1, beta2, eps, weight_decay;
  int32_t wd_mode;
  float momentum, alpha, momentum_decay;
} forge_hyper;

/* Optional per-call options (pass NULL for the defaults). */
typedef struct forge_step_opts {
  float* w_preround_out; /* if non-NULL: fp32 [N, K] device buffer receiving the updated weight
                            before it is rounded to the storage dtype (for checking) */
  int32_t sr_enable;     /* bf16 weights: 1 = stochastic rounding (default), 0 = nearest-even */
} forge_step_opts;

/*
 * forge_wgrad_step -- one fused optimizer step of a linear layer's weight.
 *
 * For every element of W: g = sum_t dY[t, n] * X[t, k] accumulated in fp32 (for fp8 inputs
 * multiplied by both per-tensor scales), then one step of rule `opt` updates W, m, v in place.
 * The gradient is never written to memory (Technical Summary section 2 "Core Mechanism").
 *
 *   X, dY   inputs, both F32, both BF16 or both FP8_E4M3.  Read only.
 *   W       [N, K], F32 (fp32 inputs only) or BF16.  BF16 is written back with stochastic
 *           rounding: element i = n*K + k draws 16 bits from Philox4x64-10 with counter
 *           (i >> 4, step, 0, 0) and key (seed, 0), field (i & 3) of word (i & 15) >> 2, and
 *           stores (bits(fp32 value) + r) >> 16 (NaN stays NaN).
 *   m, v    moments of the rule ([N, K]: both F32, or I8_B64 for m and U8_B64 for v, or
 *           I8DYN_B64 and U8DYN_B64, with their block scales); must be NULL for a moment the rule
 *           does not keep.  Zero them (codes and scales) before step 1.
 *   step    1-based step count used by bias corrections and schedules; must be >= 1.
 *   seed    stochastic-rounding key; give each weight its own seed.
 * Errors: see forge_status.  A weight with several gradient consumers in one step (tied
 * embeddings, shared experts) or a non-element-wise update (global-norm clipping) cannot use
 * this call (Technical Summary section 5, limitations).
 */
forge_status forge_wgrad_step(const forge_tensor* X, const forge_tensor* dY, forge_tensor* W,
                              forge_tensor* m, forge_tensor* v, const forge_hyper* hyper,
                              int32_t opt, int64_t step, uint64_t seed,
                              const forge_step_opts* opts, void* stream);

/*
 * forge_dgrad -- input gradient dX[T, K] = dY[T, N] . W[N, K], accumulated in fp32 and stored
 * BF16 with round-to-nearest-even.  dY [T, N], W [N, K] and dX [T, K] must all be BF16
 * (anything else: FORGE_ERR_DTYPE); N and K multiples of 128; (T + 256) N and N K each below
 * 2^31 elements (32-bit byte offsets; else FORGE_ERR_SHAPE).  It reads W as it is when the
 * kernel runs, so enqueue it before forge_wgrad_step on the same stream (Technical Summary
 * section 5: the input gradient must be read before the weight update).  dX is overwritten and
 * must not overlap dY or W (FORGE_ERR_ALIAS).
 */
forge_status forge_dgrad(const forge_tensor* dY, const forge_tensor* W, forge_tensor* dX,
                         void* stream);

/* forge_linear_backward_step -- forge_dgrad then forge_wgrad_step, in that order, on `stream`. */
forge_status forge_linear_backward_step(const forge_tensor* X, const forge_tensor* dY,
                                        forge_tensor* W, forge_tensor* dX, forge_tensor* m,
                                        forge_tensor* v, const forge_hyper* hyper, int32_t opt,
                                        int64_t step, uint64_t seed, const forge_step_opts* opts,
                                        void* stream);

/*
 * forge_linear_backward_step_fused -- what forge_linear_backward_step computes (dX from the
 * weight as it was before the step, then the fused step of W, m, v), in one kernel launch
 * after a one-workgroup clear of the workspace.  FORGE explainer (gist.science), Technical
 * Summary section 5, limitations (the input gradient is read before the weight update), and
 * section 2 "Core Mechanism" (the step).  In the launch, workgroups take the dX tiles (256
 * tokens x 128 columns) and the step's tiles of W from work queues, every dX tile before any step
 * tile; a step tile contracts dY and X, then, before it writes W, waits until every dX tile of
 * its 128 columns has finished reading them.  dX comes out bitwise as from forge_dgrad.  W, m
 * and v come out bitwise as from forge_linear_backward_step wherever that call's step runs on
 * the 256 x 128, 256 x 256 or 128 x 256 tiles (N % 256 == 0 and at least 128 tiles of
 * 256 x 128); on smaller layers it uses 128 x 128 tiles with their own token order, and the two
 * agree within the fp32 summation bound of the gradient.
 *
 * Arguments as forge_linear_backward_step (BF16 X, dY, W and dX), and N % 256 == 0, K % 128 == 0
 * (else FORGE_ERR_SHAPE).  workspace: device memory of at least
 * forge_backward_workspace_bytes(K) bytes, 4-byte aligned, owned by the caller and overlapping
 * no tensor of the call (FORGE_ERR_ARG / FORGE_ERR_LAYOUT / FORGE_ERR_ALIAS); its contents
 * before the call do not matter, and the call overwrites them.  Two calls that share a
 * workspace must not run at the same time (on different streams, say).  Once the stream has
 * passed the call, the int32 at byte offset 4 of the workspace is 0.  It is nonzero only on a
 * fault of the schedule: bit 0 if a step tile's wait reached its bound (seconds), bit 1 if a
 * workgroup found no work left (calls sharing the workspace overlapped); the tiles concerned
 * were then not updated.
 */
forge_status forge_linear_backward_step_fused(const forge_tensor* X, const forge_tensor* dY,
                                              forge_tensor* W, forge_tensor* dX, forge_tensor* m,
                                              forge_tensor* v, const forge_hyper* hyper, int32_t opt,
                                              int64_t step, uint64_t seed,
                                              const forge_step_opts* opts, void* workspace,
                                              int64_t workspace_bytes, void* stream);
/*
 * forge_linear_backward_step_fused_noalloc -- for callers that cannot allocate device memory
 * or hand over a workspace (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation): forge_linear_backward_step_fused with the counters in a static device
 * array of the library (16 KiB, one per device, held until the process ends; its address is
 * resolved on the first call on each device).  Allocates nothing.  Same arguments and results
 * as forge_linear_backward_step_fused without the workspace; K must not exceed 520960
 * ((4096 - 26) x 128 columns, else FORGE_ERR_SHAPE).  Every call on a device uses that device's
 * one array: calls on one device that overlap in time (on different streams, say) race and
 * must not be made; calls in order on one stream are fine, each clears the counters first.
 * The error word of forge_linear_backward_step_fused is kept in that array and is not
 * reported.
 */
forge_status forge_linear_backward_step_fused_noalloc(const forge_tensor* X, const forge_tensor* dY,
                                                      forge_tensor* W, forge_tensor* dX,
                                                      forge_tensor* m, forge_tensor* v,
                                                      const forge_hyper* hyper, int32_t opt,
                                                      int64_t step, uint64_t seed,
                                                      const forge_step_opts* opts, void* stream);
/* Bytes of workspace forge_linear_backward_step_fused needs for a weight of K columns
 * (4 x (26 + K / 128)); -1 for K < 0 or K > 2^40. */
int64_t forge_backward_workspace_bytes(int64_t K);

/*
 * Unfused two-phase baseline (Technical Summary section 1 "The Problem"): the gradient is
 * materialised in a caller-owned fp32 buffer dW[N, K] and a separate kernel applies the rule.
 * The contraction and the rule are the same device code as the fused path, so for the same
 * inputs forge_wgrad_gemm + forge_optimizer_step give bitwise the results of forge_wgrad_step.
 */
forge_status forge_wgrad_gemm(const forge_tensor* X, const forge_tensor* dY, forge_tensor* dW,
                              void* stream);
forge_status forge_optimizer_step(const forge_tensor* dW, forge_tensor* W, forge_tensor* m,
                                  forge_tensor* v, const forge_hyper* hyper, int32_t opt,
                                  int64_t step, uint64_t seed, const forge_step_opts* opts,
                                  void* stream);

/*
 * forge_step_scalars -- host only, no GPU needed: the per-step scalars (computed in fp64,
 * rounded to fp32) that the kernels receive for rule `opt` at step `step`.  Writes up to
 * n_out floats: {decay, l2, c1, c2, c3, b1, omb1, b2, omb2, eps, lr, rectified}.
 */
forge_status forge_step_scalars(int32_t opt, const forge_hyper* hyper, int64_t step, float* out,
                                int32_t n_out);

/* Hash of the sources the library was built from (16 hex digits); a caller can compare it
 * with the sources it ships to make sure a stale binary is never used. */
const char* forge_build_id(void);

const char* forge_status_string(forge_status s);
const char* forge_last_error(void); /* text of this thread's last error ("" if none) */
int32_t forge_version(void);
/* FORGE_OK if `device` exists and is a gfx950 part. */
forge_status forge_device_check(int32_t device);

#ifdef __cplusplus
}
#endif
#endif /* FORGE_H */
