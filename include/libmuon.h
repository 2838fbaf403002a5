/*
 * libmuon -- the Muon optimizer step on one AMD Instinct MI355X (gfx950).
 *
 * One call of muon_step() performs, for every 2-D hidden weight (or every
 * independent row block of one), the momentum update, Frobenius
 * normalization, the Newton-Schulz orthogonalization and the scaled,
 * decoupled-weight-decay update; every other parameter takes the elementwise
 * AdamW fallback.  All work is hand-written HIP for gfx950.
 *
 * Sources (web pages, cited by title and section):
 *   [Blog]      "Muon Optimizer and the Distributed Implementation"
 *   [Moonlight] the Kimi/Moonlight summary page ("...Muon优化器可替代 AdamW..."),
 *               sections "权重衰减机制", "参数更新尺度调整:一致的更新 RMS", "代码"
 *   [DeepSpeed] "DeepSpeed 集成 Muon 优化器实战..." (NS_METHODS, Gram variant)
 *   [MindSpeed] the MindSpeed "Muon 优化器" document (QKV split)
 *
 * Conventions shared by every entry point
 *   - Device pointers are HIP device addresses (e.g. torch tensors'
 *     data_ptr()).  The caller owns every buffer and the stream; the library
 *     never allocates device memory.  Scratch memory is the caller-provided
 *     workspace whose size the *_workspace_bytes queries return.
 *   - Matrices are row-major with a leading dimension equal to their column
 *     count unless an ld argument says otherwise.
 *   - Calls only enqueue work on the given stream (a hipStream_t passed as
 *     void*, NULL = the default stream); they never synchronize the host.
 *   - Every argument is validated on the host before the first launch; on any
 *     error nothing is enqueued and a negative muon_status is returned.
 *   - Non-finite values in the data are not checked; they propagate.
 *   - A workspace may not be used by two calls that overlap in time.
 */
#ifndef LIBMUON_H
#define LIBMUON_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MUON_OK = 0,
  MUON_E_ARG = -1,       /* null/misaligned pointer, bad count, non-finite hparam */
  MUON_E_SHAPE = -2,     /* negative size, split_rows not dividing rows, ... */
  MUON_E_DTYPE = -3,     /* unknown dtype code */
  MUON_E_METHOD = -4,    /* unknown ns_method */
  MUON_E_WORKSPACE = -5, /* workspace null or smaller than required */
  MUON_E_HIP = -6,       /* a HIP runtime call or kernel launch failed */
  MUON_E_PLAN = -7,      /* plan and call disagree (table size, ...) */
  MUON_E_CAPACITY = -8   /* output array too small (query calls) */
} muon_status;

/* [DeepSpeed] NS_METHODS = {standard, gram}: the standard iteration on the
 * m x n unit, or the Gram variant, which iterates on the square R = X X^T
 * (m = min, n = max of the unit's sides).  The Gram chain runs in fp16 with
 * R scaled by a power of two only where that stays within the bf16
 * tolerance on the workload gradients, m >= 512 and n >= 3m.  An explicit
 * MUON_NS_GRAM outside that region is served in a precision that meets the
 * tolerance of the requested compute dtype: with bf16 the unit's Gram
 * iteration runs in fp32 (the bucket reports compute dtype MUON_F32); with fp32 the unit
 * runs the standard iteration (the bucket reports MUON_NS_STANDARD), since
 * an fp32 Gram chain there exceeds the fp32 tolerance.  MUON_NS_AUTO picks
 * Gram exactly inside the region, where it also does less work (executed
 * cost with symmetric products: standard steps (3 m^2 n + m^3), Gram
 * 3 m^2 n + (6 steps - 5) m^3, so Gram is cheaper for n/m > 5/3), and the
 * standard method elsewhere.  MUON_NS_GRAM_RESTART is an extension (the
 * pages describe no restart): the Gram chain with one restart after
 * ceil(steps / 2) steps (steps >= 2), which forms X_r = Q X_0 explicitly,
 * recomputes R = X_r X_r^T from it and continues with Q = I, so the fp16
 * chain's rounding restarts from the rectangular iterate.  A 16-bit unit
 * with m >= 256 runs it in fp16 at any aspect ratio (at most 0.92e-2 where
 * the plain fp16 chain reaches 1.9-17e-2 on small and square shapes; the
 * bucket reports MUON_NS_GRAM_RESTART); a smaller or fp32 unit resolves as
 * for MUON_NS_GRAM.  It costs one more n x m product and one more
 * m x m x n Gram product per unit.
 * Plans report the method and compute dtype of every bucket. */
typedef enum {
  MUON_NS_STANDARD = 0,
  MUON_NS_GRAM = 1,
  MUON_NS_AUTO = 2,
  MUON_NS_GRAM_RESTART = 3
} muon_ns_method;

/* Storage dtype of parameters and gradients.  Momentum and AdamW moments are
 * always fp32. */
typedef enum { MUON_F32 = 0, MUON_BF16 = 1 } muon_dtype;

/* [Moonlight] "代码": parameters tagged use_muon take the Muon rule, the rest
 * (embeddings, heads, norms, biases) take the AdamW backup. */
typedef enum { MUON_KIND_MUON = 0, MUON_KIND_ADAMW = 1 } muon_kind;

/* One row of the shape table (plan time; no pointers).
 *   rows, cols  the 2-D view of the parameter (callers flatten ndim > 2 as
 *               [size(0), -1], as the [Moonlight] code does; vectors 1 x len).
 *   split_rows  0: the whole matrix is one unit.  h > 0: rows must be a
 *               multiple of h and each block of h consecutive rows is
 *               orthogonalized on its own ([MindSpeed] QKV split; per-head
 *               split).  Muon kind only.
 *   scale_dim   0: the update scale is rms_scale*sqrt(max(unit rows, cols));
 *               d > 0: rms_scale*sqrt(d) ([Moonlight] "参数更新尺度调整"). */
typedef struct {
  int32_t kind;   /* muon_kind */
  int32_t dtype;  /* muon_dtype of param and grad */
  int64_t rows;
  int64_t cols;
  int64_t split_rows;
  int64_t scale_dim;
} muon_param_shape;

/* Device pointers of one parameter for one step (same order as the table).
 *   param     rows x cols, dtype; updated in place.
 *   grad      rows x cols, dtype; read only.
 *   momentum  rows x cols fp32 (Muon kind); updated in place.
 *   exp_avg, exp_avg_sq  rows x cols fp32 (AdamW kind); updated in place.
 *   update_out  optional (may be NULL), Muon kind: rows x cols fp32 receives
 *             the orthogonalized update O of every unit (before scaling).
 * Alignment: param/grad to their element size, fp32 buffers to 4 bytes. */
typedef struct {
  void* param;
  const void* grad;
  float* momentum;
  float* exp_avg;
  float* exp_avg_sq;
  float* update_out;
} muon_param_ptrs;

/* Scale of the orthogonalized update O in W <- W (1 - lr wd) - lr scale O,
 * per unit, with d_out x d_in the unit's shape in parameter layout (rows x
 * cols) and D = scale_dim if set, else max(d_out, d_in):
 *   MUON_SCALE_MOONLIGHT  rms_scale * sqrt(D)            ([Moonlight]
 *                         "参数更新尺度调整": matched update RMS, 0.2)
 *   MUON_SCALE_SPECTRAL   sqrt(d_out / d_in)             ([Blog] "Variation
 *                         of Muon Optimizer": dualizing under the RMS->RMS
 *                         norm, the muP form)
 *   MUON_SCALE_UNIT_RMS   sqrt(D)                        ([Blog] DeepSeek-V4
 *                         listing, "Rescale update RMS", with gamma below)
 * each multiplied by extra_scale (the listing's update rescaling factor
 * gamma; [MindSpeed] --muon-extra-scale-factor).  MindSpeed names the modes
 * spectral / unit_rms_norm / shape_scaling without defining them; they are
 * read as SPECTRAL / UNIT_RMS / MOONLIGHT. */
typedef enum {
  MUON_SCALE_MOONLIGHT = 0,
  MUON_SCALE_SPECTRAL = 1,
  MUON_SCALE_UNIT_RMS = 2
} muon_scale_mode;

/* Hyperparameters of one step.
 *   lr, momentum, weight_decay, nesterov, ns_steps: the Muon rule
 *     ([Blog] "Formulation of Muon Optimizer"; [Moonlight] "权重衰减机制").
 *   coeffs: host array of ns_steps*3 floats (a_k, b_k, c_k) or NULL for the
 *     quintic (3.4445, -4.7750, 2.0315) at every step ([Blog] "Newton-Schulz
 *     Iteration").
 *   rms_scale: 0.2 in [Moonlight]; with the default scale mode the update
 *     is W <- W (1 - lr wd) - lr rms_scale sqrt(max(A,B)) O.
 *   scale_mode: muon_scale_mode (0 = MOONLIGHT).
 *   extra_scale: multiplier of the scale; 0 is read as 1 (so a zeroed struct
 *     keeps the default rule).  Must be finite and >= 0.
 *   adam_*: the AdamW backup of the [Moonlight] code; adam_step is t >= 1
 *     (already incremented): W <- W (1 - lr wd) - lr sqrt(1-b2^t)/(1-b1^t) *
 *     m / (eps + sqrt(v)). */
typedef struct {
  float lr;
  float momentum;
  float weight_decay;
  int32_t nesterov;
  int32_t ns_steps;
  const float* coeffs;
  float rms_scale;
  float adam_lr;
  float adam_beta1;
  float adam_beta2;
  float adam_eps;
  float adam_weight_decay;
  int64_t adam_step;
  int32_t scale_mode;
  float extra_scale;
} muon_hparams;

/* Plan options.
 *   ns_method  muon_ns_method.
 *   ns_dtype   -1: Newton-Schulz computes in the parameter dtype (bf16 MFMA
 *              for bf16 parameters, fp32 MFMA for fp32 ones); MUON_F32 or
 *              MUON_BF16 forces one. */
typedef struct {
  int32_t ns_method;
  int32_t ns_dtype;
} muon_plan_options;

typedef struct muon_plan muon_plan;

/* Build an immutable plan from a shape table of n rows (table: host array
 * owned by the caller, read only during the call): units (one per matrix
 * or row block) grouped into buckets of equal (m, n, tall, parameter
 * dtype, compute dtype, method), m = min and n = max of the unit's sides.
 * Which parameters take the Muon rule and which the AdamW backup follows
 * [Moonlight] "代码" (use_muon; Muon only for 2-D weights); a split
 * parameter's row blocks are orthogonalized independently, as the fused QKV
 * weight is in [MindSpeed] "TP 兼容适配" (Q, K, V blocks) and per attention
 * head in [DeepSpeed] (Muon Split); a tall unit is processed as its
 * transpose ([Blog] "Sign of a Matrix": msign(G) = G (G^T G)^(-1/2)).
 * Buckets are numbered by first appearance; units keep table order.  Host
 * only (no HIP call).  opts may be NULL (standard method, compute dtype of
 * the parameters).  *out receives a heap object to release with
 * muon_plan_destroy.  Errors: MUON_E_ARG (null out, n < 0, unknown kind),
 * MUON_E_DTYPE, MUON_E_METHOD, MUON_E_SHAPE (negative size, side > 2^30,
 * split_rows not dividing rows or set on an AdamW row, a unit whose
 * working copy reaches 2^31 bytes); on error *out is NULL. */
muon_status muon_plan_create(const muon_param_shape* table, int32_t n,
                             const muon_plan_options* opts, muon_plan** out);
void muon_plan_destroy(muon_plan* plan);

/* Bytes of device workspace muon_step needs with this plan (host only).
 * The workspace holds, per bucket chunk, the working copies of the
 * Newton-Schulz iteration ([Blog] "Newton-Schulz Iteration": X and its
 * transpose-side products A = X X^T and P = aI + bA + cA^2, or the Gram
 * variant's R, P and Q of [DeepSpeed]), the per-unit norms and the device
 * descriptor tables.  0 for a plan without units or AdamW parameters.
 * Errors: MUON_E_ARG (null plan or bytes). */
muon_status muon_plan_workspace_bytes(const muon_plan* plan, size_t* bytes);

/* Bit-exact view of the plan (host only).  Buckets: 8 int32 per bucket
 * (m, n, tall, param dtype, compute dtype, method, first unit, unit count);
 * units, listed bucket by bucket: 6 int64 per unit (param, row0, rows, cols,
 * tall, scale_dim as resolved).  *len receives the number of values needed;
 * with out == NULL and cap == 0 this is a size query (MUON_OK), otherwise a
 * cap below it returns MUON_E_CAPACITY and writes nothing. */
muon_status muon_plan_buckets(const muon_plan* plan, int32_t* out, size_t cap, size_t* len);
muon_status muon_plan_units(const muon_plan* plan, int64_t* out, size_t cap, size_t* len);

/* One optimizer step for every parameter of the plan's table (n must equal
 * the table size; ptrs: host array of n entries in table order, read only
 * during the call; hp: host struct, read only during the call).
 * Per Muon unit ([Blog] "Formulation of Muon Optimizer" and "Newton-Schulz
 * Iteration"; [Moonlight] "权重衰减机制", "参数更新尺度调整" and "代码"):
 *   M <- mu M + G;  U = G + mu M (nesterov) or M;  X0 = U / ||U||_F;
 *   X <- a_k X + (b_k A + c_k A^2) X, A = X X^T, k = 0 .. ns_steps-1
 *     (or the Gram variant of [DeepSpeed]);
 *   W <- W (1 - lr wd) - lr scale O, scale per muon_scale_mode;
 * a unit whose U is zero gets O = 0 (its weight only decays).  Per AdamW
 * parameter: the AdamW backup of [Moonlight] "代码" (see muon_hparams).
 * param, momentum, exp_avg, exp_avg_sq are updated in place and update_out
 * written; grad is read only.  workspace: device memory of at least
 * muon_plan_workspace_bytes bytes, owned by the caller; its contents need
 * not be initialized and are scratch between calls.  The per-unit
 * descriptors reach the workspace through the arguments of small kernel
 * launches (3 KiB each), not through a host-to-device copy, so the call
 * only enqueues work on stream (a hipStream_t, NULL = default stream) and
 * returns without waiting for the GPU.  Errors, all before the first
 * launch: MUON_E_PLAN (n
 * differs from the table), MUON_E_ARG (null plan, hp or ptrs; a required
 * pointer null or misaligned; a non-finite or out-of-range hparam),
 * MUON_E_WORKSPACE; MUON_E_HIP if a HIP call fails. */
muon_status muon_step(const muon_plan* plan, const muon_param_ptrs* ptrs, int32_t n,
                      const muon_hparams* hp, void* workspace, size_t workspace_bytes,
                      void* stream);

/* Newton-Schulz orthogonalization of one matrix X (device memory, rows x
 * cols, leading dimension ld >= cols elements, dtype MUON_F32 or MUON_BF16),
 * in place: X <- NS_steps(X / ||X||_F) ([Blog] "Newton-Schulz Iteration":
 * X <- a_k X + (b_k A + c_k A^2) X with A = X X^T), a tall X being processed
 * as its transpose ([Blog] "Sign of a Matrix"); method standard, Gram
 * ([DeepSpeed]; resolved as described above), auto, or the restarted Gram
 * chain (an extension, resolved as described above).
 * coeffs: host array of steps x 3 floats as in muon_hparams, or NULL.  A
 * zero matrix stays zero.  workspace: device memory of at least
 * ns_orthogonalize_workspace_bytes bytes, owned by the caller, contents
 * need not be initialized.  Enqueues on stream and returns.  Errors, before
 * any launch: MUON_E_DTYPE, MUON_E_METHOD, MUON_E_SHAPE (negative size,
 * ld < cols, a side above 2^30 or a working copy of 2^31 bytes or more),
 * MUON_E_ARG (X null or misaligned, steps out of [1, 64], a non-finite
 * coefficient), MUON_E_WORKSPACE; MUON_E_HIP if a launch fails. */
muon_status ns_orthogonalize(void* X, int64_t rows, int64_t cols, int64_t ld, int32_t dtype,
                             int32_t steps, const float* coeffs, int32_t method,
                             void* workspace, size_t workspace_bytes, void* stream);
muon_status ns_orthogonalize_workspace_bytes(int64_t rows, int64_t cols, int32_t dtype,
                                             int32_t method, size_t* bytes);

/* ns_orthogonalize without a workspace argument, for callers that cannot
 * allocate device memory (code under stream capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The arguments of ns_orthogonalize less
 * the workspace; the same result and errors as
 * ns_orthogonalize, with the same kernels; the scratch memory is a device
 * array of MUON_NOALLOC_SCRATCH_BYTES inside the library, one per GPU the
 * library is loaded on, held until the process ends.  The call allocates
 * nothing: no hipMalloc / hipFree, no host staging.  Matrices whose
 * ns_orthogonalize_workspace_bytes exceed MUON_NOALLOC_SCRATCH_BYTES (e.g. a
 * bf16 2048 x 4096 fits, a 4096 x 4096 does not) return MUON_E_WORKSPACE
 * before any launch.  Every call on one GPU uses that GPU's one array: calls
 * that overlap in time on the same GPU (two streams, two threads) race and
 * must be serialized by the caller.  The array's contents after a call are
 * unspecified; nothing needs to be zero before one.  MUON_E_HIP if the
 * array's device address cannot be obtained. */
#define MUON_NOALLOC_SCRATCH_BYTES (64u << 20)
muon_status ns_orthogonalize_noalloc(void* X, int64_t rows, int64_t cols, int64_t ld, int32_t dtype,
                                     int32_t steps, const float* coeffs, int32_t method, void* stream);

/* Optional per-kernel timing, for benchmarks.  While enabled (process-wide),
 * every kernel launch of the library is bracketed by two HIP events recorded
 * on the launch's stream, tagged with the kernel family and the algorithmic
 * FLOPs / HBM bytes of that launch:
 *   flops  Newton-Schulz contractions: 2*m*m*n (X X^T and P X) or 2*m^3
 *          (A A and the Gram m x m products) per unit, counted as dense
 *          products even where symmetry halves the executed work;
 *   bytes  elementwise kernels: bytes each element must move (momentum:
 *          G + M read + M write + U write; AdamW: W r/w, G, m r/w, v r/w).
 * muon_timing_collect waits for the recorded events, writes one entry per
 * family into out (up to cap), sets *n to the number of families seen, and
 * clears the records. */
typedef struct {
  char name[32];
  int64_t launches;
  double total_ms;
  double flops;
  double bytes;
} muon_kernel_timing;

muon_status muon_timing_enable(int32_t enable);
muon_status muon_timing_collect(muon_kernel_timing* out, int32_t cap, int32_t* n);

/* Measurement aids for benchmarks; not part of the optimizer step.  Both
 * only enqueue on stream (a hipStream_t, null = default stream) and return.
 * muon_probe_mfma: the device's sustained bf16 matrix-core rate.  Launches
 *   `workgroups` workgroups of 4 waves; each wave runs `iters` rounds of 8
 *   independent v_mfma_f32_32x32x16_bf16 from registers, and each workgroup
 *   writes one float to sink (device memory, `workgroups` floats, owned by
 *   the caller).  *flops (host) receives the FLOPs of the launch
 *   (workgroups * 4 * iters * 8 * 32768).  MUON_E_ARG if a count is not
 *   positive or a pointer is null; MUON_E_HIP if the launch fails.
 * muon_probe_copy: the device's streaming copy rate.  Copies `bytes` from
 *   src to dst (device memory, non-overlapping, owned by the caller) with
 *   16-byte non-temporal loads and stores, one contiguous 16 KiB block per
 *   workgroup; 2 * bytes move through HBM.
 *   MUON_E_ARG if bytes is 0 or not a multiple of 16, or a pointer is null
 *   or not 16-byte aligned; MUON_E_HIP if the launch fails. */
muon_status muon_probe_mfma(int32_t workgroups, int32_t iters, float* sink, double* flops, void* stream);
muon_status muon_probe_copy(const void* src, void* dst, size_t bytes, void* stream);
/* muon_probe_copy_lds: the same copy through the Newton-Schulz GEMMs' load
 *   path (global -> LDS with buffer_load_dwordx4 ... lds at the default cache
 *   policy, then LDS -> global with ordinary 16-byte stores), one 16 KiB
 *   block per workgroup; calibrates memory counters for those loads.  Same
 *   arguments and errors as muon_probe_copy. */
muon_status muon_probe_copy_lds(const void* src, void* dst, size_t bytes, void* stream);

/* Newton-Schulz coefficient schedules: writes steps x 3 floats (a_k, b_k,
 * c_k) to out (capacity cap floats) for muon_hparams.coeffs.
 *   MUON_COEFF_QUINTIC  (3.4445, -4.7750, 2.0315) at every step ([Blog]
 *                       "Newton-Schulz Iteration"; [MindSpeed]
 *                       --muon-coefficient-type quintic).
 *   MUON_COEFF_HYBRID   the quintic for steps-2 steps, then two refining
 *                       steps ([Blog] DeepSeek-V4 listing: HybridNewtonSchulz,
 *                       ten steps, eight with the quintic and two with an
 *                       improved Newton iteration that brings the singular
 *                       values closer to 1).  The refined coefficients are not
 *                       printed; the reading taken is (15/8, -5/4, 3/8), the
 *                       odd quintic with p(1) = 1, p'(1) = p''(1) = 0 (the
 *                       second-order expansion of [Blog] "Sign of a Matrix").
 *                       steps >= 2.
 * Errors: MUON_E_ARG (unknown kind, steps out of [1, 64], hybrid with
 * steps < 2, null out), MUON_E_CAPACITY (cap < 3 steps). */
typedef enum { MUON_COEFF_QUINTIC = 0, MUON_COEFF_HYBRID = 1 } muon_coeff_kind;
muon_status muon_ns_coefficients(int32_t kind, int32_t steps, float* out, size_t cap);

/* Static text for a status code. */
const char* muon_status_string(int32_t status);

/* Library version (major*10000 + minor*100 + patch). */
int32_t muon_version(void);

#ifdef __cplusplus
}
#endif
#endif /* LIBMUON_H */
