/*
 * muon_step.h - C ABI of an MI355X (gfx950) Muon optimizer step.
 *
 * One call performs, for every weight matrix W (n x m) it is given, the
 * DeepSeek-V4 Muon update (the Muon deep-dive page "Muon 优化器完全拆解",
 * section "V4 的完整更新公式，逐行拆解"; the DeepSeek-V4 book, ch. 6 "Muon",
 * section 5, whose expanded Algorithm 1 writes the normalisation out):
 *
 *     M_t  = mu * M_{t-1} + G_t                  momentum accumulate
 *     N_t  = mu * M_t + G_t                      Nesterov input (nesterov = 1)
 *     X    = N_t / ||N_t||_F                     (Gram taken on the smaller side)
 *     for each (a, b, c) of the schedule:  X = a X + b (X X^T) X + c (X X^T)^2 X
 *     O_t  = X * sqrt(max(n, m)) * gamma
 *     W_t  = (1 - lr * wd) * W_{t-1} - lr * O_t
 *
 * and a second entry point runs the elementwise AdamW step that the pages
 * assign to embedding and prediction-head tensors (the deep-dive page,
 * section "为什么嵌入层、输出头、bias、RMSNorm 还在用 AdamW").
 *
 * Conventions shared by every entry point:
 *   - Pointers documented as "device" point to memory of the context's GPU;
 *     "host" pointers are read before the call returns and may be freed then.
 *   - Matrices are row-major and contiguous (row pitch == cols elements).
 *   - Work is enqueued on the given HIP stream (NULL = the null stream), and
 *     by muon_step also on side streams of the context that are forked from
 *     it and joined back to it within the call, so that all of it is ordered
 *     like work of the given stream; no entry point synchronises the stream
 *     except where stated.
 *   - Every argument is validated before anything is enqueued: a non-OK
 *     status means no work was enqueued.  Launch failures return
 *     MUON_ERR_DEVICE.  No C++ exception crosses this boundary.
 *   - A context is not thread-safe; calls on one context must be ordered by
 *     the caller (one stream at a time, or explicit synchronisation).
 *   - Results are deterministic: identical inputs give bit-identical outputs
 *     (no atomics in any reduction).
 */
#ifndef MUON_STEP_H
#define MUON_STEP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MUON_STEP_ABI_VERSION 4

/* Bytes of the fixed per-GPU device scratch muon_step_noalloc works in. */
#define MUON_NOALLOC_SCRATCH_BYTES 134217728

typedef enum muon_status {
    MUON_OK = 0,
    MUON_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad size, aliasing, bad enum    */
    MUON_ERR_UNSUPPORTED = 2,      /* valid but not implemented (dtype combination)  */
    MUON_ERR_OUT_OF_MEMORY = 3,    /* workspace could not be allocated within cap    */
    MUON_ERR_DEVICE = 4            /* a HIP call or kernel launch failed             */
} muon_status;

typedef enum muon_dtype {
    MUON_F32 = 0,  /* IEEE binary32                                   */
    MUON_BF16 = 1  /* bfloat16; every cast to it rounds to nearest even */
} muon_dtype;

/* Arithmetic of the Newton-Schulz products.
 * MUON_NS_BF16: bf16 MFMA operands, fp32 accumulation; between iterations X
 *               is kept as a bf16 hi (x rounded to nearest, low halves
 *               from 0x7f80 rounding up) plus an 8-bit residual, the pair
 *               carrying x to 2^-16 of its magnitude; hi is the MFMA operand
 *               (relative Frobenius error vs fp64 ~1e-2).
 *               Matrices whose smaller side is at most 16 use the fp32
 *               products instead (too few singular directions for the bf16
 *               rounding of X to average out; their cost is negligible).
 * MUON_NS_F32:  fp32 MFMA operands and accumulation (error vs fp64 ~1e-6). */
typedef enum muon_ns_precision { MUON_NS_BF16 = 0, MUON_NS_F32 = 1 } muon_ns_precision;

/* How the orthogonalised update O'_t (n x m) is scaled into O_t.
 * MUON_SCALE_SQRT_MAX: O_t = O'_t * sqrt(max(n, m)) * gamma, the shape rule of
 *                      DeepSeek-V4's Algorithm 1 (the deep-dive page, "V4 的
 *                      完整更新公式，逐行拆解" and "更新尺度").
 * MUON_SCALE_UNIT_RMS: O_t = O'_t * gamma / RMS(O'_t), RMS(X) = ||X||_F /
 *                      sqrt(n m): the update divided by its own RMS, then
 *                      multiplied by gamma as the extra scale factor (the
 *                      deep-dive page's Megatron-Bridge recipe,
 *                      muon_scale_mode "unit_rms_norm" with
 *                      muon_extra_scale_factor 0.2).  ||O'_t|| is reduced on
 *                      the device in fp64 from the fp32 values of O'_t;
 *                      O'_t = 0 gives a zero scale (decay-only update).  Costs
 *                      one extra read of X and an unfused update pass. */
typedef enum muon_scale_mode { MUON_SCALE_SQRT_MAX = 0, MUON_SCALE_UNIT_RMS = 1 } muon_scale_mode;

/* One Newton-Schulz step X <- a X + b (X X^T) X + c (X X^T)^2 X
 * (DeepSeek-V4 book ch. 6, section 3).  Passed to kernels as fp32. */
typedef struct muon_ns_coeff {
    double a, b, c;
} muon_ns_coeff;

/* One weight matrix handed to muon_step.  Layout: row-major rows x cols.
 *   param    device, param_dtype, W_{t-1} in, W_t out (in place)
 *   grad     device, grad_dtype, G_t, read only
 *   momentum device, fp32, M_{t-1} in, M_t out (in place); the single buffer
 *            also serves the Nesterov input (the deep-dive page, Nesterov step)
 *   ns_out   optional device fp32 rows x cols; when non-NULL it receives the
 *            orthogonalised update O'_t before the sqrt(max)*gamma rescale
 *            (diagnostics and parity checks).  NULL: nothing is written.
 * grad must not overlap param, momentum or ns_out; momentum must not overlap
 * param; no two matrices of one call may share param or momentum memory. */
typedef struct muon_matrix {
    void *param;
    const void *grad;
    float *momentum;
    float *ns_out;
    int64_t rows;
    int64_t cols;
    int32_t param_dtype; /* muon_dtype */
    int32_t grad_dtype;  /* muon_dtype */
} muon_matrix;

/* Hyper-parameters of Algorithm 1 (the deep-dive page's Algorithm 1 inputs:
 * learning rate, momentum, weight decay, update scale gamma) plus the
 * Newton-Schulz schedule.
 *   schedule      host array of num_ns_steps coefficient triples, applied in
 *                 order; may be NULL only when num_ns_steps == 0.  The
 *                 DeepSeek-V4 hybrid schedule is returned by
 *                 muon_schedule("deepseekv4", ...).
 *   num_ns_steps  0..64.  0 means X = N / ||N||_F with no iteration.
 *   nesterov      1: NS input mu*M_t + G_t;  0: NS input M_t.
 *   ns_precision  muon_ns_precision.
 *   scale_mode    muon_scale_mode (other values: INVALID_ARGUMENT).
 * lr, momentum, weight_decay and gamma must be finite. */
typedef struct muon_hparams {
    double lr;
    double momentum;
    double weight_decay;
    double gamma;
    const muon_ns_coeff *schedule;
    int32_t num_ns_steps;
    int32_t nesterov;
    int32_t ns_precision;
    int32_t scale_mode; /* muon_scale_mode */
} muon_hparams;

/* One tensor handed to muon_adamw_step: numel contiguous fp32 elements each
 * of param (in/out), grad (in), exp_avg (in/out) and exp_avg_sq (in/out).
 * param_dtype and grad_dtype must be MUON_F32 (other values: UNSUPPORTED).
 * grad must not overlap the other three; no two of param, exp_avg and
 * exp_avg_sq may overlap. */
typedef struct muon_adamw_tensor {
    void *param;
    const void *grad;
    float *exp_avg;
    float *exp_avg_sq;
    int64_t numel;
    int32_t param_dtype;
    int32_t grad_dtype;
} muon_adamw_tensor;

/* AdamW with bias correction and decoupled multiplicative decay:
 *   p <- (1 - lr wd) p;  m <- b1 m + (1-b1) g;  v <- b2 v + (1-b2) g^2;
 *   p <- p - lr * (m / (1 - b1^step)) / (sqrt(v / (1 - b2^step)) + eps)
 * in fp32 with one rounding per operation in exactly this order (correctly
 * rounded division and square root); the scalars 1-lr*wd, 1-b1, 1-b2,
 * 1-b1^step, 1-b2^step are formed in double and rounded once.
 * step >= 1 counts the steps including this one. */
typedef struct muon_adamw_hparams {
    double lr;
    double beta1;
    double beta2;
    double eps;
    double weight_decay;
    int64_t step;
} muon_adamw_hparams;

typedef struct muon_context muon_context; /* opaque */

/* ABI version of the loaded library (MUON_STEP_ABI_VERSION it was built with). */
int32_t muon_abi_version(void);

/* Static, never-NULL description of a status code. */
const char *muon_status_string(muon_status status);

/* Named coefficient schedules from the pages:
 *   "deepseekv4": 8 x (3.4445, -4.7750, 2.0315) then 2 x (2, -1.5, 0.5)
 *                 (DeepSeek-V4 book ch. 6, sections 4-5)
 *   "quintic":    5 x (3.4445, -4.7750, 2.0315) (the deep-dive page,
 *                 "系数怎么调出来的" and the Megatron-Bridge recipe)
 * Writes min(count, capacity) triples to out (host; may be NULL when
 * capacity is 0) and returns the schedule's length, or -1 for an unknown
 * name.  Pure host function. */
int64_t muon_schedule(const char *name, muon_ns_coeff *out, int64_t capacity);

/* Host-only validation of a muon_step argument list: the exact checks
 * muon_step performs before it enqueues anything.  Touches no GPU.  On
 * failure writes a NUL-terminated reason into msg (host, msg_cap bytes;
 * msg may be NULL when msg_cap is 0). */
muon_status muon_check_step_args(const muon_matrix *mats, int64_t count, const muon_hparams *hp,
                                 char *msg, size_t msg_cap);

/* Host-only validation of a muon_adamw_step argument list. */
muon_status muon_check_adamw_args(const muon_adamw_tensor *ts, int64_t count,
                                  const muon_adamw_hparams *hp, char *msg, size_t msg_cap);

/* Workspace the library would allocate for this argument list when nothing
 * caps it: the largest per-group chunk of Newton-Schulz buffers (with
 * concurrent groups, the largest of each lane's groups summed over the
 * lanes) plus the per-matrix tables.  Pure host function; validates like
 * muon_check_step_args. */
muon_status muon_workspace_bytes(const muon_matrix *mats, int64_t count, const muon_hparams *hp,
                                 size_t *bytes_out);

/* Creates a context on HIP device hip_device.  workspace_cap_bytes bounds
 * the Newton-Schulz workspace the context may hold (0 = no bound); matrices
 * of one shape are processed in chunks that fit it.  *out receives the
 * context (host pointer) or NULL on failure. */
muon_status muon_create(muon_context **out, int32_t hip_device, size_t workspace_cap_bytes);

/* Waits for the context's outstanding uploads, frees its device memory and
 * the context.  NULL is accepted (no-op).  Work already enqueued by the
 * caller on its streams must be complete or ordered before the free. */
muon_status muon_destroy(muon_context *ctx);

/* Last error message of this context (host string owned by the context,
 * valid until its next call); "" when the last call succeeded. */
const char *muon_last_error(const muon_context *ctx);

/* One Muon step over `count` matrices (host array mats).  Matrices with the
 * same (rows, cols, param_dtype, grad_dtype) are batched: every stage runs
 * as one grouped launch over all of them.  A matrix whose N_t is all zero
 * gets the decay-only update W_t = (1 - lr wd) W_{t-1}.  The result does not
 * depend on the scale of N_t: any finite nonzero ||N_t|| is applied exactly
 * (an N_t outside ||N||_F^2 in [2^-40, 2^40] is normalised in double before
 * the first product).  Non-finite values propagate (IEEE): an Inf or NaN in
 * N_t makes ||N_t||^2 non-finite (muon_last_norms) and every element of
 * O'_t and W_t NaN, as the exact Algorithm 1 does (X = N / ||N|| is NaN
 * where N is infinite, and every product spreads it).  Groups of different
 * shapes are independent ("each logically independent weight", DeepSeek-V4
 * book ch. 6 §5): unless disabled (muon_set_concurrent_groups) they run
 * concurrently on up to three side streams that the context creates (at the
 * default priority), forked from hip_stream by an event and joined back to
 * it before the call returns, each lane of groups in a workspace slice of
 * its own; a nonzero workspace cap that those slices together would exceed
 * runs the groups in turn instead.  Either way the results are the same,
 * bit for bit. */
muon_status muon_step(muon_context *ctx, const muon_matrix *mats, int64_t count,
                      const muon_hparams *hp, void *hip_stream);

/* Enables (1, the default) or disables (0) the concurrent execution of a
 * muon_step call's groups described above; disabled, every group runs in
 * turn on the caller's stream in one workspace.  Per-stage timing
 * (muon_profile_enable) and muon_step_noalloc always run them in turn.
 * Returns MUON_ERR_INVALID_ARGUMENT for a NULL context or another value. */
muon_status muon_set_concurrent_groups(muon_context *ctx, int32_t enable);

/* For callers that cannot allocate device memory during a step (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * muon_step with the same arguments, results bit-identical to muon_step's,
 * that allocates nothing.  Its workspace, norm tables and descriptor table
 * live in a static device array of MUON_NOALLOC_SCRATCH_BYTES (128 MiB)
 * that every GPU the library runs on holds from muon_create until the
 * process ends; groups of same-shape matrices are processed in chunks that
 * fit it.  A call whose matrices cannot fit (one bf16 2048 x 7168 matrix
 * needs 90 MB; a 4096 x 4096 one does not fit) or that has more than 16384
 * matrices returns MUON_ERR_OUT_OF_MEMORY before anything is enqueued.
 * Every call on one GPU shares that GPU's array (across contexts too), and
 * calls that overlap on one GPU race: order them on one stream or
 * synchronise.  muon_last_norms reads from the array, so it is valid until
 * the next muon_step_noalloc on that GPU.  With per-stage timing enabled
 * (muon_profile_enable) the call may create HIP events. */
muon_status muon_step_noalloc(muon_context *ctx, const muon_matrix *mats, int64_t count,
                              const muon_hparams *hp, void *hip_stream);

/* One AdamW step over `count` tensors (host array ts), one launch. */
muon_status muon_adamw_step(muon_context *ctx, const muon_adamw_tensor *ts, int64_t count,
                            const muon_adamw_hparams *hp, void *hip_stream);

/* Normalisation + Newton-Schulz only: x_out (device fp32 rows x cols)
 * receives NS(n_in / ||n_in||_F) for the device fp32 rows x cols input n_in,
 * with hp's schedule and precision (lr, momentum, weight_decay, gamma,
 * nesterov and scale_mode are ignored).  n_in and x_out must not overlap. */
muon_status muon_ns_only(muon_context *ctx, const float *n_in, float *x_out, int64_t rows,
                         int64_t cols, const muon_hparams *hp, void *hip_stream);

/* Decay + update given an orthogonalised update x (device fp32 rows x cols,
 * the unscaled O'_t):  param <- fl(fl(d * param) - fl(s * x)) with
 * d = fl32(1 - lr*wd), s = fl32(lr * gamma * sqrt(max(rows, cols))) (unit-RMS
 * mode: s = fl32(lr * (gamma * sqrt(rows * cols) / ||x||_F)), 0 for x = 0,
 * ||x||^2 summed on the device in fp64), rounded to bf16 (nearest even) when
 * param_dtype is MUON_BF16.  Exactly the arithmetic muon_step's last stage
 * performs. */
muon_status muon_apply_update(muon_context *ctx, void *param, int32_t param_dtype, const float *x,
                              int64_t rows, int64_t cols, const muon_hparams *hp,
                              void *hip_stream);

/* Test hook: one Newton-Schulz product of the bf16 path on one matrix, with
 * its operands rounded as that path rounds them (DeepSeek-V4 book ch. 6,
 * section 3: one step is X <- a X + b A X + c A^2 X with A = X X^T, here
 * split into its three products).  X is s x l with 1 <= s <= l (X's own
 * orientation; muon_step transposes W with rows > cols into it).  All
 * pointers are device fp32, row-major; out must not overlap the inputs.
 *   MUON_STAGE_GRAM:  x (s x l) -> out (s x s):  A = X_hi X_hi^T, X_hi the
 *                     bf16 hi of x as stored in the pair (MUON_NS_BF16);
 *                     fp32 accumulation, A rounded to bf16.
 *   MUON_STAGE_POLY:  m (s x s, symmetric; rounded to bf16 as A) -> out
 *                     (s x s):  B = b A + c A A, fp32 accumulation, B
 *                     rounded to bf16.
 *   MUON_STAGE_APPLY: m (s x s, symmetric; rounded to bf16 as B), x (s x l,
 *                     kept as the pair X_hi plus its 8-bit residual) ->
 *                     out (s x l):  X' = a X + B X_hi (aX from hi + residual,
 *                     fp32 accumulation), as the value of the pair X' is
 *                     stored in.
 * The products run exactly as inside muon_step for a single matrix of this
 * shape (same tiles, same split of long K loops). */
#define MUON_STAGE_GRAM 0
#define MUON_STAGE_POLY 1
#define MUON_STAGE_APPLY 2
muon_status muon_ns_stage(muon_context *ctx, int32_t stage, const float *x, const float *m, float *out, int64_t s,
                          int64_t l, double a, double b, double c, void *hip_stream);

/* Blocks until the context's device memory holds the per-matrix squared
 * Frobenius norms of the last muon_step's N_t (matrix order of that call)
 * and copies min(count, capacity) of them to out (host doubles).  Returns
 * the count through *count_out.  Synchronises the last call's stream. */
muon_status muon_last_norms(muon_context *ctx, double *out, int64_t capacity, int64_t *count_out);

/* Measurement aid, no step of the method: streams `reads` source streams of
 * stream_bytes each (src, device; stream k starts k * pitch_bytes into it)
 * and `writes` destination streams (dst, device, the same pitch), every
 * 16-byte vector read and written once, coalesced, each written vector
 * depending on its thread's reads.  Its rate is the HBM ceiling for a kernel
 * with that read : write mix, the reference for the elementwise kernels'
 * GB/s: (reads, writes) = (6, 7) the momentum pass (bf16 G 2 + M 4 bytes
 * read, M 4 + X 3 written per element), (4, 3) AdamW, (5, 2) the separate
 * update pass, (1, 1) a copy; others UNSUPPORTED.  stream_bytes and
 * pitch_bytes (>= stream_bytes) must be multiples of 16, src and dst 16-byte
 * aligned and disjoint.  Timed as stage "stream_probe". */
muon_status muon_stream_probe(muon_context *ctx, const void *src, void *dst, int64_t stream_bytes,
                              int64_t pitch_bytes, int32_t reads, int32_t writes, void *hip_stream);

/* Per-stage timing of a context's launches.  While enabled, every kernel
 * launch the context makes is bracketed by two HIP events recorded on the
 * stream it is launched on; the stage's algorithmic work of that launch (the
 * FLOPs the method must do, counting one triangle of the symmetric X X^T and
 * A A, and the bytes it must move to and from HBM) is recorded with it.
 * Stage names: "momentum_nesterov", "norm_finalize", "normalize", "gram",
 * "poly", "apply", "apply_update" (the last product with the fused decay and
 * update), "update", "adamw", "import", "export", "unit_rms" (the per-matrix
 * ||X||^2 reduction and scale of the unit-RMS mode), "stream_probe"
 * (muon_stream_probe), "prenormalize" (the bf16
 * path's normalisation of the matrices whose ||N_t|| lies outside the range
 * in which the first step folds 1/||N_t|| into its products). */
typedef struct muon_stage_stats {
    char name[32];
    int64_t launches;
    double total_ms; /* sum of the launches' event-measured durations */
    double flops;    /* algorithmic FLOPs of those launches             */
    double bytes;    /* algorithmic HBM bytes of those launches         */
} muon_stage_stats;

/* Enables (1) or disables (0) per-stage timing and discards what was
 * recorded so far.  Disabled by default. */
muon_status muon_profile_enable(muon_context *ctx, int32_t enable);

/* Waits for the recorded events, aggregates them per stage into out (host,
 * capacity entries, stages in first-launch order), writes the number of
 * stages to *count and discards the records. */
muon_status muon_profile_read(muon_context *ctx, muon_stage_stats *out, int32_t capacity, int32_t *count);

#ifdef __cplusplus
}
#endif

#endif /* MUON_STEP_H */
