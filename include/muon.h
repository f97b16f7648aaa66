/*
 * muon.h - C ABI of an MI355X (gfx950) library that performs one Muon optimizer step over a
 * list of 2-D weight matrices.
 *
 * The step, as the pages describe it:
 *   - page "深入解析KellerJordan/modded-nanogpt中的训练架构与优化技术", section
 *     "Muon优化器：动量正交化技术", subsection "核心算法": an optimizer with defaults
 *     lr = 0.02, momentum = 0.95, nesterov = true, ns_steps = 5, whose step is (1) a
 *     standard SGD momentum update, (2) Newton-Schulz orthogonalisation, (3) the parameter
 *     update;
 *   - same page, subsection "Newton-Schulz正交化": ns_steps rounds of A = X X^T,
 *     B = b A + c A A, X = a X + B X with (a, b, c) = (3.4445, -4.7750, 2.0315), run in
 *     bfloat16;
 *   - page "Muon优化器与FP8混合精度：AI训练能效革命与绿色计算新范式", section
 *     "Muon优化器的能效突破": Muon is momentum orthogonalised by Newton-Schulz.
 *
 * What one call computes for every matrix (W param, G grad, M momentum, all rows x cols):
 *   M <- beta * M + G                                (fp32 buffer, fp32 arithmetic)
 *   U  = G + beta * M  if nesterov, else U = M
 *   X  = U / (||U||_F + eps)                         (Frobenius pre-normalisation; the
 *        printed iteration omits it, and the record analysis at lqnn.cn, section 3.2,
 *        names Frobenius normalisation in front of the quintic maps)
 *   if rows > cols the iteration runs on X^T (wide form) and the result is transposed back
 *   ns_steps rounds of the quintic iteration above
 *   W <- W - lr * O                                  (O = the iteration's result)
 * With cfg->row_equalize set, O is first passed through a per-row energy equaliser (the
 * record analysis at lqnn.cn, section 3.2, names NorMuon's per-lane energy equaliser, an
 * Adafactor-style variance estimate, after the orthogonalisation; it prints no formula, so
 * this is the plainest reading): with v the matrix's per-row state (rows fp32 values),
 *   v_i <- row_beta * v_i + (1 - row_beta) * mean_j O_ij^2      (rows of the caller's layout)
 *   D_ij = O_ij / (sqrt(v_i) + row_eps)
 *   O   <- D * ||O||_F / ||D||_F                     (total energy kept; 0 stays 0)
 *
 * Range: every finite fp32 value of U is supported. The norm is summed in double, and a
 * matrix whose ||U||_F lies outside [2^-40, 2^40] has its copy in the iteration's workspace
 * scaled by an exact power of two before the first product, with the inverse power folded
 * into 1/(||U||_F + eps); the fp32 accumulation of the products then neither overflows nor
 * underflows. (The rescale is one extra pass over that matrix, taken only for such inputs.)
 * Products whose fp32 value is subnormal (below 2^-126) may be flushed to zero.
 *
 * Conventions shared by every entry point:
 *   - All buffers are device memory on the current HIP device, row-major, contiguous, with
 *     16-byte aligned base addresses. The caller owns every buffer.
 *   - Work is enqueued on `stream` and the call returns without synchronising. Buffers must
 *     stay alive and untouched by other work until the stream has passed the call.
 *   - Calls on one plan must be ordered (same stream, or synchronised between calls).
 *   - Arguments are validated on the host before anything is enqueued: a call that returns
 *     an error has enqueued nothing. muon_last_error() then describes the failure.
 *   - NaN and Inf are propagated, not checked; they never leak from one matrix into another.
 */
#ifndef MUON_H
#define MUON_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h> /* hipStream_t */

#ifdef __cplusplus
extern "C" {
#endif

typedef struct muon_plan muon_plan; /* opaque; holds host metadata only */

typedef enum {
  MUON_OK = 0,
  MUON_ERR_INVALID_ARG = -1, /* null pointer, bad size, misalignment, overlap, mismatch */
  MUON_ERR_UNSUPPORTED = -2, /* a shape or dtype outside the library's limits */
  MUON_ERR_WORKSPACE = -3,   /* workspace missing, misaligned or too small */
  MUON_ERR_HIP = -4          /* a HIP runtime call failed (launch error, bad stream) */
} muon_status;

typedef enum { MUON_DT_BF16 = 0, MUON_DT_F32 = 1 } muon_dtype;

/* Arithmetic of the Newton-Schulz rounds.
 *   MUON_NS_BF16:      X, A and B stored in bfloat16 (the pages' precision), products on
 *                      bf16 matrix cores with fp32 accumulation, fp32 epilogues.
 *   MUON_NS_F32_DEBUG: the same rounds with fp32 storage and fp32 arithmetic, to separate
 *                      the method from its bf16 rounding. */
typedef enum { MUON_NS_BF16 = 0, MUON_NS_F32_DEBUG = 1 } muon_precision;

/* One matrix of a step.
 *   param       rows x cols, param_dtype, updated in place (W <- W - lr*O, computed in fp32
 *               and rounded to nearest even when param_dtype is bf16)
 *   grad        rows x cols, grad_dtype, read only
 *   momentum    rows x cols fp32, updated in place; zero-fill it before the first step
 *   update_out  NULL, or rows x cols fp32 that receives O (the orthogonalised update, in the
 *               matrix's own orientation, before the lr scaling; the equalised O when
 *               cfg->row_equalize is set)
 *   row_var     NULL, or rows fp32: the row equaliser's per-row state v, updated in place;
 *               zero-fill it before the first step. Required when cfg->row_equalize is set,
 *               ignored otherwise.
 * rows, cols and the dtypes must equal the plan's entry at the same index. */
typedef struct {
  void *param;
  const void *grad;
  float *momentum;
  float *update_out;
  int64_t rows;
  int64_t cols;
  muon_dtype param_dtype;
  muon_dtype grad_dtype;
  float *row_var;
} muon_matrix;

/* Hyper-parameters of a step. lr, beta (momentum), nesterov and ns_steps follow the
 * optimizer's constructor on the pages; (a, b, c) are the quintic's coefficients; eps guards
 * the normalisation of an all-zero update. ns_steps may be 0 (O = U / (||U||_F + eps)) and
 * is at most 64. Every float must be finite; eps >= 0.
 *
 * schedule: NULL (every round uses (a, b, c)), or a host array of ns_steps triples
 * {a_k, b_k, c_k}, k = 0..ns_steps-1, one quintic per round: the mechanism behind the record
 * analysed at lqnn.cn (section 3.2), which replaces the fixed quintic by a cascade of
 * re-derived quintic maps (the pages do not print their values, so they are the caller's).
 * The array is read during the call only; every value must be finite.
 *
 * row_equalize: 0, or 1 to apply the per-row energy equaliser above to O before the update
 * (muon_step only), with row_beta in [0, 1) and finite row_eps >= 0. */
typedef struct {
  float lr;
  float beta;
  int nesterov;
  int ns_steps;
  float a, b, c;
  float eps;
  const float *schedule;
  int row_equalize;
  float row_beta;
  float row_eps;
} muon_config;

/* Fills cfg with lr 0.02, beta 0.95, nesterov 1, ns_steps 5, (3.4445, -4.7750, 2.0315),
 * eps 1e-7, schedule NULL, row_equalize 0, row_beta 0.95, row_eps 1e-8. A NULL cfg is
 * ignored. */
void muon_config_default(muon_config *cfg);

/* Builds a plan for n matrices (n >= 0) of the given shapes and dtypes. The plan groups the
 * matrices by their padded wide shape (rows and cols swapped when rows > cols, each rounded
 * up to a multiple of 128) so that each group runs as one batch. rows and cols are in
 * [1, 32768] with rows*cols <= 2^28. Host-only: makes no HIP call. On success *out owns the
 * plan (release it with muon_plan_destroy); on failure *out is set to NULL. */
int muon_plan_create(muon_plan **out, const int64_t *rows, const int64_t *cols,
                     const muon_dtype *param_dtype, const muon_dtype *grad_dtype, int64_t n,
                     muon_precision precision);

/* Bytes of device workspace a call on this plan needs (0 for an empty plan). The workspace
 * base must be 256-byte aligned and must not overlap any matrix buffer. Its contents need
 * not be preserved between calls. Returns 0 for a NULL plan. */
size_t muon_plan_workspace_size(const muon_plan *plan);

/* One Muon step over mats[0..n-1]; n must equal the plan's count (n = 0 is a no-op). */
int muon_step(muon_plan *plan, const muon_matrix *mats, int64_t n, const muon_config *cfg,
              void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of the static device scratch behind muon_step_noalloc (64 MiB: the GPT-2-124M
 * matrix set's share of one GPU out of 8 needs 61.2 MiB in the bf16 rounds). */
#define MUON_STATIC_SCRATCH_BYTES ((size_t)64 << 20)

/* muon_step without a workspace argument, for callers that cannot allocate device memory
 * (code under stream capture, tight serving loops, harnesses that forbid allocation). The
 * kernels' scratch is a static device array of MUON_STATIC_SCRATCH_BYTES that the library
 * holds on every device it runs on until the process ends; the call allocates nothing (its
 * first call on a device looks up the array's address there, once). Same arguments, results
 * and conventions as muon_step otherwise, with these limits:
 *   - a plan whose muon_plan_workspace_size exceeds MUON_STATIC_SCRATCH_BYTES is rejected
 *     with MUON_ERR_WORKSPACE before anything is enqueued (use muon_step with a workspace);
 *   - nothing in the scratch has to start at zero (every step writes each scratch element it
 *     reads), and its contents after a call are unspecified;
 *   - every call on a device shares that device's scratch: calls that may overlap on one
 *     device (different streams, or host threads without ordering) race. Order them. */
int muon_step_noalloc(muon_plan *plan, const muon_matrix *mats, int64_t n,
                      const muon_config *cfg, hipStream_t stream);

/* The orthogonalisation alone (no momentum, no parameter update), for in[i] (rows x cols of
 * grad_dtype) into out[i] (rows x cols of param_dtype): out = NS(in / (||in||_F + eps)) with
 * cfg's ns_steps, a, b, c and eps; cfg's lr, beta and nesterov are ignored. This is the
 * pages' zeropower_via_newtonschulz5 with the pre-normalisation applied; row_equalize is
 * ignored. */
int muon_newton_schulz(muon_plan *plan, const void *const *in, void *const *out, int64_t n,
                       const muon_config *cfg, void *workspace, size_t workspace_bytes,
                       hipStream_t stream);

void muon_plan_destroy(muon_plan *plan); /* NULL is ignored */

/* Whether steps on this plan run all Newton-Schulz rounds as one persistent launch (enable 1,
 * the default of a new plan) where the plan allows it, or one launch per product (0). The
 * single launch takes bf16 rounds (at most 16 of them) of plans with at most 4 shape groups,
 * each a multiple of 256 on both sides with at least 8 matrices, of at most 8 apply tiles of
 * 256x256 per compute unit per round, on a 256-CU device (8 XCDs): e.g. the GPT-2-124M set,
 * 48 x 768x768 and 24 x 768x3072. It computes the same products in the same order with the
 * same instructions, so results are bitwise those of the per-product launches; it deals each
 * group's matrices to the device's 8 XCDs and runs every item of a matrix on that matrix's
 * XCD, starting each product of a matrix as soon as the products it reads are complete, with
 * no launch boundary between rounds. Its workspace (queue and completion counters) is part of
 * muon_plan_workspace_size. MUON_ERR_INVALID_ARG for a NULL plan or another value of enable.
 * Steps of a plan whose single launch is on must not overlap on one device with other steps
 * of the same plan (they share its counters, as they share the rest of its workspace).
 * Failure: a work item waits for the items it reads with a bounded poll (by default 2^22
 * polls, a few seconds, which correct operation never approaches; the environment variable
 * MUON_FUSED_MAX_POLLS, read when a plan is created, sets another count, and 0 makes every
 * wait give up at once, which tests the failure path). A wait that gives up
 * marks the launch failed, and the step's update then writes NaN to every W and O of the plan,
 * so a device that stalls the launch cannot leave silently wrong parameters. */
int muon_plan_set_fused(muon_plan *plan, int enable);

/* Upper bound of muon_plan_set_concurrency's stream count. */
#define MUON_MAX_STREAMS 4

/* Lets later calls of muon_step, muon_step_noalloc and muon_newton_schulz on this plan run
 * its shape groups concurrently: the first group stays on the call's stream, the others run
 * on up to streams - 1 streams of the plan's own (created here, at the default priority, on
 * the current device, with the events that fork them from and join them back to the call's
 * stream; muon_plan_destroy releases them). Groups share no buffer, and each group's
 * kernels and their order are unchanged, so results are bitwise those of the sequential
 * step; a concurrent step fills the device with one group's kernels while another group's
 * drain. streams = 1 (the default of a new plan) releases the streams and runs the groups
 * in sequence. Calls run in sequence all the same on another device than the one this was
 * called on, while profiling is enabled (each kernel is then timed alone), and for sets
 * larger than 16 apply tiles of 256x256 per compute unit in all, whose long kernels measured
 * faster in sequence. Plans whose groups share launches (sets too small to fill the device
 * group by group) are unaffected.
 * Returns MUON_ERR_INVALID_ARG for streams outside [1, MUON_MAX_STREAMS] and MUON_ERR_HIP if
 * the HIP runtime cannot create the streams (the plan is then left sequential). Call it
 * outside stream capture; steps on the plan may be captured afterwards. */
int muon_plan_set_concurrency(muon_plan *plan, int streams);

/* Kernel timing for measurement. When enabled, every later muon_step/muon_newton_schulz
 * times each kernel launch with a HIP event pair that the launch itself updates with the
 * kernel's start and end (hipExtLaunchKernel; no marker packets are added to the stream).
 * Events are created here, on the current device; the step itself still allocates nothing.
 * Enabling resets the totals; disabling releases the events. Not for use while the call's
 * stream is being captured into a graph: capture the step with profiling disabled. */
int muon_plan_set_profiling(muon_plan *plan, int enable);

/* Kinds of kernel, in the order of a step. */
typedef enum {
  MUON_KERNEL_MOMENTUM = 0, /* momentum + Nesterov + norm partials + X0 store  */
  MUON_KERNEL_NORM = 1,     /* per-matrix norm finish and scales              */
  MUON_KERNEL_GRAM = 2,     /* A = s X X^T (upper tiles + mirror)             */
  MUON_KERNEL_POLY = 3,     /* B = b A + c A A (upper tiles + mirror)         */
  MUON_KERNEL_APPLY = 4,    /* X' = s (a X + B X)                             */
  MUON_KERNEL_UPDATE = 5,   /* W -= lr O (and O out)                          */
  MUON_KERNEL_ROWEQ = 6,    /* row equaliser: row sums of O^2, per-row factors */
  MUON_KERNEL_ROUNDS = 7,   /* all rounds (gram, poly, apply) as one launch    */
  MUON_KERNEL_KINDS = 8
} muon_kernel_kind;

/* Waits for the recorded events and writes, per kind (up to nkinds entries), the summed
 * milliseconds and the number of launches since profiling was enabled. */
int muon_plan_read_profile(muon_plan *plan, double *ms, int64_t *launches, int nkinds);

const char *muon_status_string(int status);
/* Message for the last failing call on this thread ("" if none). */
const char *muon_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MUON_H */
