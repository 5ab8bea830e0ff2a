/*
 * muon.h -- C ABI of the MI355X (gfx950) Muon-style optimizer step.
 *
 * The method (page "きみはNanoGPT speedrunを知っているか？", prednext.com,
 * section "Muonとは"; the neo-ai.one article on the Muon author, section
 * "Muonが登場"): keep a moving average (momentum) of each 2-D weight matrix's
 * gradient, approximately orthogonalise that momentum with Newton-Schulz
 * iteration so that its singular values move towards one, and update the
 * weights with the result.  The iteration implemented is the odd polynomial
 *     X <- a_j X + (b_j A + c_j A^2) X,   A = X X^T,   j = 0 .. steps-1,
 * run on the wide orientation of each matrix (tall matrices are transposed so
 * that A is the smaller Gram matrix) after dividing by (||X||_F + eps).
 * Options cover the variant of page "Training NanoGPT in 39.9 Seconds"
 * (seosoyoung.eiaserinnys.me digest), section "ANVIL II와 가중치 평균": a fast
 * and a slow momentum, a fixed number of polynomial-map steps, weight decay
 * applied only where the weight agrees in sign with the slow momentum, and an
 * exponential moving average of the weights (the section's displayed
 * equation) with a final readout blend of final weights and average.
 *
 * Conventions for every entry point:
 *   - Matrices are row-major device buffers: element (i, j) of a muon_mat lives
 *     at ptr[i*ld + j].  ld >= cols.  Pointers must be 16-byte aligned.
 *   - The caller owns all device memory (parameters, gradients, optimizer
 *     state, workspace).  Host arrays passed in are read during the call only.
 *     The library allocates no device memory; it keeps a host-side plan cache.
 *   - Work is enqueued on `stream` (a hipStream_t, NULL = the null stream)
 *     and the call returns without synchronising.
 *   - Every argument is validated before the first launch.  On any error the
 *     function returns a nonzero MUON_E_* code, enqueues nothing and leaves
 *     the state and its counters unchanged.  MUON_E_HIP means a HIP call
 *     failed after validation; device buffers are then undefined and the
 *     counters are not advanced.
 *   - A state must not be used from two host threads at once.  Calls on one
 *     workspace must be ordered on one stream.
 *   - Results are deterministic: the same inputs give the same bits.
 */
#ifndef MUON_MI355X_H
#define MUON_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element types */
enum { MUON_BF16 = 0, MUON_F32 = 1 };

/* status codes */
enum {
  MUON_OK = 0,
  MUON_E_NULL = 1,       /* a required pointer is NULL                          */
  MUON_E_SHAPE = 2,      /* n < 0, rows/cols < 1, ld < cols, shapes differ, or
                            a matrix too large (its padded wide iterate, the
                            shape rounded up to the tile, must stay below
                            4 GiB of the Newton-Schulz element type)          */
  MUON_E_DTYPE = 3,      /* unknown element type                                */
  MUON_E_COEFFS = 4,     /* steps outside [0, MUON_MAX_STEPS] or non-finite a,b,c */
  MUON_E_HPARAM = 5,     /* non-finite lr/wd/eps, beta outside [0,1), bad option */
  MUON_E_WORKSPACE = 6,  /* workspace NULL or smaller than muon_workspace_bytes  */
  MUON_E_ALIAS = 7,      /* two buffers that must be distinct overlap          */
  MUON_E_ALIGN = 8,      /* a pointer or row pitch breaks 16-byte alignment    */
  MUON_E_HIP = 9,        /* a HIP runtime call failed                           */
  MUON_E_STATE = 10,     /* state inconsistent with the call (n, buffers)       */
  MUON_E_CAPTURE = 11    /* stream under graph capture, but the call's device
                            descriptor table is not resident (see
                            muon_step_prepare)                                 */
};

#define MUON_MAX_STEPS 16

/* One 2-D matrix on the device. */
typedef struct {
  void*   ptr;     /* device pointer, row-major                                */
  int64_t rows;
  int64_t cols;
  int64_t ld;      /* row pitch in elements; ld*element_size % 16 == 0        */
  int32_t dtype;   /* MUON_BF16 or MUON_F32                                    */
  int32_t _pad;
} muon_mat;

/* Options of the step; muon_default_options() fills the plain-Muon defaults. */
typedef struct {
  float   beta_slow;  /* slow momentum coefficient in [0,1); < 0 disables it   */
  float   beta_ema;   /* weight-average coefficient in [0,1); < 0 disables it  */
  float   eps;        /* added to the Frobenius norm (default 1e-7)            */
  int32_t nesterov;   /* 1: orthogonalise beta*M_t + (1-beta)*G instead of M_t */
  int64_t ema_start;  /* first step (1-based, after increment) that is averaged */
  int32_t cautious;   /* 1: decay only where W_{t-1} and S_t share a strict sign
                         (needs beta_slow >= 0)                                */
  int32_t ns_dtype;   /* MUON_BF16: bf16 MFMA operands with fp32 accumulation;
                         MUON_F32: fp32 operands and accumulation              */
  int32_t avg_mode;   /* weight average (when beta_ema >= 0): MUON_AVG_EMA, or
                         MUON_AVG_WEIGHTED (running weighted mean, see below)  */
  int32_t _pad;
} muon_options;

/* Weight-average recurrences E <- b*E + ob*W, E <- W at the first averaged step:
 *   MUON_AVG_EMA:      b = beta_ema, ob = 1 - b (fp32), the exponential moving
 *                      average of page "Training NanoGPT in 39.9 Seconds",
 *                      section "ANVIL II와 가중치 평균";
 *   MUON_AVG_WEIGHTED: with this step's weight w = st->avg_weight and the sum
 *                      S of the weights averaged so far (st->avg_weight_sum),
 *                      b = S/(S+w), ob = w/(S+w) (computed in double, rounded
 *                      to fp32), so E is the weighted mean of the averaged
 *                      weights: equal weights give stochastic weight averaging,
 *                      other weights weighted checkpoint averaging (both named
 *                      among the tricks of the Slowrun page's results table).
 * Components whose averages follow their own schedules (the readout, matrix
 * banks and value embeddings of the same section) use one state each. */
enum { MUON_AVG_EMA = 0, MUON_AVG_WEIGHTED = 1 };

/* Optimizer state.  The buffer arrays are HOST arrays of n DEVICE pointers;
 * every buffer is fp32, dense row-major rows x cols of the matching param. */
typedef struct {
  int32_t   n;            /* number of matrices                                */
  int32_t   _pad;
  float**   mom;          /* momentum (required)                               */
  float**   mom_slow;     /* slow momentum; required iff opt.beta_slow >= 0    */
  float**   ema;          /* weight average; required iff opt.beta_ema >= 0    */
  uint8_t** mask_out;     /* optional diagnostic (NULL = off): per matrix, a
                             dense rows x cols byte array receiving the decay
                             mask actually applied (1 = decayed)               */
  float**   update_out;   /* optional diagnostic (NULL = off): per matrix, a
                             dense rows x cols fp32 array receiving the
                             orthogonalised update O actually applied          */
  void*     workspace;    /* device scratch of >= muon_workspace_bytes bytes   */
  size_t    workspace_bytes;
  int64_t   step;         /* number of completed steps (incremented per call)  */
  int64_t   ema_count;    /* number of steps folded into the weight average    */
  muon_options opt;
  float     avg_weight;   /* MUON_AVG_WEIGHTED: weight of the next averaged step
                             (finite, >= 0; the first averaged step needs > 0) */
  int32_t   _pad2;
  double    avg_weight_sum; /* MUON_AVG_WEIGHTED: sum of the weights averaged so
                             far (advanced with ema_count)                     */
} muon_state;

/* Plain-Muon defaults: no slow momentum, no EMA, eps 1e-7, ema_start 1,
 * no Nesterov, no cautious decay, bf16 MFMA Newton-Schulz. */
void muon_default_options(muon_options* opt);

/* Workspace bytes needed by muon_step / muon_orthogonalize for this list of
 * matrix shapes (only rows and cols of params[] are read) and options.
 * `steps` is accepted for symmetry; the size does not depend on it.
 * Returns 0 if the arguments are invalid. */
size_t muon_workspace_bytes(const muon_mat* params, int32_t n,
                            const muon_options* opt, int32_t steps);

/* One optimizer step over n matrices (the whole hot path):
 *   M <- beta*M + (1-beta)*G                       (fp32, no fused ops)
 *   S <- beta_slow*S + (1-beta_slow)*G             (if enabled)
 *   U  = M, or beta*M + (1-beta)*G with Nesterov
 *   O  = orthogonalise(U) with `steps` rows of coeffs (a_j, b_j, c_j)
 *   W <- W - lr*wd*mask*W - lr*O   (mask = 1, or [W*S > 0] when cautious)
 *   step += 1;  if the average is enabled and step >= ema_start:
 *       E <- W (first averaged step) or b*E + ob*W (see MUON_AVG_*);
 *       ema_count += 1
 * params: n matrices, updated in place (bf16 is rounded to nearest even).
 * grads:  n matrices with the same shapes (any element type).
 * coeffs: HOST array of steps*3 floats.  steps in [0, MUON_MAX_STEPS].
 * lr, wd finite; beta in [0,1).  n == 0 only advances the counters.
 * The plain update (no cautious mask, no average, no update_out/mask_out)
 * of bf16 parameters whose rows, cols and ld are multiples of 8 and whose
 * base is 16-byte aligned runs in the epilogue of the last Newton-Schulz
 * launch (256-wide bf16 tiles, last iteration with b or c nonzero) instead
 * of a separate kernel; it rounds O to bf16 and applies the same fp32
 * operations, so the result is the same bit for bit.
 * The bf16 products fold the term b A (or a X) into the accumulators as
 * (b/c) A (or (a/b) X) and scale at the store; a table with a row whose ratio
 * is not finite, above 2^32 in magnitude, or whose divisor is below 2^-32
 * runs every launch of the call with the term added at the store instead
 * (same results within rounding, a little slower). */
int muon_step(const muon_mat* params, const muon_mat* grads, muon_state* st,
              const float* coeffs, int32_t steps, float lr, float wd,
              float beta, void* stream);

/* Allocation-free step, for callers that cannot allocate device memory (code
 * under graph capture, tight serving loops, harnesses that forbid it).  Same
 * arguments, validation, arithmetic and results as muon_step, but
 * st->workspace and st->workspace_bytes are ignored: the workspace is a
 * static device array of the library of MUON_NOALLOC_SCRATCH_BYTES (64 MiB),
 * one per GPU, held from the first call on that GPU until the process ends
 * (the current device when the call is made).  The descriptor table is
 * written into it by kernels on `stream`, so the call uses no pinned staging
 * memory, calls no allocation routine and may run under stream capture.  A
 * step whose muon_workspace_bytes exceeds MUON_NOALLOC_SCRATCH_BYTES returns
 * MUON_E_WORKSPACE and enqueues nothing.  Every call on one GPU shares that
 * GPU's array, which keeps the last call's contents (each call rewrites every
 * byte it reads): calls that may overlap on one GPU (other streams, other
 * host threads) race and must be ordered by the caller. */
#define MUON_NOALLOC_SCRATCH_BYTES (64u << 20)
int muon_step_noalloc(const muon_mat* params, const muon_mat* grads, muon_state* st,
                      const float* coeffs, int32_t steps, float lr, float wd, float beta,
                      void* stream);

/* Graph capture of a step (page "Training NanoGPT in 39.9 Seconds", Table A,
 * credits capturing the training step as a device graph with part of the
 * end-to-end gain).  Besides its kernel launches, muon_step enqueues one
 * host-to-device copy of a per-workspace descriptor table (matrix pointers,
 * shapes, tile offsets) from pinned staging memory, on every call; it does
 * not synchronise the stream.  The workspace holds two table regions (see
 * muon_workspace_layout): uncaptured calls send and read the eager region;
 * muon_step_prepare sends the capture region, and a call under capture makes
 * no copy and reads the capture region.  muon_step_prepare validates the
 * arguments exactly as muon_step does and sends that table for these
 * params/grads/state buffers, without launching anything or touching the
 * counters.  After it, a muon_step with the same buffers can be captured
 * (hipStreamBeginCapture, or a framework's graph capture) on `stream`; a
 * captured call whose table does not match the capture region returns
 * MUON_E_CAPTURE and enqueues nothing.  Eager muon_step, muon_orthogonalize
 * and muon_ema_blend calls on the same workspace between replays leave the
 * capture region alone; another muon_step_prepare on the workspace replaces
 * it (the earlier graph would then replay with the new table).
 * A replay repeats the captured step on the same buffers with the captured
 * scalars: lr, wd, beta, coefficients, options, the weight-average
 * coefficients, and the flags derived from the counters (whether this step is
 * averaged, and whether it is the first averaged step).  The capturing call
 * advances step/ema_count once as for an eager call; replays do not touch the
 * host state: advance the counters with muon_state_advance per replay, and
 * capture only steps whose flags and coefficients repeat (weight average
 * disabled, or an exponential average already started).  A captured step that
 * would fold into a MUON_AVG_WEIGHTED average returns MUON_E_CAPTURE (its
 * coefficients change every step).  Same errors as muon_step. */
int muon_step_prepare(const muon_mat* params, const muon_mat* grads, muon_state* st,
                      void* stream);

/* Counter advance for replayed captured steps (see muon_step_prepare): adds
 * `replays` steps to st->step and, when the weight average is on and the
 * step has reached ema_start, as many to st->ema_count, exactly as that many
 * eager calls would.  Errors: MUON_E_NULL; MUON_E_HPARAM (replays < 0 or bad
 * options); MUON_E_CAPTURE when the state's average could not have been
 * captured (a MUON_AVG_WEIGHTED average, or an exponential average that has
 * not started yet), the counters then unchanged.  Touches no device memory. */
int muon_state_advance(muon_state* st, int32_t replays);

/* Newton-Schulz part alone: out[i] = orthogonalise(in[i]) for n matrices
 * (same shapes; out may be any element type; in and out must not overlap).
 * Uses opt->eps and opt->ns_dtype; the other options are ignored. */
int muon_orthogonalize(const muon_mat* in, const muon_mat* out, int32_t n,
                       const float* coeffs, int32_t steps,
                       const muon_options* opt, void* workspace,
                       size_t workspace_bytes, void* stream);

/* Readout blend out[i] = w_final*W[i] + (1-w_final)*E[i] (fp32 operation
 * order, rounded to out's element type), with E the state's weight average
 * (page "Training NanoGPT in 39.9 Seconds", section "ANVIL II와 가중치 평균":
 * 35 % final weights and 65 % average, i.e. w_final = 0.35).
 * Requires st->ema; w_final in [0,1]. */
int muon_ema_blend(const muon_mat* out, const muon_mat* params,
                   const muon_state* st, float w_final, void* stream);

/* Human-readable name of a status code (static string). */
const char* muon_status_str(int status);

/* ---------------------------------------------------------------------------
 * Measurement hooks.  A phase's kernel launches can be bracketed with HIP
 * events recorded on the launch stream; used to time one kernel inside a
 * running step.  Not needed for normal use. */
enum {
  MUON_PHASE_PREPARE = 0,  /* momentum, cast/transpose, norm partials */
  MUON_PHASE_GRAM = 1,     /* A = X X^T                               */
  MUON_PHASE_POLY = 2,     /* B = b A + c A^2                         */
  MUON_PHASE_APPLY = 3,    /* X <- a X + B X                          */
  MUON_PHASE_FINISH = 4,   /* update, mask, EMA (or write O)          */
  MUON_PHASE_ADAMW = 5,    /* the AdamW kernel of muon_adamw_step     */
  MUON_PHASE_APPLY_UPDATE = 6, /* last APPLY with the plain update of W
                                  (see muon_step); not in MUON_PHASE_APPLY */
  MUON_PHASE_NS_SINGLE = 7     /* all iterations of a small problem in one
                                  launch (see muon_plan_info)            */
};

/* Record events around each of the next `capacity` launches of `phase`
 * (capacity in [1, 65536]).  Re-arming discards earlier records. */
int muon_probe_arm(int32_t phase, int32_t capacity);
/* Wait for the recorded events and write up to `capacity` per-launch
 * durations in milliseconds to ms[]; *count receives the number recorded. */
int muon_probe_read(float* ms, int32_t capacity, int32_t* count);
/* Stop recording and release the events. */
int muon_probe_disarm(void);

/* Workspace layout of muon_step for a shape list (byte offsets from the
 * workspace base): the descriptor-table region that uncaptured calls send and
 * read (muon_step, muon_orthogonalize, muon_ema_blend), the region that
 * muon_step_prepare sends and captured steps read, the size of one region,
 * and the first byte of the iterate and product buffers.  The two regions
 * are disjoint, so no uncaptured call on the workspace changes the table a
 * replay reads; only another muon_step_prepare on it does. */
int muon_workspace_layout(const muon_mat* params, int32_t n, const muon_options* opt,
                          size_t* eager_table, size_t* capture_table, size_t* table_bytes,
                          size_t* buffers);

/* Kernel configuration chosen for a shape list: number of effective-shape
 * groups, Newton-Schulz tile size per group (in `tiles`, up to `cap`
 * entries), and launches per step for `steps` iterations with coefficient
 * table `coeffs` (host, may be NULL for quintic): one prepare launch, the
 * Newton-Schulz launches, and one finish launch unless the plain update runs
 * inside the last APPLY launch (see muon_step; counted here for options
 * without the average). Returns a status.
 * Two environment variables, read when a shape list is first planned, override
 * the plan for experiments and tests: MUON_TILE=64|128|256 forces the tile
 * width (256 only for bf16 iterates), and MUON_GEMM_ORDER="g,p,a" sets the
 * block-order bits of the GRAM, POLY and APPLY launches (1 plain, 2 row-major
 * APPLY tiles, 4 whole matrices dealt to XCDs, 8 APPLY by column panel).
 * Results do not depend on MUON_GEMM_ORDER; MUON_TILE changes the rounding of
 * the bf16 path within its tolerance.
 * With MUON_NS_SINGLE_LAUNCH=1 (read at every call), small problems (64-wide
 * tiles with bf16 operands, at most 1024 tiles per product, at most 16
 * iterations) run all Newton-Schulz iterations in one launch whose blocks
 * meet at a grid-wide barrier between products; it computes every tile as the
 * separate launches do, so results are the same bit for bit, and counts as
 * one launch here.  It is not the default: on MI355X the barriers (device-
 * scope release and acquire across the XCDs' caches) cost more than the
 * kernel boundaries they replace.  The barrier's wait is bounded
 * (MUON_NS_SPIN_LIMIT polls, read at every call; 0 gives up at once): a block
 * that gives up marks the step failed and the finish kernel then writes NaN
 * for every O, so such a failure is never silent. */
int muon_plan_info(const muon_mat* params, int32_t n, const muon_options* opt,
                   int32_t steps, const float* coeffs, int32_t* n_groups,
                   int32_t* tiles, int32_t cap, int32_t* launches_per_step);

/* ---------------------------------------------------------------------------
 * AdamW for the parameters that are not weight matrices.  Orthogonalisation
 * applies only to matrix-shaped layers and the pages leave every other
 * parameter to AdamW (page "きみはNanoGPT speedrunを知っているか？",
 * section "Muonとは"); they give no formula, so this is the textbook update
 * with bias-corrected moments and decay decoupled from the gradient:
 *   t  = step + 1
 *   m <- b1*m + (1-b1)*g,   v <- b2*v + (1-b2)*(g*g)      (fp32, each product
 *                                                         and sum rounded)
 *   p <- p - lr*wd*p - lr * (m / (1-b1^t)) / (sqrt(v / (1-b2^t)) + eps)
 * b1, b2 are the fp32 values of beta1, beta2 and (1-b) is computed in fp32,
 * so m and v are reproducible bit for bit; the bias terms are computed on the
 * host in double precision.  One grouped launch covers all tensors. */

/* One contiguous device tensor of any shape, seen as `numel` elements. */
typedef struct {
  void*   ptr;     /* device pointer, aligned to its element size; may be NULL
                      only when numel == 0                                    */
  int64_t numel;   /* >= 0                                                    */
  int32_t dtype;   /* MUON_BF16 or MUON_F32                                   */
  int32_t _pad;
} muon_vec;

typedef struct {
  float   lr;      /* finite                                                  */
  float   beta1;   /* in [0,1)                                                */
  float   beta2;   /* in [0,1)                                                */
  float   eps;     /* finite, >= 0 (eps = 0 with v = 0 divides zero by zero)  */
  float   wd;      /* finite                                                  */
  int32_t _pad;
} muon_adamw_hparams;

/* The buffer arrays are HOST arrays of n DEVICE pointers to dense fp32
 * buffers of numel elements (NULL allowed where numel == 0). */
typedef struct {
  int32_t n;
  int32_t _pad;
  float** m;               /* first moments                                   */
  float** v;               /* second moments                                  */
  void*   workspace;       /* device scratch of >= muon_adamw_workspace_bytes  */
  size_t  workspace_bytes;
  int64_t step;            /* completed steps (incremented per call)          */
} muon_adamw_state;

/* Workspace bytes for n tensors (the per-call descriptor table); 0 if n < 0. */
size_t muon_adamw_workspace_bytes(int32_t n);

/* One AdamW step over n tensors: params[i] updated in place (bf16 rounded to
 * nearest even), grads[i] of the same numel (any element type).  All of
 * params, grads, m, v and the workspace must be pairwise disjoint.  Errors as
 * for muon_step (MUON_E_SHAPE: negative or mismatched numel; MUON_E_HPARAM:
 * the ranges above); n == 0 only advances the counter.  The bias terms
 * change with every step, so a call on a stream under graph capture returns
 * MUON_E_CAPTURE and enqueues nothing. */
int muon_adamw_step(const muon_vec* params, const muon_vec* grads, muon_adamw_state* st,
                    const muon_adamw_hparams* hp, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MUON_MI355X_H */
