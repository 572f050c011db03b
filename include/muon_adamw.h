/*
 * muon_adamw.h -- C ABI of the MI355X (gfx950) Muon + AdamW optimizer step.
 *
 * Two operations, both in place on caller-owned device memory, both
 * asynchronous on the caller's HIP stream:
 *
 *   ma_muon_step   one Muon step over groups of same-shape weight matrices
 *                  ("Chapter 4: The MuonAdamW Optimizer", sections "The Muon
 *                  Update Rule", "Polar Express: Newton-Schulz
 *                  Orthogonalization" and "The Full Muon Step"; nanochat
 *                  discussion "Stuck at the optimizer after figuring out
 *                  backward()", reply by mira687: per-step Polar Express
 *                  coefficients, cautious weight decay, MuonEq, the
 *                  max(1, rows/cols)^0.5 lr multiplier, stacked same-shape
 *                  matrices);
 *   ma_adamw_step  one AdamW step over flat buffers ("3.9 Optimizers: SGD,
 *                  Adam, Adafactor, Lion, Muon & Shampoo", section
 *                  "Implementing AdamW from scratch"; "Chapter 4", section
 *                  "The AdamW Step");
 *   ma_lion_step   one Lion step over flat buffers ("3.9 Optimizers",
 *                  section "Lion: Learning the Sign of the Update" and
 *                  exercise 5; "Muon vs AdamW, Lion and Sophia: a fair
 *                  race", section "Lion").
 *
 * Conventions for every entry point:
 *   - Pointers named "device" are HIP device pointers; "host" pointers are
 *     read during the call only and may be freed when it returns.
 *   - The library allocates no device memory and keeps no state between
 *     calls. Scratch memory is the caller's workspace.
 *   - Matrices are row-major, rows x cols, contiguous (leading dimension ==
 *     cols); rows are output features, cols input features.
 *   - Return value: MA_OK (0) or a negative MA_ERR_* code. Every argument is
 *     validated before the first launch, so a rejected call changes nothing.
 *     A kernel fault surfaces at the caller's next synchronisation.
 *     ma_last_error() returns a message for the calling thread's last
 *     failure.
 *   - `stream` is a hipStream_t passed as void* (NULL: the default stream).
 *   - Calls that overlap on one stream are ordered; concurrent calls on
 *     different streams must not share buffers or a workspace.
 */
#ifndef MUON_ADAMW_H
#define MUON_ADAMW_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define MA_OK 0
#define MA_ERR_INVALID_ARG -1   /* null pointer, bad size, bad enum, aliasing */
#define MA_ERR_UNSUPPORTED -2   /* dtype combination not provided */
#define MA_ERR_WORKSPACE -3     /* workspace null, too small or misaligned */
#define MA_ERR_HIP -4           /* a HIP runtime call or launch failed */
#define MA_ERR_NONFINITE -5     /* ma_muon_nonfinite: a matrix of the last step had
                                   non-finite norms (check_finite == 1 only) */

typedef enum { MA_F32 = 0, MA_BF16 = 1 } ma_dtype;

/* Row scalings (rows are output features, in the parameter's own layout).
 * ROWS_PRE (MuonEq): each row of the Nesterov look-ahead is divided by its
 *   Euclidean norm (+eq_eps) before the Frobenius normalisation.
 * ROWS_POST (MuonEq after the iteration): each row of the orthogonalised
 *   update U is rescaled to the matrix's mean row norm, ||U||_F/sqrt(rows),
 *   over (||U_i|| + eq_eps).
 * ROWS_RMS (NorMuon, "Chapter 4: The MuonAdamW Optimizer", section "NorMuon:
 *   Normalized Muon"): each row of U is divided by its RMS,
 *   ||U_i||/sqrt(cols), plus eq_eps (the page uses 1e-8), so that with
 *   lr_scale NONE every row of the step has RMS lr. */
typedef enum { MA_EQ_OFF = 0, MA_EQ_ROWS_PRE = 1, MA_EQ_ROWS_POST = 2, MA_EQ_ROWS_RMS = 3 } ma_eq;

/* Per-matrix lr multiplier:
 *   NONE                1
 *   SQRT_MAX1_R_OVER_C  sqrt(max(1, rows/cols)) (nanochat discussion, reply by
 *                       mira687: x2 for c_fc, x1 for c_proj)
 *   MOONSHOT            0.2 * sqrt(max(rows, cols)) ("Muon vs AdamW, Lion and
 *                       Sophia: a fair race": entries about AdamW's size)
 *   SQRT_MAX            sqrt(max(rows, cols)) ("3.9 Optimizers ...", section
 *                       "Muon: Orthogonalizing the Update": update RMS about 1) */
typedef enum {
  MA_SCALE_NONE = 0,
  MA_SCALE_SQRT_MAX1_R_OVER_C = 1,
  MA_SCALE_MOONSHOT = 2,
  MA_SCALE_SQRT_MAX = 3
} ma_scale;

/* One group: `count` matrices of identical shape rows x cols.
 * params/grads/momentum are HOST arrays of `count` DEVICE pointers; matrix i
 * of the group is params[i] (rows*cols elements of param_dtype), grads[i]
 * (grad_dtype, read only) and momentum[i] (mom_dtype, updated in place).
 * Limits (MA_ERR_INVALID_ARG beyond them): rows, cols <= 2^24,
 * rows*cols <= 2^31, count*rows*cols <= 2^40. */
typedef struct {
  int64_t rows, cols;
  int32_t count;
  int32_t param_dtype, grad_dtype, mom_dtype; /* ma_dtype */
  void* const* params;
  const void* const* grads;
  void* const* momentum;
} ma_muon_group;

/* Muon hyperparameters ("Chapter 4", section "The Full Muon Step"; the
 * nanochat discussion for the coefficient table, cautious mask and MuonEq).
 *   lr            base learning rate (multiplied per matrix by lr_scale)
 *   momentum      beta of the sum-form buffer  m <- beta*m + G
 *   weight_decay  decoupled decay; the applied factor is lr_eff*weight_decay
 *   nesterov      1: orthogonalise G + beta*m (look-ahead), 0: orthogonalise m
 *   ns_steps      number T of quintic steps, 0..MA_MAX_NS_STEPS
 *   abc           HOST array of 3*ns_steps floats: (a_k, b_k, c_k) of step k,
 *                 X <- a_k X + (b_k A + c_k A A) X with A = X X^T
 *   cautious      1: decay only where update and weight agree in sign,
 *                 mask = (U * W >= 0)
 *   equilibrate   ma_eq
 *   ns_precision  MA_BF16: iterate in bf16 with fp32 accumulation;
 *                 MA_F32: iterate in fp32
 *   lr_scale      ma_scale
 *   norm_eps      added to the Frobenius norm (the pages use 1e-7)
 *   eq_eps        added to each row norm by MuonEq (1e-7), or to each row RMS
 *                 by ROWS_RMS
 *   check_finite  1: detect non-finite values, after the fast-fail rule of
 *                 "Chapter 4", section "Fast-Fail on NaN or Loss > 100".
 *                 A matrix whose look-ahead momentum has a non-finite sum of
 *                 squares (a NaN or Inf entry, or an overflowing square) --
 *                 or, with ROWS_POST / ROWS_RMS, whose orthogonalised update
 *                 has one -- keeps its weight unchanged (no decay, no
 *                 update); its momentum buffer is updated as usual and holds
 *                 the non-finite values. Every other matrix is stepped
 *                 exactly as without the check. ma_muon_nonfinite reports
 *                 which matrices were flagged. 0: no check (non-finite
 *                 values propagate into the weights). */
typedef struct {
  float lr, momentum, weight_decay;
  int32_t nesterov, ns_steps;
  const float* abc;
  int32_t cautious, equilibrate, ns_precision, lr_scale;
  float norm_eps, eq_eps;
  int32_t check_finite;
} ma_muon_hparams;

#define MA_MAX_NS_STEPS 16
#define MA_WORKSPACE_ALIGN 256

/* Bytes of device workspace ma_muon_step needs for these groups and
 * hyperparameters (0 on invalid arguments; see ma_last_error). The
 * workspace holds the normalised momentum and the Newton-Schulz iterates
 * and Gram matrices of every matrix, padded to multiples of 256, the
 * partial sums of ma_muon_step_stats and, for fp32 groups small enough that
 * their Gram product is split along K, its per-slice partial products. */
size_t ma_muon_workspace_size(const ma_muon_group* groups, int32_t n_groups,
                              const ma_muon_hparams* hp);

/* One Muon step for every matrix of every group. Per matrix W (R x C),
 * gradient G, momentum buffer M, in this order:
 *   m1 = beta*M + G (fp32); M <- m1 rounded to mom_dtype (RNE)
 *   Mt = G + beta*m1 if nesterov else m1                      (fp32)
 *   optional MuonEq PRE; X0 = Mt / (||Mt||_F + norm_eps)
 *     (with MuonEq PRE and T >= 1, groups for which ma_muon_row_pass is 1
 *     store the row-scaled Mt rounded to the iteration's precision and apply
 *     1 / (||.||_F + norm_eps) in the first Gram product and update: the same
 *     X0 with one rounding at a different point)
 *   if R > C the iteration runs on X0^T (layout, no extra copy)
 *   T quintic steps with the caller's coefficient table
 *   optional MuonEq POST; U = final iterate in W's layout
 *   lr_eff = lr * multiplier(R, C)  (fp64 on the host, then fp32)
 *   mask = cautious ? (U*W >= 0) : 1
 *   W <- RNE( (mask ? W - (lr_eff*wd)*W : W) - lr_eff*U )   (fp32, no FMA)
 * The decay term is skipped entirely when weight_decay == 0.
 * Supported storage: param/grad/mom each MA_BF16 or MA_F32.
 * workspace: DEVICE, >= ma_muon_workspace_size bytes, MA_WORKSPACE_ALIGN
 * aligned. Parameter, gradient and momentum buffers must not overlap each
 * other or the workspace (MA_ERR_INVALID_ARG is returned for overlaps among
 * the pointers passed).
 * Results are deterministic for given inputs. The kernels a call uses depend
 * on its total work (launches of few tile jobs run smaller tiles, and an fp32
 * Gram product of few jobs is split along K), so one matrix stepped alone
 * and the same matrix stepped with many others can differ at the rounding
 * level. */
int ma_muon_step(const ma_muon_group* groups, int32_t n_groups, const ma_muon_hparams* hp,
                 void* workspace, size_t workspace_bytes, void* stream);

/* ma_muon_step with no workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation). The step's scratch memory is a fixed
 * array of MA_NOALLOC_SCRATCH_BYTES inside the library's device code, one
 * per GPU, held until the process ends; the call allocates nothing. Same
 * arguments, kernels and results as ma_muon_step. A call whose
 * ma_muon_workspace_size exceeds MA_NOALLOC_SCRATCH_BYTES is rejected with
 * MA_ERR_WORKSPACE before any launch. Every call on one GPU uses that GPU's
 * one array: calls that may overlap on one GPU (on different streams, or
 * from different host threads) race and must be ordered by the caller. Each
 * call writes every byte of scratch it later reads, so nothing carries over
 * from an earlier call. With check_finite, ma_muon_nonfinite is not available
 * for this entry point (the flags live in the shared array). The array used
 * is the current device's: a stream of another device is rejected with
 * MA_ERR_INVALID_ARG. */
#define MA_NOALLOC_SCRATCH_BYTES (64u << 20)
int ma_muon_step_noalloc(const ma_muon_group* groups, int32_t n_groups, const ma_muon_hparams* hp, void* stream);

/* ma_muon_step that also reports, per matrix, the size of the step it took:
 * the per-layer ratio ||delta theta|| / ||theta|| that "3.9 Optimizers: SGD,
 * Adam, Adafactor, Lion, Muon & Shampoo" (section "Large-batch training:
 * LARS, LAMB and the trust ratio") recommends logging. stats: DEVICE array of
 * 2 floats per matrix, groups in order and matrices in order within a group:
 *   stats[2k]   = ||W_new - W_old||_F, W_new as stored (after rounding to
 *                 param_dtype), W_old the weight before the step
 *   stats[2k+1] = ||W_old||_F
 * Per-element squares are summed in fp32 per block and the block sums in
 * fp64 in a fixed order, so the result is deterministic. stats must be
 * 4-byte aligned and must not overlap any other buffer (MA_ERR_INVALID_ARG).
 * The update itself is identical to ma_muon_step's. */
int ma_muon_step_stats(const ma_muon_group* groups, int32_t n_groups, const ma_muon_hparams* hp,
                       void* workspace, size_t workspace_bytes, float* stats, void* stream);

/* After a ma_muon_step / ma_muon_step_stats / ma_muon_adamw_step with
 * check_finite == 1 has completed (the caller has synchronised its stream),
 * the matrices it flagged: flags (HOST array of the total matrix count,
 * groups in order, or null) receives 1 for a flagged matrix and 0 otherwise.
 * groups, n_groups, hp and workspace must be those of the step. Returns MA_OK
 * when no matrix was flagged, MA_ERR_NONFINITE when one was, or
 * MA_ERR_INVALID_ARG when hp->check_finite is 0 (the step wrote no flags).
 * Synchronous: it copies the flags from device memory. */
int ma_muon_nonfinite(const ma_muon_group* groups, int32_t n_groups, const ma_muon_hparams* hp,
                      const void* workspace, int32_t* flags);

/* Whether ma_muon_step treats group `group` in one pass over G and M: the
 * momentum update, MuonEq PRE's row sums and the row-scaled X0 together, the
 * Frobenius factor of "Chapter 4: The MuonAdamW Optimizer" (section "Polar
 * Express: Newton-Schulz Orthogonalization") then applied by the first
 * Newton-Schulz products. That is the case for MuonEq PRE with T >= 1, a bf16
 * iteration, rows <= cols, cols a multiple of 8 and at most 4096 (after
 * padding to 256), 16-byte aligned buffers, unless the environment sets
 * MA_PRE_ROWS=0. Returns 1 or 0, or a negative MA_ERR_* for invalid
 * arguments (as ma_muon_workspace_size validates them). Host-only. */
int ma_muon_row_pass(const ma_muon_group* groups, int32_t n_groups, const ma_muon_hparams* hp, int32_t group);

/* Where matrix `index` of group `group` keeps the result of its Newton-Schulz
 * iteration inside a workspace after ma_muon_step (for inspection; valid
 * until the workspace is reused; with MA_EQ_ROWS_POST or MA_EQ_ROWS_RMS the
 * row scaling is applied later, in the update, and is not included). *u receives a DEVICE
 * pointer into `workspace`, in the parameter's layout (rows x cols, row pitch
 * *ld elements); *transposed (may be null) is set to 0; *elem_bytes is 2
 * (bf16 iteration) or 4 (fp32). */
int ma_muon_workspace_update(const ma_muon_group* groups, int32_t n_groups,
                             const ma_muon_hparams* hp, void* workspace, int32_t group,
                             int32_t index, void** u, int64_t* ld, int32_t* transposed,
                             int32_t* elem_bytes);

/* One flat AdamW buffer. param, grad, exp_avg, exp_avg_sq: DEVICE pointers to
 * n elements each (fp32; param_dtype and grad_dtype must be MA_F32). `step` is
 * the 1-based step count after increment (1 on the first call). */
typedef struct {
  void* param;
  const void* grad;
  void* exp_avg;
  void* exp_avg_sq;
  int64_t n;
  int32_t param_dtype, grad_dtype;
  float lr, beta1, beta2, eps, weight_decay;
  int64_t step;
} ma_adamw_segment;

/* One AdamW step over every segment (fp32 throughout), per element:
 *   p = p*(1 - lr*wd)            (only when wd != 0)
 *   m = beta1*m + (1-beta1)*g
 *   v = beta2*v + (1-beta2)*(g*g)
 *   p = p - (lr/(1-beta1^t)) * (m / (sqrt(v)/sqrt(1-beta2^t) + eps))
 * Step-dependent scalars are formed in fp64 on the host and rounded to fp32
 * once; each per-element operation is one correctly rounded fp32 operation
 * (no fused multiply-add). Segments may be in any order and of any length
 * (0 <= n <= 2^40); buffers of different segments must not overlap.
 * `segments` is a HOST array. */
int ma_adamw_step(const ma_adamw_segment* segments, int32_t n_segments, void* stream);

/* ma_adamw_step with identical results, run by at most `workgroups`
 * persistent workgroups that each keep one 16-byte chunk per buffer in
 * flight per thread: a register footprint small enough for a workgroup to
 * share a CU with a Newton-Schulz GEMM workgroup. For issuing the AdamW part
 * of a step on a second stream while ma_muon_step runs on another (the two
 * touch disjoint buffers); alone it is slower than ma_adamw_step. workgroups
 * >= 1 (MA_ERR_INVALID_ARG otherwise); 256, one per CU, suits MI355X. */
int ma_adamw_step_background(const ma_adamw_segment* segments, int32_t n_segments, int32_t workgroups,
                             void* stream);

/* One MuonAdamW step: ma_muon_step on `stream` and, on `side_stream`, the
 * AdamW update of ma_adamw_step_background (`workgroups` workgroups), which
 * starts once the Muon step's elementwise passes and first Gram and
 * polynomial products are done ("Chapter 4: The MuonAdamW Optimizer",
 * section "The Full Muon Step": the two optimizers update disjoint parameter
 * sets) and runs beside its remaining products; `stream` waits for it before
 * any later work. Results are those of ma_muon_step followed by
 * ma_adamw_step. side_stream must differ from stream (both may be captured
 * into one HIP graph: the fork and join are event records and waits on
 * events the library creates once per device and host thread; both streams
 * must belong to the current device, MA_ERR_INVALID_ARG otherwise). Every
 * argument is validated before the first launch, and no two buffers of the
 * two steps (Muon parameters, gradients, momentum, the workspace, AdamW
 * buffers) may overlap (MA_ERR_INVALID_ARG). If a launch fails after the
 * fork, `stream` still waits for what was queued on side_stream before the
 * error is returned. */
int ma_muon_adamw_step(const ma_muon_group* groups, int32_t n_groups, const ma_muon_hparams* hp,
                       void* workspace, size_t workspace_bytes, const ma_adamw_segment* segments,
                       int32_t n_segments, int32_t workgroups, void* stream, void* side_stream);

/* One flat Lion buffer. param, grad, exp_avg (the momentum, Lion's only
 * state): DEVICE pointers to n elements each, fp32 (param_dtype and
 * grad_dtype must be MA_F32), 4-byte aligned. */
typedef struct {
  void* param;
  const void* grad;
  void* exp_avg;
  int64_t n;
  int32_t param_dtype, grad_dtype;
  float lr, beta1, beta2, weight_decay;
} ma_lion_segment;

/* One Lion step over every segment (fp32 throughout), per element:
 *   p = p*(1 - lr*wd)            (only when wd != 0)
 *   c = beta1*m + (1-beta1)*g    (not stored)
 *   p = p - lr*sign(c)           sign: +1, -1, +0 for either zero, NaN for NaN
 *   m = beta2*m + (1-beta2)*g    (after the step, with the raw gradient)
 * 1 - lr*wd, 1 - beta1 and 1 - beta2 are formed in fp64 on the host and
 * rounded to fp32 once; each per-element operation is one correctly rounded
 * fp32 operation (no fused multiply-add). Requirements: finite lr and
 * weight_decay, 0 <= beta1, beta2 < 1. Segments may be in any order and of
 * any length (0 <= n <= 2^40); no two buffers, of one segment or of different
 * segments, may overlap. `segments` is a HOST array. Returns
 * MA_ERR_INVALID_ARG / MA_ERR_UNSUPPORTED before any launch on a bad
 * segment. */
int ma_lion_step(const ma_lion_segment* segments, int32_t n_segments, void* stream);

/* Status text for a code, and the calling thread's last error message. */
const char* ma_status_string(int status);
const char* ma_last_error(void);

/* Library version string, and the GPU architecture it was built for. */
const char* ma_version(void);

/* ---------------------------------------------------------------------------
 * Kernel timing. Between ma_profile_begin and ma_profile_end every kernel the
 * library launches is bracketed by two HIP events recorded on its stream
 * (host-side objects from a pool of 2*max_launches events created by
 * ma_profile_begin; no device memory). ma_profile_read synchronises on the
 * recorded events and returns, for one kernel kind, the summed duration in
 * milliseconds and the number of launches. Launches beyond max_launches are
 * not timed. Not thread-safe with concurrent library calls.
 * ------------------------------------------------------------------------- */
typedef enum {
  MA_K_ROWNORM = 0,   /* row sums of squares (momentum look-ahead or update) */
  MA_K_FINALIZE = 1,  /* per-matrix Frobenius / MuonEq factors */
  MA_K_PRE = 2,       /* momentum update and X0 in both layouts */
  MA_K_GRAM = 3,      /* A = X X^T */
  MA_K_POLY = 4,      /* B = b A + c A A */
  MA_K_AXPY = 5,      /* X' = a X + B X */
  MA_K_POST = 6,      /* cautious decay and the update */
  MA_K_ADAMW = 7,
  MA_K_LION = 8,
  MA_K_AXPY_UPDATE = 9, /* the last AXPY of a step with the update fused into it */
  MA_K_COUNT = 10
} ma_kernel_kind;

int ma_profile_begin(int32_t max_launches);
int ma_profile_end(void);
int ma_profile_read(int32_t kind, double* total_ms, int64_t* launches);

/* ---------------------------------------------------------------------------
 * Calibration (not part of the optimizer step): the bf16 MFMA rate the part
 * sustains without memory traffic, the practical ceiling the Newton-Schulz
 * GEMMs are compared with. Launches `blocks` workgroups of 4 waves; each
 * wave issues iters x 16 independent 32x32x16 bf16 MFMAs (32768 flops each)
 * on register operands and stores one float per lane into sink (DEVICE,
 * blocks x 256 floats, 4-byte aligned). changing = 0: near-constant
 * operands; 1: random operands that change from one MFMA to the next, as a
 * real product's do (more switching, more power, and under the part's power
 * limit a lower clock). Time it with events on `stream`.
 * ------------------------------------------------------------------------- */
int ma_calib_mfma(int32_t blocks, int32_t iters, int32_t changing, float* sink, void* stream);

/* ---------------------------------------------------------------------------
 * Stage entry points, used by the test suite to check single stages with
 * identical inputs on both sides. Same conventions as above.
 * ------------------------------------------------------------------------- */

/* out[i] = bf16 bits of in[i], round to nearest even (DEVICE buffers). */
int ma_test_bf16_round(const float* in, uint16_t* out, int64_t n, void* stream);

/* Momentum stage alone for one group: M <- RNE(beta*M + G) and, in
 * mt_out (DEVICE, count*rows*cols fp32, W's layout), the look-ahead
 * G + beta*m1 (or m1 when nesterov == 0), exactly as ma_muon_step forms it. */
int ma_test_muon_momentum(const ma_muon_group* group, float beta, int32_t nesterov,
                          float* mt_out, void* stream);

/* Decay-and-update stage alone for one group: W <- RNE(post(W, U)) with
 * U (DEVICE, count dense rows x cols matrices of u_dtype, W's layout) and the
 * scalars c_lr = lr_eff, c_wd = lr_eff*wd passed as they are. Only params[]
 * of the group is used. decay == 0 skips the decay term. */
int ma_test_muon_update(const ma_muon_group* group, const void* u, int32_t u_dtype,
                        float c_lr, float c_wd, int32_t cautious, int32_t decay, void* stream);

/* Makes the calling thread's next ma_muon_adamw_step fail with MA_ERR_HIP
 * right after its fork (AdamW already queued on the side stream), as a launch
 * failure there would: for testing that the join is still enqueued. */
int ma_test_fail_after_fork(void);

/* Newton-Schulz iteration alone: `count` dense m x n matrices (m <= n) in
 * x0 (DEVICE, dtype `precision`), result in u (DEVICE, same layout). */
size_t ma_test_ns_workspace_size(int64_t m, int64_t n, int32_t count, int32_t precision);
int ma_test_ns(int64_t m, int64_t n, int32_t count, int32_t precision, const void* x0, void* u,
               const float* abc, int32_t ns_steps, void* workspace, size_t workspace_bytes,
               void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MUON_ADAMW_H */
