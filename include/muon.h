/*
 * muon.h - C ABI of the MI355X (gfx950) Muon optimizer step library.
 *
 * One Muon step, as described by the HyperParallel FSDP Muon optimizer
 * performance RFC (mindspore-ai/hyper-parallel):
 *   - item 1(1): Newton-Schulz (NS) orthogonalisation runs on the gradient
 *     momentum M_t and needs every matrix whole;
 *   - item 2:    a 3-D expert slab [E, M, N] is E independent matrices;
 *   - item 3:    matrices with the same trailing [M, N] shape are processed
 *                together as one batch [B, M, N] (kernel fusion), which cuts
 *                host dispatch, small allocations and synchronisation;
 *   - item 6:    an AdamW-style decoupled weight decay term joins the update.
 * The RFC gives no formula.  The library computes, per matrix (the readings
 * are documented with the oracle):
 *     M   <- mu*M + G
 *     U    = G + mu*M   (nesterov != 0)   or   U = M
 *     X0   = U / (||U||_F + 1e-7), transposed to wide (rows <= cols) if tall
 *     X   <- a*X + (b*A + c*A^2)*X  with A = X*X^T, ns_steps times
 *     O    = X (transposed back if the parameter is tall)
 *     W   <- W - lr*(scale*O + wd*W)
 * How the NS iteration is evaluated (the result is that iteration's, up to
 * rounding):
 *   - bf16, min(M, N) <= 32: X = Q_k X0 with Q_k a polynomial in X0 X0^T,
 *     run in fp32 on the small m x m matrices (one Gram of X0 per call; in
 *     muon_step X0 = U as a bf16 hi and lo pair, in the Gram and the apply);
 *   - bf16, larger: X stored in bf16, products on bf16 MFMA with fp32
 *     accumulation.  U enters as a bf16 hi and lo pair (muon_step).  The
 *     steps run in groups (the first min(ns_steps, 5) when min(M, N) < 512,
 *     else the first min(4, ns_steps - 1); then pairs, then a single step):
 *     one Gram X X^T and one product R X per group, the A in between formed
 *     in the m x m space (A_{k+1} = P_k A_k P_k, R = P_last ... P_first).
 *     Below min(M, N) = 4096, or beyond 5 steps, the m x m products take
 *     split-bf16 operands (about 16 mantissa bits); A^2 is split except in
 *     the first min(3, ns_steps - 2) steps when min(M, N) >= 1536 and the
 *     first min(2, ns_steps - 2) when 512 <= min(M, N) < 1536;
 *   - fp32: the same sequence as the bf16 path for larger matrices but with
 *     fp32 FMA arithmetic throughout, one step at a time.
 * The bf16 O is within 1e-2 relative Frobenius (3e-2 max-abs) of the exact
 * iteration for 5 quintic steps on Gaussian inputs and on inputs whose
 * singular values spread over [1e-3, 1] or that have rank min(M, N) / 8;
 * the fp32 O within about 1e-5 (up to 3.4e-5 on rank min(M, N) / 8).
 *
 * Conventions for every entry point:
 *   - Device buffers (params, grads, momenta, outputs, workspace) belong to
 *     the caller.  The step entry points allocate and free nothing on the
 *     device and never synchronise the host with the device; they enqueue
 *     work on `stream` (a hipStream_t passed as void*, NULL = null stream)
 *     and return.  Part of a small group's work may run on the plan's side
 *     stream, which `stream` waits for within the call (muon_set_side_stream),
 *     so every call's work is ordered on `stream` as if it all ran there.
 *   - Pointer arguments named `*_ptrs` are HOST arrays of DEVICE pointers,
 *     one per parameter, in plan order.
 *   - Every tensor is dense row-major [batch, rows, cols], 16-byte aligned,
 *     and no two tensors overlap.
 *   - Arguments are validated before anything is enqueued.  A non-OK status
 *     from validation leaves every buffer untouched.  MUON_ERR_HIP means a
 *     launch failed after work may have been enqueued: buffer contents are
 *     then unspecified.
 *   - muon_last_error_detail() gives a thread-local text for the last error.
 *   - A plan holds host metadata, and (after its first eager step on a
 *     device, for plans with MFMA groups) one side stream and two events
 *     there, see muon_set_side_stream; it may be used from several host
 *     threads one call at a time.  Two calls that share a workspace must be
 *     ordered on one stream (the workspace holds per-call state).
 */
#ifndef MUON_H
#define MUON_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MUON_OK = 0,
  MUON_ERR_INVALID_ARG = 1,   /* null pointer, bad count, bad scalar */
  MUON_ERR_SHAPE = 2,         /* a dimension < 1, or shapes do not match the plan */
  MUON_ERR_DTYPE = 3,         /* dtype combination not supported */
  MUON_ERR_PLAN_MISMATCH = 4, /* n_params or shapes differ from the plan's */
  MUON_ERR_WORKSPACE = 5,     /* workspace null, too small or misaligned */
  MUON_ERR_HIP = 6,           /* a HIP runtime call or kernel launch failed */
  MUON_ERR_ALIGNMENT = 7,     /* a tensor pointer is not 16-byte aligned */
  MUON_ERR_TIMEOUT = 8        /* an earlier skinny-path launch on this device timed out */
} muon_status;

typedef enum { MUON_F32 = 0, MUON_BF16 = 1 } muon_dtype;

/* Shape of one parameter.  A 2-D matrix [rows, cols] has batch = 1; an expert
 * slab [E, rows, cols] has batch = E and is E independent matrices (RFC item 2). */
typedef struct {
  int64_t batch;
  int64_t rows;
  int64_t cols;
} muon_shape;

typedef struct muon_plan_s* muon_plan;

/* Build a plan for a fixed list of parameter shapes (RFC item 3: group by the
 * trailing shape).  Host only; no device work.
 *   shapes    : host array of n_params shapes (copied).
 *   n_params  : >= 1.
 *   param_dt  : dtype of params and grads (MUON_F32 or MUON_BF16).  The NS
 *               arithmetic follows it: fp32 params get an fp32 NS, bf16
 *               params the bf16-MFMA recipe with fp32 accumulation.
 *   grad_dt   : must equal param_dt.
 *   mom_dt    : dtype of the momenta; MUON_F32 only.
 *   out       : receives the plan.
 * Matrices are grouped by (min(rows,cols), max(rows,cols)); tall matrices
 * (rows > cols) join the group of their transpose and are handled in the wide
 * orientation.  MUON_ERR_SHAPE for a dimension < 1, a matrix of more than
 * 2^40 elements, or a bf16 matrix on the MFMA path (min > 32, or too wide
 * for the skinny path) with max(rows, cols) > 2^22 - 256.  No HIP call is made: the device is first queried (compute
 * units, co-resident capacity) by the first muon_step / muon_ns on it. */
muon_status muon_plan_create(const muon_shape* shapes, int32_t n_params, muon_dtype param_dt,
                             muon_dtype grad_dt, muon_dtype mom_dt, muon_plan* out);

/* Frees the plan, with its side streams and events.  If the plan made a side
 * stream, the host first waits for the work queued on it (launched by the
 * plan's calls, which their streams wait for). */
void muon_plan_destroy(muon_plan plan);

/* Bytes of device workspace muon_step / muon_ns need for this plan. */
muon_status muon_plan_workspace_bytes(muon_plan plan, size_t* bytes);

/* Number of shape groups, and for group g: canonical (m, n) = (min, max),
 * the number of matrices, how many of them are stored tall, and the number
 * of launches ("chunks") the group is split into. */
muon_status muon_plan_num_groups(muon_plan plan, int32_t* n_groups);
muon_status muon_plan_group_info(muon_plan plan, int32_t g, int64_t* m, int64_t* n,
                                 int64_t* count, int64_t* n_transposed, int64_t* n_chunks);

/* The workspace must be zero-filled once before its first use with any plan:
 * a small region of it holds the tagged words the skinny kernel's workgroups
 * exchange and a timeout flag, and an all-zero word carries no valid tag. */

/* One Muon step on every parameter of the plan (see the formulas above).
 *   param_ptrs : W, updated in place, dtype param_dt.
 *   grad_ptrs  : G, read only, dtype grad_dt.
 *   mom_ptrs   : M, updated in place, fp32.
 *   shapes     : must equal the plan's shapes (checked).
 *   lr, wd, scale, mu : finite; mu in [0, 1); nesterov 0 or 1.
 *   a, b, c    : NS polynomial coefficients, finite.
 *   ns_steps   : 0 .. 16 (the accuracy stated above is measured for the
 *                workloads' 5 steps; on Gaussian inputs it is checked on the
 *                GPU up to 16.  Beyond 5 steps NS carries an input's near-null
 *                directions, such as the bf16 rounding of a low-rank matrix,
 *                into its band, and bf16 arithmetic cannot follow them: on
 *                rank min(M, N) / 8 inputs O is then 2e-2 to 3e-1 from the
 *                exact iteration, finite and bounded up to 16 steps).
 *   workspace  : device buffer of at least muon_plan_workspace_bytes(),
 *                256-byte aligned, zero-filled once before first use.
 * Tensor results do not depend on how matrices are grouped or batched:
 * every matrix is computed with the same tiling and reduction order
 * whatever its batch, position or group.
 * The call may be recorded into a HIP graph (stream capture): it enqueues
 * kernels only.  Recorded skinny launches are numbered by a counter in the
 * workspace, so replays and eager calls can share one workspace, one at a
 * time. */
muon_status muon_step(muon_plan plan, void* const* param_ptrs, const void* const* grad_ptrs,
                      void* const* mom_ptrs, const muon_shape* shapes, int32_t n_params,
                      float lr, float mu, int32_t nesterov, float wd, float a, float b,
                      float c, int32_t ns_steps, float scale, void* workspace,
                      size_t workspace_bytes, void* stream);

/* muon_step without a workspace argument, for callers that cannot allocate
 * device memory (code recorded into a HIP graph, tight serving loops,
 * harnesses that forbid allocation).  The workspace is a file-scope device
 * array of the library, 64 MiB per device, held until the process ends:
 *   - plans whose muon_plan_workspace_bytes() exceeds 64 MiB are rejected
 *     with MUON_ERR_WORKSPACE before anything is enqueued (the skinny path's
 *     sets fit: 74 x [24, 10240] needs 6.5 MB; large MFMA groups do not);
 *   - the first call on a device looks up the array's device address, clears
 *     the array on `stream` and waits for it; that first call must not be
 *     recorded into a graph (MUON_ERR_INVALID_ARG);
 *   - every call on a device shares that device's array: calls that overlap
 *     in time on one device (other streams, other host threads) race and give
 *     undefined results; order them on one stream;
 *   - no hipMalloc, hipFree or other allocating routine is called, and the
 *     host-visible timeout word is used only if a muon_step / muon_ns call
 *     already created it.
 * Arguments, results and errors are otherwise those of muon_step; the
 * results are bit-identical to muon_step's. */
muon_status muon_step_noalloc(muon_plan plan, void* const* param_ptrs, const void* const* grad_ptrs,
                              void* const* mom_ptrs, const muon_shape* shapes, int32_t n_params,
                              float lr, float mu, int32_t nesterov, float wd, float a, float b,
                              float c, int32_t ns_steps, float scale, void* stream);

/* NS alone: out = NS(in) for every parameter, in fp32, same shapes as in.
 *   in_ptrs  : dtype param_dt (the NS input, e.g. a momentum), read only.
 *   out_ptrs : fp32 outputs.
 * Uses the same kernels and arithmetic as muon_step's NS. */
muon_status muon_ns(muon_plan plan, const void* const* in_ptrs, float* const* out_ptrs,
                    const muon_shape* shapes, int32_t n_params, float a, float b, float c,
                    int32_t ns_steps, void* workspace, size_t workspace_bytes, void* stream);

/* ---- Work split over ranks --------------------------------------------
 * Items 1(3) and 4 of the HyperParallel FSDP Muon optimizer RFC remove the
 * redundant NS work of data-parallel ranks: each rank orthogonalises only
 * the whole matrices assigned to it, and a greedy rule balances the load. */

/* Number of matrices of the plan: a 2-D parameter counts 1, an expert slab
 * [E, M, N] counts E.  Matrices are numbered in parameter order, the slices
 * of a slab in order. */
muon_status muon_plan_num_matrices(muon_plan plan, int64_t* n);

/* Whole-matrix assignment of the plan's matrices to n_ranks ranks.
 * Cost of a matrix: 3 m^2 n + m^3 with m = min and n = max of its two
 * dimensions (the algorithmic work of one NS step).  Matrices are taken in
 * decreasing cost, equal costs in plan order; each goes to the rank with the
 * smallest total so far, equal totals to the lowest rank.
 *   n_ranks   : >= 1.
 *   owner     : host array of n_owner entries, n_owner equal to
 *               muon_plan_num_matrices(); receives each matrix's rank.
 *   rank_cost : NULL, or a host array of n_ranks doubles that receives each
 *               rank's total cost.
 * Host only and deterministic, so every rank computes the same split.  On
 * error nothing is written. */
muon_status muon_plan_assign(muon_plan plan, int32_t n_ranks, int32_t* owner, int64_t n_owner,
                             double* rank_cost);

/* ---- One rank's shard of a sharded parameter ------------------------------
 * Item 1(1) of the RFC: after NS of the gathered momentum, each rank updates
 * the slice of the parameter at its own offset. */

/* W[i] <- W[i] * (1 - lr*wd) - lr*scale*O[offset + i] for 0 <= i < len, in
 * fp32, rounded once (to nearest even) to dt.
 *   w_shard : device, len elements of dt (MUON_BF16 or MUON_F32), in place.
 *   o_full  : device, fp32: the whole parameter's O in its own row-major
 *             layout, as muon_ns writes it; elements offset .. offset+len-1
 *             are read.
 *   offset, len : >= 0; len = 0 enqueues nothing.
 *   lr, wd, scale : finite.
 * Asynchronous on stream; no workspace; w_shard and o_full must not
 * overlap. */
muon_status muon_shard_update(void* w_shard, muon_dtype dt, const float* o_full, int64_t offset,
                              int64_t len, float lr, float wd, float scale, void* stream);

/* ---- Companion step for the 1-D parameters -------------------------------
 * The Muon sharding optimizer of PaddlePaddle/Paddle pull request 79428
 * ("Support Muon sharding optimizer comm overlap") keeps 2-D and 1-D
 * parameters in separate buffers; the 1-D ones (norm gains, biases) do not
 * go through NS and take AdamW with decoupled weight decay instead.  One call
 * updates a whole list of them. */

/* AdamW at step t >= 1 on n tensors, in fp32 per element:
 *   p <- p (1 - lr wd)
 *   m <- b1 m + (1 - b1) g;   v <- b2 v + (1 - b2) g^2
 *   p <- p - (lr / (1 - b1^t)) m / (sqrt(v) / sqrt(1 - b2^t) + eps)
 * with p rounded once to dt.
 *   params, grads   : host arrays of n device pointers, dtype dt
 *                     (MUON_BF16 or MUON_F32); params in place.
 *   exp_avg, exp_avg_sq : host arrays of n device pointers, fp32, in place.
 *   numels          : host array of n element counts (>= 0).
 *   lr, b1, b2, eps, wd : finite; 0 <= b1, b2 < 1; eps > 0.
 *   step            : t >= 1.
 * Pointers must be 4-byte aligned; tensors must not overlap.  Asynchronous
 * on stream; no workspace.  Validation happens before anything is enqueued. */
muon_status muon_adamw_step(void* const* params, const void* const* grads, float* const* exp_avg,
                            float* const* exp_avg_sq, const int64_t* numels, int32_t n, muon_dtype dt,
                            float lr, float b1, float b2, float eps, float wd, int64_t step,
                            void* stream);

/* ---- Diagnostics of the skinny path ---------------------------------------
 * The skinny path (bf16, min(rows, cols) <= 32) runs one persistent launch
 * per chunk whose workgroups exchange partial sums, so they must all be
 * resident at once.  muon_step / muon_ns check, before enqueueing anything,
 * that every chunk fits the device's co-resident capacity (compute units x
 * workgroups per unit from the occupancy query) and return MUON_ERR_HIP
 * otherwise.  The waits are bounded all the same: if one times out (another
 * stream's kernels held compute units, or the wait limit is too small), that
 * workgroup leaves its part of W (muon_step) or O (muon_ns) unwritten, the
 * momenta of the call are already updated, the launch still runs to
 * completion, and two flags are raised:
 *   - a word in the workspace, read by muon_workspace_status;
 *   - a host-visible word of the device (pinned host memory allocated by the
 *     first muon_step / muon_ns call on the device that is not being
 *     recorded into a graph).  The next muon_step / muon_ns call on the
 *     device returns MUON_ERR_TIMEOUT, enqueues nothing and clears it;
 *     muon_poll_timeout reads and clears it without a call. */

/* Sets *timed_out to 1 if a skinny-path launch on the current device that
 * has completed by now timed out since the word was last cleared, else 0,
 * and clears it.  No synchronisation: synchronise the stream first to cover
 * every launch enqueued so far. */
muon_status muon_poll_timeout(int32_t* timed_out);

/* Synchronises `stream` (the host waits for it), sets *timed_out to 1 if any
 * call on this workspace timed out since the last check, else 0, and clears
 * the flag.  Not for use inside graph capture. */
muon_status muon_workspace_status(muon_plan plan, void* workspace, size_t workspace_bytes, void* stream,
                                  int32_t* timed_out);

/* Polls a waiting workgroup makes before it gives up, for the launches that
 * follow in this process (default 1048576, about a second; 0 restores the
 * default).  Meant for tests of the timeout path. */
void muon_set_wait_limit(uint32_t polls);

/* Whether the calls that follow in this process may run part of a small
 * MFMA group's work on the plan's side stream (on by default; 0 turns it
 * off).  It changes only which launches may run at the same time, never a
 * result bit.  A group of several NS steps forms R_j = P_j R_{j-1} beside
 * the next step's products when its m x m launches leave compute units idle
 * (fewer 256-tiles than CUs): the Newton-Schulz steps of item 1(1) of the
 * HyperParallel FSDP Muon optimizer RFC, for a batch too small to fill the
 * device.  The side stream (default priority) and its two events are made
 * on the plan's first eager muon_step or muon_ns on a device (not while the
 * stream is captured, and not by muon_step_noalloc, whose launches all stay
 * on its stream) and released by muon_plan_destroy; the launch stream waits
 * for the side stream before the group's apply, so when a call returns
 * control all of its work is ordered on `stream`.  Thread-safe. */
void muon_set_side_stream(int32_t enable);

/* ---- Kernel timing for benchmarks ----------------------------------------
 * While enabled, every apply of the MFMA path (X' = P X or R X: the largest
 * launch of a large-matrix step, with its partial-round launch if any) is
 * bracketed by a pair of HIP events recorded on the launch stream, up to
 * 4096 applies between two reads.  Off by default; process-wide; not for use
 * while another host thread steps.  Enabling creates the events once. */
muon_status muon_kernel_timing(int32_t enable);

/* Waits for the recorded events and returns, over the applies recorded since
 * the last read: their summed duration in ms, their number, their algorithmic
 * flops (2 m^2 n per matrix: one m x m by m x n product) and the MFMA flops
 * they executed (one product per pair of operand planes: 2, 3 or 4 of them
 * with lo planes).  Resets the totals. */
muon_status muon_kernel_timing_read(double* ms, int64_t* launches, double* alg_flops, double* exec_flops);

const char* muon_status_str(muon_status s);
const char* muon_last_error_detail(void);

/* Library version as an integer (major*10000 + minor*100 + patch). */
int32_t muon_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MUON_H */
