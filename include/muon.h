/*
 * muon.h -- C ABI of libmuon, the owner-side Muon optimizer step on one
 * AMD Instinct MI355X (gfx950).
 *
 * One step on one matrix W (m x n) with gradient G and fp32 momentum M:
 *
 *   M' = mu M + G                      DMuon-2 §2.1 (momentum recurrence);
 *   U  = G + mu M'  (Nesterov)         the Nesterov variant that page uses;
 *   X0 = U / (||U||_F + eps)           HyperParallel-FSDP §2.3;
 *   if rows > cols iterate on X0^T     HyperParallel-FSDP §6.6 (transpose-first);
 *   X_{k+1} = a_k X + b_k (X X^T) X + c_k (X X^T)^2 X,  k = 0..K-1
 *                                      HyperParallel-FSDP §2.3, Eq. (1);
 *   O  = X_K (back in W's orientation)
 *   W' = W - lr (wd W + s O)           decoupled decay (HyperParallel-FSDP §6.3,
 *                                      §6.4 step 4; HyperParallel RFC item 6),
 *   s  = 0.2 sqrt(max(m, n))           RMS-matched scale, HyperParallel-FSDP §2.3.
 *
 * Parameters of the same core shape are batched ("shape fusion",
 * HyperParallel-FSDP §6.6 / Figure 10(a); HyperParallel RFC item 3): [A,B],
 * [A,1,B] and [E,A,B] all contribute (A,B) matrices, an expert tensor being E
 * independent matrices (HyperParallel-FSDP §6.3).  muon_plan_create does that
 * bucketing on the host; muon_step runs one batch on the caller's stream.
 *
 * Memory and ownership.  Every device pointer is owned by the caller.  For
 * muon_step, per batch, param, grad, momentum and ns_out are contiguous
 * row-major [count, M, N] regions (a parameter's matrices sit at the segment
 * offsets that muon_plan_segments reports); muon_step_ptrs takes one address
 * per matrix instead, and muon_step_rows one address per stored row of W and
 * G.  The library never allocates, frees or
 * synchronises device memory or streams; its state is the host-side plan, plus
 * a few HIP events per device that muon_step_batches creates on first use
 * (fork and join markers, no device memory) and keeps until the process ends,
 * and the static device array of muon_step_noalloc (part of the loaded code,
 * one copy per device).
 * All kernels are enqueued on `stream` (a hipStream_t; NULL = the null stream)
 * and the call returns without waiting for them.
 *
 * Errors.  Every argument is checked before anything is enqueued; on an error
 * nothing is launched and no buffer is touched.  A launch failure returns
 * MUON_ERR_HIP; a fault inside a kernel surfaces at the caller's next stream
 * synchronisation.
 *
 * Threading.  A plan is immutable after creation and may be used from several
 * threads.  Concurrent muon_step calls on different streams need separate
 * workspaces (and separate buffers).
 */
#ifndef LIBMUON_MUON_H
#define LIBMUON_MUON_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MUON_ABI_VERSION 8

typedef enum {
  MUON_OK = 0,
  MUON_ERR_INVALID_ARG = 1,        /* null pointer, bad index, non-finite or out-of-range value, aliasing */
  MUON_ERR_UNSUPPORTED = 2,        /* a shape or combination the library does not handle (1-D, 4-D, ...) */
  MUON_ERR_WORKSPACE_TOO_SMALL = 3,
  MUON_ERR_NO_MEMORY = 4,          /* host allocation of the plan failed */
  MUON_ERR_HIP = 5,                /* the HIP runtime refused a launch */
  MUON_ERR_INTERNAL = 6
} muon_status;

typedef enum { MUON_F32 = 0, MUON_BF16 = 1 } muon_dtype;

/* Where Newton-Schulz keeps X and what the matrix products take as operands.
 *  MUON_PREC_BF16     X stored in bf16; bf16 MFMA operands, fp32 accumulation.
 *  MUON_PREC_BF16_X32 a master copy of X with a 16-bit significand: bf16(X)
 *                     plus the bf16 rounding of X - bf16(X), kept beside
 *                     each other, so the a X term carries what bf16 cannot
 *                     hold; bf16 MFMA operands; for ill-conditioned inputs.
 *  MUON_PREC_F32      every product and every stored intermediate in fp32
 *                     (the check path).
 *  MUON_PREC_BF16_X32C (ABI version 8) the master of MUON_PREC_BF16_X32, and
 *                     each step also applies B to the part of X that bf16
 *                     cannot hold: X' = a X + B bf16(X) + B bf16(X - bf16(X)),
 *                     the apply running over twice the inner length.  With
 *                     only the master, that residue enters each step with
 *                     the weight a instead of the polynomial's own slope, so
 *                     on well-conditioned inputs the master mode's error is
 *                     1.1-1.7 times plain bf16's; with the second product it
 *                     is 0.86-0.99 times plain bf16's there, and on
 *                     ill-conditioned inputs it keeps the small singular
 *                     directions as the master mode does.  The apply's
 *                     flops double: the 8192 x 28672 step takes about 1.57
 *                     times as long as with MUON_PREC_BF16_X32, with the
 *                     same workspace.  Batches with a short side of at most
 *                     32 run it as MUON_PREC_BF16_X32 (their Gram-space
 *                     products are fp32 already), those from 33 to 127 as
 *                     MUON_PREC_F32.
 * Matrices whose short side is at most 32 form the Gram matrix of the stored X
 * with fp32 accumulation, run the polynomial on it in fp32 (fp64 on the check
 * path) and apply it with about 16-bit (bf16 hi + lo) or fp32 operands in
 * every mode (the small products are cheap); those
 * with a short side from 33 to 127 run every product on fp32 operands in every
 * mode, because bf16 rounding of A and B costs too much accuracy there. */
typedef enum { MUON_PREC_BF16 = 0, MUON_PREC_BF16_X32 = 1, MUON_PREC_F32 = 2, MUON_PREC_BF16_X32C = 3 } muon_precision;

/* MUON_SCALE_RMS: s = 0.2 sqrt(max(M, N)); MUON_SCALE_NONE: s = 1. */
typedef enum { MUON_SCALE_NONE = 0, MUON_SCALE_RMS = 1 } muon_scale;

/* A parameter shape: [M,N] (ndim 2), [M,1,N] or [E,M,N] (ndim 3).  A 3-D
 * shape whose middle dimension is 1 is read as [M,1,N]. */
typedef struct { int32_t ndim; int64_t dims[3]; } muon_shape;

typedef struct {
  int64_t max_batch_elems;  /* cap on elements per batch; 0 -> 2^29 ("memory-safe batching",
                               HyperParallel-FSDP §6.6).  A single matrix above the cap
                               still forms a batch of its own. */
  int32_t order;            /* 0: batches in descending element count (HyperParallel-FSDP
                               Figure 10(b)), ties in creation order; 1: creation order */
  int32_t skinny_kernel;    /* matrices with a short side <= 32 (split-K chunk kernels):
                               Newton-Schulz in Gram space (the iteration runs on the m x m
                               Gram matrix and multiplies back into X once, DMuon-2 Appendix
                               C.3) with 0 or 3: the Gram iteration and the apply in one launch
                               (2 launches in all); 1: 3 launches; 2 step by step,
                               X <- B' X each step (2K+1 launches).  All Gram-space forms give
                               bitwise the same results and report path 1. */
} muon_plan_options;

typedef struct muon_plan muon_plan;   /* opaque, host-only, immutable */

typedef struct {
  int64_t M, N;             /* stored matrix shape */
  int64_t count;            /* matrices in the batch */
  int32_t transposed;       /* 1 if M > N: Newton-Schulz runs on the transpose */
  int32_t num_segments;
  int32_t path;             /* 0 tiled products (short side > 32); 1 skinny, Gram space;
                               2 skinny, step by step */
  int32_t reserved;
} muon_batch_info;

/* A run of consecutive matrices of one parameter inside a batch. */
typedef struct {
  int32_t param_index;      /* index into the shapes given to muon_plan_create */
  int32_t reserved;
  int64_t first_matrix;     /* first expert index (0 for 2-D parameters) */
  int64_t num_matrices;
  int64_t elem_offset;      /* element offset of the run inside the batch buffers */
} muon_segment;

typedef struct {
  float lr;                 /* eta */
  float momentum;           /* mu, in [0, 1] */
  float weight_decay;       /* lambda, >= 0 */
  float eps;                /* >= 0; a zero denominator gives a zero direction */
  int32_t nesterov;         /* 1: U = G + mu M'; 0: U = M' */
  int32_t ns_steps;         /* K, 1..64 */
  const float* coeffs;      /* host array: 3 floats (a,b,c) used for every step, or 3*K floats */
  int32_t num_coeff_sets;   /* 1 or ns_steps */
  muon_scale scale;
  muon_precision precision;
  const float* lr_wd_device;  /* optional: device address of 2 floats {lr, weight_decay} that the
                               update kernels read when they run, in place of the two host
                               fields above (which are still validated).  Lets a caller capture
                               muon_step into a HIP graph once and change the learning rate
                               and decay between replays (the DMuon-2 paper, App. C.3, keeps
                               them outside its captured graphs).  4-byte aligned; the caller
                               keeps it valid until the launches have run.  NULL: use lr and
                               weight_decay as given. */
} muon_hparams;

typedef struct {
  void* param;              /* [count,M,N] of param_dtype, updated in place */
  muon_dtype param_dtype;
  const void* grad;         /* [count,M,N] of grad_dtype */
  muon_dtype grad_dtype;
  float* momentum;          /* [count,M,N] fp32, updated in place */
  float* ns_out;            /* optional [count,M,N] fp32: receives O (the orthogonalised
                               direction, in W's orientation, before the scale s); NULL to skip */
} muon_batch_buffers;

/* A batch's matrices at independent addresses (zero-copy batching: the
 * parameters need not be packed into one [count,M,N] buffer).  Each field is
 * a device array of `count` pointers; pointer i addresses matrix i of the
 * batch (in segment order) as an [M,N] row-major region of the stated type.
 * For a 3-D expert tensor the caller passes one pointer per expert.  The
 * arrays are read by the kernels when they run, never by the host, so the
 * library cannot check the addresses they hold: each must be 16-byte aligned
 * and the regions must not overlap one another or the workspace; the caller
 * keeps the arrays valid until the launches have run (as for lr_wd_device,
 * a captured graph replays with whatever they then hold). */
typedef struct {
  void* const* params;        /* device array [count]: param_dtype matrices, updated in place */
  muon_dtype param_dtype;
  const void* const* grads;   /* device array [count]: grad_dtype matrices */
  muon_dtype grad_dtype;
  float* const* momenta;      /* device array [count]: fp32 matrices, updated in place */
  float* const* ns_out;       /* optional device array [count]: fp32 matrices receiving O; NULL to skip */
} muon_batch_ptrs;

/* A batch whose matrices are row-level views of the caller's parameters and
 * gradients.  HyperParallel-FSDP §6.6 keeps the storage of a parameter apart
 * from the matrices Muon sees: one physical parameter may hold several
 * logical matrices (the heads of a fused QKV projection, the gate and up
 * matrices of an MoE FC1 weight), reached through a zero-copy view with a
 * reversible split / concatenate / interleave, and the logical updates are
 * written back into the physical parameter.  Here each logical matrix is
 * [M,N] in W's orientation and stored row r of matrix i (N contiguous
 * elements) sits at rows[i*M + r], so any split, concatenation or interleave
 * of whole rows, or a column range of each physical row, is a table of row
 * addresses; the update lands in place, which is the restore.  The tables
 * are read by the kernels, never by the host: every row address must be
 * 16-byte aligned, rows must not overlap one another, the other buffers or
 * the workspace, and the caller keeps the tables valid until the launches
 * have run.  Momentum and ns_out are the optimizer's own contiguous buffers. */
typedef struct {
  void* const* param_rows;        /* device array [count*M]: rows of param_dtype, updated in place */
  muon_dtype param_dtype;
  const void* const* grad_rows;   /* device array [count*M]: rows of grad_dtype */
  muon_dtype grad_dtype;
  float* momentum;                /* [count,M,N] fp32, contiguous, updated in place */
  float* ns_out;                  /* optional [count,M,N] fp32, contiguous: receives O; NULL to skip */
} muon_batch_rows;

int32_t muon_abi_version(void);
const char* muon_status_str(muon_status s);

/* Build the batch plan of n parameter shapes (HyperParallel-FSDP §6.6).
 * opt may be NULL (defaults).  On success *out owns a plan to be released
 * with muon_plan_destroy.  Errors: INVALID_ARG (null, n < 1, a zero or
 * negative dimension, element count overflow), UNSUPPORTED (ndim not 2 or 3). */
muon_status muon_plan_create(const muon_shape* shapes, int32_t n, const muon_plan_options* opt,
                             muon_plan** out);
void muon_plan_destroy(muon_plan* plan);
/* The plan's batches: one per chunk of a core-shape group (HyperParallel-FSDP
 * §6.6, Figure 10(a): the [A,B], [A,1,B] and [N,A,B] parameters of one (A,B)
 * group are merged into one batched tensor; the memory-safe cap splits a
 * group into chunks).  muon_plan_batch_info: the batch's stored matrix shape,
 * its matrix count, the transpose-first flag (rows > cols, §6.6) and its
 * kernel family; INVALID_ARG for a bad index or a null out.
 * muon_plan_segments: the runs of consecutive matrices of one parameter that
 * make up the batch, in the order the matrices sit in the batch buffers
 * (parameter i's matrices at elem_offset), copied into out[0 .. capacity-1];
 * INVALID_ARG for a bad index, a null out or a negative capacity.
 * muon_plan_num_batches returns -1 for a null plan. */
int32_t muon_plan_num_batches(const muon_plan* plan);
muon_status muon_plan_batch_info(const muon_plan* plan, int32_t batch, muon_batch_info* out);
muon_status muon_plan_segments(const muon_plan* plan, int32_t batch, muon_segment* out, int32_t capacity);

/* Device workspace (bytes, a multiple of 256) that muon_step / muon_stage_ns
 * need for this batch at this precision: the batched iterate X (and the
 * residues of its master with MUON_PREC_BF16_X32 and _X32C), the Gram matrix
 * A, the polynomial B and the
 * norm partials, sized once per batch as HyperParallel-FSDP §6.6 sizes the
 * workspace of one batched invocation (memory-safe batching keeps it bounded
 * by the 2^29-element cap).  Pure host computation; INVALID_ARG for a bad
 * index, precision or a null out. */
muon_status muon_workspace_bytes(const muon_plan* plan, int32_t batch, muon_precision precision,
                                 size_t* out);

/* One full Muon step on one batch, the owner-side step of the pages: the
 * momentum recurrence and Nesterov direction (DMuon-2 §2.1), normalisation
 * and K quintic Newton-Schulz steps (HyperParallel-FSDP §2.3, Eq. (1)) run
 * batched over the merged [count, M, N] tensor with transpose-first
 * (HyperParallel-FSDP §6.6; each matrix keeps its own norm, §6.3), then
 * decoupled decay and the scaled update (HyperParallel-FSDP §6.3 / §6.4 step
 * 4, §2.3).  workspace: device memory of at least muon_workspace_bytes,
 * 256-byte aligned, owned by the caller and not shared with a concurrent call.
 * Buffers must not overlap one another or the workspace; device pointers must
 * be 16-byte aligned.  Errors: INVALID_ARG (null or misaligned pointer, bad
 * index or dtype, overlap, an hparam out of range), WORKSPACE_TOO_SMALL
 * (nothing launched in either case); HIP if a launch is refused (kernels
 * already enqueued for the batch may have run). */
muon_status muon_step(const muon_plan* plan, int32_t batch, const muon_batch_buffers* bufs,
                      const muon_hparams* hp, void* workspace, size_t workspace_bytes, void* stream);

/* muon_step on per-matrix addresses (muon_batch_ptrs) instead of contiguous
 * batch buffers; the same kernels, results bitwise equal to muon_step on the
 * same data.  The pointer arrays must be non-NULL (ns_out optional), 16-byte
 * aligned and must not overlap one another or the workspace; the addresses
 * they hold are the caller's responsibility (see muon_batch_ptrs). */
muon_status muon_step_ptrs(const muon_plan* plan, int32_t batch, const muon_batch_ptrs* bufs,
                           const muon_hparams* hp, void* workspace, size_t workspace_bytes, void* stream);

/* muon_step on row-level views (muon_batch_rows); the same kernels, results
 * bitwise equal to muon_step on the same rows packed.  The row tables must be
 * non-NULL, 16-byte aligned and must not overlap one another, the momentum,
 * ns_out or the workspace. */
muon_status muon_step_rows(const muon_plan* plan, int32_t batch, const muon_batch_rows* bufs,
                           const muon_hparams* hp, void* workspace, size_t workspace_bytes, void* stream);

/* muon_step for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same step, with the workspace taken from a static device array of
 * MUON_NOALLOC_SCRATCH_BYTES that the library holds on every device it runs
 * on until the process ends.  Nothing is allocated or freed, and no library
 * routine that allocates is called.  A batch whose workspace
 * (muon_workspace_bytes) exceeds that size returns
 * MUON_ERR_WORKSPACE_TOO_SMALL before anything touches the device; other
 * arguments are checked as by muon_step.  The first call on a device (with
 * that device current) looks up the array's device address.  Every call on a
 * device shares that device's array: calls that overlap on one device (other
 * streams, other threads) race and give undefined results; calls ordered on
 * one stream are fine, and nothing carries over from one call to the next.
 * Results are bitwise those of muon_step. */
#define MUON_NOALLOC_SCRATCH_BYTES (64u << 20)
muon_status muon_step_noalloc(const muon_plan* plan, int32_t batch, const muon_batch_buffers* bufs,
                              const muon_hparams* hp, void* stream);

/* Several batches of one step on several streams.
 *
 * Each batch is its own batched Newton-Schulz iteration (HyperParallel-FSDP
 * §6.6: one sequence of batched products per core-shape group), so one batch's
 * kernels can run beside another's.  The pages run the batches of a step as
 * one stream of compute (§6.6, Figure 10(b)); here a second stream fills the
 * last, partial round of tiles that most tiled launches leave on 256 CUs with
 * another batch's tiles.
 *
 * Lanes.  Batches are taken in decreasing estimated run time (tiled: flops of
 * the K Gram, polynomial and apply products; skinny: bytes moved), ties in
 * the order given, and each goes to the lane with the least estimated time so
 * far (ties: the lowest lane).  Lane l runs its batches, in that order, on
 * streams[l] with workspaces[l].  muon_plan_lanes reports the assignment and
 * each lane's workspace size; it is a pure host computation.
 *
 * muon_step_batches: bufs[i] holds the buffers of batch batches[i] (as for
 * muon_step).  streams[0] is the caller's stream: the step runs after the work
 * already enqueued there and work enqueued there after the call runs after
 * the whole step (the other lanes wait for an event recorded on streams[0],
 * and streams[0] waits for an event recorded at the end of each of them).
 * The streams must belong to the current device; with nstreams = 1 the call
 * is muon_step on each batch in lane order.  Results are bitwise those of
 * muon_step on each batch.  Batch indices must be distinct; every buffer and
 * every used lane's workspace (workspaces[l] may be NULL for a lane with no
 * batch) must be disjoint from all others, since lanes run concurrently.
 * A HIP error part-way returns MUON_ERR_HIP with some batches enqueued; every
 * lane that was forked is still joined into streams[0] first, so work enqueued
 * there afterwards follows what was enqueued, and a capture still ends cleanly.
 * Capturable into a HIP graph on streams[0] (the fork and join are event
 * records and waits). */
#define MUON_MAX_STREAMS 8
muon_status muon_plan_lanes(const muon_plan* plan, int32_t n, const int32_t* batches, const muon_hparams* hp,
                            int32_t nstreams, int32_t* lane_of, size_t* lane_workspace_bytes);
muon_status muon_step_batches(const muon_plan* plan, int32_t n, const int32_t* batches,
                              const muon_batch_buffers* bufs, const muon_hparams* hp, void* const* workspaces,
                              const size_t* workspace_bytes, void* const* streams, int32_t nstreams);

/* Stage entry points, same validation.  They run the stages of muon_step one
 * at a time so each can be checked on its own.
 *  momentum: M' = mu M + G (in place) and u_out = U (fp32 [count,M,N]): the
 *            momentum recurrence and its Nesterov direction, DMuon-2 §2.1.
 *  ns:       o_out = O from u_in (both fp32 [count,M,N], W's orientation):
 *            normalisation, transpose-first and the K quintic steps,
 *            HyperParallel-FSDP §2.3, Eq. (1) and §6.6.
 *  update:   W' = W - lr (wd W + s O) from o_in (fp32 [count,M,N]): decoupled
 *            decay and the RMS-scaled update, HyperParallel-FSDP §6.3 / §6.4
 *            step 4 and §2.3.
 * Buffers are device memory owned by the caller, contiguous and 16-byte
 * aligned, and must not overlap; errors as for muon_step. */
muon_status muon_stage_momentum(const muon_plan* plan, int32_t batch, const void* grad, muon_dtype grad_dtype,
                                float* momentum, float* u_out, const muon_hparams* hp, void* stream);
muon_status muon_stage_ns(const muon_plan* plan, int32_t batch, const float* u_in, float* o_out,
                          const muon_hparams* hp, void* workspace, size_t workspace_bytes, void* stream);
muon_status muon_stage_update(const muon_plan* plan, int32_t batch, void* param, muon_dtype param_dtype,
                              const float* o_in, const muon_hparams* hp, void* stream);

/* Per-step Newton-Schulz coefficients, a pure host computation (no device
 * work, callable without a GPU).  The DMuon-2 page (App. C.3) steps with a
 * per-step schedule from the Polar Express method (Amsel et al., 2025) and the
 * HyperParallel-FSDP evaluation with an "asym5" set; neither prints values.
 * This call builds one by that method's greedy construction: step k uses the
 * odd quintic a x + b x^3 + c x^5 closest to 1 in the uniform norm on the
 * interval [l_k, u_k] that holds the singular values before the step, and
 * [l_{k+1}, u_{k+1}] is that polynomial's range over [l_k, u_k] (an odd
 * polynomial of X acts on each singular value).  [l_0, u_0] = [lower, 1]:
 * Frobenius normalisation leaves no singular value above 1, and `lower` is
 * the caller's bound on the smallest one.
 *  steps    K, 1..64.
 *  lower    in [1e-12, 1).
 *  safety   in [1, 2]; step k uses p_k(x / safety), so values up to safety*u_k
 *           (rounding overshoot) stay where p_k is designed.  1 = none.
 *  cushion  in [0, 1); step k is designed on [max(l_k, cushion*u_k, 1e-4*u_k),
 *           u_k], which keeps the first steps' coefficients small when `lower`
 *           is tiny (the bounds still cover [l_k, u_k]).  0 = only the fixed
 *           1e-4 floor, below which the levelled minimum of p_k would be
 *           within the coefficients' float rounding of zero.
 *  coeffs   out, host, 3*K floats (a_k, b_k, c_k), the layout muon_hparams
 *           takes with num_coeff_sets = ns_steps = K.
 *  bounds   out, host, optional (NULL): 2*K doubles, [l_{k+1}, u_{k+1}] after
 *           step k, computed for the float coefficients written.  In exact
 *           arithmetic every singular value of X_{k+1} lies in it.
 * With bf16 operands, a large first step (a = 8.47 from lower = 1e-3)
 * amplifies operand rounding on nearly square tiled matrices; safety 1.01 and
 * cushion 0.02 keep O within the usual bf16 error there.
 * Returns INVALID_ARG for an argument out of range (nothing written) and
 * INTERNAL if the construction fails to level (not seen in the ranges above). */
muon_status muon_ns_schedule(int32_t steps, double lower, double safety, double cushion, float* coeffs,
                             double* bounds);

/* Failure injection, for tests of the error paths: the (n + 1)-th batch
 * dispatch from now on (by any step call, on any thread) returns MUON_ERR_HIP
 * without launching anything, as a refused launch would, and the injection
 * is then off; n < 0 turns it off.  It lets a test drive a multi-stream step
 * into its part-way failure (muon_step_batches joins every forked lane before
 * returning) without a real launch failure. */
void muon_debug_fail_dispatch(int32_t n);

/* Launch tracing, for measurement.  muon_trace_start(n) makes the next (at
 * most n) kernel launches of the step and stage calls carry a start and a
 * stop HIP event that the runtime records at the kernel's start and end
 * (hipExtLaunchKernel), so they time its execution.  muon_trace_stop waits for
 * those events, writes up to `capacity` durations (ms) and kernel names
 * (static strings) in launch order, releases the events and returns the
 * number of launches traced (-1 if tracing was not started).  Tracing state
 * is process-wide; start returns INVALID_ARG if it is already on. */
muon_status muon_trace_start(int32_t max_launches);
int32_t muon_trace_stop(float* ms, const char** names, int32_t capacity);

#ifdef __cplusplus
}
#endif

#endif /* LIBMUON_MUON_H */
