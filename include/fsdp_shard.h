/*
 * fsdp_shard.h -- C ABI of one rank's FSDP2 sharded step on MI355X (gfx950).
 *
 * The library implements the four per-rank data movements of fully sharded
 * data parallel training with per-parameter Shard(0) sharding and a
 * bf16-param / fp32-reduce mixed-precision policy:
 *
 *   copy-in   fsdp_pack_allgather    fp32 master shards -> bf16 [S] segment
 *   copy-out  fsdp_unpack_allgather  bf16 [N, S] buffer  -> full bf16 params
 *   reduce    fsdp_reduce_shard      bf16 [N, S] grads   -> fp32 grad shards
 *   update    fsdp_adamw_shard       AdamW on fp32 master, m and v shards
 *   fused     fsdp_step_shard        reduce -> AdamW -> copy-in in one pass
 *   executor  fsdp_step_groups       a whole step over many groups, one call
 *   sets      fsdp_adamw_groups, fsdp_pack_allgather_groups,
 *             fsdp_adamw_pack_groups, fsdp_amax_groups,
 *             fsdp_pack_allgather_fp8_groups, fsdp_step_group_set
 *             AdamW, amax and copy-ins of many groups, one launch each
 *
 * and around them: the reduce-scatter copy-in (fsdp_pack_reduce_scatter),
 * fp32 contributions (fsdp_reduce_shard_f32), the FP8 E4M3 all-gather
 * (fsdp_pack_allgather_fp8, fsdp_unpack_allgather_fp8, fsdp_amax_shard),
 * gradient accumulation without sync (fsdp_accumulate_grad,
 * fsdp_pack_reduce_scatter_acc), AdamW on host shards (fsdp_adamw_host) and
 * resharding saved shards to another world size (fsdp_reshard_*); plus a
 * host-side shard-layout planner.  The collectives between these steps
 * (all-gather, reduce-scatter) are not part of the library: a caller runs
 * them on the buffers these calls read and write.
 *
 * Pages cited (by title and section):
 *   [ST] "Sharded Training: FSDP2, DTensor, Tensor and Pipeline Parallelism"
 *   [MS] "Introduction to PyTorch FSDP2 Backend Features"
 *   [AF] "PyTorch FSDP2 Guide: Distributed LLM Training with DTensor"
 *
 * Conventions for every function below.
 *  - Every call returns an fsdp_status: FSDP_OK (0) or a negative error.  No
 *    C++ exception crosses the ABI.  On error, fsdp_last_error() returns a
 *    thread-local message naming the offending argument, and nothing has been
 *    launched.
 *  - Device pointers are plain addresses of device memory on the device that
 *    was current when fsdp_bind ran; streams are hipStream_t values passed as
 *    void* (NULL = the default stream).  Hot calls only enqueue work on the
 *    stream: they never synchronize and never allocate.
 *  - The caller owns every tensor.  The library owns the plan and the device
 *    tables it uploads at bind time, and frees both in fsdp_plan_destroy.
 *  - bf16 values travel as uint16_t bit patterns; fp32 as float.
 *  - A shard's valid elements start at offset 0 of the pointer the caller
 *    binds; nothing past local_rows * cols is read or written.
 *  - Sizes and offsets are in elements unless a name says bytes.
 */
#ifndef FSDP_SHARD_H
#define FSDP_SHARD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FSDP_ABI_VERSION 1

typedef int32_t fsdp_status;
enum {
    FSDP_OK = 0,
    FSDP_E_INVAL = -1,        /* null pointer, world < 1, rank out of range,
                                 negative rows or cols, bad index           */
    FSDP_E_UNSUPPORTED = -2,  /* align_elems not 1 or 8, zero_stage not 0..3 */
    FSDP_E_ALIGN = -3,        /* fp32 pointer not 4-byte or bf16 pointer not
                                 2-byte aligned                            */
    FSDP_E_STATE = -4,        /* hot call before the roles it needs are bound,
                                 or on a device other than the bound one    */
    FSDP_E_HIP = -5,          /* HIP runtime error (launch, copy, async)    */
    FSDP_E_NOMEM = -6         /* host or device allocation failed at plan or
                                 bind time                                 */
};

/* Opaque per-(group, rank) plan. */
typedef struct fsdp_plan fsdp_plan;

/* Layout of one parameter of the group, as seen by this rank.
 * [ST] fully_shard paragraph: rank r keeps chunk r of
 * torch.chunk(param, world, dim=0), padded internally; chunk_rows is
 * ceil(rows / world), so ranks past the last chunk hold empty pieces. */
typedef struct fsdp_shard_entry_t {
    int64_t rows;         /* dim 0 of the parameter                         */
    int64_t cols;         /* product of the other dims (1 for 1-D)          */
    int64_t chunk_rows;   /* c = ceil(rows / world), 0 when rows == 0       */
    int64_t row_begin;    /* first row this rank owns: min(rank * c, rows)  */
    int64_t local_rows;   /* rows this rank owns (0 = empty chunk)          */
    int64_t shard_offset; /* element offset of the piece inside a segment   */
    int64_t shard_numel;  /* padded piece: c * cols                         */
    int64_t valid_numel;  /* local_rows * cols                              */
    int64_t pad_numel;    /* shard_numel - valid_numel                      */
    int64_t seg_numel;    /* shard_numel rounded up to align_elems          */
} fsdp_shard_entry_t;

typedef struct fsdp_plan_info_t {
    int32_t n_params;
    int32_t world;
    int32_t rank;
    int32_t align_elems;
    int64_t S;            /* segment length: sum of seg_numel (any rank)    */
    int64_t V;            /* valid elements this rank owns                  */
    int64_t F;            /* elements of the full (unsharded) parameters    */
    int64_t pad_total;    /* S - V                                          */
    int32_t n_empty;      /* parameters whose piece on this rank is empty   */
    int32_t bound;        /* bitmask of bound roles (FSDP_ROLE_*)           */
    int64_t n_tiles[4];   /* work tiles of pack, unpack, reduce, adamw      */
} fsdp_plan_info_t;

/* torch.optim.AdamW hyperparameters ([ST] ZeroRedundancyOptimizer example
 * and lab: lr = 3e-4; betas, eps and weight decay are AdamW's). */
typedef struct fsdp_adamw_hparams_t {
    double lr;
    double beta1;
    double beta2;
    double eps;
    double weight_decay;
} fsdp_adamw_hparams_t;

enum {
    FSDP_ROLE_MASTER = 1,
    FSDP_ROLE_GRAD = 2,
    FSDP_ROLE_EXP_AVG = 4,
    FSDP_ROLE_EXP_AVG_SQ = 8,
    FSDP_ROLE_FULL = 16,
    FSDP_ROLE_FULL_GRAD = 32,
    FSDP_ROLE_GRAD_ACC = 64,
    FSDP_ROLE_FULL_FP8 = 128
};

/* Element types of the reduce-scatter buffers. */
enum { FSDP_DTYPE_BF16 = 0, FSDP_DTYPE_F32 = 1 };

/* ---- library ---------------------------------------------------------- */

int32_t fsdp_abi_version(void);
/* Static string for a status code; never NULL. */
const char *fsdp_status_string(fsdp_status s);
/* Thread-local detail of this thread's last failed call ("" if none). */
const char *fsdp_last_error(void);

/* ---- planner: host only, needs no GPU ---------------------------------- */

/* Plan the communication segment of one parameter group for rank `rank`.
 * [ST] fully_shard paragraph: every parameter is a Shard(0) DTensor built
 * from torch.chunk with internal padding, and one fully_shard call makes one
 * group, one unit of communication.  The group's pieces are laid out in
 * registration order (rows[i], cols[i] for i < n_params), each padded to
 * chunk_rows * cols elements and its start rounded up to a multiple of
 * align_elems (1: no gap; 8: 16-byte starts).  S does not depend on rank.
 *   rows, cols   host arrays of n_params entries; rows >= 0, cols >= 1
 *                (cols = numel / dim 0; a 0-dim tensor cannot be sharded)
 *   world        N >= 1; rank in [0, N)
 *   out          receives a new plan; release with fsdp_plan_destroy
 * Errors: FSDP_E_INVAL, FSDP_E_UNSUPPORTED (align_elems), FSDP_E_NOMEM. */
fsdp_status fsdp_plan_create(const int64_t *rows, const int64_t *cols,
                             int32_t n_params, int32_t world, int32_t rank,
                             int32_t align_elems, fsdp_plan **out);

fsdp_status fsdp_plan_info(const fsdp_plan *plan, fsdp_plan_info_t *out);

/* Layout of parameter i on this rank.  Errors: FSDP_E_INVAL. */
fsdp_status fsdp_plan_entry(const fsdp_plan *plan, int32_t i,
                            fsdp_shard_entry_t *out);

/* Rows of parameter i owned by rank j (any j in [0, N)): the copy-out reads
 * them from row j of the all-gather buffer.  Errors: FSDP_E_INVAL. */
fsdp_status fsdp_plan_rows_of_rank(const fsdp_plan *plan, int32_t i, int32_t j,
                                   int64_t *row_begin, int64_t *local_rows);

/* Bytes of training state per rank for n_params parameters under ZeRO stage
 * 0..3 with 16 bytes per parameter (2 bf16 weights, 2 bf16 grads, 12 for the
 * fp32 master and Adam's two moments): [ST] opening paragraph, ZeRO
 * paragraph and Fence 1; [AF] "The Problem" (1,120 GB for 70B).
 * Errors: FSDP_E_INVAL (world < 1, n_params < 0, null out),
 *         FSDP_E_UNSUPPORTED (zero_stage). */
fsdp_status fsdp_state_bytes(double n_params, int32_t world, int32_t zero_stage,
                             double *per_rank_bytes);

/* Frees the plan and its device tables.  Waits for the device to finish
 * using them.  NULL is a no-op. */
void fsdp_plan_destroy(fsdp_plan *plan);

/* ---- bind: device tables, once per set of persistent tensors ------------ */

/* Record the per-parameter device tensors of this rank and upload the plan's
 * device tables (entries and work tiles) on `stream`, then wait for that
 * upload.  Each array is a host array of n_params device pointers, or NULL to
 * leave that role unbound:
 *   master, grad, exp_avg, exp_avg_sq  fp32 shards, valid_numel elements each
 *                                      (the sharded parameter, its reduced
 *                                      gradient, AdamW's m and v: [ST] the
 *                                      optimizer built after sharding sees
 *                                      only shards, so its state is sharded)
 *   full                               bf16 [rows, cols] unsharded params
 * A pointer may be NULL where its tensor has no elements.  Binding again
 * replaces the pointers (waiting for the stream first).  Allocates device
 * memory on the current device the first time.  A rejected call (bad
 * argument) keeps the previous binding; a HIP failure during the upload
 * leaves the plan unbound until a bind succeeds.
 * Errors: FSDP_E_INVAL (null pointer for a non-empty tensor), FSDP_E_ALIGN,
 *         FSDP_E_NOMEM, FSDP_E_HIP. */
fsdp_status fsdp_bind(fsdp_plan *plan, float *const *master, float *const *grad,
                      float *const *exp_avg, float *const *exp_avg_sq,
                      uint16_t *const *full, void *stream);

/* Bind each parameter's unsharded bf16 gradient [rows, cols] (the input of
 * the reduce-scatter copy-in).  full_grad is a host array of n_params device
 * pointers; NULL only where the parameter has no elements.  Uploads the
 * entry table like fsdp_bind (allocating the device tables on first use).
 * Errors: FSDP_E_INVAL, FSDP_E_ALIGN, FSDP_E_NOMEM, FSDP_E_HIP. */
fsdp_status fsdp_bind_full_grad(fsdp_plan *plan, uint16_t *const *full_grad, void *stream);

/* Bind each parameter's unsharded fp32 gradient accumulator [rows, cols]
 * (gradient accumulation without sync).  Same rules as
 * fsdp_bind_full_grad, 4-byte aligned pointers. */
fsdp_status fsdp_bind_grad_acc(fsdp_plan *plan, float *const *grad_acc, void *stream);

/* Bind each parameter's unsharded FP8 E4M3 tensor [rows, cols] (one byte per
 * element; the FP8 copy-out's destination).  Same rules as
 * fsdp_bind_full_grad, any byte alignment. */
fsdp_status fsdp_bind_full_fp8(fsdp_plan *plan, uint8_t *const *full_fp8, void *stream);

/* ---- hot path: enqueue on `stream`; no sync, no allocation ------------- */

/* All-gather copy-in.  Writes all S elements of ag_in: for each parameter,
 * ag_in[shard_offset + i] = bf16(master[i]) for i < valid_numel, rounded to
 * nearest even (a NaN stays a quiet NaN with its sign), and 0 in the piece's
 * padding and any alignment gap.  [ST] "Mixed precision": sharded parameters
 * stay fp32 and bf16 copies are all-gathered (param_dtype, half the bytes);
 * [MS] "Mixed Precision".  ag_in may be row `rank` of the [N, S] all-gather
 * output (in-place all-gather).  Needs FSDP_ROLE_MASTER.
 * Errors: FSDP_E_INVAL (null ag_in with S > 0), FSDP_E_ALIGN, FSDP_E_STATE,
 *         FSDP_E_HIP. */
fsdp_status fsdp_pack_allgather(const fsdp_plan *plan, uint16_t *ag_in,
                                void *stream);

/* All-gather copy-out.  ag_out is the [N, S] bf16 all-gather result, row j =
 * rank j's segment.  For every parameter and every rank j, copies rank j's
 * local_rows(j) * cols valid elements to rows [row_begin(j), ...) of the full
 * [rows, cols] tensor; padding is never read.  [ST] fully_shard paragraph
 * (chunks of torch.chunk, padded internally); [MS] "DTensor" (the logical
 * tensor is the whole parameter).  Bit copy, no arithmetic.
 * Needs FSDP_ROLE_FULL.  Errors: as fsdp_pack_allgather. */
fsdp_status fsdp_unpack_allgather(const fsdp_plan *plan, const uint16_t *ag_out,
                                  void *stream);

/* Reduce-scatter's local reduction for this rank.  rs_in is [N, S] bf16: row
 * j is rank j's gradient contribution laid out like a segment.  For each
 * parameter and i < valid_numel:
 *     grad[i] = ((x_0 + x_1) + ... + x_{N-1}) / N,   x_j = fp32(rs_in[j][off+i])
 * with fp32 adds in rank order and one correctly rounded fp32 division.
 * [ST] "Mixed precision" (reduce_dtype fp32), "Other controls" and "The bug
 * Adam hid" (set_force_sum_reduction_for_comms: reduce with SUM and divide by
 * the world size); [MS] "Mixed Precision".  Padding is never read.
 * Needs FSDP_ROLE_GRAD.  Errors: as fsdp_pack_allgather. */
fsdp_status fsdp_reduce_shard(const fsdp_plan *plan, const uint16_t *rs_in,
                              void *stream);

/* Reduce-scatter copy-in: writes the whole [N, S] input of the
 * reduce-scatter from this rank's unsharded gradients.  Row j gets chunk j of
 * every parameter (rows [row_begin(j), row_begin(j) + local_rows(j))) at its
 * shard offset, then zeros up to the next piece, so row j has the layout of
 * rank j's segment; the collective then hands rank j the sum of everyone's
 * row j.  [MS] "Working Principle" (Reduce-Scatter state) and "Mixed
 * Precision" (BF16 gradients cast to FP32 for the reduction); [ST] ZeRO
 * paragraph.  dtype FSDP_DTYPE_BF16 copies the bits; FSDP_DTYPE_F32 widens
 * each value exactly (reduce_dtype = fp32 on the wire); padding is 0 / +0.0.
 *   rs_out  [N, S] of the chosen dtype (2- or 4-byte aligned)
 * Needs FSDP_ROLE_FULL_GRAD.  Errors: FSDP_E_INVAL, FSDP_E_UNSUPPORTED
 * (dtype), FSDP_E_ALIGN, FSDP_E_STATE, FSDP_E_HIP. */
fsdp_status fsdp_pack_reduce_scatter(const fsdp_plan *plan, void *rs_out, int32_t dtype,
                                     void *stream);

/* FP8 all-gather copy-in ([AF] "Native FP8 Training with Float8Tensor":
 * parameters held in FP8 E4M3 and all-gathered as raw FP8 bytes, half the
 * traffic of bf16).  Writes all S bytes of ag_in: for each parameter p,
 * ag_in[shard_offset + i] = e4m3(fp32(master[i] * scales[p])) for
 * i < valid_numel, zero elsewhere.  e4m3 is the OCP e4m3fn format, round to
 * nearest even, magnitudes >= 448 and infinities saturated to +-448, NaN
 * kept as the NaN code with its sign.
 *   scales  device array of n_params fp32 per-tensor scales (e.g. 448 / amax
 *           with amax the maximum over ranks of fsdp_amax_shard's output)
 * Needs FSDP_ROLE_MASTER.  Errors: FSDP_E_INVAL, FSDP_E_ALIGN (scales),
 * FSDP_E_STATE, FSDP_E_HIP. */
fsdp_status fsdp_pack_allgather_fp8(const fsdp_plan *plan, uint8_t *ag_in, const float *scales,
                                    void *stream);

/* FP8 copy-out: [N, S] E4M3 bytes -> every parameter's bound FP8 [rows, cols]
 * tensor (bytes copied, kept FP8 for FP8 GEMMs), row mapping as
 * fsdp_unpack_allgather.  Needs FSDP_ROLE_FULL_FP8.
 * Errors: FSDP_E_INVAL, FSDP_E_STATE, FSDP_E_HIP. */
fsdp_status fsdp_unpack_allgather_fp8(const fsdp_plan *plan, const uint8_t *ag_out, void *stream);

/* Per-parameter largest |master| over this rank's shard into amax (device,
 * n_params fp32; 0 for an empty shard; a NaN propagates).  The maximum
 * across ranks (a collective, outside this library) gives tensor-wise FP8
 * scaling.  Launches a clear of amax and a reduction; amax is complete when
 * the stream reaches it.  Needs FSDP_ROLE_MASTER.
 * Errors: FSDP_E_INVAL, FSDP_E_ALIGN, FSDP_E_STATE, FSDP_E_HIP. */
fsdp_status fsdp_amax_shard(const fsdp_plan *plan, float *amax, void *stream);

/* Gradient accumulation without sync ([ST] "Other controls":
 * set_requires_gradient_sync(False) accumulates unsharded gradients and
 * skips the reduce-scatter): for every element of every parameter,
 *     acc = reset ? fp32(g) : acc + fp32(g)
 * with g the bound bf16 unsharded gradient and acc the bound fp32
 * accumulator (reduce_dtype), one fp32 rounding per add.
 * Needs FSDP_ROLE_FULL_GRAD | FSDP_ROLE_GRAD_ACC.
 * Errors: FSDP_E_INVAL, FSDP_E_STATE, FSDP_E_HIP. */
fsdp_status fsdp_accumulate_grad(const fsdp_plan *plan, int32_t reset, void *stream);

/* Reduce-scatter copy-in of the synchronizing microbatch from the fp32
 * accumulators: the [N, S] fp32 layout of fsdp_pack_reduce_scatter (row j =
 * chunk j of every parameter, +0.0 padding), values copied from acc.
 * Needs FSDP_ROLE_GRAD_ACC.  Errors: FSDP_E_INVAL, FSDP_E_ALIGN (4 bytes),
 * FSDP_E_STATE, FSDP_E_HIP. */
fsdp_status fsdp_pack_reduce_scatter_acc(const fsdp_plan *plan, float *rs_out, void *stream);

/* fsdp_reduce_shard for fp32 contributions (reduce_dtype = fp32 on the
 * wire): grad[i] = ((x_0 + x_1) + ... + x_{N-1}) / N with x_j = rs_in[j][off+i]
 * read as fp32, adds in rank order, one correctly rounded division.
 * [ST] "Mixed precision" and "Other controls"; [MS] "Mixed Precision".
 *   rs_in  [N, S] fp32, 4-byte aligned
 * Needs FSDP_ROLE_GRAD.  Errors: as fsdp_reduce_shard. */
fsdp_status fsdp_reduce_shard_f32(const fsdp_plan *plan, const float *rs_in, void *stream);

/* One AdamW step (decoupled weight decay, bias-corrected; amsgrad and
 * maximize off) on every bound shard, in place.  `step` counts from 1; m and
 * v must be zero before step 1.  Host scalars come from the hyperparameters
 * in fp64 and are rounded once to fp32; per element, each operation is one
 * fp32 rounding, no fused multiply-add:
 *     p = p * (1 - lr*wd);  m = b1*m + (1-b1)*g;  v = b2*v + (1-b2)*(g*g)
 *     p = p - (lr / (1 - b1^t)) * (m / (sqrt(v) / sqrt(1 - b2^t) + eps))
 * [ST] ZeroRedundancyOptimizer example and lab (torch.optim.AdamW at
 * lr 3e-4), fully_shard paragraph (optimizer state sharded with the
 * parameters); [MS] "Working Principle" (Update State).
 * Needs FSDP_ROLE_MASTER | GRAD | EXP_AVG | EXP_AVG_SQ.
 * Errors: FSDP_E_INVAL (null hparams, step < 1), FSDP_E_STATE, FSDP_E_HIP. */
fsdp_status fsdp_adamw_shard(const fsdp_plan *plan,
                             const fsdp_adamw_hparams_t *hp, int64_t step,
                             void *stream);

/* Flags of fsdp_step_shard and fsdp_step_groups. */
enum { FSDP_STEP_WRITE_GRAD = 1, FSDP_STEP_UNFUSED = 2 };

/* Kernel selectors for the timing hooks of fsdp_step_groups and
 * fsdp_step_group_set. */
enum {
    FSDP_KERNEL_STEP = 0,
    FSDP_KERNEL_REDUCE = 1,
    FSDP_KERNEL_ADAMW = 2,
    FSDP_KERNEL_PACK = 3,
    FSDP_KERNEL_UNPACK = 4,
    FSDP_KERNEL_ADAMW_PACK = 5
};

/* Fused sharded step: reduce -> AdamW -> copy-in in one pass over this
 * rank's pieces.  Per valid element it computes the reduced gradient exactly
 * as fsdp_reduce_shard (fp32 sum in rank order, one division by N), applies
 * the AdamW update of fsdp_adamw_shard with that gradient, and writes the
 * bf16 cast of the new master into ag_in as fsdp_pack_allgather does (zeros
 * in padding and gaps).  Results are bit-identical to the three calls in
 * sequence; the gradient is written to the bound grad shards only with
 * FSDP_STEP_WRITE_GRAD, saving its write and re-read otherwise.
 * [MS] "Working Principle" (Reduce-Scatter state, then the Update state on the
 * gradient slices; the next all-gather gathers the updated shards); [ST]
 * fully_shard paragraph (optimizer on the shards) and "Mixed precision".
 *   rs_in  [N, S] bf16 contributions, as for fsdp_reduce_shard
 *   ag_in  [S] bf16 copy-in output (may be row `rank` of the all-gather
 *          buffer); must not overlap rs_in
 * Needs FSDP_ROLE_MASTER | EXP_AVG | EXP_AVG_SQ, plus GRAD with the flag.
 * Errors: FSDP_E_INVAL (null buffer with S > 0, ag_in overlapping rs_in,
 *         null hparams, step < 1, unknown flag), FSDP_E_ALIGN, FSDP_E_STATE,
 *         FSDP_E_HIP. */
fsdp_status fsdp_step_shard(const fsdp_plan *plan, const uint16_t *rs_in,
                            uint16_t *ag_in, const fsdp_adamw_hparams_t *hp,
                            int64_t step, uint32_t flags, void *stream);

/* One rank's whole sharded step over n_groups parameter groups, launched
 * from native code in group order on one stream (one call instead of two to
 * four per group, so host launch overhead cannot starve the GPU).  For group
 * g: fsdp_step_shard(plans[g], rs_in[g], ag_in[g], ...) -- or, with
 * FSDP_STEP_UNFUSED, fsdp_reduce_shard, fsdp_adamw_shard and
 * fsdp_pack_allgather -- then, unless ag_out is NULL,
 * fsdp_unpack_allgather(plans[g], ag_out[g]).  Results equal those calls
 * made one by one.  [MS] "Working Principle" (per-group reduce-scatter,
 * sharded update, all-gather before the next use); [ST] fully_shard
 * paragraph (one group = one communication unit).
 *   plans, rs_in, ag_in, ag_out  host arrays of n_groups entries (device
 *                                buffers as in the single-group calls)
 *   timing_events  NULL, or 2*n_groups hipEvent_t (as void*): events 2g and
 *                  2g+1 are recorded on `stream` just before and after group
 *                  g's launch of kernel `timed_kernel` (FSDP_KERNEL_*), which
 *                  must be one this call runs.  A NULL pair leaves group g
 *                  untimed (each recorded pair breaks the back-to-back
 *                  dispatch of two launches, so a caller may time a few
 *                  groups per step); a pair with one NULL is an error
 * Every group is checked before anything is launched.  Errors: as the
 * single-group calls, plus FSDP_E_INVAL for null arrays, unknown flags or a
 * timed kernel the call does not run. */
fsdp_status fsdp_step_groups(fsdp_plan *const *plans, int32_t n_groups,
                             const uint16_t *const *rs_in, uint16_t *const *ag_in,
                             const uint16_t *const *ag_out,
                             const fsdp_adamw_hparams_t *hp, int64_t step,
                             uint32_t flags, int32_t timed_kernel,
                             void *const *timing_events, void *stream);

/* ---- group sets: one launch for the AdamW and the copy-in of many groups -- */

/* The optimizer is built over the whole sharded model, so one optimizer step
 * updates the shards of every group ([ST] fully_shard paragraph: build the
 * optimizer after sharding, its state sharded with the parameters; [MS]
 * "Working Principle", Update state).  A group set runs that step, and the
 * copy-in of every group, as one multi-tensor launch each over a
 * concatenated device table, instead of one launch per group.  It borrows
 * its plans (destroy the set before them) and holds their AdamW tensors as
 * bound when it was built: rebinding master, grad, exp_avg or exp_avg_sq of
 * any group makes every call on the set fail with FSDP_E_STATE. */
typedef struct fsdp_group_set fsdp_group_set;

/* Builds a set over n_groups distinct plans, each bound at least once (its
 * device tables exist), all on the current device.  Uploads the tables on
 * `stream` and waits for it.  The copy-in arena of the set holds group g's
 * S_g-element segment at an offset that fsdp_group_set_segment reports
 * (each segment starts on a multiple of 8 elements; the up to 7 elements
 * between segments are never written).
 * Errors: FSDP_E_INVAL (null or repeated plan, n_groups < 1, bound shard
 *         tensors that overlap where the AdamW update writes: a master,
 *         exp_avg or exp_avg_sq element that is also part of another bound
 *         shard of the set), FSDP_E_STATE (a plan never bound, plans on
 *         different devices or not on the current one), FSDP_E_NOMEM,
 *         FSDP_E_HIP. */
fsdp_status fsdp_group_set_create(fsdp_plan *const *plans, int32_t n_groups,
                                  void *stream, fsdp_group_set **out);

/* Waits for the device and frees the set's tables; NULL is ignored. */
void fsdp_group_set_destroy(fsdp_group_set *set);

/* The number of groups and of parameters of the set (its parameters are
 * numbered group by group, in each group's registration order) and the
 * elements of its copy-in arena.  Errors: FSDP_E_INVAL (null argument). */
fsdp_status fsdp_group_set_info(const fsdp_group_set *set, int32_t *n_groups,
                                int32_t *n_params, int64_t *arena_elems);

/* Group g's copy-in segment: elements [*offset, *offset + S_g) of the arena,
 * which holds *arena_elems elements in all.  Errors: FSDP_E_INVAL. */
fsdp_status fsdp_group_set_segment(const fsdp_group_set *set, int32_t g,
                                   int64_t *offset, int64_t *arena_elems);

/* fsdp_adamw_shard on every group of the set, in one launch; results are
 * bit-identical to the per-group calls.  Needs FSDP_ROLE_MASTER | GRAD |
 * EXP_AVG | EXP_AVG_SQ on every group.
 * Errors: as fsdp_adamw_shard, plus FSDP_E_INVAL (null set) and
 *         FSDP_E_STATE (a group rebound since the set was built). */
fsdp_status fsdp_adamw_groups(const fsdp_group_set *set,
                              const fsdp_adamw_hparams_t *hp, int64_t step,
                              void *stream);

/* fsdp_pack_allgather of every group of the set into its segment of
 * `arena` (bf16, 2-byte aligned; 16-byte aligned for full-width stores), in
 * one launch; each segment equals the per-group copy-in.  The arena may not
 * share a byte with any bound shard tensor of the set.  Needs
 * FSDP_ROLE_MASTER on every group.
 * Errors: FSDP_E_INVAL (null set, null arena, arena overlapping a shard),
 *         FSDP_E_ALIGN, FSDP_E_STATE, FSDP_E_HIP. */
fsdp_status fsdp_pack_allgather_groups(const fsdp_group_set *set, uint16_t *arena,
                                       void *stream);

/* fsdp_adamw_groups and fsdp_pack_allgather_groups in one launch: per
 * element the AdamW update, then the bf16 cast of the new master into the
 * group's arena segment (zeros in padding), so the master is read once for
 * both.  The optimizer step that writes the next all-gather's input ([ST]
 * fully_shard paragraph and "Mixed precision"; [MS] "Working Principle":
 * the update, then the all-gather of the updated shards).  Results are
 * bit-identical to the two calls.  Needs FSDP_ROLE_MASTER | GRAD | EXP_AVG |
 * EXP_AVG_SQ on every group.
 * Errors: as fsdp_adamw_groups and fsdp_pack_allgather_groups. */
fsdp_status fsdp_adamw_pack_groups(const fsdp_group_set *set,
                                   const fsdp_adamw_hparams_t *hp, int64_t step,
                                   uint16_t *arena, void *stream);

/* fsdp_amax_shard of every group in one launch: amax[k] = the largest |x|
 * of the set's parameter k (numbered as by fsdp_group_set_info) over this
 * rank's master shard, NaN if it holds one, 0 if it is empty; amax holds
 * n_params floats.  [AF] FP8 item (tensor-wise scales from the amax).
 * Needs FSDP_ROLE_MASTER.  Errors: FSDP_E_INVAL (null set or amax),
 * FSDP_E_ALIGN, FSDP_E_STATE, FSDP_E_HIP. */
fsdp_status fsdp_amax_groups(const fsdp_group_set *set, float *amax, void *stream);

/* fsdp_pack_allgather_fp8 of every group in one launch: group g's FP8 E4M3
 * segment (S_g bytes) at byte offset fsdp_group_set_segment's offset of
 * `arena`, scaled by scales[k] for the set's parameter k.  Each segment
 * equals the per-group FP8 copy-in.  The arena may not share a byte with a
 * bound shard tensor.  [AF] FP8 item; [ST] "Mixed precision".  Needs
 * FSDP_ROLE_MASTER.  Errors: FSDP_E_INVAL (null set, arena or scales; arena
 * overlapping a shard), FSDP_E_ALIGN, FSDP_E_STATE, FSDP_E_HIP. */
fsdp_status fsdp_pack_allgather_fp8_groups(const fsdp_group_set *set, uint8_t *arena,
                                           const float *scales, void *stream);

/* Flags of fsdp_step_group_set: AdamW and copy-in as one fused launch
 * (fsdp_adamw_pack_groups) instead of two. */
enum { FSDP_SET_ADAMW_COPY_IN = 1 };

/* The unfused sharded step of a set, from native code on one stream:
 * fsdp_reduce_shard of every group in order (each group's reduce-scatter
 * output arrives on its own), then fsdp_adamw_groups and
 * fsdp_pack_allgather_groups (with FSDP_SET_ADAMW_COPY_IN:
 * fsdp_adamw_pack_groups), then -- unless ag_out is NULL --
 * fsdp_unpack_allgather of every group.  Master, grad, m, v, the arena
 * segments and the full tensors equal those of fsdp_step_groups with
 * FSDP_STEP_UNFUSED and ag_in[g] = the group's segment.
 *   rs_in, ag_out  host arrays of one device buffer per group, as for
 *                  fsdp_step_groups; the arena must not overlap any rs_in
 *   timing_events  NULL, or 2*n_groups hipEvent_t: for the per-group
 *                  kernels (FSDP_KERNEL_REDUCE, FSDP_KERNEL_UNPACK) events
 *                  2g and 2g+1 bracket group g's launch; for the one-launch
 *                  kernels (FSDP_KERNEL_ADAMW, FSDP_KERNEL_PACK, or with the
 *                  flag FSDP_KERNEL_ADAMW_PACK) events 0 and 1 bracket that
 *                  launch.  A NULL pair is skipped; a pair with one NULL is
 *                  an error
 * Every argument is checked before anything is launched.  Errors: as the
 * calls it makes, plus FSDP_E_INVAL for a null rs_in array, an unknown
 * flag, an arena overlapping an rs_in buffer or a timed kernel the call
 * does not run. */
fsdp_status fsdp_step_group_set(const fsdp_group_set *set,
                                const uint16_t *const *rs_in, uint16_t *arena,
                                const uint16_t *const *ag_out,
                                const fsdp_adamw_hparams_t *hp, int64_t step,
                                uint32_t flags, int32_t timed_kernel,
                                void *const *timing_events, void *stream);

/* ---- CPU offload --------------------------------------------------------- */

/* AdamW on host-resident fp32 shards (CPU offload: [ST] "Offload" --
 * parameter shards, gradients and optimizer state in pinned host memory,
 * optimizer step on the CPU).  Same update, element for element, as
 * fsdp_adamw_shard (bit-identical results); n elements of p, g, m, v (host
 * pointers); n_threads <= 0 uses every hardware thread.  Synchronous; needs
 * no GPU; a range whose thread cannot be started runs on the calling
 * thread.  Errors: FSDP_E_INVAL (null arrays, n < 0, null hparams,
 * step < 1). */
fsdp_status fsdp_adamw_host(float *p, const float *g, float *m, float *v, int64_t n,
                            const fsdp_adamw_hparams_t *hp, int64_t step, int32_t n_threads);

/* ---- resharding a checkpoint to another world size --------------------- */

/* [ST] distributed checkpoint paragraph: every rank's Shard(0) chunks are
 * saved with their place in the global tensor; a loading rank reads only the
 * chunks that overlap its new placement, so loading into another world size
 * (2 ranks to 1, N to M) is planning, not conversion.  The reshard plan lists,
 * for target rank rank_dst of world_dst, the overlap of its rows with every
 * source rank's rows under world_src (both torch.chunk layouts), as runs of
 * elements; the executor copies them on the GPU. */
typedef struct fsdp_reshard_plan fsdp_reshard_plan;

typedef struct fsdp_reshard_run_t {
    int32_t param;       /* parameter index                                    */
    int32_t src_rank;    /* source shard the run comes from                    */
    int64_t src_offset;  /* elements from the start of that source shard       */
    int64_t dst_offset;  /* elements from the start of the target shard        */
    int64_t numel;       /* elements in the run (whole rows)                    */
} fsdp_reshard_run_t;

/* Host only.  rows/cols as in fsdp_plan_create.  Runs come in parameter
 * order, then row order, and cover the target shard exactly once.
 * Errors: FSDP_E_INVAL, FSDP_E_NOMEM. */
fsdp_status fsdp_reshard_plan_create(const int64_t *rows, const int64_t *cols, int32_t n_params,
                                     int32_t world_src, int32_t world_dst, int32_t rank_dst,
                                     fsdp_reshard_plan **out);
/* Number of runs and elements of the target shard (all parameters). */
fsdp_status fsdp_reshard_plan_runs(const fsdp_reshard_plan *plan, int64_t *n_runs,
                                   int64_t *dst_numel);
fsdp_status fsdp_reshard_plan_run(const fsdp_reshard_plan *plan, int64_t i,
                                  fsdp_reshard_run_t *out);
/* src: host array of n_params * world_src device pointers, parameter-major
 * (src[p * world_src + s] = source rank s's shard of parameter p, valid
 * elements from offset 0); dst: n_params device pointers to the target
 * shards.  elem_bytes is 2 (bf16) or 4 (fp32); pointers must be aligned to
 * it and non-NULL wherever a run reads or writes.  Builds and uploads the
 * copy table on `stream` (allocating device memory); rebinding replaces it.
 * A rejected call keeps the previous binding; a HIP or allocation failure
 * while the table is replaced leaves the plan unbound.
 * Errors: FSDP_E_INVAL, FSDP_E_UNSUPPORTED, FSDP_E_ALIGN, FSDP_E_NOMEM,
 * FSDP_E_HIP. */
fsdp_status fsdp_reshard_bind(fsdp_reshard_plan *plan, const void *const *src, void *const *dst,
                              int32_t elem_bytes, void *stream);
/* Enqueue the copies (one launch).  Errors: FSDP_E_INVAL, FSDP_E_STATE (not
 * bound, or another device), FSDP_E_HIP. */
fsdp_status fsdp_reshard_execute(const fsdp_reshard_plan *plan, void *stream);
void fsdp_reshard_plan_destroy(fsdp_reshard_plan *plan);

/* Wait for `stream` and report any asynchronous HIP error as FSDP_E_HIP. */
fsdp_status fsdp_check_stream(void *stream);

#ifdef __cplusplus
}
#endif

#endif /* FSDP_SHARD_H */
