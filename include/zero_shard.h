/*
 * zero_shard.h -- C ABI of the ZeRO / FSDP shard-local update for gfx950.
 *
 * What the library computes (page "Infra: Data Parallel", pufanyi.com):
 *   - section "Zero Redundancy Optimizer (ZeRO)": AdamW updates each element
 *     independently, so after a Reduce-Scatter with averaging hands every
 *     rank the mean gradient of its own slice, the rank updates only its
 *     slice of the parameters and of the fp32 optimizer state (master
 *     weights, first and second moments: k = 12 bytes per parameter), and an
 *     All-Gather (ZeRO-1/2) redistributes the updated 16-bit parameters;
 *     under ZeRO-3 the rank keeps its updated shard and gathers nothing.
 *   - section "Naive Data Parallelism": gradients of many parameters travel
 *     together in a bucket; with gradient accumulation (no_sync) the
 *     micro-batch gradients are summed locally, each scaled by 1/n_micro.
 *   - section "Fully Sharded Data Parallel (FSDP)", "FSDP1": parameters are
 *     flattened, concatenated and split evenly over the ranks; a split may
 *     cut a tensor, and a rank may hold none of a tensor.
 *
 * On one GPU, the N_d ranks' gradient contributions are N_d device buffers;
 * the library performs the local arithmetic of the Reduce-Scatter (a sum in
 * fixed rank order, then the division by N_d), the optimizer step and the
 * local write of the All-Gather (the rank's bf16 slice into its slot of the
 * gathered buffer), in one streaming pass over the shard (one kernel launch
 * per call for a bucketed layout with 16-byte aligned buffers; per-parameter
 * layouts take one launch per 143 to 192 tensors, or per 92 when n_d is not
 * one of 2, 4, 8, 16, 32, 64).  No collective is issued.
 *
 * Conventions for every entry point:
 *   - Returns ZERO_OK or a negative zero_status.  Arguments are validated on
 *     the host before anything is launched; on error nothing is launched and
 *     no memory is touched.
 *   - Pointers named *_dev are device pointers; everything else is host.
 *     The caller owns all memory.  The library allocates no device memory.
 *   - Work is enqueued on `stream` (NULL = the null stream) and is
 *     asynchronous; results are visible after the caller synchronises.
 *     A failed launch returns ZERO_EHIP; faults during execution surface at
 *     the caller's next synchronisation.  A HIP error already pending on the
 *     calling thread (hipPeekAtLastError) makes a call return ZERO_EHIP
 *     before it enqueues anything, leaving that error for the caller to read.
 *     A call that enqueues several kernels and sees one of its own launches
 *     fail returns ZERO_EHIP with the earlier launches already enqueued: the
 *     outputs (for a step: master, m, v and the parameters) may then be
 *     partly updated, and repeating the call would apply the update twice to
 *     that part; restore the state before retrying.
 *   - bf16 values are passed as their 16-bit patterns (uint16_t).
 *   - Arithmetic is binary32 with every operation rounded to nearest-even,
 *     no fused multiply-add, subnormals kept, correctly rounded division
 *     and square root.  Results do not depend on the launch configuration.
 *   - Any pointer alignment is accepted; 16-byte aligned buffers take the
 *     vector path, others a scalar path with the same results.
 *   - Entry points may be called from several host threads at once (no
 *     mutable global state apart from a per-device count of compute units);
 *     calls that write the same buffers must be ordered by the caller.
 *   - Every call only enqueues kernels (no allocation, memset, copy or
 *     synchronisation), so a sequence of calls can be captured in a HIP
 *     graph and replayed.
 */
#ifndef ZERO_SHARD_H
#define ZERO_SHARD_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ZERO_OK = 0,
  ZERO_EINVAL = -1,   /* null pointer, negative size, bad enum or flag, non-finite hyper-parameter */
  ZERO_ERANGE = -3,   /* rank, bucket or tensor index out of range; size limit exceeded */
  ZERO_EHIP = -4,     /* a HIP call or kernel launch failed */
  ZERO_EOVERLAP = -5  /* an output buffer overlaps an input or another output */
} zero_status;

/* Largest number of data-parallel ranks a call accepts
 * (zero_shard_step_accumulate: ZERO_MAX_ND_FUSED). */
#define ZERO_MAX_ND 256
#define ZERO_MAX_ND_FUSED 128

/* ------------------------------------------------------------------ layout
 * Bucketed flat layout ("Naive Data Parallelism": buckets; "FSDP1": flatten,
 * concatenate, split evenly; ZeRO figure: GPU i keeps the i-th part).
 *
 * The n_tensors tensors form one flat stream in list order (Psi elements).
 * The stream is cut into buckets of bucket_cap elements (the last one may be
 * shorter; bucket_cap <= 0 puts everything in one bucket), so a tensor may
 * straddle buckets.  Each bucket is zero-padded at its end to a multiple of
 * n_d: padded length P_b, slice length S_b = P_b / n_d.  The padded buckets,
 * concatenated, form the flat buffer of P = sum P_b elements that one rank's
 * gradient bucket / the All-Gather output occupies.  Rank r owns
 * [r*S_b, (r+1)*S_b) of every padded bucket; its shard is these slices in
 * bucket order, S = sum S_b elements, and all per-element state (master, m,
 * v) is stored in shard order.
 *
 * A layout is an immutable host object, a pure function of its arguments.
 */
typedef struct zero_layout zero_layout;

/* numel: host array of n_tensors element counts (>= 0; zero-sized tensors are
 * allowed).  n_d in [1, ZERO_MAX_ND], rank in [0, n_d).  On success *out
 * receives a new layout (free it with zero_layout_destroy).
 * Errors: ZERO_EINVAL (null, n_tensors < 0, numel < 0, n_d out of range),
 * ZERO_ERANGE (rank out of range or Psi overflows int64). */
int zero_layout_create(const int64_t* numel, int32_t n_tensors, int64_t bucket_cap, int32_t n_d,
                       int32_t rank, zero_layout** out);
/* FSDP2 per-parameter layout ("Fully Sharded Data Parallel (FSDP)", "FSDP2":
 * every parameter is split along dim 0 on its own; the local piece keeps the
 * parameter's trailing dimensions; the figure shows three (4, 2) weights over
 * 2 ranks as local (2, 2) pieces, the text an (8, 4) weight over 4 ranks as
 * local (2, 4)).
 *
 * Tensor t has numel[t] elements in rows[t] rows (numel[t] % rows[t] == 0;
 * rows[t] == 0 only for an empty tensor).  With c_t = ceil(rows[t] / n_d),
 * rank r owns rows [r*c_t, (r+1)*c_t) of every tensor; rows past rows[t] are
 * zero padding.  Each tensor is one bucket: padded length n_d*c_t*row_numel,
 * slice c_t*row_numel; the shard is the slices in tensor order and the
 * flat (All-Gather) buffer holds every tensor padded to n_d*c_t rows.  All
 * bucket and tensor queries below apply (bucket b is tensor b).
 * Errors: ZERO_EINVAL (null, n_d out of range, a row count that does not
 * divide numel), ZERO_ERANGE (rank out of range, Psi overflow). */
int zero_layout_create_dim0(const int64_t* numel, const int64_t* rows, int32_t n_tensors,
                            int32_t n_d, int32_t rank, zero_layout** out);

/* 0 for the bucketed flat layout, 1 for the per-parameter (dim-0) layout,
 * -1 for a null layout. */
int32_t zero_layout_kind(const zero_layout* layout);

void zero_layout_destroy(zero_layout* layout);

/* Sizes: Psi (sum of numel), P (padded flat length), S (shard length),
 * number of buckets, n_d, rank.  Return -1 for a null layout. */
int64_t zero_layout_psi(const zero_layout* layout);
int64_t zero_layout_padded(const zero_layout* layout);
int64_t zero_layout_shard(const zero_layout* layout);
int64_t zero_layout_n_buckets(const zero_layout* layout);
int32_t zero_layout_n_d(const zero_layout* layout);
int32_t zero_layout_rank(const zero_layout* layout);

/* Bucket b: stream offset and real length, offset and padded length in the
 * flat buffer, offset of its slice in the shard.  Null outputs are skipped.
 * Errors: ZERO_EINVAL (null layout), ZERO_ERANGE (b out of range). */
int zero_layout_bucket(const zero_layout* layout, int64_t b, int64_t* stream_off, int64_t* len,
                       int64_t* padded_off, int64_t* padded_len, int64_t* shard_off);

/* Tensor t: its stream offset, and the smallest shard range [lo, hi) holding
 * every element of t that this rank owns (lo == hi: the rank holds none of
 * it, the empty view of FSDP1's use_orig_params).  Inside the range there
 * are no elements of other tensors; bucket padding may occur when t runs past
 * the end of a padded bucket.  Errors as for zero_layout_bucket. */
int zero_layout_tensor(const zero_layout* layout, int32_t t, int64_t* stream_off,
                       int64_t* shard_lo, int64_t* shard_hi);

/* Tensor t in the padded flat buffer (a rank's gradient bucket buffer, the
 * All-Gather output): flat_lo is the flat offset of its first element and
 * flat_hi one past that of its last, so a tensor that lies in one bucket
 * occupies exactly [flat_lo, flat_hi); one that straddles buckets has the
 * padding of every bucket it crosses inside that range ("FSDP1": the
 * flattened parameters are concatenated and each bucket is padded at its
 * end).  For the per-parameter layout the range opens the tensor's padded
 * slot of n_d*c_t rows.  An empty tensor gets flat_lo == flat_hi, the
 * position where it would start.  Null outputs are skipped.  Errors as for
 * zero_layout_bucket. */
int zero_layout_tensor_flat(const zero_layout* layout, int32_t t, int64_t* flat_lo,
                            int64_t* flat_hi);

/* ------------------------------------------------------------- bucket pack
 * ("Naive Data Parallelism": a bucket carries the gradients of several
 * parameters; "FSDP1": flatten + concatenate.)
 *
 * For every bucket b in [bucket_begin, bucket_end): copy the bf16 gradient
 * elements of the stream range of b out of the per-tensor buffers into
 * flat_out_dev[padded_off_b ...] and write +0 into the bucket's padding.
 * Elements of flat_out_dev outside these buckets are not touched.
 *
 * tensor_grads_dev: HOST array of n_tensors DEVICE pointers, tensor t holding
 * numel[t] contiguous bf16 values; entries of tensors with no element in the
 * bucket range may be NULL.  flat_out_dev: P elements.  Sources must not
 * overlap flat_out_dev.
 * Errors: ZERO_EINVAL, ZERO_ERANGE (bucket range), ZERO_EOVERLAP, ZERO_EHIP. */
int zero_bucket_pack(const zero_layout* layout, const uint16_t* const* tensor_grads_dev,
                     int64_t bucket_begin, int64_t bucket_end, uint16_t* flat_out_dev,
                     hipStream_t stream);

/* ----------------------------------------------------- no_sync accumulation
 * ("Naive Data Parallelism": accumulate micro-batch gradients locally; with
 * n equal micro-batches of sample-mean losses divide each by n.)
 *
 * For i in [0, n):  a = (flags & ZERO_ACC_OVERWRITE) ? scale*g[i]
 *                                                    : acc[i] + scale*g[i]
 * (product and sum each rounded once); then, unless ZERO_ACC_NO_STORE,
 * acc[i] = a; if ZERO_ACC_EMIT_BF16, bf16_out[i] = bf16(a) (round to nearest
 * even).  scale is typically 1/n_micro.
 *
 * acc_dev: n floats (may be NULL only with OVERWRITE|NO_STORE);
 * grad_dev: n bf16; bf16_out_dev: n bf16, required iff EMIT_BF16, and must
 * not overlap grad_dev or acc_dev.  grad_dev must not overlap acc_dev.
 * NO_STORE requires EMIT_BF16.  Errors: ZERO_EINVAL, ZERO_EOVERLAP, ZERO_EHIP. */
#define ZERO_ACC_OVERWRITE 1u
#define ZERO_ACC_EMIT_BF16 2u
#define ZERO_ACC_NO_STORE 4u
int zero_grad_accumulate(float* acc_dev, const uint16_t* grad_dev, int64_t n, float scale,
                         uint32_t flags, uint16_t* bf16_out_dev, hipStream_t stream);

/* ---------------------------------------------------------- shard step
 * ("Zero Redundancy Optimizer (ZeRO)": Reduce-Scatter with averaging, the
 * element-wise AdamW update of the owned slice, All-Gather of the updated
 * parameters, or for ZeRO-3 keeping the updated shard in place.)
 *
 * For every shard index i of this rank, in binary32:
 *   a  = bf16->f32(G_0[i]);  a = a + bf16->f32(G_q[i])  for q = 1..n_d-1
 *   g  = a / n_d
 *   m' = B1*m + C1*g ;  v' = B2*v + C2*(g*g)
 *   d  = sqrt(v')*rho + E ;  th' = a_wd*th - s*(m'/d) ;  p = bf16(th')
 * with per-call scalars computed in binary64 and rounded once to binary32:
 *   s = lr/(1-beta1^t), rho = 1/sqrt(1-beta2^t), a_wd = 1 - lr*weight_decay,
 *   B1 = beta1, C1 = 1-beta1, B2 = beta2, C2 = 1-beta2, E = eps
 * (AdamW with decoupled weight decay, bias correction, eps outside the root.)
 *
 * t: 1-based index of this step (>= 1).
 * rank_grads_dev: HOST array of n_d DEVICE pointers to bf16 contributions:
 *   ZERO_GRAD_COMPACT: each holds S values in shard order (the rank's slice
 *                      as a Reduce-Scatter would deliver it);
 *   ZERO_GRAD_FLAT:    each is a whole padded flat buffer of P values (a
 *                      rank's gradient bucket buffer); slice r is read.
 * master_dev, exp_avg_dev, exp_avg_sq_dev: S floats each, updated in place.
 * param_out_dev: ZERO_OUT_AG_SLOT: the P-element All-Gather buffer; only
 *                      this rank's slice of each bucket is written;
 *                ZERO_OUT_SHARD:   the S-element bf16 shard, overwritten in
 *                      place (ZeRO-3).
 * reduced_grad_out_dev: NULL, or S floats receiving g (for verification).
 * Outputs must not overlap each other or any input (ZERO_EOVERLAP).
 * Errors: ZERO_EINVAL (null pointer, bad enum, t < 1, hyper-parameters not
 * finite or betas outside [0, 1)), ZERO_EOVERLAP, ZERO_EHIP. */
typedef struct {
  double lr, beta1, beta2, eps, weight_decay;
} zero_adamw;

#define ZERO_GRAD_COMPACT 0
#define ZERO_GRAD_FLAT 1
#define ZERO_OUT_AG_SLOT 0
#define ZERO_OUT_SHARD 1

int zero_shard_step(const zero_layout* layout, const zero_adamw* hp, int64_t t,
                    const uint16_t* const* rank_grads_dev, int32_t grad_layout, float* master_dev,
                    float* exp_avg_dev, float* exp_avg_sq_dev, uint16_t* param_out_dev,
                    int32_t out_mode, float* reduced_grad_out_dev, hipStream_t stream);

/* Same as zero_shard_step with options: the contributions' element type and
 * the launch shape.
 *
 * grad_dtype ZERO_DTYPE_BF16: rank_grads_dev[q] points to bf16 values, as in
 *   zero_shard_step.
 * grad_dtype ZERO_DTYPE_F32: rank_grads_dev[q] points to binary32 values (a
 *   Reduce-Scatter carried out in fp32, e.g. the ranks' no_sync fp32
 *   accumulators handed over without rounding to bf16); the reduction is
 *   a = G_0; a = a + G_q for q = 1..n_d-1, then the same update.  Reads
 *   4*n_d + 26 bytes per shard element instead of 2*n_d + 26.
 * blocks <= 0 and threads <= 0 pick the defaults; threads must be a multiple
 * of 64 and at most 256; path 0 = automatic, 1 = force element-by-element
 * (scalar) processing.
 * opt == NULL means {ZERO_DTYPE_BF16, 0, 0, 0}.  Results do not depend on
 * blocks, threads or path.  Errors as for zero_shard_step, plus ZERO_EINVAL
 * for a bad dtype or launch shape. */
#define ZERO_DTYPE_BF16 0
#define ZERO_DTYPE_F32 1

typedef struct {
  int32_t grad_dtype;
  int32_t blocks;
  int32_t threads;
  int32_t path;
} zero_step_options;

int zero_shard_step_ex(const zero_layout* layout, const zero_adamw* hp, int64_t t,
                       const void* const* rank_grads_dev, int32_t grad_layout,
                       float* master_dev, float* exp_avg_dev, float* exp_avg_sq_dev,
                       uint16_t* param_out_dev, int32_t out_mode, float* reduced_grad_out_dev,
                       const zero_step_options* opt, hipStream_t stream);

/* The last no_sync micro-batch folded into the step ("Naive Data
 * Parallelism": micro-batch gradients are accumulated locally, each scaled by
 * 1/n_micro, and the sum is what a rank contributes to the reduction).
 *
 * Rank q's contribution is computed inside the step instead of by a separate
 * accumulate call:
 *   c_q = acc_q[i] + micro_scale * bf16->f32(micro_q[i])
 *   (product and sum rounded once each, as zero_grad_accumulate's add), then
 *   contrib_dtype ZERO_DTYPE_BF16: G_q = bf16(c_q) (round to nearest even),
 *     what the rank would hand to a bf16 Reduce-Scatter: the result equals
 *     zero_grad_accumulate(acc_q, micro_q, n, micro_scale,
 *     ZERO_ACC_EMIT_BF16 | ZERO_ACC_NO_STORE, tmp_q) for every q followed by
 *     zero_shard_step on the tmp_q, bit for bit;
 *   contrib_dtype ZERO_DTYPE_F32: G_q = c_q, equal to accumulating into acc_q
 *     and calling zero_shard_step_ex with ZERO_DTYPE_F32 on the acc_q.
 * The reduction and update are those of zero_shard_step.  The accumulators
 * are read, not written (no_sync restarts them at the next step).  Moves
 * 6*n_d + 26 bytes per shard element, against 10*n_d + 26 for the separate
 * accumulate call and step (bf16 contributions).
 *
 * rank_acc_dev: HOST array of n_d DEVICE pointers to binary32 accumulators,
 * rank_micro_dev: HOST array of n_d DEVICE pointers to the bf16 gradients of
 * the last micro-batch, both in the grad_layout's shape (COMPACT: S values
 * in shard order; FLAT: whole padded flat buffers of P values).  The other
 * arguments are those of zero_shard_step_ex; opt->grad_dtype is ignored
 * (opt may be NULL).  n_d must be at most ZERO_MAX_ND_FUSED (ZERO_ERANGE).
 * Errors: as for zero_shard_step_ex, plus ZERO_EINVAL for a bad
 * contrib_dtype or a non-finite micro_scale. */
int zero_shard_step_accumulate(const zero_layout* layout, const zero_adamw* hp, int64_t t,
                               const float* const* rank_acc_dev,
                               const uint16_t* const* rank_micro_dev, float micro_scale,
                               int32_t contrib_dtype, int32_t grad_layout, float* master_dev,
                               float* exp_avg_dev, float* exp_avg_sq_dev,
                               uint16_t* param_out_dev, int32_t out_mode,
                               float* reduced_grad_out_dev, const zero_step_options* opt,
                               hipStream_t stream);

/* zero_shard_step_ex restricted to buckets [bucket_begin, bucket_end) of the
 * layout ("Zero Redundancy Optimizer (ZeRO)", ZeRO-2: gradients are reduced
 * bucket by bucket as they become ready).  The update of an element reads
 * only that element's contributions and state, so a caller may step each
 * bucket's slice as soon as its reduction has landed; stepping every bucket
 * once, in any grouping and order, gives the same bits as one
 * zero_shard_step_ex call.
 *
 * Calls on disjoint bucket ranges touch disjoint memory, so they may also
 * run concurrently on different streams.  Consecutive kernels of one stream
 * do not overlap, so one call per bucket pays each launch's ramp-up and
 * drain in turn: measured on MI355X for the Llama-3-8B shard (613 calls of
 * one 25 MiB bucket), 59 % of the HBM peak on one stream against 75 %
 * with the calls alternating between two streams (79-80 % for the whole
 * shard in one call or in calls of 32 buckets).
 *
 * All buffers are the full-size ones of zero_shard_step_ex (contributions of
 * S or P values, S-element state, S- or P-element output); only the slices
 * of the named buckets are read and written.  For a dim-0 layout a bucket is
 * a tensor.  bucket_begin == bucket_end is a no-op.
 * Errors: as for zero_shard_step_ex, plus ZERO_ERANGE when
 * 0 <= bucket_begin <= bucket_end <= n_buckets does not hold. */
int zero_shard_step_buckets(const zero_layout* layout, const zero_adamw* hp, int64_t t,
                            int64_t bucket_begin, int64_t bucket_end,
                            const void* const* rank_grads_dev, int32_t grad_layout,
                            float* master_dev, float* exp_avg_dev, float* exp_avg_sq_dev,
                            uint16_t* param_out_dev, int32_t out_mode,
                            float* reduced_grad_out_dev, const zero_step_options* opt,
                            hipStream_t stream);

/* --------------------------------------------------------- parameter gather
 * ("Zero Redundancy Optimizer (ZeRO)": ZeRO-1/2 All-Gather the updated
 * parameters after the step; ZeRO-3 All-Gathers each layer's parameters
 * before forward and again before backward.)
 *
 * The local arithmetic of that All-Gather: for every bucket b in
 * [bucket_begin, bucket_end) and every rank q, copy rank q's slice of b
 * (S_b bf16 values at shard offset shard_off_b of rank_shards_dev[q]) to
 * full_out_dev[padded_off_b + q*S_b ...].  Padding is copied as it is held
 * by the shards (+0 when the shards were produced by zero_shard_step from
 * zero-initialised padding).  Elements of full_out_dev outside the bucket
 * range are not touched.
 *
 * rank_shards_dev: HOST array of n_d DEVICE pointers, each S bf16 values
 * (a rank's shard in shard order, as zero_shard_step's ZERO_OUT_SHARD
 * output).  full_out_dev: P bf16 values; must not overlap any shard.
 * Moves 4 bytes per flat element.
 * Errors: ZERO_EINVAL, ZERO_ERANGE (bucket range), ZERO_EOVERLAP, ZERO_EHIP. */
int zero_gather_params(const zero_layout* layout, const uint16_t* const* rank_shards_dev,
                       int64_t bucket_begin, int64_t bucket_end, uint16_t* full_out_dev,
                       hipStream_t stream);

/* ----------------------------------------------------------------- reshard
 * ("Fully Sharded Data Parallel (FSDP)", "Checkpoint": every rank saves its
 * own shards; loading re-cuts them for the target layout, including a
 * different number of GPUs; optimizer state has to be saved and re-cut too.)
 *
 * Re-cut one per-element array (fp32 master / m / v, or bf16 parameters)
 * from the n_d shards of layout `src` into the shard of layout `dst` (its
 * own n_d' and rank): dst_shard_dev[i] = value of the parameter at stream
 * position x(i) taken from the src shard that owns x(i); dst padding is
 * written as 0.  Both layouts must describe the same tensor list (equal
 * numel arrays); bucket capacity, n_d and rank may differ.
 *
 * src_shards_dev: HOST array of src's n_d DEVICE pointers, each src S values.
 * dst_shard_dev: dst S values; must not overlap any source.
 * elem_bytes: 4 (fp32 state) or 2 (bf16).  Moves 2*elem_bytes bytes per
 * destination element.
 * Errors: ZERO_EINVAL (null, bad elem_bytes, different tensor lists),
 * ZERO_EOVERLAP, ZERO_EHIP. */
int zero_reshard(const zero_layout* src, const void* const* src_shards_dev,
                 const zero_layout* dst, void* dst_shard_dev, int32_t elem_bytes,
                 hipStream_t stream);

/* -------------------------------------------------------------- placement
 * Host-only planner for placing the step's buffers inside ONE device
 * allocation that the caller makes (the library allocates nothing).
 *
 * Why: every call streams all its buffers once, so its speed is set by how
 * HBM serves the concurrent streams.  Measured on MI355X (288 GB HBM3E), the
 * same buffers run up to ~15 % faster or slower depending on their position
 * in memory (a pattern with a 96 GiB period); buffers spread round-robin over
 * three lanes 32 GiB apart, each lane carrying a third of the traffic per
 * element, ran at the fast end at every shift tried.  The results of every
 * entry point are the same for any placement.
 *
 * Buffer k has nbytes[k] bytes and moves traffic[k] bytes of HBM traffic per
 * shard element (e.g. 2 for a bf16 contribution, 8 for an fp32 state array
 * that is read and written, 2 for the bf16 output).  Buffers are assigned to
 * n_lanes classes so that the classes carry equal traffic (heaviest first,
 * each to the least loaded class, ties to the lower class); class c then
 * packs its buffers, in list order and each aligned to `align`, into lane
 * slots at offsets (c + j*n_lanes) * lane_bytes, j = 0, 1, ...  A buffer
 * larger than lane_bytes is placed after all others.  offsets_out[k]
 * receives buffer k's byte offset in the pool, *pool_bytes_out the pool
 * size to allocate.  No two buffers overlap.
 *
 * Suggested values on MI355X: lane_bytes = 32 GiB, n_lanes = 3,
 * align = 2 MiB.  nbytes/traffic/offsets_out: host arrays of n entries.
 * Errors: ZERO_EINVAL (null pointer with n > 0, negative size, traffic not
 * finite or negative, n_lanes outside [1, 64], align not a power of two of
 * at least 16, lane_bytes not a positive multiple of align), ZERO_ERANGE
 * (sizes beyond 2^62 bytes). */
int zero_placement_plan(int32_t n, const int64_t* nbytes, const double* traffic,
                        int64_t lane_bytes, int32_t n_lanes, int64_t align,
                        int64_t* offsets_out, int64_t* pool_bytes_out);

/* Per-call binary32 scalars for step t, in the order
 * {s, rho, a_wd, B1, C1, B2, C2, E}.  Errors: ZERO_EINVAL. */
int zero_step_scalars(const zero_adamw* hp, int64_t t, float out[8]);

/* Static description of a status code. */
const char* zero_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* ZERO_SHARD_H */
