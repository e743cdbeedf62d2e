/*
 * zero.h -- C ABI of libzero_mi355x.so: one data-parallel rank's share of a
 * ZeRO/FSDP mixed-precision training step on an AMD Instinct MI355X (gfx950).
 *
 * The step, as the pages describe it (no collective is run here):
 *   zero_layout         map a per-tensor size list to flat shard offsets;
 *   zero_pack_grads     gather the rank's 1/N_d slice of the bf16 gradients
 *                       into one contiguous shard buffer;
 *   zero_shard_sqnorm   sum of squares of that shard (the rank's share of
 *                       the global gradient norm);
 *   zero_adamw_step     clip with the global norm, AdamW on fp32 master/m/v,
 *                       cast the new master to the bf16 parameter shard
 *                       (the state in the library's tiled buffer;
 *                       zero_adamw_step_arrays takes three separate arrays);
 *   zero_unpack_params  scatter the bf16 parameter shard back into the
 *                       per-tensor parameters.
 *
 * Conventions for every call:
 *   - bf16 values travel as raw uint16_t bit patterns; fp32 state as float.
 *   - Sizes and element offsets are int64_t; shards may exceed 2^32 elements.
 *   - Device pointers are caller-owned device memory (for example torch
 *     allocations); the library never frees them. Host pointers are read
 *     during the call only.
 *   - Device calls enqueue work on the given stream (NULL = the default
 *     stream) and return without synchronising; results are ready when the
 *     stream reaches them.
 *   - Return value: ZERO_OK or a negative error code; zero_last_error()
 *     gives a message for the calling thread. Argument errors are detected on
 *     the host before anything is enqueued.
 */
#ifndef ZERO_MI355X_H
#define ZERO_MI355X_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ZERO_OK 0
#define ZERO_EINVAL (-1)  /* bad argument: null pointer, bad size or range */
#define ZERO_EHIP (-3)    /* a HIP launch or runtime call failed */
#define ZERO_ENOMEM (-4)  /* host allocation failed */

/* Opaque, immutable description of one rank's shard (host memory only). */
typedef struct zero_layout_s* zero_layout_t;

/* Tensor elements [src_off, src_off+len) of tensor `tensor` occupy shard
 * elements [dst_off, dst_off+len). */
typedef struct {
  int64_t tensor;
  int64_t src_off;
  int64_t dst_off;
  int64_t len;
} zero_segment;

/* Facts about a layout. Byte and communication figures are per rank.
 * bytes_stage[s] is ZeRO stage s's model-state bytes on the generated layout:
 *   s=0: 16*psi;  s=1: 4*psi + 12*shard;  s=2: 2*psi + 14*shard;  s=3: 16*shard
 * bytes_stage_fp32acc[s] adds an fp32 gradient-accumulation buffer: 4*psi for
 * s<=1 (gradients replicated), 4*shard for s>=2 (gradients partitioned).
 * comm_pages[s] is the pages' per-step approximation in values (2*psi for
 * stages 0-2, 3*psi for stage 3); comm_exact[s] counts what a ring
 * reduce-scatter / all-gather sends: (n_d-1)*shard per pass, two passes for
 * stages 0-2 and three for stage 3.
 * Sources: "第 5 课：ZeRO 与 FSDP" sections 2-3; notes on the ZeRO paper,
 * sections 2.1, 4.1-4.3 and 6. */
typedef struct {
  int64_t n_tensors;
  int64_t n_d;
  int64_t rank;
  int64_t align;
  int64_t psi;          /* real parameters: sum of the sizes */
  int64_t padded;       /* P = ceil(psi / (n_d*align)) * n_d*align */
  int64_t shard;        /* S = P / n_d, elements every rank owns */
  int64_t shard_begin;  /* rank*S: first flat element of this shard */
  int64_t n_segments;
  int64_t pad_begin;    /* shard elements [pad_begin, pad_end) are padding */
  int64_t pad_end;      /* (empty when equal) */
  int64_t bytes_stage[4];
  int64_t bytes_stage_fp32acc[4];
  int64_t comm_pages[4];
  int64_t comm_exact[4];
} zero_layout_info;

/* AdamW hyperparameters. `step` is the 1-based step count used for the bias
 * corrections 1-beta1^step and 1-beta2^step (computed on the host in fp64).
 * max_norm <= 0 turns clipping off (NaN is refused); otherwise the gradient
 * is scaled by c = max_norm / (sqrt(G) + clip_eps) when that is below 1, G
 * being the global sum of squares. */
typedef struct {
  double lr;
  double beta1;
  double beta2;
  double eps;
  double weight_decay;
  double max_norm;
  double clip_eps;
  int64_t step;
} zero_adamw_hparams;

/* ---------------------------------------------------------------------------
 * zero_layout -- the partitioner (host only, no device memory).
 * Flattens the tensors in list order (notes on the ZeRO paper, sections 2.2
 * and 5.2: tensors fused into one contiguous buffer), pads the tail so the
 * buffer splits into n_d equal shards whose starts are multiples of
 * `align_elems`, and records which runs of which tensors rank `rank` owns
 * ("第 5 课：ZeRO 与 FSDP" section 2 and notes section 4.1: each rank keeps
 * 1/N_d of the state). A shard boundary may cut through a tensor.
 *   sizes       host array of n_tensors element counts (>= 0; zero-size
 *               tensors get no segment)
 *   n_d         data-parallel degree (>= 1); rank in [0, n_d)
 *   align_elems shard alignment in elements (>= 1; 128 keeps every shard
 *               start 256-byte aligned for bf16 and 512-byte for fp32)
 *   out         receives a handle to free with zero_layout_free
 * Errors: ZERO_EINVAL for a null pointer, n_tensors < 1, a negative size, a
 * total of 0, n_d < 1, rank outside [0, n_d), align_elems < 1 or an int64
 * overflow; ZERO_ENOMEM if the host allocation fails. */
int zero_layout(const int64_t* sizes, int32_t n_tensors, int32_t n_d, int32_t rank,
                int64_t align_elems, zero_layout_t* out);

/* Copy the layout's facts into *info. ZERO_EINVAL on null arguments. */
int zero_layout_query(zero_layout_t h, zero_layout_info* info);

/* Copy up to `cap` segments, in shard order, into `segs` (host) and store the
 * total count in *n_out. segs may be NULL when cap is 0. ZERO_EINVAL on a null
 * handle or n_out, or cap < 0. */
int zero_layout_segments(zero_layout_t h, zero_segment* segs, int64_t cap, int64_t* n_out);

/* Release a handle (NULL is ignored). */
void zero_layout_free(zero_layout_t h);

/* ---------------------------------------------------------------------------
 * zero_pack_grads -- flatten the rank's gradient slice.
 * Fills grad_shard[begin, begin+count) (shard coordinates) with the bf16
 * gradient elements the layout assigns there and writes 0 to padding (notes
 * on the ZeRO paper, sections 2.2 and 3.2.3: tensors are copied into a
 * pre-allocated contiguous buffer; section 4.2: the rank keeps its own 1/N_d
 * gradient slice). A pure bit copy.
 *   tensor_grads host array of n_tensors DEVICE pointers, entry i = tensor i's
 *                full gradient (sizes[i] elements, contiguous). Entries of
 *                tensors with no element in the range may be NULL.
 *   grad_shard   device pointer to the shard's element 0 (S bf16 values)
 * Reads only the segments' elements; writes only the range. Source and
 * destination must not overlap.
 * Errors: ZERO_EINVAL for a null handle/array/shard, a NULL pointer of a tensor
 * the range touches, begin < 0, count < 0 or begin+count > S; ZERO_EHIP if a
 * launch fails. count == 0 enqueues nothing. */
int zero_pack_grads(zero_layout_t h, const uint16_t* const* tensor_grads, uint16_t* grad_shard,
                    int64_t begin, int64_t count, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * zero_pack_grads_sqnorm -- zero_pack_grads and the sum of squares of the
 * packed range in one pass: the gradient norm is taken over the values as
 * they are flattened into the fused buffer (notes on the ZeRO paper, sections
 * 2.2 and 5.2: flattening feeds the gradient-norm computation), so the shard
 * is not read a second time. Writes grad_shard[begin, begin+count) exactly as
 * zero_pack_grads does, and *d_out = sum of g*g over that range (or
 * *d_out += it when accumulate != 0), each square exact in fp64, summed in
 * fp64 in an order fixed by the layout, the range and the pointers' alignment
 * (equal inputs give bit-identical results; the order differs from
 * zero_shard_sqnorm's, so the two may differ in the last bits).
 *   d_out        device pointer to one double
 *   d_workspace  device scratch of at least zero_pack_sqnorm_workspace_bytes(h,
 *                begin, count) bytes, 8-byte aligned; contents on entry do not
 *                matter
 * Errors: as zero_pack_grads, plus ZERO_EINVAL for a NULL output or workspace,
 * or a workspace that is too small. count == 0 writes 0 (or leaves *d_out
 * unchanged when accumulating). zero_pack_sqnorm_workspace_bytes returns 0
 * for a NULL handle or a range outside the shard. */
size_t zero_pack_sqnorm_workspace_bytes(zero_layout_t h, int64_t begin, int64_t count);
int zero_pack_grads_sqnorm(zero_layout_t h, const uint16_t* const* tensor_grads, uint16_t* grad_shard,
                           int64_t begin, int64_t count, double* d_out, int32_t accumulate,
                           void* d_workspace, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * zero_pack_grads_sqnorm_noalloc -- zero_pack_grads_sqnorm without a
 * workspace, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation).
 * The block partial sums go to a static device array that the library holds
 * on every GPU it runs on: ZERO_NOALLOC_PARTIALS doubles (2 MiB) per GPU,
 * kept until the process ends. The call allocates nothing (device or host)
 * and uses the same kernels in the same order as zero_pack_grads_sqnorm, so
 * its results are bit-identical to that call's.
 * Arguments, results and errors as zero_pack_grads_sqnorm, without the
 * workspace. Limit: the range may need at most ZERO_NOALLOC_PARTIALS partial
 * sums, i.e. zero_pack_sqnorm_workspace_bytes(h, begin, count) <=
 * 8 * ZERO_NOALLOC_PARTIALS (a range in one piece of up to 2,147,475,456
 * elements); a larger range is refused with ZERO_EINVAL before anything is
 * enqueued. Every call on a GPU shares that GPU's array and overwrites what
 * the previous call left (each call writes every partial it reads, so nothing
 * needs clearing): calls whose execution overlaps on one GPU (on different
 * streams, or from different host threads without ordering) race and give
 * wrong sums. ZERO_EHIP also reports a failed hipGetDevice or
 * hipGetSymbolAddress (the array's address on the current device, looked up
 * on the first call for each device). */
#define ZERO_NOALLOC_PARTIALS (1 << 18)
int zero_pack_grads_sqnorm_noalloc(zero_layout_t h, const uint16_t* const* tensor_grads, uint16_t* grad_shard,
                                   int64_t begin, int64_t count, double* d_out, int32_t accumulate,
                                   hipStream_t stream);

/* ---------------------------------------------------------------------------
 * zero_shard_sqnorm -- the rank's part of the global gradient norm.
 * *d_out = sum of g*g over the count bf16 values at d_grad (or *d_out += that
 * sum when accumulate != 0), each square exact in fp64 and the sum carried in
 * fp64. The order of additions depends only on count and on the address of
 * d_grad modulo 16, so equal inputs give bit-identical results. Gradient
 * clipping must use the norm over all ranks' slices ("ZeRO-3 核心流程",
 * pitfall 1); callers add the ranks' partial sums (an all-reduce across ranks,
 * not done here) and hand the per-rank values to zero_adamw_step.
 *   d_grad      device pointer, count bf16 values
 *   d_out       device pointer to one double
 *   d_workspace device scratch of at least zero_sqnorm_workspace_bytes(count)
 *               bytes, 8-byte aligned; contents on entry do not matter
 * Errors: ZERO_EINVAL for null pointers (d_grad may be NULL when count == 0),
 * count < 0 or a workspace that is too small; ZERO_EHIP if a launch fails.
 * count == 0 writes 0 (or leaves *d_out unchanged when accumulating). */
size_t zero_sqnorm_workspace_bytes(int64_t count);
int zero_shard_sqnorm(const uint16_t* d_grad, int64_t count, double* d_out, int32_t accumulate,
                      void* d_workspace, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * zero_sum_partials -- the combine of a bucketed sum of squares: *d_out = the
 * sum of the n doubles at d_partials (or *d_out += it when accumulate != 0),
 * in an order that depends only on n, so equal inputs give bit-identical
 * results whatever order or streams produced the partials. A shard processed
 * in constant-size buckets (notes on the ZeRO paper, section 5.2, constant
 * buffer size; "ZeRO-3 核心流程", the prefetch bucket) can write each bucket's
 * sum of squares to its own slot, on any stream, and combine the slots once
 * every bucket is done.
 *   d_partials  device array of n doubles
 *   d_out       device pointer to one double (not inside d_partials)
 * Errors: ZERO_EINVAL for n < 0, a NULL d_out, a NULL d_partials with n > 0,
 * or a pointer that is not 8-byte aligned; ZERO_EHIP if the launch fails. n == 0 writes 0 (or leaves *d_out
 * unchanged when accumulating). */
int zero_sum_partials(const double* d_partials, int64_t n, double* d_out, int32_t accumulate, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * zero_pack_grads_sqnorm_partials, zero_sum_partials_rows -- the bucketed
 * form of zero_pack_grads_sqnorm, with one final stage for all buckets. A
 * shard processed in constant-size buckets (notes on the ZeRO paper, section
 * 5.2, constant buffer size; "ZeRO-3 核心流程", the prefetch bucket) packs
 * each bucket on any stream, leaving its block partial sums in its own slice
 * of one buffer; once every bucket is done, one launch reduces each slice, and
 * zero_sum_partials combines the buckets' sums.
 *
 * zero_pack_grads_sqnorm_partials packs [begin, begin+count) exactly as
 * zero_pack_grads does and writes the sum of squares of each of its blocks to
 * d_partials[0 .. *n_partials) (device, 8-byte aligned; *n_partials is a HOST
 * int64, set before the call returns). cap_bytes, the room at d_partials, must
 * be at least zero_pack_sqnorm_workspace_bytes(h, begin, count); the count
 * depends on the layout, the range and the pointers' alignment only.
 * zero_pack_grads_sqnorm over the same range computes the same partials and
 * adds them as zero_sum_partials_rows does a row of that length, so the
 * results are bit-identical.
 * Errors: as zero_pack_grads_sqnorm, with cap_bytes for the workspace size
 * and ZERO_EINVAL for a NULL n_partials.
 *
 * zero_sum_partials_rows: for r in [0, n_rows), d_out[r] = the sum of the
 * row_len[r] doubles at d_partials + row_begin[r] (or d_out[r] += it when
 * accumulate != 0), each row in the order zero_sum_partials adds that many
 * values (bit-identical to it). row_begin, row_len: HOST arrays of n_rows
 * int64 (element offsets and counts, >= 0); d_out: device array of n_rows
 * doubles, not overlapping the rows. One launch per 192 rows.
 * Errors: ZERO_EINVAL for n_rows < 0, NULL arguments (allowed when n_rows ==
 * 0), pointers not 8-byte aligned or a negative start or length; ZERO_EHIP if
 * a launch fails. */
int zero_pack_grads_sqnorm_partials(zero_layout_t h, const uint16_t* const* tensor_grads, uint16_t* grad_shard,
                                    int64_t begin, int64_t count, double* d_partials, size_t cap_bytes,
                                    int64_t* n_partials, hipStream_t stream);
int zero_sum_partials_rows(const double* d_partials, const int64_t* row_begin, const int64_t* row_len,
                           int64_t n_rows, double* d_out, int32_t accumulate, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Layout of the fp32 optimizer state (12 bytes per element: master, m, v).
 * The state of an n-element shard is ONE buffer of 3*n floats in tiles of
 * ZERO_STATE_TILE elements. Tile k covers elements [k*T, k*T + L_k) with
 * L_k = min(T, n - k*T) and stores master[L_k], then m[L_k], then v[L_k];
 * element e (tile k = e / T, j = e % T) has master at 3*k*T + j, m at
 * 3*k*T + L_k + j and v at 3*k*T + 2*L_k + j. Only the last tile can be
 * shorter. Keeping the three values of a stretch of elements within one tile
 * lets the update stream HBM at ~80% of peak on MI355X, where three separate
 * arrays reach ~70%. zero_state_import/export convert from/to three separate
 * arrays. */
#define ZERO_STATE_TILE 8192

/* Launch granularity of the device calls. A call's work is split into
 * several kernel launches, one after another on the caller's stream, when
 * its range touches more than ZERO_PIECES_PER_LAUNCH contiguous tensor pieces
 * (pack, unpack, the fused update), or, for the updates, when the range is
 * longer than ZERO_ADAMW_LAUNCH_ELEMS elements (then equal launches of whole
 * tiles). Results do not depend on the split. */
#define ZERO_PIECES_PER_LAUNCH 64
#define ZERO_ADAMW_LAUNCH_ELEMS (1 << 27)

/* ---------------------------------------------------------------------------
 * zero_adamw_step -- fused clip + AdamW + bf16 cast over shard elements
 * [begin, begin+count).
 * The rank updates only its own 1/N_d slice of the fp32 master weights and
 * optimizer state and converts the result to bf16 ("第 5 课：ZeRO 与 FSDP"
 * section 3; notes on the ZeRO paper, section 4.1), K = 12 bytes of fp32
 * state per parameter (section 2 of the lesson; notes section 2.1).
 * Per element, with g the bf16 gradient widened to fp32:
 *   c  = clip coefficient max_norm / (sqrt(G) + clip_eps), capped at 1, in
 *        fp64, from G = d_rank_sqnorms[0] + ... + d_rank_sqnorms[n_ranks-1]
 *        in fp64, in a fixed order: for at most 64 ranks, rank order; beyond,
 *        64 lane sums (lane l adds ranks l, l+64, l+128, ... in order), then
 *        the lane sums in lane order
 *   g' = c*g;  m = beta1*m + (1-beta1)*g';  v = beta2*v + (1-beta2)*g'^2
 *   master = master*(1 - lr*wd) - (lr/(1-beta1^t)) * m / (sqrt(v)/sqrt(1-beta2^t) + eps)
 *   param  = bf16 round-to-nearest-even of the new fp32 master
 * Arithmetic is fp32 (c rounded to fp32) with correctly rounded division and
 * square root, except where the new master comes out below 2^-12 of the
 * magnitudes it is formed from (cancellation; ~2e-5 of the elements): such
 * an element is recomputed from its old values in fp64 IEEE arithmetic in the
 * order above, and stored as the fp32 roundings of the fp64 results. Every
 * bf16 parameter is then within one bf16 step of the rounding of the exactly
 * computed master.
 *   d_grad    device pointer to the bf16 gradient shard's element 0
 *   d_state   device pointer to the tiled fp32 state of all n_state elements
 *             (layout above); updated in place
 *   d_param   device pointer to the bf16 parameter shard's element 0; must not
 *             alias any other buffer
 *   n_state   elements the state buffer describes (the shard size S)
 *   begin, count  elements to update; any sub-range of [0, n_state)
 *   hp        host pointer, read during the call
 *   d_rank_sqnorms  device array of n_ranks doubles (the ranks' partial sums
 *             of squares in rank order); may be NULL when max_norm <= 0
 * Pointers with d_grad/d_param 8-byte and d_state 16-byte alignment take the
 * vector path, others a slower element path with identical results. A range
 * longer than 2^27 elements is updated in several equal launches on `stream`
 * (each element once; the results do not depend on the split).
 * Errors: ZERO_EINVAL for null pointers (all may be NULL when count == 0), a
 * range outside [0, n_state), n_ranks < 1 with clipping on, or hyperparameters
 * that PyTorch's AdamW refuses (lr, eps or weight_decay below 0, a beta
 * outside [0, 1); a NaN fails these checks), clip_eps below 0, a NaN
 * max_norm or step < 1;
 * ZERO_EHIP if a launch fails. Non-finite inputs propagate per IEEE rules (a
 * NaN norm gives a NaN coefficient). */
int zero_adamw_step(const uint16_t* d_grad, float* d_state, uint16_t* d_param, int64_t n_state,
                    int64_t begin, int64_t count, const zero_adamw_hparams* hp,
                    const double* d_rank_sqnorms, int32_t n_ranks, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * zero_adamw_step_unpack -- zero_adamw_step followed by zero_unpack_params over
 * the same range, in one pass: each new bf16 parameter goes to the parameter
 * shard (what the all-gather sends, "第 5 课：ZeRO 与 FSDP" section 3) and
 * to its position in the per-tensor parameters (the shard's share of the
 * reassembled model; notes on the ZeRO paper, section 4.1). 30 bytes per
 * element instead of 28 + 4 in two passes.
 *   d_grad .. n_ranks  as zero_adamw_step; n_state must be the layout's shard
 *   h              layout handle of this rank
 *   tensor_params  HOST array of the layout's n_tensors device pointers to the
 *                  per-tensor bf16 parameters (as zero_unpack_params)
 * Results are bit-identical to the two calls. Padding elements update state
 * and the shard only. Ranges touching more than 64 tensor pieces, or longer
 * than 2^27 elements, take more than one launch (all on `stream`).
 * Errors: as zero_adamw_step and zero_unpack_params, plus ZERO_EINVAL when
 * n_state differs from the layout's shard size. */
int zero_adamw_step_unpack(const uint16_t* d_grad, float* d_state, uint16_t* d_param, int64_t n_state,
                           int64_t begin, int64_t count, const zero_adamw_hparams* hp,
                           const double* d_rank_sqnorms, int32_t n_ranks, zero_layout_t h,
                           uint16_t* const* tensor_params, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * zero_adamw_step_arrays -- zero_adamw_step over the state as the pages hold
 * it: the fp32 master weights, m and v of the rank's slice as three separate
 * arrays, K = 12 bytes per parameter ("第 5 课：ZeRO 与 FSDP" sections 2-3;
 * notes on the ZeRO paper, sections 2.1 and 4.1). The arithmetic, the clip
 * coefficient and the rounding rule are zero_adamw_step's; the results are
 * bit-identical to it on the same values.
 *   d_grad    device pointer to count bf16 gradients
 *   d_master, d_m, d_v  device pointers to count fp32 values each; updated in
 *             place
 *   d_param   device pointer to count bf16 parameters (written)
 *   count     elements; a sub-range of larger arrays is passed as offset
 *             pointers
 *   hp, d_rank_sqnorms, n_ranks, stream  as zero_adamw_step; a caller that
 *             holds the already-combined global sum of squares G passes a
 *             one-element array holding G with n_ranks = 1
 * When the five pointers share one phase (master, m and v equally placed
 * against 16-byte boundaries, and the gradient and parameter against 8-byte
 * boundaries at the same element), the update takes the vector path; other
 * placements take a slower element path with identical results. More than
 * 2^27 elements take several launches on `stream`.
 * Errors: as zero_adamw_step; also ZERO_EINVAL when any two of the five
 * arrays overlap, or for a NULL or non-4-byte-aligned m or v with count > 0. */
int zero_adamw_step_arrays(const uint16_t* d_grad, float* d_master, float* d_m, float* d_v,
                           uint16_t* d_param, int64_t count, const zero_adamw_hparams* hp,
                           const double* d_rank_sqnorms, int32_t n_ranks, hipStream_t stream);

/* zero_state_import / zero_state_export -- copy n elements of fp32 master, m
 * and v between three separate device arrays and the tiled state buffer
 * (layout above). A bit copy; the arrays must not overlap. For callers whose
 * optimizer state lives in separate tensors (for example one rank's slice of
 * a sharded checkpoint, "別再複製本可分片的東西" on sharded checkpoints).
 * Errors: ZERO_EINVAL for n < 0, NULL or non-4-byte-aligned pointers (NULL is
 * allowed when n == 0); ZERO_EHIP if a launch fails. */
int zero_state_import(const float* d_master, const float* d_m, const float* d_v, float* d_state,
                      int64_t n, hipStream_t stream);
int zero_state_export(const float* d_state, float* d_master, float* d_m, float* d_v, int64_t n,
                      hipStream_t stream);

/* ---------------------------------------------------------------------------
 * fp32 gradient accumulation ("第 5 课：ZeRO 与 FSDP" section 2, note on fp32
 * gradient accumulation: with ZeRO-2/3 the accumulator is partitioned like
 * the gradients, 4 bytes per shard element).
 *
 * zero_accumulate_grads -- d_acc[i] = (first ? 0 : d_acc[i]) + g[i] for count
 * elements: one micro-batch's bf16 gradient slice added into the fp32
 * accumulator (fp32 add, round to nearest even; with first != 0 d_acc is not
 * read). Sub-ranges by offset pointers. 8-byte aligned d_grad and 16-byte
 * aligned d_acc take the vector path. Errors: ZERO_EINVAL for count < 0, NULL
 * buffers (allowed when count == 0) or pointers not aligned to their element
 * size; ZERO_EHIP if a launch fails. */
int zero_accumulate_grads(const uint16_t* d_grad, float* d_acc, int64_t count, int32_t first,
                          hipStream_t stream);

/* zero_shard_sqnorm_f32 -- zero_shard_sqnorm for an fp32 gradient (the
 * accumulator): *d_out (+)= sum of g*g, each square exact in fp64, fixed
 * order. The workspace is zero_sqnorm_workspace_bytes(count) bytes. Errors as
 * zero_shard_sqnorm (d_grad must be 4-byte aligned). */
int zero_shard_sqnorm_f32(const float* d_grad, int64_t count, double* d_out, int32_t accumulate,
                          void* d_workspace, size_t ws_bytes, hipStream_t stream);

/* zero_adamw_step_f32grad -- zero_adamw_step with an fp32 gradient shard
 * (d_grad: element 0 of the accumulator): the same update and arguments,
 * 30 bytes per element instead of 28. The vector path needs d_grad 16-byte
 * aligned. Errors as zero_adamw_step. */
int zero_adamw_step_f32grad(const float* d_grad, float* d_state, uint16_t* d_param, int64_t n_state,
                            int64_t begin, int64_t count, const zero_adamw_hparams* hp,
                            const double* d_rank_sqnorms, int32_t n_ranks, hipStream_t stream);

/* zero_adamw_step_f32grad_unpack -- zero_adamw_step_f32grad followed by
 * zero_unpack_params over the same range, in one pass (32 bytes per element);
 * arguments, results and errors as zero_adamw_step_unpack, with the fp32
 * gradient of zero_adamw_step_f32grad. */
int zero_adamw_step_f32grad_unpack(const float* d_grad, float* d_state, uint16_t* d_param, int64_t n_state,
                                   int64_t begin, int64_t count, const zero_adamw_hparams* hp,
                                   const double* d_rank_sqnorms, int32_t n_ranks, zero_layout_t h,
                                   uint16_t* const* tensor_params, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * zero_unpack_params -- write the updated bf16 shard back into the tensors.
 * Copies shard elements [begin, begin+count) of param_shard to the tensor
 * elements the layout maps them to (the full parameters that the all-gather
 * reassembles, "第 5 课：ZeRO 与 FSDP" section 3; notes section 4.1; the
 * updated slice is what the next forward gathers, "ZeRO-3 核心流程" section
 * 2). Padding goes nowhere; no other tensor byte is written.
 *   param_shard   device pointer to the shard's element 0
 *   tensor_params host array of n_tensors DEVICE pointers (NULL allowed for
 *                 tensors the range does not touch)
 * Errors as zero_pack_grads. */
int zero_unpack_params(zero_layout_t h, const uint16_t* param_shard, uint16_t* const* tensor_params,
                       int64_t begin, int64_t count, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * zero_cpu_adamw_step -- ZeRO-Offload: the same update as zero_adamw_step run
 * by the host cores on HOST memory (the mlqm.cn article's ZeRO-Offload
 * section: optimizer state in CPU memory, the CPU runs Adam, results return
 * over PCIe; "別再複製本可分片的東西": CPU offload of the sharded state).
 * Same update, state layout and arithmetic as zero_adamw_step (fp32 with fused
 * multiply-adds, correctly rounded sqrt and division, round-to-nearest-even
 * bf16; the same cancellation test and fp64 recomputation), so on hosts with
 * hardware FMA it matches the GPU bit for bit.
 *   h_grad    HOST array of the count bf16 gradients of the range (element
 *             begin first): a staging buffer the caller fills from the GPU
 *   h_state   HOST pointer to the tiled fp32 state of all n_state elements
 *   h_param   HOST array receiving the count bf16 parameters of the range
 *   h_rank_sqnorms  HOST array of n_ranks doubles, added in zero_adamw_step's
 *             order
 *   n_threads host threads to use (0 = all the process may run on); the
 *             library keeps its threads for the life of the process, and
 *             concurrent calls run one after another
 * Pinned staging buffers let the caller overlap the PCIe copies of one range
 * with the update of another.
 * Synchronous: returns when the range is updated. Errors: as zero_adamw_step,
 * plus ZERO_EINVAL for n_threads < 0 and ZERO_ENOMEM if threads cannot start. */
int zero_cpu_adamw_step(const uint16_t* h_grad, float* h_state, uint16_t* h_param, int64_t n_state,
                        int64_t begin, int64_t count, const zero_adamw_hparams* hp,
                        const double* h_rank_sqnorms, int32_t n_ranks, int32_t n_threads);

/* Message describing the calling thread's last error ("" if none). */
const char* zero_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ZERO_MI355X_H */
