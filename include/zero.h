/*
 * zero.h -- C ABI of the ZeRO sharded optimizer step for AMD Instinct MI355X
 * (gfx950), built as libzero.so.
 *
 * The library runs one GPU's share of the data-parallel optimizer step of
 * ZeRO stages 1-3 / FSDP, with N ranks' gradient buffers resident in that
 * GPU's memory: for every element of a rank's shard it sums the N ranks'
 * gradients in rank order (the reduction half of reduce-scatter), divides by
 * N, optionally scales by a global-norm clip coefficient, runs AdamW on the
 * fp32 master / first-moment / second-moment slice and writes the bf16 copy of
 * the updated master into its all-gather output slot.
 *
 * Pages cited below:
 *   [p1] "ZeRO and FSDP sharding" (tirogla.com): How it works; Code;
 *        Implementation notes; Pitfalls.
 *   [p3] "ZeRO: Three Ledgers, Zero Redundancy" (dominator-index.github.io):
 *        sections 1, 2 and 4.
 *   [p4] "Learn: ZeRO & FSDP" (gunjandhanuka.github.io): sections 3 and 4.
 *
 * Conventions for every entry point:
 *   - Returns zero_status: ZERO_OK (0) or a negative error code.  Nothing
 *     prints, throws or exits.
 *   - Validation happens before any device work: on an error return before a
 *     launch, no device memory has been written.
 *   - Device pointers are plain HIP device addresses (e.g. from hipMalloc or a
 *     torch tensor's data_ptr()).  The caller owns every buffer; the library
 *     allocates no device memory and keeps no pointer after a call returns.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Calls marked "async" only enqueue work on it.
 *   - The library is reentrant; its only global state is per-device caches of
 *     the compute-unit count and LDS sizes, the occupancy settings read once
 *     from the environment, and a thread-local last-HIP-error string.
 *
 * Floating point: the device code is compiled without FMA contraction, with
 * IEEE binary32 denormals and correctly rounded division and square root, so
 * that every element's result is the same bit pattern as a serial binary32
 * evaluation of the same operations in the same order.
 */
#ifndef ZERO_H
#define ZERO_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ZERO_ABI_VERSION 2

typedef int32_t zero_status;
#define ZERO_OK 0
#define ZERO_EINVAL (-1)  /* bad argument: NULL, negative size, bad enum, aliasing, N < 1 */
#define ZERO_ERANGE (-2)  /* a size or index overflows, or N > ZERO_MAX_RANKS */
#define ZERO_EALIGN (-3)  /* a pointer is not aligned to its element size */
#define ZERO_ENOSPC (-4)  /* a caller-provided buffer is too small */
#define ZERO_EHIP (-5)    /* a HIP runtime call or kernel launch failed; see zero_last_hip_error() */
#define ZERO_EIO (-6)     /* a checkpoint file could not be opened, read or written */
#define ZERO_ECORRUPT (-7) /* not a valid checkpoint shard: bad magic or version, wrong size,
                              failed checksum, or shards of different checkpoints */

#define ZERO_MAX_RANKS 256   /* largest N accepted by zero_step / zero_gradnorm */
#define ZERO_MAX_UNITS (1 << 20)

/* Element types. */
#define ZERO_F32 0
#define ZERO_BF16 1

/* Index spaces of a buffer (see the layout below).
 *   ZERO_GLOBAL: indexed by the global index j of the padded flat buffer
 *                (length P^).  For gradients this is a rank's full gradient;
 *                for the bf16 output it is the all-gather output buffer, and
 *                rank r's values land in rank r's slots.
 *   ZERO_LOCAL:  indexed by the local index k of one rank's shard (length S).
 *                For gradients this is the chunk every rank sends to this rank
 *                in the reduce-scatter; for the output it is the bf16 shard
 *                ZeRO-3 keeps. */
#define ZERO_GLOBAL 0
#define ZERO_LOCAL 1

/* ------------------------------------------------------------------------
 * Layout -- [p1 How it works]: each unit's parameters are flattened into one
 * buffer padded to a multiple of N and rank r owns slice r; [p1 Pitfalls]:
 * the flat numel must divide by N or the last rank's slice is corrupted.
 *
 * For unit u with numel P_u (the sum of its parameters' numels, in the
 * caller's order) and granule g_u (1 for the flat layout; the row length for
 * the row-aligned layout of zero_pack_rows):
 *   padded_u  = ceil(P_u / (N g_u)) * N g_u     shard_u = padded_u / N
 *   offset_u  = sum of padded_{u'} over u' < u   (start in the flat buffer)
 *   local_u   = sum of shard_{u'}  over u' < u   (start inside a rank's shard)
 * Rank r's slice of unit u is global [offset_u + r*shard_u, +shard_u); its
 * local index k in [local_u, local_u + shard_u) maps to global index
 * j = offset_u + r*shard_u + (k - local_u).  P^ = sum padded_u, S = sum shard_u.
 * ------------------------------------------------------------------------ */

typedef struct zero_unit {
    int64_t numel;         /* P_u */
    int64_t padded;        /* padded_u */
    int64_t shard;         /* shard_u (a multiple of granule) */
    int64_t offset;        /* offset_u */
    int64_t local_offset;  /* local_u */
    int64_t granule;       /* g_u: elements per row the shards are aligned to */
} zero_unit;

typedef struct zero_layout {
    uint32_t magic;        /* ZERO_LAYOUT_MAGIC once filled by zero_pack */
    int32_t n_ranks;       /* N */
    int32_t n_units;       /* U */
    int32_t reserved;
    int64_t numel;         /* sum P_u */
    int64_t padded;        /* P^ */
    int64_t shard;         /* S */
    zero_unit unit[];      /* U entries */
} zero_layout;

#define ZERO_LAYOUT_MAGIC 0x5a45524fu /* "ZERO" */

/* Bytes a layout of n_units units occupies. */
size_t zero_layout_bytes(int32_t n_units);

/* Fill a caller-owned layout.  Host only.
 *   n_ranks    N >= 1 (any value up to 2^31-1; zero_step itself caps N).
 *   unit_numel U non-negative numels (host array).
 *   layout     caller memory of layout_bytes bytes, or NULL to query the size.
 *   bytes_needed (may be NULL) receives zero_layout_bytes(n_units).
 * Errors: EINVAL (bad N, U < 0, negative numel, NULL unit_numel with U > 0),
 *         ERANGE (a padded size overflows int64), ENOSPC (layout_bytes short;
 *         bytes_needed is still filled). */
zero_status zero_pack(int32_t n_ranks, int32_t n_units, const int64_t *unit_numel,
                      zero_layout *layout, size_t layout_bytes, size_t *bytes_needed);

/* Row-aligned layout -- [p4 section 5, FSDP1 vs FSDP2]: FSDP2 shards each
 * parameter on its own along dim 0 (torch.chunk over the rows) instead of
 * FSDP1's flatten-concat-chunk buffer; [p3, the note after section 5] calls
 * this row-aligned sharding.  Give
 * each parameter its own unit with granule = its row length (numel / rows):
 * rank r then owns rows [r c, (r+1) c) of the parameter, c = ceil(rows / N),
 * zero-padded to c rows -- FSDP2's shard of that parameter.  unit_granule[u]
 * >= 1 must divide unit_numel[u] (EINVAL otherwise).  The step, the norm and
 * the packer work unchanged on row-aligned layouts.  Errors as zero_pack. */
zero_status zero_pack_rows(int32_t n_ranks, int32_t n_units, const int64_t *unit_numel,
                           const int64_t *unit_granule, zero_layout *layout,
                           size_t layout_bytes, size_t *bytes_needed);

/* Index maps of the layout (host only).  zero_global_index: global j of rank
 * r's local k (EINVAL unless 0 <= r < N and 0 <= k < S).  zero_owner: owning
 * rank and local index of global j (EINVAL unless 0 <= j < P^). */
zero_status zero_global_index(const zero_layout *layout, int32_t rank, int64_t k, int64_t *j);
zero_status zero_owner(const zero_layout *layout, int64_t j, int32_t *rank, int64_t *k);

/* Pack parameters into a flat buffer on the device (async) -- [p1 How it
 * works] flattening, with the padding zero-filled.
 *   params: n_params device pointers; param p has src_numel[p] elements of
 *     src_dtype and belongs to unit src_unit[p].  Within a unit, parameters
 *     are laid out in the order they appear in this list; the numels of each
 *     unit's parameters must add up to that unit's numel.
 *   rank < 0: dst is the whole padded flat buffer (ZERO_GLOBAL, P^ elements).
 *   rank r:   dst is rank r's shard (ZERO_LOCAL, S elements): only the
 *             elements rank r owns are copied.
 *   dst_dtype: ZERO_F32 or ZERO_BF16 (F32 -> BF16 rounds to nearest even;
 *     BF16 -> F32 widens exactly).
 * Errors: EINVAL (bad arguments, unit numels do not add up, dst overlaps a
 *   source), EALIGN, EHIP. */
zero_status zero_pack_copy(const zero_layout *layout, int32_t rank, int32_t n_params,
                           const void *const *params, const int64_t *src_numel,
                           const int32_t *src_unit, int32_t src_dtype,
                           void *dst, int32_t dst_dtype, void *stream);

/* Inverse of zero_pack_copy: copy each parameter's elements out of a flat
 * buffer (rank < 0: GLOBAL P^ buffer; rank r: rank r's LOCAL shard, only the
 * elements rank r owns are written).  Async. */
zero_status zero_unpack_copy(const zero_layout *layout, int32_t rank, const void *src,
                             int32_t src_dtype, int32_t n_params, void *const *params,
                             const int64_t *dst_numel, const int32_t *dst_unit,
                             int32_t dst_dtype, void *stream);

/* Reshard -- [p1 Implementation notes]: a sharded checkpoint (each rank
 * writes its own shard) is resharded to a different N at load time; [p4
 * section 5, FSDP1 vs FSDP2]: checkpoints carry over between the flat and the
 * per-parameter layouts.
 *
 * An element is identified by its stream position: its index in the
 * concatenation of all units' unpadded elements, in unit order.  `from` and
 * `to` must hold the same number of elements (layout->numel); their units, N
 * and granules may differ (e.g. one unit per block, flat, N = 64 -> one unit
 * per parameter, row-aligned, N = 32).  src holds from->n_ranks pointers, rank
 * q's LOCAL shard in layout `from` (from->shard elements each).  dst receives
 * rank dst_rank's LOCAL shard in layout `to` (to->shard elements): each
 * element is copied from the rank and local index that hold the same stream
 * position in `from`; padding is zero.  dtype: ZERO_F32 (state) or ZERO_BF16
 * (parameters); values are copied bit for bit, not converted.  zero_reshard:
 * device pointers, asynchronous on `stream`; zero_reshard_host: host pointers,
 * synchronous.  dst may be NULL when to->shard is 0, and src[q] when
 * from->shard is 0.  Errors: EINVAL (element counts differ, bad rank, NULL, dst
 * overlapping a source), EALIGN (a pointer not aligned to the element size),
 * EHIP. */
zero_status zero_reshard(const zero_layout *from, const void *const *src,
                         const zero_layout *to, int32_t dst_rank, void *dst, int32_t dtype,
                         void *stream);
zero_status zero_reshard_host(const zero_layout *from, const void *const *src,
                              const zero_layout *to, int32_t dst_rank, void *dst, int32_t dtype);

/* Algorithmic HBM bytes of one zero_reshard: elem * (elements copied from the
 * sources + to->shard elements written), elem = 4 (ZERO_F32) or 2 (ZERO_BF16);
 * *elements = to->shard.  EINVAL as zero_reshard. */
zero_status zero_reshard_traffic(const zero_layout *from, const zero_layout *to, int32_t dst_rank,
                                 int32_t dtype, double *bytes, int64_t *elements);

/* Placement of the step's buffers in one device allocation (host only) --
 * [p1 How it works]: the step streams flat per-rank gradient buffers and the
 * flat fp32 master / m / v / bf16 buffers side by side.  How such buffers sit
 * relative to each other in HBM is a property of MI355X, not of the method:
 * device memory is mapped in 2 MiB pages, so a buffer's phase inside its
 * page is the same physically as virtually, and buffers that start at the
 * same phase are streamed through the same HBM channels at the same moment.
 * Measured with the N = 64 step (the fused kernel, 65 streamed buffers): 67 %
 * of the 8 TB/s peak with every buffer 2 MiB-aligned (what one allocation per
 * buffer gives), 73-74 % with staggered phases; the staged N = 64 step 75.2 /
 * 78.0 % and the N = 8 step 82.2 / 83.4 % without / with the stagger.  The
 * stagger was chosen on those two rank counts; no single rule measured won
 * at every N (the exception below covers the largest dips found).
 *
 * Lays out n_buffers buffers of bytes[i] bytes, in the given order, in one
 * allocation: buffer i starts at the first offset at or after the end of
 * buffer i - 1 whose remainder modulo 2 MiB is (i * 256 KiB) mod 2 MiB, with
 * one exception: in a run of more than 32 consecutive buffers of one size,
 * a buffer whose start would lie a multiple of 2 MiB plus 32 MiB (modulo 64
 * MiB) past the previous one's, beyond the stagger, starts 2 MiB later (the
 * staged step at the rank counts with that spacing, 96 and 160 bf16 or 64
 * and 192 fp32 gradients, measured 1.2 to 7.2 points faster; any extra space
 * cost the fused 32-rank step 1 to 3 points, hence only for runs longer than
 * 32).  offsets[i] receives the byte offset of buffer i (every offset is a
 * multiple of 256 KiB), *total_bytes the size to allocate (the end of the
 * last buffer).  Order the buffers as the step reads them: the gradients,
 * then master, exp_avg, exp_avg_sq, then the output.  EINVAL: n_buffers < 0,
 * a negative size, NULL pointers; ERANGE: the total overflows int64. */
zero_status zero_arena_plan(int32_t n_buffers, const int64_t *bytes, int64_t *offsets,
                            int64_t *total_bytes);

/* ------------------------------------------------------------------------
 * AdamW step scalars -- [p1 Code]: AdamW with b1, b2, eps, decoupled weight
 * decay wd, a step counter t that is 1 at the first step, and bias
 * corrections 1 - b1^t and sqrt(1 - b2^t).
 *
 * Computed on the host in binary32, one rounding per operation:
 *   one_minus_b1 = 1 - b1, one_minus_b2 = 1 - b2 (from the binary32 betas);
 *   pow1 = b1^t, pow2 = b2^t as running products (p_t = p_{t-1} * b, p_0 = 1);
 *   bc1 = 1 - pow1;  bc2 = sqrtf(1 - pow2);
 *   step_size = lr / bc1;  decay = 1 - lr * wd.
 * clip_coef multiplies the averaged gradient (1 = no clipping).
 * ------------------------------------------------------------------------ */

typedef struct zero_adamw_scalars {
    int32_t t;
    float lr, b1, b2, eps, wd;
    float one_minus_b1, one_minus_b2;
    float pow1, pow2;
    float bc1, bc2;
    float step_size;
    float decay;
    float clip_coef;
} zero_adamw_scalars;

/* Scalars of step t >= 1 (O(t) host work).  EINVAL: t < 1, NULL out, or a
 * hyperparameter that is NaN. */
zero_status zero_adamw_scalars_for(int32_t t, float lr, float b1, float b2, float eps, float wd,
                                   float clip_coef, zero_adamw_scalars *out);

/* Scalars of step prev->t + 1 from those of step prev->t (O(1); equal to
 * zero_adamw_scalars_for(prev->t + 1, ...)).  clip_coef is copied. */
zero_status zero_adamw_scalars_next(const zero_adamw_scalars *prev, zero_adamw_scalars *out);

/* ------------------------------------------------------------------------
 * The fused step -- [p1 Code] reduce-scatter, divide by N, AdamW on the
 * local slice, all-gather; [p1 How it works] the updated fp32 master is
 * cast to a bf16 copy for the gather; [p3 section 1] the update is
 * elementwise, so any partition of the elements gives the same result.
 *
 * For every processed element, with G_q the binary32 value of gradient q:
 *   s = G_0 + G_1 + ... + G_{n_grads-1}   (left to right, binary32)
 *   g = s / divisor  (a multiply by 1/divisor when divisor is a power of two,
 *                     which is the same correctly rounded value)
 *   g = g * clip_coef
 *   m = b1*m + (1-b1)*g
 *   v = b2*v + ((1-b2)*g)*g
 *   w = w*decay - (step_size*m) / (sqrt(v)/bc2 + eps)
 *   out = bf16(w), rounded to nearest even
 *
 *   rank < 0:  every shard of every unit -- all N simulated ranks' steps at
 *              once.  grads, state and out must all be ZERO_GLOBAL.
 *   rank r:    rank r's shard only (S elements).
 *   grads:     host array of n_grads device pointers (1 <= n_grads <=
 *              ZERO_MAX_RANKS), summed in array order; each of grad_dtype and
 *              in the grad_index space.  n_grads is normally N; pass 1 with
 *              divisor 1 for a gradient that is already reduced.
 *   divisor:   > 0 and finite (normally N).
 *   master, exp_avg, exp_avg_sq: fp32 state in the state_index space, updated
 *              in place.
 *   out:       bf16 bits in the out_index space, or NULL.
 *   sc:        the step's scalars.
 * Async on `stream`.  Errors: EINVAL (NULL, bad enum, rank >= N, rank < 0 with
 *   a LOCAL index, divisor not > 0, gradient range overlapping state or out,
 *   state/out ranges overlapping each other), ERANGE (n_grads out of range),
 *   EALIGN (pointer not aligned to its element size), EHIP (launch failed). */
zero_status zero_step(const zero_layout *layout, int32_t rank,
                      const void *const *grads, int32_t n_grads, int32_t grad_dtype,
                      int32_t grad_index, float divisor,
                      float *master, float *exp_avg, float *exp_avg_sq, int32_t state_index,
                      uint16_t *out, int32_t out_index,
                      const zero_adamw_scalars *sc, void *stream);

/* zero_step with the clip multiplier read from device memory (a float the
 * stream has produced, e.g. by zero_clip_coef_async) instead of
 * sc->clip_coef.  With zero_gradnorm_async and zero_clip_coef_async this
 * makes the whole clipped step free of host synchronization, so it can be
 * enqueued ahead or captured in a graph.  A NaN multiplier (the coefficient
 * of a non-finite norm) skips the step: master, exp_avg, exp_avg_sq and out
 * are left unchanged, as a loss scaler skips the step of an overflowed
 * gradient; the caller can read the multiplier to see that it happened (and
 * not advance t).  clip_coef_dev must not overlap any buffer the step writes
 * (EINVAL).  Otherwise as zero_step. */
zero_status zero_step_device_clip(const zero_layout *layout, int32_t rank,
                                  const void *const *grads, int32_t n_grads, int32_t grad_dtype,
                                  int32_t grad_index, float divisor,
                                  float *master, float *exp_avg, float *exp_avg_sq,
                                  int32_t state_index, uint16_t *out, int32_t out_index,
                                  const zero_adamw_scalars *sc, const float *clip_coef_dev,
                                  void *stream);

/* The staged step -- the same step as zero_step ([p1 Code]: reduce-scatter,
 * divide by N, AdamW on the local slice, bf16 for the gather), every element
 * with the same bits, split for large N into two kernels per chunk of
 * elements: the first sums the N gradients in rank order and divides
 * (writing g, fp32, to `workspace`), the second runs the fused step on that
 * one reduced gradient.  Each kernel streams a simpler mix than the fused
 * one, and a chunk of up to 32M elements (128 MB) fits MI355X's 256 MB
 * memory-side cache (chunks larger than the cache measured 2 points slower):
 * at N = 64 the step runs about 6 % faster than fused (3.08 against 3.28 ms
 * on an 8B-parameter model's 125M-element shard).
 *   workspace:  caller device memory, 16-byte aligned, not overlapping any
 *               other buffer of the call; its size sets the chunk (whole
 *               512-element tiles, at most 32M elements; at least 2048 bytes).
 *               With 16 bytes to spare beyond the chunk, each chunk's reduced
 *               gradient is placed at the state's 16-byte phase, so both
 *               kernels take their vector paths whenever the gradients and
 *               the state share a phase (as the fused step needs too).
 *               zero_step_staged_workspace_bytes gives the size that needs a
 *               single chunk up to that limit, spare bytes included.
 * For n_grads <= 32 with bf16 gradients, and n_grads <= 24 with fp32
 * gradients (twice the bytes per rank), the fused step is as fast or faster
 * and runs instead; the workspace is then not used and may be NULL.  The size
 * query does not know the gradient type: it returns 0 up to 24 gradients and
 * one chunk's size from 25 on.  Async on `stream`.  Errors as zero_step,
 * plus, where the staged step runs: EINVAL (NULL workspace, workspace
 * overlapping another buffer), EALIGN (workspace not 16-byte aligned),
 * ENOSPC (workspace_bytes < 2048). */
zero_status zero_step_staged_workspace_bytes(const zero_layout *layout, int32_t rank,
                                             int32_t n_grads, size_t *bytes);
zero_status zero_step_staged(const zero_layout *layout, int32_t rank,
                             const void *const *grads, int32_t n_grads, int32_t grad_dtype,
                             int32_t grad_index, float divisor,
                             float *master, float *exp_avg, float *exp_avg_sq, int32_t state_index,
                             uint16_t *out, int32_t out_index,
                             const zero_adamw_scalars *sc, void *workspace, size_t workspace_bytes,
                             void *stream);

/* The step of a range of units, from gradient buckets -- [p1 How it works]:
 * each unit's gradients are reduce-scattered as soon as backward has produced
 * them, and the unit's shards can be stepped then; [p3 section 4]: with
 * bucketed reduce-scatter each bucket is freed once reduced, so gradients are
 * transient.  Steps units [unit_begin, unit_end) of the selection (rank < 0:
 * every rank's slices of those units; rank r: rank r's slices) with the same
 * arithmetic as zero_step.  grads[q] is a bucket holding only those units in
 * the grad_index space: element j of the layout (ZERO_GLOBAL) at bucket index
 * j - offset_{unit_begin}, local index k (ZERO_LOCAL) at k -
 * local_offset_{unit_begin}; a bucket spans offset_{unit_end} -
 * offset_{unit_begin} (resp. local_offset) elements, and may be NULL when
 * that is 0.  master, exp_avg,
 * exp_avg_sq and out are the whole buffers, indexed as in zero_step.  Steps of
 * disjoint unit ranges that together cover every unit, in any order and on any
 * streams, give the bits of one zero_step call, so a caller can step unit k
 * on a side stream while backward still writes the buckets of the next units.
 * workspace: as zero_step_staged, used where that call stages (bf16
 * gradients above 32, fp32 above 24; NULL: the fused step at any N).  Async on `stream`.  Errors as zero_step / zero_step_staged,
 * plus EINVAL for a unit range outside 0 <= unit_begin <= unit_end <= U. */
zero_status zero_step_units(const zero_layout *layout, int32_t rank, int32_t unit_begin,
                            int32_t unit_end, const void *const *grads, int32_t n_grads,
                            int32_t grad_dtype, int32_t grad_index, float divisor,
                            float *master, float *exp_avg, float *exp_avg_sq, int32_t state_index,
                            uint16_t *out, int32_t out_index, const zero_adamw_scalars *sc,
                            void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * The step on host cores, for ZeRO-Offload -- [p4 section 6]: the optimizer
 * state and the fp32 step live in CPU memory; gradients come down from the
 * GPU and updated parameters go back; [p1 Implementation notes]: offload
 * trades PCIe bandwidth for capacity.
 *
 * Same selection, index rules, validation and arithmetic as zero_step (every
 * element bit-identical to it), on host pointers, by n_threads worker threads
 * (<= 0: all hardware threads; fewer are used for small selections).  The
 * result does not depend on the thread count.  Synchronous: returns when the
 * step is done.  Errors as zero_step (EHIP cannot occur).
 * ------------------------------------------------------------------------ */
zero_status zero_step_host(const zero_layout *layout, int32_t rank,
                           const void *const *grads, int32_t n_grads, int32_t grad_dtype,
                           int32_t grad_index, float divisor,
                           float *master, float *exp_avg, float *exp_avg_sq, int32_t state_index,
                           uint16_t *out, int32_t out_index,
                           const zero_adamw_scalars *sc, int32_t n_threads);

/* The offload step with its PCIe transfers, pipelined -- [p4 section 6]: the
 * reduced gradient comes down, the host steps the fp32 state, the bf16
 * parameters go back up; the PCIe link is the bottleneck.
 *
 * For rank r's shard (S = layout->shard elements, LOCAL indexing): d_grad is
 * the reduced fp32 gradient on the device (e.g. written by the norm pass),
 * already averaged and, if clipping, to be scaled by sc->clip_coef; master,
 * exp_avg, exp_avg_sq are host arrays of S floats; d_out receives the S bf16
 * parameters on the device.  The shard moves in chunks of `chunk` elements
 * through two staging slots the caller provides in pinned host memory
 * (h_grad_stage: 2 * chunk floats; h_out_stage: 2 * chunk bf16): the copy
 * down of chunk c + 1 (stream_down), the host step of chunk c and the copy up
 * of chunk c - 1 (stream_up) overlap.  Every element is bit-identical to
 * zero_step with one fp32 gradient and divisor 1.  Ordering: the copies read
 * d_grad in stream_down's order and write d_out in stream_up's order, so the
 * kernel producing d_grad must run on stream_down (or be complete) and
 * readers of d_out must follow stream_up (the call returns after both
 * streams are drained).  Synchronous: returns when the last chunk is on the
 * device.  Errors: EINVAL, EALIGN, EHIP. */
zero_status zero_offload_step(const zero_layout *layout, int32_t rank,
                              const float *d_grad, float *h_grad_stage,
                              float *master, float *exp_avg, float *exp_avg_sq,
                              uint16_t *h_out_stage, uint16_t *d_out,
                              int64_t chunk, const zero_adamw_scalars *sc, int32_t n_threads,
                              void *stream_down, void *stream_up);

/* ------------------------------------------------------------------------
 * Global gradient norm -- [p1 Implementation notes]: clipping needs the
 * global norm, the sum of the shards' squared norms (all-reduced across
 * ranks); [p3 section 2] a norm is a decomposable sum of squares.
 *
 * Sum of squares, accumulated in binary64, of g = (rank-ordered binary32 sum
 * of the gradients) / divisor over the processed elements (same selection and
 * index rules as zero_step).  Two stages: one wave of the first reduces each
 * 512-element tile of a contiguous run to one binary64 partial (each lane
 * sums the squares of 8 consecutive elements in order, the wave adds its
 * lanes in a fixed butterfly); a run's tiles start 0 to 56 elements before
 * it (its first gradient element's index modulo a 128-byte line, in whole
 * 8-element groups), and elements outside the run add nothing.  The second
 * stage adds the partials in a fixed-order tree of 1024-way workgroups.  The
 * partition depends only on the layout, the rank and the index spaces (not
 * on the device, pointer alignment or whether g_out is written), so the
 * result is bitwise reproducible.
 *   g_out:      if not NULL, g is also written (fp32, g_index space), so the
 *               step can read one reduced gradient instead of N.
 *   workspace:  caller device memory of at least zero_gradnorm_workspace_bytes.
 *   sumsq:      host pointer; receives the binary64 sum.
 * Synchronizes `stream` (the host needs the value to form the clip
 * coefficient).  Errors as zero_step, plus ENOSPC for a short workspace. */
zero_status zero_gradnorm_workspace_bytes(const zero_layout *layout, int32_t rank,
                                          size_t *bytes);
zero_status zero_gradnorm(const zero_layout *layout, int32_t rank,
                          const void *const *grads, int32_t n_grads, int32_t grad_dtype,
                          int32_t grad_index, float divisor,
                          float *g_out, int32_t g_index,
                          void *workspace, size_t workspace_bytes,
                          double *sumsq, void *stream);

/* The same pass without the host synchronization (async): the binary64 sum
 * of squares is written to the device pointer sumsq_dev (8-byte aligned,
 * outside the workspace), bitwise equal to what zero_gradnorm returns.  For
 * callers that keep the norm on the stream (a later kernel, a graph, an
 * all-reduce of the per-rank sums) or time it with events. */
zero_status zero_gradnorm_async(const zero_layout *layout, int32_t rank,
                                const void *const *grads, int32_t n_grads, int32_t grad_dtype,
                                int32_t grad_index, float divisor,
                                float *g_out, int32_t g_index,
                                void *workspace, size_t workspace_bytes,
                                double *sumsq_dev, void *stream);

/* zero_gradnorm_async for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  No workspace is passed: the partial sums live in a
 * library-owned device array of ZERO_NOALLOC_SCRATCH_BYTES per GPU (static
 * device memory of the library's code object, held by every GPU the library
 * runs on until the process ends).  The selection's partials must fit
 * (zero_gradnorm_workspace_bytes <= ZERO_NOALLOC_SCRATCH_BYTES, about 1.07G
 * elements; ENOSPC otherwise, before any device work).  The call allocates
 * nothing and calls no allocating routine.  Every call on one GPU shares that
 * GPU's array, which keeps the last call's contents (every partial is written
 * before it is read, so nothing needs clearing): calls that overlap on one GPU
 * (different streams without ordering, or threads) race and give wrong sums.
 * The first call on a device looks the array's address up
 * (hipGetSymbolAddress); make one call on that device before capturing a
 * graph.  Result, g_out and errors otherwise as zero_gradnorm_async. */
#define ZERO_NOALLOC_SCRATCH_BYTES (16u << 20)
zero_status zero_gradnorm_async_noalloc(const zero_layout *layout, int32_t rank,
                                        const void *const *grads, int32_t n_grads,
                                        int32_t grad_dtype, int32_t grad_index, float divisor,
                                        float *g_out, int32_t g_index, double *sumsq_dev,
                                        void *stream);

/* Clip coefficient from a sum of squares (host): norm = sqrt(sumsq) and
 * coef = min(1, max_norm / (norm + 1e-6)) in binary64, rounded once to
 * binary32 -- the convention of the clip_grad_norm_ routine [p1
 * Implementation notes] names.  EINVAL: sumsq negative, NaN or infinite (a
 * non-finite gradient has no coefficient), max_norm <= 0. */
zero_status zero_clip_coef(double sumsq, double max_norm, float *coef);

/* The same coefficient on the device (async): reads the binary64 sum of
 * squares at sumsq_dev (8-byte aligned) and writes the binary32 coefficient
 * to coef_dev (4-byte aligned) -- bitwise equal to zero_clip_coef.  Where
 * the host function refuses the sum (negative, NaN or infinite), a NaN is
 * written, which makes zero_step_device_clip skip the step.  EINVAL: NULL
 * pointers or max_norm <= 0. */
zero_status zero_clip_coef_async(const double *sumsq_dev, double max_norm, float *coef_dev,
                                 void *stream);

/* The clip coefficient across ranks -- [p1 Implementation notes]: the global
 * norm is the square root of the sum of every shard's sum of squares.  Each
 * of N ranks computes its own shard's sum (zero_gradnorm / _async with its
 * rank); after they exchange the N binary64 sums (an all-gather of N doubles),
 * every rank adds them in rank order, sums[0] + sums[1] + ... + sums[N-1],
 * and forms the coefficient as zero_clip_coef does, so every rank scales by
 * the same binary32 value.  The total is written to *total when total is not
 * NULL.  Host: EINVAL for NULL pointers, n_ranks < 1 or > ZERO_MAX_UNITS, a
 * negative or NaN sum, an infinite total, max_norm <= 0. */
zero_status zero_clip_coef_ranks(const double *rank_sums, int32_t n_ranks, double max_norm,
                                 float *coef, double *total);

/* The same on the device (async): reads n_ranks binary64 sums at
 * rank_sums_dev (8-byte aligned), writes the coefficient to coef_dev and,
 * if total_dev is not NULL, the total -- bitwise equal to
 * zero_clip_coef_ranks on the same sums.  A total the host function refuses
 * (a negative, NaN or infinite sum) gives a NaN coefficient instead, which
 * makes zero_step_device_clip skip the step.  EINVAL: NULL
 * pointers, n_ranks out of range, max_norm <= 0; EALIGN; EHIP. */
zero_status zero_clip_coef_ranks_async(const double *rank_sums_dev, int32_t n_ranks,
                                       double max_norm, float *coef_dev, double *total_dev,
                                       void *stream);

/* ------------------------------------------------------------------------
 * Sharded checkpoint -- [p1 Implementation notes]: each rank writes its own
 * shard of the checkpoint, and a checkpoint saved at one N is resharded to a
 * different N when it is loaded; [p4 section 5, FSDP1 vs FSDP2]: the state
 * carries over between the flat and the per-parameter dim-0 layouts.
 *
 * One file per rank holds that rank's fp32 master, exp_avg and exp_avg_sq
 * shards (layout->shard elements each, bit for bit), the step count and the
 * layout's unit table (numel and granule per unit, N), after a 64-byte header
 * (magic "ZEROCKPT", format 1, the ABI version), and ends with a CRC-32C
 * (Castagnoli) of every byte before it.  Host memory only, synchronous; the
 * caller moves device state to or from host memory.
 * ------------------------------------------------------------------------ */

typedef struct zero_ckpt_info {
    int32_t format;   /* file format version (1) */
    int32_t abi;      /* ZERO_ABI_VERSION of the writer */
    int32_t n_ranks;  /* N of the saved layout: the checkpoint has N files */
    int32_t n_units;
    int32_t rank;     /* whose shard this file holds */
    int32_t step;     /* the AdamW step count t of the saved state */
    int64_t numel;    /* parameter elements (sum of the unit numels) */
    int64_t shard;    /* elements per array (the saved layout's S) */
} zero_ckpt_info;

/* Write rank `rank`'s shard to `path` (written to path.tmp, flushed, then
 * renamed).  master / exp_avg / exp_avg_sq: host arrays of layout->shard
 * floats (may be NULL when that is 0).  step >= 0.  EINVAL, EIO. */
zero_status zero_ckpt_save(const char *path, const zero_layout *layout, int32_t rank,
                           int32_t step, const float *master, const float *exp_avg,
                           const float *exp_avg_sq);

/* Read one shard file's header and rebuild its saved layout (two-call size
 * query as zero_pack: layout NULL -> *bytes_needed only).  verify != 0 also
 * checks the CRC-32C over the whole file.  EINVAL, EIO, ECORRUPT, ENOSPC. */
zero_status zero_ckpt_inspect(const char *path, int32_t verify, zero_ckpt_info *info,
                              zero_layout *layout, size_t layout_bytes, size_t *bytes_needed);

/* Load rank dst_rank's shard of layout `to` from a checkpoint's n_files shard
 * files (paths[q] must hold rank q's shard; n_files is the saved N),
 * resharding at load time: each element comes from the file and position
 * that hold the same stream position in the saved layout (as zero_reshard),
 * padding is zero.  Only the byte runs the destination needs are read.
 * verify != 0 checks every file's CRC-32C first.  master / exp_avg /
 * exp_avg_sq: host arrays of to->shard floats; *step (may be NULL) receives
 * the saved step count.  EINVAL (bad arguments, files out of rank order or
 * of another N, a destination layout with another element count), EIO,
 * ECORRUPT.  Every file is opened and checked before the first byte of the
 * destination is written; a read that fails after that (EIO) leaves the
 * destination partly filled. */
zero_status zero_ckpt_load(const char *const *paths, int32_t n_files, const zero_layout *to,
                           int32_t dst_rank, int32_t verify, int32_t *step, float *master,
                           float *exp_avg, float *exp_avg_sq);

/* ------------------------------------------------------------------------
 * Ledger -- [p4 section 3]: model state is (2 + 2 + K) psi bytes with K = 12
 * (bf16 params 2, bf16 grads 2, fp32 master + m + v 12); [p4 section 4]:
 * stage 1 shards the optimizer state, stage 2 also the gradients, stage 3
 * also the parameters; communication per step is 2 psi elements for stages
 * 0-2 and 3 psi for stage 3, times (N-1)/N for ring collectives [p3 section
 * 2]; [p3 section 4]: with bucketed reduce-scatter the gradients are
 * transient and drop out of the resident ledger; [p1 Complexity and
 * constants]: ZeRO-3 needs about two units of gathered bf16 weights.
 * ------------------------------------------------------------------------ */

typedef struct zero_ledger_out {
    double params_bytes;        /* bf16 working parameters held per GPU */
    double grads_bytes;         /* bf16 gradients held per GPU (0 if transient) */
    double optim_bytes;         /* fp32 master + m + v held per GPU */
    double model_state_bytes;   /* the sum of the three */
    double comm_elements;       /* 2 psi (stages 0-2) or 3 psi (stage 3) */
    double comm_elements_ring;  /* the same times (N-1)/N */
    double optimizer_floats_per_rank;  /* 3 psi / N floats (master, m, v) for stages >= 1, 3 psi for 0 */
} zero_ledger_out;

/* EINVAL: psi < 0, N < 1, stage outside 0..3, NULL out. */
zero_status zero_ledger(double psi, int32_t n_ranks, int32_t stage, int32_t grads_transient,
                        zero_ledger_out *out);

/* Device memory the one-GPU simulation of the step keeps resident -- [p4
 * section 3]: per element, 2 bytes of bf16 gradient, 12 bytes of fp32 master
 * + m + v and 2 bytes of bf16 parameters, applied to the simulation's own
 * buffers rather than to one model replica: n_grads gradient buffers over the
 * grad_index space (2 bytes per element for ZERO_BF16, 4 for ZERO_F32),
 * master, m and v over the state_index space, the bf16 output over the
 * out_index space (if with_out) and the clipped step's reduced fp32 gradient
 * over the state_index space (if with_g).  Extents: P^ elements for
 * ZERO_GLOBAL, S for ZERO_LOCAL.  N simulated ranks' bf16 gradients with
 * every buffer GLOBAL hold (2N + 14) P^ bytes; one rank's LOCAL shard (2N +
 * 14) S.  Workspaces (norm partials, staged chunk) are not counted.  Host
 * only.  EINVAL: bad layout, n_grads < 1, bad dtype or index, NULL out. */
typedef struct zero_footprint_out {
    double grads_bytes;
    double state_bytes;
    double out_bytes;
    double g_bytes;
    double total_bytes;
} zero_footprint_out;

zero_status zero_sim_footprint(const zero_layout *layout, int32_t n_grads, int32_t grad_dtype,
                               int32_t grad_index, int32_t state_index, int32_t out_index,
                               int32_t with_out, int32_t with_g, zero_footprint_out *out);

/* Overlap condition of one FSDP unit -- [p1 Complexity and constants]: the
 * unit's all-gather, 2 psi_unit (N-1)/N bytes of bf16 weights received per
 * rank, takes gather_bytes / busbw; it is hidden behind the unit's compute,
 * 6 psi_unit flops per token (forward + backward) for tokens_per_gpu tokens at
 * flops_per_s, when gather_s <= compute_s.  EINVAL: negative or zero rates,
 * N < 1, NULL out. */
typedef struct zero_overlap_out {
    double gather_bytes;
    double gather_s;
    double compute_flops;
    double compute_s;
    double ratio;      /* gather_s / compute_s */
    int32_t hidden;    /* 1 if gather_s <= compute_s */
    int32_t reserved;
} zero_overlap_out;

zero_status zero_overlap(double psi_unit, int32_t n_ranks, double busbw_bytes_per_s,
                         double tokens_per_gpu, double flops_per_s, zero_overlap_out *out);

/* ZeRO-3 gather working set: `units_in_flight` units of bf16 weights of the
 * largest unit of the layout (bytes). */
zero_status zero_gather_buffer_bytes(const zero_layout *layout, int32_t units_in_flight,
                                     double *bytes);

/* Algorithmic HBM bytes one zero_step call moves, and the elements it
 * processes: n_grads * grad_size (reads) + 12 (master, m, v reads) + 12
 * (writes) + 2 (bf16 out, if with_out) per processed element. */
zero_status zero_step_traffic(const zero_layout *layout, int32_t rank, int32_t n_grads,
                              int32_t grad_dtype, int32_t with_out,
                              double *bytes, int64_t *elements);

/* Algorithmic bytes of one zero_gradnorm call: n_grads * grad_size reads per
 * element plus 4 bytes written per element when g_out is requested. */
zero_status zero_gradnorm_traffic(const zero_layout *layout, int32_t rank, int32_t n_grads,
                                  int32_t grad_dtype, int32_t with_g_out,
                                  double *bytes, int64_t *elements);

/* ------------------------------------------------------------------------
 * Launch shape.  Every streaming kernel runs one wave64 per workgroup and
 * caps how many are resident per compute unit (through a dynamic LDS
 * reservation the kernels never touch): fewer tiles in flight keep fewer DRAM
 * rows competing, too few starve the memory pipeline.  The defaults were
 * measured on MI355X per kernel family, from the number of streams a wave
 * keeps in flight; these calls let a caller read them and sweep them
 * (bench.py --sweep-waves).  The environment variables
 * ZERO_STEP_WAVES_PER_CU, ZERO_STEP1_WAVES_PER_CU and ZERO_NORM_WAVES_PER_CU
 * (read once) set the same three families.
 *   ZERO_CAP_STEP   the fused step over N gradients
 *   ZERO_CAP_STEP1  the step on one fp32 gradient (the clipped step after
 *                   the norm pass, the staged step's second half)
 *   ZERO_CAP_NORM   the norm pass and the staged step's reduction
 * ------------------------------------------------------------------------ */
#define ZERO_CAP_STEP 0
#define ZERO_CAP_STEP1 1
#define ZERO_CAP_NORM 2

/* Set a family's cap for later launches of this process: waves 1..64, 0 = no
 * cap, -1 = back to the environment / default.  Not ordered with launches on
 * other threads.  EINVAL: bad kind or value. */
zero_status zero_set_waves_per_cu(int32_t kind, int32_t waves);

/* The cap a launch of the family over n_grads bf16 gradients would use now
 * (for ZERO_CAP_STEP1 the clipped step's).  EINVAL: bad kind, n_grads out of
 * 1..ZERO_MAX_RANKS, NULL. */
zero_status zero_get_waves_per_cu(int32_t kind, int32_t n_grads, int32_t *waves);

/* The same for n_grads gradients of grad_dtype (ZERO_BF16 or ZERO_F32) and,
 * when staged is nonzero, for the staged step's kernels: ZERO_CAP_STEP1 its
 * second half (whose default differs from the clipped step's), ZERO_CAP_NORM
 * its reduction (compiled for fewer rank counts than the norm pass); staged
 * does not change ZERO_CAP_STEP.  For 16-byte aligned buffers (the vector
 * kernels).  zero_get_waves_per_cu(kind, n, w) equals
 * zero_get_waves_per_cu_for(kind, n, ZERO_BF16, 0, w).  EINVAL: as
 * zero_get_waves_per_cu, or a bad grad_dtype. */
zero_status zero_get_waves_per_cu_for(int32_t kind, int32_t n_grads, int32_t grad_dtype,
                                      int32_t staged, int32_t *waves);

/* ------------------------------------------------------------------------
 * Diagnostics.
 * ------------------------------------------------------------------------ */

const char *zero_strerror(zero_status status);
/* Text of the last HIP error seen by this thread ("" if none). */
const char *zero_last_hip_error(void);
int32_t zero_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ZERO_H */
