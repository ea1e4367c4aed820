/*
 * fp8z1 -- blockwise-FP8 ZeRO-1 shard-local optimizer step for MI355X (gfx950).
 *
 * The operations follow "面向 Blockwise FP8 量化的 ZeRO 优化器设计" (A ZeRO
 * optimizer design for blockwise FP8 quantization, beipo.top/blog/fp8-zero1):
 *   - section "块粒度切分" (block-wise split): params are cut in 128x128
 *     units, each quantized dimension padded to a multiple of 128, and a
 *     lookup table records real sizes and padding  -> fp8z1_build_table
 *   - section "参数粒度切分" (param-wise split): greedy assignment of whole
 *     params to DP buckets, padded to the largest bucket -> split FP8Z1_SPLIT_PARAM
 *   - section "参数布局变换" (layout transform): fold turns row-major weights
 *     into 128x128-block-contiguous order, unfold is the inverse
 *                                                    -> fp8z1_fold, fp8z1_unfold
 *   - section "总结" (the step flow): after the update each rank quantizes
 *     its FP32 master into FP8 weights plus one scale per block -> fp8z1_step
 * and "DeepSpeed ZeRO 优化" (gitcode.csdn.net) for the optimizer-step order
 * (section 3.2), loss scaling (section 6), gradient clipping (section 7) and
 * the overflow check (section 9, Q6).
 *
 * Conventions
 *   - Every call returns an int status: FP8Z1_OK (0) or a negative error.
 *     fp8z1_last_error() gives a detail string for the calling thread.
 *   - Argument errors are found before anything is launched; a failed
 *     launch or HIP runtime error returns FP8Z1_EHIP.
 *   - GPU calls are asynchronous on the caller's stream (`stream` is a
 *     hipStream_t; NULL is the default stream).  Host waits happen only in
 *     fp8z1_state_read / fp8z1_state_write, at the first GPU use of a table
 *     (its plan is uploaded), in fp8z1_table_free, and when a call passes
 *     param pointers that differ from the last call of the same kind (the
 *     library waits for its previous upload of that pointer list).
 *   - Data buffers are caller-owned device memory.  The library owns the
 *     table handle: its host arrays, and (from the first GPU call that uses
 *     it) one device copy of the table plus small device arrays that hold the
 *     per-param pointer lists passed to fold/unfold.  fp8z1_table_free
 *     releases all of it.
 *   - A table is bound to the device current at its first GPU use.  All GPU
 *     calls that use one table must be issued on one stream, or ordered by
 *     the caller; calls on distinct tables are independent and thread-safe.
 *     fp8z1_table_free waits for the table's own pending work (the pointer
 *     list uploads and the kernels of its last uncaptured call) before
 *     releasing, not for the whole device; replays of a captured graph that
 *     uses the table must have finished before it is freed.
 *   - Graph capture: fp8z1_fold, fp8z1_step, fp8z1_step_rowmajor,
 *     fp8z1_unfold, fp8z1_state_init and fp8z1_dequantize only launch
 *     kernels once a table is set up on the device and its pointer lists
 *     are current, so they may be captured into a HIP graph after the same
 *     call (same table, same param pointer arrays) has run once outside the
 *     capture.  A captured call that would need set-up (first device use of
 *     the table, or param pointers that differ from the last call of the
 *     same kind) returns FP8Z1_EINVAL instead.  A replayed graph reads the
 *     table's current pointer lists: a later uncaptured call of the same
 *     kind with other param pointers retargets it, so keep them fixed while
 *     the graph is in use.  Each kind of call has its own lists (fold
 *     sources, step grads, FP8 unfold destinations and scales, FP32 unfold
 *     destinations and scales), so a call of one kind never retargets
 *     another kind's graph.  fp8z1_state_read/state_write synchronize and cannot be captured.
 *   - Rows of row-major arrays may start at any element alignment: kernels
 *     use 16-byte accesses (gfx950 runs in unaligned-access mode) but never
 *     touch a byte outside the block row segment they own.
 *   - Layouts: a param is row-major [E, R, C] (a 2-D param has E = 1).
 *     A folded shard is shard_slots blocks of 128 x 128 elements, each block
 *     row-major, blocks in table order; padding positions are +0.
 */
#ifndef FP8Z1_H
#define FP8Z1_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define FP8Z1_OK 0
#define FP8Z1_EINVAL (-1)  /* bad argument (NULL pointer, out-of-range value) */
#define FP8Z1_ENOMEM (-2)  /* host or device allocation failed */
#define FP8Z1_EHIP (-3)    /* HIP runtime or launch error */
#define FP8Z1_ESHAPE (-4)  /* shape outside the supported limits, or a mismatch */
#define FP8Z1_EDEVICE (-5) /* table used on a device other than the one it is bound to */

/* splits (section "块粒度切分" / "参数粒度切分") */
#define FP8Z1_SPLIT_BLOCK 0
#define FP8Z1_SPLIT_PARAM 1
#define FP8Z1_ALL_RANKS (-1) /* rank value: the table of the whole flat buffer (all ranks' slots) */

/* element types */
#define FP8Z1_F32 0
#define FP8Z1_BF16 1
#define FP8Z1_E4M3 2 /* OCP FP8 E4M3 codes, one byte each */

#define FP8Z1_BLOCK 128 /* block edge */
#define FP8Z1_STAT_PARTS 4 /* float64 partial sums of squares per slot (one per 32 rows) */

/* block scale rules */
#define FP8Z1_SCALE_AMAX 0 /* scale = amax / 448 in float32 (1 if amax = 0) */
#define FP8Z1_SCALE_POW2 1 /* scale = 2^(floor(log2 amax) - 8), an E8M0 power of two kept in
                              [2^-127, 2^119] (1 if amax = 0, +inf if amax = +inf); the block's
                              largest magnitude lands in [256, 512) and saturates at 448 */

typedef struct fp8z1_table fp8z1_table; /* opaque */

typedef struct {
  int64_t E, R, C;
} fp8z1_shape;

/* One slot of a shard, 16 bytes.  param = -1 marks a padding slot (all other
 * fields 0).  Otherwise the slot holds block (brow, bcol) of expert `expert`
 * of param `param`: rows 128*brow .. +vrows and columns 128*bcol .. +vcols are
 * real, the rest of the 128x128 block is padding. */
typedef struct {
  int32_t param;
  int32_t expert;
  uint16_t brow, bcol;
  uint8_t vrows, vcols;
  uint16_t reserved;
} fp8z1_block;

typedef struct {
  int32_t split, dp, rank, n_params;
  int64_t total_blocks;     /* blocks of all params */
  int64_t slots_per_rank;   /* every rank's shard has this many slots */
  int64_t shard_first_slot; /* global index of this shard's first slot */
  int64_t shard_slots;      /* slots in this table (slots_per_rank, or dp*slots_per_rank for FP8Z1_ALL_RANKS) */
  int64_t valid_elems;      /* real elements in this shard */
  int64_t pad_elems;        /* shard_slots*16384 - valid_elems */
} fp8z1_table_info;

/* AdamW / clipping / loss-scaling settings.  Float fields are float32 values;
 * every scalar the step derives from them is computed in float64 and rounded
 * once to float32. */
typedef struct {
  float lr, beta1, beta2, eps, weight_decay;
  float max_grad_norm;     /* <= 0: no clipping; NaN is rejected (FP8Z1_EINVAL) */
  int32_t loss_scaling;    /* 0: off (S = 1) */
  float init_scale;        /* loss scale S at fp8z1_state_init */
  float growth_factor;     /* S *= growth_factor after growth_interval clean steps */
  float backoff_factor;    /* S *= backoff_factor on overflow; with loss_scaling on, both
                              factors must be finite and > 0 (else FP8Z1_EINVAL) */
  int32_t growth_interval;
  int32_t extra_found_inf; /* overflow flag of the other ranks (the all-reduced flag) */
  int32_t scale_rule;      /* FP8Z1_SCALE_AMAX (0) or FP8Z1_SCALE_POW2 (1) */
  double extra_sumsq;      /* sum of squares of the other ranks' grads (the all-reduced sum) */
  /* NULL, or a device pointer to the global float64 sum of squares over all
   * ranks (the all-reduced fp8z1_shard_sumsq outputs), read by the step on
   * the device when it runs; the step then takes no statistics of its own and
   * ignores extra_sumsq (extra_found_inf still applies).  Lets the cross-rank
   * reduction stay on the device, and a captured step see each replay's sum. */
  const double* d_global_sumsq;
} fp8z1_hparams;

/* Optimizer step state, 64 bytes, kept in device memory between steps. */
typedef struct {
  int64_t step;        /* successful (non-skipped) steps t */
  double beta1_pow;    /* beta1^t */
  double beta2_pow;    /* beta2^t */
  double global_sumsq; /* this step's global sum of squares of the (scaled) grads */
  float loss_scale;    /* S for the next step */
  float k;             /* factor applied to the grads at the last update (clip / S) */
  float step_size;     /* lr / (1 - beta1^t) */
  float bc2_sqrt;      /* sqrt(1 - beta2^t) */
  float decay;         /* 1 - lr * weight_decay */
  int32_t good_steps;  /* clean steps since the last scale change */
  int32_t found_inf;   /* 1 if this step overflowed (and was skipped) */
  int32_t skipped_total;
} fp8z1_state;

const char* fp8z1_status_string(int status);
const char* fp8z1_last_error(void);

/* Build the lookup table of rank `rank` of `dp` (or FP8Z1_ALL_RANKS) over
 * `n_params` params (host arrays; host-only call, no GPU needed).
 * Section "块粒度切分": blocks of each param in (expert, block_row,
 * block_col) order, params in the given order; block split = DP equal
 * contiguous ranges of ceil(nblocks/DP) slots, empty slots at the global tail.
 * Section "参数粒度切分": param split = params sorted by block count
 * (descending, ties by id), each to the least loaded bucket (lowest index on
 * ties); a bucket lists its params by ascending id then padding slots up to
 * the largest bucket; bucket r is rank r.
 * Limits: E, R, C >= 1, R and C < 2^23, blocks per param < 2^31.
 * On success *out owns the table (free with fp8z1_table_free). */
int fp8z1_build_table(const fp8z1_shape* shapes, int32_t n_params, int32_t dp, int32_t rank, int32_t split,
                      fp8z1_table** out);
int fp8z1_table_info_get(const fp8z1_table* table, fp8z1_table_info* out);
/* Host view of the shard's shard_slots entries, valid until fp8z1_table_free. */
int fp8z1_table_entries(const fp8z1_table* table, const fp8z1_block** entries);
void fp8z1_table_free(fp8z1_table* table);

/* Fold (section "参数布局变换"): gather the shard's blocks from row-major
 * params into dst (device, shard_slots*16384 float32, 16-byte aligned),
 * widening BF16 to float32 exactly.  src: host array of n_params device
 * pointers to row-major [E,R,C] params of type src_dtype (FP8Z1_F32 or
 * FP8Z1_BF16), aligned to their element size (rows need not be 16-byte aligned);
 * an entry may be NULL if the shard holds no block of that param.  Padding
 * positions and padding slots are written +0.  Used on the FP32/BF16
 * weights at init and on the reduced FP32 grads every step.
 * If slot_sumsq is not NULL (device, 4*shard_slots doubles, 8-byte aligned),
 * the float64 sum of squares of the real elements of each quarter of each
 * slot (rows 32q..32q+31 of slot s at index 4s+q, in a fixed order) is
 * written there as well, in the form fp8z1_step takes as its statistics.
 * With dst NULL (FP32 src, slot_sumsq not NULL) only those sums are taken:
 * the statistics pass over row-major grads that are not folded. */
int fp8z1_fold(const fp8z1_table* table, const void* const* src, int32_t src_dtype, float* dst, double* slot_sumsq,
               void* stream);

/* Write the initial step state (t = 0, S = init_scale or 1) into d_state
 * (device, 64 bytes). */
int fp8z1_state_init(const fp8z1_hparams* hp, fp8z1_state* d_state, void* stream);

/* Bytes of device workspace fp8z1_step needs (the float64 partial sums of
 * squares, one per quarter slot: 32 bytes per slot). */
int fp8z1_step_workspace_bytes(const fp8z1_table* table, size_t* bytes);

/* This shard's float64 sum of squares of its real grads (level 2 of the
 * statistics, in the order the step's finalize uses): the sum of d_partials
 * (device, fp8z1_step_workspace_bytes() bytes written by fp8z1_fold with
 * slot_sumsq) written to d_sum (device, one double).  Clipping across ranks
 * ("DeepSpeed ZeRO 优化" section 7) all-reduces these sums; the reduced value
 * goes to fp8z1_step through hp->d_global_sumsq.  A non-finite grad makes the
 * sum non-finite, and so the reduced sum, which is the overflow test. */
int fp8z1_shard_sumsq(const fp8z1_table* table, const double* d_partials, double* d_sum, void* stream);

/* One optimizer step on the shard (section "总结"; step order of
 * "DeepSpeed ZeRO 优化" section 3.2).  All buffers are device memory laid out
 * as the folded shard: grad/master/m/v shard_slots*16384 float32, fp8
 * shard_slots*16384 bytes, scales shard_slots float32.  (Placement: with
 * grad, master, m and v back to back in one allocation the MoE expert shard's
 * update ran 2 % faster on MI355X than with four separate allocations.)
 *  1. statistics (only if hp->max_grad_norm > 0 or hp->loss_scaling): the
 *     float64 sum of squares of the shard's real grads, plus hp->extra_sumsq
 *     (or the value at hp->d_global_sumsq instead of both);
 *     overflow if that sum is not finite or hp->extra_found_inf is set.
 *     If `presummed` is nonzero, d_workspace already holds the partial sums
 *     from fp8z1_fold(slot_sumsq = d_workspace) of this same grad and the
 *     grad is not read for them again.
 *  2. on overflow: skip (master, m, v, fp8, scales untouched), S *= backoff.
 *     Else k = clip / S with clip = min(1, max_norm / (norm + 1e-6)),
 *     norm = sqrt(sum)/S, and the scalars advance.
 *  3. AdamW on every real element (float32, one rounding per operation):
 *       g = g_raw*k; m = b1*m + (1-b1)*g; v = b2*v + (1-b2)*(g*g);
 *       p = p*decay - step_size*(m / (sqrt(v)/bc2_sqrt + eps))
 *     Padding positions of master, m, v are neither read for the result nor
 *     changed.
 *  4. per slot: amax = max |p| over real elements, scale = amax/448 (1 if
 *     amax = 0; or the power of two of FP8Z1_SCALE_POW2 when hp->scale_rule
 *     asks for it), code = E4M3(p / scale) (round to nearest even,
 *     saturating at 448, NaN kept); padding codes 0; padding slots scale 1.
 * d_workspace: fp8z1_step_workspace_bytes() bytes (may be NULL when no
 * statistics are taken or hp->d_global_sumsq is set).  The state at d_state is updated in place. */
int fp8z1_step(const fp8z1_table* table, const fp8z1_hparams* hp, fp8z1_state* d_state, const float* grad,
               float* master, float* m, float* v, uint8_t* fp8, float* scales, void* d_workspace,
               size_t workspace_bytes, int32_t presummed, void* stream);

/* The same step with the grads read straight from the row-major reduced
 * grads: the fold of section "参数布局变换" happens on read inside the
 * update, and no folded copy of the grads is written.  grads: host array of
 * n_params device pointers to row-major FP32 [E,R,C] grads, 4-byte aligned
 * (NULL allowed for params the shard holds no block of).  With statistics
 * on, a first pass over the same grads writes the partial sums of squares
 * into d_workspace, in the order fp8z1_fold uses.  Results (state, master,
 * m, v, fp8, scales) are bit-identical to fp8z1_fold followed by
 * fp8z1_step. */
int fp8z1_step_rowmajor(const fp8z1_table* table, const fp8z1_hparams* hp, fp8z1_state* d_state,
                        const void* const* grads, float* master, float* m, float* v, uint8_t* fp8, float* scales,
                        void* d_workspace, size_t workspace_bytes, void* stream);

/* fp8z1_step_rowmajor for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  The call allocates nothing: the statistics partials live in a
 * device array of the library (FP8Z1_NOALLOC_MAX_SLOTS * FP8Z1_STAT_PARTS
 * float64 = 8 MiB on each GPU that runs the call, held until the process
 * ends) instead of a caller workspace.  Same arguments, results and errors as
 * fp8z1_step_rowmajor, and bit-identical results, with these limits:
 *   - tables of more than FP8Z1_NOALLOC_MAX_SLOTS slots: FP8Z1_ESHAPE;
 *   - the table must already be set up on the current device (any earlier
 *     GPU call with it, e.g. the init fp8z1_fold of the masters), because
 *     setting it up allocates: else FP8Z1_EINVAL;
 *   - every call on one GPU uses that GPU's one array, which keeps the last
 *     call's partials (each call writes all the partials it reads before it
 *     reads them): calls that may overlap on one GPU (other streams, other
 *     threads, not ordered by the caller) race on it. */
#define FP8Z1_NOALLOC_MAX_SLOTS 262144
int fp8z1_step_rowmajor_noalloc(const fp8z1_table* table, const fp8z1_hparams* hp, fp8z1_state* d_state,
                                const void* const* grads, float* master, float* m, float* v, uint8_t* fp8,
                                float* scales, void* stream);

/* Unfold (section "参数布局变换", and the scale unfold of section "总结"):
 * write the shard's real elements from `folded` (device, shard_slots*16384
 * elements of dtype FP8Z1_E4M3 or FP8Z1_F32) into row-major params.
 * dst: host array of n_params device pointers to [E,R,C] arrays of that
 * dtype (NULL allowed for params the shard does not hold); only the shard's
 * real positions are written.  If scales (device, shard_slots float32) and
 * dst_scales (host array of n_params device pointers to [E,Rb,Cb] float32)
 * are both non-NULL, each slot's scale goes to its block's position. */
int fp8z1_unfold(const fp8z1_table* table, const void* folded, int32_t dtype, const float* scales,
                 void* const* dst, float* const* dst_scales, void* stream);

/* Dequantize row-major FP8 weights (section "Blockwise 量化": one scale per
 * 128x128 block, the scale being the dequantization multiplier):
 * out[e,r,c] = decode(codes[e,r,c]) * scales[e, r/128, c/128], rounded once to
 * float32 and, for out_dtype FP8Z1_BF16, then to bfloat16 (nearest, ties to
 * even; NaN stays NaN).  codes: device [E,R,C] bytes; scales: device
 * [E,ceil(R/128),ceil(C/128)] float32; out: device [E,R,C] of out_dtype
 * (FP8Z1_F32 or FP8Z1_BF16).  For reading back what the gathered FP8 weights
 * stand for. */
int fp8z1_dequantize(const uint8_t* codes, const float* scales, int64_t E, int64_t R, int64_t C, int32_t out_dtype,
                     void* out, void* stream);

/* Copy the device state to the host (synchronizes the stream) / from the host
 * (resume from a checkpoint). */
int fp8z1_state_read(const fp8z1_state* d_state, fp8z1_state* out, void* stream);
int fp8z1_state_write(fp8z1_state* d_state, const fp8z1_state* in, void* stream);

/* The device E4M3 encoder the step uses, over n float32 values (device to
 * device), so it can be checked exhaustively. */
int fp8z1_encode_e4m3(const float* in, uint8_t* out, int64_t n, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FP8Z1_H */
