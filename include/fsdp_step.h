/*
 * fsdp_step.h -- C ABI of librank_step.so: one data-parallel rank's share of an
 * FSDP FULL_SHARD (ZeRO-3) training step on an AMD Instinct MI355X (gfx950).
 *
 * The rank's work between the backward reduce-scatter and the next forward
 * all-gather, as the pages describe it:
 *   1. fsdp_shard_layout      where the rank's 1/N shard of each parameter lies
 *   2. fsdp_reduce_grad_shard the fp32 mean of the N gradient slices of that shard
 *   3. fsdp_adamw_shard_step  decoupled-weight-decay AdamW on the shard only
 *   4. fsdp_cast_unshard_bf16 the updated shard cast to bf16, into the buffer the
 *                             next all-gather reads
 * plus a multi-tensor plan (fsdp_mt_*) that runs 2+3+4 fused, in one pass over
 * memory, for many per-parameter shards in a single kernel launch.
 *
 * Page citations use the pages' titles:
 *   [FSDP ch.18]   "PyTorch 训练框架内核深度解析 -- 第18章 FSDP：ZeRO 风格的参数分片"
 *   [ZeRO post]    NCCL ZeRO / FSDP state sharding (blog.cptz.space)
 *   [FSDP2 doc]    "PyTorch FSDP2 后端特性介绍" (MindSpeed-LLM docs)
 *   [titan FSDP2]  torchtitan FSDP2 / HSDP / meta-init article (gsyq.cn)
 *
 * Conventions for every call:
 *   - Return value: FSDP_OK (0) or a negative FSDP_E_* code; on error
 *     fsdp_last_error() gives a message (thread-local, valid until the next
 *     failing call on the same thread).  Nothing aborts, nothing throws: a
 *     host allocation that fails returns FSDP_E_CAPACITY.
 *   - All arguments are checked on the host before any device work is queued.
 *   - Device pointers are plain HIP device addresses on the current device.
 *     The caller owns every buffer it passes; the library never allocates or
 *     frees them (a plan allocates only its own tables, from the
 *     stream-ordered allocator, see fsdp_mt_plan_create).
 *   - Work is queued on the caller's stream (NULL = the null stream) and is
 *     asynchronous; no call synchronises the host except fsdp_mt_plan_create
 *     (one upload) and fsdp_mt_plan_destroy (which waits for the plan's own
 *     last launch, and for nothing else).
 *   - Sizes and offsets are in elements unless a name says bytes.
 *   - Padding: positions [valid, shard_numel) of every buffer the call writes
 *     are set to +0.0 (all-zero bits); inputs are never read there.  NaN and
 *     Inf in inputs are not errors: they propagate per IEEE 754.
 *   - Floating point: fp32 with IEEE-correct division and square root, no
 *     flush of denormals.  Results are deterministic run to run (no atomics).
 *   - Speed, not correctness: every call streams in 16-byte vectors when the
 *     fp32 buffers it streams are 16-byte aligned: grad_shard_out for
 *     fsdp_reduce_grad_shard and fsdp_reduce_sqnorm_noalloc; param_fp32,
 *     exp_avg and exp_avg_sq for fsdp_adamw_shard_step; param_fp32 for
 *     fsdp_cast_unshard_bf16; acc for fsdp_grad_accumulate; for a plan, the
 *     rule given at fsdp_mt_tensor.  Gradient slices, the gradient read by
 *     fsdp_adamw_shard_step, micro-batch gradients and bf16/fp8 copies may
 *     start at any element.  Otherwise the call runs element by element,
 *     bit-identical.
 *   - Resources: the streaming kernels run one wave64 per workgroup and,
 *     except the fp8 code pass, reserve up to 36 KB of LDS per workgroup that
 *     they never touch.  The reservation caps how many of their workgroups
 *     share a compute unit (4 to 16, from the bytes the launch moves per
 *     element), which is where HBM serves their read/write mix best; kernels
 *     running concurrently on the same CUs have that much less LDS.  A
 *     compute-bound kernel on another stream progresses at a small fraction
 *     of its solo rate while a large step runs, with the cap or without it:
 *     the step's waves hold the CUs either way.
 */
#ifndef FSDP_STEP_H
#define FSDP_STEP_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

struct ihipStream_t;
typedef struct ihipStream_t* hipStream_t; /* the HIP stream handle type */

enum {
    FSDP_OK = 0,
    FSDP_E_ARG = -1,      /* null pointer, negative size, value out of range */
    FSDP_E_DTYPE = -2,    /* unknown dtype, or mixed dtypes in one flat unit */
    FSDP_E_ALIGN = -3,    /* pointer not aligned to its element size */
    FSDP_E_ALIAS = -4,    /* a written buffer overlaps another buffer of the call */
    FSDP_E_HIP = -5,      /* a HIP runtime call or kernel launch failed */
    FSDP_E_CAPACITY = -6, /* a size exceeds what the call supports */
    FSDP_E_STATE = -7     /* plan used on a device other than the one it was made on */
};

typedef enum { FSDP_DT_F32 = 0, FSDP_DT_BF16 = 1 } fsdp_dtype;
typedef enum { FSDP_LAYOUT_FLAT = 0, FSDP_LAYOUT_SHARD0 = 1, FSDP_LAYOUT_OWNER = 2 } fsdp_layout_mode;

/* Message of the last failing call on this thread ("" if none). */
const char* fsdp_last_error(void);

/* ------------------------------------------------------------------ layout */

/* One original parameter: total element count, size of dim 0 (a 0-d tensor
 * is numel=1, dim0=1; numel must be a multiple of dim0 when numel > 0), and
 * its dtype (fsdp_dtype). */
typedef struct {
    int64_t numel;
    int64_t dim0;
    int32_t dtype;
    int32_t reserved; /* must be 0 */
} fsdp_tensor_shape;

/* Where one parameter's data lies on one rank.
 *   shard_numel    length of the local buffer holding it (FLAT: the rank's
 *                  whole flat shard S; SHARD0: ceil(dim0/N) rows)
 *   valid          leading elements of that buffer that are real data; the
 *                  rest, [valid, shard_numel), is zero padding
 *   global_offset  offset of the parameter in the unpadded concatenation of
 *                  all parameters in the order given
 *   view_offset    where its local piece starts in the rank's local storage
 *                  (FLAT: in the flat shard; SHARD0: in the concatenation of
 *                  the rank's shards in the order given)
 *   view_numel     elements of the parameter the rank holds (may be 0)
 *   tensor_offset  index, in the flattened parameter, of the first one held
 *   owner          OWNER mode: the rank that holds and updates the whole
 *                  parameter; -1 in the other modes (every rank holds a piece)
 * For an empty FLAT view, with lo = max(global_offset, rank*S):
 * view_offset = min(lo - rank*S, S), tensor_offset = min(lo - global_offset, numel).
 * In OWNER mode a parameter the rank does not own has shard_numel = valid =
 * view_numel = tensor_offset = 0 and view_offset = where it would be packed. */
typedef struct {
    int64_t shard_numel, valid, global_offset, view_offset, view_numel, tensor_offset;
    int64_t owner;
} fsdp_shard_view;

/* Per-rank totals.  logical_numel: sum of numel; physical_numel: padded
 * element count over all N ranks; shard_numel / pad_numel: this rank's local
 * elements and the padding among them; bytes_param: local parameter bytes in
 * the parameters' dtypes; bytes_grad: the fp32 reduced-gradient shard;
 * bytes_optim: exp_avg + exp_avg_sq (fp32); bytes_master: fp32 master copy
 * (0 when has_master is 0).  All per rank, padding included.
 * bytes_grad_unsharded: the fp32 gradient a rank holds while it accumulates
 * micro-batches without reducing ([FSDP ch.18] §18.26 no_sync /
 * set_requires_gradient_sync(False), §18.39: the unsharded gradient is the
 * full size, N times the sharded one): the padded flat vector in FLAT mode,
 * the full parameters in SHARD0 mode. */
typedef struct {
    int64_t logical_numel, physical_numel, shard_numel, pad_numel;
    int64_t bytes_param, bytes_grad, bytes_optim, bytes_master;
    int64_t bytes_grad_unsharded;
} fsdp_layout_summary;

/* Shard layout of `rank` among `world_size` ranks.  Host only: no device
 * work, deterministic, thread-safe.
 *
 * FSDP_LAYOUT_FLAT -- [FSDP ch.18] §18.12 FlatParameter: the parameters are
 *   flattened and concatenated in the order given into one vector of P
 *   elements, which must share one dtype (else FSDP_E_DTYPE); [ZeRO post]
 *   section "FlatParameter 与 Padding": it is padded at its end to
 *   N*ceil(P/N) and rank r owns [r*S, r*S+S), S = ceil(P/N); the rank's view
 *   of a parameter may be empty.
 * FSDP_LAYOUT_SHARD0 -- [FSDP2 doc] section "DTensor", [titan FSDP2] §2.3:
 *   each parameter is sharded on its own along dim 0, (d0, ...) ->
 *   (d0/N, ...); when N does not divide d0, every rank gets ceil(d0/N) rows
 *   and the trailing ranks' missing rows are padding.
 * FSDP_LAYOUT_OWNER -- ZeRO-1 (ZeroRedundancyOptimizer), [ZeRO post] "ZeRO-1：
 *   Optimizer State Sharding" and "Optimizer Step 的所有权": whole parameters
 *   are given to owner ranks; only the owner keeps their optimizer state and
 *   updates them (then broadcasts them).  Ownership is balanced by bytes, not
 *   by parameter count (the post lists count-balancing among its mistakes):
 *   parameters in decreasing byte size (ties: lower index first) each go to
 *   the rank with the fewest bytes so far (ties: lower rank).  A rank's owned
 *   parameters are packed whole, in the order given.  Parameters and
 *   gradients stay replicated: bytes_param and bytes_grad count every
 *   parameter; bytes_optim and bytes_master count the owned ones.
 * Byte totals follow [ZeRO post] tables "Canonical ZeRO 状态公式" /
 * "实测状态因子" (stage 3: P/N params, P/N grads, 2P/N optimizer state per
 * rank) and [titan FSDP2] §2.3 (master + moments = 12 bytes per parameter).
 *
 * views_out: caller array of n_tensors records (may be NULL if n_tensors is
 * 0); summary_out may be NULL.  n_tensors may be 0.  Errors: FSDP_E_ARG for
 * a bad mode, world_size < 1, rank outside [0, world_size), negative sizes,
 * numel not a multiple of dim0, nonzero reserved, or int64 overflow;
 * FSDP_E_DTYPE as above.  Outputs are untouched on error. */
int32_t fsdp_shard_layout(int32_t mode, int32_t world_size, int32_t rank,
                          const fsdp_tensor_shape* tensors, int32_t n_tensors,
                          int32_t has_master, fsdp_shard_view* views_out,
                          fsdp_layout_summary* summary_out);

/* Where to place one rank's step buffers in device memory: one allocation of
 * total_bytes, carved into a region per buffer class, each region starting
 * on a region_align (2 MiB) boundary of the allocation, in this order: fp32
 * param, exp_avg, exp_avg_sq; the gradient slices, n_slices rows of
 * slice_stride elements; the bf16 all-gather buffer (bf16_slots slots of
 * shard_numel elements: 1 for this rank's slot alone, world_size for the
 * whole packed buffer, 0 for none); the fp32 stored gradient; the fp8 copy
 * (bytes).  slice_stride is shard_numel rounded up to 64 elements (a
 * 128-byte line for bf16 slices) plus 256 when n_slices > 1, and
 * shard_numel when n_slices is 1.  A shard_numel of the form above is what
 * fsdp_shard_layout's summary gives (its shard_numel); the plan's shards
 * then sit at their view offsets inside each region.
 *
 * Why (a performance rule, not a correctness one; any placement steps the
 * same values): the fused step streams a dozen arrays in lockstep, element k
 * of each at once, so their relative placement on HBM channels and banks
 * sets its speed.  Separate allocations leave it to the allocator: the 7B
 * rank shard's step took 5.34-5.93 ms over such placements on MI355X; carved
 * this way, 5.34-5.45 ms in every placement measured, and with slice rows
 * exactly shard_numel apart up to 5.57 ms.
 *
 * Offsets are in bytes from the allocation's start; a buffer class that is
 * absent (bf16_slots 0, grad_out or fp8_out 0) has offset -1.  Host only.
 * Errors: FSDP_E_ARG for shard_numel < 0, n_slices outside [1, 1024],
 * bf16_slots < 0, grad_out or fp8_out not 0 or 1, a null out, or sizes that
 * overflow int64; FSDP_E_DTYPE for an unknown slice dtype.  out is untouched
 * on error. */
typedef struct {
    int64_t total_bytes;        /* bytes of the one allocation */
    int64_t region_align;       /* alignment of every region's start (2 MiB) */
    int64_t slice_stride;       /* elements between consecutive slice rows */
    int64_t param_offset;       /* fp32 [shard_numel] */
    int64_t exp_avg_offset;     /* fp32 [shard_numel] */
    int64_t exp_avg_sq_offset;  /* fp32 [shard_numel] */
    int64_t slices_offset;      /* [n_slices][slice_stride] of the slice dtype */
    int64_t bf16_offset;        /* bf16 [bf16_slots * shard_numel], or -1 */
    int64_t grad_out_offset;    /* fp32 [shard_numel], or -1 */
    int64_t fp8_offset;         /* uint8 [shard_numel], or -1 */
} fsdp_rank_buffers;

int32_t fsdp_rank_buffer_layout(int64_t shard_numel, int32_t n_slices, int32_t slice_dtype,
                                int32_t bf16_slots, int32_t grad_out, int32_t fp8_out,
                                fsdp_rank_buffers* out);

/* ------------------------------------------------------------------ step */

/* AdamW hyperparameters.  step is the 1-based count of this update.
 * Required: all finite, lr >= 0, 0 <= beta1 < 1, 0 <= beta2 < 1, eps >= 0,
 * weight_decay >= 0, step >= 1 (else FSDP_E_ARG).  Derived scalars
 * (1 - lr*wd, lr/(1 - beta1^step), 1/sqrt(1 - beta2^step)) are computed on
 * the host in double (beta^step by binary powering) and rounded to fp32, and
 * reach the kernel by value.  A launch captured into a HIP graph therefore
 * keeps them as they were at capture: every replay applies the captured
 * step's bias corrections and learning rate (a graph captured at step 3 and
 * replayed at step 1000 steps 3.7x too far, with 1/sqrt(1 - beta2^3) = 18.3
 * where 1.0 is due), and nothing reports it.  To step a graph through
 * t = 1, 2, ..., capture the _capturable forms of the step calls, which read
 * the count (and, if asked, the learning rate) from device memory
 * (fsdp_mt_step_capturable and the clipped and fp8 forms), or make the calls
 * eagerly. */
typedef struct {
    double lr, beta1, beta2, eps, weight_decay;
    int64_t step;
} fsdp_adamw_hparams;

/* Reduce the N gradient slices of a shard to their fp32 mean:
 *   grad_shard_out[k] = (x_0[k] + x_1[k] + ... + x_{N-1}[k]) / N,  k < valid
 *   grad_shard_out[k] = +0,                                        k >= valid
 * with x_q[k] = grad_slices[q*slice_stride + k] widened exactly to fp32, the
 * sum taken in fp32 in the order q = 0..N-1 and one correctly rounded
 * division by N.  This is the arithmetic a rank does in a reduce-scatter with
 * reduce_dtype=float32: [FSDP ch.18] §18.3 / §18.6, [ZeRO post] "ZeRO-2
 * 方向：Gradient Sharding", [FSDP2 doc] "混合精度"; the mean (not the sum)
 * per [ZeRO post] "Optimizer Step 的所有权" (replicas step with averaged
 * gradients).
 *   grad_shard_out  device fp32 [shard_numel], written
 *   grad_slices     device [n_slices][slice_stride] of slice_dtype, read in
 *                   [0, valid) of each slice only
 *   n_slices        N >= 1 (1 = already reduced: a copy); at most 1024
 *   slice_stride    elements between slices, >= shard_numel when N > 1
 * The output must not overlap the slices (FSDP_E_ALIAS).  shard_numel = 0 is
 * a no-op. */
int32_t fsdp_reduce_grad_shard(float* grad_shard_out, const void* grad_slices,
                               int32_t slice_dtype, int64_t slice_stride,
                               int32_t n_slices, int64_t shard_numel, int64_t valid,
                               hipStream_t stream);

/* One decoupled-weight-decay AdamW step on the local shard only, in place
 * ([FSDP ch.18] §18.21, [ZeRO post] "FSDP Sharded Optimizer", [FSDP2 doc]
 * "工作原理": each rank updates its own 1/N with its 1/N gradient and state,
 * with no communication).  The optimizer is torch.optim.AdamW
 * ([FSDP ch.18] §18.43); with t = hp->step, for k < valid:
 *   p1 = p*(1 - lr*wd);  m = b1*m + (1-b1)*g;  v = b2*v + (1-b2)*g*g
 *   p  = p1 - (lr/(1-b1^t)) * m / (sqrt(v)/sqrt(1-b2^t) + eps)
 * and p = m = v = +0 for k >= valid.
 *   param_fp32, exp_avg, exp_avg_sq  device fp32 [shard_numel], read/written
 *   grad_shard                       device fp32 [shard_numel], read in [0, valid)
 * The three state buffers must be pairwise disjoint and not overlap the
 * gradient (FSDP_E_ALIAS).  shard_numel = 0 is a no-op. */
int32_t fsdp_adamw_shard_step(float* param_fp32, float* exp_avg, float* exp_avg_sq,
                              const float* grad_shard, int64_t shard_numel, int64_t valid,
                              const fsdp_adamw_hparams* hp, hipStream_t stream);

/* Cast the updated fp32 shard to bf16 into this rank's slot of the next
 * all-gather's input ([FSDP ch.18] §18.6: bf16 on the wire, fp32 master;
 * §18.10: the low-precision cast runs before the all-gather).
 *   out[k] = RNE_bf16(param_fp32[k]) for k < valid, 0x0000 for k >= valid
 * Round to nearest, ties to even; overflow gives +-Inf; NaN gives the quiet
 * NaN 0x7FC0 with the input's sign.
 *   unshard_bf16_out  device bf16 [shard_numel] (e.g. offset rank*S of a
 *                     packed [N*S] all-gather buffer), written
 *   param_fp32        device fp32 [shard_numel], read in [0, valid)
 * The two must not overlap (FSDP_E_ALIAS).  shard_numel = 0 is a no-op. */
int32_t fsdp_cast_unshard_bf16(uint16_t* unshard_bf16_out, const float* param_fp32,
                               int64_t shard_numel, int64_t valid, hipStream_t stream);

/* ------------------------------------------------------------------ multi-tensor */

/* One local shard in a multi-tensor plan.  The plan runs, per element and in
 * one pass over memory: the reduce of fsdp_reduce_grad_shard, the update of
 * fsdp_adamw_shard_step and the cast of fsdp_cast_unshard_bf16 -- with
 * bit-identical results to calling the three in that order.
 *   param_fp32, exp_avg, exp_avg_sq  device fp32 [shard_numel], read/written
 *   grad_slices, slice_stride        as in fsdp_reduce_grad_shard
 *   unshard_bf16_out                 device bf16 [shard_numel] or NULL (no cast)
 *   grad_shard_out                   device fp32 [shard_numel] or NULL (the
 *                                    reduced gradient is not stored)
 *   unshard_fp8_out                  device fp8 codes [shard_numel] or NULL:
 *                                    written only by fsdp_mt_cast_fp8 and
 *                                    fsdp_mt_step_fp8
 *   grad_slice_ptrs                  NULL: slice q starts at grad_slices +
 *                                    q*slice_stride.  Else a host array of
 *                                    n_slices device pointers: slice q starts at
 *                                    grad_slice_ptrs[q], and grad_slices and
 *                                    slice_stride are ignored.  This is the form
 *                                    for N receive buffers that do not share one
 *                                    allocation: in the backward reduce-scatter
 *                                    the rank receives its 1/N of every rank's
 *                                    gradient ([FSDP ch.18] §18.3), and FSDP-2
 *                                    lets a custom reduce-scatter replace the
 *                                    built-in one (§18.5), e.g. one in which the
 *                                    rank reads its slices from its peers' buffers.
 *                                    The plan copies the array; entries may be
 *                                    NULL only when valid is 0, must be aligned
 *                                    to the element size, and are read in
 *                                    [0, valid) only. */
/* Speed, not correctness: a shard streams in 16-byte vectors when
 * param_fp32, exp_avg, exp_avg_sq and grad_shard_out start at the same
 * element phase (address / 4 mod 4): all 16-byte aligned, or all 1-3
 * elements past, when the plan splits off a head of the 1-3 elements before
 * the boundary.  The slices and the bf16 and fp8 copies may start at any
 * element (e.g. slot rank*S of a packed buffer with S not a multiple of 4).
 * A shard whose fp32 buffers disagree runs element by element.  Results are
 * bit-identical either way. */
typedef struct {
    float* param_fp32;
    float* exp_avg;
    float* exp_avg_sq;
    const void* grad_slices;
    int64_t slice_stride;
    uint16_t* unshard_bf16_out;
    float* grad_shard_out;
    int64_t shard_numel;
    int64_t valid;
    uint8_t* unshard_fp8_out;     /* NULL => no fp8 copy (see fsdp_mt_cast_fp8, fsdp_mt_step_fp8) */
    const void* const* grad_slice_ptrs; /* NULL => grad_slices + q*slice_stride */
} fsdp_mt_tensor;

typedef struct fsdp_mt_plan fsdp_mt_plan; /* opaque */

typedef struct {
    int64_t n_tensors;   /* shards in the plan */
    int64_t n_chunks;    /* entries of the chunk-descriptor table */
    int64_t n_blocks;    /* workgroups of a launch through the chunk table (8 per entry; a
                            one-range step launches ceil(total_numel / 256)) */
    int64_t total_numel; /* sum of shard_numel */
    int64_t total_valid; /* sum of valid */
    int64_t chunk_numel; /* elements per chunk (the last of a shard may be shorter) */
    int32_t n_slices;
    int32_t slice_dtype;
    int32_t step_one_range; /* 1: fsdp_mt_step runs the shards as one range (see fsdp_mt_step) */
    int32_t store_policy;   /* fsdp_mt_step's state stores: 0 plain, 1 write-through,
                               2 non-temporal write-through */
} fsdp_mt_plan_info;

/* Build a plan over n_tensors shards sharing N = n_slices and slice_dtype
 * (the multi-tensor "fused optimizer" batching of [FSDP ch.18] §18.12 and
 * §18.43: many parameters per launch instead of one by one).  Copies the
 * records, checks them as the single-shard calls would (no written buffer
 * may overlap any other buffer of any shard in the plan; read-only slices
 * may overlap each other), builds the chunk-descriptor table and uploads it
 * to device memory the plan owns on the current device.  When every
 * non-empty shard has a grad_shard_out the plan also owns one fp64 partial
 * sum per workgroup for fsdp_mt_reduce_sqnorm, and every non-empty plan a
 * 48-byte slot for the scalars of the _capturable calls.  Synchronises
 * `stream` once.  The caller keeps every referenced buffer alive and in
 * place while the plan exists.  n_tensors may be 0 (an empty plan).
 * The plan keeps the byte ranges of its shards' buffers: the further device
 * buffers that the calls on it take (grad_scale, scale_in, amax_ranks and
 * the lr_dev of the _capturable calls as inputs; sqnorm_out, amax_out,
 * scale_out and their step_dev as outputs) are checked against them.  An
 * input may overlap only the read-only gradient slices, an output
 * no buffer of the plan (else FSDP_E_ALIAS, before any work is queued).
 * Errors: as the single-shard calls; FSDP_E_CAPACITY if one launch cannot
 * hold the plan's workgroups (checked before any table is built); FSDP_E_HIP
 * if the upload fails.
 * One plan steps with one set of hyperparameters.  Shards that need others
 * (torch's parameter groups, e.g. no weight decay on norms and biases) go in
 * a plan of their own, one step call per plan.  With the _capturable calls
 * each such plan takes its own step count: every call advances the count it
 * is given, so plans sharing one count would advance it once per plan. */
int32_t fsdp_mt_plan_create(fsdp_mt_plan** plan_out, const fsdp_mt_tensor* tensors,
                            int32_t n_tensors, int32_t n_slices, int32_t slice_dtype,
                            hipStream_t stream);

/* One step over every shard of the plan: exactly one kernel launch on
 * `stream` (none for an empty plan), no host synchronisation.  The plan must
 * be used on the device it was made on (FSDP_E_STATE).  When the shards lie
 * back to back in every buffer (state, copies, stored gradient, slices with
 * one stride), all but the last unpadded, and those that start off a
 * chunk_numel boundary of the whole hold at most 1/256 of its elements, the
 * launch takes them as one range from its arguments instead of through the
 * chunk table (step_one_range in the plan's info).  The elements and their
 * arithmetic are the same either way, so the results are bit-identical;
 * only which workgroups run which tiles may differ, in those few shards.
 * Two steps of one plan on different streams without ordering between them race.  Under HIP
 * graph capture the launch is recorded with hp's derived scalars fixed (see
 * fsdp_adamw_hparams). */
int32_t fsdp_mt_step(fsdp_mt_plan* plan, const fsdp_adamw_hparams* hp, hipStream_t stream);

/* fsdp_mt_step with the step count in device memory, for a HIP graph that
 * replays the step (torch's "capturable" AdamW keeps its count on the device
 * for the same reason).  step_dev: device int64 [1] holding the number of
 * steps taken so far, 0 <= *step_dev < 2^62, not checked on the device.  The
 * call first advances *step_dev by one, then steps with t = the new count:
 * a one-lane launch derives t's scalars on the device, with the host's
 * operations (so the results are bit-identical to fsdp_mt_step with
 * hp->step = t), into a slot the plan owns, and the step launch reads them
 * there.  hp->step is ignored; betas, eps and weight_decay are taken at the
 * call (a captured graph keeps them).
 *   lr_dev  NULL: the learning rate is hp->lr, taken at the call.  Else a
 *           device double [1] read by the one-lane launch, in stream order,
 *           in place of hp->lr (which must still be valid): a learning-rate
 *           schedule for a replayed graph, whose caller writes the step's
 *           rate there before each replay.  The decay factor 1 - lr*wd and
 *           lr/(1 - beta1^t) are then derived from it on the device, so the
 *           results are bit-identical to fsdp_mt_step with hp->lr = *lr_dev.
 *           Finite and >= 0, not checked on the device.  8-byte aligned
 *           (FSDP_E_ALIGN); it may overlap only the plan's read-only
 *           gradient slices and not step_dev (FSDP_E_ALIAS).
 * Two launches, no allocation, no host synchronisation; an empty plan
 * advances the count only (and does not read lr_dev).  The step waits for
 * the one-lane launch: about 6 us more per step than fsdp_mt_step, and about
 * 5 us more per replay of a one-step graph (measured on MI355X, with or
 * without lr_dev), a share only small steps notice.  step_dev must not overlap
 * the plan's buffers (FSDP_E_ALIAS); null is FSDP_E_ARG, misaligned
 * FSDP_E_ALIGN.  Calls on one plan must not overlap (they share the slot). */
int32_t fsdp_mt_step_capturable(fsdp_mt_plan* plan, const fsdp_adamw_hparams* hp,
                                int64_t* step_dev, const double* lr_dev, hipStream_t stream);

/* ------------------------------------------------------------------ clipping */

/* Global gradient-norm clipping across the ranks' shards, [FSDP ch.18] §18.18:
 * each rank takes the sum of squares of its own reduced gradient shard, an
 * all-reduce sums those over the ranks, the square root is the global norm,
 * and every rank scales its own shard by one coefficient.  The page names
 * clip_grad_norm_(max_norm, norm_type=2.0); its formula is taken as torch's:
 * coef = min(1, max_norm / (norm + 1e-6)), g <- g * coef.  A clipped step is
 * two passes over memory (the update needs the global norm first):
 *   fsdp_mt_reduce_sqnorm  slices -> grad_shard_out, and the rank's sum of squares
 *   (all-reduce of the per-rank sums: outside this library)
 *   fsdp_clip_coef         per-rank sums -> norm and coefficient, on the device
 *   fsdp_mt_step_clipped   AdamW + cast from grad_shard_out * coef
 * No host synchronisation anywhere in the sequence. */

/* Pass 1 over every shard of `plan`: write the reduced gradient (as
 * fsdp_reduce_grad_shard) to each shard's grad_shard_out and the rank's sum
 * of its squares to sqnorm_out (device, one fp64).  Squares are exact in fp64
 * and summed in fp64 in a fixed order, so the result is deterministic.  Every
 * non-empty shard of the plan must have a grad_shard_out (else FSDP_E_ARG).
 * Uses the plan's own per-workgroup partial-sum buffer: two calls on one plan
 * must not overlap.  An empty plan writes 0. */
int32_t fsdp_mt_reduce_sqnorm(fsdp_mt_plan* plan, double* sqnorm_out, hipStream_t stream);

/* Global norm and clip coefficient from n_ranks per-rank sums of squares
 * (device fp64 [n_ranks], summed in index order -- the all-reduce's result
 * when n_ranks is 1, or the ranks' own sums when one device holds them all):
 *   norm = sqrt(sum), coef = min(1, max_norm / (norm + 1e-6))
 * coef_out: device fp32 [1]; norm_out: device fp64 [1] or NULL.  A NaN norm
 * gives a NaN coefficient; an infinite norm gives 0.  max_norm must be finite
 * and >= 0, 1 <= n_ranks <= 2^20; outputs must not overlap the input. */
int32_t fsdp_clip_coef(float* coef_out, double* norm_out, const double* sqnorms,
                       int32_t n_ranks, double max_norm, hipStream_t stream);

/* Pass 2: AdamW and the bf16 cast on every shard of `plan`, from the reduced
 * gradient that fsdp_mt_reduce_sqnorm (or fsdp_mt_reduce_accumulate) stored
 * in grad_shard_out, multiplied in fp32 by
 * *grad_scale (device fp32, e.g. fsdp_clip_coef's output).  With a scale of
 * exactly 1 the results are bit-identical to fsdp_mt_step's.  The gradient
 * buffers are read, not written.  One kernel launch. */
int32_t fsdp_mt_step_clipped(fsdp_mt_plan* plan, const fsdp_adamw_hparams* hp,
                             const float* grad_scale, hipStream_t stream);

/* fsdp_mt_step_clipped with the step count (and optionally the learning
 * rate) in device memory, as fsdp_mt_step_capturable: advances *step_dev,
 * then the scaled update at the new count.  step_dev must not overlap
 * grad_scale either. */
int32_t fsdp_mt_step_clipped_capturable(fsdp_mt_plan* plan, const fsdp_adamw_hparams* hp,
                                        int64_t* step_dev, const double* lr_dev,
                                        const float* grad_scale, hipStream_t stream);

/* ------------------------------------------------------------------ gradient accumulation */

/* Gradient accumulation over micro-batches, [FSDP ch.18] §18.26 and §18.39.
 * Synchronised (the default): every micro-batch reduce-scatters and the
 * reduced 1/N gradient accumulates in the shard:
 *   fsdp_mt_reduce_accumulate(plan, 0, ...) on the first micro-batch,
 *   fsdp_mt_reduce_accumulate(plan, 1, ...) on the others,
 *   then fsdp_mt_step_clipped with a scale of 1 (or a clip coefficient).
 * no_sync (set_requires_gradient_sync(False)): each rank accumulates its
 * unsharded gradient in place with fsdp_grad_accumulate, and only the last
 * micro-batch reduce-scatters the sums (which reach this rank as fp32
 * slices for fsdp_mt_step).  Both give the shard sum_k (1/N) sum_q x_{q,k} up
 * to rounding; no_sync holds the full-size gradient (bytes_grad_unsharded of
 * the layout summary, N times the shard) and saves N-1 collectives. */

/* For every shard of `plan`: grad_shard_out = mean of the slices
 * (accumulate = 0) or grad_shard_out + mean of the slices (accumulate = 1;
 * one fp32 add, old + new); the padding stays +0.  sqnorm_out (device fp64
 * [1], or NULL): the rank's sum of squares of the stored values, as in
 * fsdp_mt_reduce_sqnorm, for clipping the accumulated gradient.  Every
 * non-empty shard needs a grad_shard_out.  Calls on one plan must not
 * overlap. */
int32_t fsdp_mt_reduce_accumulate(fsdp_mt_plan* plan, int32_t accumulate, double* sqnorm_out,
                                  hipStream_t stream);

/* In-place accumulation of one micro-batch's unsharded gradient:
 *   acc[k] = acc[k] + x[k]   (accumulate = 1; one fp32 add)
 *   acc[k] = x[k]            (accumulate = 0; exact copy of the widened value)
 * acc: device fp32 [numel], read/written; micro: device [numel] of
 * micro_dtype (fp32 or bf16, widened exactly), read.  They must not overlap.
 * numel = 0 is a no-op. */
int32_t fsdp_grad_accumulate(float* acc, const void* micro, int32_t micro_dtype, int64_t numel,
                             int32_t accumulate, hipStream_t stream);

/* ------------------------------------------------------------------ fp8 all-gather copy */

/* fp8 all-gather copy of the updated shards with a per-tensor scale,
 * [FSDP ch.18] §18.27: an fp8 all-gather moves half the bytes of a bf16 one,
 * but fp8's range is narrow, so every tensor carries its own scale with the
 * quantised data.  The page gives no recipe; the one taken is dynamic
 * per-tensor scaling over the whole tensor (all ranks' shards) in OCP FP8
 * E4M3 ("e4m3fn": bias 7, 3 fraction bits, largest finite 448, no inf):
 *   amax  = max |p| over tensor i on every rank (NaN propagates)
 *   scale = 448 / max(amax, 1e-12)                       (fp32)
 *   code  = RNE_e4m3(clamp(fp32(p * scale), -448, 448)), 0 in the padding
 * A consumer recovers p ~ value(code) / scale.  Sequence:
 *   fsdp_mt_step_amax   the fused step, plus each tensor's local amax of the
 *                       updated parameter (no extra pass over memory)
 *   (all-reduce max of the per-rank amax arrays: outside this library)
 *   fsdp_mt_cast_fp8    reads the updated fp32 shards, writes the codes
 * or, with the scale fixed before the step (delayed scaling: the scale the
 * previous step derived from its amax), in one pass:
 *   fsdp_mt_step_fp8    the fused step writing the codes with the given
 *                       scales, plus this step's amax for the next scales */

/* The step of fsdp_mt_step (same outputs, bit-identical), and for every
 * shard i of the plan, in input order, the largest |p'| of its updated local
 * shard to amax_out[i] (device fp32 [n_tensors]; 0 for an empty shard; NaN if
 * any updated value is NaN).  The plan must have at least one fp8 output.
 * Uses the plan's per-workgroup scratch: calls on one plan must not overlap. */
int32_t fsdp_mt_step_amax(fsdp_mt_plan* plan, const fsdp_adamw_hparams* hp, float* amax_out,
                          hipStream_t stream);

/* fsdp_mt_step_amax with the step count (and optionally the learning rate)
 * in device memory, as fsdp_mt_step_capturable: advances *step_dev, then
 * steps at the new count.  Neither step_dev nor lr_dev may overlap amax_out. */
int32_t fsdp_mt_step_amax_capturable(fsdp_mt_plan* plan, const fsdp_adamw_hparams* hp,
                                     int64_t* step_dev, const double* lr_dev, float* amax_out,
                                     hipStream_t stream);

/* Write every shard's fp8 codes from its updated fp32 parameter.  The amax
 * of shard i is the maximum over r of amax_ranks[r * n_tensors + i] (device
 * fp32 [n_ranks][n_tensors]: the ranks' fsdp_mt_step_amax outputs, or one
 * row that an all-reduce max already combined).  scale_out: device fp32
 * [n_tensors] for the scales, or NULL.  Every non-empty shard must have an
 * unshard_fp8_out (else FSDP_E_ARG).  One kernel launch. */
int32_t fsdp_mt_cast_fp8(fsdp_mt_plan* plan, const float* amax_ranks, int32_t n_ranks,
                         float* scale_out, hipStream_t stream);

/* The step of fsdp_mt_step (same fp32 outputs and bf16 copies,
 * bit-identical), which also writes every shard's fp8 codes in the same pass:
 *   code = RNE_e4m3(clamp(fp32(p' * scale_in[i]), -448, 448)), 0 in the pad
 * and, as fsdp_mt_step_amax does, each shard's largest |p'| to amax_out[i].
 *   scale_in  device fp32 [n_tensors], read: shard i's scale, chosen before
 *             the step (e.g. the scale_out of the previous step's
 *             fsdp_mt_cast_fp8, or 448 / max(amax, 1e-12) of the previous
 *             step's all-reduced amax)
 *   amax_out  device fp32 [n_tensors], written; must not overlap scale_in
 * This is the delayed-scaling reading of [FSDP ch.18] §18.27 (the page fixes
 * neither recipe): values that grew past the previous amax saturate to
 * +-448 until the next scale catches up.  Every non-empty shard must have an
 * unshard_fp8_out (else FSDP_E_ARG).  Two kernel launches (the step and the
 * per-shard amax), none when the plan is empty.  Uses the plan's
 * per-workgroup scratch: calls on one plan must not overlap. */
int32_t fsdp_mt_step_fp8(fsdp_mt_plan* plan, const fsdp_adamw_hparams* hp, const float* scale_in,
                         float* amax_out, hipStream_t stream);

/* fsdp_mt_step_fp8 with the step count (and optionally the learning rate)
 * in device memory, as fsdp_mt_step_capturable: advances *step_dev, then
 * steps at the new count.  step_dev must not overlap scale_in or amax_out
 * either, nor lr_dev amax_out. */
int32_t fsdp_mt_step_fp8_capturable(fsdp_mt_plan* plan, const fsdp_adamw_hparams* hp,
                                    int64_t* step_dev, const double* lr_dev, const float* scale_in,
                                    float* amax_out, hipStream_t stream);

/* ------------------------------------------------------------------ no device allocation */

/* For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  A plan's
 * tables and its per-workgroup partial sums are allocated when the plan is
 * made; this call needs no plan and allocates nothing.
 *
 * Pass 1 of a clipped step for one shard: the reduced gradient, exactly as
 * fsdp_reduce_grad_shard writes it, to grad_shard_out, and the sum of its
 * squares to sqnorm_out (device, one fp64).  Its results are bit-identical
 * to fsdp_mt_reduce_sqnorm's on a plan holding this one shard (same kernel
 * body, same per-workgroup partials, same fixed summation order) when the
 * shard's fp32 buffers of that plan are 16-byte aligned.
 *   grad_shard_out  device fp32 [shard_numel], written (+0 in the padding)
 *   sqnorm_out      device fp64 [1], written (0 for shard_numel = 0)
 *   the slices      as in fsdp_reduce_grad_shard
 * The per-workgroup partial sums live in one fixed device array of the
 * library, FSDP_NOALLOC_SCRATCH_BYTES (1 MiB) on each device, held until the
 * process ends, so shard_numel is at most FSDP_NOALLOC_MAX_NUMEL (else
 * FSDP_E_CAPACITY, nothing queued).  Every call on a device shares that
 * device's array: calls that overlap on one device (different streams
 * without ordering between them, or different host threads) race.  Each
 * call writes every partial it reads, so nothing is cleared between calls.
 * No hipMalloc, hipFree or other allocating call is made; the array's device
 * address is looked up once per device, on the first call there.  Errors:
 * as fsdp_reduce_grad_shard; FSDP_E_ARG for a null sqnorm_out, FSDP_E_ALIGN
 * if it is not 8-byte aligned, FSDP_E_ALIAS if it overlaps the gradient or
 * the slices. */
#define FSDP_NOALLOC_SCRATCH_BYTES (1 << 20)
#define FSDP_NOALLOC_MAX_NUMEL ((int64_t)33292288) /* 16,256 chunk entries of 2048 */
int32_t fsdp_reduce_sqnorm_noalloc(float* grad_shard_out, double* sqnorm_out,
                                   const void* grad_slices, int32_t slice_dtype,
                                   int64_t slice_stride, int32_t n_slices, int64_t shard_numel,
                                   int64_t valid, hipStream_t stream);

/* Sizes of a plan (host only). */
int32_t fsdp_mt_plan_get_info(const fsdp_mt_plan* plan, fsdp_mt_plan_info* info_out);

/* Free a plan's device tables.  Waits until the plan's last launch made
 * outside a HIP graph capture has finished (its completion event is bound to
 * that kernel), and for nothing else on the device: no device-wide
 * synchronisation.  The tables come from the stream-ordered allocator and
 * are freed in stream order after that wait.  Calls on one plan are ordered
 * (they race otherwise), so the last launch finishing means all have.  A HIP
 * graph holding launches of the plan must not be replayed once the plan is
 * destroyed.  NULL is a no-op. */
int32_t fsdp_mt_plan_destroy(fsdp_mt_plan* plan);

#ifdef __cplusplus
}
#endif

#endif /* FSDP_STEP_H */
