/*
 * zero.h - C ABI of the MI355X (gfx950) ZeRO-2 shard-step library, libzero.so.
 *
 * One data-parallel rank's ZeRO-2 optimizer step, as described on the page
 * "ZeRO and FSDP: partitioning the optimizer states, the gradients and the
 * parameters" (AI infra handbook), section "Implementing ZeRO's Adam from
 * scratch" (class ZeroAdam), and in lesson "9. ZeRO Stage 1 and 2", section
 * "Know this" (stage 2 partitions optimizer state and gradients):
 *
 *   flatten   the tensor list into one vector of shard*world elements,
 *             zero-padded at the end;
 *   reduce    the world data-parallel gradient copies onto this rank's slice
 *             (sum in rank order 0..world-1, then divide by world);
 *   Adam      with bias correction on the fp32 master/m/v slice;
 *   write     the updated slice into the flat parameter buffer (this rank's
 *             all-gather contribution), as bf16 or fp32.
 *
 * Conventions for every function:
 *   - The return value is a status: ZERO_OK (0) or a negative ZERO_E* code.
 *     No function throws, aborts or exits. On failure, zero_last_error()
 *     returns a message for the calling thread.
 *   - Argument checks run before any device work; a call that fails a check
 *     has launched nothing and changed nothing.
 *   - "device pointer" means memory on the device the context was created
 *     on (hipMalloc or a torch CUDA/HIP tensor's storage); "host array" means
 *     ordinary host memory that is read during the call only.
 *   - Device work is stream-ordered and asynchronous on the hipStream_t the
 *     caller passes (0 = the null stream). A fault inside a kernel surfaces
 *     at the caller's next synchronisation, not as a return code here.
 *   - Element counts are int64: shards of more than 2^31 elements are fine.
 *   - Device pointers need only bf16 (2-byte) or fp32 (4-byte) natural
 *     alignment. The step runs 16-byte vectors whatever the buffers'
 *     offsets, after a head of at most 63 elements that puts the streams on
 *     128-byte lines where they share a phase, and shards or ranges shorter
 *     than about 16 elements run element by element. The state sits at the
 *     phase that element lo has in a full flat buffer starting on a 128-byte
 *     line; a slice-only buffer stored at that phase (lo mod 64 bf16, or
 *     lo mod 32 fp32, elements past a line) keeps every stream on whole
 *     lines. Buffers at other 16-byte phases take a shifted path: on the
 *     7e9-element shard at N = 8, seven replicas one element off ran at
 *     about 78% of 8 TB/s and one replica with the output three off at
 *     about 75%, against 80-81% with every stream on its lines. Buffers
 *     whose slices start on 4 KiB pages run fastest (each replica 512 bytes
 *     off its page costs about 0.4% of the step).
 *   - The library owns the context and its master/m/v buffers; the caller
 *     owns every pointer it passes, and its streams.
 *   - Output buffers must not overlap any input of the same call (the
 *     kernels assume no aliasing).
 *   - A context is not locked: calls on one context must not run from
 *     several host threads at once. Different contexts are independent.
 */
#ifndef ZERO_SHARD_H
#define ZERO_SHARD_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct zero_ctx zero_ctx;   /* opaque, one per (rank, device) */

typedef enum {
    ZERO_F32 = 0,   /* IEEE binary32, 4 bytes */
    ZERO_BF16 = 1   /* bfloat16 (top half of binary32), 2 bytes */
} zero_dtype;

enum {
    ZERO_OK = 0,
    ZERO_EINVAL = -1,        /* an argument is out of range or null */
    ZERO_ENOMEM = -2,        /* device or host allocation failed */
    ZERO_EHIP = -3,          /* a HIP runtime call failed */
    ZERO_EUNSUPPORTED = -4   /* valid request the library cannot serve */
};

/* Largest world (number of gradient replicas) a step accepts. */
#define ZERO_MAX_WORLD 256

/* Shard geometry, host only ([ZeRO and FSDP], ZeroAdam constructor):
 *   shard  = ceil(numel / world)     elements this rank owns
 *   lo     = rank * shard            first flat index of its slice
 *   padded = shard * world           length of the zero-padded flat vector
 * Any out-pointer may be NULL. EINVAL unless numel >= 1, 1 <= world,
 * 0 <= rank < world. */
int zero_shard_geometry(int64_t numel, int32_t world, int32_t rank,
                        int64_t *shard, int64_t *lo, int64_t *padded);

/* Create a rank's context on the current HIP device: computes the
 * geometry, allocates fp32 master, m and v of `shard` elements each and
 * sets all three to zero (the page's m = v = 0; call zero_load_master to
 * set master). Hyperparameters as in the page's constructor
 * (lr, betas=(beta1, beta2), eps). Synchronous.
 * EINVAL: geometry as above, !(0 < beta1 < 1), !(0 < beta2 < 1), eps < 0,
 * lr or eps not finite, world > ZERO_MAX_WORLD, out == NULL.
 * ENOMEM: device allocation failed. EHIP: no usable device. */
int zero_shard_init(int64_t numel, int32_t world, int32_t rank,
                    double lr, double beta1, double beta2, double eps,
                    zero_ctx **out);

/* Geometry of a context (any out-pointer may be NULL). */
int zero_shard_info(const zero_ctx *ctx, int64_t *shard, int64_t *lo,
                    int64_t *padded);

/* Bytes of optimizer state this rank holds ([ZeRO and FSDP], ZeroAdam's
 * state_bytes: fp32 master, m and v of its elements, 12 bytes each): 12 *
 * shard for the flat layout, 12 * (its rows of every parameter) for the
 * per-parameter layout. Host only. EINVAL: null context or bytes. */
int zero_shard_state_bytes(const zero_ctx *ctx, int64_t *bytes);

/* Change the learning rate used by later steps (schedules). EINVAL if not
 * finite. Host only. */
int zero_set_lr(zero_ctx *ctx, double lr);

/* master[i] = fp32(flat_params[flat_offset + i]) for i < shard, m = v = 0
 * ([ZeRO and FSDP], ZeroAdam constructor: master is a copy of this rank's
 * slice of the flattened parameters). flat_params: device pointer of
 * `dtype` holding at least flat_offset + shard elements; flat_offset = lo
 * for the full padded flat vector, 0 for a buffer holding the slice only.
 * bf16 widens exactly. EINVAL: null pointer, unknown dtype, negative
 * offset, or a buffer shorter than its allocation allows. */
int zero_load_master(zero_ctx *ctx, const void *flat_params, zero_dtype dtype,
                     int64_t flat_offset, hipStream_t stream);

/* Flatten and pad ([ZeRO and FSDP], ZeroAdam._flatten): dst[k] is element
 * k of the concatenation of srcs[0..ntensors) (each contiguous, row-major)
 * for k < numel, and zero for numel <= k < padded. A bit copy: the dtype
 * only fixes the element size. srcs: host array of ntensors device
 * pointers (NULL allowed where numels[t] == 0); numels: host array;
 * dst: device pointer to `padded` elements, which must not overlap any
 * source. EINVAL unless ntensors >= 1, every numels[t] >= 0 and their sum
 * equals the context's numel. */
int zero_flatten(const zero_ctx *ctx, const void *const *srcs,
                 const int64_t *numels, int32_t ntensors, zero_dtype dtype,
                 void *dst, hipStream_t stream);

/* zero_flatten restricted to flat elements [flat_begin, flat_begin +
 * flat_count) of the padded vector (pad included): a window of the flatten,
 * e.g. one gradient bucket, or this rank's slice ahead of the rest. Windows
 * that tile [0, padded) give exactly zero_flatten's result; disjoint
 * windows may run on different streams. Same argument rules as
 * zero_flatten, plus 0 <= flat_begin, 0 <= flat_count, flat_begin +
 * flat_count <= padded (EINVAL otherwise). */
int zero_flatten_range(const zero_ctx *ctx, const void *const *srcs,
                       const int64_t *numels, int32_t ntensors, zero_dtype dtype,
                       void *dst, int64_t flat_begin, int64_t flat_count,
                       hipStream_t stream);

/* The inverse ([ZeRO and FSDP], ZeroAdam.step, the copy of the gathered
 * vector back into each parameter): dsts[t] receives flat elements
 * [off_t, off_t + numels[t]) with off_t the sum of the earlier numels.
 * Same argument rules as zero_flatten; the pad is not read. */
int zero_unflatten(const zero_ctx *ctx, const void *flat, int32_t ntensors,
                   const int64_t *numels, zero_dtype dtype,
                   void *const *dsts, hipStream_t stream);

/* One optimizer step on this rank's slice ([ZeRO and FSDP], ZeroAdam.step):
 *   g      = (sum over q = 0..world-1, in that order, of
 *             fp32(grad_replicas[q][grad_offset + i])) / world
 *   m      = b1*m + (1-b1)*g ;  v = b2*v + (1-b2)*g*g
 *   master = master - lr * (m/(1-b1^t)) / (sqrt(v/(1-b2^t)) + eps)
 *   param_out[param_offset + i] = master, rounded to bf16 (nearest, ties to
 *                                  even) or stored as fp32
 * for every i < shard, all in binary32 with correctly rounded division and
 * square root (the exact operation order is given in the library source).
 * grad_replicas: host array of n_replicas device pointers (replica q =
 * data-parallel rank q's gradient). grad_offset = lo when each replica is a
 * full padded flat vector, 0 when it holds this rank's slice only; the same
 * offset applies to every replica. param_out: device pointer; param_offset =
 * lo for a full flat parameter buffer, 0 for a slice-only one.
 * t >= 1 is the step number used for bias correction (the page's counter,
 * incremented before use). Precondition: the pad elements of the replicas
 * are zero (zero_flatten guarantees it); they are not masked.
 * EINVAL: n_replicas != world, t < 1, NULL pointers, unknown dtypes. */
int zero_step(zero_ctx *ctx, const void *const *grad_replicas,
              int32_t n_replicas, zero_dtype grad_dtype, int64_t grad_offset,
              void *param_out, zero_dtype param_dtype, int64_t param_offset,
              int64_t t, hipStream_t stream);

/* The step of zero_step restricted to shard elements [shard_begin,
 * shard_begin + count), for gradients that arrive in buckets ([ZeRO and
 * FSDP], the note after the 4-process test: real ZeRO-2 reduce-scatters
 * bucket by bucket during the backward pass and frees each full-gradient
 * bucket once it has gone out). Element shard_begin + i of the state is
 * updated from grad_replicas[q][grad_offset + i] and written to
 * param_out[param_offset + i], for i < count, with the same arithmetic, so
 * covering the shard with disjoint ranges gives results bit-identical to
 * one zero_step. Ranges launched on different streams must be disjoint;
 * the library does not order them. Neighbouring ranges running at once
 * write different elements of the same cache lines (state and output), so
 * param_out must be ordinary device memory (hipMalloc, torch): an output
 * from hipExtMallocWithFlags(..., hipDeviceMallocContiguous) was seen to
 * lose such writes when the library's own state lived there. Any range
 * start takes the vector path after a head of at most 63 elements.
 * EINVAL: as zero_step, plus shard_begin < 0, count < 0 or
 * shard_begin + count > shard. count == 0 is a no-op. */
int zero_step_range(zero_ctx *ctx, int64_t shard_begin, int64_t count,
                    const void *const *grad_replicas, int32_t n_replicas,
                    zero_dtype grad_dtype, int64_t grad_offset,
                    void *param_out, zero_dtype param_dtype,
                    int64_t param_offset, int64_t t, hipStream_t stream);

/* Cap the workgroups of later flat-layout steps (zero_step,
 * zero_step_range and their scheduled forms) at per_cu times the device's
 * compute units; 0 (the default) removes the cap. Uncapped, the fused step
 * makes one pass over its range with one workgroup per 512-element block
 * and fills every compute unit, so kernels on other streams (a backward
 * pass's GEMMs next to gradient buckets, [ZeRO and FSDP], the note after
 * the 4-process test) only start as it drains. Capped, each workgroup walks
 * blocks at a stride of the cap, leaving room on every compute unit; the
 * results are bit-identical (the update is elementwise). Host only; EINVAL
 * unless 0 <= per_cu <= 64. */
int zero_set_step_workgroups(zero_ctx *ctx, int32_t per_cu);

/* ---- Per-parameter (dim-0) layout ------------------------------------
 * [ZeRO and FSDP], section "ZeRO-3 and FSDP": FSDP2 keeps every parameter
 * as a tensor partitioned along dimension 0, and the optimizer acts on the
 * local pieces, so its state is partitioned the same way. Rank r holds
 * rows [r*c, min((r+1)*c, dim0)) of a parameter with dim0 rows, where
 * c = ceil(dim0 / world); trailing ranks may hold fewer rows or none. */

/* Largest world the per-parameter layout accepts. */
#define ZERO_FSDP_MAX_WORLD 16

/* This rank's rows of a dim0-row parameter (host only). Out-pointers may be
 * NULL. EINVAL unless dim0 >= 0, world >= 1, 0 <= rank < world. */
int zero_dim0_split(int64_t dim0, int32_t world, int32_t rank,
                    int64_t *first_row, int64_t *rows);

/* Context for `ntensors` parameters, parameter k having dim0[k] rows of
 * row_numel[k] elements (row-major). The library allocates fp32 master, m
 * and v for this rank's rows of every parameter, concatenated in order with
 * each piece starting on a multiple of 32 elements (a 128-byte line), all
 * zero.
 * zero_shard_info reports the state length as `shard` (lo = 0).
 * zero_get_state / zero_set_state / zero_set_lr / zero_destroy apply;
 * the flat-layout calls (zero_load_master, zero_flatten, zero_unflatten,
 * zero_step, zero_step_range) return EINVAL on this context.
 * EINVAL: ntensors < 1, a dim0 < 0 or row_numel < 1, bad rank/world or
 * hyperparameters (as zero_shard_init). EUNSUPPORTED: world >
 * ZERO_FSDP_MAX_WORLD. ENOMEM / EHIP as zero_shard_init. Synchronous. */
int zero_fsdp_init(int32_t ntensors, const int64_t *dim0,
                   const int64_t *row_numel, int32_t world, int32_t rank,
                   double lr, double beta1, double beta2, double eps,
                   zero_ctx **out);

/* Parameter k's local rows and the offset of its piece in master/m/v. */
int zero_fsdp_local(const zero_ctx *ctx, int32_t k, int64_t *first_row,
                    int64_t *rows, int64_t *state_offset);

/* master = fp32(this rank's rows of each full parameter), m = v = 0.
 * params: host array of ntensors device pointers to the full parameters of
 * `dtype` (NULL allowed for parameters of which this rank holds no rows). */
int zero_fsdp_load_master(zero_ctx *ctx, const void *const *params,
                          zero_dtype dtype, hipStream_t stream);

/* One step on every local piece, with the arithmetic of zero_step: for
 * each parameter k and each of its local elements, the gradient is the
 * mean over replicas q (in rank order) of replica q's full gradient of k
 * at that element; the updated master is written to params_out[k] (this
 * rank's rows only, bf16 or fp32). grads: host array of n_replicas *
 * ntensors device pointers, replica-major (grads[q * ntensors + k] is
 * replica q's full gradient of parameter k). params_out: host array of
 * ntensors device pointers (NULL allowed where this rank holds no rows).
 * EINVAL: not a per-parameter context, n_replicas != world, t < 1, null or
 * misaligned pointers, ranges past their allocations. */
int zero_fsdp_step(zero_ctx *ctx, const void *const *grads, int32_t n_replicas,
                   zero_dtype grad_dtype, void *const *params_out,
                   zero_dtype param_dtype, int64_t t, hipStream_t stream);

/* ---- Device-resident step schedule (graph-replayable steps) ----------
 * The step count t and the learning rate can live in device memory, so a
 * captured HIP graph of a step replays as successive steps ([ZeRO and
 * FSDP], "Implementing ZeRO's Adam from scratch": ZeroAdam keeps its own
 * step count and increments it on every step). The scheduled calls below
 * take t and lr from the device instead of their arguments; their
 * arithmetic, and so their results, equal zero_step's at that t and lr bit
 * for bit: the bias corrections come from a table the library builds on
 * the host at zero_schedule_init exactly as it forms them for a host t.
 * Between zero_schedule_init and zero_destroy the scheduled calls launch
 * kernels only (no allocation, no memset, no host synchronisation), so
 * they can be recorded by HIP stream capture. Scheduled calls on one
 * context must be ordered among themselves (one stream, or events between
 * streams): every zero_step_begin advances the same device counter and
 * rewrites the same block of scalars. */

/* Longest bias-correction table (in steps) the schedule accepts; betas for
 * which 1 - b^t has not reached 1 in binary32 by then are EUNSUPPORTED. */
#define ZERO_SCHEDULE_MAX_TABLE (1 << 22)

/* Create the schedule if the context has none (device allocation and a
 * synchronous upload: not capturable), then set, stream-ordered, the next
 * step count to next_t and the device learning rate to the context's lr.
 * EINVAL: next_t < 1. EUNSUPPORTED: see ZERO_SCHEDULE_MAX_TABLE. */
int zero_schedule_init(zero_ctx *ctx, int64_t next_t, hipStream_t stream);

/* zero_schedule_init for callers that cannot allocate device memory
 * (code under HIP stream capture, tight serving loops, harnesses that
 * forbid hipMalloc): the schedule lives in a static block of 2 MiB that
 * the library holds on each device it runs on until the process ends,
 * instead of an allocation per context. The call allocates nothing and
 * waits for nothing: it fills the bias-correction table with kernels on
 * `stream` and sets the next step to next_t and the device lr to the
 * context's lr, stream-ordered. Scheduled calls then behave exactly as
 * with zero_schedule_init, bit for bit.
 * One block per device: a later zero_schedule_init_noalloc by another
 * context on the same device takes the block over, and this context's
 * scheduled calls then return EINVAL until it is initialised again (with
 * either call). Calls that use the block from several streams or contexts
 * at once race. The block keeps the last call's contents: a scheduled
 * range step before the first begin-step after this call returns EINVAL.
 * Limit: the table holds at most 262,080 steps (betas whose 1 - b^t has
 * not reached 1 in binary32 by then return EUNSUPPORTED; b2 = 0.9999 needs
 * 180,210). EINVAL: null context, next_t < 1. EHIP: a launch failed. */
int zero_schedule_init_noalloc(zero_ctx *ctx, int64_t next_t,
                               hipStream_t stream);

/* Set the learning rate of later scheduled steps (stream-ordered; also the
 * context's host lr). A captured graph takes the lr the device holds when
 * it replays. EINVAL: no schedule, lr not finite. */
int zero_schedule_lr(zero_ctx *ctx, double lr, hipStream_t stream);

/* Read back the next step count (waits for `stream`; not capturable), for
 * checkpoints. EINVAL: no schedule or null output. */
int zero_schedule_get(const zero_ctx *ctx, int64_t *next_t, hipStream_t stream);

/* Begin the schedule's next step: resolve its scalars on the device and
 * advance the step count by one. One single-lane kernel. */
int zero_step_begin(zero_ctx *ctx, hipStream_t stream);

/* zero_step_begin followed by zero_step at the step just begun. Arguments,
 * checks and errors as zero_step, without t; EINVAL also without a
 * schedule. */
int zero_step_sched(zero_ctx *ctx, const void *const *grad_replicas,
                    int32_t n_replicas, zero_dtype grad_dtype,
                    int64_t grad_offset, void *param_out,
                    zero_dtype param_dtype, int64_t param_offset,
                    hipStream_t stream);

/* zero_step_range at the schedule's current step (the one the last
 * zero_step_begin began); covering the shard with disjoint ranges after
 * one zero_step_begin equals one zero_step_sched. The ranges read the
 * scalars zero_step_begin wrote: a range on another stream must be ordered
 * after that zero_step_begin (e.g. by an event), and must have finished
 * before the next zero_step_begin runs. EINVAL as zero_step_range, and
 * also while no step has begun on this context's schedule (no
 * zero_step_begin, zero_step_sched or zero_fsdp_step_sched issued since
 * zero_schedule_init created it): the scalar block then holds no step. */
int zero_step_range_sched(zero_ctx *ctx, int64_t shard_begin, int64_t count,
                          const void *const *grad_replicas,
                          int32_t n_replicas, zero_dtype grad_dtype,
                          int64_t grad_offset, void *param_out,
                          zero_dtype param_dtype, int64_t param_offset,
                          hipStream_t stream);

/* zero_step_begin followed by zero_fsdp_step at the step just begun. */
int zero_fsdp_step_sched(zero_ctx *ctx, const void *const *grads,
                         int32_t n_replicas, zero_dtype grad_dtype,
                         void *const *params_out, zero_dtype param_dtype,
                         hipStream_t stream);

/* Copy the fp32 state out of / into the context (checkpoint and resume):
 * the master copy of this rank's slice and the two moments that [ZeRO and
 * FSDP], ZeroAdam constructor, creates per rank (master = the slice of the
 * flat parameters, m = v = 0). The step count is the caller's (the t of
 * zero_step) or the schedule's (zero_schedule_get / zero_schedule_init).
 * master, m, v: device pointers to `shard` floats each; any may be NULL to
 * skip that buffer. Stream-ordered device-to-device copies. EINVAL: null
 * context, or a buffer shorter than `shard` floats within its allocation. */
int zero_get_state(const zero_ctx *ctx, float *master, float *m, float *v,
                   hipStream_t stream);
int zero_set_state(zero_ctx *ctx, const float *master, const float *m,
                   const float *v, hipStream_t stream);

/* Model-state bytes per card for `numel` parameters and data-parallel
 * degree `world` under mixed-precision Adam ([ZeRO and FSDP], table "The
 * three stages"): stage 0 (plain data parallelism) 16*numel; 1: 4*numel +
 * 12*numel/world; 2: 2*numel + 14*numel/world; 3: 16*numel/world.
 * EINVAL for another stage, numel < 0, world < 1 or bytes == NULL. */
int zero_state_bytes(int32_t stage, double numel, double world, double *bytes);

/* Release the context and its device buffers (synchronises the device
 * first). NULL is ignored. */
void zero_destroy(zero_ctx *ctx);

/* Message describing this thread's most recent failure ("" if none). The
 * string stays valid until the next call on this thread. */
const char *zero_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ZERO_SHARD_H */
