// Internal interface between the host API (zero_api.hip) and the gfx950
// kernels (zero_kernels.hip). Not installed; callers use include/zero.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/zero.h"

namespace zk {

// Step scalars, each formed in binary64 on the host and rounded once to
// binary32: b1, 1-b1, b2, 1-b2, lr, eps, 1-b1^t, 1-b2^t, world, and 1/world
// (used only when world is a power of two, where x*(1/world) == x/world
// exactly).
struct StepScalars {
    float b1, c1, b2, c2, lr, eps, bc1, bc2, nf, inv_n;
    int n_pow2;
};

// Device-resident step schedule (graph-replayable steps): the step count
// of the next step and the fp32 learning rate, in device memory.
struct DevSchedule {
    int64_t t;
    float lr;
    int32_t pad;
};

// One step over `shard` elements. grads[q] already points at element 0 of
// replica q's slice; out at element 0 of the output slice. With sc_dev
// non-null the kernels read their scalars from that device address
// (written by launch_begin_step) and `sc` is unused.
struct StepArgs {
    const void *const *grads;   // host array, n entries
    int n;
    bool grad_bf16;
    float *master, *m, *v;      // library buffers, 256-byte aligned
    void *out;
    bool out_bf16;
    int64_t shard;
    StepScalars sc;
    const StepScalars *sc_dev;
    int num_cus;
    // Non-temporal hints on master/m/v in the vector path. Set when the
    // context's whole state, not just this launch's range, is larger than
    // the Infinity Cache: it cannot stay cached from one step to the next.
    bool stream_state;
    // Cap on the workgroups that take the vector path's full blocks (0: one
    // per block, a single pass). A capped launch leaves room on every CU
    // for work on other streams; each workgroup then walks the blocks at a
    // stride of the cap, with the same per-element arithmetic.
    int64_t max_workgroups;
    // Non-temporal hints on the replica loads of the vector path (set by
    // the launcher from the streams' alignment).
    bool nt_grad;
};
// MI355X's last-level (Infinity) cache in front of HBM.
constexpr int64_t kInfinityCacheBytes = (int64_t)256 << 20;
// Whether a state of `elems` fp32 master/m/v elements is streamed.
inline bool state_streams(int64_t elems) { return elems * 12 > kInfinityCacheBytes; }
hipError_t launch_step(const StepArgs &a, hipStream_t stream);

// Resolve the scalars of the schedule's current step into *out: `base`
// supplies the step-independent ones, ds->lr the learning rate, and
// table[min(t, len) - 1] the bias corrections (1-b1^t, 1-b2^t); then
// advance ds->t by one. One lane of one workgroup.
hipError_t launch_begin_step(DevSchedule *ds, const float *table, int64_t len,
                             const StepScalars &base, StepScalars *out, hipStream_t stream);
// ds->t = t (if t >= 1) and ds->lr = lr, stream-ordered.
hipError_t launch_set_schedule(DevSchedule *ds, int64_t t, float lr, hipStream_t stream);

// Up to kWordChunk 32-bit words carried in the kernel arguments (which
// stay under 4 KiB) and stored at dst, stream-ordered: fills device memory
// from the host without a copy call or a staging buffer.
constexpr int kWordChunk = 1000;
struct WordChunk {
    uint32_t w[kWordChunk];
    int n;
};
static_assert(sizeof(WordChunk) <= 4096, "word chunk must fit the kernel arguments");
hipError_t launch_fill_words(uint32_t *dst, const WordChunk &c, hipStream_t stream);

// Per-parameter (dim-0) layout: one segment per parameter's local shard.
constexpr int kFsdpMaxWorld = 16;
struct FsdpSegment {
    const void *grads[kFsdpMaxWorld];   // replica q's gradient at this rank's first row
    void *out;                          // this rank's output shard
    int64_t state_off;                  // first element in master/m/v
    int64_t numel;                      // local elements
};
struct FsdpArgs {
    const FsdpSegment *segs;
    int nseg;
    int n;
    bool grad_bf16, out_bf16;
    float *master, *m, *v;
    StepScalars sc;
    const StepScalars *sc_dev;    // as in StepArgs
    bool stream_state;            // as in StepArgs
};
hipError_t launch_fsdp_step(const FsdpArgs &a, hipStream_t stream);

// Batched segment copy: segment s copies nbytes[s] bytes from src[s] to
// dst[s], or writes zeros when src[s] is null. esize (2 or 4) is the
// granularity every pointer and length is a multiple of.
struct Segment {
    const void *src;
    void *dst;
    int64_t nbytes;
};
hipError_t launch_copy_segments(const Segment *segs, int nseg, int esize,
                                hipStream_t stream);

// master[i] = fp32(flat[i]) (flat already offset to lo), m = v = 0.
hipError_t launch_load_master(const void *flat, bool flat_bf16, float *master,
                              float *m, float *v, int64_t shard,
                              hipStream_t stream);

}  // namespace zk
