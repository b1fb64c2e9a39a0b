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

// One step over `shard` elements. grads[q] already points at element 0 of
// replica q's slice; out at element 0 of the output slice.
struct StepArgs {
    const void *const *grads;   // host array, n entries
    int n;
    bool grad_bf16;
    float *master, *m, *v;      // library buffers, 256-byte aligned
    void *out;
    bool out_bf16;
    int64_t shard;
    StepScalars sc;
    int num_cus;
};
hipError_t launch_step(const StepArgs &a, hipStream_t stream);

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
