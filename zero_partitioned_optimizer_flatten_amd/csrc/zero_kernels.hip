// gfx950 kernels for one rank's ZeRO-2 optimizer step.
//
// K2  fused step: reduce the N gradient replicas onto this rank's slice,
//     Adam with bias correction on fp32 master/m/v, write the slice back as
//     bf16 or fp32 -- one pass over HBM, every intermediate in registers.
// K1  batched segment copy: flatten (tensor list -> zero-padded flat vector)
//     and its inverse are lists of (src, dst, bytes) segments.
// K0  master initialisation from the flat parameters.
//
// The update follows the page "ZeRO and FSDP: partitioning the optimizer
// states, the gradients and the parameters" (AI infra handbook), section
// "Implementing ZeRO's Adam from scratch", ZeroAdam.step, in binary32 with
// the operation order PyTorch uses for those lines on a CPU:
//     g  = (g_0 + g_1 + ... + g_{N-1}) / N          (left fold, rank order)
//     m  = fma(g, 1-b1, m*b1)
//     v  = fma((1-b2)*g, g, v*b2)
//     mh = m / (1-b1^t);  vh = v / (1-b2^t)
//     master = master - (lr*mh) / (sqrt(vh) + eps)
// Division and square root are the correctly rounded IEEE operations (this
// file is built with -fhip-fp32-correctly-rounded-divide-sqrt and
// -ffp-contract=off; f32 denormals are kept). The step is HBM-bound
// (about 0.5 flop per byte), so the kernels are written for streaming:
// 16-byte loads and stores, coalesced across each 64-lane wavefront, with
// every replica's load for a vector issued before the fold consumes it.
// Full blocks of the fused step read and write through buffer instructions
// on per-block descriptors, which carry the whole cache-policy field
// (device-scope streaming stores), where HIP's flat global instructions
// only carry the non-temporal hint.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "zero_internal.h"

namespace zk {

namespace {

#ifndef ZK_BLOCK
#define ZK_BLOCK 64
#endif
constexpr int kBlock = ZK_BLOCK;     // fused-step workgroup size (wavefronts of 64 lanes)
constexpr int kElemBlock = 256;      // element path
constexpr int kVec = 8;              // elements per lane per vector step
constexpr int kGroup = 8;            // replicas loaded together

// Launch shape of the fused step: one 8-element vector per lane and one pass
// over the shard, one block per workgroup (a workgroup cap, which leaves room
// for kernels on other streams, makes each workgroup stride over blocks), so
// the waves in flight at any moment cover one contiguous, sliding window of
// every stream.
//
// Dynamic LDS reserved (unused) per fused-step workgroup: caps how many
// workgroups share a CU (160 KiB of LDS per CU). The default keeps six
// one-wave workgroups per CU: measured best (with the block's buffer
// instructions 80.2% of peak HBM bandwidth against 79.1% at eight, 78.8% at
// seven and 72.3% at five; earlier with flat global instructions 79.0%
// against 77.9% at seven, 77.3% at eight and 75.4% at ten, on the 7e9/N=8
// shard), since more waves put more of the step's 12 streams' requests in
// flight than the HBM serves well, and fewer leave it idle.
#ifndef ZK_STEP_LDS
#define ZK_STEP_LDS 26624
#endif
// Sixteen replicas put twice the loads of eight in flight per wave (the
// block's pinned load order, below): four workgroups per CU gave 77.6% of
// peak against 77.1% at five, 74.0% at six and 71.3% at three (7e9/N=16
// shard; the earlier global-load kernel at six: 77.4%).
#ifndef ZK_STEP_LDS_WIDE
#define ZK_STEP_LDS_WIDE 40960
#endif
// The same for the shifted path, which does more per lane (cross-lane
// realignment, the last lane's own loads, narrow stores) and measured best
// with more waves. With its state behind the block's buffer instructions,
// ten per CU gave 77.0-77.4% of peak HBM bandwidth against 72.0-72.9% at
// twelve and 75.9-76.3% at eleven on the Llama-13B rank-7 mixed layout,
// 75.1-76.3% against 72.5-75.3% with one replica and the output three
// elements off, and 76.5% against 76.2-77.2% (eleven: 78.4-78.9%) with
// seven replicas one element off (7e9-element shard, N = 8; three states
// per variant, interleaved in one process). Earlier, with flat global state
// accesses, twelve had led ten by 0.9-3.0 points on the last two layouts.
#ifndef ZK_SHIFT_LDS
#define ZK_SHIFT_LDS 16384
#endif
// The same for the per-parameter step, whose workgroups first search the
// segment table (dependent scalar loads) before their first vector load:
// ten per CU gave 78.1% of peak against 76.9% at seven and 73.2% at six;
// twelve to sixteen 77.7-78.1%, uncapped 77.1% (Llama-7B list, N = 8).
#ifndef ZK_FSDP_LDS
#define ZK_FSDP_LDS 16384
#endif
// Non-temporal (streaming) hints. The replicas are read once and the
// parameter output written once (replica loads take the hint where every
// stream sits on whole 128-byte lines; see StepArgs::nt_grad). For
// master/m/v the launcher chooses (see StepArgs::stream_state): in the split
// lane layout of a full wavefront block, where every store instruction
// writes whole lines, non-temporal loads and stores on them together
// measured 6% faster than the default policy on a 875M-element shard
// (either hint alone: no gain, or slower), but slower on shards whose state
// fits in the 256 MB Infinity Cache and stays there between steps. Where a
// lane owns 32 contiguous bytes (the last partial block, the element and
// shifted paths), the hints measured slower, so those accesses keep the
// default policy.
#ifndef ZK_NT_GRAD
#define ZK_NT_GRAD 1
#endif
#ifndef ZK_NT_OUT
#define ZK_NT_OUT 1
#endif
// Cache-policy bits of the buffer instructions of a full wavefront block of
// the fused step (gfx950 encoding: sc0 = 1, nt = 2, sc1 = 16). Streamed
// state and the output are stored non-temporal at device scope (nt sc1):
// 80.2-80.7% of peak HBM bandwidth on the 7e9/N=8 shard against 79.5-79.6%
// with nt alone and 79.0% for the same access pattern through flat global
// instructions (interleaved in one process, three runs). Device scope on
// the state stores alone gave 80.3%, on the output alone 77.9%; sc0 nt sc1
// 80.3%, sc0 nt 79.7%, sc1 alone 79.0%; the same bits on the loads
// (nt sc1, sc0 nt) 79.1-79.2%, and default-policy loads of the replicas or
// of the state 79.3-79.4%. Global loads with these buffer stores gave
// 78.8%: the gain needs the buffer loads as well.
#ifndef ZK_POL_STORE_STREAM
#define ZK_POL_STORE_STREAM 18
#endif
// State that stays in the Infinity Cache between steps (12 S bytes within
// its 256 MB) is loaded and stored at device scope without the streaming
// hint (sc1): 83.8% of peak on the GPT-2-small shard (N = 8, rank 3)
// against 79.0% with default-policy loads and 83.2% with both default; sc1
// stores with default loads 87.0% / 79.0% in two runs, sc0 sc1 stores
// 78.9%, nt sc1 stores 72.6-78.4%, nt stores 77.8-81.6%, sc0 loads 80.1%.
// Its output keeps the plain non-temporal hint (nt sc1 or no hint: within
// 0.3 points).
#ifndef ZK_POL_STORE_CACHED
#define ZK_POL_STORE_CACHED 16
#endif
#ifndef ZK_POL_LOAD_CACHED
#define ZK_POL_LOAD_CACHED 16
#endif
#ifndef ZK_POL_OUT_CACHED
#define ZK_POL_OUT_CACHED 2
#endif
// Replica counts up to this take the pinned load order of a block (the
// replicas, m and v in one round trip, then master).
// Segment copy: cache policy of its 16-byte stores. Non-temporal at device
// scope (nt sc1), through buffer instructions with non-temporal loads: the
// one-tensor 7e9 bf16 flatten ran at 85.0% of peak HBM bandwidth against
// 81.3% for flat global non-temporal loads and stores, the GPT-2-small list
// at 69.4% against 67.4%, the Llama-7B list at 82.0% / 80.2% against
// 81.8% / 79.4% (aligned / one element off); sc0 nt sc1 stores measured
// the same (interleaved in one process).
#ifndef ZK_POL_COPY_STORE
#define ZK_POL_COPY_STORE 18
#endif
#ifndef ZK_PIN_MAX
#define ZK_PIN_MAX 16
#endif
// Master initialisation: dynamic LDS reserved (unused) per one-wave
// workgroup, six per compute unit as for the fused step. Its three write
// streams (master, m, v) and one read stream measured 80.7% / 80.1% of peak
// HBM bandwidth at six per CU against 70.2% / 65.5% uncapped (7e9/N=8 and
// 70e9/N=64 shards; four, five, eight and ten per CU 65.7-80.6%).
#ifndef ZK_K0_LDS
#define ZK_K0_LDS 26624
#endif
// Segment copy: workgroup size (one 16-byte vector per lane per chunk).
#ifndef ZK_COPY_BLOCK
#define ZK_COPY_BLOCK 64
#endif

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

template <bool NT>
__device__ __forceinline__ uint2 ld_u2(const void *p) {
    if (NT) {
        u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t *>(p));
        return make_uint2(v.x, v.y);
    }
    return *reinterpret_cast<const uint2 *>(p);
}

template <bool NT>
__device__ __forceinline__ uint4 ld_u4(const void *p) {
    if (NT) {
        u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
        return make_uint4(v.x, v.y, v.z, v.w);
    }
    return *reinterpret_cast<const uint4 *>(p);
}

template <bool NT>
__device__ __forceinline__ float4 ld_f4(const void *p) {
    if (NT) {
        f32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t *>(p));
        return make_float4(v.x, v.y, v.z, v.w);
    }
    return *reinterpret_cast<const float4 *>(p);
}

template <bool NT>
__device__ __forceinline__ void st_u4(void *p, uint4 v) {
    if (NT) {
        u32x4_t w = {v.x, v.y, v.z, v.w};
        __builtin_nontemporal_store(w, reinterpret_cast<u32x4_t *>(p));
    } else {
        *reinterpret_cast<uint4 *>(p) = v;
    }
}

template <bool NT>
__device__ __forceinline__ void st_f4(void *p, float4 v) {
    if (NT) {
        f32x4_t w = {v.x, v.y, v.z, v.w};
        __builtin_nontemporal_store(w, reinterpret_cast<f32x4_t *>(p));
    } else {
        *reinterpret_cast<float4 *>(p) = v;
    }
}

// Buffer instructions over one wave-uniform span: the descriptor (base in
// scalar registers, byte addressing, range = the span) is built per span,
// and each lane passes a 32-bit byte offset into it. An access past the
// span reads zero and writes nothing. Word 3 is the gfx9 family's raw
// (untyped) buffer format.
constexpr int kPolDefault = 0;
constexpr int kPolNT = 2;
typedef __amdgpu_buffer_rsrc_t span_t;

__device__ __forceinline__ span_t span_of(const void *base, int nbytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, nbytes,
                                             0x00020000);
}

template <int POL>
__device__ __forceinline__ uint2 bld_u2(span_t r, int off) {
    u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, POL);
    return make_uint2(v.x, v.y);
}

template <int POL>
__device__ __forceinline__ float4 bld_f4(span_t r, int off) {
    u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, POL);
    return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z),
                       __uint_as_float(v.w));
}

template <int POL>
__device__ __forceinline__ uint4 bld_u4(span_t r, int off) {
    u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, POL);
    return make_uint4(v.x, v.y, v.z, v.w);
}

template <int POL>
__device__ __forceinline__ void bst_u4(span_t r, int off, uint4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{v.x, v.y, v.z, v.w}, r, off, 0, POL);
}

template <int POL>
__device__ __forceinline__ void bst_u2(span_t r, int off, uint2 v) {
    __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{v.x, v.y}, r, off, 0, POL);
}

template <int POL>
__device__ __forceinline__ void bst_f4(span_t r, int off, float4 v) {
    u32x4_t w = {__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z),
                 __float_as_uint(v.w)};
    __builtin_amdgcn_raw_buffer_store_b128(w, r, off, 0, POL);
}

__device__ __forceinline__ float widen_bf16(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// binary32 -> bf16 bits, round to nearest, ties to even. NaN keeps its sign
// and gets the quiet bit; overflow rounds to infinity through the carry.
__device__ __forceinline__ uint32_t round_bf16(float x) {
    uint32_t u = __float_as_uint(x);
    uint32_t r = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
    return ((u & 0x7FFFFFFFu) > 0x7F800000u) ? ((u >> 16) | 0x40u) : r;
}

// One element of the Adam update in two parts: the moments (m, v updated in
// place) give the step u, which the parameter then takes (p - u).
__device__ __forceinline__ float adam_moments(float g, float &m, float &v,
                                              const StepScalars &sc) {
    float mm = __builtin_fmaf(g, sc.c1, m * sc.b1);
    float vv = __builtin_fmaf(sc.c2 * g, g, v * sc.b2);
    float mh = mm / sc.bc1;
    float vh = vv / sc.bc2;
    float den = __builtin_sqrtf(vh) + sc.eps;
    m = mm;
    v = vv;
    return (sc.lr * mh) / den;
}

// One element of the Adam update; p/m/v updated in place.
__device__ __forceinline__ void adam_update(float g, float &p, float &m,
                                            float &v, const StepScalars &sc) {
    const float u = adam_moments(g, m, v, sc);
    p = p - u;
}

// Replica pointer table passed by value in the kernel arguments, so each
// pointer is a wave-uniform scalar (SGPR base + per-lane offset).
template <int NR>
struct Reps {
    const void *p[NR > 0 ? NR : ZERO_MAX_WORLD];
};

// Where a step kernel takes its scalars from: by value in the kernel
// arguments, or (DS) from device memory written by the begin-step kernel,
// which lets a captured graph replay successive steps.
template <bool DS> struct ScalarArg;
template <> struct ScalarArg<false> { StepScalars v; };
template <> struct ScalarArg<true> { const StepScalars *p; };

__device__ __forceinline__ StepScalars scalars(const ScalarArg<false> &a) { return a.v; }
__device__ __forceinline__ StepScalars scalars(const ScalarArg<true> &a) { return *a.p; }

// Raw 8-element gradient vector of one replica: 16 bytes of bf16 or 32
// bytes of fp32.
template <bool GB> struct RawVec;
template <> struct RawVec<true> { uint4 a; };
template <> struct RawVec<false> { float4 a, b; };

template <bool GB>
__device__ __forceinline__ RawVec<GB> load_vec(const void *base, int64_t j);

template <>
__device__ __forceinline__ RawVec<true> load_vec<true>(const void *base, int64_t j) {
    RawVec<true> r;
    r.a = ld_u4<ZK_NT_GRAD>(reinterpret_cast<const uint4 *>(base) + j);
    return r;
}

template <>
__device__ __forceinline__ RawVec<false> load_vec<false>(const void *base, int64_t j) {
    RawVec<false> r;
    const float4 *p = reinterpret_cast<const float4 *>(base);
    r.a = ld_f4<ZK_NT_GRAD>(p + 2 * j);
    r.b = ld_f4<ZK_NT_GRAD>(p + 2 * j + 1);
    return r;
}

__device__ __forceinline__ void unpack(const RawVec<true> &r, float (&x)[kVec]) {
    x[0] = widen_bf16(r.a.x & 0xFFFFu); x[1] = widen_bf16(r.a.x >> 16);
    x[2] = widen_bf16(r.a.y & 0xFFFFu); x[3] = widen_bf16(r.a.y >> 16);
    x[4] = widen_bf16(r.a.z & 0xFFFFu); x[5] = widen_bf16(r.a.z >> 16);
    x[6] = widen_bf16(r.a.w & 0xFFFFu); x[7] = widen_bf16(r.a.w >> 16);
}

__device__ __forceinline__ void unpack(const RawVec<false> &r, float (&x)[kVec]) {
    x[0] = r.a.x; x[1] = r.a.y; x[2] = r.a.z; x[3] = r.a.w;
    x[4] = r.b.x; x[5] = r.b.y; x[6] = r.b.z; x[7] = r.b.w;
}

__device__ __forceinline__ void load8(const float *base, int64_t j, float (&x)[kVec]) {
    const float4 *p = reinterpret_cast<const float4 *>(base);
    float4 a = ld_f4<false>(p + 2 * j), b = ld_f4<false>(p + 2 * j + 1);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

template <bool NT>
__device__ __forceinline__ void store8(float *base, int64_t j, const float (&x)[kVec]) {
    float4 *p = reinterpret_cast<float4 *>(base);
    st_f4<NT>(p + 2 * j, make_float4(x[0], x[1], x[2], x[3]));
    st_f4<NT>(p + 2 * j + 1, make_float4(x[4], x[5], x[6], x[7]));
}

// Fold one group of up to kGroup replicas into s (rank order). The group's
// loads are all issued before the first add consumes them.
template <int NR, bool GB>
__device__ __forceinline__ void fold_group(const Reps<NR> &reps, int q0, int n, int64_t j,
                                           float (&s)[kVec]) {
    RawVec<GB> raw[kGroup];
#pragma unroll
    for (int k = 0; k < kGroup; ++k)
        if (q0 + k < n) raw[k] = load_vec<GB>(reps.p[q0 + k], j);
#pragma unroll
    for (int k = 0; k < kGroup; ++k) {
        if (q0 + k < n) {
            float x[kVec];
            unpack(raw[k], x);
            if (q0 + k == 0) {
#pragma unroll
                for (int e = 0; e < kVec; ++e) s[e] = x[e];
            } else {
#pragma unroll
                for (int e = 0; e < kVec; ++e) s[e] = s[e] + x[e];
            }
        }
    }
}

// One 8-element vector j of the fused step.
template <int NR, bool GB, bool PB>
__device__ __forceinline__ void step_vector(const Reps<NR> &reps, int n, bool pow2,
                                            float *__restrict__ master, float *__restrict__ mom,
                                            float *__restrict__ var, void *__restrict__ out,
                                            int64_t j, const StepScalars &sc) {
    float p[kVec], m[kVec], v[kVec];
    load8(master, j, p);
    load8(mom, j, m);
    load8(var, j, v);

    float s[kVec];
    if constexpr (NR > 0 && NR <= 2 * kGroup) {
#pragma unroll
        for (int q0 = 0; q0 < NR; q0 += kGroup) fold_group<NR, GB>(reps, q0, n, j, s);
    } else {
#pragma unroll 1
        for (int q0 = 0; q0 < n; q0 += kGroup) fold_group<NR, GB>(reps, q0, n, j, s);
    }

    float g[kVec];
    if (pow2) {
#pragma unroll
        for (int e = 0; e < kVec; ++e) g[e] = s[e] * sc.inv_n;   // exact scaling
    } else {
#pragma unroll
        for (int e = 0; e < kVec; ++e) g[e] = s[e] / sc.nf;
    }
#pragma unroll
    for (int e = 0; e < kVec; ++e) adam_update(g[e], p[e], m[e], v[e], sc);

    store8<false>(master, j, p);
    store8<false>(mom, j, m);
    store8<false>(var, j, v);
    if (PB) {
        uint4 o;
        o.x = round_bf16(p[0]) | (round_bf16(p[1]) << 16);
        o.y = round_bf16(p[2]) | (round_bf16(p[3]) << 16);
        o.z = round_bf16(p[4]) | (round_bf16(p[5]) << 16);
        o.w = round_bf16(p[6]) | (round_bf16(p[7]) << 16);
        st_u4<ZK_NT_OUT>(reinterpret_cast<uint4 *>(out) + j, o);
    } else {
        store8<ZK_NT_OUT>(reinterpret_cast<float *>(out), j, p);
    }
}

// Split lane layout of a full wavefront block (kBlock vectors, 8*kBlock
// elements): lane l owns the 4-element quads l and l + kBlock of the block,
// so every load and store instruction of the wavefront covers one
// contiguous span of its stream (1 KiB of fp32, 512 B of bf16) instead of
// every other 16 bytes of a span twice as long. Each element still takes
// the same arithmetic, so results do not depend on the layout.
template <bool GB> struct SplitRaw;
template <> struct SplitRaw<true> { uint2 a, b; };
template <> struct SplitRaw<false> { float4 a, b; };

// Bytes of one full wavefront block of a stream of the given element size.
template <int ES> constexpr int kSpanBytes = kBlock * kVec * ES;

// A lane's two quads of one replica's block (GPOL: its cache policy).
template <bool GB, int GPOL>
__device__ __forceinline__ SplitRaw<GB> load_split(span_t r) {
    const int l = threadIdx.x;
    SplitRaw<GB> x;
    if constexpr (GB) {
        x.a = bld_u2<GPOL>(r, 8 * l);
        x.b = bld_u2<GPOL>(r, 8 * (kBlock + l));
    } else {
        x.a = bld_f4<GPOL>(r, 16 * l);
        x.b = bld_f4<GPOL>(r, 16 * (kBlock + l));
    }
    return x;
}

__device__ __forceinline__ void unpack(const SplitRaw<true> &r, float (&x)[kVec]) {
    x[0] = widen_bf16(r.a.x & 0xFFFFu); x[1] = widen_bf16(r.a.x >> 16);
    x[2] = widen_bf16(r.a.y & 0xFFFFu); x[3] = widen_bf16(r.a.y >> 16);
    x[4] = widen_bf16(r.b.x & 0xFFFFu); x[5] = widen_bf16(r.b.x >> 16);
    x[6] = widen_bf16(r.b.y & 0xFFFFu); x[7] = widen_bf16(r.b.y >> 16);
}

__device__ __forceinline__ void unpack(const SplitRaw<false> &r, float (&x)[kVec]) {
    x[0] = r.a.x; x[1] = r.a.y; x[2] = r.a.z; x[3] = r.a.w;
    x[4] = r.b.x; x[5] = r.b.y; x[6] = r.b.z; x[7] = r.b.w;
}

template <int POL>
__device__ __forceinline__ void load8_split(span_t r, float (&x)[kVec]) {
    const int l = threadIdx.x;
    float4 a = bld_f4<POL>(r, 16 * l), b = bld_f4<POL>(r, 16 * (kBlock + l));
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

template <int POL>
__device__ __forceinline__ void store8_split(span_t r, const float (&x)[kVec]) {
    const int l = threadIdx.x;
    bst_f4<POL>(r, 16 * l, make_float4(x[0], x[1], x[2], x[3]));
    bst_f4<POL>(r, 16 * (kBlock + l), make_float4(x[4], x[5], x[6], x[7]));
}

// Fold replicas q0r .. q0r + kGroup - 1 of block blk into s (rank order).
// The group's loads are all issued before the first add consumes them.
template <int NR, bool GB, int GPOL>
__device__ __forceinline__ void fold_group_split(const Reps<NR> &reps, int q0r, int n,
                                                 int64_t blk, float (&s)[kVec]) {
    constexpr int gbytes = kSpanBytes<GB ? 2 : 4>;
    SplitRaw<GB> raw[kGroup];
#pragma unroll
    for (int k = 0; k < kGroup; ++k)
        if (q0r + k < n)
            raw[k] = load_split<GB, GPOL>(
                span_of(static_cast<const char *>(reps.p[q0r + k]) + blk * gbytes, gbytes));
#pragma unroll
    for (int k = 0; k < kGroup; ++k) {
        if (q0r + k < n) {
            float x[kVec];
            unpack(raw[k], x);
            if (q0r + k == 0) {
#pragma unroll
                for (int e = 0; e < kVec; ++e) s[e] = x[e];
            } else {
#pragma unroll
                for (int e = 0; e < kVec; ++e) s[e] = s[e] + x[e];
            }
        }
    }
}

// The fused step on full wavefront block blk (elements blk * 8 * kBlock
// onwards of every stream, which lie on 16-byte boundaries) in the split
// lane layout, through buffer instructions over each stream's block.
// NTS: master/m/v streamed (non-temporal loads, stores at the streaming
// policy) rather than kept in the Infinity Cache; NTG: non-temporal replica
// loads.
template <int NR, bool GB, bool PB, bool NTS, bool NTG>
__device__ __forceinline__ void step_block_split(const Reps<NR> &reps, int n, bool pow2,
                                                 float *master, float *mom, float *var, void *out,
                                                 int64_t blk, const StepScalars &sc) {
    constexpr int kGPol = NTG ? kPolNT : kPolDefault;
    constexpr int kSLoad = NTS ? kPolNT : ZK_POL_LOAD_CACHED;
    constexpr int kSStore = NTS ? ZK_POL_STORE_STREAM : ZK_POL_STORE_CACHED;
    constexpr int kOStore = !ZK_NT_OUT ? kPolDefault
                                       : (NTS ? ZK_POL_STORE_STREAM : ZK_POL_OUT_CACHED);
    constexpr int sbytes = kSpanBytes<4>;
    constexpr int obytes = kSpanBytes<PB ? 2 : 4>;
    constexpr int gbytes = kSpanBytes<GB ? 2 : 4>;
    const int64_t so = blk * (kBlock * kVec);
    const span_t rp = span_of(master + so, sbytes), rm = span_of(mom + so, sbytes),
                 rv = span_of(var + so, sbytes);
    float s[kVec], p[kVec], m[kVec], v[kVec], g[kVec];
    if constexpr (NR > 0 && NR <= ZK_PIN_MAX) {
        // Up to ZK_PIN_MAX replicas: the replicas, m and v in one round
        // trip, and master, whose value is needed last, loaded once the
        // moments are done; scheduling barriers keep that order. Measured
        // 80.3% of peak HBM bandwidth against 79.2% with every load in one
        // round trip (7e9/N=8 shard, interleaved in one process).
        // NR is a capacity where the count comes at run time (n <= NR): only
        // the first n table entries are replicas
        SplitRaw<GB> raw[NR];
#pragma unroll
        for (int k = 0; k < NR; ++k)
            if (k < n)
                raw[k] = load_split<GB, kGPol>(
                    span_of(static_cast<const char *>(reps.p[k]) + blk * gbytes, gbytes));
        load8_split<kSLoad>(rm, m);
        load8_split<kSLoad>(rv, v);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = 0; k < NR; ++k) {
            if (k < n) {
                float x[kVec];
                unpack(raw[k], x);
#pragma unroll
                for (int e = 0; e < kVec; ++e) s[e] = k == 0 ? x[e] : s[e] + x[e];
            }
        }
        if (pow2) {
#pragma unroll
            for (int e = 0; e < kVec; ++e) g[e] = s[e] * sc.inv_n;
        } else {
#pragma unroll
            for (int e = 0; e < kVec; ++e) g[e] = s[e] / sc.nf;
        }
        float u[kVec];
#pragma unroll
        for (int e = 0; e < kVec; ++e) u[e] = adam_moments(g[e], m[e], v[e], sc);
        __builtin_amdgcn_sched_barrier(0);
        load8_split<kSLoad>(rp, p);
#pragma unroll
        for (int e = 0; e < kVec; ++e) p[e] = p[e] - u[e];
    } else {
        // Replicas first, then the state: measured 0.3-1% faster than the
        // reverse order (issuing every load before the first wait, pinned
        // with a scheduling barrier, measured 6% slower than either).
        if constexpr (NR > 0 && NR <= 2 * kGroup) {
#pragma unroll
            for (int r = 0; r < NR; r += kGroup)
                fold_group_split<NR, GB, kGPol>(reps, r, n, blk, s);
        } else {
#pragma unroll 1
            for (int r = 0; r < n; r += kGroup)
                fold_group_split<NR, GB, kGPol>(reps, r, n, blk, s);
        }
        load8_split<kSLoad>(rp, p);
        load8_split<kSLoad>(rm, m);
        load8_split<kSLoad>(rv, v);
        if (pow2) {
#pragma unroll
            for (int e = 0; e < kVec; ++e) g[e] = s[e] * sc.inv_n;
        } else {
#pragma unroll
            for (int e = 0; e < kVec; ++e) g[e] = s[e] / sc.nf;
        }
#pragma unroll
        for (int e = 0; e < kVec; ++e) adam_update(g[e], p[e], m[e], v[e], sc);
    }

    store8_split<kSStore>(rp, p);
    store8_split<kSStore>(rm, m);
    store8_split<kSStore>(rv, v);
    const span_t ro = span_of(static_cast<char *>(out) + blk * obytes, obytes);
    if constexpr (PB) {
        uint2 a, b;
        a.x = round_bf16(p[0]) | (round_bf16(p[1]) << 16);
        a.y = round_bf16(p[2]) | (round_bf16(p[3]) << 16);
        b.x = round_bf16(p[4]) | (round_bf16(p[5]) << 16);
        b.y = round_bf16(p[6]) | (round_bf16(p[7]) << 16);
        const int l = threadIdx.x;
        bst_u2<kOStore>(ro, 8 * l, a);
        bst_u2<kOStore>(ro, 8 * (kBlock + l), b);
    } else {
        store8_split<kOStore>(ro, p);
    }
}

// One element i of the fused step (any alignment). R is a replica table:
// rep_base(reps, q, element size) gives replica q's element 0.
template <int NR, bool GB, bool PB, class R>
__device__ __forceinline__ void step_one(const R &reps, int n, float *__restrict__ master,
                                         float *__restrict__ mom, float *__restrict__ var,
                                         void *__restrict__ out, int64_t i, const StepScalars &sc);

template <int NR>
__device__ __forceinline__ const void *rep_base(const Reps<NR> &r, int q, int) {
    return r.p[q];
}

// Vector path: every stream 16-byte aligned. A full wavefront block takes
// the split lane layout; the last, partial block has lane j - 64*block
// handle elements [8j, 8j+8) of vector j. NR > 0 fixes the replica count at
// compile time (N <= 16 fully unrolled; larger N walks the groups in a loop
// to bound register use); NR == 0 reads it from `nrep`. Workgroups [0, nbw) take
// the full blocks: block w, then w + nbw, ... (nbw = the number of full
// blocks unless the launch is capped, so normally one block each, one pass
// over the shard). The next workgroup takes the partial block, if any, and
// one more, launched when head + tail > 0, steps the `head` elements just
// before element 0 and the `tail` elements after the last vector one by
// one, so a shard takes one launch whatever its alignment.
template <int NR, bool GB, bool PB, bool DS, bool NTG>
__global__ void __launch_bounds__(kBlock)
step_vec_kernel(Reps<NR> reps, int nrep, float *__restrict__ master,
                float *__restrict__ mom, float *__restrict__ var,
                void *__restrict__ out, int64_t nvec, int64_t nbw, int head, int tail,
                int nt_state, ScalarArg<DS> sa) {
    const StepScalars sc = scalars(sa);
    const int n = NR > 0 ? NR : nrep;
    constexpr bool kPow2 = NR > 0 && (NR & (NR - 1)) == 0;
    const bool pow2 = kPow2 || (NR == 0 && sc.n_pow2);
    const int64_t nfull = nvec / kBlock;
    const int64_t w = blockIdx.x;
    if (w < nbw) {
        // one loop per state policy: with the branch inside the loop body the
        // compiler hoists the replica loads, common to both, above it, and
        // the state loads can no longer share their round trip
        if (nt_state) {
            for (int64_t blk = w; blk < nfull; blk += nbw)
                step_block_split<NR, GB, PB, true, NTG>(reps, n, pow2, master, mom, var, out, blk,
                                                        sc);
        } else {
            for (int64_t blk = w; blk < nfull; blk += nbw)
                step_block_split<NR, GB, PB, false, NTG>(reps, n, pow2, master, mom, var, out,
                                                         blk, sc);
        }
        return;
    }
    if (w == nbw && nfull * kBlock < nvec) {
        const int64_t j = nfull * kBlock + threadIdx.x;
        if (j < nvec) step_vector<NR, GB, PB>(reps, n, pow2, master, mom, var, out, j, sc);
        return;
    }
    for (int k = threadIdx.x; k < head + tail; k += kBlock) {
        const int64_t e = k < head ? (int64_t)(k - head) : nvec * kVec + (k - head);
        step_one<NR, GB, PB>(reps, n, master, mom, var, out, e, sc);
    }
}

template <int NR, bool GB, bool PB, class R>
__device__ __forceinline__ void step_one(const R &reps, int n, float *__restrict__ master,
                                         float *__restrict__ mom, float *__restrict__ var,
                                         void *__restrict__ out, int64_t i, const StepScalars &sc) {
    constexpr int es = GB ? 2 : 4;
    float s;
    if (GB) s = widen_bf16(reinterpret_cast<const uint16_t *>(rep_base(reps, 0, es))[i]);
    else s = reinterpret_cast<const float *>(rep_base(reps, 0, es))[i];
    for (int q = 1; q < n; ++q) {
        float x;
        if (GB) x = widen_bf16(reinterpret_cast<const uint16_t *>(rep_base(reps, q, es))[i]);
        else x = reinterpret_cast<const float *>(rep_base(reps, q, es))[i];
        s = s + x;
    }
    float p = master[i], m = mom[i], v = var[i];
    const float g = sc.n_pow2 ? s * sc.inv_n : s / sc.nf;
    adam_update(g, p, m, v, sc);
    master[i] = p;
    mom[i] = m;
    var[i] = v;
    if (PB) reinterpret_cast<uint16_t *>(out)[i] = (uint16_t)round_bf16(p);
    else reinterpret_cast<float *>(out)[i] = p;
}

// Element path: any alignment, and the tail of the vector path. Lane
// handles element i, consecutive lanes consecutive elements.
template <bool GB, bool PB, bool DS>
__global__ void __launch_bounds__(kElemBlock)
step_elem_kernel(Reps<0> reps, int nrep, float *__restrict__ master,
                 float *__restrict__ mom, float *__restrict__ var,
                 void *__restrict__ out, int64_t begin, int64_t end,
                 ScalarArg<DS> sa) {
    const StepScalars sc = scalars(sa);
    const int64_t stride = (int64_t)gridDim.x * kElemBlock;
    for (int64_t i = begin + (int64_t)blockIdx.x * kElemBlock + threadIdx.x; i < end; i += stride)
        step_one<0, GB, PB>(reps, nrep, master, mom, var, out, i, sc);
}

// ------------------------------------------------------ shifted vector path
// For caller buffers that do not share one 16-byte phase with the state
// (e.g. replicas holding only this rank's slice next to a full flat output
// at an odd offset lo). The vector partition follows the state, so master,
// m and v keep their aligned 16-byte accesses.
//
// A bf16 replica whose vector j starts d elements past a 16-byte boundary
// spans aligned blocks j and j+1 of its aligned base. Each lane loads block
// j; block j+1 is the next lane's block j, taken across lanes (DPP wave
// shift), so a wavefront still issues one 16-byte load per lane per
// replica (measured 10-15% faster than loading both blocks in every lane).
// The wave's last lane and the lane of the last vector load block j+1
// themselves; that block holds at least one of the lane's own elements, so
// no read leaves the 16-byte blocks of the buffer's own elements.
//
// An output at another phase is written with 2-, 4- and 8-byte stores that
// cover exactly the lane's elements (measured no slower than a cross-lane
// realignment into whole blocks). An fp32 replica's 32 bytes span three
// aligned blocks: the lane loads two and takes the third, the next lane's
// first, across lanes in the same way.

// Replica pointer table: each base 16-byte aligned, and d[q] the number of
// elements between it and the replica's element 0 of the vector range.
template <int NR>
struct ShiftReps {
    const void *p[NR > 0 ? NR : ZERO_MAX_WORLD];
    uint8_t d[NR > 0 ? NR : ZERO_MAX_WORLD];
};

template <int NR>
__device__ __forceinline__ const void *rep_base(const ShiftReps<NR> &r, int q, int es) {
    return static_cast<const char *>(r.p[q]) + (int)r.d[q] * es;
}

// Value of v in the next lane of the wavefront (DPP wave shift left by one;
// lanes without a next lane get 0 and do not use it).
__device__ __forceinline__ uint32_t next_lane(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x130, 0xf, 0xf, false);
}

__device__ __forceinline__ uint4 next_lane(uint4 v) {
    return make_uint4(next_lane(v.x), next_lane(v.y), next_lane(v.z), next_lane(v.w));
}

template <bool GB> struct ShiftRaw;
template <> struct ShiftRaw<true> { uint4 a, b; };             // blocks j, j+1 (8 bf16 each)
template <> struct ShiftRaw<false> { float4 a, b, c; };        // 3 blocks of 4 fp32

__device__ __forceinline__ ShiftRaw<true> load_shift(const void *base, int d, int64_t j,
                                                     bool self_next, ShiftRaw<true> *) {
    const uint4 *p = reinterpret_cast<const uint4 *>(base) + j;
    ShiftRaw<true> r;
    r.a = ld_u4<false>(p);
    r.b = make_uint4(0u, 0u, 0u, 0u);
    if (d && self_next) r.b = ld_u4<false>(p + 1);
    return r;
}

__device__ __forceinline__ ShiftRaw<false> load_shift(const void *base, int d, int64_t j,
                                                      bool self_next, ShiftRaw<false> *) {
    const float4 *p = reinterpret_cast<const float4 *>(base) + 2 * j;
    ShiftRaw<false> r;
    r.a = ld_f4<false>(p);
    r.b = ld_f4<false>(p + 1);
    r.c = make_float4(0.f, 0.f, 0.f, 0.f);
    if (d && self_next) r.c = ld_f4<false>(p + 2);
    return r;
}

// Block j+1 from the next lane, for the lanes that did not load it.
__device__ __forceinline__ void complete_shift(ShiftRaw<true> &r, int d, bool self_next) {
    if (!d) return;
    const uint4 nb = next_lane(r.a);
    if (!self_next) r.b = nb;
}

// fp32: the third block is the next lane's first.
__device__ __forceinline__ void complete_shift(ShiftRaw<false> &r, int d, bool self_next) {
    if (!d) return;
    const uint4 nb = next_lane(make_uint4(__float_as_uint(r.a.x), __float_as_uint(r.a.y),
                                          __float_as_uint(r.a.z), __float_as_uint(r.a.w)));
    if (!self_next)
        r.c = make_float4(__uint_as_float(nb.x), __uint_as_float(nb.y), __uint_as_float(nb.z),
                          __uint_as_float(nb.w));
}

// Four words (eight bf16) starting D elements into the 16 elements of c:
// word k is bytes [2D + 4k, 2D + 4k + 4).
template <int D>
__device__ __forceinline__ uint4 take_words(const uint32_t (&c)[8]) {
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
        w[k] = (D % 2 == 0) ? c[k + D / 2]
                            : __builtin_amdgcn_alignbyte(c[k + D / 2 + 1], c[k + D / 2], 2);
    return make_uint4(w[0], w[1], w[2], w[3]);
}

__device__ __forceinline__ uint4 take_words(const uint32_t (&c)[8], int d) {
    switch (d) {
    case 0: return take_words<0>(c);
    case 1: return take_words<1>(c);
    case 2: return take_words<2>(c);
    case 3: return take_words<3>(c);
    case 4: return take_words<4>(c);
    case 5: return take_words<5>(c);
    case 6: return take_words<6>(c);
    default: return take_words<7>(c);
    }
}

__device__ __forceinline__ void unpack_shift(const ShiftRaw<true> &r, int d, float (&x)[kVec]) {
    const uint32_t c[8] = {r.a.x, r.a.y, r.a.z, r.a.w, r.b.x, r.b.y, r.b.z, r.b.w};
    RawVec<true> v;
    v.a = take_words(c, d);
    unpack(v, x);
}

template <int D>
__device__ __forceinline__ void take_f32(const float (&c)[12], float (&x)[kVec]) {
#pragma unroll
    for (int e = 0; e < kVec; ++e) x[e] = c[D + e];
}

__device__ __forceinline__ void unpack_shift(const ShiftRaw<false> &r, int d, float (&x)[kVec]) {
    const float c[12] = {r.a.x, r.a.y, r.a.z, r.a.w, r.b.x, r.b.y,
                         r.b.z, r.b.w, r.c.x, r.c.y, r.c.z, r.c.w};
    switch (d) {
    case 0: take_f32<0>(c, x); break;
    case 1: take_f32<1>(c, x); break;
    case 2: take_f32<2>(c, x); break;
    default: take_f32<3>(c, x); break;
    }
}

template <int NR, bool GB>
__device__ __forceinline__ void fold_group_shift(const ShiftReps<NR> &reps, int q0, int n,
                                                 int64_t j, bool self_next, float (&s)[kVec]) {
    ShiftRaw<GB> raw[kGroup];
#pragma unroll
    for (int k = 0; k < kGroup; ++k)
        if (q0 + k < n)
            raw[k] = load_shift(reps.p[q0 + k], reps.d[q0 + k], j, self_next,
                                (ShiftRaw<GB> *)nullptr);
#pragma unroll
    for (int k = 0; k < kGroup; ++k) {
        if (q0 + k < n) {
            complete_shift(raw[k], reps.d[q0 + k], self_next);
            float x[kVec];
            unpack_shift(raw[k], reps.d[q0 + k], x);
            if (q0 + k == 0) {
#pragma unroll
                for (int e = 0; e < kVec; ++e) s[e] = x[e];
            } else {
#pragma unroll
                for (int e = 0; e < kVec; ++e) s[e] = s[e] + x[e];
            }
        }
    }
}

template <typename T>
__device__ __forceinline__ void st_nt(T *p, T v) {
    if (ZK_NT_OUT) __builtin_nontemporal_store(v, p);
    else *p = v;
}


// Eight packed bf16 values (o.x = elements 0,1, ...) to q, which sits
// d elements past a 16-byte boundary.
__device__ __forceinline__ void store_bf16x8_at(uint16_t *q, int d, uint4 o) {
    if (d == 0) {
        st_u4<ZK_NT_OUT>(q, o);
    } else if (d == 4) {                                 // 8-byte aligned
        st_nt(reinterpret_cast<u32x2_t *>(q), u32x2_t{o.x, o.y});
        st_nt(reinterpret_cast<u32x2_t *>(q + 4), u32x2_t{o.z, o.w});
    } else if ((d & 1) == 0) {                           // 4-byte aligned
        uint32_t *w = reinterpret_cast<uint32_t *>(q);
        st_nt(w, o.x);
        st_nt(w + 1, o.y);
        st_nt(w + 2, o.z);
        st_nt(w + 3, o.w);
    } else {                                             // 2 mod 4: q + 1 is 4-byte aligned
        uint32_t *w = reinterpret_cast<uint32_t *>(q + 1);
        st_nt(q, (uint16_t)(o.x & 0xFFFFu));
        st_nt(w, __builtin_amdgcn_alignbyte(o.y, o.x, 2));
        st_nt(w + 1, __builtin_amdgcn_alignbyte(o.z, o.y, 2));
        st_nt(w + 2, __builtin_amdgcn_alignbyte(o.w, o.z, 2));
        st_nt(q + 7, (uint16_t)(o.w >> 16));
    }
}

// Eight fp32 values to q, which sits d elements past a 16-byte boundary.
__device__ __forceinline__ void store_f32x8_at(float *q, int d, const float (&x)[kVec]) {
    if (d == 0) {
        st_f4<ZK_NT_OUT>(q, make_float4(x[0], x[1], x[2], x[3]));
        st_f4<ZK_NT_OUT>(q + 4, make_float4(x[4], x[5], x[6], x[7]));
    } else if (d == 2) {                                 // 8-byte aligned
#pragma unroll
        for (int k = 0; k < 4; ++k)
            st_nt(reinterpret_cast<f32x2_t *>(q + 2 * k), f32x2_t{x[2 * k], x[2 * k + 1]});
    } else {                                             // q + 1 is 8-byte aligned
        st_nt(q, x[0]);
#pragma unroll
        for (int k = 0; k < 3; ++k)
            st_nt(reinterpret_cast<f32x2_t *>(q + 1 + 2 * k), f32x2_t{x[1 + 2 * k], x[2 + 2 * k]});
        st_nt(q + 7, x[7]);
    }
}

// ---- split lane layout on the shifted path (full wavefront blocks)
// Lane l owns the quads l and l + kBlock of the block, as in the vector
// path. A replica is read in 4-element units: 8 bytes of bf16, 16 bytes of
// fp32. A replica d elements past its 16-byte base starts its quads r =
// d mod 4 elements into a unit, so a lane's quad spans its own unit and
// the next. The next unit of half 0 and of half 1 is the next lane's (DPP
// wave shift). For lane 63, half 0's next unit is lane 0's unit of half 1
// (read across lanes; loading it again measured 0.8 points slower), and
// half 1's next unit, past the block, it loads itself: that unit holds the
// block's last element, so no read leaves the units of the buffer's own
// elements.
template <bool GB> struct UnitT;
template <> struct UnitT<true> { typedef uint2 T; };
template <> struct UnitT<false> { typedef uint4 T; };

__device__ __forceinline__ uint2 next_lane(uint2 v) {
    return make_uint2(next_lane(v.x), next_lane(v.y));
}

// Lane 0's value of v, in every lane.
__device__ __forceinline__ uint2 first_lane(uint2 v) {
    return make_uint2((uint32_t)__builtin_amdgcn_readlane((int)v.x, 0),
                      (uint32_t)__builtin_amdgcn_readlane((int)v.y, 0));
}

__device__ __forceinline__ uint4 first_lane(uint4 v) {
    return make_uint4((uint32_t)__builtin_amdgcn_readlane((int)v.x, 0),
                      (uint32_t)__builtin_amdgcn_readlane((int)v.y, 0),
                      (uint32_t)__builtin_amdgcn_readlane((int)v.z, 0),
                      (uint32_t)__builtin_amdgcn_readlane((int)v.w, 0));
}

// Off-phase replicas straddle 128-byte lines: the line a block shares with
// the next block (on another XCD) is fetched twice. With the default cache
// policy the second fetch finds it in the Infinity Cache; non-temporal
// loads measured slower here (75.1% against 75.7% of peak HBM bandwidth,
// seven replicas one element off, 7e9-element shard).
template <bool GB>
__device__ __forceinline__ typename UnitT<GB>::T load_unit(const void *base, int64_t u) {
    if constexpr (GB) {
        return ld_u2<false>(reinterpret_cast<const uint2 *>(base) + u);
    } else {
        return ld_u4<false>(reinterpret_cast<const uint4 *>(base) + u);
    }
}

template <bool GB> struct ShiftUnits {
    typename UnitT<GB>::T a[2], nx[2];     // own unit and next unit of each half
};

// Four elements starting r elements into unit a (then nx).
__device__ __forceinline__ void take4(uint2 a, uint2 nx, int r, float *x) {
    uint32_t w0, w1;
    switch (r) {
    case 0: w0 = a.x; w1 = a.y; break;
    case 1: w0 = __builtin_amdgcn_alignbyte(a.y, a.x, 2);
            w1 = __builtin_amdgcn_alignbyte(nx.x, a.y, 2); break;
    case 2: w0 = a.y; w1 = nx.x; break;
    default: w0 = __builtin_amdgcn_alignbyte(nx.x, a.y, 2);
             w1 = __builtin_amdgcn_alignbyte(nx.y, nx.x, 2); break;
    }
    x[0] = widen_bf16(w0 & 0xFFFFu); x[1] = widen_bf16(w0 >> 16);
    x[2] = widen_bf16(w1 & 0xFFFFu); x[3] = widen_bf16(w1 >> 16);
}

__device__ __forceinline__ void take4(uint4 a, uint4 nx, int r, float *x) {
    const uint32_t c[8] = {a.x, a.y, a.z, a.w, nx.x, nx.y, nx.z, nx.w};
    switch (r) {
    case 0: x[0] = __uint_as_float(c[0]); x[1] = __uint_as_float(c[1]);
            x[2] = __uint_as_float(c[2]); x[3] = __uint_as_float(c[3]); break;
    case 1: x[0] = __uint_as_float(c[1]); x[1] = __uint_as_float(c[2]);
            x[2] = __uint_as_float(c[3]); x[3] = __uint_as_float(c[4]); break;
    case 2: x[0] = __uint_as_float(c[2]); x[1] = __uint_as_float(c[3]);
            x[2] = __uint_as_float(c[4]); x[3] = __uint_as_float(c[5]); break;
    default: x[0] = __uint_as_float(c[3]); x[1] = __uint_as_float(c[4]);
             x[2] = __uint_as_float(c[5]); x[3] = __uint_as_float(c[6]); break;
    }
}

template <int NR, bool GB>
__device__ __forceinline__ void fold_group_split_shift(const ShiftReps<NR> &reps, int q0, int n,
                                                       int64_t ub, float (&s)[kVec]) {
    const int lane = threadIdx.x % 64;
    ShiftUnits<GB> raw[kGroup];
#pragma unroll
    for (int k = 0; k < kGroup; ++k) {
        if (q0 + k < n) {
            const int d = reps.d[q0 + k];
            const int64_t u = ub + (GB ? d / 4 : 0);
            raw[k].a[0] = load_unit<GB>(reps.p[q0 + k], u);
            raw[k].a[1] = load_unit<GB>(reps.p[q0 + k], u + kBlock);
            if ((d & 3) && lane == 63)         // past the block: lane 63 loads it
                raw[k].nx[1] = load_unit<GB>(reps.p[q0 + k], u + kBlock + 1);
        }
    }
#pragma unroll
    for (int k = 0; k < kGroup; ++k) {
        if (q0 + k < n) {
            const int r = reps.d[q0 + k] & 3;
            if (r) {
                const typename UnitT<GB>::T n0 = next_lane(raw[k].a[0]);
                const typename UnitT<GB>::T n1 = next_lane(raw[k].a[1]);
                // the unit after half 0 is lane 0's unit of half 1
                const typename UnitT<GB>::T h1 = first_lane(raw[k].a[1]);
                if (lane != 63) {
                    raw[k].nx[0] = n0;
                    raw[k].nx[1] = n1;
                } else {
                    raw[k].nx[0] = h1;
                }
            } else {
                raw[k].nx[0] = raw[k].a[0];
                raw[k].nx[1] = raw[k].a[1];
            }
            float x[kVec];
            take4(raw[k].a[0], raw[k].nx[0], r, x);
            take4(raw[k].a[1], raw[k].nx[1], r, x + 4);
            if (q0 + k == 0) {
#pragma unroll
                for (int e = 0; e < kVec; ++e) s[e] = x[e];
            } else {
#pragma unroll
                for (int e = 0; e < kVec; ++e) s[e] = s[e] + x[e];
            }
        }
    }
}

// Four bf16 (packed in x, y) to q, which sits d elements past an 8-byte
// boundary (d = 0..3).
__device__ __forceinline__ void store_bf16x4_at(uint16_t *q, int d, uint32_t x, uint32_t y) {
    if (d == 0) {
        st_nt(reinterpret_cast<u32x2_t *>(q), u32x2_t{x, y});
    } else if (d == 2) {
        st_nt(reinterpret_cast<uint32_t *>(q), x);
        st_nt(reinterpret_cast<uint32_t *>(q) + 1, y);
    } else {                                             // q + 1 is 4-byte aligned
        st_nt(q, (uint16_t)(x & 0xFFFFu));
        st_nt(reinterpret_cast<uint32_t *>(q + 1), __builtin_amdgcn_alignbyte(y, x, 2));
        st_nt(q + 3, (uint16_t)(y >> 16));
    }
}

// Four fp32 to q, which sits d elements past a 16-byte boundary.
__device__ __forceinline__ void store_f32x4_at(float *q, int d, const float *x) {
    if (d == 0) {
        st_f4<ZK_NT_OUT>(q, make_float4(x[0], x[1], x[2], x[3]));
    } else if (d == 2) {
        st_nt(reinterpret_cast<f32x2_t *>(q), f32x2_t{x[0], x[1]});
        st_nt(reinterpret_cast<f32x2_t *>(q + 2), f32x2_t{x[2], x[3]});
    } else {                                             // q + 1 is 8-byte aligned
        st_nt(q, x[0]);
        st_nt(reinterpret_cast<f32x2_t *>(q + 1), f32x2_t{x[1], x[2]});
        st_nt(q + 3, x[3]);
    }
}

// Full block blk of the shifted path in the split lane layout.
template <int NR, bool GB, bool PB, bool NTS>
__device__ __forceinline__ void step_block_split_shift(const ShiftReps<NR> &reps, int n,
                                                       bool pow2, float *__restrict__ master,
                                                       float *__restrict__ mom,
                                                       float *__restrict__ var,
                                                       void *__restrict__ out, int dout,
                                                       int64_t blk, const StepScalars &sc) {
    const int64_t q0 = blk * 2 * kBlock + threadIdx.x;    // state quad of half 0
    const int64_t ub = blk * 2 * kBlock + threadIdx.x;    // replica unit of half 0 at d = 0
    constexpr int kSLoad = NTS ? kPolNT : ZK_POL_LOAD_CACHED;
    constexpr int kSStore = NTS ? ZK_POL_STORE_STREAM : ZK_POL_STORE_CACHED;
    constexpr int sbytes = kSpanBytes<4>;
    const int64_t so = blk * (kBlock * kVec);
    const span_t rp = span_of(master + so, sbytes), rm = span_of(mom + so, sbytes),
                 rv = span_of(var + so, sbytes);
    float s[kVec], p[kVec], m[kVec], v[kVec], g[kVec];
    if constexpr (NR > 0 && NR <= 2 * kGroup) {
#pragma unroll
        for (int r = 0; r < NR; r += kGroup) fold_group_split_shift<NR, GB>(reps, r, n, ub, s);
    } else {
#pragma unroll 1
        for (int r = 0; r < n; r += kGroup) fold_group_split_shift<NR, GB>(reps, r, n, ub, s);
    }
    // m and v, then master once the moments are done. Issuing m and v before
    // the replica work, or all three state loads after it, or flat global
    // state accesses measured within a point of this either way (7e9/N=8
    // shard, 7 replicas one element off and 1 replica with the output 3 off,
    // three states per variant interleaved in one process).
    load8_split<kSLoad>(rm, m);
    load8_split<kSLoad>(rv, v);
    if (pow2) {
#pragma unroll
        for (int e = 0; e < kVec; ++e) g[e] = s[e] * sc.inv_n;
    } else {
#pragma unroll
        for (int e = 0; e < kVec; ++e) g[e] = s[e] / sc.nf;
    }
    float u[kVec];
#pragma unroll
    for (int e = 0; e < kVec; ++e) u[e] = adam_moments(g[e], m[e], v[e], sc);
    load8_split<kSLoad>(rp, p);
#pragma unroll
    for (int e = 0; e < kVec; ++e) p[e] = p[e] - u[e];
    store8_split<kSStore>(rp, p);
    store8_split<kSStore>(rm, m);
    store8_split<kSStore>(rv, v);
    const int64_t e0 = 4 * q0, e1 = 4 * (q0 + kBlock);    // first element of each quad
    if (PB) {
        uint16_t *o = reinterpret_cast<uint16_t *>(out);
        const int d = dout & 3;
        store_bf16x4_at(o + e0, d, round_bf16(p[0]) | (round_bf16(p[1]) << 16),
                        round_bf16(p[2]) | (round_bf16(p[3]) << 16));
        store_bf16x4_at(o + e1, d, round_bf16(p[4]) | (round_bf16(p[5]) << 16),
                        round_bf16(p[6]) | (round_bf16(p[7]) << 16));
    } else {
        float *o = reinterpret_cast<float *>(out);
        store_f32x4_at(o + e0, dout, p);
        store_f32x4_at(o + e1, dout, p + 4);
    }
}

// Vector j of the shifted path: state aligned; replicas read through
// their aligned bases; the output (element pointer of the range's first
// element, dout elements past a 16-byte boundary) written at its phase.
template <int NR, bool GB, bool PB, bool DS>
__global__ void __launch_bounds__(kBlock)
step_shift_kernel(ShiftReps<NR> reps, int nrep, float *__restrict__ master,
                  float *__restrict__ mom, float *__restrict__ var, void *__restrict__ out,
                  int dout, int64_t nvec, int64_t nbw, int head, int tail, int nt_state,
                  ScalarArg<DS> sa) {
    const StepScalars sc = scalars(sa);
    const int n = NR > 0 ? NR : nrep;
    constexpr bool kPow2 = NR > 0 && (NR & (NR - 1)) == 0;
    const bool pow2 = kPow2 || (NR == 0 && sc.n_pow2);
    const int64_t nfull = nvec / kBlock;
    const int64_t w = blockIdx.x;
    if (w < nbw) {                                   // full blocks, as step_vec_kernel
        if (nt_state) {
            for (int64_t blk = w; blk < nfull; blk += nbw)
                step_block_split_shift<NR, GB, PB, true>(reps, n, pow2, master, mom, var, out,
                                                         dout, blk, sc);
        } else {
            for (int64_t blk = w; blk < nfull; blk += nbw)
                step_block_split_shift<NR, GB, PB, false>(reps, n, pow2, master, mom, var, out,
                                                          dout, blk, sc);
        }
        return;
    }
    if (!(w == nbw && nfull * kBlock < nvec)) {      // head and tail, as step_vec_kernel
        for (int k = threadIdx.x; k < head + tail; k += kBlock) {
            const int64_t e = k < head ? (int64_t)(k - head) : nvec * kVec + (k - head);
            step_one<NR, GB, PB>(reps, n, master, mom, var, out, e, sc);
        }
        return;
    }
    const int64_t j = nfull * kBlock + threadIdx.x;  // the partial block
    if (j >= nvec) return;
    const bool self_next = (threadIdx.x % 64) == 63 || j + 1 == nvec;
    float p[kVec], m[kVec], v[kVec];
    load8(master, j, p);
    load8(mom, j, m);
    load8(var, j, v);

    float s[kVec];
    if constexpr (NR > 0 && NR <= 2 * kGroup) {
#pragma unroll
        for (int q0 = 0; q0 < NR; q0 += kGroup)
            fold_group_shift<NR, GB>(reps, q0, n, j, self_next, s);
    } else {
#pragma unroll 1
        for (int q0 = 0; q0 < n; q0 += kGroup)
            fold_group_shift<NR, GB>(reps, q0, n, j, self_next, s);
    }
    float g[kVec];
    if (pow2) {
#pragma unroll
        for (int e = 0; e < kVec; ++e) g[e] = s[e] * sc.inv_n;
    } else {
#pragma unroll
        for (int e = 0; e < kVec; ++e) g[e] = s[e] / sc.nf;
    }
#pragma unroll
    for (int e = 0; e < kVec; ++e) adam_update(g[e], p[e], m[e], v[e], sc);

    store8<false>(master, j, p);
    store8<false>(mom, j, m);
    store8<false>(var, j, v);
    if (PB) {
        uint4 o;
        o.x = round_bf16(p[0]) | (round_bf16(p[1]) << 16);
        o.y = round_bf16(p[2]) | (round_bf16(p[3]) << 16);
        o.z = round_bf16(p[4]) | (round_bf16(p[5]) << 16);
        o.w = round_bf16(p[6]) | (round_bf16(p[7]) << 16);
        store_bf16x8_at(reinterpret_cast<uint16_t *>(out) + kVec * j, dout, o);
    } else {
        store_f32x8_at(reinterpret_cast<float *>(out) + kVec * j, dout, p);
    }
}

// ------------------------------------------------ per-parameter (dim-0) layout
// Each segment is one parameter's local row shard: its replica pointers
// (already at this rank's first row), its output shard, and its place in
// the rank's master/m/v. A workgroup takes one kBlock*8-element chunk of
// one segment. In segments whose streams are all 16-byte aligned, a full
// chunk takes the split lane layout and a partial one the vector step on
// its whole vectors; the rest, and every segment's last partial vector,
// take the element step.
// Segments per launch: as many as keep the table within 4 KiB of kernel
// arguments (32 with up to 8 replica pointers each, 16 with 16).
constexpr int fsdp_batch(int nr) { return nr <= 8 ? 32 : 16; }

template <int NR>
struct FsdpBatch {
    static constexpr int kMax = fsdp_batch(NR);
    Reps<NR> reps[kMax];
    void *out[kMax];
    int64_t state_off[kMax];
    int64_t numel[kMax];
    int64_t blk0[kMax + 1];
    int nseg;
};
static_assert(sizeof(FsdpBatch<8>) <= 4096 && sizeof(FsdpBatch<kFsdpMaxWorld>) <= 4096,
              "segment table must fit the kernel arguments");

template <int NR, bool EXACT, bool GB, bool PB, bool DS>
__global__ void __launch_bounds__(kBlock)
fsdp_step_kernel(FsdpBatch<NR> b, int nrep, float *__restrict__ master,
                 float *__restrict__ mom, float *__restrict__ var, int nt_state,
                 ScalarArg<DS> sa) {
    const StepScalars sc = scalars(sa);
    const int64_t w = blockIdx.x;
    int lo = 0, hi = b.nseg - 1;                 // last segment with blk0 <= w
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (b.blk0[mid] <= w) lo = mid;
        else hi = mid - 1;
    }
    const int sgi = lo;
    const int n = EXACT ? NR : nrep;
    constexpr bool kPow2 = EXACT && (NR & (NR - 1)) == 0;
    const bool pow2 = kPow2 || (!EXACT && sc.n_pow2);
    const int64_t numel = b.numel[sgi];
    float *ms = master + b.state_off[sgi];
    float *mm = mom + b.state_off[sgi];
    float *vs = var + b.state_off[sgi];
    void *out = b.out[sgi];
    const Reps<NR> &reps = b.reps[sgi];
    bool aligned = ((uintptr_t)out % 16) == 0 && ((uintptr_t)ms % 16) == 0;
    for (int q = 0; q < n; ++q) aligned = aligned && ((uintptr_t)reps.p[q] % 16) == 0;
    const int64_t chunk = w - b.blk0[sgi];
    if (aligned && (chunk + 1) * kBlock * kVec <= numel) {
        if (nt_state)
            step_block_split<NR, GB, PB, true, ZK_NT_GRAD>(reps, n, pow2, ms, mm, vs, out, chunk,
                                                           sc);
        else
            step_block_split<NR, GB, PB, false, ZK_NT_GRAD>(reps, n, pow2, ms, mm, vs, out, chunk,
                                                            sc);
        return;
    }
    const int64_t j = chunk * kBlock + threadIdx.x;     // vector index
    if (j * kVec >= numel) return;
    if (aligned && (j + 1) * kVec <= numel) {
        step_vector<NR, GB, PB>(reps, n, pow2, ms, mm, vs, out, j, sc);
    } else {
        const int64_t end = (j + 1) * kVec < numel ? (j + 1) * kVec : numel;
        for (int64_t i = j * kVec; i < end; ++i) step_one<NR, GB, PB>(reps, n, ms, mm, vs, out, i, sc);
    }
}

template <bool DS>
ScalarArg<DS> scalar_arg(const StepScalars &sc, const StepScalars *dev);
template <>
inline ScalarArg<false> scalar_arg<false>(const StepScalars &sc, const StepScalars *) {
    return ScalarArg<false>{sc};
}
template <>
inline ScalarArg<true> scalar_arg<true>(const StepScalars &, const StepScalars *dev) {
    return ScalarArg<true>{dev};
}

template <int NR, bool EXACT, bool GB, bool PB, bool DS>
hipError_t launch_fsdp_typed(const FsdpArgs &a, hipStream_t stream) {
    const int64_t per_block = (int64_t)kBlock * kVec;
    int i = 0;
    while (i < a.nseg) {
        FsdpBatch<NR> b = {};
        b.nseg = 0;
        int64_t blocks = 0;
        while (i < a.nseg && b.nseg < FsdpBatch<NR>::kMax) {
            const FsdpSegment &sg = a.segs[i++];
            if (sg.numel <= 0) continue;
            for (int q = 0; q < a.n; ++q) b.reps[b.nseg].p[q] = sg.grads[q];
            b.out[b.nseg] = sg.out;
            b.state_off[b.nseg] = sg.state_off;
            b.numel[b.nseg] = sg.numel;
            b.blk0[b.nseg] = blocks;
            blocks += (sg.numel + per_block - 1) / per_block;
            b.nseg++;
        }
        if (b.nseg == 0) continue;
        b.blk0[b.nseg] = blocks;
        if (blocks > (int64_t)(0xFFFFFFFFu / kBlock)) return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL((fsdp_step_kernel<NR, EXACT, GB, PB, DS>), dim3((unsigned)blocks),
                           dim3(kBlock), ZK_FSDP_LDS, stream, b, a.n, a.master, a.m, a.v,
                           a.stream_state ? 1 : 0, scalar_arg<DS>(a.sc, a.sc_dev));
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <bool GB, bool PB, bool DS>
hipError_t launch_fsdp_dtype(const FsdpArgs &a, hipStream_t stream) {
    switch (a.n) {
    case 1: return launch_fsdp_typed<1, true, GB, PB, DS>(a, stream);
    case 2: return launch_fsdp_typed<2, true, GB, PB, DS>(a, stream);
    case 4: return launch_fsdp_typed<4, true, GB, PB, DS>(a, stream);
    case 8: return launch_fsdp_typed<8, true, GB, PB, DS>(a, stream);
    default: return launch_fsdp_typed<kFsdpMaxWorld, false, GB, PB, DS>(a, stream);
    }
}

// Workgroups that take the full blocks of a vector-path launch: one per
// block, or at most a.max_workgroups (each then walks blocks at that stride).
inline int64_t block_workgroups(const StepArgs &a, int64_t nfull) {
    return (a.max_workgroups > 0 && a.max_workgroups < nfull) ? a.max_workgroups : nfull;
}

// Dynamic LDS a step launch reserves (and never touches) to cap the
// workgroups per compute unit. A capped launch already holds few
// workgroups per compute unit and reserves none, so that kernels on other
// streams find LDS beside it.
inline unsigned occupancy_lds(const StepArgs &a, unsigned lds) {
    return a.max_workgroups > 0 ? 0u : lds;
}

template <int NR, bool GB, bool PB, bool DS>
hipError_t launch_vec(const StepArgs &a, int64_t nvec, int head, int tail,
                      hipStream_t stream) {
    Reps<NR> reps = {};
    for (int q = 0; q < a.n; ++q) reps.p[q] = a.grads[q];
    const int64_t nfull = nvec / kBlock, nbw = block_workgroups(a, nfull);
    const int64_t grid = nbw + (nfull * kBlock < nvec ? 1 : 0) + (head + tail > 0 ? 1 : 0);
    // a dispatch holds at most 2^32-1 work-items
    if (grid > (int64_t)(0xFFFFFFFFu / kBlock)) return hipErrorInvalidConfiguration;
    // replica cache policy as a template parameter: a runtime choice inside
    // the kernel measured 2 points slower on line-aligned streams
    const dim3 g((unsigned)grid), b(kBlock);
    constexpr unsigned kLds = (NR > kGroup && NR <= 2 * kGroup) ? ZK_STEP_LDS_WIDE : ZK_STEP_LDS;
    const unsigned lds = occupancy_lds(a, kLds);
    const int nts = a.stream_state ? 1 : 0;
    if (a.nt_grad)
        hipLaunchKernelGGL((step_vec_kernel<NR, GB, PB, DS, true>), g, b, lds, stream, reps, a.n,
                           a.master, a.m, a.v, a.out, nvec, nbw, head, tail, nts,
                           scalar_arg<DS>(a.sc, a.sc_dev));
    else
        hipLaunchKernelGGL((step_vec_kernel<NR, GB, PB, DS, false>), g, b, lds, stream, reps,
                           a.n, a.master, a.m, a.v, a.out, nvec, nbw, head, tail, nts,
                           scalar_arg<DS>(a.sc, a.sc_dev));
    return hipGetLastError();
}

template <bool GB, bool PB, bool DS>
hipError_t dispatch_vec(const StepArgs &a, int64_t nvec, int head, int tail,
                        hipStream_t stream) {
    switch (a.n) {
    case 1: return launch_vec<1, GB, PB, DS>(a, nvec, head, tail, stream);
    case 2: return launch_vec<2, GB, PB, DS>(a, nvec, head, tail, stream);
    case 4: return launch_vec<4, GB, PB, DS>(a, nvec, head, tail, stream);
    case 8: return launch_vec<8, GB, PB, DS>(a, nvec, head, tail, stream);
    case 16: return launch_vec<16, GB, PB, DS>(a, nvec, head, tail, stream);
    case 64: return launch_vec<64, GB, PB, DS>(a, nvec, head, tail, stream);
    default: return launch_vec<0, GB, PB, DS>(a, nvec, head, tail, stream);
    }
}

template <bool GB, bool PB, bool DS>
hipError_t launch_elem(const StepArgs &a, int64_t begin, int64_t end, hipStream_t stream) {
    Reps<0> reps = {};
    for (int q = 0; q < a.n; ++q) reps.p[q] = a.grads[q];
    int64_t want = (end - begin + kElemBlock - 1) / kElemBlock;
    int64_t cap = (int64_t)a.num_cus * 8;
    int grid = (int)(want < cap ? want : cap);
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL((step_elem_kernel<GB, PB, DS>), dim3(grid), dim3(kElemBlock), 0, stream,
                       reps, a.n, a.master, a.m, a.v, a.out, begin, end,
                       scalar_arg<DS>(a.sc, a.sc_dev));
    return hipGetLastError();
}

// Cache-line size of the L2: a wavefront's block of a stream (1 KiB of
// bf16, 2 KiB of fp32) fills whole lines when the vector range starts on a
// line. Adjacent workgroups run on different XCDs, each with its own L2, so
// a line shared by two blocks is fetched, or written, twice.
constexpr uintptr_t kLine = 128;
constexpr int kLineHead = 64;        // bf16 elements per line: heads below this

inline bool at(const void *p, int esize, int h, uintptr_t align) {
    return ((uintptr_t)p + (uintptr_t)esize * (uintptr_t)h) % align == 0;
}

inline bool state_at(const StepArgs &a, int h, uintptr_t align) {
    return at(a.master, 4, h, align) && at(a.m, 4, h, align) && at(a.v, 4, h, align);
}

// Every stream (replicas, master/m/v, output) at element h on an `align`
// boundary (element h of a bf16 stream at byte 2h, of an fp32 stream at 4h).
inline bool all_at(const StepArgs &a, int h, uintptr_t align) {
    const int ge = a.grad_bf16 ? 2 : 4, oe = a.out_bf16 ? 2 : 4;
    bool ok = state_at(a, h, align) && at(a.out, oe, h, align);
    for (int q = 0; q < a.n && ok; ++q) ok = at(a.grads[q], ge, h, align);
    return ok;
}

// Head of the vector path: the smallest h < 64 at which every stream sits
// on a 128-byte line and at least one vector follows; failing that, the
// smallest h < 8 at which every stream sits on a 16-byte boundary; -1 if
// neither exists.
inline int common_head(const StepArgs &a) {
    for (int h = 0; h < kLineHead && a.shard - h >= kVec; ++h)
        if (all_at(a, h, kLine)) return h;
    for (int h = 0; h < kVec; ++h)
        if (all_at(a, h, 16)) return h;
    return -1;
}

// Head for the shifted path: an h < 64 at which master, m and v are 16-byte
// aligned, chosen for, in order: the state on a 128-byte line, the most
// caller streams on a line (the output counts double: its unaligned form
// also costs more instructions than a replica's), the most on a 16-byte
// boundary; the smallest such h. -1 if no h aligns the state or a buffer
// is not naturally aligned.
inline int shifted_head(const StepArgs &a) {
    const int ge = a.grad_bf16 ? 2 : 4, oe = a.out_bf16 ? 2 : 4;
    if ((uintptr_t)a.out % oe) return -1;
    for (int q = 0; q < a.n; ++q)
        if ((uintptr_t)a.grads[q] % ge) return -1;
    int best = -1;
    int64_t best_score = -1;
    for (int h = 0; h < kLineHead; ++h) {
        if (!state_at(a, h, 16)) continue;
        int64_t lines = 2 * at(a.out, oe, h, kLine), vecs = 2 * at(a.out, oe, h, 16);
        for (int q = 0; q < a.n; ++q) {
            lines += at(a.grads[q], ge, h, kLine);
            vecs += at(a.grads[q], ge, h, 16);
        }
        const int64_t score = (int64_t)state_at(a, h, kLine) * (1 << 20) + lines * 1024 + vecs;
        if (score > best_score) {
            best = h;
            best_score = score;
        }
    }
    return best;
}

template <int NR, bool GB, bool PB, bool DS>
hipError_t launch_shift(const StepArgs &a, int h, int64_t nvec, int tail, hipStream_t stream) {
    const int ge = a.grad_bf16 ? 2 : 4, oe = a.out_bf16 ? 2 : 4;
    ShiftReps<NR> reps = {};
    for (int q = 0; q < a.n; ++q) {
        const uintptr_t e0 = (uintptr_t)a.grads[q] + (uintptr_t)ge * h;
        reps.d[q] = (uint8_t)((e0 % 16) / ge);
        reps.p[q] = (const void *)(e0 - e0 % 16);
    }
    void *out = (char *)a.out + (int64_t)oe * h;
    const int dout = (int)(((uintptr_t)out % 16) / oe);
    const int64_t nfull = nvec / kBlock, nbw = block_workgroups(a, nfull);
    const int64_t grid = nbw + (nfull * kBlock < nvec ? 1 : 0) + (h + tail > 0 ? 1 : 0);
    if (grid > (int64_t)(0xFFFFFFFFu / kBlock)) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((step_shift_kernel<NR, GB, PB, DS>), dim3((unsigned)grid), dim3(kBlock),
                       occupancy_lds(a, ZK_SHIFT_LDS), stream, reps, a.n, a.master + h, a.m + h, a.v + h, out, dout,
                       nvec, nbw, h, tail, a.stream_state ? 1 : 0,
                       scalar_arg<DS>(a.sc, a.sc_dev));
    return hipGetLastError();
}

template <bool GB, bool PB, bool DS>
hipError_t dispatch_shift(const StepArgs &a, int h, int64_t nvec, int tail, hipStream_t stream) {
    switch (a.n) {
    case 1: return launch_shift<1, GB, PB, DS>(a, h, nvec, tail, stream);
    case 2: return launch_shift<2, GB, PB, DS>(a, h, nvec, tail, stream);
    case 4: return launch_shift<4, GB, PB, DS>(a, h, nvec, tail, stream);
    case 8: return launch_shift<8, GB, PB, DS>(a, h, nvec, tail, stream);
    case 16: return launch_shift<16, GB, PB, DS>(a, h, nvec, tail, stream);
    case 64: return launch_shift<64, GB, PB, DS>(a, h, nvec, tail, stream);
    default: return launch_shift<0, GB, PB, DS>(a, h, nvec, tail, stream);
    }
}

// Element head [0, h), vector range and element tail, in one launch.
template <bool GB, bool PB, bool DS>
hipError_t step_shifted(const StepArgs &a, int h, hipStream_t stream) {
    const int64_t nvec = (a.shard - h) / kVec;
    const int tail = (int)(a.shard - h - nvec * kVec);
    return dispatch_shift<GB, PB, DS>(a, h, nvec, tail, stream);
}

template <bool GB, bool PB, bool DS>
hipError_t step_typed(const StepArgs &a, hipStream_t stream) {
    // Vector path from the head h that common_head chooses; the h elements
    // before it and the ragged tail take the element step (same arithmetic)
    // in one extra workgroup of the same launch. Buffers at mixed phases
    // take the shifted vector path; only buffers that are not naturally
    // aligned, or shards shorter than the head plus one vector, run on the
    // element path alone.
    const int h = common_head(a);
    if (h < 0) {
        const int hs = shifted_head(a);
        if (hs >= 0 && a.shard - hs >= kVec) return step_shifted<GB, PB, DS>(a, hs, stream);
        return launch_elem<GB, PB, DS>(a, 0, a.shard, stream);
    }
    if (a.shard - h < kVec) return launch_elem<GB, PB, DS>(a, 0, a.shard, stream);
    const int64_t nvec = (a.shard - h) / kVec;
    const int tail = (int)(a.shard - h - nvec * kVec);
    StepArgs b = a;
    // non-temporal replica loads only where every stream sits on whole
    // 128-byte lines: with the 16-byte head, blocks straddle lines and the
    // default policy lets a shared line's second fetch hit the Infinity
    // Cache (measured 76.7% against 73.9% of peak HBM bandwidth, eight
    // replicas 16 bytes off a line, 7e9-element shard; level on lines)
    b.nt_grad = ZK_NT_GRAD && all_at(a, h, kLine);
    const void *shifted[ZERO_MAX_WORLD];
    const int ge = a.grad_bf16 ? 2 : 4, oe = a.out_bf16 ? 2 : 4;
    for (int q = 0; q < a.n; ++q) shifted[q] = (const char *)a.grads[q] + (int64_t)ge * h;
    b.grads = shifted;
    b.master = a.master + h;
    b.m = a.m + h;
    b.v = a.v + h;
    b.out = (char *)a.out + (int64_t)oe * h;
    return dispatch_vec<GB, PB, DS>(b, nvec, h, tail, stream);
}

// ------------------------------------------------------------ segment copy

// Segments per launch. 120 would fit the arguments, but every 1 KiB
// workgroup's binary search then takes one more dependent step: measured
// 2.7% slower on the 291- and 364-tensor Llama flattens (5% faster on the
// 148-tensor GPT-2 list, which needs one launch fewer).
constexpr int kSegBatch = 64;
constexpr int kCopyBlock = ZK_COPY_BLOCK;
constexpr int64_t kChunk = (int64_t)kCopyBlock * 16;   // bytes per workgroup
constexpr int64_t kCopyLine = 128;

// A segment's chunks are cut on its destination's 128-byte lines: chunk k
// covers the bytes from line boundary base + k * kChunk on, where base is the
// start of the line holding the first destination byte. Every chunk but a
// segment's first and last then writes whole lines, whatever the
// destination's alignment, and no line is written by two workgroups inside
// the segment. (Cut from the segment's first byte instead, the chunks of an
// unflatten into tensors 2 bytes off a line each began and ended with
// element stores into lines shared with the next workgroup: 55% of 8 TB/s
// on the Llama-7B list, against 79% on the line grid.) A batch whose
// destinations all start on a line takes the plain grid, chunk k at byte
// k * kChunk: the same chunks, with a shorter scalar prologue (0.6 points
// of 8 TB/s on the aligned Llama-7B flatten).
__host__ __device__ __forceinline__ int64_t chunk_back(const void *dst) {
    return (int64_t)((uintptr_t)dst & (uintptr_t)(kCopyLine - 1));
}

struct SegBatch {
    const char *src[kSegBatch];
    char *dst[kSegBatch];
    int64_t nbytes[kSegBatch];
    int64_t blk0[kSegBatch + 1];              // prefix of workgroup counts
    int nseg;
    int esize;
};
static_assert(sizeof(SegBatch) <= 4096, "segment table must fit the kernel arguments");

template <typename T>
__device__ __forceinline__ void copy_elems(const char *src, char *dst, int64_t nbytes) {
    const int64_t n = nbytes / (int64_t)sizeof(T);
    for (int64_t k = threadIdx.x; k < n; k += kCopyBlock) {
        T x = src ? reinterpret_cast<const T *>(src)[k] : T(0);
        reinterpret_cast<T *>(dst)[k] = x;
    }
}

__device__ __forceinline__ void copy_elems_any(const char *src, char *dst, int64_t nbytes, int esize) {
    if (esize == 4) copy_elems<uint32_t>(src, dst, nbytes);
    else copy_elems<uint16_t>(src, dst, nbytes);
}

// Workgroup w copies one chunk of one segment: an element-wise head up to
// the destination's next 16-byte boundary, then one 16-byte
// vector per lane, then an element-wise tail. Where source and destination
// share their offset within 16 bytes, the vector loads are aligned and
// non-temporal; otherwise each is one plain 16-byte load at the source's
// own alignment (gfx950 takes wide global loads at any element alignment;
// an element-by-element copy of such segments, as from tensors that sit an
// odd number of elements apart, reached 35% of 8 TB/s on the Llama-7B list
// against 79% this way).
template <bool LG>
__global__ void __launch_bounds__(kCopyBlock) copy_segments_kernel(SegBatch b) {
    const int64_t w = blockIdx.x;
    int lo = 0, hi = b.nseg - 1;              // last segment with blk0 <= w
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (b.blk0[mid] <= w) lo = mid;
        else hi = mid - 1;
    }
    const int s = lo;
    const int64_t back = LG ? chunk_back(b.dst[s]) : 0;
    const int64_t k = w - b.blk0[s];
    const int64_t beg = (LG && k == 0) ? 0 : k * kChunk - back;
    int64_t end = (k + 1) * kChunk - back;
    if (end > b.nbytes[s]) end = b.nbytes[s];
    const int64_t len = end - beg;
    if (len <= 0) return;
    const char *src = b.src[s] ? b.src[s] + beg : nullptr;
    char *dst = b.dst[s] + beg;

    const unsigned da = (unsigned)((uintptr_t)dst & 15u);
    const unsigned sa = src ? (unsigned)((uintptr_t)src & 15u) : da;
    int64_t head = (int64_t)((16u - da) & 15u);
    if (head > len) head = len;
    copy_elems_any(src, dst, head, b.esize);
    const int64_t nv = (len - head) / 16;
    // a chunk is one 16-byte vector per lane, through buffer instructions
    // over the chunk (stores non-temporal at device scope)
    const span_t rd = span_of(dst + head, (int)(nv * 16));
    if (!src) {
        for (int64_t k = threadIdx.x; k < nv; k += kCopyBlock)
            bst_u4<ZK_POL_COPY_STORE>(rd, (int)(16 * k), make_uint4(0u, 0u, 0u, 0u));
    } else if (sa == da) {
        const span_t rs = span_of(src + head, (int)(nv * 16));
        for (int64_t k = threadIdx.x; k < nv; k += kCopyBlock)
            bst_u4<ZK_POL_COPY_STORE>(rd, (int)(16 * k), bld_u4<kPolNT>(rs, (int)(16 * k)));
    } else {
        const char *s1 = src + head;
        for (int64_t k = threadIdx.x; k < nv; k += kCopyBlock) {
            uint4 v;
            __builtin_memcpy(&v, s1 + 16 * k, sizeof v);
            bst_u4<ZK_POL_COPY_STORE>(rd, (int)(16 * k), v);
        }
    }
    const int64_t done = head + nv * 16;
    copy_elems_any(src ? src + done : nullptr, dst + done, len - done, b.esize);
}

// ---------------------------------------------------------- master load
// master[i] = fp32(flat[i]), m[i] = v[i] = 0. The launcher starts the vector
// range at the first element h where master, m and v sit on a 128-byte
// line, so that every store instruction writes whole lines (blocks that
// split lines with the next block's workgroup, on another XCD, measured
// 60% of peak HBM bandwidth on the Llama-13B rank-7 shard).
// A full wavefront block (8 * kBlock elements) takes the split lane layout
// of the fused step: lane l writes the quads l and l + kBlock, so every
// store instruction covers one contiguous 1 KiB span of each state array.
// A lane reads its source quad (8 bytes of bf16, 16 of fp32) with one wide
// load: non-temporal where the source shares the state's 16-byte phase
// (SA), a plain one at the source's own alignment otherwise (gfx950 takes
// wide global loads at any element alignment). The h head elements and the
// tail after the last full block take one extra workgroup, element by
// element.
template <bool FB>
__device__ __forceinline__ float src_elem(const void *flat, int64_t i) {
    return FB ? widen_bf16(reinterpret_cast<const uint16_t *>(flat)[i])
              : reinterpret_cast<const float *>(flat)[i];
}

template <bool FB, bool SA>
__device__ __forceinline__ float4 src_quad(const void *flat, int64_t e) {
    if constexpr (FB) {
        const uint16_t *p = reinterpret_cast<const uint16_t *>(flat) + e;
        uint2 w;
        if constexpr (SA) w = ld_u2<true>(p);
        else __builtin_memcpy(&w, p, sizeof w);
        return make_float4(widen_bf16(w.x & 0xFFFFu), widen_bf16(w.x >> 16),
                           widen_bf16(w.y & 0xFFFFu), widen_bf16(w.y >> 16));
    } else {
        const float *p = reinterpret_cast<const float *>(flat) + e;
        if constexpr (SA) return ld_f4<true>(p);
        float4 v;
        __builtin_memcpy(&v, p, sizeof v);
        return v;
    }
}

template <bool FB, bool SA>
__global__ void __launch_bounds__(kBlock)
load_master_kernel(const void *__restrict__ flat, float *__restrict__ master,
                   float *__restrict__ mom, float *__restrict__ var, int64_t shard, int head,
                   int64_t nblk) {
    constexpr int64_t per = (int64_t)kVec * kBlock;
    if ((int64_t)blockIdx.x >= nblk) {                 // head and tail
        const int64_t t0 = head + nblk * per;
        const int64_t rest = head + (shard - t0);
        for (int64_t k = threadIdx.x; k < rest; k += kBlock) {
            const int64_t i = k < head ? k : t0 + (k - head);
            master[i] = src_elem<FB>(flat, i);
            mom[i] = 0.0f;
            var[i] = 0.0f;
        }
        return;
    }
    const int64_t e0 = head + (int64_t)blockIdx.x * per + 4 * (int64_t)threadIdx.x;
    const int64_t e1 = e0 + 4 * kBlock;
    const float4 a = src_quad<FB, SA>(flat, e0), b = src_quad<FB, SA>(flat, e1);
    const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
    st_f4<true>(master + e0, a);
    st_f4<true>(master + e1, b);
    st_f4<true>(mom + e0, z);
    st_f4<true>(mom + e1, z);
    st_f4<true>(var + e0, z);
    st_f4<true>(var + e1, z);
}

// ------------------------------------------------------ device step schedule
// One lane: the scalars of the schedule's current step, then t advances.
// Bias corrections come from the host-built table (binary64 power, one
// rounding to binary32); past its end both are exactly 1.
__global__ void __launch_bounds__(64)
begin_step_kernel(DevSchedule *ds, const float *__restrict__ table, int64_t len,
                  StepScalars base, StepScalars *out) {
    if (threadIdx.x != 0) return;
    const int64_t t = ds->t;
    int64_t i = t < 1 ? 1 : t;
    if (i > len) i = len;
    StepScalars sc = base;
    sc.lr = ds->lr;
    sc.bc1 = table[2 * (i - 1)];
    sc.bc2 = table[2 * (i - 1) + 1];
    *out = sc;
    ds->t = t + 1;
}

// dst[i] = c.w[i] for i < c.n: words passed by value in the kernel
// arguments, so a host table reaches device memory without a copy call.
__global__ void __launch_bounds__(256) fill_words_kernel(uint32_t *dst, WordChunk c) {
    for (int i = threadIdx.x; i < c.n; i += 256) dst[i] = c.w[i];
}

__global__ void __launch_bounds__(64)
set_schedule_kernel(DevSchedule *ds, int64_t t, float lr) {
    if (threadIdx.x != 0) return;
    if (t >= 1) ds->t = t;
    ds->lr = lr;
}

}  // namespace

hipError_t launch_begin_step(DevSchedule *ds, const float *table, int64_t len,
                             const StepScalars &base, StepScalars *out, hipStream_t stream) {
    hipLaunchKernelGGL(begin_step_kernel, dim3(1), dim3(64), 0, stream, ds, table, len, base, out);
    return hipGetLastError();
}

hipError_t launch_fill_words(uint32_t *dst, const WordChunk &c, hipStream_t stream) {
    if (c.n < 0 || c.n > kWordChunk) return hipErrorInvalidValue;
    if (c.n == 0) return hipSuccess;
    hipLaunchKernelGGL(fill_words_kernel, dim3(1), dim3(256), 0, stream, dst, c);
    return hipGetLastError();
}

hipError_t launch_set_schedule(DevSchedule *ds, int64_t t, float lr, hipStream_t stream) {
    hipLaunchKernelGGL(set_schedule_kernel, dim3(1), dim3(64), 0, stream, ds, t, lr);
    return hipGetLastError();
}

hipError_t launch_step(const StepArgs &a, hipStream_t stream) {
    if (a.shard <= 0) return hipSuccess;
    if (a.sc_dev) {
        if (a.grad_bf16)
            return a.out_bf16 ? step_typed<true, true, true>(a, stream)
                              : step_typed<true, false, true>(a, stream);
        return a.out_bf16 ? step_typed<false, true, true>(a, stream)
                          : step_typed<false, false, true>(a, stream);
    }
    if (a.grad_bf16) {
        return a.out_bf16 ? step_typed<true, true, false>(a, stream)
                          : step_typed<true, false, false>(a, stream);
    }
    return a.out_bf16 ? step_typed<false, true, false>(a, stream)
                      : step_typed<false, false, false>(a, stream);
}

hipError_t launch_fsdp_step(const FsdpArgs &a, hipStream_t stream) {
    if (a.n < 1 || a.n > kFsdpMaxWorld) return hipErrorInvalidValue;
    if (a.sc_dev) {
        if (a.grad_bf16)
            return a.out_bf16 ? launch_fsdp_dtype<true, true, true>(a, stream)
                              : launch_fsdp_dtype<true, false, true>(a, stream);
        return a.out_bf16 ? launch_fsdp_dtype<false, true, true>(a, stream)
                          : launch_fsdp_dtype<false, false, true>(a, stream);
    }
    if (a.grad_bf16) {
        return a.out_bf16 ? launch_fsdp_dtype<true, true, false>(a, stream)
                          : launch_fsdp_dtype<true, false, false>(a, stream);
    }
    return a.out_bf16 ? launch_fsdp_dtype<false, true, false>(a, stream)
                      : launch_fsdp_dtype<false, false, false>(a, stream);
}

hipError_t launch_copy_segments(const Segment *segs, int nseg, int esize, hipStream_t stream) {
    // A dispatch holds at most 2^32-1 work-items; long segments are cut into
    // pieces at multiples of the chunk size (which keeps every piece's
    // source/destination alignment relation and its destination's line
    // phase) and batched under that limit.
    const int64_t max_blocks = (int64_t)(0xFFFFFFFFu / kCopyBlock);
    const int64_t max_piece = kChunk * (max_blocks / 4);
    int i = 0;
    int64_t done = 0;                          // bytes of segs[i] already issued
    while (i < nseg) {
        SegBatch b;
        b.esize = esize;
        b.nseg = 0;
        int64_t blocks = 0;
        bool lg = false;
        while (i < nseg && b.nseg < kSegBatch) {
            const Segment &s = segs[i];
            int64_t len = s.nbytes - done;
            if (len <= 0) { ++i; done = 0; continue; }
            if (len > max_piece) len = max_piece;
            char *dst = static_cast<char *>(s.dst) + done;
            const int64_t nb = (len + chunk_back(dst) + kChunk - 1) / kChunk;
            lg = lg || chunk_back(dst) != 0;
            if (blocks + nb > max_blocks) break;
            b.src[b.nseg] = s.src ? static_cast<const char *>(s.src) + done : nullptr;
            b.dst[b.nseg] = dst;
            b.nbytes[b.nseg] = len;
            b.blk0[b.nseg] = blocks;
            blocks += nb;
            b.nseg++;
            done += len;
            if (done >= s.nbytes) { ++i; done = 0; }
        }
        if (b.nseg == 0) continue;
        b.blk0[b.nseg] = blocks;
        if (lg)
            hipLaunchKernelGGL(copy_segments_kernel<true>, dim3((unsigned)blocks),
                               dim3(kCopyBlock), 0, stream, b);
        else
            hipLaunchKernelGGL(copy_segments_kernel<false>, dim3((unsigned)blocks),
                               dim3(kCopyBlock), 0, stream, b);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_load_master(const void *flat, bool flat_bf16, float *master, float *m,
                              float *v, int64_t shard, hipStream_t stream) {
    if (shard <= 0) return hipSuccess;
    constexpr int64_t per = (int64_t)kVec * kBlock;
    // master, m and v share their phase within a line (the context
    // allocates them that way); h puts them on a 128-byte line
    const uintptr_t ph = (uintptr_t)master & 127u;
    int head = (int)(((128u - ph) & 127u) / 4u);
    if (((uintptr_t)m & 127u) != ph || ((uintptr_t)v & 127u) != ph) return hipErrorInvalidValue;
    if (head > shard) head = (int)shard;
    const int64_t nblk = (shard - head) / per;
    const int64_t grid = nblk + ((shard - nblk * per) > 0 ? 1 : 0);
    if (grid > (int64_t)(0xFFFFFFFFu / kBlock)) return hipErrorInvalidConfiguration;
    const int es = flat_bf16 ? 2 : 4;
    const uintptr_t src_h = (uintptr_t)flat + (uintptr_t)es * (uintptr_t)head;
    const bool sa = src_h % (uintptr_t)(4 * es) == 0;
    const dim3 g((unsigned)grid), blk(kBlock);
    if (flat_bf16) {
        if (sa)
            hipLaunchKernelGGL((load_master_kernel<true, true>), g, blk, ZK_K0_LDS, stream, flat, master,
                               m, v, shard, head, nblk);
        else
            hipLaunchKernelGGL((load_master_kernel<true, false>), g, blk, ZK_K0_LDS, stream, flat, master,
                               m, v, shard, head, nblk);
    } else {
        if (sa)
            hipLaunchKernelGGL((load_master_kernel<false, true>), g, blk, ZK_K0_LDS, stream, flat, master,
                               m, v, shard, head, nblk);
        else
            hipLaunchKernelGGL((load_master_kernel<false, false>), g, blk, ZK_K0_LDS, stream, flat,
                               master, m, v, shard, head, nblk);
    }
    return hipGetLastError();
}

}  // namespace zk
