/*
 * CPU oracle for one data-parallel rank's ZeRO-2 optimizer step.
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg load this library. It shares no source with the HIP
 * library (no headers, helpers or constants): it is written from the pages'
 * description alone, as plain loops, so that a reader can check it by eye.
 *
 * Sources (the pages this follows):
 *   [ZF]  "ZeRO and FSDP: partitioning the optimizer states, the gradients
 *         and the parameters" (AI infra handbook), table "The three stages",
 *         section "Implementing ZeRO's Adam from scratch" (class ZeroAdam:
 *         constructor, _flatten, step, state_bytes), and the first exercise's
 *         answer (13B model on 16 cards).
 *   [L9]  "9. ZeRO Stage 1 and 2: Partitioning Optimizer State and
 *         Gradients", section "Know this".
 *
 * Precision. The pages' optimizer holds its master copy and both moments as
 * fp32 tensors (ZeroAdam keeps `flat[lo:lo+shard]` of a default-dtype flat
 * vector and calls these "the fp32 master parameters"), so the update is
 * evaluated in IEEE binary32 with the operation order of the page's step as
 * PyTorch evaluates it on a CPU:
 *     m <- fma(g, 1-b1, m*b1)            m.mul_(b1).add_(g, alpha=1-b1)
 *     v <- fma((1-b2)*g, g, v*b2)        v.mul_(b2).addcmul_(g, g, value=1-b2)
 *     mh = m / (1-b1^t)   vh = v / (1-b2^t)   (true divisions)
 *     master <- master - (lr*mh) / (sqrt(vh) + eps)
 * Every scalar (b1, 1-b1, b2, 1-b2, lr, eps, 1-b1^t, 1-b2^t, N) is formed in
 * binary64 and rounded once to binary32. Divisions and square roots are the
 * correctly rounded IEEE operations; denormals are kept.
 * This file must be compiled with -ffp-contract=off (no implicit fusion).
 *
 * The bf16 write-back rounds to nearest, ties to even, written here from the
 * definition (compare the discarded half against one half-ulp).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_EINVAL (-1)

/* ---------------------------------------------------------------- geometry
 * [ZF] ZeroAdam constructor: shard = ceil(numel / world); this rank's slice
 * starts at lo = rank * shard; the flat vector has shard * world elements,
 * zero-padded at the end.
 * out[0] = shard, out[1] = lo, out[2] = padded length, out[3] = pad count,
 * out[4] = real (non-pad) elements inside this rank's slice.               */
int oracle_geometry(int64_t numel, int64_t world, int64_t rank, int64_t *out)
{
    if (numel < 1 || world < 1 || rank < 0 || rank >= world || !out)
        return ORACLE_EINVAL;
    int64_t shard = numel / world;
    if (shard * world < numel)
        shard += 1;                     /* ceiling */
    int64_t lo = rank * shard;
    int64_t padded = shard * world;
    int64_t valid = numel - lo;
    if (valid < 0) valid = 0;
    if (valid > shard) valid = shard;
    out[0] = shard;
    out[1] = lo;
    out[2] = padded;
    out[3] = padded - numel;
    out[4] = valid;
    return ORACLE_OK;
}

/* -------------------------------------------------- per-parameter dim-0 split
 * [ZF] section "ZeRO-3 and FSDP": FSDP2 keeps each parameter as a tensor
 * partitioned along dimension 0. Rank r holds rows [r*c, min((r+1)*c, d0))
 * with c = ceil(d0 / world); trailing ranks may hold fewer rows or none.
 * out[0] = first row, out[1] = number of rows.                             */
int oracle_dim0_split(int64_t d0, int64_t world, int64_t rank, int64_t *out)
{
    if (d0 < 0 || world < 1 || rank < 0 || rank >= world || !out)
        return ORACLE_EINVAL;
    int64_t c = d0 / world;
    if (c * world < d0)
        c += 1;
    int64_t first = rank * c;
    if (first > d0) first = d0;
    int64_t last = first + c;
    if (last > d0) last = d0;
    out[0] = first;
    out[1] = last - first;
    return ORACLE_OK;
}

/* ------------------------------------------------------------ stage bytes
 * [ZF] table "The three stages": model-state bytes per card under
 * mixed-precision Adam with psi parameters and data-parallel degree n.
 * stage 0 = plain data parallelism, 1..3 = ZeRO-1..3.                      */
double oracle_stage_bytes(int stage, double psi, double n)
{
    switch (stage) {
    case 0: return 16.0 * psi;
    case 1: return 4.0 * psi + 12.0 * psi / n;
    case 2: return 2.0 * psi + 14.0 * psi / n;
    case 3: return 16.0 * psi / n;
    default: return -1.0;
    }
}

/* [ZF] ZeroAdam.state_bytes: master, m and v of `shard` fp32 elements each. */
int64_t oracle_state_bytes(int64_t shard)
{
    return 3 * shard * (int64_t)sizeof(float);
}

/* ----------------------------------------------------------------- flatten
 * [ZF] ZeroAdam._flatten: concatenate the tensors' elements in list order
 * (each tensor row-major), then zeros up to the padded length. The copy is a
 * byte copy, so the dtype is kept bit for bit.                             */
int oracle_flatten(const void *const *srcs, const int64_t *numels,
                   int32_t ntensors, int32_t elem_size, void *dst,
                   int64_t padded)
{
    if (ntensors < 0 || elem_size < 1 || !dst || padded < 0)
        return ORACLE_EINVAL;
    unsigned char *out = (unsigned char *)dst;
    int64_t off = 0;
    for (int32_t t = 0; t < ntensors; t++) {
        if (numels[t] < 0) return ORACLE_EINVAL;
        if (off + numels[t] > padded) return ORACLE_EINVAL;
        if (numels[t] > 0)
            memcpy(out + off * elem_size, srcs[t], (size_t)(numels[t] * elem_size));
        off += numels[t];
    }
    memset(out + off * elem_size, 0, (size_t)((padded - off) * elem_size));
    return ORACLE_OK;
}

/* The inverse: cut the flat vector back into the tensors, in list order
 * ([ZF] ZeroAdam.step, the copy of the gathered vector into each p.data). */
int oracle_unflatten(const void *src, int32_t ntensors, const int64_t *numels,
                     int32_t elem_size, void *const *dsts)
{
    if (ntensors < 0 || elem_size < 1 || !src) return ORACLE_EINVAL;
    const unsigned char *in = (const unsigned char *)src;
    int64_t off = 0;
    for (int32_t t = 0; t < ntensors; t++) {
        if (numels[t] > 0)
            memcpy(dsts[t], in + off * elem_size, (size_t)(numels[t] * elem_size));
        off += numels[t];
    }
    return ORACLE_OK;
}

/* -------------------------------------------------------------------- bf16 */
static float bf16_bits_to_float(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;     /* bf16 is the top half of binary32 */
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Round binary32 to bf16, nearest with ties to even. NaN stays NaN (quiet,
 * sign kept); values past the largest bf16 round to infinity.              */
uint16_t oracle_bf16_round(float x)
{
    uint32_t u;
    memcpy(&u, &x, sizeof u);
    uint32_t hi = u >> 16;
    uint32_t lo = u & 0xFFFFu;
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0)
        return (uint16_t)(hi | 0x0040u);            /* NaN: force quiet bit */
    if (lo > 0x8000u || (lo == 0x8000u && (hi & 1u)))
        hi += 1;                                     /* carries into exponent */
    return (uint16_t)hi;
}

void oracle_bf16_round_array(const float *x, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = oracle_bf16_round(x[i]);
}

/* ------------------------------------------------------------ step scalars
 * sc[0]=b1  sc[1]=1-b1  sc[2]=b2  sc[3]=1-b2  sc[4]=lr  sc[5]=eps
 * sc[6]=1-b1^t  sc[7]=1-b2^t  sc[8]=N   (each: binary64, rounded once)     */
int oracle_step_scalars(double lr, double b1, double b2, double eps,
                        int64_t t, int32_t world, float *sc)
{
    if (t < 1 || world < 1 || !sc) return ORACLE_EINVAL;
    sc[0] = (float)b1;
    sc[1] = (float)(1.0 - b1);
    sc[2] = (float)b2;
    sc[3] = (float)(1.0 - b2);
    sc[4] = (float)lr;
    sc[5] = (float)eps;
    sc[6] = (float)(1.0 - pow(b1, (double)t));
    sc[7] = (float)(1.0 - pow(b2, (double)t));
    sc[8] = (float)world;
    return ORACLE_OK;
}

/* -------------------------------------------------------- per-element work */
static float grad_at(const void *rep, int32_t is_bf16, int64_t idx)
{
    if (is_bf16)
        return bf16_bits_to_float(((const uint16_t *)rep)[idx]);
    return ((const float *)rep)[idx];
}

/* [ZF] ZeroAdam.step, reduce-scatter then `g /= world`: this rank's slice of
 * the sum over the N replicas, added in rank order 0..N-1, then divided by N. */
static float reduce_mean_one(const void *const *reps, int32_t n,
                             int32_t is_bf16, int64_t idx, float nf)
{
    float s = grad_at(reps[0], is_bf16, idx);
    for (int32_t q = 1; q < n; q++)
        s = s + grad_at(reps[q], is_bf16, idx);
    return s / nf;
}

/* [ZF] ZeroAdam.step, the Adam lines: moments, bias correction, update.    */
static void adam_one(float g, float *master, float *m, float *v,
                     const float *sc)
{
    float b1 = sc[0], c1 = sc[1], b2 = sc[2], c2 = sc[3];
    float lr = sc[4], eps = sc[5], bc1 = sc[6], bc2 = sc[7];
    float mm = fmaf(g, c1, *m * b1);
    float vv = fmaf(c2 * g, g, *v * b2);
    float mh = mm / bc1;
    float vh = vv / bc2;
    float den = sqrtf(vh) + eps;
    float u = (lr * mh) / den;
    *m = mm;
    *v = vv;
    *master = *master - u;
}

/* g[i] = mean over replicas of reps[q][off + i], i < shard.                */
int oracle_reduce_mean(const void *const *reps, int32_t n, int32_t is_bf16,
                       int64_t off, int64_t shard, float nf, float *g)
{
    if (n < 1 || shard < 0 || !g) return ORACLE_EINVAL;
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < shard; i++)
        g[i] = reduce_mean_one(reps, n, is_bf16, off + i, nf);
    return ORACLE_OK;
}

/* One full shard step ([ZF] ZeroAdam.step): reduce, Adam, and this rank's
 * contribution to the all-gather (its updated slice written into the flat
 * parameter buffer at `out_off`, bf16 rounded or fp32), element by element
 * in one loop (so large shards need no g buffer).                          */
int oracle_shard_step(const void *const *reps, int32_t n, int32_t is_bf16,
                      int64_t grad_off, float *master, float *m, float *v,
                      int64_t shard, const float *sc, void *out,
                      int32_t out_bf16, int64_t out_off)
{
    if (n < 1 || shard < 0 || !sc || !out) return ORACLE_EINVAL;
    float nf = sc[8];
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < shard; i++) {
        float g = reduce_mean_one(reps, n, is_bf16, grad_off + i, nf);
        adam_one(g, &master[i], &m[i], &v[i], sc);
        if (out_bf16)
            ((uint16_t *)out)[out_off + i] = oracle_bf16_round(master[i]);
        else
            ((float *)out)[out_off + i] = master[i];
    }
    return ORACLE_OK;
}

/* Master initialisation ([ZF] constructor): the fp32 master is this rank's
 * slice of the flat parameters (bf16 inputs widen exactly); m = v = 0.     */
int oracle_load_master(const void *flat, int32_t is_bf16, int64_t lo,
                       int64_t shard, float *master, float *m, float *v)
{
    if (!flat || shard < 0) return ORACLE_EINVAL;
    for (int64_t i = 0; i < shard; i++) {
        master[i] = grad_at(flat, is_bf16, lo + i);
        m[i] = 0.0f;
        v[i] = 0.0f;
    }
    return ORACLE_OK;
}

/* Set the number of threads the parallel loops use (timing only). */
void oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* Threads the parallel loops above use (for reporting). */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
