// Host side of libzero.so: argument checks, the rank context (geometry,
// hyperparameters, fp32 master/m/v), step scalars, and kernel dispatch.
// The C ABI is declared and documented in include/zero.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "../../include/zero.h"
#include "zero_internal.h"

// One parameter of a per-parameter (dim-0) layout context.
struct zero_fsdp_tensor {
    int64_t dim0, row_numel;     // full shape: dim0 rows of row_numel elements
    int64_t first_row, rows;     // this rank's rows
    int64_t state_off;           // first element in master/m/v (multiple of 32)
};

struct zero_ctx {
    int64_t numel, shard, lo, padded;
    bool fsdp;                               // per-parameter layout
    std::vector<zero_fsdp_tensor> tensors;   // fsdp only
    int32_t world, rank;
    double lr, beta1, beta2, eps;
    int device;
    int num_cus;
    int32_t step_wgs_per_cu;     // zero_set_step_workgroups (0: no cap)
    void *state;                 // one allocation: master | m | v
    float *master, *m, *v;
    // device-resident step schedule, one block: schedule | scalars of the
    // current step | bias-correction table. It is either the context's own
    // allocation (zero_schedule_init: sched_mem, sched_mem_len) or the
    // device's static block (zero_schedule_init_noalloc: sched_static);
    // ds, sc_dev, bc_table and bc_len describe the one in use.
    void *sched_mem;
    int64_t sched_mem_len;
    bool sched_static;
    zk::DevSchedule *ds;
    zk::StepScalars *sc_dev;
    float *bc_table;             // (1-b1^t, 1-b2^t) for t = 1..bc_len
    int64_t bc_len;
    // Set once a begin-step kernel has been launched on the schedule: until
    // then the scalar block holds no step, and a range step that reads it
    // is refused. Host call order is the launch order on a stream, also
    // under capture.
    bool begun;
};

// The static schedule block of zero_schedule_init_noalloc: one per device
// that loads the library, held until the process ends. Host code never
// uses the array's name as an address (in host code it is a stand-in, not
// device memory): the device address comes from hipGetSymbolAddress, once
// per device with that device current, and only that address is used.
constexpr size_t kScratchBytes = (size_t)2 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

thread_local std::string g_last_error;

int fail(int code, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    try {
        g_last_error = buf;
    } catch (...) {
        g_last_error.clear();
    }
    return code;
}

int hip_fail(hipError_t e, const char *what) {
    return fail(ZERO_EHIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

bool valid_dtype(zero_dtype d) { return d == ZERO_F32 || d == ZERO_BF16; }
size_t dtype_size(zero_dtype d) { return d == ZERO_BF16 ? 2 : 4; }

int geometry(int64_t numel, int32_t world, int32_t rank, int64_t *shard, int64_t *lo,
             int64_t *padded) {
    if (numel < 1) return fail(ZERO_EINVAL, "numel must be >= 1 (got %lld)", (long long)numel);
    if (world < 1) return fail(ZERO_EINVAL, "world must be >= 1 (got %d)", world);
    if (rank < 0 || rank >= world)
        return fail(ZERO_EINVAL, "rank must be in [0, world) (got rank %d, world %d)", rank, world);
    const int64_t s = numel / world + (numel % world != 0 ? 1 : 0);
    if (shard) *shard = s;
    if (lo) *lo = (int64_t)rank * s;
    if (padded) *padded = s * world;
    return ZERO_OK;
}

void dim0_split(int64_t d0, int32_t world, int32_t rank, int64_t *first, int64_t *rows) {
    const int64_t c = d0 / world + (d0 % world != 0 ? 1 : 0);
    int64_t f = (int64_t)rank * c;
    if (f > d0) f = d0;
    int64_t e = f + c;
    if (e > d0) e = d0;
    *first = f;
    *rows = e - f;
}

int reject_fsdp(const zero_ctx *c) {
    if (c && c->fsdp)
        return fail(ZERO_EINVAL, "this context holds the per-parameter (dim-0) layout; "
                                 "use the zero_fsdp_* calls");
    return ZERO_OK;
}

// Make the context's device current for the duration of a call.
class DeviceGuard {
  public:
    explicit DeviceGuard(int dev) {
        if (hipGetDevice(&prev_) != hipSuccess) prev_ = -1;
        if (prev_ != dev) err_ = hipSetDevice(dev);
    }
    ~DeviceGuard() {
        if (prev_ >= 0 && err_ == hipSuccess) (void)hipSetDevice(prev_);
    }
    hipError_t error() const { return err_; }

  private:
    int prev_ = -1;
    hipError_t err_ = hipSuccess;
};

// Range checks query the runtime's allocation table, which a stream
// capture in global mode may not allow. While the caller's stream is being
// captured they are skipped (every other argument check still runs); the
// buffers of a captured call are normally those of an earlier eager call.
thread_local bool g_skip_range = false;

class CaptureScope {
  public:
    explicit CaptureScope(hipStream_t s) : prev_(g_skip_range) {
        hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(s, &st) != hipSuccess) {
            (void)hipGetLastError();
            st = hipStreamCaptureStatusNone;
        }
        g_skip_range = st == hipStreamCaptureStatusActive;
    }
    ~CaptureScope() { g_skip_range = prev_; }

  private:
    bool prev_;
};

// Reject a device range that runs past the allocation holding its first
// byte (an undersized buffer would otherwise fault on the GPU). Memory the
// runtime cannot describe (e.g. imported or virtually mapped) is accepted.
int check_range(const void *p, int64_t nbytes, const char *what) {
    if (nbytes <= 0 || g_skip_range) return ZERO_OK;
    hipDeviceptr_t base = nullptr;
    size_t size = 0;
    hipError_t e = hipMemGetAddressRange(&base, &size, (hipDeviceptr_t)p);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return ZERO_OK;
    }
    const uintptr_t b = (uintptr_t)base, q = (uintptr_t)p;
    if (q < b || q - b + (uint64_t)nbytes > (uint64_t)size)
        return fail(ZERO_EINVAL, "%s: %lld bytes at %p run past the end of its allocation "
                    "(%zu bytes at %p)", what, (long long)nbytes, p, size, (void *)base);
    return ZERO_OK;
}

zk::StepScalars make_scalars(const zero_ctx *c, int64_t t) {
    zk::StepScalars sc;
    sc.b1 = (float)c->beta1;
    sc.c1 = (float)(1.0 - c->beta1);
    sc.b2 = (float)c->beta2;
    sc.c2 = (float)(1.0 - c->beta2);
    sc.lr = (float)c->lr;
    sc.eps = (float)c->eps;
    sc.bc1 = (float)(1.0 - std::pow(c->beta1, (double)t));
    sc.bc2 = (float)(1.0 - std::pow(c->beta2, (double)t));
    sc.nf = (float)c->world;
    sc.n_pow2 = (c->world & (c->world - 1)) == 0;
    sc.inv_n = (float)(1.0 / (double)c->world);
    return sc;
}

// Where a step takes its scalars from.
enum StepMode {
    kHostT = 0,          // the step count passed by the caller
    kBeginDevice = 1,    // begin the schedule's next step, then use its scalars
    kCurrentDevice = 2,  // the scalars of the schedule's current step
};

// Layout of a schedule block: DevSchedule at 0, the current step's scalars
// at 256, the bias-correction table from 512.
constexpr size_t kSchedHead = 512;
constexpr size_t kSchedScalars = 256;

constexpr int64_t kScratchMaxTable = (int64_t)((kScratchBytes - kSchedHead) / (2 * sizeof(float)));
constexpr int kMaxDevices = 256;

std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];              // device address of `scratch`, per device
const zero_ctx *g_scratch_owner[kMaxDevices];  // context whose schedule it holds

// Resolve the static block's address on the current device `dev` (once).
int scratch_address(int dev, void **out) {
    if (dev < 0 || dev >= kMaxDevices)
        return fail(ZERO_EUNSUPPORTED, "device %d beyond the %d the library tracks", dev,
                    kMaxDevices);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr) {
            (void)hipGetLastError();
            return fail(ZERO_EHIP, "hipGetSymbolAddress of the static schedule block: %s",
                        hipGetErrorString(e));
        }
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return ZERO_OK;
}

bool owns_scratch(const zero_ctx *c) {
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    return c->device >= 0 && c->device < kMaxDevices && g_scratch_owner[c->device] == c;
}

int need_schedule(const zero_ctx *c) {
    if (!c->ds)
        return fail(ZERO_EINVAL, "no device step schedule: call zero_schedule_init (or "
                                 "zero_schedule_init_noalloc) first");
    if (c->sched_static && !owns_scratch(c))
        return fail(ZERO_EINVAL, "this context's static step schedule was taken over by "
                                 "another context on the same device "
                                 "(zero_schedule_init_noalloc); initialise it again");
    return ZERO_OK;
}

hipError_t begin_device_step(const zero_ctx *c, hipStream_t stream) {
    return zk::launch_begin_step(c->ds, c->bc_table, c->bc_len, make_scalars(c, 1), c->sc_dev,
                                 stream);
}

int build_flat_segments(const zero_ctx *c, const void *const *tensors, const int64_t *numels,
                        int32_t ntensors, zero_dtype dtype, const void *flat,
                        std::vector<zk::Segment> &segs, bool to_flat) {
    if (!c) return fail(ZERO_EINVAL, "null context");
    if (c->fsdp) return reject_fsdp(c);
    if (!tensors || !numels) return fail(ZERO_EINVAL, "null tensor or numel array");
    if (ntensors < 1) return fail(ZERO_EINVAL, "ntensors must be >= 1 (got %d)", ntensors);
    if (!valid_dtype(dtype)) return fail(ZERO_EINVAL, "unknown dtype %d", (int)dtype);
    if (!flat) return fail(ZERO_EINVAL, "null flat buffer");
    const int64_t es = (int64_t)dtype_size(dtype);
    int64_t off = 0;
    segs.clear();
    try {
        segs.reserve((size_t)ntensors + 1);
    } catch (...) {
        return fail(ZERO_ENOMEM, "host allocation failed");
    }
    for (int32_t t = 0; t < ntensors; ++t) {
        const int64_t n = numels[t];
        if (n < 0) return fail(ZERO_EINVAL, "numels[%d] is negative", t);
        if (n > c->numel - off)
            return fail(ZERO_EINVAL, "tensor sizes exceed the context's numel %lld",
                        (long long)c->numel);
        if (n > 0) {
            if (!tensors[t]) return fail(ZERO_EINVAL, "tensor %d is null", t);
            if ((uintptr_t)tensors[t] % (uintptr_t)es)
                return fail(ZERO_EINVAL, "tensor %d is not %lld-byte aligned", t, (long long)es);
            int rc = check_range(tensors[t], n * es, "tensor");
            if (rc) return rc;
            char *fp = (char *)flat + off * es;
            if (to_flat) segs.push_back({tensors[t], fp, n * es});
            else segs.push_back({fp, const_cast<void *>(tensors[t]), n * es});
        }
        off += n;
    }
    if (off != c->numel)
        return fail(ZERO_EINVAL, "tensor sizes sum to %lld, context numel is %lld", (long long)off,
                    (long long)c->numel);
    if ((uintptr_t)flat % (uintptr_t)es)
        return fail(ZERO_EINVAL, "flat buffer is not %lld-byte aligned", (long long)es);
    int rc = check_range(flat, (to_flat ? c->padded : c->numel) * es, "flat buffer");
    if (rc) return rc;
    if (to_flat && c->padded > c->numel)
        segs.push_back({nullptr, (char *)flat + c->numel * es, (c->padded - c->numel) * es});
    return ZERO_OK;
}

}  // namespace

extern "C" {

const char *zero_last_error(void) { return g_last_error.c_str(); }

int zero_shard_geometry(int64_t numel, int32_t world, int32_t rank, int64_t *shard, int64_t *lo,
                        int64_t *padded) {
    return geometry(numel, world, rank, shard, lo, padded);
}

int zero_state_bytes(int32_t stage, double numel, double world, double *bytes) {
    if (!bytes) return fail(ZERO_EINVAL, "null output");
    if (!(numel >= 0) || !(world >= 1)) return fail(ZERO_EINVAL, "need numel >= 0 and world >= 1");
    switch (stage) {
    case 0: *bytes = 16.0 * numel; break;                        // replicated
    case 1: *bytes = 4.0 * numel + 12.0 * numel / world; break;  // optimizer state split
    case 2: *bytes = 2.0 * numel + 14.0 * numel / world; break;  // + gradients split
    case 3: *bytes = 16.0 * numel / world; break;                // + parameters split
    default: return fail(ZERO_EINVAL, "stage must be 0..3 (got %d)", stage);
    }
    return ZERO_OK;
}

static int check_hparams(int32_t world, double lr, double beta1, double beta2, double eps) {
    if (world > ZERO_MAX_WORLD)
        return fail(ZERO_EINVAL, "world %d exceeds ZERO_MAX_WORLD (%d)", world, ZERO_MAX_WORLD);
    if (!(beta1 > 0.0 && beta1 < 1.0) || !(beta2 > 0.0 && beta2 < 1.0))
        return fail(ZERO_EINVAL, "betas must lie in (0, 1) (got %g, %g)", beta1, beta2);
    if (!std::isfinite(lr)) return fail(ZERO_EINVAL, "lr must be finite");
    if (!std::isfinite(eps) || eps < 0.0) return fail(ZERO_EINVAL, "eps must be finite and >= 0");
    return ZERO_OK;
}

// Device, master/m/v (`shard` elements each, zeroed) for a filled-in context.
// Each of master | m | v starts on a 2 MiB boundary of the allocation
// (measured: arrays packed at 256-byte granularity, which leaves m and v
// off 4 KiB pages, run the fused step 1.5-3% slower than 4 KiB or larger).
static const size_t kStateAlign = (size_t)2 << 20;
// m starts this far past master's phase within kStateAlign, and v twice as
// far: measured about 1 point of HBM peak faster for the fused step than
// all three arrays at one phase (7e9-element shard, N = 8; a 2 MiB offset,
// i.e. the same phase on other pages, was not).
static const size_t kStateStagger = (size_t)1 << 20;

// Each array starts `shift` elements past that boundary (m and v also
// kStateStagger and 2 kStateStagger past it). With shift =
// lo mod 32 the state lines up with full flat buffers that start on a
// 128-byte line: at h = (-lo) mod 64, element lo + h of such a buffer is at
// a multiple of 128 bytes (bf16: 2(lo + h); fp32: 4(lo + h)), and so is
// state element h (4(shift + h), with shift + h = lo + h mod 32). A step on
// full flat buffers at any lo therefore runs, after a head of fewer than 64
// elements, on wavefront blocks that fill whole 128-byte lines of every
// stream.
static int alloc_state(zero_ctx *c, int shift) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    int cus = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
    c->device = dev;
    c->num_cus = cus > 0 ? cus : 256;
    // the static schedule block's address on this device, resolved at set-up
    // so that zero_schedule_init_noalloc makes no runtime query later; a
    // failure here only matters to that call, which resolves it again and
    // reports it
    if (dev >= 0 && dev < kMaxDevices) {
        void *unused = nullptr;
        if (scratch_address(dev, &unused) != ZERO_OK) g_last_error.clear();
    }
    // master | m | v, each segment a whole number of kStateAlign blocks plus
    // kStateStagger, the first starting on a kStateAlign boundary inside the
    // allocation
    const size_t seg = ((((size_t)c->shard + (size_t)shift) * sizeof(float) + kStateAlign - 1) &
                        ~(kStateAlign - 1)) + kStateStagger;
    const size_t bytes = 3 * seg + kStateAlign;
    e = hipMalloc(&c->state, bytes);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        c->state = nullptr;
        return fail(ZERO_ENOMEM, "hipMalloc of %zu bytes for master/m/v failed: %s", bytes,
                    hipGetErrorString(e));
    }
    char *base = (char *)(((uintptr_t)c->state + kStateAlign - 1) & ~(uintptr_t)(kStateAlign - 1));
    c->master = (float *)base + shift;
    c->m = (float *)(base + seg) + shift;
    c->v = (float *)(base + 2 * seg) + shift;
    e = hipMemset(c->state, 0, bytes);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) {
        (void)hipFree(c->state);
        c->state = nullptr;
        return hip_fail(e, "clearing master/m/v");
    }
    return ZERO_OK;
}

int zero_shard_init(int64_t numel, int32_t world, int32_t rank, double lr, double beta1,
                    double beta2, double eps, zero_ctx **out) {
    if (!out) return fail(ZERO_EINVAL, "null output pointer");
    *out = nullptr;
    int64_t shard, lo, padded;
    int rc = geometry(numel, world, rank, &shard, &lo, &padded);
    if (rc) return rc;
    rc = check_hparams(world, lr, beta1, beta2, eps);
    if (rc) return rc;
    zero_ctx *c = new (std::nothrow) zero_ctx();
    if (!c) return fail(ZERO_ENOMEM, "host allocation failed");
    c->numel = numel;
    c->shard = shard;
    c->lo = lo;
    c->padded = padded;
    c->fsdp = false;
    c->world = world;
    c->rank = rank;
    c->lr = lr;
    c->beta1 = beta1;
    c->beta2 = beta2;
    c->eps = eps;
    rc = alloc_state(c, (int)(lo % 32));
    if (rc) {
        delete c;
        return rc;
    }
    *out = c;
    return ZERO_OK;
}

int zero_dim0_split(int64_t dim0, int32_t world, int32_t rank, int64_t *first_row,
                    int64_t *rows) {
    if (dim0 < 0) return fail(ZERO_EINVAL, "dim0 must be >= 0");
    if (world < 1) return fail(ZERO_EINVAL, "world must be >= 1");
    if (rank < 0 || rank >= world) return fail(ZERO_EINVAL, "rank must be in [0, world)");
    int64_t f, r;
    dim0_split(dim0, world, rank, &f, &r);
    if (first_row) *first_row = f;
    if (rows) *rows = r;
    return ZERO_OK;
}

int zero_fsdp_init(int32_t ntensors, const int64_t *dim0, const int64_t *row_numel,
                   int32_t world, int32_t rank, double lr, double beta1, double beta2, double eps,
                   zero_ctx **out) {
    if (!out) return fail(ZERO_EINVAL, "null output pointer");
    *out = nullptr;
    if (ntensors < 1 || !dim0 || !row_numel)
        return fail(ZERO_EINVAL, "need ntensors >= 1 and both shape arrays");
    if (world < 1 || rank < 0 || rank >= world)
        return fail(ZERO_EINVAL, "rank must be in [0, world) with world >= 1");
    if (world > ZERO_FSDP_MAX_WORLD)
        return fail(ZERO_EUNSUPPORTED, "the per-parameter layout supports world <= %d",
                    ZERO_FSDP_MAX_WORLD);
    int rc = check_hparams(world, lr, beta1, beta2, eps);
    if (rc) return rc;
    zero_ctx *c = new (std::nothrow) zero_ctx();
    if (!c) return fail(ZERO_ENOMEM, "host allocation failed");
    c->fsdp = true;
    c->world = world;
    c->rank = rank;
    c->lr = lr;
    c->beta1 = beta1;
    c->beta2 = beta2;
    c->eps = eps;
    int64_t off = 0, total = 0;
    try {
        c->tensors.resize((size_t)ntensors);
    } catch (...) {
        delete c;
        return fail(ZERO_ENOMEM, "host allocation failed");
    }
    for (int32_t k = 0; k < ntensors; ++k) {
        if (dim0[k] < 0 || row_numel[k] < 1) {
            delete c;
            return fail(ZERO_EINVAL, "tensor %d: need dim0 >= 0 and row_numel >= 1", k);
        }
        zero_fsdp_tensor &t = c->tensors[(size_t)k];
        t.dim0 = dim0[k];
        t.row_numel = row_numel[k];
        dim0_split(t.dim0, world, rank, &t.first_row, &t.rows);
        t.state_off = off;
        off += (t.rows * t.row_numel + 31) / 32 * 32;   // every piece on a 128-byte line
        total += t.dim0 * t.row_numel;
    }
    c->numel = total;
    c->shard = off;
    c->lo = 0;
    c->padded = off;
    rc = alloc_state(c, 0);
    if (rc) {
        delete c;
        return rc;
    }
    *out = c;
    return ZERO_OK;
}

int zero_fsdp_local(const zero_ctx *c, int32_t k, int64_t *first_row, int64_t *rows,
                    int64_t *state_offset) {
    if (!c || !c->fsdp) return fail(ZERO_EINVAL, "not a per-parameter layout context");
    if (k < 0 || k >= (int32_t)c->tensors.size()) return fail(ZERO_EINVAL, "tensor index out of range");
    const zero_fsdp_tensor &t = c->tensors[(size_t)k];
    if (first_row) *first_row = t.first_row;
    if (rows) *rows = t.rows;
    if (state_offset) *state_offset = t.state_off;
    return ZERO_OK;
}

int zero_fsdp_load_master(zero_ctx *c, const void *const *params, zero_dtype dtype,
                          hipStream_t stream) {
    if (!c || !c->fsdp) return fail(ZERO_EINVAL, "not a per-parameter layout context");
    if (!params) return fail(ZERO_EINVAL, "null parameter array");
    CaptureScope cs(stream);
    if (!valid_dtype(dtype)) return fail(ZERO_EINVAL, "unknown dtype %d", (int)dtype);
    const int64_t es = (int64_t)dtype_size(dtype);
    for (size_t k = 0; k < c->tensors.size(); ++k) {
        const zero_fsdp_tensor &t = c->tensors[k];
        if (t.rows == 0) continue;
        if (!params[k]) return fail(ZERO_EINVAL, "parameter %zu is null", k);
        if ((uintptr_t)params[k] % (uintptr_t)es) return fail(ZERO_EINVAL, "parameter %zu misaligned", k);
        int rc = check_range(params[k], t.dim0 * t.row_numel * es, "parameter");
        if (rc) return rc;
    }
    DeviceGuard g(c->device);
    if (g.error() != hipSuccess) return hip_fail(g.error(), "hipSetDevice");
    for (size_t k = 0; k < c->tensors.size(); ++k) {
        const zero_fsdp_tensor &t = c->tensors[k];
        if (t.rows == 0) continue;
        const char *base = (const char *)params[k] + t.first_row * t.row_numel * es;
        hipError_t e = zk::launch_load_master(base, dtype == ZERO_BF16, c->master + t.state_off,
                                              c->m + t.state_off, c->v + t.state_off,
                                              t.rows * t.row_numel, stream);
        if (e != hipSuccess) return hip_fail(e, "load_master launch");
    }
    return ZERO_OK;
}

static int fsdp_step_common(zero_ctx *c, const void *const *grads, int32_t n_replicas,
                            zero_dtype grad_dtype, void *const *params_out,
                            zero_dtype param_dtype, int64_t t, StepMode mode,
                            hipStream_t stream) {
    if (!c || !c->fsdp) return fail(ZERO_EINVAL, "not a per-parameter layout context");
    CaptureScope cs(stream);
    if (n_replicas != c->world)
        return fail(ZERO_EINVAL, "n_replicas (%d) must equal world (%d)", n_replicas, c->world);
    if (mode == kHostT && t < 1)
        return fail(ZERO_EINVAL, "step t must be >= 1 (got %lld)", (long long)t);
    if (mode != kHostT) {
        int rc = need_schedule(c);
        if (rc) return rc;
    }
    if (!grads || !params_out) return fail(ZERO_EINVAL, "null gradient or output array");
    if (!valid_dtype(grad_dtype) || !valid_dtype(param_dtype))
        return fail(ZERO_EINVAL, "unknown dtype");
    const int64_t ge = (int64_t)dtype_size(grad_dtype), pe = (int64_t)dtype_size(param_dtype);
    const size_t nt = c->tensors.size();
    std::vector<zk::FsdpSegment> segs;
    try {
        segs.reserve(nt);
    } catch (...) {
        return fail(ZERO_ENOMEM, "host allocation failed");
    }
    for (size_t k = 0; k < nt; ++k) {
        const zero_fsdp_tensor &tt = c->tensors[k];
        if (tt.rows == 0) continue;
        zk::FsdpSegment sg;
        const int64_t local = tt.rows * tt.row_numel;
        for (int q = 0; q < n_replicas; ++q) {
            const void *gp = grads[(size_t)q * nt + k];
            if (!gp) return fail(ZERO_EINVAL, "gradient of replica %d, tensor %zu is null", q, k);
            if ((uintptr_t)gp % (uintptr_t)ge)
                return fail(ZERO_EINVAL, "gradient of replica %d, tensor %zu misaligned", q, k);
            int rc = check_range(gp, tt.dim0 * tt.row_numel * ge, "gradient");
            if (rc) return rc;
            sg.grads[q] = (const char *)gp + tt.first_row * tt.row_numel * ge;
        }
        if (!params_out[k]) return fail(ZERO_EINVAL, "output shard %zu is null", k);
        if ((uintptr_t)params_out[k] % (uintptr_t)pe)
            return fail(ZERO_EINVAL, "output shard %zu misaligned", k);
        int rc = check_range(params_out[k], local * pe, "output shard");
        if (rc) return rc;
        sg.out = params_out[k];
        sg.state_off = tt.state_off;
        sg.numel = local;
        segs.push_back(sg);
    }
    DeviceGuard g(c->device);
    if (g.error() != hipSuccess) return hip_fail(g.error(), "hipSetDevice");
    if (mode == kBeginDevice) {
        hipError_t e = begin_device_step(c, stream);
        if (e != hipSuccess) return hip_fail(e, "begin-step launch");
        c->begun = true;
    }
    if (segs.empty()) return ZERO_OK;
    zk::FsdpArgs a;
    a.segs = segs.data();
    a.nseg = (int)segs.size();
    a.n = n_replicas;
    a.grad_bf16 = grad_dtype == ZERO_BF16;
    a.out_bf16 = param_dtype == ZERO_BF16;
    a.master = c->master;
    a.m = c->m;
    a.v = c->v;
    a.sc = make_scalars(c, mode == kHostT ? t : 1);
    a.sc_dev = mode == kHostT ? nullptr : c->sc_dev;
    a.stream_state = zk::state_streams(c->shard);
    hipError_t e = zk::launch_fsdp_step(a, stream);
    return e == hipSuccess ? ZERO_OK : hip_fail(e, "per-parameter step launch");
}

int zero_fsdp_step(zero_ctx *c, const void *const *grads, int32_t n_replicas,
                   zero_dtype grad_dtype, void *const *params_out, zero_dtype param_dtype,
                   int64_t t, hipStream_t stream) {
    return fsdp_step_common(c, grads, n_replicas, grad_dtype, params_out, param_dtype, t, kHostT,
                            stream);
}

int zero_fsdp_step_sched(zero_ctx *c, const void *const *grads, int32_t n_replicas,
                         zero_dtype grad_dtype, void *const *params_out, zero_dtype param_dtype,
                         hipStream_t stream) {
    return fsdp_step_common(c, grads, n_replicas, grad_dtype, params_out, param_dtype, 0,
                            kBeginDevice, stream);
}

int zero_shard_info(const zero_ctx *c, int64_t *shard, int64_t *lo, int64_t *padded) {
    if (!c) return fail(ZERO_EINVAL, "null context");
    if (shard) *shard = c->shard;
    if (lo) *lo = c->lo;
    if (padded) *padded = c->padded;
    return ZERO_OK;
}

int zero_shard_state_bytes(const zero_ctx *c, int64_t *bytes) {
    if (!c || !bytes) return fail(ZERO_EINVAL, "null context or output pointer");
    int64_t elems = c->shard;
    if (c->fsdp) {
        elems = 0;
        for (const zero_fsdp_tensor &t : c->tensors) elems += t.rows * t.row_numel;
    }
    *bytes = 3 * (int64_t)sizeof(float) * elems;
    return ZERO_OK;
}

int zero_set_lr(zero_ctx *c, double lr) {
    if (!c) return fail(ZERO_EINVAL, "null context");
    if (!std::isfinite(lr)) return fail(ZERO_EINVAL, "lr must be finite");
    c->lr = lr;
    return ZERO_OK;
}

int zero_set_step_workgroups(zero_ctx *c, int32_t per_cu) {
    if (!c) return fail(ZERO_EINVAL, "null context");
    if (per_cu < 0 || per_cu > 64)
        return fail(ZERO_EINVAL, "workgroups per compute unit must be in [0, 64] (got %d)", per_cu);
    c->step_wgs_per_cu = per_cu;
    return ZERO_OK;
}

int zero_load_master(zero_ctx *c, const void *flat, zero_dtype dtype, int64_t flat_offset,
                     hipStream_t stream) {
    if (!c) return fail(ZERO_EINVAL, "null context");
    if (!flat) return fail(ZERO_EINVAL, "null flat parameter buffer");
    CaptureScope cs(stream);
    if (!valid_dtype(dtype)) return fail(ZERO_EINVAL, "unknown dtype %d", (int)dtype);
    if (flat_offset < 0) return fail(ZERO_EINVAL, "negative offset");
    const size_t es = dtype_size(dtype);
    if ((uintptr_t)flat % es) return fail(ZERO_EINVAL, "flat buffer misaligned for its dtype");
    int rc = check_range(flat, (flat_offset + c->shard) * (int64_t)es, "flat parameter buffer");
    if (rc) return rc;
    DeviceGuard g(c->device);
    if (g.error() != hipSuccess) return hip_fail(g.error(), "hipSetDevice");
    rc = reject_fsdp(c);
    if (rc) return rc;
    const char *base = (const char *)flat + (size_t)flat_offset * es;
    hipError_t e = zk::launch_load_master(base, dtype == ZERO_BF16, c->master, c->m, c->v,
                                          c->shard, stream);
    return e == hipSuccess ? ZERO_OK : hip_fail(e, "load_master launch");
}

int zero_flatten(const zero_ctx *c, const void *const *srcs, const int64_t *numels,
                 int32_t ntensors, zero_dtype dtype, void *dst, hipStream_t stream) {
    if (!c) return fail(ZERO_EINVAL, "null context");
    CaptureScope cs(stream);
    std::vector<zk::Segment> segs;
    int rc = build_flat_segments(c, srcs, numels, ntensors, dtype, dst, segs, true);
    if (rc) return rc;
    DeviceGuard g(c->device);
    if (g.error() != hipSuccess) return hip_fail(g.error(), "hipSetDevice");
    hipError_t e = zk::launch_copy_segments(segs.data(), (int)segs.size(),
                                            (int)dtype_size(dtype), stream);
    return e == hipSuccess ? ZERO_OK : hip_fail(e, "flatten launch");
}

int zero_flatten_range(const zero_ctx *c, const void *const *srcs, const int64_t *numels,
                       int32_t ntensors, zero_dtype dtype, void *dst, int64_t flat_begin,
                       int64_t flat_count, hipStream_t stream) {
    if (!c) return fail(ZERO_EINVAL, "null context");
    CaptureScope cs(stream);
    std::vector<zk::Segment> segs;
    int rc = build_flat_segments(c, srcs, numels, ntensors, dtype, dst, segs, true);
    if (rc) return rc;
    if (flat_begin < 0 || flat_count < 0 || flat_begin > c->padded - flat_count)
        return fail(ZERO_EINVAL, "window [%lld, %lld) outside the padded length %lld",
                    (long long)flat_begin, (long long)(flat_begin + flat_count),
                    (long long)c->padded);
    // clip every segment to the window (segments are laid out in flat order)
    const int64_t es = (int64_t)dtype_size(dtype);
    const char *base = (const char *)dst;
    const int64_t wb = flat_begin * es, we = (flat_begin + flat_count) * es;
    std::vector<zk::Segment> clipped;
    try {
        clipped.reserve(segs.size());
    } catch (...) {
        return fail(ZERO_ENOMEM, "host allocation failed");
    }
    for (const zk::Segment &sg : segs) {
        const int64_t b = (const char *)sg.dst - base, e = b + sg.nbytes;
        const int64_t cb = b > wb ? b : wb, ce = e < we ? e : we;
        if (cb >= ce) continue;
        zk::Segment x;
        x.src = sg.src ? (const char *)sg.src + (cb - b) : nullptr;
        x.dst = (char *)sg.dst + (cb - b);
        x.nbytes = ce - cb;
        clipped.push_back(x);
    }
    if (clipped.empty()) return ZERO_OK;
    DeviceGuard g(c->device);
    if (g.error() != hipSuccess) return hip_fail(g.error(), "hipSetDevice");
    hipError_t e = zk::launch_copy_segments(clipped.data(), (int)clipped.size(), (int)es, stream);
    return e == hipSuccess ? ZERO_OK : hip_fail(e, "flatten launch");
}

int zero_unflatten(const zero_ctx *c, const void *flat, int32_t ntensors, const int64_t *numels,
                   zero_dtype dtype, void *const *dsts, hipStream_t stream) {
    if (!c) return fail(ZERO_EINVAL, "null context");
    CaptureScope cs(stream);
    std::vector<zk::Segment> segs;
    int rc = build_flat_segments(c, (const void *const *)dsts, numels, ntensors, dtype, flat,
                                 segs, false);
    if (rc) return rc;
    DeviceGuard g(c->device);
    if (g.error() != hipSuccess) return hip_fail(g.error(), "hipSetDevice");
    hipError_t e = zk::launch_copy_segments(segs.data(), (int)segs.size(),
                                            (int)dtype_size(dtype), stream);
    return e == hipSuccess ? ZERO_OK : hip_fail(e, "unflatten launch");
}

static int step_common(zero_ctx *c, int64_t begin, int64_t count, const void *const *grads,
                       int32_t n_replicas, zero_dtype grad_dtype, int64_t grad_offset,
                       void *param_out, zero_dtype param_dtype, int64_t param_offset, int64_t t,
                       StepMode mode, hipStream_t stream) {
    if (!c) return fail(ZERO_EINVAL, "null context");
    CaptureScope cs(stream);
    if (c->fsdp) return reject_fsdp(c);
    if (begin < 0 || count < 0 || begin > c->shard - count)
        return fail(ZERO_EINVAL, "range [%lld, %lld) outside the shard of %lld elements",
                    (long long)begin, (long long)(begin + count), (long long)c->shard);
    if (n_replicas != c->world)
        return fail(ZERO_EINVAL, "n_replicas (%d) must equal world (%d)", n_replicas, c->world);
    if (mode == kHostT && t < 1)
        return fail(ZERO_EINVAL, "step t must be >= 1 (got %lld)", (long long)t);
    if (mode != kHostT) {
        int rc = need_schedule(c);
        if (rc) return rc;
    }
    if (mode == kCurrentDevice && !c->begun)
        return fail(ZERO_EINVAL, "no scheduled step has begun: call zero_step_begin (or "
                                 "zero_step_sched) before a scheduled range step");
    if (!grads) return fail(ZERO_EINVAL, "null replica array");
    if (!param_out) return fail(ZERO_EINVAL, "null parameter output");
    if (!valid_dtype(grad_dtype) || !valid_dtype(param_dtype))
        return fail(ZERO_EINVAL, "unknown dtype");
    if (grad_offset < 0 || param_offset < 0) return fail(ZERO_EINVAL, "negative offset");
    const size_t ge = dtype_size(grad_dtype), pe = dtype_size(param_dtype);
    const void *slices[ZERO_MAX_WORLD];
    for (int q = 0; q < n_replicas; ++q) {
        if (!grads[q]) return fail(ZERO_EINVAL, "replica %d is null", q);
        if ((uintptr_t)grads[q] % ge) return fail(ZERO_EINVAL, "replica %d misaligned", q);
        slices[q] = (const char *)grads[q] + (size_t)grad_offset * ge;
        int rc = check_range(grads[q], (grad_offset + count) * (int64_t)ge, "gradient replica");
        if (rc) return rc;
    }
    if ((uintptr_t)param_out % pe) return fail(ZERO_EINVAL, "parameter output misaligned");
    int rc = check_range(param_out, (param_offset + count) * (int64_t)pe, "parameter output");
    if (rc) return rc;
    DeviceGuard g(c->device);
    if (g.error() != hipSuccess) return hip_fail(g.error(), "hipSetDevice");
    if (mode == kBeginDevice) {
        hipError_t e = begin_device_step(c, stream);
        if (e != hipSuccess) return hip_fail(e, "begin-step launch");
        c->begun = true;
    }
    if (count == 0) return ZERO_OK;

    zk::StepArgs a = {};
    a.grads = slices;
    a.n = n_replicas;
    a.grad_bf16 = grad_dtype == ZERO_BF16;
    a.master = c->master + begin;
    a.m = c->m + begin;
    a.v = c->v + begin;
    a.out = (char *)param_out + (size_t)param_offset * pe;
    a.out_bf16 = param_dtype == ZERO_BF16;
    a.shard = count;
    a.sc = make_scalars(c, mode == kHostT ? t : 1);
    a.sc_dev = mode == kHostT ? nullptr : c->sc_dev;
    a.num_cus = c->num_cus;
    a.stream_state = zk::state_streams(c->shard);
    a.max_workgroups = (int64_t)c->step_wgs_per_cu * c->num_cus;
    hipError_t e = zk::launch_step(a, stream);
    return e == hipSuccess ? ZERO_OK : hip_fail(e, "step launch");
}

int zero_step(zero_ctx *c, const void *const *grads, int32_t n_replicas, zero_dtype grad_dtype,
              int64_t grad_offset, void *param_out, zero_dtype param_dtype, int64_t param_offset,
              int64_t t, hipStream_t stream) {
    if (!c) return fail(ZERO_EINVAL, "null context");
    return step_common(c, 0, c->shard, grads, n_replicas, grad_dtype, grad_offset, param_out,
                       param_dtype, param_offset, t, kHostT, stream);
}

int zero_step_range(zero_ctx *c, int64_t shard_begin, int64_t count, const void *const *grads,
                    int32_t n_replicas, zero_dtype grad_dtype, int64_t grad_offset,
                    void *param_out, zero_dtype param_dtype, int64_t param_offset, int64_t t,
                    hipStream_t stream) {
    return step_common(c, shard_begin, count, grads, n_replicas, grad_dtype, grad_offset,
                       param_out, param_dtype, param_offset, t, kHostT, stream);
}

int zero_step_sched(zero_ctx *c, const void *const *grads, int32_t n_replicas,
                    zero_dtype grad_dtype, int64_t grad_offset, void *param_out,
                    zero_dtype param_dtype, int64_t param_offset, hipStream_t stream) {
    if (!c) return fail(ZERO_EINVAL, "null context");
    return step_common(c, 0, c->shard, grads, n_replicas, grad_dtype, grad_offset, param_out,
                       param_dtype, param_offset, 0, kBeginDevice, stream);
}

int zero_step_range_sched(zero_ctx *c, int64_t shard_begin, int64_t count,
                          const void *const *grads, int32_t n_replicas, zero_dtype grad_dtype,
                          int64_t grad_offset, void *param_out, zero_dtype param_dtype,
                          int64_t param_offset, hipStream_t stream) {
    return step_common(c, shard_begin, count, grads, n_replicas, grad_dtype, grad_offset,
                       param_out, param_dtype, param_offset, 0, kCurrentDevice, stream);
}

int zero_step_begin(zero_ctx *c, hipStream_t stream) {
    if (!c) return fail(ZERO_EINVAL, "null context");
    int rc = need_schedule(c);
    if (rc) return rc;
    DeviceGuard g(c->device);
    if (g.error() != hipSuccess) return hip_fail(g.error(), "hipSetDevice");
    hipError_t e = begin_device_step(c, stream);
    if (e != hipSuccess) return hip_fail(e, "begin-step launch");
    c->begun = true;
    return ZERO_OK;
}

// Bias-correction table: entry t-1 holds (f32(1 - b1^t), f32(1 - b2^t)),
// formed exactly as for a host step count. It ends at the first t where
// both b^t < 2^-26: from there on 1 - b^t rounds to 1 in binary32 for every
// later t, and the last entry is (1, 1).
static int bias_table_len(const zero_ctx *c, int64_t cap, int64_t *len_out) {
    const double tiny = std::ldexp(1.0, -26);
    int64_t len = 1;
    while (std::pow(c->beta1, (double)len) >= tiny || std::pow(c->beta2, (double)len) >= tiny) {
        if (++len > cap)
            return fail(ZERO_EUNSUPPORTED, "betas (%g, %g) need a bias-correction table of more "
                        "than %lld steps", c->beta1, c->beta2, (long long)cap);
    }
    const zk::StepScalars last = make_scalars(c, len);
    if (last.bc1 != 1.0f || last.bc2 != 1.0f)
        return fail(ZERO_EHIP, "bias-correction table does not end at (1, 1)");
    *len_out = len;
    return ZERO_OK;
}

static int bias_table(const zero_ctx *c, std::vector<float> &tab) {
    int64_t len = 0;
    int rc = bias_table_len(c, ZERO_SCHEDULE_MAX_TABLE, &len);
    if (rc) return rc;
    try {
        tab.resize((size_t)(2 * len));
    } catch (...) {
        return fail(ZERO_ENOMEM, "host allocation failed");
    }
    for (int64_t t = 1; t <= len; ++t) {
        const zk::StepScalars sc = make_scalars(c, t);
        tab[(size_t)(2 * (t - 1))] = sc.bc1;
        tab[(size_t)(2 * (t - 1) + 1)] = sc.bc2;
    }
    return ZERO_OK;
}

// Point the context's schedule at a block (its own or the static one).
static void use_schedule_block(zero_ctx *c, void *mem, int64_t len, bool is_static) {
    c->ds = (zk::DevSchedule *)mem;
    c->sc_dev = (zk::StepScalars *)((char *)mem + kSchedScalars);
    c->bc_table = (float *)((char *)mem + kSchedHead);
    c->bc_len = len;
    c->sched_static = is_static;
}

int zero_schedule_init(zero_ctx *c, int64_t next_t, hipStream_t stream) {
    if (!c) return fail(ZERO_EINVAL, "null context");
    if (next_t < 1) return fail(ZERO_EINVAL, "next step must be >= 1 (got %lld)", (long long)next_t);
    DeviceGuard g(c->device);
    if (g.error() != hipSuccess) return hip_fail(g.error(), "hipSetDevice");
    if (!c->sched_mem) {
        std::vector<float> tab;
        int rc = bias_table(c, tab);
        if (rc) return rc;
        const size_t bytes = kSchedHead + tab.size() * sizeof(float);
        void *mem = nullptr;
        hipError_t e = hipMalloc(&mem, bytes);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            return fail(ZERO_ENOMEM, "hipMalloc of %zu bytes for the step schedule failed", bytes);
        }
        e = hipMemset(mem, 0, kSchedHead);
        if (e == hipSuccess)
            e = hipMemcpy((char *)mem + kSchedHead, tab.data(), tab.size() * sizeof(float),
                          hipMemcpyHostToDevice);
        if (e != hipSuccess) {
            (void)hipFree(mem);
            return hip_fail(e, "uploading the step schedule");
        }
        c->sched_mem = mem;
        c->sched_mem_len = (int64_t)(tab.size() / 2);
    }
    if (c->ds != (zk::DevSchedule *)c->sched_mem) {
        use_schedule_block(c, c->sched_mem, c->sched_mem_len, false);
        c->begun = false;    // this block's scalars were resolved for no step of ours
    }
    hipError_t e = zk::launch_set_schedule(c->ds, next_t, (float)c->lr, stream);
    return e == hipSuccess ? ZERO_OK : hip_fail(e, "schedule launch");
}

int zero_schedule_init_noalloc(zero_ctx *c, int64_t next_t, hipStream_t stream) {
    if (!c) return fail(ZERO_EINVAL, "null context");
    if (next_t < 1) return fail(ZERO_EINVAL, "next step must be >= 1 (got %lld)", (long long)next_t);
    int64_t len = 0;
    int rc = bias_table_len(c, kScratchMaxTable, &len);
    if (rc == ZERO_EUNSUPPORTED)
        return fail(ZERO_EUNSUPPORTED, "betas (%g, %g) need a bias-correction table longer than "
                    "the %lld steps the static schedule block (%zu bytes) holds; use "
                    "zero_schedule_init", c->beta1, c->beta2, (long long)kScratchMaxTable,
                    kScratchBytes);
    if (rc) return rc;
    DeviceGuard g(c->device);
    if (g.error() != hipSuccess) return hip_fail(g.error(), "hipSetDevice");
    void *base = nullptr;
    rc = scratch_address(c->device, &base);
    if (rc) return rc;
    {
        std::lock_guard<std::mutex> lk(g_scratch_mu);
        g_scratch_owner[c->device] = c;
    }
    use_schedule_block(c, base, len, true);
    c->begun = false;        // the block holds whatever the last call left there
    // the table, entry t-1 = (f32(1 - b1^t), f32(1 - b2^t)), in chunks carried
    // by the fill kernel's arguments
    zk::WordChunk chunk;
    uint32_t *dst = reinterpret_cast<uint32_t *>(c->bc_table);
    int64_t done = 0;                        // words issued
    const int64_t words = 2 * len;
    static_assert(zk::kWordChunk % 2 == 0, "whole table entries per chunk");
    while (done < words) {
        chunk.n = (int)(words - done < zk::kWordChunk ? words - done : zk::kWordChunk);
        for (int k = 0; k < chunk.n; k += 2) {
            const zk::StepScalars sc = make_scalars(c, (done + k) / 2 + 1);
            std::memcpy(&chunk.w[k], &sc.bc1, sizeof(float));
            std::memcpy(&chunk.w[k + 1], &sc.bc2, sizeof(float));
        }
        hipError_t e = zk::launch_fill_words(dst + done, chunk, stream);
        if (e != hipSuccess) return hip_fail(e, "uploading the static step schedule");
        done += chunk.n;
    }
    hipError_t e = zk::launch_set_schedule(c->ds, next_t, (float)c->lr, stream);
    return e == hipSuccess ? ZERO_OK : hip_fail(e, "schedule launch");
}

int zero_schedule_lr(zero_ctx *c, double lr, hipStream_t stream) {
    if (!c) return fail(ZERO_EINVAL, "null context");
    if (!std::isfinite(lr)) return fail(ZERO_EINVAL, "lr must be finite");
    int rc = need_schedule(c);
    if (rc) return rc;
    DeviceGuard g(c->device);
    if (g.error() != hipSuccess) return hip_fail(g.error(), "hipSetDevice");
    c->lr = lr;
    hipError_t e = zk::launch_set_schedule(c->ds, 0, (float)lr, stream);
    return e == hipSuccess ? ZERO_OK : hip_fail(e, "schedule launch");
}

int zero_schedule_get(const zero_ctx *c, int64_t *next_t, hipStream_t stream) {
    if (!c) return fail(ZERO_EINVAL, "null context");
    if (!next_t) return fail(ZERO_EINVAL, "null output pointer");
    int rc = need_schedule(c);
    if (rc) return rc;
    DeviceGuard g(c->device);
    if (g.error() != hipSuccess) return hip_fail(g.error(), "hipSetDevice");
    zk::DevSchedule h;
    hipError_t e = hipMemcpyAsync(&h, c->ds, sizeof h, hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return hip_fail(e, "reading the step schedule");
    *next_t = h.t;
    return ZERO_OK;
}

static int copy_state(const zero_ctx *c, const float *const src[3], float *const dst[3],
                      hipStream_t stream, const char *what) {
    CaptureScope cs(stream);
    DeviceGuard g(c->device);
    if (g.error() != hipSuccess) return hip_fail(g.error(), "hipSetDevice");
    for (int k = 0; k < 3; ++k) {
        if (!src[k] || !dst[k]) continue;
        int rc = check_range(src[k], c->shard * (int64_t)sizeof(float), what);
        if (!rc) rc = check_range(dst[k], c->shard * (int64_t)sizeof(float), what);
        if (rc) return rc;
        hipError_t e = hipMemcpyAsync(dst[k], src[k], (size_t)c->shard * sizeof(float),
                                      hipMemcpyDeviceToDevice, stream);
        if (e != hipSuccess) return hip_fail(e, what);
    }
    return ZERO_OK;
}

int zero_get_state(const zero_ctx *c, float *master, float *m, float *v, hipStream_t stream) {
    if (!c) return fail(ZERO_EINVAL, "null context");
    const float *src[3] = {c->master, c->m, c->v};
    float *dst[3] = {master, m, v};
    return copy_state(c, src, dst, stream, "get_state copy");
}

int zero_set_state(zero_ctx *c, const float *master, const float *m, const float *v,
                   hipStream_t stream) {
    if (!c) return fail(ZERO_EINVAL, "null context");
    const float *src[3] = {master, m, v};
    float *dst[3] = {c->master, c->m, c->v};
    return copy_state(c, src, dst, stream, "set_state copy");
}

void zero_destroy(zero_ctx *c) {
    if (!c) return;
    DeviceGuard g(c->device);
    (void)hipDeviceSynchronize();
    if (c->state) (void)hipFree(c->state);
    if (c->sched_mem) (void)hipFree(c->sched_mem);
    {
        std::lock_guard<std::mutex> lk(g_scratch_mu);
        if (c->device >= 0 && c->device < kMaxDevices && g_scratch_owner[c->device] == c)
            g_scratch_owner[c->device] = nullptr;
    }
    delete c;
}

}  // extern "C"
