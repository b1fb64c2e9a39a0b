"""MI355X (gfx950) ZeRO-2 shard step: Python binding of libzero.so.

Argument marshalling only: every step of the path runs in the library's HIP
kernels. PyTorch supplies device memory (tensor storage) and streams; the
binding checks tensor device/dtype/size so that a mistake becomes a Python
error instead of an out-of-bounds GPU access, then calls the C ABI declared
in include/zero.h with raw pointers.

There is no CPU fallback: if libzero.so is missing or cannot be loaded, the
first call raises ZeroError.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libzero.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "zero.h")

ZERO_F32, ZERO_BF16 = 0, 1
ZERO_OK, ZERO_EINVAL, ZERO_ENOMEM, ZERO_EHIP, ZERO_EUNSUPPORTED = 0, -1, -2, -3, -4
MAX_WORLD = 256

_CODES = {ZERO_EINVAL: "EINVAL", ZERO_ENOMEM: "ENOMEM", ZERO_EHIP: "EHIP",
          ZERO_EUNSUPPORTED: "EUNSUPPORTED"}


class ZeroError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"zero [{_CODES.get(code, code)}]: {msg}")
        self.code = code
        self.msg = msg


_lib = None


def lib():
    """Load libzero.so (built in-tree by build.py) and declare signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ZeroError(ZERO_EUNSUPPORTED,
                        f"{LIB_PATH} is not built; run __graft_entry__.build() or "
                        "python -m zero_partitioned_optimizer_flatten_amd.build")
    L = ctypes.CDLL(LIB_PATH)
    i64, i32, vp, dbl = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_double
    p64 = ctypes.POINTER(ctypes.c_int64)
    L.zero_last_error.restype = ctypes.c_char_p
    L.zero_shard_geometry.argtypes = [i64, i32, i32, p64, p64, p64]
    L.zero_shard_init.argtypes = [i64, i32, i32, dbl, dbl, dbl, dbl, ctypes.POINTER(vp)]
    L.zero_shard_info.argtypes = [vp, p64, p64, p64]
    L.zero_shard_state_bytes.argtypes = [vp, p64]
    L.zero_set_lr.argtypes = [vp, dbl]
    L.zero_load_master.argtypes = [vp, vp, ctypes.c_int, i64, vp]
    L.zero_flatten.argtypes = [vp, vp, vp, i32, ctypes.c_int, vp, vp]
    L.zero_unflatten.argtypes = [vp, vp, i32, vp, ctypes.c_int, vp, vp]
    L.zero_flatten_range.argtypes = [vp, vp, vp, i32, ctypes.c_int, vp, i64, i64, vp]
    L.zero_step.argtypes = [vp, vp, i32, ctypes.c_int, i64, vp, ctypes.c_int, i64, i64, vp]
    L.zero_step_range.argtypes = [vp, i64, i64, vp, i32, ctypes.c_int, i64, vp, ctypes.c_int,
                                  i64, i64, vp]
    L.zero_dim0_split.argtypes = [i64, i32, i32, p64, p64]
    L.zero_fsdp_init.argtypes = [i32, vp, vp, i32, i32, dbl, dbl, dbl, dbl, ctypes.POINTER(vp)]
    L.zero_fsdp_local.argtypes = [vp, i32, p64, p64, p64]
    L.zero_fsdp_load_master.argtypes = [vp, vp, ctypes.c_int, vp]
    L.zero_fsdp_step.argtypes = [vp, vp, i32, ctypes.c_int, vp, ctypes.c_int, i64, vp]
    L.zero_set_step_workgroups.argtypes = [vp, i32]
    L.zero_schedule_init.argtypes = [vp, i64, vp]
    L.zero_schedule_init_noalloc.argtypes = [vp, i64, vp]
    L.zero_schedule_lr.argtypes = [vp, dbl, vp]
    L.zero_schedule_get.argtypes = [vp, p64, vp]
    L.zero_step_begin.argtypes = [vp, vp]
    L.zero_step_sched.argtypes = [vp, vp, i32, ctypes.c_int, i64, vp, ctypes.c_int, i64, vp]
    L.zero_step_range_sched.argtypes = [vp, i64, i64, vp, i32, ctypes.c_int, i64, vp,
                                        ctypes.c_int, i64, vp]
    L.zero_fsdp_step_sched.argtypes = [vp, vp, i32, ctypes.c_int, vp, ctypes.c_int, vp]
    L.zero_get_state.argtypes = [vp, vp, vp, vp, vp]
    L.zero_set_state.argtypes = [vp, vp, vp, vp, vp]
    L.zero_state_bytes.argtypes = [i32, dbl, dbl, ctypes.POINTER(dbl)]
    L.zero_destroy.argtypes = [vp]
    L.zero_destroy.restype = None
    _lib = L
    return L


def _check(rc: int):
    if rc != ZERO_OK:
        raise ZeroError(rc, lib().zero_last_error().decode(errors="replace"))


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return ZERO_BF16
    if dt == torch.float32:
        return ZERO_F32
    raise TypeError(f"only float32 and bfloat16 are supported, got {dt}")


def _stream_handle(stream: Optional[torch.cuda.Stream]) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr_array(ptrs: Sequence[int]):
    arr = (ctypes.c_void_p * max(1, len(ptrs)))()
    for i, p in enumerate(ptrs):
        arr[i] = p
    return arr


def shard_geometry(numel: int, world: int, rank: int) -> Tuple[int, int, int]:
    """(shard, lo, padded) for this rank (host computation in the library)."""
    s, lo, p = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    _check(lib().zero_shard_geometry(numel, world, rank, ctypes.byref(s),
                                     ctypes.byref(lo), ctypes.byref(p)))
    return s.value, lo.value, p.value


def state_bytes(stage: int, numel: float, world: float) -> float:
    """Model-state bytes per card for ZeRO stage 0..3."""
    out = ctypes.c_double()
    _check(lib().zero_state_bytes(stage, float(numel), float(world), ctypes.byref(out)))
    return out.value


class ShardState:
    """One data-parallel rank's ZeRO-2 optimizer state on the current GPU.

    Mirrors the pages' ZeroAdam(params, lr, betas, eps) for one rank: the
    library owns fp32 master/m/v of `shard` elements; gradients, flat
    buffers and streams belong to the caller. The step number t is passed
    explicitly (first step t = 1), or kept on the device with schedule()
    for the *_sched calls, which a captured HIP graph can replay.
    """

    def __init__(self, numel: int, world: int, rank: int, lr: float,
                 betas: Tuple[float, float] = (0.9, 0.999), eps: float = 1e-8,
                 device=None):
        self.device = torch.device("cuda", torch.cuda.current_device()) if device is None \
            else torch.device(device)
        self.numel, self.world, self.rank = int(numel), int(world), int(rank)
        h = ctypes.c_void_p()
        with torch.cuda.device(self.device):
            _check(lib().zero_shard_init(self.numel, self.world, self.rank, float(lr),
                                         float(betas[0]), float(betas[1]), float(eps),
                                         ctypes.byref(h)))
        self._h = h
        s, lo, p = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
        _check(lib().zero_shard_info(self._h, ctypes.byref(s), ctypes.byref(lo),
                                     ctypes.byref(p)))
        self.shard, self.lo, self.padded = s.value, lo.value, p.value

    # ------------------------------------------------------------ helpers
    def _dev(self, t: torch.Tensor, what: str):
        if t.device != self.device:
            raise ValueError(f"{what} is on {t.device}, state is on {self.device}")
        if not t.is_contiguous():
            raise ValueError(f"{what} must be contiguous")

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            lib().zero_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    # ------------------------------------------------------------- calls
    def set_step_workgroups(self, per_cu: int):
        """Cap later flat-layout steps at per_cu workgroups per compute unit
        (0: uncapped); results are unchanged."""
        _check(lib().zero_set_step_workgroups(self._h, int(per_cu)))

    def state_bytes(self) -> int:
        """Bytes of fp32 master, m and v this rank holds (12 per element)."""
        out = ctypes.c_int64()
        _check(lib().zero_shard_state_bytes(self._h, ctypes.byref(out)))
        return out.value

    def set_lr(self, lr: float):
        _check(lib().zero_set_lr(self._h, float(lr)))

    def load_master(self, flat_params: torch.Tensor, flat_offset: Optional[int] = None,
                    stream=None):
        """master = fp32(flat_params[flat_offset : flat_offset+shard]); m = v = 0.
        flat_offset defaults to lo for a full padded buffer, 0 otherwise."""
        self._dev(flat_params, "flat_params")
        off = flat_offset
        if off is None:
            off = self.lo if flat_params.numel() >= self.padded else 0
        if flat_params.numel() < off + self.shard:
            raise ValueError(f"flat_params has {flat_params.numel()} elements, "
                             f"need {off + self.shard}")
        _check(lib().zero_load_master(self._h, flat_params.data_ptr(),
                                      _dtype_code(flat_params.dtype), off,
                                      _stream_handle(stream)))

    def flatten(self, tensors: Sequence[torch.Tensor], out: torch.Tensor, stream=None,
                window: Optional[Tuple[int, int]] = None):
        """out[:numel] = concatenation of the tensors; out[numel:padded] = 0.
        window=(begin, count) writes only flat elements [begin, begin+count)."""
        dt = out.dtype
        self._dev(out, "out")
        if out.numel() < self.padded:
            raise ValueError(f"out has {out.numel()} elements, need {self.padded}")
        for i, t in enumerate(tensors):
            self._dev(t, f"tensors[{i}]")
            if t.dtype != dt:
                raise TypeError(f"tensors[{i}] is {t.dtype}, out is {dt}")
        numels = (ctypes.c_int64 * max(1, len(tensors)))(*[t.numel() for t in tensors])
        ptrs = _ptr_array([t.data_ptr() for t in tensors])
        if window is None:
            _check(lib().zero_flatten(self._h, ptrs, numels, len(tensors), _dtype_code(dt),
                                      out.data_ptr(), _stream_handle(stream)))
        else:
            b, n = window
            _check(lib().zero_flatten_range(self._h, ptrs, numels, len(tensors), _dtype_code(dt),
                                            out.data_ptr(), int(b), int(n),
                                            _stream_handle(stream)))

    def unflatten(self, flat: torch.Tensor, tensors: Sequence[torch.Tensor], stream=None):
        """Copy flat[off_t : off_t + numel_t] into each tensor, in order."""
        dt = flat.dtype
        self._dev(flat, "flat")
        if flat.numel() < self.numel:
            raise ValueError(f"flat has {flat.numel()} elements, need {self.numel}")
        for i, t in enumerate(tensors):
            self._dev(t, f"tensors[{i}]")
            if t.dtype != dt:
                raise TypeError(f"tensors[{i}] is {t.dtype}, flat is {dt}")
        numels = (ctypes.c_int64 * max(1, len(tensors)))(*[t.numel() for t in tensors])
        ptrs = _ptr_array([t.data_ptr() for t in tensors])
        _check(lib().zero_unflatten(self._h, flat.data_ptr(), len(tensors), numels,
                                    _dtype_code(dt), ptrs, _stream_handle(stream)))

    def _step_args(self, replicas, param_out, grad_offset, param_offset):
        if len(replicas) != self.world:
            raise ValueError(f"need {self.world} replicas, got {len(replicas)}")
        gdt = replicas[0].dtype
        go = grad_offset
        if go is None:
            go = self.lo if replicas[0].numel() >= self.padded else 0
        po = param_offset
        if po is None:
            po = self.lo if param_out.numel() >= self.padded else 0
        for q, r in enumerate(replicas):
            self._dev(r, f"replicas[{q}]")
            if r.dtype != gdt:
                raise TypeError("replicas must share one dtype")
            if r.numel() < go + self.shard:
                raise ValueError(f"replicas[{q}] has {r.numel()} elements, need {go + self.shard}")
        self._dev(param_out, "param_out")
        if param_out.numel() < po + self.shard:
            raise ValueError(f"param_out has {param_out.numel()} elements, need {po + self.shard}")
        return _ptr_array([r.data_ptr() for r in replicas]), gdt, int(go), int(po)

    def _range_args(self, shard_begin, count, replicas, param_out, grad_offset, param_offset):
        if len(replicas) != self.world:
            raise ValueError(f"need {self.world} replicas, got {len(replicas)}")
        if shard_begin < 0 or count < 0 or shard_begin + count > self.shard:
            raise ValueError(f"range [{shard_begin}, {shard_begin + count}) outside the shard")
        gdt = replicas[0].dtype
        for q, r in enumerate(replicas):
            self._dev(r, f"replicas[{q}]")
            if r.dtype != gdt:
                raise TypeError("replicas must share one dtype")
            if r.numel() < grad_offset + count:
                raise ValueError(f"replicas[{q}] has {r.numel()} elements, need {grad_offset + count}")
        self._dev(param_out, "param_out")
        if param_out.numel() < param_offset + count:
            raise ValueError(f"param_out has {param_out.numel()} elements, need {param_offset + count}")
        return _ptr_array([r.data_ptr() for r in replicas]), gdt

    def step(self, replicas: Sequence[torch.Tensor], t: int, param_out: torch.Tensor,
             grad_offset: Optional[int] = None, param_offset: Optional[int] = None,
             stream=None):
        """One shard step. replicas[q][grad_offset + i] is rank q's gradient of
        slice element i; writes param_out[param_offset + i]. Offsets default
        to lo for full padded buffers and 0 for slice-sized ones."""
        ptrs, gdt, go, po = self._step_args(replicas, param_out, grad_offset, param_offset)
        _check(lib().zero_step(self._h, ptrs, len(replicas), _dtype_code(gdt), go,
                               param_out.data_ptr(), _dtype_code(param_out.dtype), po,
                               int(t), _stream_handle(stream)))

    def step_range(self, shard_begin: int, count: int, replicas: Sequence[torch.Tensor],
                   t: int, param_out: torch.Tensor, grad_offset: int = 0,
                   param_offset: int = 0, stream=None):
        """The step on shard elements [shard_begin, shard_begin+count):
        replicas[q][grad_offset + i] feeds element shard_begin + i, which is
        written to param_out[param_offset + i]. Disjoint ranges on different
        streams may run concurrently."""
        ptrs, gdt = self._range_args(shard_begin, count, replicas, param_out, grad_offset,
                                     param_offset)
        _check(lib().zero_step_range(self._h, int(shard_begin), int(count), ptrs, len(replicas),
                                     _dtype_code(gdt), int(grad_offset), param_out.data_ptr(),
                                     _dtype_code(param_out.dtype), int(param_offset), int(t),
                                     _stream_handle(stream)))

    # ------------------------------------------- device-resident schedule
    def schedule(self, next_t: int = 1, stream=None):
        """Keep the step count and lr on the device (created on first use,
        outside any graph capture): the next scheduled step is next_t."""
        with torch.cuda.device(self.device):
            _check(lib().zero_schedule_init(self._h, int(next_t), _stream_handle(stream)))

    def schedule_noalloc(self, next_t: int = 1, stream=None):
        """schedule() in the device's static block: allocates nothing (one
        such schedule per device at a time)."""
        with torch.cuda.device(self.device):
            _check(lib().zero_schedule_init_noalloc(self._h, int(next_t),
                                                    _stream_handle(stream)))

    def schedule_lr(self, lr: float, stream=None):
        """Learning rate of later scheduled steps (stream-ordered)."""
        _check(lib().zero_schedule_lr(self._h, float(lr), _stream_handle(stream)))

    def schedule_next_t(self, stream=None) -> int:
        """The next scheduled step count (waits for the stream)."""
        out = ctypes.c_int64()
        _check(lib().zero_schedule_get(self._h, ctypes.byref(out), _stream_handle(stream)))
        return out.value

    def step_begin(self, stream=None):
        """Begin the next scheduled step (before step_range_sched calls)."""
        _check(lib().zero_step_begin(self._h, _stream_handle(stream)))

    def step_sched(self, replicas: Sequence[torch.Tensor], param_out: torch.Tensor,
                   grad_offset: Optional[int] = None, param_offset: Optional[int] = None,
                   stream=None):
        """step() at the device schedule's next step count and lr; advances
        the count. Capturable in a HIP graph."""
        ptrs, gdt, go, po = self._step_args(replicas, param_out, grad_offset, param_offset)
        _check(lib().zero_step_sched(self._h, ptrs, len(replicas), _dtype_code(gdt), go,
                                     param_out.data_ptr(), _dtype_code(param_out.dtype), po,
                                     _stream_handle(stream)))

    def step_range_sched(self, shard_begin: int, count: int, replicas: Sequence[torch.Tensor],
                         param_out: torch.Tensor, grad_offset: int = 0, param_offset: int = 0,
                         stream=None):
        """step_range() at the step the last step_begin began."""
        ptrs, gdt = self._range_args(shard_begin, count, replicas, param_out, grad_offset,
                                     param_offset)
        _check(lib().zero_step_range_sched(self._h, int(shard_begin), int(count), ptrs,
                                           len(replicas), _dtype_code(gdt), int(grad_offset),
                                           param_out.data_ptr(), _dtype_code(param_out.dtype),
                                           int(param_offset), _stream_handle(stream)))

    def bucket_ranges(self, bucket_bounds: Sequence[int]) -> List[Tuple[int, int, int, int]]:
        """For gradient buckets given as flat-vector boundaries
        [b0=0, b1, ..., bk=padded], the part of each bucket this rank owns:
        (bucket index, shard_begin, count, offset of that part inside the
        bucket). Buckets that miss this rank's slice are left out."""
        out = []
        lo, hi = self.lo, self.lo + self.shard
        for k in range(len(bucket_bounds) - 1):
            a, b = int(bucket_bounds[k]), int(bucket_bounds[k + 1])
            s, e = max(a, lo), min(b, hi)
            if s < e:
                out.append((k, s - lo, e - s, s - a))
        return out

    def get_state(self, stream=None) -> List[torch.Tensor]:
        """Fresh fp32 copies of (master, m, v)."""
        out = [torch.empty(self.shard, dtype=torch.float32, device=self.device)
               for _ in range(3)]
        _check(lib().zero_get_state(self._h, out[0].data_ptr(), out[1].data_ptr(),
                                    out[2].data_ptr(), _stream_handle(stream)))
        return out

    def set_state(self, master: torch.Tensor, m: torch.Tensor, v: torch.Tensor, stream=None):
        for name, x in (("master", master), ("m", m), ("v", v)):
            self._dev(x, name)
            if x.dtype != torch.float32 or x.numel() != self.shard:
                raise ValueError(f"{name} must be float32 with {self.shard} elements")
        _check(lib().zero_set_state(self._h, master.data_ptr(), m.data_ptr(), v.data_ptr(),
                                    _stream_handle(stream)))


def dim0_split(dim0: int, world: int, rank: int) -> Tuple[int, int]:
    """(first row, rows) of this rank's dim-0 shard of a parameter."""
    f, r = ctypes.c_int64(), ctypes.c_int64()
    _check(lib().zero_dim0_split(dim0, world, rank, ctypes.byref(f), ctypes.byref(r)))
    return f.value, r.value


class FsdpShardState(ShardState):
    """One rank of the per-parameter (FSDP2-style) layout: every parameter
    is split along dim 0 and this rank keeps fp32 master/m/v for its rows.
    Inherits get_state / set_state / set_lr / close from ShardState."""

    def __init__(self, shapes, world: int, rank: int, lr: float,
                 betas: Tuple[float, float] = (0.9, 0.999), eps: float = 1e-8, device=None):
        self.device = torch.device("cuda", torch.cuda.current_device()) if device is None \
            else torch.device(device)
        self.shapes = [tuple(int(d) for d in s) for s in shapes]
        self.world, self.rank = int(world), int(rank)
        n = len(self.shapes)
        dim0 = (ctypes.c_int64 * max(1, n))(*[s[0] if s else 1 for s in self.shapes])
        rown = (ctypes.c_int64 * max(1, n))(*[
            int(torch.Size(s[1:]).numel()) if len(s) > 1 else 1 for s in self.shapes])
        h = ctypes.c_void_p()
        with torch.cuda.device(self.device):
            _check(lib().zero_fsdp_init(n, dim0, rown, self.world, self.rank, float(lr),
                                        float(betas[0]), float(betas[1]), float(eps),
                                        ctypes.byref(h)))
        self._h = h
        s_, lo, p = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
        _check(lib().zero_shard_info(self._h, ctypes.byref(s_), ctypes.byref(lo), ctypes.byref(p)))
        self.shard, self.lo, self.padded = s_.value, lo.value, p.value
        self.numel = sum(int(torch.Size(s).numel()) for s in self.shapes)
        self.local = []
        for k in range(n):
            f, r, off = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
            _check(lib().zero_fsdp_local(self._h, k, ctypes.byref(f), ctypes.byref(r),
                                         ctypes.byref(off)))
            self.local.append((f.value, r.value, off.value))

    def local_shape(self, k: int) -> Tuple[int, ...]:
        return (self.local[k][1],) + self.shapes[k][1:]

    def local_numel(self, k: int) -> int:
        return int(torch.Size(self.local_shape(k)).numel())

    def _check_full(self, ts, what):
        if len(ts) != len(self.shapes):
            raise ValueError(f"{what}: need {len(self.shapes)} tensors, got {len(ts)}")
        for k, x in enumerate(ts):
            if x is None:
                if self.local[k][1]:
                    raise ValueError(f"{what}[{k}] is None but this rank holds rows of it")
                continue
            self._dev(x, f"{what}[{k}]")
            if tuple(x.shape) != self.shapes[k] and x.numel() != torch.Size(self.shapes[k]).numel():
                raise ValueError(f"{what}[{k}] has shape {tuple(x.shape)}, need {self.shapes[k]}")

    def load_master(self, params: Sequence[torch.Tensor], stream=None):
        """master = this rank's rows of each full parameter; m = v = 0."""
        self._check_full(params, "params")
        dts = {p.dtype for p in params if p is not None}
        if len(dts) != 1:
            raise TypeError("params must share one dtype")
        ptrs = _ptr_array([p.data_ptr() if p is not None else 0 for p in params])
        _check(lib().zero_fsdp_load_master(self._h, ptrs, _dtype_code(dts.pop()),
                                           _stream_handle(stream)))

    def _fsdp_args(self, replica_grads, params_out):
        if len(replica_grads) != self.world:
            raise ValueError(f"need {self.world} replicas, got {len(replica_grads)}")
        gdts = set()
        for q, gl in enumerate(replica_grads):
            self._check_full(gl, f"replica_grads[{q}]")
            gdts |= {g.dtype for g in gl if g is not None}
        if len(gdts) != 1:
            raise TypeError("gradients must share one dtype")
        if len(params_out) != len(self.shapes):
            raise ValueError("need one output shard per parameter")
        pdts = set()
        for k, o in enumerate(params_out):
            if self.local[k][1] == 0:
                continue
            self._dev(o, f"params_out[{k}]")
            if o.numel() < self.local_numel(k):
                raise ValueError(f"params_out[{k}] has {o.numel()} elements, "
                                 f"need {self.local_numel(k)}")
            pdts.add(o.dtype)
        if len(pdts) > 1:
            raise TypeError("outputs must share one dtype")
        pdt = pdts.pop() if pdts else torch.float32
        gptrs = _ptr_array([g.data_ptr() if g is not None else 0
                            for gl in replica_grads for g in gl])
        optrs = _ptr_array([o.data_ptr() if (o is not None and self.local[k][1]) else 0
                            for k, o in enumerate(params_out)])
        return gptrs, gdts.pop(), optrs, pdt

    def step(self, replica_grads: Sequence[Sequence[torch.Tensor]], t: int,
             params_out: Sequence[torch.Tensor], stream=None):
        """replica_grads[q][k]: replica q's full gradient of parameter k;
        params_out[k]: this rank's local shard of parameter k (written)."""
        gptrs, gdt, optrs, pdt = self._fsdp_args(replica_grads, params_out)
        _check(lib().zero_fsdp_step(self._h, gptrs, self.world, _dtype_code(gdt), optrs,
                                    _dtype_code(pdt), int(t), _stream_handle(stream)))

    def step_sched(self, replica_grads: Sequence[Sequence[torch.Tensor]],
                   params_out: Sequence[torch.Tensor], stream=None):
        """step() at the device schedule's next step count and lr."""
        gptrs, gdt, optrs, pdt = self._fsdp_args(replica_grads, params_out)
        _check(lib().zero_fsdp_step_sched(self._h, gptrs, self.world, _dtype_code(gdt), optrs,
                                          _dtype_code(pdt), _stream_handle(stream)))

    def state_pieces(self, state: Sequence[torch.Tensor]):
        """Split (master, m, v) from get_state into per-parameter local pieces."""
        out = []
        for x in state:
            out.append([x[off:off + r * (int(torch.Size(self.shapes[k][1:]).numel())
                                          if len(self.shapes[k]) > 1 else 1)]
                        for k, (_, r, off) in enumerate(self.local)])
        return out
