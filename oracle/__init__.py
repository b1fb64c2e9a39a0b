"""CPU oracle for one rank's ZeRO-2 optimizer step (TEST INFRASTRUCTURE).

Only `tests/`, `__graft_entry__.smoke()` and the CPU-baseline leg of
`bench.py` may import this package. It wraps `oracle.c` (plain C, compiled
with gcc, -ffp-contract=off, OpenMP) through ctypes and works on numpy
arrays; it never imports the HIP library or its binding.

bf16 data is carried as numpy uint16 bit patterns.

Pages followed: "ZeRO and FSDP: partitioning the optimizer states, the
gradients and the parameters" (AI infra handbook), section "Implementing
ZeRO's Adam from scratch", class ZeroAdam (constructor, _flatten, step,
state_bytes) and table "The three stages".

Parity pins (tests/oracle_pins.py, run by tests/test_oracle_pins.py; each
planted mistake in tests/test_oracle_mutants.py fails at least one):
  geometry       brute force over small sizes, exact Fraction ceilings
  dim0_split     torch.chunk, the page's 128-row FSDP2 example
  stage_bytes    the page's 13B/16-card worked example, per-component bytes
  state_bytes    the page's toy model (state_bytes and its 1/4 ratio)
  flatten        torch.cat plus a zero tail, brute force
  unflatten      round trip through the pinned flatten
  bf16_round     torch's bf16 cast over every high half and the tie cases
  step_scalars   dyadic closed forms; binary64 power rounded once
  reduce_mean    N = 1, identical replicas, a rank-order example, an error bound
  shard_step     closed forms, torch.optim.Adam, the page's step lines in torch,
                 the sharded == unsharded invariant at non-zero offsets
  load_master    a slice taken at lo (not at 0) of a known vector
Unpinned: the NaN payload bits of the bf16 cast (only NaN-ness, the sign and
the quiet bit are compared).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import List, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
          "-fno-fast-math", "-fopenmp", "-Wall", "-Wextra"]


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so next to it."""
    if force or not os.path.exists(_LIB) or (
            os.path.getmtime(_LIB) < os.path.getmtime(_SRC)):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def load(path: str):
    """Load a compiled oracle library and declare its signatures."""
    L = ctypes.CDLL(path)
    i64, i32, vp, dbl = (ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                         ctypes.c_double)
    L.oracle_geometry.argtypes = [i64, i64, i64, vp]
    L.oracle_dim0_split.argtypes = [i64, i64, i64, vp]
    L.oracle_stage_bytes.argtypes = [ctypes.c_int, dbl, dbl]
    L.oracle_stage_bytes.restype = dbl
    L.oracle_state_bytes.argtypes = [i64]
    L.oracle_state_bytes.restype = i64
    L.oracle_flatten.argtypes = [vp, vp, i32, i32, vp, i64]
    L.oracle_unflatten.argtypes = [vp, i32, vp, i32, vp]
    L.oracle_bf16_round.argtypes = [ctypes.c_float]
    L.oracle_bf16_round.restype = ctypes.c_uint16
    L.oracle_bf16_round_array.argtypes = [vp, i64, vp]
    L.oracle_step_scalars.argtypes = [dbl, dbl, dbl, dbl, i64, i32, vp]
    L.oracle_reduce_mean.argtypes = [vp, i32, i32, i64, i64, ctypes.c_float, vp]
    L.oracle_shard_step.argtypes = [vp, i32, i32, i64, vp, vp, vp, i64, vp,
                                    vp, i32, i64]
    L.oracle_load_master.argtypes = [vp, i32, i64, i64, vp, vp, vp]
    L.oracle_num_threads.restype = ctypes.c_int
    L.oracle_set_threads.argtypes = [ctypes.c_int]
    return L


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        _lib = load(_LIB)
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"], "oracle needs contiguous arrays"
    return a.ctypes.data


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what}: invalid arguments (rc={rc})")


def _ptr_array(arrays: Sequence[np.ndarray]):
    arr = (ctypes.c_void_p * max(1, len(arrays)))()
    for i, a in enumerate(arrays):
        arr[i] = _ptr(a)
    return arr


def _is_bf16(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return 1
    if a.dtype == np.float32:
        return 0
    raise TypeError(f"oracle takes float32 or bf16-as-uint16, got {a.dtype}")


# ----------------------------------------------------------------- geometry

def geometry(numel: int, world: int, rank: int) -> dict:
    out = np.zeros(5, dtype=np.int64)
    _check(lib().oracle_geometry(numel, world, rank, _ptr(out)), "geometry")
    return dict(shard=int(out[0]), lo=int(out[1]), padded=int(out[2]),
                pad=int(out[3]), valid=int(out[4]))


def dim0_split(d0: int, world: int, rank: int):
    """(first row, rows) of this rank's dim-0 shard of a parameter."""
    out = np.zeros(2, dtype=np.int64)
    _check(lib().oracle_dim0_split(d0, world, rank, _ptr(out)), "dim0_split")
    return int(out[0]), int(out[1])


def stage_bytes(stage: int, psi: float, n: float) -> float:
    return lib().oracle_stage_bytes(stage, float(psi), float(n))


def state_bytes(shard: int) -> int:
    return lib().oracle_state_bytes(shard)


def num_threads() -> int:
    return lib().oracle_num_threads()


def set_threads(n: int) -> None:
    lib().oracle_set_threads(int(n))


# ------------------------------------------------------------------ flatten

def flatten(tensors: Sequence[np.ndarray], padded: int, fill=None) -> np.ndarray:
    """Concatenate (row-major, list order) and zero-pad to `padded`.
    `fill` pre-fills the output bytes (to show every byte is written)."""
    if not tensors:
        raise ValueError("empty list")
    dt = tensors[0].dtype
    srcs = [np.ascontiguousarray(t).reshape(-1) for t in tensors]
    for s in srcs:
        if s.dtype != dt:
            raise TypeError("mixed dtypes")
    numels = np.array([s.size for s in srcs], dtype=np.int64)
    out = np.empty(padded, dtype=dt)
    if fill is not None:
        out.view(np.uint8)[:] = fill
    _check(lib().oracle_flatten(_ptr_array(srcs), _ptr(numels), len(srcs),
                                dt.itemsize, _ptr(out), padded), "flatten")
    return out


def unflatten(flat: np.ndarray, shapes) -> List[np.ndarray]:
    outs = [np.empty(int(np.prod(s)), dtype=flat.dtype) for s in shapes]
    numels = np.array([o.size for o in outs], dtype=np.int64)
    flat = np.ascontiguousarray(flat)
    _check(lib().oracle_unflatten(_ptr(flat), len(outs), _ptr(numels),
                                  flat.dtype.itemsize, _ptr_array(outs)),
           "unflatten")
    return [o.reshape(s) for o, s in zip(outs, shapes)]


# --------------------------------------------------------------------- bf16

def bf16_round(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().oracle_bf16_round_array(_ptr(x), x.size, _ptr(out))
    return out


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------- step

def step_scalars(lr, b1, b2, eps, t, world) -> np.ndarray:
    sc = np.zeros(9, dtype=np.float32)
    _check(lib().oracle_step_scalars(lr, b1, b2, eps, t, world, _ptr(sc)),
           "step_scalars")
    return sc


def reduce_mean(replicas: Sequence[np.ndarray], offset: int, shard: int,
                world: int) -> np.ndarray:
    isb = _is_bf16(replicas[0])
    for r in replicas:
        if r.size < offset + shard:
            raise ValueError("replica shorter than offset + shard")
    g = np.empty(shard, dtype=np.float32)
    nf = np.float32(world)
    _check(lib().oracle_reduce_mean(_ptr_array(replicas), len(replicas), isb,
                                    offset, shard, ctypes.c_float(nf), _ptr(g)),
           "reduce_mean")
    return g


class ShardOracle:
    """One rank's slice of the pages' ZeroAdam, on the CPU.

    State: fp32 master/m/v of `shard` elements (owned here). The caller owns
    gradients and the flat parameter buffer and passes t explicitly (the
    page's counter starts at 0 and is incremented before use, so the first
    step is t = 1).

    `n_replicas` defaults to `world`; ShardOracle(P, 1, 0, ..., n_replicas=N)
    is one owner updating a whole padded vector from N replicas (the
    unsharded reference for the sharding invariant).
    """

    def __init__(self, numel, world, rank, lr, betas=(0.9, 0.999), eps=1e-8,
                 n_replicas=None):
        self.geo = geometry(numel, world, rank)
        self.numel, self.world, self.rank = numel, world, rank
        self.n_replicas = world if n_replicas is None else n_replicas
        self.lr, self.betas, self.eps = lr, betas, eps
        S = self.geo["shard"]
        self.master = np.zeros(S, dtype=np.float32)
        self.m = np.zeros(S, dtype=np.float32)
        self.v = np.zeros(S, dtype=np.float32)

    @property
    def shard(self):
        return self.geo["shard"]

    @property
    def lo(self):
        return self.geo["lo"]

    def load_master(self, flat_params: np.ndarray):
        if flat_params.size < self.geo["padded"]:
            raise ValueError("flat params shorter than the padded length")
        flat_params = np.ascontiguousarray(flat_params)
        _check(lib().oracle_load_master(_ptr(flat_params), _is_bf16(flat_params),
                                        self.lo, self.shard, _ptr(self.master),
                                        _ptr(self.m), _ptr(self.v)),
               "load_master")

    def scalars(self, t):
        return step_scalars(self.lr, self.betas[0], self.betas[1], self.eps,
                            t, self.n_replicas)

    def step(self, replicas: Sequence[np.ndarray], t: int, out: np.ndarray,
             grad_offset: int = None, out_offset: int = None):
        """replicas[q][grad_offset + i] is replica q's gradient of slice
        element i; writes out[out_offset + i]. Defaults: both offsets = lo
        (full flat buffers)."""
        if len(replicas) != self.n_replicas:
            raise ValueError("need one replica per rank")
        go = self.lo if grad_offset is None else grad_offset
        oo = self.lo if out_offset is None else out_offset
        isb = _is_bf16(replicas[0])
        for r in replicas:
            if _is_bf16(r) != isb or r.size < go + self.shard:
                raise ValueError("replica dtype/size mismatch")
        if out.size < oo + self.shard:
            raise ValueError("output too short")
        sc = self.scalars(t)
        _check(lib().oracle_shard_step(_ptr_array(replicas), len(replicas), isb,
                                       go, _ptr(self.master), _ptr(self.m),
                                       _ptr(self.v), self.shard, _ptr(sc),
                                       _ptr(out), _is_bf16(out), oo),
               "shard_step")


class FsdpShardOracle:
    """One rank of the per-parameter (FSDP2-style) layout: each parameter is
    split along dim 0 (dim0_split) and the rank keeps fp32 master/m/v for
    its rows of every parameter. The update of each local shard is the same
    elementwise step as ShardOracle's, fed by the mean over the N replicas
    of that parameter's gradient rows."""

    def __init__(self, shapes, world, rank, lr, betas=(0.9, 0.999), eps=1e-8):
        self.shapes = [tuple(s) for s in shapes]
        self.world, self.rank = world, rank
        self.rows = []
        self.parts = []
        for shp in self.shapes:
            d0 = shp[0] if shp else 1
            row = int(np.prod(shp[1:])) if len(shp) > 1 else 1
            first, nrows = dim0_split(d0, world, rank)
            self.rows.append((first, nrows, row))
            self.parts.append(ShardOracle(max(1, nrows * row), 1, 0, lr, betas, eps,
                                          n_replicas=world) if nrows * row > 0 else None)

    def local_numels(self):
        return [n * r for (_, n, r) in self.rows]

    def _local(self, full: np.ndarray, k: int) -> np.ndarray:
        first, nrows, row = self.rows[k]
        return np.ascontiguousarray(full.reshape(-1)[first * row:(first + nrows) * row])

    def load_master(self, params_full):
        for k, p in enumerate(params_full):
            if self.parts[k] is not None:
                self.parts[k].load_master(self._local(p, k))

    def step(self, replica_grads, t, outs):
        """replica_grads[q][k]: replica q's full gradient of parameter k;
        outs[k]: this rank's local shard of parameter k (written)."""
        for k, part in enumerate(self.parts):
            if part is None:
                continue
            local = [self._local(replica_grads[q][k], k) for q in range(self.world)]
            part.step(local, t, outs[k], grad_offset=0, out_offset=0)

    def state(self):
        keys = ("master", "m", "v")
        return [np.concatenate([getattr(p, key) for p in self.parts if p is not None]
                               or [np.zeros(0, np.float32)]) for key in keys]
