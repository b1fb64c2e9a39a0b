"""Shared helpers for the GPU parity tests: bit views, the error metrics the
parity bar is stated in, and drivers that run the HIP path and the CPU
oracle on the same seeded inputs."""
from __future__ import annotations

import sys
import time

import numpy as np
import torch

import oracle
import synth
import zero_partitioned_optimizer_flatten_amd as zero

# Parity bar: fp32 master/m/v within 2e-6 relative error, written bf16
# parameters within 1 ulp, flatten bit-exact. The kernels run the oracle's
# exact operation sequence, so 0 differing elements is expected as well.
REL_TOL = 2e-6
BF16_ULP_TOL = 1


def log(msg: str):
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


def bits(t: torch.Tensor) -> np.ndarray:
    """Host copy of a tensor as numpy: bf16 -> uint16 bit patterns, fp32 ->
    float32."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    if t.dtype == torch.float32:
        return t.numpy().copy()
    raise TypeError(t.dtype)


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max |got - ref| / max(|ref|, 2^-126); matching NaNs count as equal,
    +0 and -0 compare equal."""
    got = got.astype(np.float64)
    ref = ref.astype(np.float64)
    both_nan = np.isnan(got) & np.isnan(ref)
    with np.errstate(invalid="ignore"):
        d = np.abs(got - ref) / np.maximum(np.abs(ref), 2.0**-126)
        same_inf = np.isinf(got) & np.isinf(ref) & (np.sign(got) == np.sign(ref))
    d[both_nan | same_inf] = 0.0
    d[np.isnan(d)] = np.inf
    return float(d.max()) if d.size else 0.0


def _ordered_bf16(b: np.ndarray) -> np.ndarray:
    b = b.astype(np.int64)
    neg = (b & 0x8000) != 0
    return np.where(neg, 0x8000 - (b & 0x7FFF), 0x8000 + (b & 0x7FFF))


def bf16_ulp(got: np.ndarray, ref: np.ndarray) -> int:
    """Largest distance between bf16 bit patterns in ordered order (NaN
    against NaN counts 0)."""
    g_nan = ((got & 0x7F80) == 0x7F80) & ((got & 0x007F) != 0)
    r_nan = ((ref & 0x7F80) == 0x7F80) & ((ref & 0x007F) != 0)
    d = np.abs(_ordered_bf16(got) - _ordered_bf16(ref))
    d[g_nan & r_nan] = 0
    d[g_nan ^ r_nan] = 1 << 20
    return int(d.max()) if d.size else 0


def _isnan_bits(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.uint16:
        return ((a & 0x7F80) == 0x7F80) & ((a & 0x007F) != 0)
    return np.isnan(a)


def mismatches(got: np.ndarray, ref: np.ndarray) -> int:
    """Elements whose bit patterns differ; a NaN against a NaN counts as
    equal (NaN payload and sign are not part of the parity bar)."""
    gv = got.view(np.uint32 if got.dtype == np.float32 else np.uint16)
    rv = ref.view(np.uint32 if ref.dtype == np.float32 else np.uint16)
    both_nan = _isnan_bits(got) & _isnan_bits(ref)
    return int(np.count_nonzero((gv != rv) & ~both_nan))


def assert_state_parity(label, gpu_state, ref_state, out_got=None, out_ref=None):
    """gpu_state/ref_state: (master, m, v) float32 arrays."""
    report = []
    for name, g, r in zip(("master", "m", "v"), gpu_state, ref_state):
        e = rel_err(g, r)
        mm = mismatches(g, r)
        report.append(f"{name}: rel {e:.3g}, {mm} differ")
        assert e <= REL_TOL, f"{label}: {name} max rel err {e} > {REL_TOL}"
    if out_got is not None:
        if out_got.dtype == np.uint16:
            u = bf16_ulp(out_got, out_ref)
            report.append(f"out: {u} ulp, {mismatches(out_got, out_ref)} differ")
            assert u <= BF16_ULP_TOL, f"{label}: bf16 output {u} ulp apart"
        else:
            e = rel_err(out_got, out_ref)
            report.append(f"out: rel {e:.3g}")
            assert e <= REL_TOL, f"{label}: fp32 output rel err {e}"
    log(f"{label}: " + "; ".join(report))
    return report


def assert_bitexact_state(label, gpu_state, ref_state, out_got=None, out_ref=None):
    for name, g, r in zip(("master", "m", "v"), gpu_state, ref_state):
        assert mismatches(g, r) == 0, f"{label}: {name} not bit-exact"
    if out_got is not None:
        assert mismatches(out_got, out_ref) == 0, f"{label}: output not bit-exact"


def gpu_state(st: zero.ShardState):
    return [x.cpu().numpy() for x in st.get_state()]


def run_small_parity(numel, world, rank, grad_dtype, out_dtype, steps, std,
                     shapes=None, lr=1e-3, betas=(0.9, 0.999), eps=1e-8,
                     outliers=False, full_out=True, label="", check_every=1):
    """Full-size parity for shards the oracle finishes in seconds: every
    replica is a full padded flat vector built by the HIP flatten from a
    tensor list; every element is compared."""
    dev = torch.device("cuda", torch.cuda.current_device())
    shapes = shapes or [(numel,)]
    st = zero.ShardState(numel, world, rank, lr, betas, eps)
    orc = oracle.ShardOracle(numel, world, rank, lr, betas, eps)
    S, lo, P = st.shard, st.lo, st.padded
    p_flat_cpu = synth.params(numel)
    plist = synth.split_to_shapes(p_flat_cpu, shapes)
    flat_p = torch.empty(P, dtype=torch.float32, device=dev)
    st.flatten([x.to(dev) for x in plist], flat_p)
    st.load_master(flat_p)
    orc.load_master(oracle.flatten([x.numpy().reshape(-1) for x in plist], P))
    if out_dtype == torch.bfloat16:
        out = torch.full((P if full_out else S,), -1, dtype=torch.int16, device=dev).view(torch.bfloat16)
        out_ref = np.full(P if full_out else S, 0xFFFF, dtype=np.uint16)
    else:
        out = torch.full((P if full_out else S,), float("nan"), dtype=torch.float32, device=dev)
        out_ref = np.full(P if full_out else S, np.nan, dtype=np.float32)
    for t in range(1, steps + 1):
        reps, reps_h = [], []
        for q in range(world):
            if outliers:
                g = synth.gaussian_with_outliers(numel, std, synth.grad_seed(t, q),
                                                 synth.mask_seed(t, q), dtype=grad_dtype,
                                                 device=dev)
            else:
                g = synth.gaussian(numel, std, synth.grad_seed(t, q), grad_dtype, device=dev)
            flat = torch.empty(P, dtype=grad_dtype, device=dev)
            st.flatten(synth.split_to_shapes(g, shapes), flat)
            reps.append(flat)
            reps_h.append(bits(flat))
        st.step(reps, t, out)
        orc.step(reps_h, t, out_ref, out_offset=lo if full_out else 0)
        if t % check_every == 0 or t == steps:
            torch.cuda.synchronize()
            assert_state_parity(f"{label} t={t}", gpu_state(st), [orc.master, orc.m, orc.v],
                                bits(out), out_ref)
    res = dict(state=gpu_state(st), ref=[orc.master.copy(), orc.m.copy(), orc.v.copy()],
               out=bits(out), out_ref=out_ref, S=S, lo=lo, P=P)
    st.close()
    return res
