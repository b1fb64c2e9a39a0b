"""The C ABI on a machine without a GPU: the library loads, exports every
function include/zero.h declares, and its host-only logic and argument
checks behave as documented. No kernel is launched here."""
import ctypes
import os
import re

import pytest
import torch

import zero_partitioned_optimizer_flatten_amd as zero
import oracle


def _declared_functions():
    with open(zero.HEADER_PATH) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b(zero_[a-z_]+)\s*\(", text)
    return sorted(set(names))


def test_library_exports_every_declared_function():
    names = _declared_functions()
    assert len(names) >= 13, names
    L = zero.lib()
    missing = [n for n in names if not hasattr(L, n)]
    assert not missing, missing


def test_header_is_plain_c():
    """The header compiles as C (no C++ or torch types in the ABI)."""
    import subprocess
    import tempfile
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "t.c")
        with open(c, "w") as f:
            f.write('#include "zero.h"\nint main(void){zero_ctx *c = 0; (void)c; return 0;}\n')
        subprocess.check_call(["gcc", "-std=c99", "-D__HIP_PLATFORM_AMD__", "-fsyntax-only",
                               "-I", os.path.dirname(zero.HEADER_PATH),
                               "-I", "/opt/rocm/include", c])


def test_geometry_matches_oracle():
    for numel in (1, 2, 7, 8, 9, 1000, 1_000_003, 13_015_864_321, 70_000_000_000):
        for world in (1, 3, 4, 8, 64, 256):
            for rank in {0, world // 2, world - 1}:
                g = oracle.geometry(numel, world, rank)
                assert zero.shard_geometry(numel, world, rank) == (g["shard"], g["lo"], g["padded"])


def test_state_bytes_matches_oracle():
    for stage in range(4):
        for psi, n in ((13e9, 16), (7e9, 8), (70e9, 64), (1.0, 1)):
            assert zero.state_bytes(stage, psi, n) == pytest.approx(
                oracle.stage_bytes(stage, psi, n), rel=1e-15)


@pytest.mark.parametrize("args", [
    (0, 4, 0), (-5, 4, 0), (10, 0, 0), (10, 4, 4), (10, 4, -1)])
def test_geometry_rejects(args):
    with pytest.raises(zero.ZeroError) as e:
        zero.shard_geometry(*args)
    assert e.value.code == zero.ZERO_EINVAL


def test_state_bytes_rejects():
    with pytest.raises(zero.ZeroError):
        zero.state_bytes(4, 1e9, 8)
    with pytest.raises(zero.ZeroError):
        zero.state_bytes(2, 1e9, 0)
    out = ctypes.c_int64(-1)
    assert zero.lib().zero_shard_state_bytes(None, ctypes.byref(out)) == zero.ZERO_EINVAL
    assert out.value == -1


def _init(*a):
    h = ctypes.c_void_p()
    rc = zero.lib().zero_shard_init(*a, ctypes.byref(h))
    return rc, h


@pytest.mark.parametrize("args", [
    (0, 4, 0, 1e-3, 0.9, 0.999, 1e-8),          # numel
    (100, 4, 4, 1e-3, 0.9, 0.999, 1e-8),        # rank
    (100, 300, 0, 1e-3, 0.9, 0.999, 1e-8),      # world above the maximum
    (100, 4, 0, 1e-3, 1.0, 0.999, 1e-8),        # beta1
    (100, 4, 0, 1e-3, 0.9, 0.0, 1e-8),          # beta2
    (100, 4, 0, 1e-3, 0.9, 0.999, -1.0),        # eps
    (100, 4, 0, float("nan"), 0.9, 0.999, 1e-8),  # lr
])
def test_init_rejects_before_touching_a_device(args):
    rc, h = _init(*args)
    assert rc == zero.ZERO_EINVAL and not h.value
    assert zero.lib().zero_last_error()


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-device path")
def test_init_without_device_reports_hip_error():
    rc, h = _init(100, 4, 0, 1e-3, 0.9, 0.999, 1e-8)
    assert rc == zero.ZERO_EHIP and not h.value
    assert b"hip" in zero.lib().zero_last_error().lower()


def test_null_context_calls_are_rejected():
    L = zero.lib()
    assert L.zero_step(None, None, 4, 1, 0, None, 1, 0, 1, None) == zero.ZERO_EINVAL
    assert L.zero_load_master(None, None, 0, 0, None) == zero.ZERO_EINVAL
    assert L.zero_flatten(None, None, None, 1, 0, None, None) == zero.ZERO_EINVAL
    assert L.zero_get_state(None, None, None, None, None) == zero.ZERO_EINVAL
    assert L.zero_set_lr(None, 1e-3) == zero.ZERO_EINVAL
    assert L.zero_schedule_init(None, 1, None) == zero.ZERO_EINVAL
    assert L.zero_schedule_lr(None, 1e-3, None) == zero.ZERO_EINVAL
    assert L.zero_schedule_get(None, None, None) == zero.ZERO_EINVAL
    assert L.zero_step_begin(None, None) == zero.ZERO_EINVAL
    assert L.zero_step_sched(None, None, 4, 1, 0, None, 1, 0, None) == zero.ZERO_EINVAL
    assert L.zero_step_range_sched(None, 0, 1, None, 4, 1, 0, None, 1, 0, None) == zero.ZERO_EINVAL
    assert L.zero_fsdp_step_sched(None, None, 4, 1, None, 1, None) == zero.ZERO_EINVAL
    L.zero_destroy(None)


def test_dim0_split_matches_oracle():
    for d0 in (0, 1, 5, 10, 255, 256, 32000):
        for world in (1, 2, 3, 4, 8, 16):
            for rank in range(world):
                assert zero.dim0_split(d0, world, rank) == oracle.dim0_split(d0, world, rank)
    with pytest.raises(zero.ZeroError):
        zero.dim0_split(-1, 2, 0)
