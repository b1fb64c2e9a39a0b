"""The step schedule that allocates nothing (zero_schedule_init_noalloc),
called through the C ABI, against the allocating zero_schedule_init on a
twin context: two initialisations in a row on the device's one static block,
the second on a smaller shard with other betas, each followed by scheduled
steps whose master/m/v and bf16 output must equal the allocating
schedule's bit for bit, and the oracle's."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import synth
import zero_partitioned_optimizer_flatten_amd as zero
from gpu_harness import assert_bitexact_state, bits, gpu_state, log

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    assert torch.cuda.is_available()
    zero.lib()
    yield
    torch.cuda.synchronize()


def _noalloc_init(st, next_t):
    """The entry point under test, called through the C ABI."""
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return zero.lib().zero_schedule_init_noalloc(st._h, int(next_t), stream)


class Twin:
    """Two contexts with the same geometry, hyperparameters and master: `a`
    takes the allocating schedule, `b` the static one; plus the oracle."""

    def __init__(self, numel, world, rank, lr, betas, eps=1e-8):
        self.a = zero.ShardState(numel, world, rank, lr, betas, eps)
        self.b = zero.ShardState(numel, world, rank, lr, betas, eps)
        self.orc = oracle.ShardOracle(numel, world, rank, lr, betas, eps)
        S = self.a.shard
        self.valid = max(0, min(S, numel - self.a.lo))
        p = torch.zeros(S, dtype=torch.float32, device="cuda")
        p[:self.valid] = synth.gaussian(self.valid, synth.PARAM_STD, synth.PARAM_SEED,
                                        torch.float32, "cuda")
        self.a.load_master(p, flat_offset=0)
        self.b.load_master(p, flat_offset=0)
        self.orc.master[:] = bits(p)
        self.reps = [torch.zeros(S, dtype=torch.bfloat16, device="cuda") for _ in range(world)]
        self.out_a = torch.zeros(S, dtype=torch.bfloat16, device="cuda")
        self.out_b = torch.full((S,), -1.0, dtype=torch.bfloat16, device="cuda")

    def fill(self, t):
        for q, r in enumerate(self.reps):
            synth.fill_gaussian(r[:self.valid], 1e-3, synth.grad_seed(t, q))

    def check(self, label, t):
        torch.cuda.synchronize()
        out_ref = np.zeros(self.a.shard, np.uint16)
        self.orc.step([bits(r) for r in self.reps], t, out_ref, grad_offset=0, out_offset=0)
        sa, sb = gpu_state(self.a), gpu_state(self.b)
        assert_bitexact_state(f"{label} t={t} static vs allocating", sb, sa,
                              bits(self.out_b), bits(self.out_a))
        assert_bitexact_state(f"{label} t={t} static vs oracle", sb,
                              [self.orc.master, self.orc.m, self.orc.v], bits(self.out_b), out_ref)
        log(f"{label} t={t}: static schedule == allocating schedule == oracle")

    def close(self):
        self.a.close()
        self.b.close()


def _steps(tw, t0, count, label):
    for t in range(t0, t0 + count):
        tw.fill(t)
        tw.a.step_sched(tw.reps, tw.out_a)
        tw.b.step_sched(tw.reps, tw.out_b)
        tw.check(label, t)


def _range_step(tw, t, label):
    """One step as a begin plus two scheduled ranges on each context."""
    tw.fill(t)
    S = tw.a.shard
    cut = S // 3
    for st, out in ((tw.a, tw.out_a), (tw.b, tw.out_b)):
        st.step_begin()
        st.step_range_sched(0, cut, [r[:cut] for r in tw.reps], out[:cut], grad_offset=0,
                            param_offset=0)
        st.step_range_sched(cut, S - cut, [r[cut:] for r in tw.reps], out[cut:],
                            grad_offset=0, param_offset=0)
    tw.check(label, t)


def test_noalloc_schedule_equals_allocating_schedule_twice():
    # first call: 100,003 elements, N = 4, rank 1, resuming at t = 5
    tw1 = Twin(100_003, 4, 1, 1e-3, (0.9, 0.999))
    tw1.a.schedule(5)
    assert _noalloc_init(tw1.b, 5) == zero.ZERO_OK, zero.lib().zero_last_error()
    _steps(tw1, 5, 3, "first")
    _range_step(tw1, 8, "first, ranges")
    assert tw1.b.schedule_next_t() == tw1.a.schedule_next_t() == 9

    # second call, smaller: 10,001 elements, N = 2, rank 1 (one pad element),
    # other betas and lr; the static block still holds the first call's table
    tw2 = Twin(10_001, 2, 1, 3e-4, (0.8, 0.99))
    tw2.a.schedule(1)
    assert _noalloc_init(tw2.b, 1) == zero.ZERO_OK, zero.lib().zero_last_error()
    with pytest.raises(zero.ZeroError) as ei:           # no step has begun yet
        tw2.b.step_range_sched(0, tw2.b.shard, tw2.reps, tw2.out_b, grad_offset=0,
                               param_offset=0)
    assert ei.value.code == zero.ZERO_EINVAL
    _steps(tw2, 1, 3, "second")
    _range_step(tw2, 4, "second, ranges")

    # the first static schedule was taken over by the second context
    with pytest.raises(zero.ZeroError) as ei:
        tw1.b.step_sched(tw1.reps, tw1.out_b)
    assert ei.value.code == zero.ZERO_EINVAL and "taken over" in str(ei.value)
    # ... and it continues on its own allocation where it left off
    tw1.b.schedule(9)
    _steps(tw1, 9, 1, "first, reallocated")
    tw1.close()
    tw2.close()


def test_noalloc_schedule_rejects_a_table_beyond_its_block():
    """b2 = 0.99999 needs a table of about 1.8M steps, more than the static
    block's 262,080: refused before any device work; the allocating call
    serves it."""
    st = zero.ShardState(1000, 1, 0, 1e-3, (0.9, 0.99999), 1e-8)
    rc = _noalloc_init(st, 1)
    assert rc == zero.ZERO_EUNSUPPORTED
    msg = zero.lib().zero_last_error().decode()
    assert "262080" in msg, msg
    with pytest.raises(zero.ZeroError):
        st.step_begin()                                 # still no schedule
    st.schedule(1)
    st.close()
