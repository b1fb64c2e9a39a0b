"""Seeded random bucketings of the step (zero_step_range) against one whole
step and the oracle.

Each case draws the replica count, rank, a ragged shard, both dtypes, the
number of buckets and their boundaries (anywhere, one-element buckets
included), one to three streams and a workgroup cap. Two steps; after each,
the bucketed context's master/m/v and output equal the whole-step
context's bit for bit, and both equal the oracle."""
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


@pytest.mark.parametrize("case", range(24))
def test_random_buckets(case):
    rng = np.random.default_rng(40_000 + case)
    dev = torch.device("cuda")
    world = int(rng.choice([1, 2, 3, 4, 7, 8, 16, 64]))
    rank = int(rng.integers(0, world))
    numel = int(rng.integers(world, 400_000))
    gdt = torch.bfloat16 if rng.random() < 0.7 else torch.float32
    odt = torch.bfloat16 if rng.random() < 0.7 else torch.float32
    cap = int(rng.choice([0, 0, 1, 2, 4]))
    nstreams = int(rng.integers(1, 4))
    whole = zero.ShardState(numel, world, rank, 1e-3)
    buck = zero.ShardState(numel, world, rank, 1e-3)
    buck.set_step_workgroups(cap)
    orc = oracle.ShardOracle(numel, world, rank, 1e-3)
    S, lo = whole.shard, whole.lo
    valid = max(0, min(S, numel - lo))
    cuts = sorted(set(int(c) for c in rng.integers(0, S + 1, size=int(rng.integers(0, 40)))))
    if rng.random() < 0.3 and S > 2:
        cuts += [1, 2]                          # one-element buckets at the start
    bounds = sorted(set([0, S] + [c for c in cuts if 0 < c < S]))
    log(f"case {case}: N={world} r={rank} S={S} {gdt}->{odt} cap={cap} "
        f"{len(bounds) - 1} buckets on {nstreams} streams")

    p = torch.zeros(S, dtype=torch.float32, device=dev)
    p[:valid] = synth.gaussian(valid, synth.PARAM_STD, synth.PARAM_SEED + case, torch.float32, dev)
    for st in (whole, buck):
        st.load_master(p, flat_offset=0)
    orc.master[:] = bits(p)
    reps = [torch.zeros(S, dtype=gdt, device=dev) for _ in range(world)]
    out_w = torch.zeros(S, dtype=odt, device=dev)
    out_b = torch.zeros(S, dtype=odt, device=dev)
    out_ref = bits(out_w)
    streams = [torch.cuda.Stream() for _ in range(nstreams)]
    cur = torch.cuda.current_stream()
    for t in (1, 2):
        for q, r in enumerate(reps):
            synth.fill_gaussian(r[:valid], 1e-3, synth.grad_seed(t, q + 1000 * case))
        whole.step(reps, t, out_w)
        for s in streams:
            s.wait_stream(cur)
        for i, (a, b) in enumerate(zip(bounds[:-1], bounds[1:])):
            buck.step_range(a, b - a, [r[a:] for r in reps], t, out_b, grad_offset=0,
                            param_offset=a, stream=streams[i % nstreams])
        for s in streams:
            cur.wait_stream(s)
        orc.step([bits(r) for r in reps], t, out_ref, grad_offset=0, out_offset=0)
        torch.cuda.synchronize()
        sw, sb = gpu_state(whole), gpu_state(buck)
        for x, y in zip(sw, sb):
            assert x.tobytes() == y.tobytes(), f"case {case} t={t}: bucketed state differs"
        assert bits(out_w).tobytes() == bits(out_b).tobytes(), f"case {case} t={t}: output"
        assert_bitexact_state(f"case {case} t={t}", sw, [orc.master, orc.m, orc.v],
                              bits(out_w), out_ref)
    whole.close()
    buck.close()
