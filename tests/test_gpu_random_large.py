"""Seeded random large shards of the fused step against the oracle.

The other random sweeps stop at a few hundred thousand elements. Here the
shard runs from about twenty thousand to several million elements, and the
workgroup cap is drawn from {uncapped, 1, 2, 4}, so a capped launch makes
each workgroup stride over thousands of blocks. Replica and output views
sit at independent element offsets; the buffers hold either this rank's
slice or the full flat vector. Two steps; master/m/v and the output slice
equal the oracle bit for bit."""
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
    torch.cuda.empty_cache()


@pytest.mark.parametrize("case", range(12))
def test_random_large_shard(case):
    rng = np.random.default_rng(70_000 + case)
    dev = torch.device("cuda")
    world = int(rng.choice([2, 4, 8, 16, 64]))
    rank = int(rng.integers(0, world))
    numel = int(rng.integers(1_000_000, 20_000_000))
    gdt = torch.bfloat16 if rng.random() < 0.7 else torch.float32
    odt = torch.bfloat16 if rng.random() < 0.7 else torch.float32
    full = bool(rng.random() < 0.3)
    cap = int(rng.choice([0, 0, 1, 2, 4]))
    st = zero.ShardState(numel, world, rank, 1e-3)
    st.set_step_workgroups(cap)
    orc = oracle.ShardOracle(numel, world, rank, 1e-3)
    S, lo, P = st.shard, st.lo, st.padded
    valid = max(0, min(S, numel - lo))
    L, off = (P, lo) if full else (S, 0)
    label = (f"case {case}: N={world} r={rank} S={S} {gdt} -> {odt} "
             f"{'full' if full else 'slice'} cap={cap}")

    p = torch.zeros(S, dtype=torch.float32, device=dev)
    p[:valid] = synth.gaussian(valid, synth.PARAM_STD, synth.PARAM_SEED + case,
                               torch.float32, dev)
    st.load_master(p, flat_offset=0)
    orc.master[:] = bits(p)
    rep_offs = [int(rng.integers(0, 64)) for _ in range(world)]
    reps = []
    for q in range(world):
        buf = torch.zeros(L + 64, dtype=gdt, device=dev)
        reps.append(buf[rep_offs[q]:rep_offs[q] + L])
    out_off = int(rng.integers(0, 64))
    out = torch.zeros(L + 64, dtype=odt, device=dev)[out_off:out_off + L]
    ref = bits(out).copy()
    log(f"{label} output offset {out_off}")
    for t in (1, 2):
        for q, r in enumerate(reps):
            synth.fill_gaussian(r[off:off + valid], 1e-3, synth.grad_seed(t, q + 100 * case))
        st.step(reps, t, out, grad_offset=off, param_offset=off)
        orc.step([bits(r) for r in reps], t, ref, grad_offset=off, out_offset=off)
        torch.cuda.synchronize()
        assert_bitexact_state(f"{label} t={t}", gpu_state(st), [orc.master, orc.m, orc.v],
                              bits(out)[off:off + S], ref[off:off + S])
    st.close()
