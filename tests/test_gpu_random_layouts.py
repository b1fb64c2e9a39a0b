"""Seeded random layouts of the fused step against the oracle.

Each case draws the replica count, rank, shard size (ragged, pad included),
gradient and output dtypes, full flat or slice-only buffers, and for every
replica and for the output an independent element offset within 64 of a
freshly allocated buffer. That mixes the vector, shifted and element paths,
every compiled replica count and the runtime-count kernel, heads and tails,
in combinations the enumerated tests do not reach. Two steps at a random
step count; master/m/v and the output equal the oracle bit for bit, and
the output buffer's elements outside this rank's slice keep their sentinel
bits (nothing outside the slice is written)."""
import numpy as np
import pytest
import torch

import oracle
import synth
import zero_partitioned_optimizer_flatten_amd as zero
from gpu_harness import assert_bitexact_state, bits, gpu_state, log

pytestmark = pytest.mark.gpu

WORLDS = (1, 2, 3, 4, 5, 7, 8, 9, 16, 17, 32, 64, 100)


@pytest.fixture(autouse=True)
def _gpu():
    assert torch.cuda.is_available()
    zero.lib()
    yield
    torch.cuda.synchronize()


def _sentinel(n, dtype, dev):
    """n elements of a recognisable NaN pattern (bf16 0x7FC1, fp32 0x7FC00001)."""
    if dtype == torch.bfloat16:
        return torch.full((n,), 0x7FC1, dtype=torch.int16, device=dev).view(dtype)
    return torch.full((n,), 0x7FC00001, dtype=torch.int32, device=dev).view(dtype)


@pytest.mark.parametrize("case", range(48))
def test_random_layout(case):
    rng = np.random.default_rng(20_000 + case)
    dev = torch.device("cuda")
    world = int(rng.choice(WORLDS))
    rank = int(rng.integers(0, world))
    numel = int(rng.integers(1, 120_000))
    gdt = torch.bfloat16 if rng.random() < 0.7 else torch.float32
    odt = torch.bfloat16 if rng.random() < 0.7 else torch.float32
    full = bool(rng.random() < 0.5)
    t0 = int(rng.integers(1, 2000))
    lr = float(rng.choice([1e-3, 3e-4, 1e-2]))
    st = zero.ShardState(numel, world, rank, lr)
    orc = oracle.ShardOracle(numel, world, rank, lr)
    S, lo, P = st.shard, st.lo, st.padded
    valid = max(0, min(S, numel - lo))
    L, off = (P, lo) if full else (S, 0)
    label = (f"case {case}: N={world} r={rank} numel={numel} {gdt} -> {odt} "
             f"{'full' if full else 'slice'} t0={t0}")

    p = torch.zeros(S, dtype=torch.float32, device=dev)
    p[:valid] = synth.gaussian(valid, synth.PARAM_STD, synth.PARAM_SEED + case,
                               torch.float32, dev)
    st.load_master(p, flat_offset=0)
    orc.master[:] = bits(p)

    # replica q: a view at a random element offset into its own buffer;
    # only this rank's valid elements are non-zero (the pad stays zero)
    rep_offs = [int(rng.integers(0, 64)) for _ in range(world)]
    reps = []
    for q in range(world):
        buf = torch.zeros(L + 64, dtype=gdt, device=dev)
        reps.append(buf[rep_offs[q]:rep_offs[q] + L])
    out_off = int(rng.integers(0, 64))
    out_buf = _sentinel(L + 128, odt, dev)
    out = out_buf[out_off:out_off + L]
    want = bits(out_buf)
    log(f"{label} replica offsets {rep_offs[:8]} output offset {out_off}")

    for t in (t0, t0 + 1):
        for q, r in enumerate(reps):
            synth.fill_gaussian(r[off:off + valid], 1e-3, synth.grad_seed(t, q + 100 * case))
        st.step(reps, t, out, grad_offset=off, param_offset=off)
        ref = want[out_off:out_off + L].copy()
        orc.step([bits(r) for r in reps], t, ref, grad_offset=off, out_offset=off)
        want[out_off:out_off + L] = ref
        torch.cuda.synchronize()
        got = bits(out_buf)
        assert_bitexact_state(f"{label} t={t}", gpu_state(st), [orc.master, orc.m, orc.v],
                              got[out_off + off:out_off + off + S],
                              want[out_off + off:out_off + off + S])
        outside = np.ones(got.size, dtype=bool)
        outside[out_off + off:out_off + off + S] = False
        assert got[outside].tobytes() == want[outside].tobytes(), f"{label}: write outside the slice"
    st.close()
