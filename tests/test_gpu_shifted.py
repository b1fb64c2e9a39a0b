"""Buffers at mixed 16-byte phases: the shifted vector path, and launches
whose blocks straddle 128-byte lines.

The state's phase is fixed by the library (lo mod 32 elements past a 1 MiB
boundary); replicas and output here sit at every element phase relative to
it, each replica at its own phase. Every combination must give the oracle's
values bit for bit, and the output must touch exactly its own elements
(sentinels before and after the output view stay intact)."""
import numpy as np
import pytest
import torch

import oracle
import synth
import zero_partitioned_optimizer_flatten_amd as zero
from gpu_harness import assert_bitexact_state, assert_state_parity, bits, gpu_state, log

pytestmark = pytest.mark.gpu
LR, BETAS, EPS = 1e-3, (0.9, 0.999), 1e-8
SENTINEL = -1                      # 0xFFFF in bf16 bits, NaN pattern 0xFFFFFFFF in fp32


@pytest.fixture(autouse=True)
def _gpu():
    assert torch.cuda.is_available()
    zero.lib()
    yield
    torch.cuda.synchronize()


def _run_phases(world, rank, S, gdt, odt, combos, label):
    """One shard state; step t uses the t-th (replica offsets, output offset)
    combination, each replica a view at that element offset into a fresh
    allocation."""
    dev = torch.device("cuda")
    numel = world * S - (1 if world > 1 else 0)
    st = zero.ShardState(numel, world, rank, LR, BETAS, EPS)
    assert st.shard == S
    orc = oracle.ShardOracle(numel, world, rank, LR, BETAS, EPS)
    valid = max(0, min(S, numel - st.lo))
    p = torch.zeros(S, dtype=torch.float32, device=dev)
    p[:valid] = synth.gaussian(valid, synth.PARAM_STD, synth.PARAM_SEED + rank, torch.float32, dev)
    st.load_master(p, flat_offset=0)
    orc.master[:] = bits(p)
    ivt = torch.int16 if odt == torch.bfloat16 else torch.int32
    for t, (roffs, ooff) in enumerate(combos, start=1):
        reps, reps_h = [], []
        for q in range(world):
            buf = torch.zeros(S + 64, dtype=gdt, device=dev)
            g = buf[roffs[q]:roffs[q] + S]
            g[:valid] = synth.gaussian(valid, 1e-3, synth.grad_seed(t, q), gdt, dev)
            reps.append(g)
            reps_h.append(bits(g))
        obuf = torch.full((S + 64,), SENTINEL, dtype=ivt, device=dev).view(odt)
        out = obuf[ooff:ooff + S]
        st.step(reps, t, out)
        out_ref = np.zeros(S, np.uint16 if odt == torch.bfloat16 else np.float32)
        orc.step(reps_h, t, out_ref, grad_offset=0, out_offset=0)
        torch.cuda.synchronize()
        whole = obuf.view(ivt).cpu().numpy()
        assert np.all(whole[:ooff] == SENTINEL) and np.all(whole[ooff + S:] == SENTINEL), \
            f"{label} t={t}: output store left its view (offset {ooff})"
        got = bits(out)
        tag = f"{label} t={t} reps@{list(roffs)} out@{ooff}"
        assert_bitexact_state(tag, gpu_state(st), [orc.master, orc.m, orc.v], got, out_ref)
    assert_state_parity(label, gpu_state(st), [orc.master, orc.m, orc.v])
    st.close()


@pytest.mark.parametrize("gdt,odt", [(torch.bfloat16, torch.bfloat16),
                                     (torch.bfloat16, torch.float32),
                                     (torch.float32, torch.bfloat16),
                                     (torch.float32, torch.float32)])
def test_every_phase_against_every_state_shift(gdt, odt):
    """N = 4, S = 5001 (= 1 mod 4, so rank r's state sits r elements past a
    16-byte boundary), ranks 0..3; for each, all 8 replica base phases
    (replica q at (base + 3q) mod 8) against all 8 output phases."""
    S, world = 5001, 4
    combos = [(tuple((rp + 3 * q) % 8 for q in range(world)), op)
              for rp in range(8) for op in range(8)]
    for rank in range(world):
        _run_phases(world, rank, S, gdt, odt, combos, f"phases N=4 r{rank} {gdt}->{odt}")


@pytest.mark.parametrize("world", [1, 2, 3, 8, 16, 64])
def test_phases_every_compiled_replica_count(world):
    """Each compiled replica count (and the runtime-N kernel at N = 3) on
    the shifted path: bf16 replicas at mixed phases, bf16 output."""
    S = 4097
    rng = np.random.default_rng(world)
    combos = [(tuple(int(x) for x in rng.integers(0, 8, world)), int(rng.integers(0, 8)))
              for _ in range(6)]
    combos.append((tuple([1] * world), 0))
    combos.append((tuple([0] * world), 7))
    rank = world - 1
    _run_phases(world, rank, S, torch.bfloat16, torch.bfloat16, combos,
                f"phases N={world} r{rank}")


def test_shifted_path_short_shards():
    """Shards of 8..40 elements: head, at most a few vectors, tail."""
    for S in (8, 9, 15, 16, 17, 23, 40):
        combos = [((1, 2), 3), ((0, 5), 0), ((7, 7), 6)]
        _run_phases(2, 1, S, torch.bfloat16, torch.bfloat16, combos, f"short S={S}")
        log(f"short shard S={S} ok")


def test_line_straddling_blocks_large_shard():
    """Launches whose streams straddle 128-byte lines, on a shard of 200,003
    elements (390 full wavefront blocks in the split lane layout, a partial
    block and the head/tail workgroup):
      - rank 0, every buffer 16-byte aligned but off its line by 8, 24, 40
        or 56 elements (the vector path's 16-byte tier);
      - ranks 1 and 3, replicas and output at mixed 16-byte phases (the
        shifted path)."""
    S, world = 200_003, 4
    _run_phases(world, 0, S, torch.bfloat16, torch.bfloat16,
                [((8, 24, 40, 56), 8), ((8, 8, 8, 8), 24), ((56, 40, 24, 8), 40)],
                "16-byte tier")
    for rank in (1, 3):
        _run_phases(world, rank, S, torch.bfloat16, torch.bfloat16,
                    [((1, 2, 3, 4), 5), ((0, 0, 0, 7), 3), ((7, 0, 7, 0), 0)],
                    f"shifted r{rank}")
    _run_phases(world, 1, S, torch.float32, torch.float32,
                [((1, 2, 3, 0), 1), ((0, 0, 0, 2), 3)], "shifted fp32")


def test_arbitrary_bit_patterns_through_the_shifted_path():
    """Replicas of random 16-bit patterns (every bf16 class: zeros,
    subnormals, normals, infinities, NaNs) at mixed phases, output at an odd
    phase: the realignment in registers and the narrow stores move bits, so
    the result must match the oracle on every element (NaN against NaN
    counting as equal)."""
    dev = torch.device("cuda")
    S, world, rank = 70_001, 4, 2
    numel = world * S - 1
    st = zero.ShardState(numel, world, rank, LR, BETAS, EPS)
    orc = oracle.ShardOracle(numel, world, rank, LR, BETAS, EPS)
    valid = min(S, numel - st.lo)
    p = synth.gaussian(S, synth.PARAM_STD, synth.PARAM_SEED, torch.float32, dev)
    p[valid:] = 0
    st.load_master(p, flat_offset=0)
    orc.master[:] = bits(p)
    gen = torch.Generator(device="cpu").manual_seed(77)
    for t, (roffs, ooff) in enumerate([((1, 4, 6, 3), 5), ((7, 0, 2, 5), 1)], start=1):
        reps = []
        for q in range(world):
            buf = torch.zeros(S + 64, dtype=torch.int16, device=dev)
            g = buf[roffs[q]:roffs[q] + S]
            g[:valid] = torch.randint(-32768, 32768, (valid,), generator=gen,
                                      dtype=torch.int32).to(torch.int16).to(dev)
            reps.append(g.view(torch.bfloat16))
        obuf = torch.full((S + 64,), SENTINEL, dtype=torch.int16, device=dev)
        out = obuf[ooff:ooff + S].view(torch.bfloat16)
        st.step(reps, t, out)
        out_ref = np.zeros(S, np.uint16)
        orc.step([bits(r) for r in reps], t, out_ref, grad_offset=0, out_offset=0)
        torch.cuda.synchronize()
        whole = obuf.cpu().numpy()
        assert np.all(whole[:ooff] == SENTINEL) and np.all(whole[ooff + S:] == SENTINEL)
        assert_bitexact_state(f"bit patterns t={t}", gpu_state(st), [orc.master, orc.m, orc.v],
                              bits(out), out_ref)
        log(f"arbitrary bit patterns t={t}: matches the oracle")
    st.close()
