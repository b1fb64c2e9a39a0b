"""Per-parameter (FSDP2-style, dim-0) layout on the GPU against the CPU
oracle: each parameter split by rows across ranks, the fused update run
over the list of local row shards."""
import numpy as np
import pytest
import torch

import oracle
import synth
import zero_partitioned_optimizer_flatten_amd as zero
from gpu_harness import assert_bitexact_state, assert_state_parity, bits, log

pytestmark = pytest.mark.gpu

RAGGED = [(10, 7), (5,), (1, 3), (13, 2, 2), (3, 4), (256, 64), (256,), (4099,), (2, 1000),
          (37, 129), (8, 8)]


@pytest.fixture(autouse=True)
def _gpu():
    assert torch.cuda.is_available()
    zero.lib()
    torch.cuda.empty_cache()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _run(shapes, world, rank, gdt, odt, steps, std=1e-3, seed=0):
    dev = torch.device("cuda")
    st = zero.FsdpShardState(shapes, world, rank, 1e-3)
    orc = oracle.FsdpShardOracle(shapes, world, rank, 1e-3)
    assert [st.local_numel(k) for k in range(len(shapes))] == orc.local_numels()
    params = [synth.gaussian(int(np.prod(s)), synth.PARAM_STD, seed + k).reshape(s)
              for k, s in enumerate(shapes)]
    st.load_master([p.to(dev) for p in params])
    orc.load_master([p.numpy() for p in params])
    outs = [torch.full((max(1, st.local_numel(k)),), -1, dtype=torch.int16 if odt == torch.bfloat16
                       else torch.int32, device=dev).view(odt) for k in range(len(shapes))]
    outs_h = [np.zeros(n, np.uint16 if odt == torch.bfloat16 else np.float32)
              for n in orc.local_numels()]
    for t in range(1, steps + 1):
        grads = [[synth.gaussian(int(np.prod(s)), std, synth.grad_seed(t, q) * 1000 + k, gdt,
                                 dev).reshape(s) for k, s in enumerate(shapes)]
                 for q in range(world)]
        st.step(grads, t, outs)
        orc.step([[bits(g) for g in gl] for gl in grads], t, outs_h)
    torch.cuda.synchronize()
    state = st.get_state()
    pieces = st.state_pieces(state)
    got = [np.concatenate([bits(x) for x in pl] or [np.zeros(0, np.float32)]) for pl in pieces]
    ref = orc.state()
    out_got = np.concatenate([bits(o)[:n] for o, n in zip(outs, orc.local_numels())])
    out_ref = np.concatenate(outs_h)
    label = f"fsdp N={world} r{rank} {gdt}->{odt}"
    assert_state_parity(label, got, ref, out_got, out_ref)
    assert_bitexact_state(label, got, ref, out_got, out_ref)
    st.close()


@pytest.mark.parametrize("world", [2, 4])
@pytest.mark.parametrize("gdt", [torch.bfloat16, torch.float32])
def test_ragged_list_every_rank(world, gdt):
    for rank in range(world):
        _run(RAGGED, world, rank, gdt, torch.bfloat16, 4)


@pytest.mark.parametrize("world", [3, 5, 7, 16])
def test_ragged_list_other_worlds(world):
    """Runtime replica count (not 1/2/4/8); ranks with no rows of some
    parameters."""
    for rank in (0, world - 1):
        _run(RAGGED, world, rank, torch.bfloat16, torch.float32, 3)


def test_gpt2_small_rank3():
    shapes = synth.gpt2_small_shapes()
    _run(shapes, 8, 3, torch.bfloat16, torch.bfloat16, 3)


def test_fsdp_flat_calls_rejected_and_geometry():
    st = zero.FsdpShardState([(10, 3), (5,)], 4, 3, 1e-3)
    assert [st.local[k][:2] for k in range(2)] == [oracle.dim0_split(10, 4, 3),
                                                   oracle.dim0_split(5, 4, 3)]
    n = st.shard                     # the concatenated local state, in whole lines
    assert n == 32
    with pytest.raises(zero.ZeroError) as e:
        zero.ShardState.step(st, [torch.zeros(n, device="cuda")] * 4, 1,
                             torch.zeros(n, device="cuda"))
    assert e.value.code == zero.ZERO_EINVAL
    st.close()


def test_llama7b_list_full_size_subset():
    """Llama-7B-shaped list (291 parameters), N = 8, rank 5: the full list is
    stepped on the GPU; the oracle checks the embedding, a layer's seven
    matrices and two norms, the final norm and the LM head."""
    shapes = synth.llama_shapes(32, 4096, 11008)
    world, rank = 8, 5
    dev = torch.device("cuda")
    st = zero.FsdpShardState(shapes, world, rank, 1e-3)
    check = [0, 1, 2, 3, 4, 5, 6, 7, 8, 9, len(shapes) - 2, len(shapes) - 1]
    sub = [shapes[k] for k in check]
    orc = oracle.FsdpShardOracle(sub, world, rank, 1e-3)
    # full-size buffers; only this rank's rows are ever read, so only those
    # rows are filled (the rest stays as allocated)
    params = [torch.empty(s, dtype=torch.bfloat16, device=dev) for s in shapes]
    for k, p in enumerate(params):
        f, r, _ = st.local[k]
        synth.fill_gaussian(p.view(p.shape[0], -1)[f:f + r], synth.PARAM_STD, k)
    st.load_master(params)
    orc.load_master([bits(params[k]).reshape(-1) for k in check])
    del params
    grads = [[torch.empty(s, dtype=torch.bfloat16, device=dev) for s in shapes]
             for _ in range(world)]
    outs = [torch.empty(st.local_numel(k), dtype=torch.bfloat16, device=dev)
            for k in range(len(shapes))]
    outs_h = [np.zeros(n, np.uint16) for n in orc.local_numels()]
    for t in range(1, 4):
        for q in range(world):
            for k, g in enumerate(grads[q]):
                f, r, _ = st.local[k]
                synth.fill_gaussian(g.view(g.shape[0], -1)[f:f + r], 1e-3,
                                    synth.grad_seed(t, q) * 1000 + k)
        st.step(grads, t, outs)
        sub_grads = [[bits(grads[q][k]).reshape(-1) for k in check] for q in range(world)]
        orc.step(sub_grads, t, outs_h)
        log(f"fsdp llama7b: step {t} done")
    torch.cuda.synchronize()
    pieces = st.state_pieces(st.get_state())
    got = [np.concatenate([bits(pl[k]) for k in check]) for pl in pieces]
    out_got = np.concatenate([bits(outs[k]) for k in check])
    label = "fsdp llama7b subset"
    assert_state_parity(label, got, orc.state(), out_got, np.concatenate(outs_h))
    assert_bitexact_state(label, got, orc.state(), out_got, np.concatenate(outs_h))
    st.close()


def test_zero_row_parameters():
    """Parameters with no rows at all ((0,), (0, 5)) next to ordinary ones:
    no rank holds any of them, and the rest steps as usual."""
    shapes = [(0,), (9, 4), (0, 5), (3,), (130, 2)]
    for rank in range(4):
        _run(shapes, 4, rank, torch.bfloat16, torch.bfloat16, 2)


def _random_shapes(rng):
    shapes = []
    for _ in range(int(rng.choice([1, 5, 33, 70]))):
        kind = rng.random()
        if kind < 0.1:
            shapes.append((0,) if rng.random() < 0.5 else (0, int(rng.integers(1, 9))))
        elif kind < 0.5:
            shapes.append((int(rng.integers(1, 5000)),))
        elif kind < 0.9:
            shapes.append((int(rng.integers(1, 300)), int(rng.integers(1, 300))))
        else:
            shapes.append((int(rng.integers(1, 40)), int(rng.integers(1, 9)), int(rng.integers(1, 70))))
    return shapes


@pytest.mark.parametrize("case", range(16))
def test_random_parameter_lists(case):
    """Seeded random parameter lists (zero-row, 1-D, 2-D and 3-D shapes; up
    to 70 parameters, so several launches of 32 or 16), world and rank
    (ranks that hold no rows of some parameters), both dtypes: 3 steps,
    bit-exact against the per-parameter oracle."""
    rng = np.random.default_rng(50_000 + case)
    world = int(rng.choice([1, 2, 3, 4, 5, 7, 8, 9, 13, 16]))
    rank = int(rng.integers(0, world))
    gdt = torch.bfloat16 if rng.random() < 0.7 else torch.float32
    odt = torch.bfloat16 if rng.random() < 0.7 else torch.float32
    shapes = _random_shapes(rng)
    log(f"fsdp case {case}: {len(shapes)} parameters, N={world} r{rank} {gdt}->{odt}")
    _run(shapes, world, rank, gdt, odt, 3, seed=case)
