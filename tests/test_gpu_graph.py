"""Device-resident step schedule and HIP graph replay.

The scheduled calls take t and lr from device memory, so one captured graph
of a step replays as successive steps. Every replay, and every eager
scheduled step between replays, must equal the oracle at that step bit for
bit. Replays are interleaved with the program's own eager work and
synchronisations, and lr changes between replays reach the next replay."""
import numpy as np
import pytest
import torch

import oracle
import synth
import zero_partitioned_optimizer_flatten_amd as zero
from gpu_harness import assert_bitexact_state, bits, gpu_state, log

pytestmark = pytest.mark.gpu
BETAS, EPS = (0.9, 0.999), 1e-8


@pytest.fixture(autouse=True)
def _gpu():
    assert torch.cuda.is_available()
    zero.lib()
    yield
    torch.cuda.synchronize()


def _setup(numel, world, rank, lr, gdt=torch.bfloat16, dev="cuda"):
    st = zero.ShardState(numel, world, rank, lr, BETAS, EPS)
    orc = oracle.ShardOracle(numel, world, rank, lr, BETAS, EPS)
    S = st.shard
    valid = max(0, min(S, numel - st.lo))
    p = torch.zeros(S, dtype=torch.float32, device=dev)
    p[:valid] = synth.gaussian(valid, synth.PARAM_STD, synth.PARAM_SEED, torch.float32, dev)
    st.load_master(p, flat_offset=0)
    orc.master[:] = bits(p)
    reps = [torch.zeros(S, dtype=gdt, device=dev) for _ in range(world)]
    out = torch.zeros(S, dtype=torch.bfloat16, device=dev)
    return st, orc, reps, out, valid


def _fill(reps, valid, t):
    for q, r in enumerate(reps):
        synth.fill_gaussian(r[:valid], 1e-3, synth.grad_seed(t, q))


def _check(label, st, orc, reps, out, t):
    out_ref = np.zeros(st.shard, np.uint16)
    orc.step([bits(r) for r in reps], t, out_ref, grad_offset=0, out_offset=0)
    torch.cuda.synchronize()
    assert_bitexact_state(f"{label} t={t}", gpu_state(st), [orc.master, orc.m, orc.v],
                          bits(out), out_ref)


def test_scheduled_steps_equal_host_steps():
    """Eager scheduled steps against the oracle, with a learning-rate change
    and a schedule reset (resume at a later t) on the way."""
    st, orc, reps, out, valid = _setup(100_003, 4, 3, 1e-3)
    st.schedule(1)
    for t in range(1, 13):
        if t == 6:
            st.schedule_lr(3e-4)
            orc.lr = 3e-4
        if t == 9:
            assert st.schedule_next_t() == 9
            st.schedule(40)                       # resume at step 40
        tt = t if t < 9 else 40 + (t - 9)
        _fill(reps, valid, tt)
        st.step_sched(reps, out)
        _check("sched", st, orc, reps, out, tt)
    assert st.schedule_next_t() == 44
    st.close()


def test_range_step_before_any_begin_is_refused():
    """A scheduled range step reads the scalars that a begin-step wrote; on
    a fresh schedule there are none, so the call must fail its argument
    check and leave the state and the output untouched. After a begin it
    runs and equals the oracle."""
    st, orc, reps, out, valid = _setup(10_007, 2, 0, 1e-3)
    st.schedule(1)
    _fill(reps, valid, 1)
    out.fill_(0)
    before = [x.clone() for x in st.get_state()]
    with pytest.raises(zero.ZeroError) as ei:
        st.step_range_sched(0, st.shard, reps, out, grad_offset=0, param_offset=0)
    assert ei.value.code == zero.ZERO_EINVAL
    assert "begun" in str(ei.value)
    torch.cuda.synchronize()
    after = st.get_state()
    for a, b in zip(before, after):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    assert int(out.view(torch.int16).abs().sum()) == 0
    st.step_begin()
    st.step_range_sched(0, st.shard, reps, out, grad_offset=0, param_offset=0)
    _check("range after begin", st, orc, reps, out, 1)
    st.close()


def test_scheduled_steps_past_the_bias_table():
    """Steps far past the point where both bias corrections round to 1
    (the table's end), against the oracle at those t."""
    st, orc, reps, out, valid = _setup(20_001, 2, 1, 1e-3)
    for t0 in (17_000, 17_400, 1_000_000, 2**40):
        st.schedule(t0)
        _fill(reps, valid, 7)
        st.step_sched(reps, out)
        _check("late", st, orc, reps, out, t0)
    st.close()


def test_graph_replays_successive_steps():
    """One captured scheduled step, replayed as steps 2..9 with eager
    scheduled steps and other eager work between some replays."""
    st, orc, reps, out, valid = _setup(200_003, 8, 5, 1e-3)
    st.schedule(1)
    _fill(reps, valid, 1)
    st.step_sched(reps, out)                      # eager step 1 (also loads the code)
    _check("graph warm-up", st, orc, reps, out, 1)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st.step_sched(reps, out)
    torch.cuda.synchronize()
    assert st.schedule_next_t() == 2              # capture launched nothing
    scratch = torch.empty(1 << 20, device="cuda")
    for t in range(2, 10):
        _fill(reps, valid, t)
        scratch.normal_()                         # unrelated eager work
        if t == 5:
            st.step_sched(reps, out)              # eager step between replays
        else:
            if t == 7:
                st.schedule_lr(5e-4)              # reaches the next replay
                orc.lr = 5e-4
            g.replay()
        _check("graph", st, orc, reps, out, t)
        log(f"graph replay t={t} bit-exact")
    assert st.schedule_next_t() == 10
    del g
    st.close()


def test_graph_of_bucketed_step():
    """step_begin + ragged step_range_sched buckets captured once; each
    replay is one whole step."""
    st, orc, reps, out, valid = _setup(300_007, 4, 2, 1e-3)
    S = st.shard
    bounds = [0, 1, 9, 4096, 33_333, 60_001, S]
    st.schedule(1)
    _fill(reps, valid, 1)
    st.step_begin()
    for a, b in zip(bounds[:-1], bounds[1:]):
        st.step_range_sched(a, b - a, [r[a:] for r in reps], out, param_offset=a)
    _check("buckets eager", st, orc, reps, out, 1)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st.step_begin()
        for a, b in zip(bounds[:-1], bounds[1:]):
            st.step_range_sched(a, b - a, [r[a:] for r in reps], out, param_offset=a)
    for t in range(2, 7):
        _fill(reps, valid, t)
        g.replay()
        _check("buckets graph", st, orc, reps, out, t)
    del g
    # the same buckets alternating between two branches of one graph
    side = torch.cuda.Stream()
    g2 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g2):
        cur = torch.cuda.current_stream()
        st.step_begin()
        side.wait_stream(cur)
        for i, (a, b) in enumerate(zip(bounds[:-1], bounds[1:])):
            st.step_range_sched(a, b - a, [r[a:] for r in reps], out, param_offset=a,
                                stream=(cur, side)[i % 2])
        cur.wait_stream(side)
    for t in range(7, 11):
        _fill(reps, valid, t)
        g2.replay()
        _check("buckets graph, 2 branches", st, orc, reps, out, t)
    del g2
    st.close()


def test_graph_of_the_whole_hot_path():
    """One training step's optimizer path captured as one graph: flatten of
    this rank's gradient list into its full flat buffer, the scheduled step
    over the N full flat replicas (the pages' layout) writing bf16 into the
    full flat parameter buffer at lo, and unflatten of that buffer into the
    parameter tensors. The gradient list is ragged and carved from one
    buffer at an odd element offset; rank 3 holds the pad. Each replay, with
    new gradients and eager work between replays and an lr change before
    one of them, equals the oracle's flatten, step and unflatten."""
    shapes = synth.ragged_shapes(5, 23, 30_000) + [(1,), (7, 3)]
    numel = synth.numel_of(shapes)
    world, rank = 4, 3
    dev = "cuda"
    st = zero.ShardState(numel, world, rank, 1e-3, BETAS, EPS)
    orc = oracle.ShardOracle(numel, world, rank, 1e-3, BETAS, EPS)
    S, lo, P = st.shard, st.lo, st.padded
    assert P > numel, "rank 3 should hold pad elements"
    flat_p = torch.zeros(P, dtype=torch.float32, device=dev)
    flat_p[:numel] = synth.gaussian(numel, synth.PARAM_STD, synth.PARAM_SEED, torch.float32, dev)
    st.load_master(flat_p)
    orc.load_master(bits(flat_p))
    storage = torch.zeros(numel + 1, dtype=torch.bfloat16, device=dev)
    own_list = synth.split_views(storage[1:], shapes)
    own_flat = torch.full((P,), -1, dtype=torch.int16, device=dev).view(torch.bfloat16)
    peers = {q: torch.zeros(P, dtype=torch.bfloat16, device=dev) for q in range(world) if q != rank}
    reps = [own_flat if q == rank else peers[q] for q in range(world)]
    param_flat = flat_p.to(torch.bfloat16)
    params = [torch.empty(s, dtype=torch.bfloat16, device=dev) for s in shapes]
    want_flat = bits(param_flat)

    def fill(t):
        synth.fill_gaussian(storage[1:], 1e-3, synth.grad_seed(t, rank))
        for q, b in peers.items():
            synth.fill_gaussian(b[:numel], 1e-3, synth.grad_seed(t, q))

    def path():
        st.flatten(own_list, own_flat)
        st.step_sched(reps, param_flat)
        st.unflatten(param_flat, params)

    def check(label, t):
        own_ref = oracle.flatten([bits(x) for x in own_list], P)
        orc.step([own_ref if q == rank else bits(peers[q]) for q in range(world)], t, want_flat)
        torch.cuda.synchronize()
        assert bits(own_flat).tobytes() == own_ref.tobytes(), (label, t)
        assert_bitexact_state(f"{label} t={t}", gpu_state(st), [orc.master, orc.m, orc.v],
                              bits(param_flat), want_flat)
        for a, b in zip(params, oracle.unflatten(want_flat, shapes)):
            assert bits(a).tobytes() == b.tobytes(), (label, t)

    st.schedule(1)
    fill(1)
    path()                                        # eager step 1 (also loads the code)
    check("whole path eager", 1)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        path()
    torch.cuda.synchronize()
    assert st.schedule_next_t() == 2              # capture launched nothing
    scratch = torch.empty(1 << 20, device=dev)
    for t in range(2, 8):
        fill(t)
        scratch.normal_()                         # unrelated eager work
        if t == 5:
            st.schedule_lr(5e-4)                  # reaches the next replay
            orc.lr = 5e-4
        g.replay()
        check("whole path graph", t)
        log(f"whole-path graph replay t={t} bit-exact")
    del g
    st.close()


def test_fsdp_scheduled_and_graph():
    """The per-parameter layout: scheduled steps, eager and replayed,
    against host-t steps on an identical second state."""
    shapes = [(37, 5), (64,), (3, 7, 2), (1,), (130, 8)]
    world, rank = 4, 1
    dev = torch.device("cuda")
    a = zero.FsdpShardState(shapes, world, rank, 1e-3, BETAS, EPS)
    b = zero.FsdpShardState(shapes, world, rank, 1e-3, BETAS, EPS)
    params = [synth.gaussian(int(np.prod(s)), 0.02, k, torch.float32, dev).view(s)
              for k, s in enumerate(shapes)]
    a.load_master(params)
    b.load_master(params)
    grads = [[torch.empty(s, dtype=torch.bfloat16, device=dev) for s in shapes]
             for _ in range(world)]
    outs_a = [torch.zeros(max(1, a.local_numel(k)), dtype=torch.bfloat16, device=dev)
              for k in range(len(shapes))]
    outs_b = [torch.zeros_like(o) for o in outs_a]

    def fill(t):
        for q in range(world):
            for k, g in enumerate(grads[q]):
                synth.fill_gaussian(g, 1e-3, 1000 * t + 10 * q + k)

    a.schedule(1)
    fill(1)
    a.step_sched(grads, outs_a)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        a.step_sched(grads, outs_a)
    b.step(grads, 1, outs_b)
    for t in range(2, 6):
        fill(t)
        g.replay()
        b.step(grads, t, outs_b)
        torch.cuda.synchronize()
        for x, y in zip(a.get_state(), b.get_state()):
            assert torch.equal(x.view(torch.int32), y.view(torch.int32)), f"state t={t}"
        for x, y in zip(outs_a, outs_b):
            assert torch.equal(x.view(torch.int16), y.view(torch.int16)), f"out t={t}"
    del g
    a.close()
    b.close()


def test_schedule_errors():
    st = zero.ShardState(1000, 2, 0, 1e-3)
    reps = [torch.zeros(st.shard, dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    out = torch.zeros(st.shard, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(zero.ZeroError) as e:
        st.step_sched(reps, out)                  # no schedule yet
    assert e.value.code == zero.ZERO_EINVAL
    with pytest.raises(zero.ZeroError):
        st.step_begin()
    with pytest.raises(zero.ZeroError):
        st.schedule(0)
    st.schedule(3)
    with pytest.raises(zero.ZeroError):
        st.schedule_lr(float("inf"))
    assert st.schedule_next_t() == 3
    st.close()
    with pytest.raises(zero.ZeroError) as e:
        zero.ShardState(1000, 2, 0, 1e-3, betas=(0.9, 0.99999999)).schedule(1)
    assert e.value.code == zero.ZERO_EUNSUPPORTED


def test_scheduled_steps_on_every_path():
    """The scheduled (device-scalar) instantiation of each launch path
    against the oracle: the shifted vector path (replicas and output at
    mixed 16-byte phases, grouped workgroup order), the vector path with a
    head and a tail, the element path (a shard shorter than one vector),
    and a graph replay of the shifted path."""
    dev = torch.device("cuda")
    # shifted path: rank 1 of 4, S = 200,003
    S, world, rank = 200_003, 4, 1
    numel = world * S - 1
    st = zero.ShardState(numel, world, rank, 1e-3, BETAS, EPS)
    orc = oracle.ShardOracle(numel, world, rank, 1e-3, BETAS, EPS)
    p = synth.gaussian(S, synth.PARAM_STD, synth.PARAM_SEED, torch.float32, dev)
    st.load_master(p, flat_offset=0)
    orc.master[:] = bits(p)
    bufs = [torch.zeros(S + 64, dtype=torch.bfloat16, device=dev) for _ in range(world)]
    reps = [b[1 + 2 * q:1 + 2 * q + S] for q, b in enumerate(bufs)]       # phases 1, 3, 5, 7
    obuf = torch.zeros(S + 64, dtype=torch.bfloat16, device=dev)
    out = obuf[3:3 + S]
    st.schedule(1)

    def fill(t):
        for q, r in enumerate(reps):
            synth.fill_gaussian(r, 1e-3, synth.grad_seed(t, q))

    def check(t):
        out_ref = np.zeros(S, np.uint16)
        orc.step([bits(r) for r in reps], t, out_ref, grad_offset=0, out_offset=0)
        torch.cuda.synchronize()
        assert_bitexact_state(f"shifted sched t={t}", gpu_state(st), [orc.master, orc.m, orc.v],
                              bits(out), out_ref)

    for t in (1, 2):
        fill(t)
        st.step_sched(reps, out)
        check(t)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st.step_sched(reps, out)
    for t in (3, 4):
        fill(t)
        g.replay()
        check(t)
    del g
    st.close()
    # vector path with head and tail, and the element path
    for numel, world, rank in ((100_003, 4, 3), (9, 2, 1), (3, 8, 0)):
        st, orc, reps, out, valid = _setup(numel, world, rank, 1e-3)
        st.schedule(1)
        for t in (1, 2, 3):
            _fill(reps, valid, t)
            st.step_sched(reps, out)
            _check(f"sched numel={numel}", st, orc, reps, out, t)
        st.close()
