"""HIP path against the CPU oracle through the C ABI, on shards the oracle
finishes in seconds (every element compared), plus edge cases."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import synth
import zero_partitioned_optimizer_flatten_amd as zero
from gpu_harness import (assert_bitexact_state, assert_state_parity, bits, gpu_state,
                         log, run_small_parity)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    zero.lib()          # fail loudly if the HIP library is missing
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


# ------------------------------------------------------ flat 1M, N = 4

@pytest.mark.parametrize("rank", [0, 3])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_flat1m_n4(rank, out_dtype):
    """1,000,003 fp32 parameters (one flat tensor, padded to 1,000,004),
    N = 4, fp32 gradients N(0, 0.01), 10 steps. Rank 3 holds the pad
    element and an odd offset lo = 750,003 (misaligned element path)."""
    log(f"flat1m_n4 rank={rank} out={out_dtype}")
    r = run_small_parity(1_000_003, 4, rank, torch.float32, out_dtype, 10, 0.01,
                         label=f"flat1m_n4 r{rank} {out_dtype}")
    assert_bitexact_state("flat1m", r["state"], r["ref"], r["out"], r["out_ref"])
    if rank == 3:      # pad element: all state and output exactly zero
        for a in r["state"]:
            assert a[-1] == 0 and not np.signbit(a[-1])
        assert r["out"].view(np.uint16 if r["out"].dtype == np.uint16 else np.uint32)[-1] == 0


def test_gpt2_small_n8_rank3():
    """GPT-2-small list (148 tensors, 124,439,808 elements), N = 8, rank 3,
    bf16 gradients N(0, 1e-3), bf16 parameter output, 10 steps."""
    shapes = synth.gpt2_small_shapes()
    numel = synth.numel_of(shapes)
    assert len(shapes) == 148 and numel == 124_439_808
    log("gpt2s_n8 rank 3")
    r = run_small_parity(numel, 8, 3, torch.bfloat16, torch.bfloat16, 10, 1e-3,
                         shapes=shapes, label="gpt2s_n8", check_every=5)
    assert_bitexact_state("gpt2s", r["state"], r["ref"], r["out"], r["out_ref"])


@pytest.mark.parametrize("shard", [22_369_621, 22_369_622])
def test_state_hints_on_both_sides_of_the_cache_size(shard):
    """The launcher streams master/m/v (non-temporal loads and stores) when
    the context's state, 12 B per shard element, exceeds 256 MiB, and keeps
    the default cache policy otherwise. 22,369,621 elements are 268,435,452
    bytes of state (default policy), one more element 268,435,464 (streamed):
    both equal the oracle bit for bit. N = 2, rank 1 at an odd offset (a
    head before the vector range), bf16 gradients and output, 2 steps."""
    numel = 2 * shard - 1
    log(f"state hints: shard={shard} state bytes={12 * shard}")
    r = run_small_parity(numel, 2, 1, torch.bfloat16, torch.bfloat16, 2, 1e-3,
                         label=f"state hints shard={shard}")
    assert_bitexact_state(f"shard {shard}", r["state"], r["ref"], r["out"], r["out_ref"])


# ------------------------------------------------- every replica count

@pytest.mark.parametrize("world", [1, 2, 3, 4, 5, 7, 8, 16, 32, 64, 100, 256])
@pytest.mark.parametrize("gdt", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("last_rank", [False, True])
def test_replica_counts(world, gdt, last_rank):
    """Each compile-time replica count and the runtime-count kernel, power
    of two and not; shard sizes with a ragged tail (not a multiple of 8).
    Rank 0 takes the vector path plus a tail; the last rank sits at an odd
    offset and takes the element path."""
    numel = 8 * 1237 * world + 5
    rank = world - 1 if last_rank else 0
    r = run_small_parity(numel, world, rank, gdt, torch.bfloat16, 3, 1e-3,
                         label=f"world={world} rank={rank} {gdt}")
    assert_bitexact_state(f"world {world}", r["state"], r["ref"], r["out"], r["out_ref"])


@pytest.mark.parametrize("numel,world", [(1, 1), (1, 8), (3, 8), (7, 8), (9, 8), (17, 2),
                                         (4096 * 8 + 3, 8)])
def test_degenerate_sizes(numel, world):
    """Psi < N (ranks holding only pad), Psi = 1, single-vector shards."""
    for rank in range(world):
        r = run_small_parity(numel, world, rank, torch.bfloat16, torch.bfloat16, 2, 1e-3,
                             label=f"numel={numel} N={world} r{rank}")
        assert_bitexact_state("degenerate", r["state"], r["ref"], r["out"], r["out_ref"])
        geo = oracle.geometry(numel, world, rank)
        valid = geo["valid"]
        for a in r["state"]:
            assert not np.any(a[valid:].view(np.uint32)), "pad state not zero"


def test_slice_only_buffers_and_offsets():
    """Replicas and output holding only this rank's slice (offsets 0) give
    the same result as full buffers with offset lo."""
    numel, world, rank = 200_003, 8, 5
    dev = torch.device("cuda")
    a = zero.ShardState(numel, world, rank, 1e-3)
    b = zero.ShardState(numel, world, rank, 1e-3)
    S, lo, P = a.shard, a.lo, a.padded
    flat_p = torch.zeros(P, device=dev)
    flat_p[:numel] = synth.params(numel, device=dev)
    a.load_master(flat_p)
    b.load_master(flat_p[lo:lo + S].clone(), flat_offset=0)
    out_a = torch.zeros(P, dtype=torch.bfloat16, device=dev)
    out_b = torch.zeros(S, dtype=torch.bfloat16, device=dev)
    for t in range(1, 4):
        full = []
        for q in range(world):
            f = torch.zeros(P, dtype=torch.bfloat16, device=dev)
            f[:numel] = synth.gaussian(numel, 1e-3, synth.grad_seed(t, q), torch.bfloat16, dev)
            full.append(f)
        a.step(full, t, out_a)
        b.step([f[lo:lo + S].clone() for f in full], t, out_b)
    sa, sb = gpu_state(a), gpu_state(b)
    for x, y in zip(sa, sb):
        assert x.tobytes() == y.tobytes()
    assert torch.equal(out_a[lo:lo + S].view(torch.int16), out_b.view(torch.int16))
    a.close()
    b.close()


def test_misaligned_bf16_offsets():
    """Odd element offsets into bf16 buffers (2-byte aligned only) take the
    element path and still match the oracle bit for bit."""
    numel, world, rank = 100_001, 4, 1
    dev = torch.device("cuda")
    st = zero.ShardState(numel, world, rank, 1e-3)
    orc = oracle.ShardOracle(numel, world, rank, 1e-3)
    S, P = st.shard, st.padded
    p = synth.params(S)
    st.load_master(p.to(dev), flat_offset=0)
    orc.master[:] = p.numpy()
    base = [torch.zeros(S + 3, dtype=torch.bfloat16, device=dev) for _ in range(world)]
    out = torch.zeros(S + 5, dtype=torch.bfloat16, device=dev)
    out_ref = np.zeros(S + 5, np.uint16)
    for t in range(1, 4):
        for q in range(world):
            base[q][3:] = synth.gaussian(S, 1e-3, synth.grad_seed(t, q), torch.bfloat16, dev)
        st.step(base, t, out, grad_offset=3, param_offset=5)
        orc.step([bits(x) for x in base], t, out_ref, grad_offset=3, out_offset=5)
    torch.cuda.synchronize()
    assert_bitexact_state("misaligned", gpu_state(st), [orc.master, orc.m, orc.v], bits(out), out_ref)
    st.close()


# --------------------------------------------- determinism, resume, lr

def _run_steps(st, reps_by_t, out, ts):
    for t in ts:
        st.step(reps_by_t[t], t, out)


def test_determinism_and_resume():
    """Two runs give identical bits; 5 steps + get/set state into a fresh
    context + 5 steps == 10 straight steps, bit for bit."""
    numel, world, rank = 300_007, 8, 2
    dev = torch.device("cuda")
    geo = oracle.geometry(numel, world, rank)
    P = geo["padded"]
    flat_p = torch.zeros(P, device=dev)
    flat_p[:numel] = synth.params(numel, device=dev)
    reps = {}
    for t in range(1, 11):
        reps[t] = []
        for q in range(world):
            f = torch.zeros(P, dtype=torch.bfloat16, device=dev)
            f[:numel] = synth.gaussian(numel, 1e-3, synth.grad_seed(t, q), torch.bfloat16, dev)
            reps[t].append(f)
    outs, states = [], []
    for _ in range(2):
        st = zero.ShardState(numel, world, rank, 1e-3)
        st.load_master(flat_p)
        out = torch.zeros(P, dtype=torch.bfloat16, device=dev)
        _run_steps(st, reps, out, range(1, 11))
        outs.append(out.clone())
        states.append(gpu_state(st))
        st.close()
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
    for x, y in zip(*states):
        assert x.tobytes() == y.tobytes()
    a = zero.ShardState(numel, world, rank, 1e-3)
    a.load_master(flat_p)
    out = torch.zeros(P, dtype=torch.bfloat16, device=dev)
    _run_steps(a, reps, out, range(1, 6))
    saved = a.get_state()
    a.close()
    b = zero.ShardState(numel, world, rank, 1e-3)
    b.set_state(*saved)
    _run_steps(b, reps, out, range(6, 11))
    for x, y in zip(gpu_state(b), states[0]):
        assert x.tobytes() == y.tobytes()
    assert torch.equal(out.view(torch.int16), outs[0].view(torch.int16))
    b.close()


def test_set_lr_matches_oracle():
    numel, world = 50_000, 2
    dev = torch.device("cuda")
    st = zero.ShardState(numel, world, 0, 1e-3)
    orc = oracle.ShardOracle(numel, world, 0, 1e-3)
    p = synth.params(st.padded)
    st.load_master(p.to(dev))
    orc.load_master(p.numpy())
    out = torch.zeros(st.padded, device=dev)
    out_h = np.zeros(st.padded, np.float32)
    for t, lr in ((1, 1e-3), (2, 3e-4), (3, 1e-5)):
        st.set_lr(lr)
        orc.lr = lr
        reps = [synth.gaussian(st.padded, 1e-2, synth.grad_seed(t, q), device=dev) for q in range(world)]
        st.step(reps, t, out)
        orc.step([bits(r) for r in reps], t, out_h)
    torch.cuda.synchronize()
    assert_bitexact_state("set_lr", gpu_state(st), [orc.master, orc.m, orc.v], bits(out), out_h)
    st.close()


def test_nonfinite_gradients_stay_local():
    numel, world = 4096, 4
    dev = torch.device("cuda")
    st = zero.ShardState(numel, world, 0, 1e-3)
    orc = oracle.ShardOracle(numel, world, 0, 1e-3)
    p = synth.params(st.padded)
    st.load_master(p.to(dev))
    orc.load_master(p.numpy())
    reps = [synth.gaussian(numel, 1e-3, q, torch.bfloat16, dev) for q in range(world)]
    reps[2][10] = float("nan")
    reps[1][20] = float("inf")
    reps[0][30] = float("-inf")
    reps[3][30] = float("inf")
    out = torch.zeros(numel, dtype=torch.bfloat16, device=dev)
    out_h = np.zeros(numel, np.uint16)
    st.step(reps, 1, out)
    orc.step([bits(r) for r in reps], 1, out_h)
    torch.cuda.synchronize()
    state = gpu_state(st)
    assert_state_parity("nonfinite", state, [orc.master, orc.m, orc.v], bits(out), out_h)
    bad = set(np.nonzero(~np.isfinite(state[0]))[0])
    assert bad == {10, 20, 30}
    st.close()


# ------------------------------------------------------------ flatten

@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_flatten_ragged_bitexact(dtype):
    """Odd sizes and offsets: every tensor's destination misaligned in turn,
    sources at odd element offsets too, single-element tensors, a pad."""
    dev = torch.device("cuda")
    for seed in range(4):
        shapes = synth.ragged_shapes(seed, 37, 20_000) + [(1,), (1,), (3,)]
        numel = synth.numel_of(shapes)
        for world in (1, 3, 8):
            st = zero.ShardState(numel, world, 0, 1e-3)
            P = st.padded
            vals = synth.gaussian(numel + 64, 1.0, seed, dtype)
            # sources carved from one buffer at odd offsets (not 16-byte aligned)
            pool = vals.to(dev)
            srcs, off = [], 1
            for s in shapes:
                k = int(np.prod(s))
                srcs.append(pool[off:off + k])
                off += k
            out = torch.full((P,), -1, dtype=torch.int16 if dtype == torch.bfloat16 else torch.int32,
                             device=dev).view(dtype)
            st.flatten(srcs, out)
            want = oracle.flatten([bits(x) for x in srcs], P, fill=0x5A)
            assert bits(out).tobytes() == want.tobytes(), (seed, world)
            # unflatten into fresh tensors gives the sources back
            dsts = [torch.empty_like(x) for x in srcs]
            st.unflatten(out, dsts)
            for a, b in zip(dsts, srcs):
                assert bits(a).tobytes() == bits(b).tobytes()
            st.close()


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_flatten_every_phase_pair(dtype):
    """Every pair of (source, destination) offsets within 16 bytes, plus
    destinations deeper into a 128-byte line: the destination flat buffer is
    a view at element offset b, the sources are carved from one buffer
    starting at element offset a. The list holds a
    tensor of several copy chunks and a ragged tail, a 1-element tensor and
    a tensor shorter than 16 bytes, so heads, wide bodies and tails all run.
    flatten equals the oracle byte for byte and the guard elements before
    and after the destination keep their fill; unflatten back into views at
    offset a gives the sources back and leaves their neighbours alone."""
    dev = torch.device("cuda")
    ph = 16 // (2 if dtype == torch.bfloat16 else 4)
    ity = torch.int16 if dtype == torch.bfloat16 else torch.int32
    nty = np.int16 if dtype == torch.bfloat16 else np.int32
    sizes = [5 * 1024 + 13, 1, 3, 777]
    numel = sum(sizes)
    st = zero.ShardState(numel, 3, 0, 1e-3)
    P = st.padded
    vals = synth.gaussian(numel + ph, 1.0, 11, dtype).to(dev)
    for a in range(ph):
        srcs, off = [], a
        for k in sizes:
            srcs.append(vals[off:off + k])
            off += k
        src_bits = [bits(x) for x in srcs]
        want = oracle.flatten(src_bits, P, fill=0x5A)
        for b in list(range(ph)) + [5 * ph + 2, 8 * ph - 1]:
            buf = torch.full((P + 9 * ph,), -1, dtype=ity, device=dev).view(dtype)
            st.flatten(srcs, buf[b:b + P])
            got = bits(buf)
            assert got[b:b + P].tobytes() == want.tobytes(), (a, b)
            guard = np.concatenate([got[:b], got[b + P:]])
            assert (guard.view(nty) == -1).all(), (a, b)
            back = torch.full((numel + 2 * ph,), -1, dtype=ity, device=dev).view(dtype)
            dsts, off = [], a
            for k in sizes:
                dsts.append(back[off:off + k])
                off += k
            st.unflatten(buf[b:b + P], dsts)
            bb = bits(back)
            assert bb[a:a + numel].tobytes() == np.concatenate(src_bits).tobytes(), (a, b)
            assert (np.concatenate([bb[:a], bb[a + numel:]]).view(nty) == -1).all(), (a, b)
    log(f"flatten/unflatten {dtype}: all {ph}x{ph} phase pairs equal the oracle")
    st.close()


def test_flatten_gpt2_list():
    shapes = synth.gpt2_small_shapes()
    numel = synth.numel_of(shapes)
    dev = torch.device("cuda")
    st = zero.ShardState(numel, 8, 3, 1e-3)
    g = synth.gaussian(numel, 1e-3, 1, torch.bfloat16, dev)
    ts = synth.split_to_shapes(g, shapes)
    out = torch.empty(st.padded, dtype=torch.bfloat16, device=dev)
    st.flatten(ts, out)
    ref = torch.cat([t.flatten() for t in ts])
    assert torch.equal(out[:numel].view(torch.int16), ref.view(torch.int16))
    # and the oracle, on the host
    want = oracle.flatten([bits(t).reshape(-1) for t in ts], st.padded)
    assert bits(out).tobytes() == want.tobytes()
    st.close()


# --------------------------------------------------------- error paths

def test_binding_rejects_bad_arguments():
    """Undersized or mismatched buffers and t < 1 are refused before any
    launch."""
    dev = torch.device("cuda")
    numel, world = 1 << 20, 4
    st = zero.ShardState(numel, world, 3, 1e-3)
    short = [torch.empty(st.shard // 2, dtype=torch.bfloat16, device=dev) for _ in range(world)]
    out = torch.empty(st.padded, dtype=torch.bfloat16, device=dev)
    with pytest.raises(ValueError):
        st.step(short, 1, out)
    with pytest.raises(ValueError):
        st.step(short[:2], 1, out)
    full = [torch.zeros(st.padded, dtype=torch.bfloat16, device=dev) for _ in range(world)]
    with pytest.raises(zero.ZeroError) as e:
        st.step(full, 0, out)
    assert e.value.code == zero.ZERO_EINVAL
    with pytest.raises(zero.ZeroError) as e:
        st.flatten([out[:10]], out)              # sizes do not sum to numel
    assert e.value.code == zero.ZERO_EINVAL
    torch.cuda.synchronize()
    st.close()


def test_library_range_check_on_exact_allocations():
    """Called through the C ABI directly (no binding checks), a range that
    runs past the end of a hipMalloc allocation is refused with EINVAL
    before any launch; the in-range call on the same buffers succeeds."""
    hip = ctypes.CDLL("libamdhip64.so")
    nbytes = 4096
    g = ctypes.c_void_p()
    o = ctypes.c_void_p()
    assert hip.hipMalloc(ctypes.byref(g), ctypes.c_size_t(nbytes)) == 0
    assert hip.hipMalloc(ctypes.byref(o), ctypes.c_size_t(nbytes)) == 0
    try:
        numel, world = 4096, 2           # shard = 2048 bf16 = 4096 bytes
        st = zero.ShardState(numel, world, 0, 1e-3)
        L = zero.lib()
        ptrs = (ctypes.c_void_p * world)(g.value, g.value)
        stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        assert hip.hipMemset(g, 0, ctypes.c_size_t(nbytes)) == 0
        rc = L.zero_step(st._h, ptrs, world, zero.ZERO_BF16, 1, o.value, zero.ZERO_BF16, 0, 1,
                         stream)
        assert rc == zero.ZERO_EINVAL and b"allocation" in L.zero_last_error()
        rc = L.zero_step(st._h, ptrs, world, zero.ZERO_BF16, 0, o.value, zero.ZERO_BF16, 1, 1,
                         stream)
        assert rc == zero.ZERO_EINVAL
        rc = L.zero_step(st._h, ptrs, world, zero.ZERO_BF16, 0, o.value, zero.ZERO_BF16, 0, 1,
                         stream)
        assert rc == 0
        torch.cuda.synchronize()
        st.close()
    finally:
        hip.hipFree(g)
        hip.hipFree(o)


@pytest.mark.parametrize("lr,betas,eps,t0", [
    (3e-4, (0.85, 0.98), 1e-6, 1),
    (1e-2, (0.5, 0.75), 0.0, 1),
    (1e-3, (0.9, 0.999), 1e-8, 997),       # far into training: 1-b^t near 1
    (5e-5, (0.95, 0.9999), 1e-12, 20000),
])
def test_hyperparameters_and_late_steps(lr, betas, eps, t0):
    """Other Adam hyperparameters and step numbers far from 1 (bias
    correction near 1; the page's counter passed explicitly)."""
    numel, world, rank = 100_003, 4, 2
    dev = torch.device("cuda")
    st = zero.ShardState(numel, world, rank, lr, betas, eps)
    orc = oracle.ShardOracle(numel, world, rank, lr, betas, eps)
    P = st.padded
    p = torch.zeros(P, device=dev)
    p[:numel] = synth.params(numel, device=dev)
    st.load_master(p)
    orc.load_master(bits(p))
    out = torch.zeros(P, dtype=torch.bfloat16, device=dev)
    out_h = np.zeros(P, np.uint16)
    for t in range(t0, t0 + 4):
        reps = []
        for q in range(world):
            f = torch.zeros(P, dtype=torch.bfloat16, device=dev)
            f[:numel] = synth.gaussian(numel, 1e-3, synth.grad_seed(t % 1000, q), torch.bfloat16, dev)
            reps.append(f)
        st.step(reps, t, out)
        orc.step([bits(r) for r in reps], t, out_h)
    torch.cuda.synchronize()
    assert_bitexact_state(f"hparams {lr} {betas} {eps} t0={t0}", gpu_state(st),
                          [orc.master, orc.m, orc.v], bits(out), out_h)
    st.close()


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_flatten_windows(dtype):
    """Windows tiling [0, padded) on 3 streams give zero_flatten's bytes;
    a single window writes nothing outside itself."""
    dev = torch.device("cuda")
    shapes = synth.ragged_shapes(7, 29, 50_000) + [(1,)]
    numel = synth.numel_of(shapes)
    st = zero.ShardState(numel, 8, 0, 1e-3)
    P = st.padded
    srcs = [synth.gaussian(int(np.prod(s)), 1.0, k, dtype, dev) for k, s in enumerate(shapes)]
    fill = -1 if dtype == torch.bfloat16 else -7
    idt = torch.int16 if dtype == torch.bfloat16 else torch.int32
    whole = torch.full((P,), fill, dtype=idt, device=dev).view(dtype)
    st.flatten(srcs, whole)
    tiled = torch.full((P,), fill, dtype=idt, device=dev).view(dtype)
    g = torch.Generator().manual_seed(3)
    cuts = sorted(set(int(x) for x in torch.randint(1, P, (12,), generator=g)))
    bounds = [0] + cuts + [P]
    streams = [torch.cuda.Stream() for _ in range(3)]
    cur = torch.cuda.current_stream()
    for i in range(len(bounds) - 1):
        s = streams[i % 3]
        s.wait_stream(cur)
        st.flatten(srcs, tiled, stream=s, window=(bounds[i], bounds[i + 1] - bounds[i]))
    for s in streams:
        cur.wait_stream(s)
    torch.cuda.synchronize()
    assert torch.equal(whole.view(idt), tiled.view(idt))
    one = torch.full((P,), fill, dtype=idt, device=dev).view(dtype)
    b, n = P // 3 + 1, P // 5
    st.flatten(srcs, one, window=(b, n))
    torch.cuda.synchronize()
    assert torch.equal(one[b:b + n].view(idt), whole[b:b + n].view(idt))
    assert bool((one[:b].view(idt) == fill).all()) and bool((one[b + n:].view(idt) == fill).all())
    with pytest.raises(zero.ZeroError):
        st.flatten(srcs, one, window=(P - 2, 3))
    st.close()


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_flatten_with_empty_tensors(dtype):
    """Zero-element tensors anywhere in the list (first, between, last, a
    (3, 0) matrix) take no room in the flat vector; flatten and unflatten
    stay bit-exact and the step over that flat vector matches the oracle."""
    dev = torch.device("cuda")
    shapes = [(0,), (5,), (3, 0), (1,), (0,), (1000, 3), (7,), (0, 4)]
    numel = synth.numel_of(shapes)
    assert numel == 3013
    st = zero.ShardState(numel, 4, 3, 1e-3)
    P = st.padded
    vals = synth.gaussian(numel, 1.0, 3, dtype).to(dev)
    srcs = synth.split_to_shapes(vals, shapes)
    assert [x.numel() for x in srcs] == [0, 5, 0, 1, 0, 3000, 7, 0]
    out = torch.full((P,), -1, dtype=torch.int16 if dtype == torch.bfloat16 else torch.int32,
                     device=dev).view(dtype)
    st.flatten(srcs, out)
    want = oracle.flatten([bits(x) for x in srcs], P, fill=0x5A)
    assert bits(out).tobytes() == want.tobytes()
    dsts = [torch.full_like(x, 7) for x in srcs]
    st.unflatten(out, dsts)
    for a, b in zip(dsts, srcs):
        assert bits(a).tobytes() == bits(b).tobytes()
    r = run_small_parity(numel, 4, 3, dtype, torch.bfloat16, 2, 1e-3, shapes=shapes,
                         label=f"empty tensors {dtype}")
    assert_bitexact_state("empty tensors", r["state"], r["ref"], r["out"], r["out_ref"])
    st.close()


def test_all_ranks_concurrently_on_separate_streams():
    """Contexts are independent: the N = 4 ranks' contexts step at the same
    time, each on its own stream, reading the same full flat replicas and
    writing disjoint slices of one shared full flat output (the all-gather's
    result). 3 steps of 400,013 elements (ragged shard, pad in rank 3);
    every rank's state and the whole output equal the oracle bit for bit,
    and the pad stays +0."""
    dev = torch.device("cuda")
    numel, world, steps = 400_013, 4, 3
    states = [zero.ShardState(numel, world, r, 1e-3) for r in range(world)]
    orcs = [oracle.ShardOracle(numel, world, r, 1e-3) for r in range(world)]
    P = states[0].padded
    p = torch.zeros(P, dtype=torch.float32, device=dev)
    p[:numel] = synth.gaussian(numel, synth.PARAM_STD, synth.PARAM_SEED, torch.float32, dev)
    for st, o in zip(states, orcs):
        st.load_master(p)
        o.load_master(bits(p))
    streams = [torch.cuda.Stream() for _ in range(world)]
    out = torch.zeros(P, dtype=torch.bfloat16, device=dev)
    out_ref = np.zeros(P, np.uint16)
    torch.cuda.synchronize()
    for t in range(1, steps + 1):
        reps = []
        for q in range(world):
            g = torch.zeros(P, dtype=torch.bfloat16, device=dev)
            g[:numel] = synth.gaussian(numel, 1e-3, synth.grad_seed(t, q), torch.bfloat16, dev)
            reps.append(g)
        torch.cuda.synchronize()
        for st, s in zip(states, streams):
            st.step(reps, t, out, stream=s)
        reps_h = [bits(g) for g in reps]
        for o in orcs:
            o.step(reps_h, t, out_ref)
        torch.cuda.synchronize()
        assert bits(out).tobytes() == out_ref.tobytes(), f"shared output differs at t={t}"
        for r, (st, o) in enumerate(zip(states, orcs)):
            assert_bitexact_state(f"concurrent rank {r} t={t}", gpu_state(st),
                                  [o.master, o.m, o.v], None, None)
        assert not np.any(out_ref[numel:])
        log(f"concurrent ranks: step {t} bit-exact")
    for st in states:
        st.close()
