"""Bucketed ZeRO-2 step: the fused update applied bucket by bucket as
gradient buckets arrive, on several streams, each bucket's gradient
buffers released right after use. The result must be bit-identical to one
whole-shard step (the update is elementwise) and to the oracle."""
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
    torch.cuda.empty_cache()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _bucketed_step(st, full_reps, t, out, bounds, streams, out_offset_is_flat=True):
    """Feed this rank's part of every bucket through step_range. Each
    bucket's replica pieces are fresh buffers (what a bucketed
    reduce-scatter would hand this rank) that die after the bucket."""
    cur = torch.cuda.current_stream()
    for i, (k, sb, cnt, _) in enumerate(st.bucket_ranges(bounds)):
        s = streams[i % len(streams)]
        pieces = [r[st.lo + sb: st.lo + sb + cnt].clone() for r in full_reps]
        s.wait_stream(cur)
        for pc in pieces:
            pc.record_stream(s)
        po = st.lo + sb if out_offset_is_flat else sb
        st.step_range(sb, cnt, pieces, t, out, grad_offset=0, param_offset=po, stream=s)
        del pieces
    for s in streams:
        cur.wait_stream(s)


@pytest.mark.parametrize("cap", [0, 1])
@pytest.mark.parametrize("rank", [1, 3])
@pytest.mark.parametrize("gdt", [torch.float32, torch.bfloat16])
def test_bucketed_equals_whole_step_and_oracle(rank, gdt, cap):
    """cap: workgroups per compute unit for the bucketed context (0: none)."""
    numel, world = 1_000_003, 4
    dev = torch.device("cuda")
    whole = zero.ShardState(numel, world, rank, 1e-3)
    buck = zero.ShardState(numel, world, rank, 1e-3)
    buck.set_step_workgroups(cap)
    orc = oracle.ShardOracle(numel, world, rank, 1e-3)
    P = whole.padded
    flat_p = torch.zeros(P, device=dev)
    flat_p[:numel] = synth.params(numel, device=dev)
    whole.load_master(flat_p)
    buck.load_master(flat_p)
    orc.load_master(bits(flat_p))
    # bucket boundaries: ragged, some mid-vector, one tiny bucket
    g = torch.Generator().manual_seed(rank)
    cuts = sorted(set(int(x) for x in torch.randint(1, P, (9,), generator=g)) | {P // 2 + 3, P // 2 + 4})
    bounds = [0] + cuts + [P]
    streams = [torch.cuda.Stream() for _ in range(3)]
    out_w = torch.zeros(P, dtype=torch.bfloat16, device=dev)
    out_b = torch.zeros(P, dtype=torch.bfloat16, device=dev)
    out_h = np.zeros(P, np.uint16)
    for t in range(1, 6):
        reps = []
        for q in range(world):
            f = torch.zeros(P, dtype=gdt, device=dev)
            f[:numel] = synth.gaussian(numel, 1e-3, synth.grad_seed(t, q), gdt, dev)
            reps.append(f)
        whole.step(reps, t, out_w)
        _bucketed_step(buck, reps, t, out_b, bounds, streams)
        orc.step([bits(r) for r in reps], t, out_h)
    torch.cuda.synchronize()
    sw, sb = gpu_state(whole), gpu_state(buck)
    for x, y in zip(sw, sb):
        assert x.tobytes() == y.tobytes()
    assert torch.equal(out_w.view(torch.int16), out_b.view(torch.int16))
    assert_bitexact_state("bucketed", sb, [orc.master, orc.m, orc.v], bits(out_b), out_h)
    whole.close()
    buck.close()


def test_bucketed_full_size_7b():
    """7e9/N=8 rank-0 shard in 64M-element buckets on 2 streams, 3 steps:
    identical bits to the whole-shard step, compared on the GPU."""
    numel, world = 7_000_000_000, 8
    dev = torch.device("cuda")
    whole = zero.ShardState(numel, world, 0, 1e-3)
    buck = zero.ShardState(numel, world, 0, 1e-3)
    S = whole.shard
    p = synth.gaussian(S, synth.PARAM_STD, synth.PARAM_SEED, torch.float32, dev)
    whole.load_master(p, flat_offset=0)
    buck.load_master(p, flat_offset=0)
    del p
    reps = [torch.empty(S, dtype=torch.bfloat16, device=dev) for _ in range(world)]
    out_w = torch.empty(S, dtype=torch.bfloat16, device=dev)
    out_b = torch.empty(S, dtype=torch.bfloat16, device=dev)
    bucket = 1 << 26
    streams = [torch.cuda.Stream() for _ in range(2)]
    cur = torch.cuda.current_stream()
    for t in range(1, 4):
        for q in range(world):
            synth.fill_gaussian(reps[q], 1e-3, synth.grad_seed(t, q))
        whole.step(reps, t, out_w)
        for i, b0 in enumerate(range(0, S, bucket)):
            cnt = min(bucket, S - b0)
            s = streams[i % 2]
            s.wait_stream(cur)
            buck.step_range(b0, cnt, [r[b0:] for r in reps], t, out_b, grad_offset=0,
                            param_offset=b0, stream=s)
        for s in streams:
            cur.wait_stream(s)
        log(f"bucketed 7b: step {t} done")
    torch.cuda.synchronize()
    for x, y in zip(whole.get_state(), buck.get_state()):
        assert torch.equal(x.view(torch.int32), y.view(torch.int32))
    assert torch.equal(out_w.view(torch.int16), out_b.view(torch.int16))
    whole.close()
    buck.close()


@pytest.mark.parametrize("phase", ["lo", 0, 1])
def test_capped_step_equals_uncapped_and_oracle(phase):
    """Steps capped at 1 and 3 workgroups per compute unit (each workgroup
    walking many blocks) against the uncapped step and the oracle. The
    slice-only replicas and output start `phase` elements past a 128-byte
    line: "lo" puts them at the phase element lo has in a full flat buffer,
    which the state shares (vector path); 0 and 1 put them off it (shifted
    path)."""
    numel, world, rank = 2_000_003, 4, 3
    dev = torch.device("cuda")
    sts = [zero.ShardState(numel, world, rank, 1e-3) for _ in range(3)]
    sts[1].set_step_workgroups(1)
    sts[2].set_step_workgroups(3)
    orc = oracle.ShardOracle(numel, world, rank, 1e-3)
    S, valid = sts[0].shard, numel - sts[0].lo
    p = torch.zeros(S, device=dev)
    p[:valid] = synth.gaussian(valid, synth.PARAM_STD, synth.PARAM_SEED, torch.float32, dev)
    for st in sts:
        st.load_master(p, flat_offset=0)
    orc.master[:] = bits(p)
    ph = sts[0].lo % 64 if phase == "lo" else phase
    bufs = [torch.zeros(S + 64, dtype=torch.bfloat16, device=dev) for _ in range(world)]
    reps = [b[ph:ph + S] for b in bufs]
    outs = [torch.zeros(S + 64, dtype=torch.bfloat16, device=dev)[ph:ph + S] for _ in sts]
    out_h = np.zeros(S, np.uint16)
    for t in range(1, 4):
        for q, r in enumerate(reps):
            synth.fill_gaussian(r[:valid], 1e-3, synth.grad_seed(t, q))
        for st, o in zip(sts, outs):
            st.step(reps, t, o, grad_offset=0, param_offset=0)
        orc.step([bits(r) for r in reps], t, out_h, grad_offset=0, out_offset=0)
    torch.cuda.synchronize()
    ref = gpu_state(sts[0])
    for k in (1, 2):
        for x, y in zip(ref, gpu_state(sts[k])):
            assert x.tobytes() == y.tobytes(), (phase, k)
        assert torch.equal(outs[0].view(torch.int16), outs[k].view(torch.int16)), (phase, k)
    assert_bitexact_state(f"capped phase {phase}", gpu_state(sts[1]),
                          [orc.master, orc.m, orc.v], bits(outs[1]), out_h)
    for st in sts:
        st.close()


def test_capped_step_full_size_7b():
    """The 7e9/N=8 rank-0 shard with 2 workgroups per compute unit (each
    walking about 3,300 blocks, offsets past 2^31 elements) equals the
    uncapped step bit for bit, compared on the GPU."""
    numel, world = 7_000_000_000, 8
    dev = torch.device("cuda")
    whole = zero.ShardState(numel, world, 0, 1e-3)
    capd = zero.ShardState(numel, world, 0, 1e-3)
    capd.set_step_workgroups(2)
    S = whole.shard
    p = synth.gaussian(S, synth.PARAM_STD, synth.PARAM_SEED, torch.float32, dev)
    whole.load_master(p, flat_offset=0)
    capd.load_master(p, flat_offset=0)
    del p
    reps = [torch.empty(S, dtype=torch.bfloat16, device=dev) for _ in range(world)]
    out_w = torch.empty(S, dtype=torch.bfloat16, device=dev)
    out_c = torch.empty(S, dtype=torch.bfloat16, device=dev)
    for t in range(1, 3):
        for q in range(world):
            synth.fill_gaussian(reps[q], 1e-3, synth.grad_seed(t, q))
        whole.step(reps, t, out_w)
        capd.step(reps, t, out_c)
        log(f"capped 7b: step {t} done")
    torch.cuda.synchronize()
    for x, y in zip(whole.get_state(), capd.get_state()):
        assert torch.equal(x.view(torch.int32), y.view(torch.int32))
    assert torch.equal(out_w.view(torch.int16), out_c.view(torch.int16))
    whole.close()
    capd.close()


def test_step_range_rejects_out_of_shard():
    dev = torch.device("cuda")
    st = zero.ShardState(1000, 2, 0, 1e-3)
    reps = [torch.zeros(st.shard, device=dev) for _ in range(2)]
    out = torch.zeros(st.shard, device=dev)
    with pytest.raises(ValueError):
        st.step_range(400, 200, reps, 1, out)
    import ctypes
    ptrs = (ctypes.c_void_p * 2)(*[r.data_ptr() for r in reps])
    rc = zero.lib().zero_step_range(st._h, 400, 200, ptrs, 2, zero.ZERO_F32, 0, out.data_ptr(),
                                    zero.ZERO_F32, 0, 1, None)
    assert rc == zero.ZERO_EINVAL
    st.step_range(0, 0, reps, 1, out)        # empty range is a no-op
    torch.cuda.synchronize()
    st.close()
