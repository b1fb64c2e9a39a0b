"""Full-size shards (the 7e9 / N=8, Llama-13B / N=8 and 70e9 / N=64
workloads) on the GPU, checked against the oracle on sampled elements.

The update is elementwise, so the oracle run on the gathered elements of
every input gives exactly the full-shard oracle's values at those
positions. Samples: 2^20 random positions plus the first and last 4096
(which hold the pad, where there is one)."""
import numpy as np
import pytest
import torch

import oracle
import synth
import zero_partitioned_optimizer_flatten_amd as zero
from gpu_harness import assert_bitexact_state, assert_state_parity, bits, log

pytestmark = pytest.mark.gpu
LR, BETAS, EPS = 1e-3, (0.9, 0.999), 1e-8


@pytest.fixture(autouse=True)
def _gpu():
    assert torch.cuda.is_available()
    zero.lib()
    torch.cuda.empty_cache()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _sample(S, dev, seed=99):
    g = torch.Generator(device="cpu").manual_seed(seed)
    r = torch.randint(0, S, (1 << 20,), generator=g)
    edge = torch.cat([torch.arange(min(4096, S)), torch.arange(max(0, S - 4096), S)])
    return torch.unique(torch.cat([r, edge])).to(dev)


def _check_sampled(label, st, orc, idx, out, out_off, out_ref):
    torch.cuda.synchronize()
    state = st.get_state()
    got = [bits(x[idx]) for x in state]
    del state
    out_got = bits(out[out_off + idx])
    assert_state_parity(label, got, [orc.master, orc.m, orc.v], out_got, out_ref)
    assert_bitexact_state(label, got, [orc.master, orc.m, orc.v], out_got, out_ref)


def _slice_only_run(numel, world, rank, steps, label):
    """Slice-only replicas and output, 16-byte aligned: the vector path in
    the launch configuration the benchmark times."""
    dev = torch.device("cuda")
    st = zero.ShardState(numel, world, rank, LR, BETAS, EPS)
    S = st.shard
    assert st.lo + S <= numel                      # no pad in these shards
    idx = _sample(S, dev)
    K = idx.numel()
    p = synth.gaussian(S, synth.PARAM_STD, synth.PARAM_SEED, torch.float32, dev)
    st.load_master(p, flat_offset=0)
    orc = oracle.ShardOracle(K, 1, 0, LR, BETAS, EPS, n_replicas=world)
    orc.load_master(bits(p[idx]))
    del p
    reps = [torch.empty(S, dtype=torch.bfloat16, device=dev) for _ in range(world)]
    out = torch.empty(S, dtype=torch.bfloat16, device=dev)
    out_ref = np.zeros(K, np.uint16)
    for t in range(1, steps + 1):
        for q in range(world):
            synth.fill_gaussian(reps[q], 1e-3, synth.grad_seed(t, q))
        st.step(reps, t, out)
        orc.step([bits(r[idx]) for r in reps], t, out_ref, grad_offset=0, out_offset=0)
        log(f"{label}: step {t} done")
    _check_sampled(label, st, orc, idx, out, 0, out_ref)
    st.close()


def test_flat7b_n8_rank0_full_size():
    """7e9-element flat vector, N = 8, rank 0: S = 875,000,000, eight bf16
    slice-only replicas N(0, 1e-3), fp32 master/m/v, bf16 output, 10 steps."""
    _slice_only_run(7_000_000_000, 8, 0, 10, "flat7b_n8")


def test_flat70b_n64_rank0_full_size():
    """70e9-element state at N = 64, rank 0: S = 1,093,750,000, 64 bf16
    slice-only replicas (140 GB), 3 steps."""
    _slice_only_run(70_000_000_000, 64, 0, 3, "flat70b_n64")


@pytest.mark.parametrize("peer_phase", ["zero", "lo"])
def test_llama13b_n8_last_rank_full_size(peer_phase):
    """Llama-13B list + 1 scalar (364 tensors, 13,015,864,321 elements),
    N = 8, rank 7 (7 pad elements at the end of its slice, odd lo). This
    rank's own gradient is a real tensor list flattened by the HIP path into
    a full padded vector; the seven peers hold this slice only, either at
    address phase 0 (mixed 16-byte phases: the shifted path) or at the
    offset within a 128-byte line that element lo has in a full flat buffer
    (every stream at the state's phase: the vector path). bf16 gradients
    N(0, 1e-3) with 1% of elements x100, bf16 output into the full flat
    parameter buffer at offset lo, 5 steps."""
    shapes = synth.llama_shapes(40, 5120, 13824, trailing_scalar=True)
    numel = synth.numel_of(shapes)
    assert len(shapes) == 364 and numel == 13_015_864_321
    world, rank = 8, 7
    dev = torch.device("cuda")
    st = zero.ShardState(numel, world, rank, LR, BETAS, EPS)
    S, lo, P = st.shard, st.lo, st.padded
    assert (S, lo, P - numel) == (1_626_983_041, 11_388_881_287, 7)
    valid = numel - lo
    idx = _sample(S, dev)
    K = idx.numel()
    p = torch.zeros(S, dtype=torch.float32, device=dev)
    synth.fill_gaussian(p[:valid], synth.PARAM_STD, synth.PARAM_SEED)
    st.load_master(p, flat_offset=0)
    orc = oracle.ShardOracle(K, 1, 0, LR, BETAS, EPS, n_replicas=world)
    orc.load_master(bits(p[idx]))
    del p
    own_list_storage = torch.empty(numel, dtype=torch.bfloat16, device=dev)
    own_flat = torch.empty(P, dtype=torch.bfloat16, device=dev)
    ph = lo % 64 if peer_phase == "lo" else 0
    peers = [torch.zeros(S + 64, dtype=torch.bfloat16, device=dev)[ph:ph + S]
             for _ in range(world - 1)]
    out = torch.zeros(P, dtype=torch.bfloat16, device=dev)
    out_ref = np.zeros(K, np.uint16)
    for t in range(1, 6):
        synth.fill_gaussian(own_list_storage, 1e-3, synth.grad_seed(t, rank),
                            synth.mask_seed(t, rank))
        tensors = synth.split_views(own_list_storage, shapes)
        own_flat.fill_(float("nan"))              # every element must be written
        st.flatten(tensors, own_flat)
        if t == 1:   # the flatten itself: bit-exact against its definition
            torch.cuda.synchronize()
            assert torch.equal(own_flat[:numel].view(torch.int16),
                               own_list_storage.view(torch.int16))
            assert not torch.any(own_flat[numel:].view(torch.int16))
            log(f"llama13b_n8 peers@{peer_phase}: flatten of 364 tensors bit-exact")
        for k, q in enumerate(q for q in range(world) if q != rank):
            synth.fill_gaussian(peers[k][:valid], 1e-3, synth.grad_seed(t, q),
                                synth.mask_seed(t, q))
        reps = peers[:rank] + [own_flat[lo:]] + peers[rank:]
        st.step(reps, t, out, grad_offset=0, param_offset=lo)
        orc.step([bits(r[idx]) for r in reps], t, out_ref, grad_offset=0, out_offset=0)
        log(f"llama13b_n8 peers@{peer_phase}: step {t} done")
    _check_sampled(f"llama13b_n8 peers@{peer_phase}", st, orc, idx, out, lo, out_ref)
    tail = bits(st.get_state()[0][valid:])
    assert not np.any(tail.view(np.uint32)), "pad master not zero"
    st.close()


def test_flatten_single_tensor_beyond_one_dispatch():
    """A one-tensor list of 9,000,000,001 bf16 elements (18 GB) flattened
    to 9,000,000,008 (N = 8): longer than one copy dispatch may cover, so
    the library splits it; result bit-exact and pad zero."""
    dev = torch.device("cuda")
    numel, world = 9_000_000_001, 8
    st = zero.ShardState(numel, world, 0, LR)
    src = torch.empty(numel, dtype=torch.bfloat16, device=dev)
    synth.fill_gaussian(src, 1.0, 3)
    dst = torch.full((st.padded,), -1, dtype=torch.int16, device=dev).view(torch.bfloat16)
    st.flatten([src], dst)
    torch.cuda.synchronize()
    assert torch.equal(dst[:numel].view(torch.int16), src.view(torch.int16))
    assert not torch.any(dst[numel:].view(torch.int16))
    log("flatten of an 18 GB tensor bit-exact")
    st.close()
