"""The page's 4-process experiment ([ZeRO and FSDP], "Implementing ZeRO's
Adam from scratch": the MLP 64 -> 256 -> 10 on a batch of 32 split across 4
ranks, 3 steps, compared with single-process torch.optim.Adam), run through
the HIP library on one GPU.

Each simulated rank computes its quarter-batch gradient on the GPU and the
library flattens it into that rank's padded flat vector (zero_flatten).
Every rank's shard state then steps its slice from the 4 vectors
(zero_step) and writes the updated fp32 slice into one full flat parameter
buffer (the all-gather's result), which the library cuts back into the
model's tensors (zero_unflatten). After 3 steps the model must be within
the page's 1e-5 of torch.optim.Adam on the full batch, and every rank's
master/m/v and the flat parameters must equal the CPU oracle fed the same
gradient bits, bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import zero_partitioned_optimizer_flatten_amd as zero
from gpu_harness import bits, log

pytestmark = pytest.mark.gpu
WORLD, LR, STEPS = 4, 1e-2, 3


def _model(dev):
    torch.manual_seed(0)
    return torch.nn.Sequential(torch.nn.Linear(64, 256), torch.nn.GELU(),
                               torch.nn.Linear(256, 10)).to(dev)


def test_page_experiment_through_the_library():
    dev = torch.device("cuda")
    torch.manual_seed(123)
    X, Y = torch.randn(32, 64).to(dev), torch.randint(0, 10, (32,)).to(dev)
    loss_fn = torch.nn.CrossEntropyLoss()

    ref = _model(dev)
    opt = torch.optim.Adam(ref.parameters(), lr=LR)
    model = _model(dev)
    params = list(model.parameters())
    numel = sum(p.numel() for p in params)
    states = [zero.ShardState(numel, WORLD, r, LR) for r in range(WORLD)]
    S, P = states[0].shard, states[0].padded
    assert (numel, S) == (19_210, 4_803)                 # the page's toy model
    # the page's state_bytes per rank (12 bytes per shard element: 57,636)
    assert [st.state_bytes() for st in states] == [oracle.state_bytes(S)] * WORLD == [57_636] * WORLD

    flat_params = torch.empty(P, dtype=torch.float32, device=dev)
    states[0].flatten([p.detach() for p in params], flat_params)
    for st in states:
        st.load_master(flat_params)                      # each rank's fp32 slice
    orcs = [oracle.ShardOracle(numel, WORLD, r, LR) for r in range(WORLD)]
    for o in orcs:
        o.load_master(bits(flat_params))
    replicas = [torch.empty(P, dtype=torch.float32, device=dev) for _ in range(WORLD)]
    flat_ref = np.zeros(P, np.float32)

    for t in range(1, STEPS + 1):
        opt.zero_grad()
        loss_fn(ref(X), Y).backward()
        opt.step()
        for r in range(WORLD):                           # each rank's backward
            model.zero_grad()
            sl = slice(r * 8, (r + 1) * 8)
            loss_fn(model(X[sl]), Y[sl]).backward()
            states[r].flatten([p.grad for p in params], replicas[r])
        reps_h = [bits(x) for x in replicas]
        for r, st in enumerate(states):
            st.step(replicas, t, flat_params)            # writes [lo_r, lo_r + S)
            orcs[r].step(reps_h, t, flat_ref)
        states[0].unflatten(flat_params, [p.data for p in params])
        torch.cuda.synchronize()
        for r, st in enumerate(states):
            got = [x.cpu().numpy() for x in st.get_state()]
            for g, w in zip(got, (orcs[r].master, orcs[r].m, orcs[r].v)):
                assert g.tobytes() == w.tobytes(), f"rank {r} state differs from the oracle at t={t}"
        assert bits(flat_params).tobytes() == flat_ref.tobytes()
        assert not np.any(bits(flat_params)[numel:])    # the pad stays +0
        log(f"page experiment: step {t} bit-exact against the oracle")

    diff = max(float((a - b).detach().abs().max()) for a, b in zip(ref.parameters(), model.parameters()))
    log(f"page experiment: max |param - torch.optim.Adam| = {diff:.3g}")
    assert diff < 1e-5                                   # the page's own threshold
    for st in states:
        st.close()


def test_page_fsdp_experiment_through_the_library():
    """The page's FSDP2 comparison ([ZeRO and FSDP], section "ZeRO-3 and
    FSDP"): the same MLP, each parameter split by rows across the 4 ranks.
    Each rank's per-parameter shard state steps its rows from the 4 ranks'
    full gradients and writes them into the model (the gather of the row
    shards); after 3 steps the model is within 1e-5 of torch.optim.Adam, and
    every rank's outputs equal the per-parameter oracle bit for bit."""
    dev = torch.device("cuda")
    torch.manual_seed(123)
    X, Y = torch.randn(32, 64).to(dev), torch.randint(0, 10, (32,)).to(dev)
    loss_fn = torch.nn.CrossEntropyLoss()
    ref = _model(dev)
    opt = torch.optim.Adam(ref.parameters(), lr=LR)
    model = _model(dev)
    params = list(model.parameters())
    shapes = [tuple(p.shape) for p in params]
    states = [zero.FsdpShardState(shapes, WORLD, r, LR) for r in range(WORLD)]
    orcs = [oracle.FsdpShardOracle(shapes, WORLD, r, LR) for r in range(WORLD)]
    # state bytes count this rank's rows only (not the line padding between
    # pieces), and over all ranks they cover every parameter once
    held = [st.state_bytes() for st in states]
    assert held == [12 * sum(st.local_numel(k) for k in range(len(shapes))) for st in states]
    assert sum(held) == 12 * sum(int(np.prod(s)) for s in shapes)
    for st, o in zip(states, orcs):
        st.load_master([p.detach() for p in params])
        o.load_master([bits(p.detach()).reshape(-1) for p in params])
    outs = [[torch.empty(max(1, st.local_numel(k)), dtype=torch.float32, device=dev)
             for k in range(len(shapes))] for st in states]
    outs_h = [[np.zeros(n, np.float32) for n in o.local_numels()] for o in orcs]
    grads = [[torch.empty(s, dtype=torch.float32, device=dev) for s in shapes]
             for _ in range(WORLD)]
    for t in range(1, STEPS + 1):
        opt.zero_grad()
        loss_fn(ref(X), Y).backward()
        opt.step()
        for r in range(WORLD):
            model.zero_grad()
            sl = slice(r * 8, (r + 1) * 8)
            loss_fn(model(X[sl]), Y[sl]).backward()
            for g, p in zip(grads[r], params):
                g.copy_(p.grad)
        grads_h = [[bits(g).reshape(-1) for g in gl] for gl in grads]
        for r in range(WORLD):
            states[r].step(grads, t, outs[r])
            orcs[r].step(grads_h, t, outs_h[r])
        torch.cuda.synchronize()
        with torch.no_grad():                             # gather the row shards
            for r, st in enumerate(states):
                for k, p in enumerate(params):
                    f, rows, _ = st.local[k]
                    n = st.local_numel(k)
                    if rows:
                        p.view(p.shape[0], -1)[f:f + rows] = outs[r][k][:n].view(rows, -1)
                        assert bits(outs[r][k][:n]).tobytes() == outs_h[r][k].tobytes(), \
                            f"rank {r} parameter {k} differs from the oracle at t={t}"
        log(f"page FSDP experiment: step {t} bit-exact against the oracle")
    diff = max(float((a - b).detach().abs().max()) for a, b in zip(ref.parameters(), model.parameters()))
    log(f"page FSDP experiment: max |param - torch.optim.Adam| = {diff:.3g}")
    assert diff < 1e-5
    for st in states:
        st.close()
