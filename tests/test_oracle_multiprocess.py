"""The toy experiment of [ZF] "Implementing ZeRO's Adam from scratch" with
real collectives: 4 processes over gloo on the CPU, each with a quarter of
the batch of a 64-256-10 MLP.

Each process steps two copies of the model:
  * torch: the sharded step written from the method's definition with torch
    collectives (reduce-scatter of the padded flat gradient, divide by the
    world size, the Adam equations on this rank's slice, all-gather of the
    updated slices);
  * oracle: all-gather of every rank's flat gradient (the N replicas),
    ShardOracle.step for this rank's slice, all-gather of the updated slices.
After 3 steps both must match single-process torch.optim.Adam on the full
batch within the page's 1e-5, and the oracle's shards must reassemble into
a vector that equals the oracle run unsharded on the gathered replicas,
bit for bit."""
import math
import os
import socket
import sys

import numpy as np
import torch
import torch.distributed as dist
import torch.multiprocessing as mp
from torch.nn.utils import parameters_to_vector, vector_to_parameters

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _free_port():
    with socket.socket() as s:
        s.bind(("127.0.0.1", 0))
        return s.getsockname()[1]


def _make_model():
    torch.manual_seed(0)
    return torch.nn.Sequential(torch.nn.Linear(64, 256), torch.nn.GELU(),
                               torch.nn.Linear(256, 10))


def _padded(vec, length):
    """vec followed by zeros up to `length` (the zero-padded flat vector)."""
    return torch.nn.functional.pad(vec, (0, length - vec.numel()))


def _torch_sharded_step(model, state, t, world, rank, lr, betas, eps):
    """One data-parallel rank's ZeRO-2 step from the definitions, in torch.
    state: this rank's fp32 slice (master, m, v) and the padded length."""
    from oracle_pins import torch_adam
    master, m, v, padded = state["master"], state["m"], state["v"], state["padded"]
    shard = padded // world
    grads = _padded(parameters_to_vector(p.grad for p in model.parameters()), padded)
    g = torch.empty(shard)
    dist.reduce_scatter_tensor(g, grads)                   # sum over the ranks
    g = g / world
    master, m, v = torch_adam(master, m, v, g, t, lr, betas[0], betas[1], eps)
    state.update(master=master, m=m, v=v)
    full = torch.empty(padded)
    dist.all_gather_into_tensor(full, master)
    vector_to_parameters(full[:sum(p.numel() for p in model.parameters())],
                         model.parameters())


def _torch_sharded_state(model, world, rank):
    numel = sum(p.numel() for p in model.parameters())
    shard = math.ceil(numel / world)
    flat = _padded(parameters_to_vector(model.parameters()).detach(), shard * world)
    master = flat[rank * shard:(rank + 1) * shard].clone()
    return dict(master=master, m=torch.zeros(shard), v=torch.zeros(shard),
                padded=shard * world)


def _worker(rank, world, port, outdir):
    os.environ.update(MASTER_ADDR="127.0.0.1", MASTER_PORT=str(port))
    sys.path[:0] = [ROOT, os.path.join(ROOT, "tests")]
    import oracle
    dist.init_process_group("gloo", rank=rank, world_size=world)
    torch.manual_seed(123)
    X, Y = torch.randn(32, 64), torch.randint(0, 10, (32,))
    sl = slice(rank * 32 // world, (rank + 1) * 32 // world)
    loss_fn = torch.nn.CrossEntropyLoss()
    ref, torch_model, orc_model = _make_model(), _make_model(), _make_model()
    opt_ref = torch.optim.Adam(ref.parameters(), lr=1e-2)
    torch_state = _torch_sharded_state(torch_model, world, rank)
    numel = sum(p.numel() for p in orc_model.parameters())
    geo = oracle.geometry(numel, world, rank)
    P = geo["padded"]
    flat_p = oracle.flatten([p.detach().numpy().reshape(-1) for p in orc_model.parameters()], P)
    orc = oracle.ShardOracle(numel, world, rank, 1e-2)
    orc.load_master(flat_p)
    whole = oracle.ShardOracle(P, 1, 0, 1e-2, n_replicas=world)
    whole.load_master(flat_p)
    bitexact = True
    for t in range(1, 4):
        opt_ref.zero_grad()
        loss_fn(ref(X), Y).backward()
        opt_ref.step()
        for p in torch_model.parameters():
            p.grad = None
        loss_fn(torch_model(X[sl]), Y[sl]).backward()
        with torch.no_grad():
            _torch_sharded_step(torch_model, torch_state, t, world, rank, 1e-2, (0.9, 0.999), 1e-8)
        for p in orc_model.parameters():
            p.grad = None
        loss_fn(orc_model(X[sl]), Y[sl]).backward()
        mine = torch.from_numpy(oracle.flatten(
            [p.grad.numpy().reshape(-1) for p in orc_model.parameters()], P))
        reps = [torch.empty(P) for _ in range(world)]
        dist.all_gather(reps, mine)
        reps_np = [r.numpy() for r in reps]
        out = np.zeros(P, np.float32)
        orc.step(reps_np, t, out)
        slices = [torch.empty(geo["shard"]) for _ in range(world)]
        dist.all_gather(slices, torch.from_numpy(out[geo["lo"]:geo["lo"] + geo["shard"]].copy()))
        full = torch.cat(slices).numpy()
        out_whole = np.zeros(P, np.float32)
        whole.step(reps_np, t, out_whole, grad_offset=0, out_offset=0)
        bitexact = bitexact and full.tobytes() == out_whole.tobytes()
        with torch.no_grad():
            off = 0
            for p in orc_model.parameters():
                p.copy_(torch.from_numpy(full[off:off + p.numel()]).view_as(p))
                off += p.numel()
    d_torch = max(float((a - b).detach().abs().max()) for a, b in
                  zip(ref.parameters(), torch_model.parameters()))
    d_orc = max(float((a - b).detach().abs().max()) for a, b in
                zip(ref.parameters(), orc_model.parameters()))
    d_to = max(float((a - b).detach().abs().max()) for a, b in
               zip(torch_model.parameters(), orc_model.parameters()))
    np.save(os.path.join(outdir, f"r{rank}.npy"),
            np.array([d_torch, d_orc, d_to, float(bitexact)]))
    dist.destroy_process_group()


def test_toy_experiment_four_processes(tmp_path):
    world = 4
    mp.spawn(_worker, args=(world, _free_port(), str(tmp_path)), nprocs=world, join=True)
    for r in range(world):
        d_torch, d_orc, d_to, bitexact = np.load(tmp_path / f"r{r}.npy")
        assert d_torch < 1e-5, d_torch         # the page's bound, torch sharded step
        assert d_orc < 1e-5, d_orc             # the oracle, sharded over 4 processes
        assert d_to < 1e-6, d_to               # oracle vs the torch sharded step
        assert bitexact == 1.0                 # shards reassemble the unsharded update
