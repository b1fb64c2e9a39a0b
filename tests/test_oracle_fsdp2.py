"""The per-parameter dim-0 layout against FSDP2 itself, on the CPU with the
gloo backend (the pages run their FSDP2 script the same way): the local
shard shapes FSDP2 assigns, and the page's 3-step comparison with the
oracle's per-parameter shards in place of FSDP2's optimizer."""
import os
import socket

import numpy as np
import pytest
import torch
import torch.distributed as dist
import torch.multiprocessing as mp


def _free_port():
    with socket.socket() as s:
        s.bind(("127.0.0.1", 0))
        return s.getsockname()[1]


def _make_model():
    torch.manual_seed(0)
    return torch.nn.Sequential(torch.nn.Linear(64, 256), torch.nn.GELU(),
                               torch.nn.Linear(256, 10), torch.nn.Linear(10, 5))


def _worker(rank, world, port, outdir):
    os.environ.update(MASTER_ADDR="127.0.0.1", MASTER_PORT=str(port))
    import sys
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    from torch.distributed.device_mesh import init_device_mesh
    from torch.distributed.fsdp import fully_shard
    dist.init_process_group("gloo", rank=rank, world_size=world)
    mesh = init_device_mesh("cpu", (world,))
    torch.manual_seed(123)
    X, Y = torch.randn(32, 64), torch.randint(0, 10, (32,))
    model = _make_model()
    for layer in model:
        if isinstance(layer, torch.nn.Linear):
            fully_shard(layer, mesh=mesh)
    fully_shard(model, mesh=mesh)
    head = torch.nn.Linear(5, 10)
    loss_fn = torch.nn.CrossEntropyLoss()
    opt = torch.optim.Adam(model.parameters(), lr=1e-2, foreach=False)
    local0 = [p.to_local().detach().clone().numpy() for p in model.parameters()]
    sl = slice(rank * 32 // world, (rank + 1) * 32 // world)
    grads = []
    for _ in range(3):
        opt.zero_grad()
        loss_fn(head(model(X[sl])), Y[sl]).backward()
        grads.append([p.grad.to_local().detach().clone().numpy() for p in model.parameters()])
        opt.step()
    local3 = [p.to_local().detach().clone().numpy() for p in model.parameters()]
    np.savez(os.path.join(outdir, f"rank{rank}.npz"),
             **{f"s{k}": np.array(a.shape) for k, a in enumerate(local0)},
             **{f"p0_{k}": a for k, a in enumerate(local0)},
             **{f"p3_{k}": a for k, a in enumerate(local3)},
             **{f"g{t}_{k}": a for t, gl in enumerate(grads) for k, a in enumerate(gl)})
    dist.destroy_process_group()


@pytest.mark.parametrize("world", [2, 4])
def test_fsdp2_local_shards(world, tmp_path):
    import oracle
    mp.spawn(_worker, args=(world, _free_port(), str(tmp_path)), nprocs=world, join=True)
    shapes = [tuple(p.shape) for p in _make_model().parameters()]
    for r in range(world):
        z = np.load(tmp_path / f"rank{r}.npz")
        for k, shp in enumerate(shapes):
            first, rows = oracle.dim0_split(shp[0], world, r)
            want = (rows,) + tuple(shp[1:])
            assert tuple(z[f"s{k}"]) == want, (world, r, k)
    # FSDP2 hands each rank its reduced (averaged) local gradient rows; the
    # oracle's per-parameter shard step on those rows must track FSDP2's own
    # torch.optim.Adam on the shards within the page's 1e-5 after 3 steps.
    for r in range(world):
        z = np.load(tmp_path / f"rank{r}.npz")
        for k, shp in enumerate(shapes):
            if z[f"p0_{k}"].size == 0:
                continue
            o = oracle.ShardOracle(z[f"p0_{k}"].size, 1, 0, 1e-2, n_replicas=1)
            o.load_master(np.ascontiguousarray(z[f"p0_{k}"].reshape(-1)))
            out = np.zeros(o.shard, np.float32)
            for t in range(3):
                g = np.ascontiguousarray(z[f"g{t}_{k}"].reshape(-1).astype(np.float32))
                o.step([g], t + 1, out, grad_offset=0, out_offset=0)
            diff = np.abs(out - z[f"p3_{k}"].reshape(-1)).max()
            assert diff < 1e-5, (world, r, k, diff)
