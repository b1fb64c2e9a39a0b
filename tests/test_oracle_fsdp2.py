"""The per-parameter dim-0 layout ([ZF] "ZeRO-3 and FSDP") against FSDP2
itself, on the CPU with the gloo backend: the local shard shapes FSDP2
assigns, and 3 Adam steps of FSDP2's own optimizer on those pieces against
the oracle's shard step on the same reduced gradients (the page's 1e-5)."""
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


def _local(t):
    """This rank's dim-0 piece of an FSDP2 parameter or gradient (a DTensor)."""
    return t.to_local().detach().clone().numpy()


def _worker(rank, world, port, outdir):
    """Shard the model with FSDP2 (one group at the root: the per-parameter
    dim-0 layout does not depend on the grouping), run 3 steps of its own
    Adam on this rank's quarter of the batch, and save the local pieces:
    shapes, initial values, the reduced gradients and the final values."""
    os.environ.update(MASTER_ADDR="127.0.0.1", MASTER_PORT=str(port))
    from torch.distributed.device_mesh import init_device_mesh
    from torch.distributed.fsdp import fully_shard
    dist.init_process_group("gloo", rank=rank, world_size=world)
    model = fully_shard(_make_model(), mesh=init_device_mesh("cpu", (world,)))
    head = torch.nn.Linear(5, 10)
    torch.manual_seed(123)
    X, Y = torch.randn(32, 64), torch.randint(0, 10, (32,))
    rows = slice(rank * 32 // world, (rank + 1) * 32 // world)
    params = list(model.parameters())
    opt = torch.optim.Adam(params, lr=1e-2, foreach=False)
    saved = {f"s{k}": np.array(p.to_local().shape) for k, p in enumerate(params)}
    saved.update({f"p0_{k}": _local(p) for k, p in enumerate(params)})
    for t in range(3):
        opt.zero_grad()
        torch.nn.functional.cross_entropy(head(model(X[rows])), Y[rows]).backward()
        saved.update({f"g{t}_{k}": _local(p.grad) for k, p in enumerate(params)})
        opt.step()
    saved.update({f"p3_{k}": _local(p) for k, p in enumerate(params)})
    np.savez(os.path.join(outdir, f"rank{rank}.npz"), **saved)
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
