"""The page's 4-process experiment with real collectives (gloo, CPU), the
oracle doing each rank's shard step.

Each of 4 processes builds the page's MLP, computes the gradient of its
quarter of the batch, and then:
  * ZeroAdam as the page writes it in torch: reduce_scatter_tensor (SUM),
    divide by world, Adam on the slice, all_gather_into_tensor;
  * the oracle: all_gather of every rank's flat gradient (the N replicas),
    ShardOracle.step for this rank's slice, all_gather of the updated
    slices.
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

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _free_port():
    with socket.socket() as s:
        s.bind(("127.0.0.1", 0))
        return s.getsockname()[1]


def _make_model():
    torch.manual_seed(0)
    return torch.nn.Sequential(torch.nn.Linear(64, 256), torch.nn.GELU(),
                               torch.nn.Linear(256, 10))


class PageZeroAdam:
    """The page's ZeroAdam, restated in torch for the comparison."""

    def __init__(self, params, lr, betas=(0.9, 0.999), eps=1e-8):
        self.params = list(params)
        self.lr, self.betas, self.eps, self.t = lr, betas, eps, 0
        self.rank, self.world = dist.get_rank(), dist.get_world_size()
        self.numel = sum(p.numel() for p in self.params)
        self.shard = math.ceil(self.numel / self.world)
        flat = self._flatten([p.data for p in self.params])
        lo = self.rank * self.shard
        self.master = flat[lo:lo + self.shard].clone()
        self.m = torch.zeros_like(self.master)
        self.v = torch.zeros_like(self.master)

    def _flatten(self, tensors):
        flat = torch.zeros(self.shard * self.world)
        flat[:self.numel] = torch.cat([t.flatten() for t in tensors])
        return flat

    def step(self):
        grads = self._flatten([p.grad for p in self.params])
        g = torch.empty(self.shard)
        dist.reduce_scatter_tensor(g, grads)
        g /= self.world
        self.t += 1
        b1, b2 = self.betas
        self.m.mul_(b1).add_(g, alpha=1 - b1)
        self.v.mul_(b2).addcmul_(g, g, value=1 - b2)
        m_hat = self.m / (1 - b1 ** self.t)
        v_hat = self.v / (1 - b2 ** self.t)
        self.master -= self.lr * m_hat / (v_hat.sqrt() + self.eps)
        full = torch.empty(self.shard * self.world)
        dist.all_gather_into_tensor(full, self.master)
        offset = 0
        for p in self.params:
            p.data.copy_(full[offset:offset + p.numel()].view_as(p))
            offset += p.numel()


def _worker(rank, world, port, outdir):
    os.environ.update(MASTER_ADDR="127.0.0.1", MASTER_PORT=str(port))
    sys.path.insert(0, ROOT)
    import oracle
    dist.init_process_group("gloo", rank=rank, world_size=world)
    torch.manual_seed(123)
    X, Y = torch.randn(32, 64), torch.randint(0, 10, (32,))
    sl = slice(rank * 32 // world, (rank + 1) * 32 // world)
    loss_fn = torch.nn.CrossEntropyLoss()
    ref, page_model, orc_model = _make_model(), _make_model(), _make_model()
    opt_ref = torch.optim.Adam(ref.parameters(), lr=1e-2)
    opt_page = PageZeroAdam(page_model.parameters(), lr=1e-2)
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
        for p in page_model.parameters():
            p.grad = None
        loss_fn(page_model(X[sl]), Y[sl]).backward()
        opt_page.step()
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
    d_page = max(float((a - b).detach().abs().max()) for a, b in
                 zip(ref.parameters(), page_model.parameters()))
    d_orc = max(float((a - b).detach().abs().max()) for a, b in
                zip(ref.parameters(), orc_model.parameters()))
    d_po = max(float((a - b).detach().abs().max()) for a, b in
               zip(page_model.parameters(), orc_model.parameters()))
    np.save(os.path.join(outdir, f"r{rank}.npy"),
            np.array([d_page, d_orc, d_po, float(bitexact)]))
    dist.destroy_process_group()


def test_page_four_process_experiment(tmp_path):
    world = 4
    mp.spawn(_worker, args=(world, _free_port(), str(tmp_path)), nprocs=world, join=True)
    for r in range(world):
        d_page, d_orc, d_po, bitexact = np.load(tmp_path / f"r{r}.npy")
        assert d_page < 1e-5, d_page           # the page's own claim
        assert d_orc < 1e-5, d_orc             # the oracle, sharded over 4 processes
        assert d_po < 1e-6, d_po               # oracle vs the page's torch ZeroAdam
        assert bitexact == 1.0                 # shards reassemble the unsharded update
