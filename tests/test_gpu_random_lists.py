"""Seeded random tensor lists through flatten, windowed flatten and
unflatten, against the oracle.

Each case draws a list of ragged shapes (empty tensors and single elements
included, sometimes more than one launch's worth of segments), the element
type, the world size (so the pad varies), an element offset for the source
pool and one for the destination flat buffer (every 16-byte and 128-byte
phase relation between them), and a random tiling of the padded vector
into windows. The flat vector equals the oracle's flatten byte for byte,
the windows on two streams give the same bytes, unflatten into views at
another offset gives the sources back, and guard elements around every
destination keep their sentinel bits."""
import numpy as np
import pytest
import torch

import oracle
import zero_partitioned_optimizer_flatten_amd as zero
from gpu_harness import bits, log

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    assert torch.cuda.is_available()
    zero.lib()
    yield
    torch.cuda.synchronize()


def _shapes(rng):
    count = int(rng.choice([1, 3, 17, 70, 150]))
    out = []
    for _ in range(count):
        r = rng.random()
        if r < 0.1:
            out.append((0,) if rng.random() < 0.5 else (int(rng.integers(1, 4)), 0))
        elif r < 0.2:
            out.append((1,))
        elif r < 0.7:
            out.append((int(rng.integers(1, 3000)),))
        else:
            out.append((int(rng.integers(1, 200)), int(rng.integers(1, 300))))
    if sum(int(np.prod(s)) for s in out) == 0:
        out.append((5,))
    return out


@pytest.mark.parametrize("case", range(32))
def test_random_list(case):
    rng = np.random.default_rng(30_000 + case)
    dev = torch.device("cuda")
    dt = torch.bfloat16 if rng.random() < 0.6 else torch.float32
    ity, nty = (torch.int16, np.int16) if dt == torch.bfloat16 else (torch.int32, np.int32)
    shapes = _shapes(rng)
    sizes = [int(np.prod(s)) for s in shapes]
    numel = sum(sizes)
    world = int(rng.choice([1, 2, 3, 8, 13]))
    st = zero.ShardState(numel, world, int(rng.integers(0, world)), 1e-3)
    P = st.padded
    a = int(rng.integers(0, 64))          # source pool offset (elements)
    b = int(rng.integers(0, 64))          # destination offset (elements)
    log(f"case {case}: {len(shapes)} tensors, numel {numel}, P {P}, {dt}, offsets {a}/{b}")

    pool = torch.randint(-30000, 30000, (numel + 64,), dtype=torch.int32, device=dev)
    pool = pool.to(ity).view(dt) if dt == torch.bfloat16 else pool.view(dt)
    srcs, off = [], a
    for s, k in zip(shapes, sizes):
        srcs.append(pool[off:off + k].view(s))
        off += k
    src_bits = [bits(x).reshape(-1) for x in srcs]
    want = oracle.flatten(src_bits, P, fill=0x5A)

    buf = torch.full((P + 128,), -1, dtype=ity, device=dev).view(dt)
    st.flatten(srcs, buf[b:b + P])
    got = bits(buf)
    assert got[b:b + P].tobytes() == want.tobytes(), f"case {case}: flatten"
    assert (np.concatenate([got[:b], got[b + P:]]).view(nty) == -1).all(), f"case {case}: guard"

    # random tiling into windows, alternating between two streams
    cuts = sorted(set(int(c) for c in rng.integers(0, P + 1, size=int(rng.integers(1, 6)))))
    bounds = [0] + [c for c in cuts if 0 < c < P] + [P]
    win = torch.full((P + 128,), -1, dtype=ity, device=dev).view(dt)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    cur = torch.cuda.current_stream()
    for s in streams:
        s.wait_stream(cur)
    for i, (lo, hi) in enumerate(zip(bounds[:-1], bounds[1:])):
        st.flatten(srcs, win[b:b + P], stream=streams[i % 2], window=(lo, hi - lo))
    for s in streams:
        cur.wait_stream(s)
    assert bits(win)[b:b + P].tobytes() == want.tobytes(), f"case {case}: windows {bounds}"

    # unflatten into views at another offset of a guarded buffer
    c = int(rng.integers(0, 64))
    back = torch.full((numel + 128,), -1, dtype=ity, device=dev).view(dt)
    dsts, off = [], c
    for s, k in zip(shapes, sizes):
        dsts.append(back[off:off + k].view(s))
        off += k
    st.unflatten(buf[b:b + P], dsts)
    bb = bits(back)
    assert bb[c:c + numel].tobytes() == np.concatenate(src_bits).tobytes(), f"case {case}: unflatten"
    assert (np.concatenate([bb[:c], bb[c + numel:]]).view(nty) == -1).all(), f"case {case}: guard"
    for d, ref in zip(dsts, oracle.unflatten(want, shapes)):
        assert bits(d).tobytes() == ref.tobytes(), f"case {case}: unflatten vs oracle"
    st.close()
