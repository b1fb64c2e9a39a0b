"""Correct rounding of the fused step's square root and division, checked
through the kernel itself over every non-negative binary32 pattern.

With beta1 = beta2 = 1/2, eps = 0, lr = 1, t = 1 and a zero gradient, the
step computes, exactly up to its roundings,
    m' = m/2,  v' = v/2,  m_hat = m'/(1/2),  v_hat = v'/(1/2),
    master' = master - (1 * m_hat) / sqrt(v_hat),
so with master = 0 and v set to each pattern (through zero_set_state) the
result is -RN(m / RN(sqrt(v))) for normal v, and the same operation
sequence for the rest. Both the kernel and the CPU oracle run it on all
2^31 patterns 0x00000000..0x7FFFFFFF (zero, subnormals, normals, +inf,
NaNs), with m = 1 and with random m; results must agree bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import zero_partitioned_optimizer_flatten_amd as zero
from gpu_harness import log

pytestmark = pytest.mark.gpu

CHUNK = 1 << 27


@pytest.fixture(autouse=True)
def _gpu():
    assert torch.cuda.is_available()
    zero.lib()
    torch.cuda.empty_cache()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("m_kind", ["one", "random"])
def test_sqrt_and_divide_all_nonnegative_patterns(m_kind):
    dev = torch.device("cuda")
    lr, betas, eps = 1.0, (0.5, 0.5), 0.0
    st = zero.ShardState(CHUNK, 1, 0, lr, betas, eps)
    grad = torch.zeros(CHUNK, dtype=torch.float32, device=dev)
    out = torch.empty(CHUNK, dtype=torch.float32, device=dev)
    zeros = torch.zeros(CHUNK, dtype=torch.float32, device=dev)
    gen = torch.Generator(device=dev).manual_seed(5)
    orc = oracle.ShardOracle(CHUNK, 1, 0, lr, betas, eps)
    grad_h = np.zeros(CHUNK, np.float32)
    out_h = np.empty(CHUNK, np.float32)
    mismatches = 0
    for c in range(1 << 31 >> 27):
        v = torch.arange(c * CHUNK, (c + 1) * CHUNK, dtype=torch.int64, device=dev).to(torch.int32)
        v = v.view(torch.float32)
        if m_kind == "one":
            m = torch.ones(CHUNK, dtype=torch.float32, device=dev)
        else:
            m = (torch.rand(CHUNK, generator=gen, device=dev) * 2 - 1) * 10.0 ** (
                torch.randint(-30, 30, (CHUNK,), generator=gen, device=dev).float())
        st.set_state(zeros, m, v)
        st.step([grad], 1, out)
        torch.cuda.synchronize()
        got = [x.cpu().numpy() for x in st.get_state()]
        orc.master[:] = 0.0
        orc.m[:] = m.cpu().numpy()
        orc.v[:] = v.cpu().numpy()
        orc.step([grad_h], 1, out_h, grad_offset=0, out_offset=0)
        for g, r in zip(got, (orc.master, orc.m, orc.v)):
            d = g.view(np.uint32) != r.view(np.uint32)
            both_nan = np.isnan(g) & np.isnan(r)
            mismatches += int(np.count_nonzero(d & ~both_nan))
        log(f"exhaustive {m_kind}: chunk {c + 1}/16, mismatches so far {mismatches}")
    assert mismatches == 0
    st.close()
