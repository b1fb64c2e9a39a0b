"""Pins for the CPU oracle: each check ties one oracle function to something
other than the oracle itself (the pages' worked example, closed forms,
brute force, invariants, or a library routine).

Every check is a plain function that raises AssertionError on failure, so
`test_oracle_pins.py` runs them and `test_oracle_mutants.py` re-runs them
against deliberately broken builds of the oracle to show that a plausible
mistake is caught.
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _bf16_bits(x: torch.Tensor) -> np.ndarray:
    return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def _f32_from_bits(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


# ============================================================== geometry

def check_geometry_bruteforce():
    """shard = smallest s with s*world >= numel; the rest by counting."""
    for numel in range(1, 201):
        for world in range(1, 10):
            s = 1
            while s * world < numel:
                s += 1
            for rank in range(world):
                g = oracle.geometry(numel, world, rank)
                lo = rank * s
                valid = sum(1 for k in range(lo, lo + s) if k < numel)
                assert g == dict(shard=s, lo=lo, padded=s * world,
                                 pad=s * world - numel, valid=valid), \
                    (numel, world, rank, g)


def check_geometry_large():
    """int64 sizes of the named workloads (Psi up to 7e10)."""
    cases = [  # numel, world, rank -> shard, lo, pad, valid
        (1_000_003, 4, 3, 250_001, 750_003, 1, 250_000),
        (124_439_808, 8, 3, 15_554_976, 46_664_928, 0, 15_554_976),
        (7_000_000_000, 8, 0, 875_000_000, 0, 0, 875_000_000),
        (13_015_864_321, 8, 7, 1_626_983_041, 11_388_881_287, 7,
         1_626_983_034),
        (70_000_000_000, 64, 0, 1_093_750_000, 0, 0, 1_093_750_000),
    ]
    for numel, world, rank, s, lo, pad, valid in cases:
        # exact integer ceiling by Fraction, independent of the oracle
        assert s == math.ceil(Fraction(numel, world))
        g = oracle.geometry(numel, world, rank)
        assert (g["shard"], g["lo"], g["pad"], g["valid"]) == (s, lo, pad, valid), g


def check_geometry_toy_state_bytes():
    """The page's own test model on 4 ranks: per-rank optimizer state versus
    the unsharded count, which the page prints as 1/round(ratio)."""
    gold = _golden("toy_model.json")
    torch.manual_seed(0)
    model = torch.nn.Sequential(torch.nn.Linear(64, 256), torch.nn.GELU(),
                                torch.nn.Linear(256, 10))
    numel = sum(p.numel() for p in model.parameters())
    world = gold["world"]
    g = oracle.geometry(numel, world, 0)
    # the page's state_bytes: numel * element_size summed over master, m, v
    tensors = [torch.zeros(g["shard"]) for _ in range(3)]
    page_bytes = sum(t.numel() * t.element_size() for t in tensors)
    assert oracle.state_bytes(g["shard"]) == page_bytes
    full = 3 * numel * 4
    assert round(full / oracle.state_bytes(g["shard"])) == gold["expected_round_ratio"]


# =========================================================== stage bytes

def check_stage_bytes_worked_example():
    gold = _golden("stage_bytes_worked_example.json")
    psi, n, unit = gold["psi"], gold["n"], gold["gb_unit_bytes"]
    for k, stage in (("zero1", 1), ("zero2", 2), ("zero3", 3)):
        got = oracle.stage_bytes(stage, psi, n) / unit
        dec = gold["printed_decimals"][k]
        assert round(got, dec) == gold["printed_gb"][k], (k, got)
    # the answer's intermediate terms: unpartitioned part + partitioned part
    z1 = oracle.stage_bytes(1, psi, n) / unit
    z2 = oracle.stage_bytes(2, psi, n) / unit
    assert abs(z1 - sum(gold["printed_terms_gb"]["zero1"])) < 1e-9
    assert abs(z2 - 26.0 - 11.375) < 1e-9 and round(11.375, 1) == 11.4


def check_stage_bytes_components():
    """Each stage = sum over components of bytes/param, divided by N for the
    components that stage partitions."""
    gold = _golden("state_components.json")
    bpp = gold["bytes_per_param"]
    assert sum(bpp.values()) == 16
    assert sum(bpp[c] for c in gold["optimizer_components"]) == 12
    rng = np.random.default_rng(5)
    for _ in range(200):
        psi = float(rng.integers(1, 10**12))
        n = float(rng.integers(1, 4097))
        for stage in range(4):
            parts = gold["partitioned"][str(stage)]
            want = sum(Fraction(b) * Fraction(int(psi)) / (int(n) if c in parts else 1)
                       for c, b in bpp.items())
            got = oracle.stage_bytes(stage, psi, n)
            assert abs(got - float(want)) <= 1e-12 * float(want), (stage, psi, n)


def check_reduction_factors():
    gold = _golden("reduction_factors.json")
    psi = 7e9
    dp = oracle.stage_bytes(0, psi, 8)
    for k, stage in (("zero1", 1), ("zero2", 2)):
        big = dp / oracle.stage_bytes(stage, psi, 1e15)
        assert abs(big - gold["large_n_limits"][k]) < 1e-9, (k, big)
    # optimizer states alone at N = 8: (ZeRO-1 bytes minus its unsplit 4 psi)
    ex = gold["optimizer_only_example"]
    opt_split = oracle.stage_bytes(1, psi, ex["n"]) - 4 * psi
    assert abs(12 * psi / opt_split - ex["factor"]) < 1e-9
    # no saving at N = 1; strictly ordered savings for N > 1
    for stage in range(4):
        assert oracle.stage_bytes(stage, psi, 1) == 16 * psi
    for n in (2, 8, 64):
        vals = [oracle.stage_bytes(s, psi, n) for s in range(4)]
        assert vals[0] > vals[1] > vals[2] > vals[3]


# =============================================================== flatten

def _ragged(rng, count, maxn):
    return [int(rng.integers(1, maxn + 1)) for _ in range(count)]


def check_flatten_vs_torch_cat():
    """Library routine: torch.cat of the flattened tensors + a zero tail,
    compared byte for byte, for fp32 and bf16 lists with odd sizes."""
    rng = np.random.default_rng(11)
    for dtype in (torch.float32, torch.bfloat16):
        for trial in range(6):
            sizes = _ragged(rng, int(rng.integers(1, 40)), 3000)
            gen = torch.Generator().manual_seed(trial)
            ts = [torch.randn(s, generator=gen).to(dtype) for s in sizes]
            ts[0] = ts[0].reshape(1, -1)        # shapes do not matter
            numel = sum(sizes)
            padded = numel + int(rng.integers(0, 9))
            ref = torch.cat([t.flatten() for t in ts] +
                            [torch.zeros(padded - numel, dtype=dtype)])
            if dtype == torch.bfloat16:
                arrs = [t.view(torch.int16).numpy().view(np.uint16) for t in ts]
                want = ref.view(torch.int16).numpy().view(np.uint16)
            else:
                arrs = [t.numpy() for t in ts]
                want = ref.numpy()
            got = oracle.flatten(arrs, padded, fill=0xAB)
            assert got.tobytes() == want.tobytes(), (dtype, trial)


def check_flatten_bruteforce():
    """Tiny lists against an element-by-element loop."""
    rng = np.random.default_rng(3)
    for _ in range(50):
        sizes = _ragged(rng, int(rng.integers(1, 6)), 7)
        arrs = [rng.standard_normal(s).astype(np.float32) for s in sizes]
        numel = sum(sizes)
        padded = numel + int(rng.integers(0, 4))
        want = []
        for a in arrs:
            for x in a:
                want.append(x)
        while len(want) < padded:
            want.append(np.float32(0))
        got = oracle.flatten(arrs, padded, fill=0xCD)
        assert np.array_equal(got.view(np.uint32),
                              np.array(want, dtype=np.float32).view(np.uint32))


def check_unflatten_roundtrip():
    rng = np.random.default_rng(4)
    shapes = [(3, 5), (7,), (1,), (2, 2, 3), (11,)]
    arrs = [rng.standard_normal(s).astype(np.float32) for s in shapes]
    numel = sum(a.size for a in arrs)
    flat = oracle.flatten(arrs, numel + 5)
    back = oracle.unflatten(flat, shapes)
    for a, b in zip(arrs, back):
        assert a.shape == b.shape and a.tobytes() == b.tobytes()


def check_flatten_rejects_overflow():
    try:
        oracle.flatten([np.zeros(5, np.float32)], 4)
    except ValueError:
        return
    raise AssertionError("flatten accepted a list longer than the padded length")


# ================================================================== bf16

def check_bf16_vs_torch():
    """Library routine: torch's float32 -> bfloat16 cast (round to nearest,
    ties to even) over every high half with the critical low halves, plus
    random patterns. NaN compared by NaN-ness only."""
    hi = np.arange(65536, dtype=np.uint32) << 16
    lows = np.array([0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF], dtype=np.uint32)
    pats = (hi[:, None] | lows[None, :]).reshape(-1)
    rng = np.random.default_rng(9)
    pats = np.concatenate([pats, rng.integers(0, 2**32, 500_000,
                                              dtype=np.uint64).astype(np.uint32)])
    x = pats.view(np.float32)
    got = oracle.bf16_round(x)
    want = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    isnan = np.isnan(x)
    assert np.array_equal(got[~isnan], want[~isnan])
    gnan = _f32_from_bits(got[isnan])
    assert np.all(np.isnan(gnan))
    # quiet bit set, sign kept
    assert np.all(got[isnan] & 0x0040)
    assert np.array_equal(got[isnan] >> 15, (pats[isnan] >> 31).astype(np.uint16))


def check_bf16_specials():
    cases = [  # (value, expected bf16 bits)
        (0.0, 0x0000), (-0.0, 0x8000), (1.0, 0x3F80), (-2.0, 0xC000),
        (float("inf"), 0x7F80), (float("-inf"), 0xFF80),
        (1.0 + 2**-8, 0x3F80),          # exact tie, even stays
        (1.0 + 3 * 2**-8, 0x3F82),      # tie, odd rounds up
        (3.4e38, 0x7F80),               # past the largest bf16
        (-3.4e38, 0xFF80),
        (2**-133, 0x0001),              # smallest bf16 subnormal
        (2**-134, 0x0000),              # subnormal tie to even (zero)
        (3 * 2**-134, 0x0002),          # subnormal tie, odd rounds up
    ]
    for val, bits in cases:
        got = int(oracle.bf16_round(np.array([val], np.float32))[0])
        assert got == bits, (val, hex(got), hex(bits))


# ================================================================ reduce

def check_reduce_identity_n1():
    rng = np.random.default_rng(0)
    for dt in ("f32", "bf16"):
        x = rng.standard_normal(1000).astype(np.float32)
        rep = _bf16_bits(torch.from_numpy(x)) if dt == "bf16" else x
        g = oracle.reduce_mean([rep], 0, 1000, 1)
        want = _f32_from_bits(rep) if dt == "bf16" else x
        assert np.array_equal(g.view(np.uint32), want.view(np.uint32))


def check_reduce_identical_replicas():
    """N identical bf16 replicas average back to the replica exactly: k*x is
    exact in fp32 for an 8-bit significand and k <= 2^16, and (k*x)/k = x."""
    rng = np.random.default_rng(1)
    x = _bf16_bits(torch.from_numpy(rng.standard_normal(4096).astype(np.float32)))
    for n in (2, 3, 4, 5, 7, 8, 16, 64):
        g = oracle.reduce_mean([x] * n, 0, x.size, n)
        assert np.array_equal(g.view(np.uint32), _f32_from_bits(x).view(np.uint32)), n


def check_reduce_rank_order():
    """Left fold over ranks 0..N-1: 1 + 2^-24 rounds back to 1 at every
    step, so the mean is exactly 1/4; any other order gives more."""
    reps = [np.array([v], np.float32) for v in (1.0, 2**-24, 2**-24, 2**-24)]
    g = oracle.reduce_mean(reps, 0, 1, 4)
    assert g[0] == np.float32(0.25), g
    reps = reps[::-1]
    g = oracle.reduce_mean(reps, 0, 1, 4)
    assert g[0] == np.float32((1.0 + 2**-22) / 4), g


def check_reduce_error_bound():
    """Random replicas: the fp32 left fold stays within (N-1) u sum|g_q| of
    the exact sum (u = 2^-24), and the division adds at most half an ulp."""
    rng = np.random.default_rng(2)
    for n in (3, 8, 64):
        for dt in ("f32", "bf16"):
            xs = [rng.standard_normal(5000).astype(np.float32) * 10 ** rng.uniform(-3, 3)
                  for _ in range(n)]
            reps = [_bf16_bits(torch.from_numpy(x)) if dt == "bf16" else x for x in xs]
            vals = [(_f32_from_bits(r) if dt == "bf16" else r).astype(np.float64) for r in reps]
            exact = np.sum(vals, axis=0) / n
            bound = (n - 1) * 2.0**-24 * np.sum(np.abs(vals), axis=0) / n \
                + np.abs(exact) * 2.0**-23 + 1e-45
            g = oracle.reduce_mean(reps, 0, 5000, n).astype(np.float64)
            assert np.all(np.abs(g - exact) <= bound), (n, dt)


def check_reduce_offset():
    rng = np.random.default_rng(8)
    reps = [rng.standard_normal(100).astype(np.float32) for _ in range(3)]
    g_off = oracle.reduce_mean(reps, 37, 50, 3)
    g_cut = oracle.reduce_mean([np.ascontiguousarray(r[37:87]) for r in reps], 0, 50, 3)
    assert np.array_equal(g_off, g_cut)


# ================================================================== adam

def _run_oracle_steps(grads_per_step, master0, lr, b1, b2, eps, world=1):
    """Drive the oracle's shard step with one replica per rank on a single
    shard covering everything; returns master, m, v after each step."""
    n = master0.size
    o = oracle.ShardOracle(n, 1, 0, lr, (b1, b2), eps)
    o.load_master(master0)
    out = np.zeros(n, np.float32)
    hist = []
    for t, g in enumerate(grads_per_step, start=1):
        o.step([np.ascontiguousarray(g, np.float32)], t, out)
        hist.append((o.master.copy(), o.m.copy(), o.v.copy(), out.copy()))
    return hist


def check_adam_dyadic_exact():
    """b1 = 1/2, b2 = 3/4, eps = 0, lr = 2^-4 and g = +-2^k make every
    intermediate exact: m_hat = g, v_hat = g^2, sqrt(v_hat) = |g|, so each
    step moves master by exactly -lr*sign(g)."""
    rng = np.random.default_rng(6)
    n = 64
    g = (np.where(rng.random(n) < 0.5, -1.0, 1.0) *
         2.0 ** rng.integers(-20, 10, n)).astype(np.float32)
    master0 = (rng.integers(-64, 64, n) / 4.0).astype(np.float32)
    lr = 2.0**-4
    hist = _run_oracle_steps([g] * 12, master0, lr, 0.5, 0.75, 0.0)
    for t, (master, m, v, out) in enumerate(hist, start=1):
        want = master0.astype(np.float64) - t * lr * np.sign(g)
        assert np.array_equal(master.astype(np.float64), want), t
        assert np.array_equal(m.astype(np.float64), g * (1 - 0.5**t)), t
        assert np.array_equal(v.astype(np.float64),
                              g.astype(np.float64)**2 * (1 - 0.75**t)), t
        assert np.array_equal(out, master)


def check_adam_step1_sign():
    """Step 1 with b1 = 1/2, b2 = 3/4, eps = 0 and lr = 2^-k: for any g the
    update is exactly lr*sign(g) (sqrt of a correctly rounded square gives
    |g| back), so master_1 = RN(master_0 - lr*sign(g))."""
    rng = np.random.default_rng(12)
    g = (rng.standard_normal(10000) * 10 ** rng.uniform(-6, 3, 10000)).astype(np.float32)
    master0 = rng.standard_normal(10000).astype(np.float32)
    lr = np.float32(2.0**-7)
    (master, m, v, out), = _run_oracle_steps([g], master0, float(lr), 0.5, 0.75, 0.0)
    want = master0 - np.float32(lr) * np.sign(g).astype(np.float32)
    assert np.array_equal(master, want)


def _closed_form(gs, master0, lr, b1, b2, eps):
    """Unrolled recurrences in float64: m_t = (1-b1) sum_k b1^(t-k) g_k,
    v_t = (1-b2) sum_k b2^(t-k) g_k^2, and the running master."""
    T = len(gs)
    gs = [g.astype(np.float64) for g in gs]
    out = []
    master = master0.astype(np.float64).copy()
    for t in range(1, T + 1):
        m = (1 - b1) * sum(b1 ** (t - k) * gs[k - 1] for k in range(1, t + 1))
        v = (1 - b2) * sum(b2 ** (t - k) * gs[k - 1] ** 2 for k in range(1, t + 1))
        mabs = (1 - b1) * sum(b1 ** (t - k) * np.abs(gs[k - 1]) for k in range(1, t + 1))
        mh = m / (1 - b1 ** t)
        vh = v / (1 - b2 ** t)
        u = lr * mh / (np.sqrt(vh) + eps)
        master = master - u
        out.append((master.copy(), m, v, mabs, vh))
    return out


def check_adam_closed_form_random():
    """Random gradients for 10 steps against the unrolled closed forms, with
    error bounds from fp32 rounding. eps is comparable to |g| so its
    placement (outside the root, after bias correction) matters."""
    rng = np.random.default_rng(7)
    n = 20000
    lr, b1, b2, eps = 1e-3, 0.9, 0.999, 1e-3
    gs = [(rng.standard_normal(n) * 1e-3).astype(np.float32) for _ in range(10)]
    master0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    hist = _run_oracle_steps(gs, master0, lr, b1, b2, eps)
    cf = _closed_form(gs, master0, lr, b1, b2, eps)
    u = 2.0**-24
    for t, ((master, m, v, _), (cm, mm, vv, mabs, vh)) in enumerate(zip(hist, cf), start=1):
        # each recurrence step adds <= ~3u relative error on its terms
        assert np.all(np.abs(m - mm) <= 4 * t * u * mabs + 1e-30), t
        assert np.all(np.abs(v - vv) <= 4 * t * u * vv + 1e-30), t
        # master: per-step update error is bounded by lr times the m error
        # scaled by the denominator, plus rounding of master itself
        den = np.sqrt(vh) + eps
        step_err = lr * (8 * t * u * mabs / (1 - b1 ** t)) / den
        assert np.all(np.abs(master - cm) <= t * (step_err + 2 * u * np.abs(cm)) + 1e-12), t


def check_adam_constant_gradient():
    """Constant g: m_hat = g and v_hat = g^2 exactly in real arithmetic, so
    master_t = master_0 - t*lr*g/(|g| + eps)."""
    rng = np.random.default_rng(13)
    n = 5000
    g = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    master0 = rng.standard_normal(n).astype(np.float32)
    lr, eps = 1e-3, 1e-5
    hist = _run_oracle_steps([g] * 10, master0, lr, 0.9, 0.999, eps)
    for t, (master, *_rest) in enumerate(hist, start=1):
        g64 = g.astype(np.float64)
        want = master0 - t * lr * g64 / (np.abs(g64) + eps)
        assert np.all(np.abs(master - want) <= t * (1e-6 * lr + 2**-23 * np.abs(want))), t


def check_adam_step1_bounded():
    """Step 1: |u| = lr*|g|/(|g|+eps) < lr in exact arithmetic."""
    rng = np.random.default_rng(14)
    g = (rng.standard_normal(100000) * 10 ** rng.uniform(-9, 4, 100000)).astype(np.float32)
    master0 = np.zeros(100000, np.float32)
    lr = 1e-3
    (master, *_r), = _run_oracle_steps([g], master0, lr, 0.9, 0.999, 1e-8)
    assert np.all(np.abs(master) <= np.float32(lr) * (1 + 8 * 2.0**-24))
    assert np.all(np.sign(master) == -np.sign(g))


def check_adam_vs_torch_optim():
    """Library routine: torch.optim.Adam (fp32 CPU, single tensor path) on
    the unsharded averaged gradient. The page asserts a difference below
    1e-5 after 3 steps; both 3 and 10 steps are checked, plus a tight bound."""
    rng = np.random.default_rng(15)
    n, world = 30001, 4
    lr, betas, eps = 1e-3, (0.9, 0.999), 1e-8
    master0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    p = torch.nn.Parameter(torch.from_numpy(master0.copy()))
    opt = torch.optim.Adam([p], lr=lr, betas=betas, eps=eps, foreach=False)
    o = oracle.ShardOracle(n, 1, 0, lr, betas, eps, n_replicas=world)
    o.load_master(master0)
    out = np.zeros(n, np.float32)
    for t in range(1, 11):
        reps = [(rng.standard_normal(n) * 0.01).astype(np.float32) for _ in range(world)]
        g = oracle.reduce_mean(reps, 0, n, world)
        o.step(reps, t, out)
        p.grad = torch.from_numpy(g.copy())
        opt.step()
        diff = np.max(np.abs(p.detach().numpy() - o.master))
        if t == 3:
            assert diff < 1e-5, diff
        assert diff < 2e-8, (t, diff)


def torch_adam(master, m, v, g, t, lr, b1, b2, eps, root=torch.sqrt):
    """The Adam update of [ZF] "Implementing ZeRO's Adam from scratch"
    (ZeroAdam.step) as equations over torch CPU tensors, returning new
    (master, m, v):
        m <- b1*m + (1-b1)*g            torch's scaled add
        v <- b2*v + (1-b2)*g*g          torch's addcmul
        master <- master - lr * (m/(1-b1^t)) / (root(v/(1-b2^t)) + eps)
    with the bias corrections formed from Python floats, as the page does.
    `root` is the square root used (torch's own by default)."""
    m = torch.add(m * b1, g, alpha=1 - b1)
    v = torch.addcmul(v * b2, g, g, value=1 - b2)
    m_hat = m / (1 - b1 ** t)
    v_hat = v / (1 - b2 ** t)
    return master - lr * m_hat / (root(v_hat) + eps), m, v


def _sqrt_rn(x: torch.Tensor) -> torch.Tensor:
    """Correctly rounded binary32 square root: the root in binary64 (53 >=
    2*24 + 2 bits, so one rounding to binary32 is correct)."""
    return torch.from_numpy(np.sqrt(x.numpy().astype(np.float64)).astype(np.float32))


def check_adam_equations_in_torch():
    """The update equations evaluated by PyTorch on the CPU, against the
    oracle over 10 steps of 8 bf16 replicas. m and v must agree bit for bit
    (this fixes where the two fused multiply-adds sit). torch's CPU square
    root is not always correctly rounded, so master is compared twice:
    with a correctly rounded root (bit for bit) and with torch's own root
    (within a few ulp)."""
    rng = np.random.default_rng(16)
    n, world = 200003, 8
    lr, (b1, b2), eps = 1e-3, (0.9, 0.999), 1e-8
    master0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    o = oracle.ShardOracle(n, 1, 0, lr, (b1, b2), eps, n_replicas=world)
    o.load_master(master0)
    out = np.zeros(n, np.float32)
    zero_t = torch.zeros(n)
    cr = (torch.from_numpy(master0.copy()), zero_t, zero_t)      # (master, m, v)
    tq = cr
    for t in range(1, 11):
        reps = [_bf16_bits(torch.randn(n, generator=torch.Generator().manual_seed(100 * t + q)) * 1e-3)
                for q in range(world)]
        g_np = oracle.reduce_mean(reps, 0, n, world)
        o.step(reps, t, out)
        # the reduce-scatter's sum in fp32 in rank order, then the division
        g = torch.stack([torch.from_numpy(_f32_from_bits(r)) for r in reps])
        s_ = g[0].clone()
        for q in range(1, world):
            s_ = s_ + g[q]
        g = s_ / world
        assert np.array_equal(g.numpy().view(np.uint32), g_np.view(np.uint32))
        cr = torch_adam(*cr, g, t, lr, b1, b2, eps, root=_sqrt_rn)
        tq = torch_adam(*tq, g, t, lr, b1, b2, eps)
        assert np.array_equal(cr[1].numpy().view(np.uint32), o.m.view(np.uint32)), t
        assert np.array_equal(cr[2].numpy().view(np.uint32), o.v.view(np.uint32)), t
        assert np.array_equal(cr[0].numpy().view(np.uint32), o.master.view(np.uint32)), t
        # a 1-ulp root error moves u by ~lr * 2^-23; master may then round
        # the other way (one ulp of master)
        diff = np.abs(tq[0].numpy().astype(np.float64) - o.master)
        tol = t * (lr * 2.0**-21 + np.spacing(np.abs(o.master)).astype(np.float64))
        assert np.all(diff <= tol), (t, diff.max())
        assert np.array_equal(out.view(np.uint32), o.master.view(np.uint32))


def check_toy_model_four_ranks():
    """The toy experiment of [ZF] "Implementing ZeRO's Adam from scratch"
    (a 64-256-10 MLP, a batch of 32 split over 4 ranks, 3 steps), with the 4
    ranks simulated in one process: one ShardOracle per rank writing its fp32
    slice, against torch.optim.Adam on the full batch."""
    gold = _golden("toy_model.json")
    world, lr, steps = gold["world"], gold["lr"], gold["steps"]

    def make_model():
        torch.manual_seed(0)
        return torch.nn.Sequential(torch.nn.Linear(64, 256), torch.nn.GELU(),
                                   torch.nn.Linear(256, 10))
    torch.manual_seed(123)
    X, Y = torch.randn(32, 64), torch.randint(0, 10, (32,))
    loss_fn = torch.nn.CrossEntropyLoss()
    ref = make_model()
    opt_ref = torch.optim.Adam(ref.parameters(), lr=lr)
    models = [make_model() for _ in range(world)]
    params0 = [p.detach().numpy().copy() for p in models[0].parameters()]
    numel = sum(p.size for p in params0)
    geo = oracle.geometry(numel, world, 0)
    flat_p = oracle.flatten([p.reshape(-1) for p in params0], geo["padded"])
    shards = []
    for r in range(world):
        o = oracle.ShardOracle(numel, world, r, lr)
        o.load_master(flat_p)
        shards.append(o)
    shapes = [p.shape for p in params0]
    for t in range(1, steps + 1):
        opt_ref.zero_grad()
        loss_fn(ref(X), Y).backward()
        opt_ref.step()
        reps = []
        for r, mod in enumerate(models):
            mod.zero_grad()
            sl = slice(r * 32 // world, (r + 1) * 32 // world)
            loss_fn(mod(X[sl]), Y[sl]).backward()
            reps.append(oracle.flatten([p.grad.numpy().reshape(-1)
                                        for p in mod.parameters()], geo["padded"]))
        full = np.zeros(geo["padded"], np.float32)
        for o in shards:
            o.step(reps, t, full)          # each rank writes its own slice
        new = oracle.unflatten(full[:numel], shapes)
        for mod in models:
            with torch.no_grad():
                for p, w in zip(mod.parameters(), new):
                    p.copy_(torch.from_numpy(w))
    diff = max(float((a - b).detach().abs().max()) for a, b in
               zip(ref.parameters(), models[0].parameters()))
    assert diff < gold["max_abs_param_diff_below"], diff
    full_state = 3 * numel * 4
    assert round(full_state / oracle.state_bytes(geo["shard"])) == gold["expected_round_ratio"]


def _sharded_run(numel, world, steps, dt, seed):
    """Returns (concatenated shard results per step, unsharded results)."""
    rng = np.random.default_rng(seed)
    lr, betas, eps = 1e-3, (0.9, 0.999), 1e-8
    geo = oracle.geometry(numel, world, 0)
    P = geo["padded"]
    params = (rng.standard_normal(numel) * 0.02).astype(np.float32)
    flat_p = oracle.flatten([params], P)
    shards = []
    for r in range(world):
        o = oracle.ShardOracle(numel, world, r, lr, betas, eps)
        o.load_master(flat_p)
        shards.append(o)
    whole = oracle.ShardOracle(P, 1, 0, lr, betas, eps, n_replicas=world)
    whole.load_master(flat_p)
    res = []
    for t in range(1, steps + 1):
        reps = []
        for q in range(world):
            x = (rng.standard_normal(numel) * 0.01).astype(np.float32)
            if dt == "bf16":
                x = _bf16_bits(torch.from_numpy(x))
            reps.append(oracle.flatten([x], P))
        out_sh = np.full(P, 0xFFFF if dt == "bf16" else np.nan,
                         np.uint16 if dt == "bf16" else np.float32)
        out_wh = out_sh.copy()
        for o in shards:
            o.step(reps, t, out_sh)
        whole.step(reps, t, out_wh, grad_offset=0, out_offset=0)
        cat = [np.concatenate([getattr(o, k) for o in shards]) for k in ("master", "m", "v")]
        res.append((cat, out_sh, [whole.master.copy(), whole.m.copy(), whole.v.copy()], out_wh, geo))
    return res


def check_sharding_invariant():
    """Concatenating the N ranks' shard results equals one owner updating
    the whole padded vector with the averaged gradient, bit for bit; the
    pad elements stay exactly zero."""
    for numel, world in ((3, 8), (1, 4), (64, 8), (1001, 4), (100_003, 8)):
        for dt in ("f32", "bf16"):
            for cat, out_sh, wh, out_wh, geo in _sharded_run(numel, world, 4, dt, numel):
                for a, b in zip(cat, wh):
                    assert a.tobytes() == b.tobytes(), (numel, world, dt)
                assert out_sh.tobytes() == out_wh.tobytes()
                pad = slice(numel, geo["padded"])
                for a in cat:
                    assert not np.any(a[pad].view(np.uint32)), "pad not zero"
                assert not np.any(out_sh[pad].view(np.uint16 if dt == "bf16" else np.uint32))


def check_resume():
    """5 steps, copy state out and into a fresh shard, 5 more == 10 steps."""
    rng = np.random.default_rng(17)
    n, world = 10007, 4
    geo = oracle.geometry(n, world, 2)
    flat = oracle.flatten([(rng.standard_normal(n) * 0.02).astype(np.float32)], geo["padded"])
    gs = [[oracle.flatten([(rng.standard_normal(n) * 0.01).astype(np.float32)], geo["padded"])
           for _ in range(world)] for _ in range(10)]
    a = oracle.ShardOracle(n, world, 2, 1e-3)
    a.load_master(flat)
    out = np.zeros(geo["padded"], np.float32)
    for t in range(1, 11):
        a.step(gs[t - 1], t, out)
    b = oracle.ShardOracle(n, world, 2, 1e-3)
    b.load_master(flat)
    for t in range(1, 6):
        b.step(gs[t - 1], t, out)
    saved = [x.copy() for x in (b.master, b.m, b.v)]
    c = oracle.ShardOracle(n, world, 2, 1e-3)
    c.master[:], c.m[:], c.v[:] = saved
    for t in range(6, 11):
        c.step(gs[t - 1], t, out)
    for k in ("master", "m", "v"):
        assert getattr(a, k).tobytes() == getattr(c, k).tobytes()


def check_nonfinite_stays_local():
    """A NaN or Inf in one replica poisons that element only."""
    n, world = 1000, 4
    reps = [np.full(n, 0.001, np.float32) for _ in range(world)]
    reps[2][10] = np.nan
    reps[1][20] = np.inf
    o = oracle.ShardOracle(n, 1, 0, 1e-3, n_replicas=world)
    o.load_master(np.zeros(n, np.float32))
    out = np.zeros(n, np.float32)
    o.step(reps, 1, out, grad_offset=0, out_offset=0)
    bad = ~np.isfinite(o.master)
    assert set(np.nonzero(bad)[0]) == {10, 20}
    assert np.isnan(o.master[10]) and np.isnan(o.master[20])   # inf/inf in the update


# ======================================================= dim-0 layout

def check_dim0_split_vs_torch_chunk():
    """Library routine: torch.chunk along dim 0, with empty chunks for the
    ranks it leaves out (the way FSDP2 pads its shard list)."""
    for d0 in range(0, 41):
        for world in range(1, 10):
            chunks = torch.chunk(torch.arange(d0), world, dim=0)
            rows = [int(c.numel()) for c in chunks] + [0] * (world - len(chunks))
            first = 0
            for r in range(world):
                f, n = oracle.dim0_split(d0, world, r)
                assert n == rows[r], (d0, world, r)
                if n:
                    assert f == first, (d0, world, r)
                first += n


def check_dim0_split_page_example():
    gold = _golden("fsdp2_rows.json")
    d0 = gold["weight_shape"][0]
    for r in range(gold["world"]):
        assert oracle.dim0_split(d0, gold["world"], r)[1] == gold["local_rows"]


def check_fsdp_layout_equals_whole_update():
    """Every rank's dim-0 shards of every parameter, put back in row order,
    equal the update of whole parameters, bit for bit (ragged shapes,
    ranks with no rows)."""
    rng = np.random.default_rng(21)
    shapes = [(10, 7), (5,), (1, 3), (13, 2, 2), (3, 4)]
    world = 4
    params = [(rng.standard_normal(s) * 0.02).astype(np.float32) for s in shapes]
    ranks = [oracle.FsdpShardOracle(shapes, world, r, 1e-3) for r in range(world)]
    for o in ranks:
        o.load_master(params)
    whole = [oracle.ShardOracle(int(np.prod(s)), 1, 0, 1e-3, n_replicas=world) for s in shapes]
    for w, p in zip(whole, params):
        w.load_master(p.reshape(-1))
    for t in range(1, 4):
        grads = [[(rng.standard_normal(s) * 1e-2).astype(np.float32) for s in shapes]
                 for _ in range(world)]
        outs = [[np.zeros(n, np.float32) for n in o.local_numels()] for o in ranks]
        for o, out in zip(ranks, outs):
            o.step(grads, t, out)
        for k, w in enumerate(whole):
            w.step([grads[q][k].reshape(-1) for q in range(world)], t,
                   np.zeros(w.shard, np.float32), grad_offset=0, out_offset=0)
            got = np.concatenate([outs[r][k] for r in range(world)])
            assert got.tobytes() == w.master.tobytes(), (t, k)


ALL_CHECKS = [v for k, v in sorted(globals().items()) if k.startswith("check_")]
