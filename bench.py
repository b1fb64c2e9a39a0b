"""Benchmark: one data-parallel rank's ZeRO-2 step on the 7e9-parameter,
N = 8, rank-0 shard (875,000,000 elements), on one MI355X.

A timed step is one pass of the whole hot path over one batch of gradients:
  1. flatten this rank's gradient (the 7e9-element flat vector, a one-tensor
     list) into its zero-padded flat buffer            -> flatten kernel
  2. reduce the 8 replicas onto the slice, Adam with bias correction on the
     fp32 master/m/v, write the bf16 slice into the full flat parameter
     buffer                                            -> fused step kernel
Replica 0 is the buffer step 1 wrote; replicas 1..7 (the other ranks'
contributions to this slice) are slice-only buffers. All inputs are seeded
synthetic data resident in HBM before timing starts.

Prints one JSON line. `value` is shard elements updated per second over the
whole step; `roofline` describes the fused step kernel (HIP events on the
launch stream); `cpu_baseline` times the CPU oracle on a bounded window of
the same workload on this host.

`--workload` times one of the other shards instead (the 1,000,003-element,
GPT-2-small, Llama-13B and 70e9/N=64 cases, built as in the parity tests);
those lines carry no CPU baseline and no extras. The Llama-13B shard comes
twice: with the peers' slices at address phase 0 (mixed 16-byte phases, the
shifted path) and at the phase they have inside full flat buffers.

The default workload also times extras, each selectable with `--extras`:
the bucketed step eager on 2 streams (buckets), replayed from a HIP graph
(graph), beside bf16 GEMMs with and without a workgroup cap (gemm) and on
CU-partitioned streams (partition), the Llama-7B tensor-list flatten and
unflatten (lists), and the per-parameter dim-0 layout step (fsdp).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402
import zero_partitioned_optimizer_flatten_amd as zero  # noqa: E402

NUMEL, WORLD, RANK = 7_000_000_000, 8, 0
LR, BETAS, EPS = 1e-3, (0.9, 0.999), 1e-8
PEAK_HBM_GBPS = 8000.0
KERNEL_SRC = os.path.join(ROOT, "zero_partitioned_optimizer_flatten_amd", "csrc",
                          "zero_kernels.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_step_flat7b_n8.md")


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def step_bytes_per_elem(world, grad_bytes=2, param_bytes=2):
    """Algorithmic bytes per shard element of the fused step: read the N
    replica values, read and write fp32 master/m/v, write the parameter."""
    return world * grad_bytes + 12 + 12 + param_bytes


def kernel_source_digest():
    """First 16 hex digits of the sha256 of the kernel source's code, with
    comments removed and whitespace collapsed: an edit that changes no code
    keeps the committed counters valid, any other edit invalidates them."""
    with open(KERNEL_SRC) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return hashlib.sha256(" ".join(text.split()).encode()).hexdigest()[:16]


def measured_traffic():
    """HBM bytes per fused-step launch from the committed rocprofv3 counter
    summary, or None if absent or taken on a different kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            text = f.read()
    except OSError:
        return None
    src = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    val = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not src or not val or src.group(1) != kernel_source_digest():
        return None
    return float(val.group(1))


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(window: int, min_seconds: float):
    """The CPU oracle as it stands, on a window of the same workload: the
    flatten of the matching 8*window gradient elements plus the shard step
    on `window` elements with all 8 replicas, repeated for min_seconds, on
    all OpenMP threads and then on one thread."""
    import oracle
    rng_g = torch.Generator().manual_seed(1)
    own = (torch.randn(WORLD * window, generator=rng_g) * 1e-3).to(torch.bfloat16)
    own_bits = own.view(torch.int16).numpy().view(np.uint16)
    peers = [(torch.randn(window, generator=rng_g) * 1e-3).to(torch.bfloat16)
             .view(torch.int16).numpy().view(np.uint16).copy() for _ in range(WORLD - 1)]
    orc = oracle.ShardOracle(window, 1, 0, LR, BETAS, EPS, n_replicas=WORLD)
    orc.master[:] = (torch.randn(window, generator=rng_g) * 0.02).numpy()
    out = np.zeros(window, np.uint16)

    def run(seconds):
        iters, t = 0, 1
        t0 = time.perf_counter()
        while True:
            flat = oracle.flatten([own_bits], WORLD * window)
            orc.step([flat[:window]] + peers, t, out, grad_offset=0, out_offset=0)
            iters += 1
            t += 1
            el = time.perf_counter() - t0
            if el >= seconds and iters >= 2:
                return iters, el

    threads = oracle.num_threads()
    iters, el = run(min_seconds)
    oracle.set_threads(1)
    iters1, el1 = run(min_seconds / 2)
    oracle.set_threads(threads)
    # host bytes per iteration with the GPU kernels' formulas: the fused
    # step's 42 B per shard element plus the flatten's read and write
    host_bytes = step_bytes_per_elem(WORLD) * window + 2 * 2 * WORLD * window
    return dict(value=window * iters / el, unit="shard elements/s", cores=threads,
                kind="oracle", host_gbps=host_bytes * iters / el / 1e9,
                sample=(f"{iters} steps of a {window}-element window of the 7e9/N=8 shard: "
                        f"flatten of {WORLD * window} bf16 gradient elements + reduce/Adam/bf16 "
                        f"over {WORLD} replicas, {el:.1f} s wall on {threads} OpenMP threads"),
                single_thread_value=window * iters1 / el1,
                cpu_model=_cpu_model(), host_cpus=os.cpu_count())


def _time_ms(fn, reps=5):
    fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def _time_ms_steady(fn, reps=5):
    """Per-call GPU time once calls are queued back to back: one call is in
    flight before the first event, so the host work of each later call
    overlaps the GPU work of the one before (as in a training loop). For
    calls whose host side is not negligible against their GPU time."""
    fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    fn()
    a.record()
    for _ in range(reps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def bucketed_extras(st, reps, out, t0, sizes=(1 << 22, 1 << 24, 1 << 26), nstreams=2):
    """The same step applied bucket by bucket (zero_step_range) on
    `nstreams` streams: time of a whole shard's worth of buckets."""
    S = st.shard
    streams = [torch.cuda.Stream() for _ in range(nstreams)]
    cur = torch.cuda.current_stream()
    res = {}
    t = [t0]

    def run(bucket):
        for s in streams:
            s.wait_stream(cur)
        for i, b0 in enumerate(range(0, S, bucket)):
            st.step_range(b0, min(bucket, S - b0), reps, t[0], out, grad_offset=b0,
                          param_offset=b0, stream=streams[i % nstreams])
        for s in streams:
            cur.wait_stream(s)
        t[0] += 1

    for bucket in sizes:
        ms = _time_ms(lambda: run(bucket), reps=3)
        res[str(bucket)] = {"buckets": (S + bucket - 1) // bucket, "ms": ms,
                            "gbps": step_bytes_per_elem(WORLD) * S / (ms * 1e-3) / 1e9}
    return res


def bucketed_graph_extras(st, reps, out, t0, sizes=(1 << 20, 1 << 22, 1 << 24),
                          nstreams=(1, 2)):
    """The bucketed step with the step count on the device: step_begin plus
    one step_range_sched per bucket, captured once as a HIP graph and
    replayed (each replay is one whole step); with 2 streams, buckets
    alternate between two branches of the graph after step_begin."""
    S = st.shard
    st.schedule(t0)
    res = {}
    for ns in nstreams:
        for bucket in sizes:
            g = torch.cuda.CUDAGraph()
            side = torch.cuda.Stream()
            with torch.cuda.graph(g):
                cur = torch.cuda.current_stream()
                st.step_begin()
                streams = [cur] + ([side] if ns > 1 else [])
                if ns > 1:
                    side.wait_stream(cur)
                for i, b0 in enumerate(range(0, S, bucket)):
                    cnt = min(bucket, S - b0)
                    st.step_range_sched(b0, cnt, [r[b0:] for r in reps], out, grad_offset=0,
                                        param_offset=b0, stream=streams[i % ns])
                if ns > 1:
                    cur.wait_stream(side)
            ms = _time_ms(g.replay, reps=3)
            res[f"{bucket}x{ns}"] = {"buckets": (S + bucket - 1) // bucket, "streams": ns,
                                     "ms": ms,
                                     "gbps": step_bytes_per_elem(WORLD) * S / (ms * 1e-3) / 1e9}
            del g
    return res


def overlap_extras(st, reps, out, t0, bucket=1 << 26, n=4096, gemms=48, caps=(0, 1, 2, 4)):
    """Why buckets: the step is HBM-bound, a backward pass mostly MFMA-bound.
    bf16 GEMMs (n x n x n, about as long in all as the step) on one stream
    and the bucketed step on another, timed alone and together, with the
    step's workgroups uncapped (cap 0) and capped at `cap` per compute unit
    (zero_set_step_workgroups)."""
    S = st.shard
    a = torch.randn(n, n, device="cuda").to(torch.bfloat16)
    b = torch.randn(n, n, device="cuda").to(torch.bfloat16)
    c = torch.empty(n, n, dtype=torch.bfloat16, device="cuda")
    gs, ss = torch.cuda.Stream(), torch.cuda.Stream()
    cur = torch.cuda.current_stream()
    t = [t0]

    def launch_gemms():
        with torch.cuda.stream(gs):
            for _ in range(gemms):
                torch.matmul(a, b, out=c)

    def launch_steps():
        for b0 in range(0, S, bucket):
            st.step_range(b0, min(bucket, S - b0), reps, t[0], out, grad_offset=b0,
                          param_offset=b0, stream=ss)
        t[0] += 1

    def run_gemms():
        gs.wait_stream(cur)
        launch_gemms()
        cur.wait_stream(gs)

    def run_steps():
        ss.wait_stream(cur)
        launch_steps()
        cur.wait_stream(ss)

    def both():
        # both side streams start after the current stream's work; the
        # current stream then waits for both (no order between the two)
        gs.wait_stream(cur)
        ss.wait_stream(cur)
        launch_gemms()
        launch_steps()
        cur.wait_stream(gs)
        cur.wait_stream(ss)

    ms_g = _time_ms(run_gemms, reps=3)
    res = {"gemm": {"n": n, "count": gemms, "ms": ms_g,
                    "tflops": 2.0 * n ** 3 * gemms / (ms_g * 1e-3) / 1e12},
           "bucket": bucket, "by_cap": {}}
    for cap in caps:
        st.set_step_workgroups(cap)
        ms_s = _time_ms(run_steps, reps=3)
        ms_b = _time_ms(both, reps=3)
        res["by_cap"][str(cap)] = {
            "bucketed_step_ms": ms_s, "together_ms": ms_b,
            "step_gbps": step_bytes_per_elem(WORLD) * S / (ms_s * 1e-3) / 1e9,
            "hidden_fraction_of_step": (ms_g + ms_s - ms_b) / ms_s}
    st.set_step_workgroups(0)
    del a, b, c
    return res


_HIP = None


def _hip_runtime():
    """The HIP runtime library this process already loaded (through torch),
    for the stream calls torch does not expose."""
    global _HIP
    if _HIP is None:
        import ctypes
        path = None
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64.so" in line:
                    path = line.split()[-1]
                    break
        if path is None:
            raise RuntimeError("HIP runtime not loaded")
        L = ctypes.CDLL(path)
        L.hipExtStreamCreateWithCUMask.argtypes = [ctypes.POINTER(ctypes.c_void_p),
                                                   ctypes.c_uint32,
                                                   ctypes.POINTER(ctypes.c_uint32)]
        L.hipStreamDestroy.argtypes = [ctypes.c_void_p]
        _HIP = L
    return _HIP


def cu_partition(n_cus, share):
    """Two CU masks: share/8 of the CUs for the first, the rest for the
    second, such that each of the 8 XCDs holds share/8 of its CUs in the
    first whether mask bit c belongs to XCD c // (n_cus / 8) or to XCD c % 8."""
    per = n_cus // 8
    pick = [((c % 8) + c // per) % 8 < share for c in range(n_cus)]
    return ([c for c in range(n_cus) if pick[c]], [c for c in range(n_cus) if not pick[c]])


def cu_masked_stream(cus, n_cus):
    """A default-priority stream whose kernels run only on the listed CUs."""
    import ctypes
    words = (n_cus + 31) // 32
    mask = (ctypes.c_uint32 * words)()
    for c in cus:
        mask[c // 32] |= 1 << (c % 32)
    h = ctypes.c_void_p()
    rc = _hip_runtime().hipExtStreamCreateWithCUMask(ctypes.byref(h), words, mask)
    if rc != 0:
        raise RuntimeError(f"hipExtStreamCreateWithCUMask failed ({rc})")
    return torch.cuda.ExternalStream(h.value), h


def partition_extras(st, reps, out, t0, bucket=1 << 26, n=4096, gemms=48,
                     shares=((1, 2), (2, 0), (2, 4), (4, 4), (4, 8))):
    """The bucketed step and bf16 GEMMs on CU-partitioned streams: the step
    on share/8 of the CUs (capped at `cap` workgroups per device CU, all of
    which land on its share), the GEMMs on the rest. Against the two run
    one after the other on the whole device."""
    S = st.shard
    n_cus = torch.cuda.get_device_properties(0).multi_processor_count
    a = torch.randn(n, n, device="cuda").to(torch.bfloat16)
    b = torch.randn(n, n, device="cuda").to(torch.bfloat16)
    c = torch.empty(n, n, dtype=torch.bfloat16, device="cuda")
    cur = torch.cuda.current_stream()
    t = [t0]

    def launch_gemms(gs):
        with torch.cuda.stream(gs):
            for _ in range(gemms):
                torch.matmul(a, b, out=c)

    def launch_steps(ss):
        for b0 in range(0, S, bucket):
            st.step_range(b0, min(bucket, S - b0), reps, t[0], out, grad_offset=b0,
                          param_offset=b0, stream=ss)
        t[0] += 1

    def on(launch, *streams):
        # the side streams start after the current stream's work, and the
        # current stream waits for all of them (no order among them)
        def run():
            for x in streams:
                x.wait_stream(cur)
            launch()
            for x in streams:
                cur.wait_stream(x)
        return run

    def gemm_on(gs):
        return on(lambda: launch_gemms(gs), gs)

    def step_on(ss):
        return on(lambda: launch_steps(ss), ss)

    whole_g, whole_s = torch.cuda.Stream(), torch.cuda.Stream()
    ms_g = _time_ms(gemm_on(whole_g), reps=3)
    st.set_step_workgroups(0)
    ms_s = _time_ms(step_on(whole_s), reps=3)
    ms_b = _time_ms(on(lambda: (launch_gemms(whole_g), launch_steps(whole_s)), whole_g,
                       whole_s), reps=3)
    res = {"gemm_ms": ms_g, "step_ms": ms_s, "serial_ms": ms_g + ms_s, "n_cus": n_cus,
           "unpartitioned_together_ms": ms_b, "by_partition": {}}
    for share, cap in shares:
        sc, gc = cu_partition(n_cus, share)
        ss, sh = cu_masked_stream(sc, n_cus)
        gs, gh = cu_masked_stream(gc, n_cus)
        st.set_step_workgroups(cap)
        ms_ps = _time_ms(step_on(ss), reps=3)
        ms_pg = _time_ms(gemm_on(gs), reps=3)
        ms_b = _time_ms(on(lambda: (launch_gemms(gs), launch_steps(ss)), gs, ss), reps=3)
        torch.cuda.synchronize()
        _hip_runtime().hipStreamDestroy(sh)
        _hip_runtime().hipStreamDestroy(gh)
        res["by_partition"][f"step_cus={len(sc)},cap={cap}"] = {
            "step_alone_ms": ms_ps, "gemm_alone_ms": ms_pg, "together_ms": ms_b,
            "hidden_fraction_of_step": (ms_g + ms_s - ms_b) / ms_s}
    st.set_step_workgroups(0)
    del a, b, c
    return res


def list_extras(dev):
    """Multi-tensor flatten and unflatten on the Llama-7B-shaped list
    (291 tensors, 6,738,415,616 bf16 elements)."""
    shapes = synth.llama_shapes(32, 4096, 11008)
    numel = synth.numel_of(shapes)
    st = zero.ShardState(numel, WORLD, 0, LR, BETAS, EPS)
    storage = torch.empty(numel, dtype=torch.bfloat16, device=dev)
    synth.fill_gaussian(storage, 1e-3, 11)
    tensors = synth.split_views(storage, shapes)
    flat = torch.empty(st.padded, dtype=torch.bfloat16, device=dev)
    ms_f = _time_ms(lambda: st.flatten(tensors, flat))
    ok = torch.equal(flat[:numel].view(torch.int16), storage.view(torch.int16))
    dst_storage = torch.empty(numel, dtype=torch.bfloat16, device=dev)
    dsts = synth.split_views(dst_storage, shapes)
    ms_u = _time_ms(lambda: st.unflatten(flat, dsts))
    ok = ok and torch.equal(dst_storage.view(torch.int16), storage.view(torch.int16))
    res = {"tensors": len(shapes), "numel": numel,
           "flatten": {"ms": ms_f, "gbps": (2 * numel + 2 * st.padded) / (ms_f * 1e-3) / 1e9},
           "unflatten": {"ms": ms_u, "gbps": 4 * numel / (ms_u * 1e-3) / 1e9},
           "bit_exact": bool(ok)}
    del storage, flat, dst_storage, tensors, dsts
    st.close()
    torch.cuda.empty_cache()
    return res


def fsdp_extras(dev, steps=5):
    """Per-parameter (dim-0) layout: the fused step over this rank's row
    shards of the Llama-7B-shaped list (291 parameters), N = 8, rank 0.
    Replica gradients are full-size tensors; only this rank's rows are read."""
    shapes = synth.llama_shapes(32, 4096, 11008)
    st = zero.FsdpShardState(shapes, WORLD, 0, LR, BETAS, EPS)
    local = sum(st.local_numel(k) for k in range(len(shapes)))
    params = [torch.empty(s, dtype=torch.float32, device=dev) for s in shapes]
    for k, p in enumerate(params):
        f, r, _ = st.local[k]
        synth.fill_gaussian(p.view(p.shape[0], -1)[f:f + r], synth.PARAM_STD, k)
    st.load_master(params)
    del params
    grads = [[torch.empty(s, dtype=torch.bfloat16, device=dev) for s in shapes]
             for _ in range(WORLD)]
    for q in range(WORLD):
        for k, g in enumerate(grads[q]):
            f, r, _ = st.local[k]
            synth.fill_gaussian(g.view(g.shape[0], -1)[f:f + r], 1e-3, 1000 * q + k)
    outs = [torch.empty(max(1, st.local_numel(k)), dtype=torch.bfloat16, device=dev)
            for k in range(len(shapes))]
    t = [1]

    def one():
        st.step(grads, t[0], outs)
        t[0] += 1
    one()
    torch.cuda.synchronize()
    h0 = time.perf_counter()
    one()                       # host side of a call: checks, pointer table, 10 launches
    host_ms = (time.perf_counter() - h0) * 1e3
    ms = _time_ms_steady(one, reps=steps)
    res = {"tensors": len(shapes), "local_elements": local, "ms": ms,
           "gbps": step_bytes_per_elem(WORLD) * local / (ms * 1e-3) / 1e9,
           "host_ms_per_call": host_ms}
    del grads, outs
    st.close()
    torch.cuda.empty_cache()
    return res


def copy_ceiling(nbytes: int, reps: int = 5):
    """Plain-copy context figures: the library's own copy kernel (the flatten
    of one bf16 tensor of nbytes, no pad: a plain copy of known size) and
    torch's device-to-device copy, in GB/s counting bytes read + written."""
    numel = nbytes // 2
    st = zero.ShardState(numel, 1, 0, LR, BETAS, EPS)
    src = torch.empty(numel, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty(numel, dtype=torch.bfloat16, device="cuda")
    src.view(torch.int16).random_(-30000, 30000)
    ms_lib = _time_ms(lambda: st.flatten([src], dst), reps=reps)
    assert torch.equal(src.view(torch.int16), dst.view(torch.int16))
    ms_torch = _time_ms(lambda: dst.copy_(src), reps=reps)
    st.close()
    del src, dst
    torch.cuda.empty_cache()
    return (2 * numel * 2 / (ms_lib * 1e-3) / 1e9, 2 * numel * 2 / (ms_torch * 1e-3) / 1e9)


EXTRAS = ("buckets", "graph", "gemm", "partition", "lists", "fsdp")

WORKLOADS = {
    "flat7b_n8_rank0": dict(
        desc="7e9-element flat vector, N=8 simulated ranks, rank 0 shard of 875,000,000",
        numel=7_000_000_000, world=8, rank=0, shapes=None, gdt=torch.bfloat16, std=1e-3,
        outliers=False, peers="slice", out="full", flatten=True),
    "flat1m_n4_rank3": dict(
        desc="1,000,003-element flat vector (one tensor), N=4, rank 3 (one pad element), fp32 "
             "gradients N(0,0.01), full flat replicas; cache-resident (10.5 MB per step)",
        numel=1_000_003, world=4, rank=3, shapes=None, gdt=torch.float32, std=1e-2,
        outliers=False, peers="full", out="full", flatten=True),
    "gpt2s_n8_rank3": dict(
        desc="GPT-2-small list (148 tensors, 124,439,808 elements), N=8, rank 3, full flat "
             "replicas; 653 MB per step (partly cache-resident)",
        numel=None, world=8, rank=3, shapes="gpt2", gdt=torch.bfloat16, std=1e-3,
        outliers=False, peers="full", out="full", flatten=True),
    "llama13b_n8_rank7": dict(
        desc="Llama-13B list + one scalar (364 tensors, 13,015,864,321 elements), N=8, rank 7 "
             "(odd lo, 7 pad elements); own gradient flattened from the list, peers hold the "
             "slice only, bf16 output into the full flat buffer; 1% of gradients x100",
        numel=None, world=8, rank=7, shapes="llama13b", gdt=torch.bfloat16, std=1e-3,
        outliers=True, peers="slice", out="full", flatten=True),
    "llama13b_n8_rank7_lo": dict(
        desc="Llama-13B list + one scalar (364 tensors, 13,015,864,321 elements), N=8, rank 7 "
             "(odd lo, 7 pad elements); own gradient flattened from the list, each peer's "
             "slice stored at the address phase (lo mod 64 elements) it has in a full flat "
             "buffer, bf16 output into the full flat buffer; 1% of gradients x100",
        numel=None, world=8, rank=7, shapes="llama13b", gdt=torch.bfloat16, std=1e-3,
        outliers=True, peers="slice_at_lo", out="full", flatten=True),
    "flat70b_n64_rank0": dict(
        desc="70e9-element flat vector, N=64, rank 0 shard of 1,093,750,000, slice-only "
             "replicas and output; flatten not timed (the full own gradient and its flat copy, "
             "280 GB, do not fit beside the 64 replica slices)",
        numel=70_000_000_000, world=64, rank=0, shapes=None, gdt=torch.bfloat16, std=1e-3,
        outliers=False, peers="slice", out="slice", flatten=False),
}
DEFAULT_WORKLOAD = "flat7b_n8_rank0"


def _shapes(kind):
    if kind == "gpt2":
        return synth.gpt2_small_shapes()
    if kind == "llama13b":
        return synth.llama_shapes(40, 5120, 13824, trailing_scalar=True)
    return None


def build_inputs(w, dev):
    """Seeded inputs of a workload, resident on the device: the shard
    state, this rank's gradient as a tensor list plus its flat buffer, the
    other ranks' replicas, and the parameter output."""
    shapes = _shapes(w["shapes"])
    numel = synth.numel_of(shapes) if shapes else w["numel"]
    world, rank, gdt = w["world"], w["rank"], w["gdt"]
    st = zero.ShardState(numel, world, rank, LR, BETAS, EPS)
    S, lo, P = st.shard, st.lo, st.padded
    valid = max(0, min(S, numel - lo))
    p = torch.zeros(S, dtype=torch.float32, device=dev)
    synth.fill_gaussian(p[:valid], synth.PARAM_STD, synth.PARAM_SEED)
    st.load_master(p, flat_offset=0)
    del p
    # return the staging block, so the buffers below start on fresh
    # 2 MiB-aligned segments instead of inside its halves (measured: a
    # replica 512 bytes off a 4 KiB page costs the fused step)
    torch.cuda.synchronize()
    torch.cuda.empty_cache()

    def grad_fill(buf, q):
        synth.fill_gaussian(buf, w["std"], synth.grad_seed(1, q),
                            synth.mask_seed(1, q) if w["outliers"] else None)

    own_tensors, own_flat = None, None
    if w["flatten"]:
        storage = torch.empty(numel, dtype=gdt, device=dev)
        grad_fill(storage, rank)
        own_tensors = synth.split_views(storage, shapes) if shapes else [storage]
        own_flat = torch.empty(P, dtype=gdt, device=dev)
        own = own_flat[lo:lo + S]
    else:
        own = torch.zeros(S, dtype=gdt, device=dev)
        grad_fill(own[:valid], rank)
    reps = []
    for q in range(world):
        if q == rank:
            reps.append(own)
            continue
        if w["peers"] == "full":
            buf = torch.zeros(P, dtype=gdt, device=dev)
            grad_fill(buf[lo:lo + valid], q)
            reps.append(buf[lo:lo + S])
        elif w["peers"] == "slice_at_lo":
            # the part of a full flat buffer that the step reads, at the
            # offset within a 128-byte line that element lo has there
            ph = lo % 64
            buf = torch.zeros(S + 64, dtype=gdt, device=dev)
            grad_fill(buf[ph:ph + valid], q)
            reps.append(buf[ph:ph + S])
        else:
            buf = torch.zeros(S, dtype=gdt, device=dev)
            grad_fill(buf[:valid], q)
            reps.append(buf)
    if w["out"] == "full":
        out = torch.zeros(P, dtype=torch.bfloat16, device=dev)[lo:lo + S]
    else:
        out = torch.zeros(S, dtype=torch.bfloat16, device=dev)
    return dict(st=st, numel=numel, S=S, lo=lo, P=P, own_tensors=own_tensors,
                own_flat=own_flat, reps=reps, out=out, ntensors=len(shapes) if shapes else 1)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", choices=sorted(WORKLOADS), default=DEFAULT_WORKLOAD,
                    help="shard to time; the others than the default skip the CPU baseline "
                         "and the extras")
    ap.add_argument("--cpu-window", type=int, default=1 << 24)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-context", action="store_true",
                    help="skip the plain-copy context measurement")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the bucketed-step and tensor-list measurements")
    ap.add_argument("--extras", default=",".join(EXTRAS),
                    help="comma-separated subset of the default workload's extra "
                         "measurements to run: " + ", ".join(EXTRAS))
    args = ap.parse_args()
    chosen = set() if args.no_extras else {e for e in args.extras.split(",") if e}
    unknown = chosen - set(EXTRAS)
    if unknown:
        ap.error(f"unknown extras: {', '.join(sorted(unknown))}")
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one rank's shard step on one GPU; runs on more than one "
              "GPU are not supported (the other ranks are simulated as gradient replicas "
              "on the same device).", file=sys.stderr)
        sys.exit(2)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    zero.lib()
    default = args.workload == DEFAULT_WORKLOAD
    w = WORKLOADS[args.workload]
    world = w["world"]
    gsize = torch.tensor([], dtype=w["gdt"]).element_size()

    log(f"{args.workload}: generating inputs")
    inp = build_inputs(w, dev)
    st, S, lo, P, numel = inp["st"], inp["S"], inp["lo"], inp["P"], inp["numel"]
    reps, out = inp["reps"], inp["out"]
    own_tensors, own_flat = inp["own_tensors"], inp["own_flat"]
    ntensors = inp["ntensors"]
    torch.cuda.synchronize()
    log(f"shard={S} lo={lo} padded={P}; inputs resident; warming up")

    stream = torch.cuda.current_stream()
    n_total = args.warmup + args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n_total)]

    def one(i):
        ev[i][0].record(stream)
        if own_tensors is not None:
            st.flatten(own_tensors, own_flat)
        ev[i][1].record(stream)
        st.step(reps, i + 1, out, grad_offset=0, param_offset=0)
        ev[i][2].record(stream)

    for i in range(args.warmup):
        one(i)
    torch.cuda.synchronize()

    log(f"timing {args.steps} steps")
    t0 = time.perf_counter()
    for i in range(args.warmup, n_total):
        one(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    flat_ms = np.array([ev[i][0].elapsed_time(ev[i][1]) for i in range(args.warmup, n_total)])
    step_ms = np.array([ev[i][1].elapsed_time(ev[i][2]) for i in range(args.warmup, n_total)])

    ms_per_step = wall * 1e3 / args.steps
    value = S * args.steps / wall
    bpe = step_bytes_per_elem(world, gsize)
    k2_bytes = bpe * S
    k1_bytes = gsize * (numel + P) if own_tensors is not None else 0
    k2_gbps = k2_bytes / (step_ms.mean() * 1e-3) / 1e9
    traffic = measured_traffic() if default else None

    # the step must have produced finite parameters
    assert torch.isfinite(out[:max(0, min(S, numel - lo))].float()).all().item()

    extras = {}
    if not default:
        chosen = set()
    if "buckets" in chosen:
        log("bucketed step")
        extras["bucketed_step_2_streams"] = bucketed_extras(
            st, reps, out, n_total + 1, sizes=(1 << 20, 1 << 22, 1 << 24, 1 << 26))
    if "graph" in chosen:
        log("bucketed step, graph replay")
        extras["bucketed_step_graph"] = bucketed_graph_extras(st, reps, out, n_total + 100)
    if "gemm" in chosen:
        log("bucketed step beside bf16 GEMMs")
        extras["bucketed_step_beside_gemm"] = overlap_extras(st, reps, out, n_total + 200)
    if "partition" in chosen:
        log("bucketed step and bf16 GEMMs on CU-partitioned streams")
        extras["bucketed_step_cu_partition"] = partition_extras(st, reps, out, n_total + 300)

    del inp, reps, out, own_tensors, own_flat
    st.close()
    torch.cuda.empty_cache()

    context = {}
    if not args.no_context:
        lib_gbps, torch_gbps = copy_ceiling(8 << 30)
        context["plain_copy_gbps"] = round(lib_gbps, 1)
        context["plain_copy_frac_of_peak"] = round(lib_gbps / PEAK_HBM_GBPS, 4)
        context["torch_copy_gbps"] = round(torch_gbps, 1)
        context["note"] = ("plain_copy: the library's copy kernel on one 8 GiB bf16 tensor "
                           "(read + written bytes), the achievable-bandwidth ceiling for a "
                           "2-stream copy; torch_copy: torch's own device copy of the same")
    if "lists" in chosen:
        log("tensor-list flatten/unflatten")
        extras["llama7b_list"] = list_extras(dev)
    if "fsdp" in chosen:
        log("per-parameter (dim-0) layout step")
        extras["fsdp_llama7b_n8_rank0"] = fsdp_extras(dev)

    kernels = {
        "fused_step": {"ms_mean": float(step_ms.mean()), "ms_median": float(np.median(step_ms)),
                       "ms_min": float(step_ms.min()),
                       "bytes_per_launch": k2_bytes, "bytes_per_elem": bpe,
                       "gbps": k2_gbps, "elements_per_s": S / (step_ms.mean() * 1e-3)},
    }
    if k1_bytes:
        kernels["flatten"] = {"ms_mean": float(flat_ms.mean()), "ms_median": float(np.median(flat_ms)),
                              "ms_min": float(flat_ms.min()),
                              "bytes_per_launch": k1_bytes, "tensors": ntensors,
                              "gbps": k1_bytes / (flat_ms.mean() * 1e-3) / 1e9}
    result = {
        "metric": "sharded Adam step: elements/s and achieved HBM GB/s (% of peak), 7B N=8",
        "value": value,
        "unit": "shard elements/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32 (%s gradients, bf16 parameter output)" % ("bf16" if gsize == 2 else "f32"),
        "data": "synthetic: seeded N(0,%g) %s gradients, N(0,0.02) fp32 parameters"
                % (w["std"], "bf16" if gsize == 2 else "fp32"),
        "config": {"workload": f"{args.workload}: {w['desc']}",
                   "numel": numel, "world": world, "rank": w["rank"], "shard": S,
                   "parallelism": "zero2-shard, 1 GPU"},
        "step_hbm_gbps": (k1_bytes + k2_bytes) / (ms_per_step * 1e-3) / 1e9,
        "kernels": kernels,
        "roofline": {"bound": "hbm", "achieved": k2_gbps, "peak": PEAK_HBM_GBPS,
                     "unit": "GB/s", "frac": k2_gbps / PEAK_HBM_GBPS,
                     "traffic": traffic,
                     "kernel": ("fused reduce+Adam+bf16 step (step_vec_kernel<8,bf16,bf16>)"
                                if default else "fused reduce+Adam step")},
        "context": context,
        "extras": extras,
    }
    if default and not args.no_cpu_baseline:
        log("timing the CPU oracle")
        result["cpu_baseline"] = cpu_baseline(args.cpu_window, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
