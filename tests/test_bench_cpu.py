"""bench.py's contract pieces that need no GPU: more than one GPU is refused
with a message, and the algorithmic bytes behind roofline.achieved."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    for n in ("2", "8"):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", n],
                           capture_output=True, text=True, timeout=300)
        assert r.returncode == 2, r
        assert "one GPU" in r.stderr and not r.stdout.strip()


def test_step_bytes_per_element():
    # N replica reads + fp32 master/m/v read and written + the parameter write
    assert bench.step_bytes_per_elem(8) == 8 * 2 + 12 + 12 + 2 == 42
    assert bench.step_bytes_per_elem(64) == 154
    assert bench.step_bytes_per_elem(4, grad_bytes=4) == 4 * 4 + 24 + 2
    # the 7e9/N=8 shard: 875,000,000 elements, 36.75 GB per fused-step launch
    assert bench.step_bytes_per_elem(8) * 875_000_000 == 36_750_000_000


def test_workloads_cover_the_shard_configurations():
    w = bench.WORKLOADS
    assert bench.DEFAULT_WORKLOAD == "flat7b_n8_rank0"
    assert (w["flat7b_n8_rank0"]["numel"], w["flat7b_n8_rank0"]["world"]) == (7_000_000_000, 8)
    assert (w["flat70b_n64_rank0"]["numel"], w["flat70b_n64_rank0"]["world"]) == (70_000_000_000, 64)
    assert w["llama13b_n8_rank7"]["rank"] == 7 and w["llama13b_n8_rank7"]["outliers"]
    assert w["llama13b_n8_rank7_lo"]["peers"] == "slice_at_lo"
    assert {k: v for k, v in w["llama13b_n8_rank7_lo"].items() if k not in ("peers", "desc")} \
        == {k: v for k, v in w["llama13b_n8_rank7"].items() if k not in ("peers", "desc")}
    assert w["flat1m_n4_rank3"]["numel"] == 1_000_003
    assert w["gpt2s_n8_rank3"]["shapes"] == "gpt2"


def test_unknown_extras_are_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--extras", "fsdp,nope"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2 and "unknown extras: nope" in r.stderr
    assert set(bench.EXTRAS) == {"buckets", "graph", "gemm", "partition", "lists", "fsdp"}


def test_kernel_code_digest(tmp_path, monkeypatch):
    """The digest that gates the committed counters ignores comments and
    whitespace and changes with any code edit."""
    src = tmp_path / "k.hip"
    code = "// header\n__global__ void k(int *p) {\n  p[0] = 1; /* store */\n}\n"
    src.write_text(code)
    monkeypatch.setattr(bench, "KERNEL_SRC", str(src))
    d0 = bench.kernel_source_digest()
    src.write_text("// other words\n\n__global__  void k(int *p)\n{ p[0] = 1;\n}\n")
    assert bench.kernel_source_digest() == d0
    src.write_text(code.replace("= 1", "= 2"))
    assert bench.kernel_source_digest() != d0
