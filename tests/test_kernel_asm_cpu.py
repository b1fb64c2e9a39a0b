"""The gfx950 assembly of the kernels, compiled here on the CPU, keeps the
properties the design relies on:

- no packed fp32 arithmetic (v_pk_add/mul/fma_f32), which the build turns
  off;
- no kernel uses scratch (no register spills);
- the fused and per-parameter step kernels and the segment copy carry no
  readfirstlane loop: every buffer descriptor they build is wave-uniform, so
  no load or store is wrapped in a loop over the distinct descriptors of a
  wave;
- the segment copy stores its 16-byte vectors non-temporal at device scope;
- the streamed-state N = 8 bf16 step stores master/m/v and the parameter
  output non-temporal at device scope (nt sc1), and loads the state and the
  line-aligned replicas non-temporal."""
import os
import re
import shutil

import pytest

from zero_partitioned_optimizer_flatten_amd import build as zb


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    if not (os.path.exists(zb.HIPCC) or shutil.which(zb.HIPCC)):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm")
    zb.asm(str(out))
    return (out / "zero_kernels.s").read_text()


def _kernels(asm):
    """(name, body, trailer) per kernel."""
    for m in re.finditer(r"^(_Z\w+):", asm, re.M):
        end = asm.index(".Lfunc_end", m.end())
        yield m.group(1), asm[m.end():end], asm[end:end + 4000]


def test_no_packed_fp32(asm):
    assert not re.search(r"\bv_pk_(add|mul|fma)_f32\b", asm)


def test_no_scratch(asm):
    sizes = {name: int(re.search(r"; ScratchSize: (\d+)", tail).group(1))
             for name, _, tail in _kernels(asm)}
    assert sizes, "no kernels found"
    assert all(v == 0 for v in sizes.values()), {k: v for k, v in sizes.items() if v}


def test_step_kernels_have_no_waterfall_loops(asm):
    found = 0
    for name, body, _ in _kernels(asm):
        if ("step_vec_kernel" in name or "fsdp_step_kernel" in name
                or "copy_segments_kernel" in name):
            found += 1
            assert "v_readfirstlane" not in body, name
    assert found >= 100


def test_copy_store_policy(asm):
    bodies = [b for n, b, _ in _kernels(asm) if "copy_segments_kernel" in n]
    assert len(bodies) == 2                      # both destination chunk grids
    for body in bodies:
        stores = re.findall(r"buffer_store_dwordx4 [^\n]*offen([^\n]*)", body)
        assert stores and all(t.split() == ["nt", "sc1"] for t in stores), stores


def test_streamed_step_cache_policy(asm):
    name = ("_ZN2zk12_GLOBAL__N_115step_vec_kernelILi8ELb1ELb1ELb0ELb1EEEvNS0_4RepsIXT_EEEiPfS4_"
            "S4_PvlliiiNS0_9ScalarArgIXT2_EEE")
    body = dict((n, b) for n, b, _ in _kernels(asm))[name]
    stores = re.findall(r"buffer_store_dwordx(\d) [^\n]*offen([^\n]*)", body)
    loads = re.findall(r"buffer_load_dwordx(\d) [^\n]*offen([^\n]*)", body)

    def policy(bits):
        return [t for t in bits.split() if not t.startswith("offset:")]

    streamed = [w for w, bits in stores if policy(bits) == ["nt", "sc1"]]
    # per block: 6 state stores (dwordx4) and 2 output stores (dwordx2)
    assert streamed.count("4") >= 6 and streamed.count("2") >= 2
    nt_loads = [w for w, bits in loads if policy(bits) == ["nt"]]
    # 16 replica loads (dwordx2) and 6 state loads (dwordx4)
    assert nt_loads.count("2") >= 16 and nt_loads.count("4") >= 6
