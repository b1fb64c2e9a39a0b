"""Build libzero.so for gfx950 with hipcc, in-tree (next to this file)."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libzero.so")
SOURCES = ["zero_api.hip", "zero_kernels.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Numerics: no implicit fusion, correctly rounded fp32 divide and sqrt,
# denormals kept. Packed-fp32 instructions are disabled for the device.
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fno-fast-math",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def build(verbose: bool = False) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


def asm(out_dir: str) -> None:
    """Write the gfx950 assembly of the kernels (for inspection)."""
    os.makedirs(out_dir, exist_ok=True)
    src = os.path.join(CSRC, "zero_kernels.hip")
    flags = [f for f in FLAGS if f not in ("-shared", "-fPIC")]
    subprocess.check_call([HIPCC, *flags, "--cuda-device-only", "-S", src,
                           "-o", os.path.join(out_dir, "zero_kernels.s")])


if __name__ == "__main__":
    build(verbose=True)
    if len(sys.argv) > 1 and sys.argv[1] == "--asm":
        asm(sys.argv[2] if len(sys.argv) > 2 else "_work/asm")
