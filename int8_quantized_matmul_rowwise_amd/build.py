"""Build the llmint8 shared library (HIP, gfx950 only) in-tree.

    python -m int8_quantized_matmul_rowwise_amd.build

compiles csrc/*.hip with hipcc into int8_quantized_matmul_rowwise_amd/libllmint8.so.
Numeric flags are part of the contract: no floating-point contraction (every product
and sum in the epilogue rounds once), no fast-math, IEEE division (hipcc's default
correctly rounded fp32 divide is kept), no denormal flushing, and no packed-fp32
instructions.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libllmint8.so")
SOURCES = ["api.hip", "xpass.hip", "weight.hip", "gemm.hip", "gemm_small.hip", "codec.hip", "gemm_group.hip",
           "gemm_group_small.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-fvisibility=hidden",
    "-ffp-contract=off", "-fno-fast-math", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def build(verbose: bool = False, extra=()) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, *extra, "-I", os.path.join(ROOT, "include"), *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True, extra=sys.argv[1:]))
