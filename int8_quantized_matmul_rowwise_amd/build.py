"""Build the llmint8 shared library (HIP, gfx950 only) in-tree.

    python -m int8_quantized_matmul_rowwise_amd.build [--sanitize OUT.so]

compiles csrc/*.hip with hipcc (one process per source, in parallel) and links
int8_quantized_matmul_rowwise_amd/libllmint8.so.  Numeric flags are part of the
contract: no floating-point contraction (every product and sum in the epilogue rounds
once), no fast-math, IEEE division (hipcc's default correctly rounded fp32 divide is
kept), no denormal flushing, and no packed-fp32 instructions.

--sanitize OUT.so builds a copy whose HOST code carries AddressSanitizer and
UndefinedBehaviorSanitizer (the device code is the same); it is a test build for the
argument validation and error paths, run on the CPU with the sanitizer runtime preloaded.
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libllmint8.so")
# the benchmark's measurement probes (MFMA rate and clock, stream read), a library of their own
PROBE_LIB = os.path.join(HERE, "libllmint8_probe.so")
PROBE_SOURCES = ["probe.hip"]
SOURCES = ["api.hip", "xpass.hip", "weight.hip", "gemm.hip", "gemm_small.hip", "codec.hip", "gemm_group.hip",
           "gemm_group_small.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-ffp-contract=off", "-fno-fast-math", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]
# host-only sanitizers (each -fsanitize= right after -Xarch_host: the GPU code is not instrumented)
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _jobs() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, int(os.environ.get("MAX_JOBS") or 16), len(SOURCES)))


def build(verbose: bool = False, extra=(), out: str = LIB, sanitize: bool = False, sources=SOURCES) -> str:
    flags = FLAGS + (SANITIZE if sanitize else []) + list(extra)
    inc = ["-I", os.path.join(ROOT, "include")]
    with tempfile.TemporaryDirectory(prefix="llmint8_build_") as tmpd:
        def compile_one(src: str) -> str:
            obj = os.path.join(tmpd, src.replace(".hip", ".o"))
            cmd = [HIPCC, *flags, *inc, "-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            subprocess.check_call(cmd)
            return obj

        with ThreadPoolExecutor(_jobs()) as ex:
            objs = list(ex.map(compile_one, sources))
        tmp = out + ".tmp%d" % os.getpid()
        cmd = [HIPCC, *flags, "-shared", *objs, "-o", tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.check_call(cmd)
    os.replace(tmp, out)
    return out


def build_probe(verbose: bool = False) -> str:
    return build(verbose=verbose, out=PROBE_LIB, sources=PROBE_SOURCES)


if __name__ == "__main__":
    args = sys.argv[1:]
    if args[:1] == ["--sanitize"]:
        print(build(verbose=True, out=os.path.abspath(args[1]), sanitize=True, extra=args[2:]))
    else:
        print(build(verbose=True, extra=args))
        print(build_probe(verbose=True))
