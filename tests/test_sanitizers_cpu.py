"""Sanitizer runs on the CPU (no GPU code is instrumented or run).

- The library's host code (argument validation, workspace layout, the stage sequencing and
  the error path) built with AddressSanitizer and UndefinedBehaviorSanitizer
  (`-Xarch_host -fsanitize=...`), driven by the boundary and failure tests.
- The CPU oracle built with the same sanitizers by gcc, driven by its pin tests.

Each run is a child process with the sanitizer runtime preloaded (the Python interpreter
itself is not instrumented); any report aborts it (UBSan without recovery), so the child's
exit status and output decide."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang"


def _runtime(cmd):
    try:
        p = subprocess.run(cmd, capture_output=True, text=True, check=True).stdout.strip()
    except (OSError, subprocess.CalledProcessError):
        return None
    return p if os.path.isabs(p) and os.path.exists(p) else None


def _run_child(env_extra, tests, timeout=600):
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env.pop("LLMINT8_FAULT", None)
    env.pop("LLMINT8_LOG", None)
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu", *tests]
    p = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=timeout)
    out = p.stdout + p.stderr
    assert p.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out
    return out


def test_library_host_code_under_asan_and_ubsan(tmp_path):
    rt = _runtime([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"])
    if rt is None:
        pytest.skip("clang's AddressSanitizer runtime is not installed")
    from int8_quantized_matmul_rowwise_amd import build
    lib = build.build(out=str(tmp_path / "libllmint8_san.so"), sanitize=True)
    _run_child({"LD_PRELOAD": rt, "LLMINT8_LIB": lib}, ["tests/test_abi_cpu.py", "tests/test_fault_cpu.py"])


def test_oracle_under_asan_and_ubsan(tmp_path):
    rt = _runtime(["gcc", "-print-file-name=libasan.so"])
    if rt is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    import oracle
    lib = oracle.build(out=str(tmp_path / "liborc_san.so"), sanitize=True)
    _run_child({"LD_PRELOAD": rt, "LLMINT8_ORACLE_LIB": lib, "OMP_NUM_THREADS": "4"},
               ["tests/test_oracle_pipeline.py", "tests/test_oracle_formats.py", "tests/test_oracle_group.py",
                "tests/test_oracle_codec.py", "tests/test_oracle_fixed.py", "tests/test_oracle_quantizer.py"],
               timeout=900)
