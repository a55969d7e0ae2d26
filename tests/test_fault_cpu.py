"""Failure handling of the host layer, on the CPU.

LLMINT8_FAULT=<stage> turns a call into a dry run in which the named launch (or copy)
fails: the call must return LLMINT8_EHIP, enqueue nothing after the failed stage and
report nothing as done (int8_matmul_stats leaves its host output alone).  LLMINT8_LOG=1
prints each call's path and stages, which is how these tests learn the stage sequence of
every entry point.  Nothing here touches a GPU: in a dry run no HIP call is made, and
argument validation runs before any stage."""
import ctypes
import re

import pytest

import int8_quantized_matmul_rowwise_amd as L

MB = 0x100000
X, WQ, SW, Y, WS, OL, WO = MB, 64 * MB, 128 * MB, 192 * MB, 256 * MB, 1024 * MB, 1100 * MB  # fake device addresses
BIG = 1 << 34


def _calls():
    lib = L.lib()
    n = ctypes.c_int32(-5)
    return {
        "matmul_tiled": (lambda: lib.int8_matmul(X, 300, 1024, 0, WQ, SW, 520, 6.0, Y, WS, BIG, None),
                         ["detect", "compact", "code_rows", "gemm"]),
        "matmul_small": (lambda: lib.int8_matmul(X, 16, 1024, 1, WQ, SW, 520, 6.0, Y, WS, BIG, None),
                         ["xpass_small", "gemm_small"]),
        "matmul_mid": (lambda: lib.int8_matmul(X, 64, 1024, 0, WQ, SW, 65536, 6.0, Y, WS, BIG, None),
                       ["xpass_small", "gemm"]),
        "matmul_long_rows": (lambda: lib.int8_matmul(X, 8192, 28672, 1, WQ, SW, 8192, 6.0, 8192 * MB, 4096 * MB,
                                                     BIG, None), ["detect", "compact", "code_rows", "gemm"]),
        "accumulators": (lambda: lib.int8_matmul_accumulators(X, 300, 1024, 0, WQ, 520, 6.0, Y, WO, WS, BIG, None),
                         ["detect", "compact", "code_rows", "gemm"]),
        "prepare": (lambda: lib.int8_matmul_prepare(X, 300, 1024, 0, WQ, 520, 6.0, WS, BIG, None),
                    ["detect", "compact", "code_rows"]),
        "products_small": (lambda: lib.int8_matmul_products(16, 1024, 0, WQ, SW, 520, Y, WS, BIG, None),
                           ["gemm_small"]),
        "weight": (lambda: lib.int8_quantize_weight(X, 1024, 520, 0, WQ, SW, None), ["weight"]),
        "weight_fixed": (lambda: lib.int8_quantize_weight_fixed(X, 1024, 520, 0, OL, 5, WQ, SW, WO, WS, BIG, None),
                         ["list_bitmap", "weight", "gather_wo"]),
        "matmul_fixed": (lambda: lib.int8_matmul_fixed(X, 300, 1024, 0, OL, 5, WQ, SW, WO, 520, Y, WS, BIG, None),
                         ["list_bitmap", "compact", "code_rows", "gemm"]),
        "weight_group": (lambda: lib.int8_quantize_weight_group(X, 1024, 520, 0, 128, WQ, SW, None),
                         ["group_colmax", "quantize_weight_groups"]),
        "matmul_group": (lambda: lib.int8_matmul_group(X, 300, 1024, 0, 128, WQ, SW, 520, Y, WS, BIG, None),
                         ["group_xpass", "gemm_group"]),
        "matmul_group_small": (lambda: lib.int8_matmul_group(X, 16, 1024, 0, 128, WQ, SW, 520, Y, WS, BIG, None),
                               ["group_xpass", "gemm_group_small"]),
        "group_k0": (lambda: lib.int8_matmul_group(X, 16, 0, 0, 128, WQ, SW, 520, Y, WS, BIG, None), ["fill_zero"]),
        "codec_q": (lambda: lib.int8_blockwise_quantize(X, 1 << 20, 2048, WQ, SW, None), ["block_quantize"]),
        "codec_d": (lambda: lib.int8_blockwise_dequantize(WQ, SW, 1 << 20, 2048, X, None), ["block_dequantize"]),
        "stats": (lambda: lib.int8_matmul_stats(X, 300, 1024, 0, 6.0, ctypes.byref(n), OL, WS, BIG, None),
                  ["detect", "compact", "stats_copy", "stats_sync", "stats_copy_cols"]),
    }, n


def _stages(err: str):
    return re.findall(r"^\[llmint8\]   stage (\w+)", err, flags=re.M)


@pytest.fixture
def dry(monkeypatch):
    monkeypatch.setenv("LLMINT8_LOG", "1")

    def set_fault(stage):
        monkeypatch.setenv("LLMINT8_FAULT", stage)
    return set_fault


@pytest.mark.parametrize("name", sorted(_calls()[0]))
def test_dry_run_lists_the_stages(name, dry, capfd):
    """With a fault on no stage of the path, the dry run passes every stage, enqueues
    nothing and returns OK; the log names the path's stages in order."""
    calls, _ = _calls()
    fn, expected = calls[name]
    dry("no_such_stage")
    capfd.readouterr()
    assert fn() == L.OK
    err = capfd.readouterr().err
    assert _stages(err) == expected, err
    assert "(dry run)" in err


@pytest.mark.parametrize("name", sorted(_calls()[0]))
def test_every_stage_failure_returns_ehip_and_stops(name, dry, capfd):
    calls, _ = _calls()
    fn, expected = calls[name]
    for i, st in enumerate(expected):
        dry(st)
        capfd.readouterr()
        assert fn() == L.EHIP, st
        err = capfd.readouterr().err
        # the failed stage is the last one reached: nothing is enqueued after it
        assert _stages(err) == expected[:i + 1], (st, err)
        assert f"stage {st}: injected failure" in err


def test_stats_reports_nothing_on_failure(dry, capfd):
    calls, n = _calls()
    fn, expected = calls["stats"]
    for st in expected:
        n.value = -5
        dry(st)
        assert fn() == L.EHIP
        assert n.value == -5, st  # the host output is left unwritten
    n.value = -5
    dry("no_such_stage")
    assert fn() == L.OK and n.value == 0


def test_validation_comes_before_any_stage(dry, capfd):
    """A bad argument is reported as such, not as a HIP failure, and reaches no stage."""
    lib = L.lib()
    dry("detect")
    capfd.readouterr()
    assert lib.int8_matmul(X, 300, 1000, 0, WQ, SW, 520, 6.0, Y, WS, BIG, None) == L.EINVAL   # K % 16
    assert lib.int8_matmul(X, 300, 1024, 0, WQ, SW, 520, float("nan"), Y, WS, BIG, None) == L.EINVAL
    assert lib.int8_matmul(X, 300, 1024, 0, WQ, SW, 520, 6.0, Y, WS, 1024, None) == L.EWORKSPACE
    assert lib.int8_quantize_weight(X, 1024, 520, 0, X + 64, SW, None) == L.EINVAL            # Wq overlaps W
    assert _stages(capfd.readouterr().err) == []


def test_log_names_the_call(monkeypatch, capfd):
    monkeypatch.setenv("LLMINT8_LOG", "1")
    monkeypatch.setenv("LLMINT8_FAULT", "no_such_stage")
    capfd.readouterr()
    assert L.lib().int8_matmul(X, 300, 1024, 1, WQ, SW, 520, 6.0, Y, WS, BIG, None) == L.OK
    err = capfd.readouterr().err
    assert "M=300 K=1024 N=520 dtype=bf16 threshold=6 path=tiled" in err
    assert "path=small_batch" not in err


def test_no_log_and_no_fault_by_default(monkeypatch, capfd):
    monkeypatch.delenv("LLMINT8_LOG", raising=False)
    monkeypatch.delenv("LLMINT8_FAULT", raising=False)
    capfd.readouterr()
    assert L.lib().int8_matmul(X, 300, 1000, 0, WQ, SW, 520, 6.0, Y, WS, BIG, None) == L.EINVAL
    assert capfd.readouterr().err == ""
