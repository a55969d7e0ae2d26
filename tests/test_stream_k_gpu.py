"""Stream-K on the tiled path (fewer 256 x 256 output tiles than twice the 256 workgroups,
and not a multiple of them): the tiles' K stages are split over all workgroups, the parts
of a tile exchange exact int32 partial sums and the last one runs the epilogue.  Against
the oracle through the C ABI (O, s_x, Xq, X[:,O], W_O bit for bit, C exactly, Y within the
gates of tests/parity.py), including the batch sizes of a mid-size call on the 175B-like
QKV weight; the log confirms the route.  Calls of at most 128 rows also take the half-tile
mode (the waves of tile rows 128..255 only load and wait), with and without the split."""
import numpy as np
import pytest
import torch

import int8_quantized_matmul_rowwise_amd as lm
import oracle
import workloads
from tests import parity

pytestmark = pytest.mark.gpu


def _route(M, K, N, capfd, monkeypatch):
    monkeypatch.setenv("LLMINT8_LOG", "1")
    monkeypatch.setenv("LLMINT8_FAULT", "no_such_stage")  # a dry run: the route, nothing enqueued
    capfd.readouterr()
    MB = 0x100000
    assert lm.lib().int8_matmul(MB, M, K, 0, 2048 * MB, 4096 * MB, N, 6.0, 8192 * MB, 16384 * MB, 1 << 40,
                                None) == lm.OK
    err = capfd.readouterr().err
    monkeypatch.delenv("LLMINT8_LOG")
    monkeypatch.delenv("LLMINT8_FAULT")
    return "stream_k" if "path=tiled_stream_k" in err else ("tiled" if "path=tiled" in err else "small")


def _case(M, K, N, dt, seed):
    x, _ = workloads.make_x(M, K, dt, n_outliers=4, outlier_range=(6.5, 40.0), seed=seed, wid=97)
    w = workloads.make_w(K, N, dt, sigma=0.02, seed=seed, wid=97)
    return x, w


@pytest.mark.parametrize("M,K,N,dt", [
    (200, 2048, 8192, "fp16"),   # 32 tiles of 16 stages: 2 stages per workgroup, 8 parts per tile
    (256, 12288, 4096, "bf16"),  # 16 tiles of 96 stages: 16 parts per tile
    (130, 4096, 9000, "fp16"),   # 36 ragged tiles: parts cross tile boundaries unevenly
    (300, 1040, 520, "bf16"),    # 6 tiles of 9 stages (the last partial): one stage per part
    (513, 400, 2056, "fp16"),    # 27 tiles in 3 row tiles, 4 stages
    (24, 1024, 36864, "bf16"),   # a small batch on a wide weight: 144 tiles
])
def test_stream_k_parity(M, K, N, dt, capfd, monkeypatch):
    assert _route(M, K, N, capfd, monkeypatch) == "stream_k"
    print(f"\n[case] stream-K {M}x{K}x{N} {dt}", flush=True)
    x, w = _case(M, K, N, dt, seed=M + N)
    rows = None if M * N * K <= 2 ** 31 else np.unique(np.concatenate([[0, M - 1], np.arange(1, M, 37)]))
    st = parity.run_case(x, w, 6.0, rows=rows)
    assert st["n_outliers"] >= 4


def test_whole_tiles_past_twice_the_grid():
    # 522 tiles (18 x 29, ragged in M and N): the persistent kernel without the split, two or
    # three tiles per workgroup
    M, K, N = 4600, 256, 7200
    print(f"\n[case] whole tiles {M}x{K}x{N}", flush=True)
    x, w = _case(M, K, N, "bf16", seed=3)
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, 255, 256, M - 1], rng.integers(0, M, 12)]))
    parity.run_case(x, w, 6.0, rows=rows)


def test_half_tiles_without_the_split(capfd, monkeypatch):
    # 40 rows on 256 whole tiles (as many as the workgroups: no split), half-tile mode
    M, K, N = 40, 256, 65536
    assert _route(M, K, N, capfd, monkeypatch) == "tiled"
    print(f"\n[case] half tiles {M}x{K}x{N}", flush=True)
    x, w = _case(M, K, N, "fp16", seed=17)
    parity.run_case(x, w, 6.0)


_QKV = {}


def _qkv_weight():
    if not _QKV:
        x, w, cols, wl = workloads.make_workload("qkv_175b", rows=1)
        Wq, s_w = lm.int8_quantize_weight(w.cuda())
        torch.cuda.synchronize()
        Wq_o, s_w_o = parity.check_weight(w, Wq, s_w)
        _QKV["w"] = (Wq, s_w, Wq_o, s_w_o)
        _QKV["wl"] = wl
    return _QKV["w"], _QKV["wl"]


@pytest.mark.parametrize("M", [32, 64, 128, 256])
def test_mid_size_batches_on_the_qkv_weight(M, capfd, monkeypatch):
    """A mid-size call (M rows of the workload's X) on the 175B-like QKV weight, 12288 x
    36864: 144 tiles, split over all workgroups; 8 sampled rows against the oracle."""
    wq, wl = _qkv_weight()
    assert _route(M, wl.K, wl.N, capfd, monkeypatch) == "stream_k"
    print(f"\n[case] mid-size M={M} on the qkv weight", flush=True)
    x, w, cols, _ = workloads.make_workload("qkv_175b", rows=M)
    rng = np.random.default_rng(M)
    rows = np.unique(np.concatenate([[0, M - 1], rng.integers(0, M, 6)]))
    st = parity.run_case(x, w, wl.tau, rows=rows, Wq_s=wq)
    assert st["n_outliers"] >= len(cols)


@pytest.mark.parametrize("M,K,N", [(130, 4096, 9000),   # the row coding zeroes the counters
                                   (64, 2048, 36864)])  # the slab X pass zeroes them
def test_repeated_products_on_one_workspace(M, K, N):
    # the tile counters are left at zero by every call: the products run three times on one
    # prepared workspace and give the same bits each time
    x, w = _case(M, K, N, "fp16", seed=11)
    Xd = x.cuda()
    Wq, s_w = lm.int8_quantize_weight(w.cuda())
    ws = lm.int8_matmul_prepare(Xd, Wq, 6.0)
    Ys = [lm.int8_matmul_products(M, K, torch.float16, Wq, s_w, ws) for _ in range(3)]
    ref = lm.int8_matmul(Xd, Wq, s_w, 6.0)
    torch.cuda.synchronize()
    for Y in Ys:
        assert torch.equal(Y.view(torch.int16), ref.view(torch.int16))
