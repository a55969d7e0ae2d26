"""Which product kernel (small-batch, tiled, tiled with stream-K) each size takes, read
from the log of a dry run (LLMINT8_FAULT naming no stage: nothing is enqueued, no GPU)."""
import pytest

import int8_quantized_matmul_rowwise_amd as lm

MB = 0x100000


def route(M, K, N, monkeypatch, capfd):
    monkeypatch.setenv("LLMINT8_LOG", "1")
    monkeypatch.setenv("LLMINT8_FAULT", "no_such_stage")
    capfd.readouterr()
    assert lm.lib().int8_matmul(MB, M, K, 0, 2048 * MB, 4096 * MB, N, 6.0, 8192 * MB, 16384 * MB, 1 << 40,
                                None) == lm.OK
    err = capfd.readouterr().err
    line = [l for l in err.splitlines() if l.startswith("[llmint8] products")][0]
    return line.split("path=")[1].split()[0]


@pytest.mark.parametrize("M,K,N,path", [
    (4096, 12288, 36864, "tiled"),           # 2304 tiles: 9 per workgroup
    (8192, 28672, 8192, "tiled"),            # 1024 tiles
    (2048, 4096, 16384, "tiled"),            # 512 tiles
    (4600, 256, 7200, "tiled"),              # 522 tiles: past twice the grid
    (40, 256, 65536, "tiled"),               # 256 tiles, as many as the workgroups
    (32, 12288, 36864, "tiled_stream_k"),    # mid-size batches on the 175B-like QKV weight: 144 tiles
    (64, 12288, 36864, "tiled_stream_k"),
    (256, 12288, 36864, "tiled_stream_k"),
    (512, 12288, 36864, "tiled_stream_k"),   # 288 tiles
    (300, 1040, 520, "tiled_stream_k"),      # 6 tiles
    (16, 8192, 8192, "small_batch"),
    (64, 2048, 8192, "small_batch"),
    # past 64 rows: the small-batch path where the stream-K grid would fill under half the
    # compute units and X has under 2^20 elements (32 tiles, 2 or 3 workgroups each), else
    # stream-K
    (112, 8192, 8192, "small_batch"),
    (128, 8192, 8192, "tiled_stream_k"),
    (112, 4096, 8192, "small_batch"),
    (128, 2064, 7424, "small_batch"),
    (128, 16384, 8192, "tiled_stream_k"),
    (96, 4096, 16384, "tiled_stream_k"),
    (128, 12288, 36864, "tiled_stream_k"),
])
def test_product_kernel_routes(M, K, N, path, monkeypatch, capfd):
    assert route(M, K, N, monkeypatch, capfd) == path
