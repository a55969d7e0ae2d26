"""int8_matmul_noalloc: int8_matmul on the library's own static device scratch (for callers
that cannot allocate).  Checked through the C-ABI against int8_matmul with a caller
workspace -- the same kernels, so bitwise -- on consecutive calls whose sizes shrink (the
scratch keeps the previous call's contents), on both batch paths; and its argument checks,
including the size limit, on the CPU."""
import ctypes

import pytest
import torch

import int8_quantized_matmul_rowwise_amd as lm
import workloads

LIMIT = lm.NOALLOC_SCRATCH_BYTES


def _inputs(M, K, N, dt, seed):
    x, _ = workloads.make_x(M, K, dt, n_outliers=3, outlier_range=(6.5, 40.0), seed=seed, wid=61)
    w = workloads.make_w(K, N, dt, sigma=0.02, seed=seed, wid=61)
    return x, w


def test_noalloc_rejects_sizes_beyond_its_scratch():
    # argument checks run before any HIP call: these need no GPU
    lib = lm.lib()
    MB = 0x100000
    M, K, N = 4096, 12288, 36864
    assert lm.int8_matmul_workspace_bytes(M, K, N) > LIMIT
    assert lib.int8_matmul_noalloc(MB, M, K, 0, 512 * MB, 1024 * MB, N, 6.0, 2048 * MB, None) == lm.EWORKSPACE
    assert lm.int8_matmul_workspace_bytes(16, 8192, 8192) <= LIMIT  # a decode step fits
    assert lib.int8_matmul_noalloc(MB, 16, 8190, 0, 512 * MB, 1024 * MB, 64, 6.0, 2048 * MB, None) == lm.EINVAL
    assert lib.int8_matmul_noalloc(MB, 16, 8192, 0, 512 * MB, 1024 * MB, 64, float("nan"), 2048 * MB,
                                   None) == lm.EINVAL
    assert lib.int8_matmul_noalloc(MB, 16, 8192, 0, 512 * MB, 1024 * MB, 64, 6.0, None, None) == lm.EINVAL
    assert lib.int8_matmul_noalloc(None, 0, 8192, 0, 512 * MB, 1024 * MB, 64, 6.0, None, None) == lm.OK


def test_noalloc_dry_run_stages(monkeypatch, capfd):
    MB = 0x100000
    monkeypatch.setenv("LLMINT8_LOG", "1")
    lib = lm.lib()
    for fault, rc in (("no_such_stage", lm.OK), ("scratch_symbol", lm.EHIP), ("gemm_small", lm.EHIP)):
        monkeypatch.setenv("LLMINT8_FAULT", fault)
        capfd.readouterr()
        assert lib.int8_matmul_noalloc(MB, 16, 8192, 1, 512 * MB, 1024 * MB, 8192, 6.0, 2048 * MB, None) == rc
        err = capfd.readouterr().err
        assert "stage scratch_symbol" in err
        assert ("stage xpass_small" in err) == (fault != "scratch_symbol")


@pytest.mark.gpu
@pytest.mark.parametrize("shapes", [
    # small-batch path (a decode step, then a smaller one), tiled path (ragged, then smaller),
    # and a tiled call followed by a small-batch one
    [(16, 8192, 8192, "bf16"), (5, 4096, 1024, "bf16")],
    [(300, 1040, 520, "fp16"), (257, 272, 264, "fp16")],
    [(520, 512, 1032, "bf16"), (33, 1024, 264, "bf16")],
    [(300, 1024, 264, "fp16"), (260, 1024, 264, "fp16")],
])
def test_noalloc_equals_int8_matmul(shapes):
    for i, (M, K, N, dt) in enumerate(shapes):
        print(f"\n[case] noalloc call {i}: {M}x{K}x{N} {dt}", flush=True)
        assert lm.int8_matmul_workspace_bytes(M, K, N) <= LIMIT
        x, w = _inputs(M, K, N, dt, seed=M + K + N)
        X, W = x.cuda(), w.cuda()
        Wq, s_w = lm.int8_quantize_weight(W)
        # the reference call's workspace starts as garbage: no region needs to start at zero
        ws = torch.full((lm.int8_matmul_workspace_bytes(M, K, N),), 0x5A, dtype=torch.uint8, device="cuda")
        Y_ref = lm.int8_matmul(X, Wq, s_w, 6.0, workspace=ws)
        Y = torch.full((M, N), 3.0, dtype=X.dtype, device="cuda")
        lm.int8_matmul_noalloc(X, Wq, s_w, 6.0, Y=Y)
        torch.cuda.synchronize()
        assert torch.equal(Y.view(torch.int16), Y_ref.view(torch.int16)), (i, M, K, N)


@pytest.mark.gpu
def test_noalloc_too_large_leaves_y_alone():
    M, K, N = 1024, 4096, 8192
    assert lm.int8_matmul_workspace_bytes(M, K, N) > LIMIT
    X = torch.zeros((M, K), dtype=torch.float16, device="cuda")
    Wq = torch.zeros((N, K), dtype=torch.int8, device="cuda")
    s_w = torch.ones(N, device="cuda")
    Y = torch.full((M, N), 7.0, dtype=torch.float16, device="cuda")
    with pytest.raises(lm.LLMInt8Error) as e:
        lm.int8_matmul_noalloc(X, Wq, s_w, 6.0, Y=Y)
    assert e.value.status == lm.EWORKSPACE
    torch.cuda.synchronize()
    assert torch.all(Y == 7.0)


@pytest.mark.gpu
@pytest.mark.parametrize("M,K,N,dt", [(16, 2048, 264, "bf16"), (300, 1040, 520, "fp16")])
def test_noalloc_call_replays_from_a_graph(M, K, N, dt):
    """Captured once in a HIP graph (the case it is for) and replayed on new X contents, with
    eager work between the replays: every replay equals the eager int8_matmul bit for bit."""
    print(f"\n[case] graph int8_matmul_noalloc {M}x{K}x{N} {dt}", flush=True)
    x, w = _inputs(M, K, N, dt, seed=M)
    X, W = x.cuda(), w.cuda()
    Wq, s_w = lm.int8_quantize_weight(W)
    Y = torch.empty((M, N), dtype=X.dtype, device="cuda")
    lm.int8_matmul_noalloc(X, Wq, s_w, 6.0, Y=Y)  # the first call on the device, outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        lm.int8_matmul_noalloc(X, Wq, s_w, 6.0, Y=Y)
    torch.cuda.synchronize()
    for r in range(3):
        X.copy_(_inputs(M, K, N, dt, seed=300 + r)[0].cuda())
        ref = lm.int8_matmul(X, Wq, s_w, 6.0)
        torch.cuda.synchronize()
        Y.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(Y.view(torch.int16), ref.view(torch.int16)), f"replay {r} differs"
