"""The product path under HIP graph capture: every library call only enqueues kernels on
the caller's stream (no allocation, no memset node, no host synchronisation), so a caller
can capture it once and replay it.  Each replay runs on the inputs' current contents and
must equal the eager call bit for bit; eager work and synchronisations run between the
replays."""
import pytest
import torch

import int8_quantized_matmul_rowwise_amd as lm
import workloads

pytestmark = pytest.mark.gpu


def _inputs(M, K, N, dt, seed):
    x, _ = workloads.make_x(M, K, dt, n_outliers=3, outlier_range=(8.0, 30.0), seed=seed, wid=80)
    w = workloads.make_w(K, N, dt, sigma=0.02, seed=seed, wid=80)
    return x.cuda(), w.cuda()


@pytest.mark.parametrize("M,K,N,dt", [(300, 1040, 520, "fp16"), (16, 2048, 264, "bf16"),
                                      (300, 4096, 264, "fp16"),
                                      # tiled stream-K after the slab X pass, whose coding launch
                                      # zeroes the tile counters and gathers W_O
                                      (64, 1024, 36864, "bf16")])
def test_vectorwise_call_replays_from_a_graph(M, K, N, dt):
    print(f"\n[case] graph int8_matmul {dt} {M}x{K}x{N}", flush=True)
    X, W = _inputs(M, K, N, dt, seed=M)
    Wq, s_w = lm.int8_quantize_weight(W)
    ws = torch.empty(lm.int8_matmul_workspace_bytes(M, K, N), dtype=torch.uint8, device="cuda")
    Y = torch.empty((M, N), dtype=X.dtype, device="cuda")
    lm.int8_matmul(X, Wq, s_w, 6.0, Y=Y, workspace=ws)  # warm up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        lm.int8_matmul(X, Wq, s_w, 6.0, Y=Y, workspace=ws)
    torch.cuda.synchronize()
    for r in range(4):
        # new contents for X (a different outlier pattern each time), eager reference first
        X.copy_(_inputs(M, K, N, dt, seed=100 + r)[0])
        ref = lm.int8_matmul(X, Wq, s_w, 6.0)
        torch.cuda.synchronize()
        Y.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(Y.view(torch.int16), ref.view(torch.int16)), f"replay {r} differs"


@pytest.mark.parametrize("M,K,N,G", [(300, 2048, 264, 512),   # the tiled group kernel
                                     (24, 2048, 264, 256)])   # the split-N small-batch group kernel
def test_groupwise_call_replays_from_a_graph(M, K, N, G):
    assert lm.int8_matmul_group_small_batch(M, K, N, G) == (M <= 64)
    print(f"\n[case] graph int8_matmul_group fp16 {M}x{K}x{N} G={G}", flush=True)
    X, W = _inputs(M, K, N, "fp16", seed=7)
    Wq, s_w = lm.int8_quantize_weight_group(W, G)
    ws = torch.empty(lm.int8_matmul_group_workspace_bytes(M, K, G), dtype=torch.uint8, device="cuda")
    Y = torch.empty((M, N), dtype=X.dtype, device="cuda")
    lm.int8_matmul_group(X, Wq, s_w, G, Y=Y, workspace=ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        lm.int8_matmul_group(X, Wq, s_w, G, Y=Y, workspace=ws)
    torch.cuda.synchronize()
    for r in range(3):
        X.copy_(_inputs(M, K, N, "fp16", seed=200 + r)[0])
        ref = lm.int8_matmul_group(X, Wq, s_w, G)
        torch.cuda.synchronize()
        Y.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(Y.view(torch.int16), ref.view(torch.int16)), f"replay {r} differs"
