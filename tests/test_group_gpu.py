"""Parity of the group-wise path (one scale per group of G features along K for every row
of X and column of W) with the CPU oracle, through the C ABI.  The codes, the scales and
the dequantization factors are compared bit for bit; so is Y: the kernel takes the same
fp32 operations in the same order as the oracle (per group: the exact int32 partial, two
products, one sum, groups ascending), so any difference is a defect."""
import numpy as np
import pytest
import torch

import int8_quantized_matmul_rowwise_amd as lm
import oracle
import workloads

pytestmark = pytest.mark.gpu


def _u32(a):
    return np.ascontiguousarray(a, np.float32).view(np.uint32)


def _run(X, W, dt, G, rows=None, check_weight=True):
    M, K = X.shape
    N = W.shape[1]
    Xd, Wd = X.cuda(), W.cuda()
    Wq, s_w = lm.int8_quantize_weight_group(Wd, G)
    ws = torch.empty(lm.int8_matmul_group_workspace_bytes(M, K, G), dtype=torch.uint8, device="cuda")
    Y = lm.int8_matmul_group(Xd, Wq, s_w, G, workspace=ws)
    torch.cuda.synchronize()
    Xb, Wb = workloads.bits(X), workloads.bits(W)
    Wq_c, s_w_c = Wq.cpu().numpy(), s_w.cpu().numpy()
    if check_weight:
        Wq_o, s_w_o = oracle.group_quantize_weight(Wb, dt, G)
        assert np.array_equal(_u32(s_w_c), _u32(s_w_o)), "s_w differs"
        assert np.array_equal(Wq_c, Wq_o), "Wq differs"
    Xq_o, s_x_o = oracle.group_quantize_rows(Xb, dt, G)
    v = lm.group_workspace_views(ws, M, K, G)
    assert np.array_equal(_u32(v["s_x"].cpu().numpy()), _u32(s_x_o)), "s_x differs"
    assert np.array_equal(v["Xq"].cpu().numpy(), Xq_o), "Xq differs"
    r_o = (s_x_o / np.float32(127.0)).astype(np.float32).T  # fp32 division, correctly rounded
    assert np.array_equal(_u32(v["r"].cpu().numpy()), _u32(r_o)), "dequantization factors differ"
    # the products take the oracle's weight codes: equal to the kernel's when checked above
    y_o, Y_o = oracle.group_gemm(Xq_o, s_x_o, Wq_c, s_w_c, G, dt, rows)
    Yg = workloads.bits(Y.cpu())
    Yg = Yg if rows is None else Yg[np.asarray(rows)]
    assert np.count_nonzero(Y_o) > 0 or not (Xq_o.any() and Wq_c.any()), "degenerate case"
    bad = np.argwhere(Yg != Y_o)
    assert bad.size == 0, f"Y differs at {bad.shape[0]} elements, first {bad[:4].tolist()}"
    return Y


def _case(M, K, N, dt, seed, n_outliers=3):
    x, _ = workloads.make_x(M, K, dt, n_outliers=n_outliers, outlier_range=(8.0, 40.0), seed=seed, wid=70)
    w = workloads.make_w(K, N, dt, sigma=0.02, seed=seed, wid=70)
    return x, w


@pytest.mark.parametrize("dt", ["fp16", "bf16"])
@pytest.mark.parametrize("M,K,N,G", [
    (300, 1024, 264, 128),    # 2 x 3 tiles, ragged in M and N; one stage per group
    (300, 2048, 520, 512),    # four stages per group
    (257, 768, 136, 256),     # three groups of two stages
    (64, 8192, 128, 4096),    # the largest group
    (513, 3072, 392, 1024),   # three groups of 1024 (the group size the pages' GPTQ snippet uses)
    (1, 128, 8, 128),         # one row, one group, one 8-column segment
    # small batches (the split-N group kernel): 16-step groups, 2-step groups split over two
    # of the four waves, three row groups with a ragged last column group
    (16, 8192, 512, 1024),
    (48, 2048, 264, 128),
    (33, 1536, 8200, 512),
    # 17 to 32 rows: two row groups of the split-N group kernel
    (24, 2048, 264, 256),
])
def test_group_parity(dt, M, K, N, G):
    print(f"\n[case] group {dt} {M}x{K}x{N} G={G}", flush=True)
    x, w = _case(M, K, N, dt, seed=M + K + G)
    _run(x, w, dt, G)


@pytest.mark.parametrize("K,G,dt", [(128, 128, "fp16"), (256, 128, "bf16"), (384, 128, "fp16")])
def test_group_several_tiles_per_workgroup(K, G, dt):
    # 17 x 17 = 289 tiles of 256 x 128 on 256 workgroups: some take two tiles, and the
    # operand loads run one (K = 128: one stage per tile) or two tiles ahead; ragged in M
    # and N; rows sampled in the first, a middle and the last row tile
    M, N = 4200, 2056
    print(f"\n[case] group several tiles per workgroup {dt} {M}x{K}x{N} G={G}", flush=True)
    x, w = _case(M, K, N, dt, seed=K + 1)
    rng = np.random.default_rng(K)
    rows = np.unique(np.concatenate([[0, 255, 256, 2047, 4095, 4096, M - 1], rng.integers(0, M, 5)]))
    _run(x, w, dt, G, rows=rows)


def test_group_equals_vectorwise_at_one_group():
    # G = K: one scale per row and column, the vector-wise code; with no outlier above the
    # threshold the vector-wise path's Y is RN_T(RN32(RN32(C * r) * c)), the same as one group
    x, w = _case(200, 1024, 136, "fp16", seed=5, n_outliers=0)
    Y = _run(x, w, "fp16", 1024)
    Wq, s = lm.int8_quantize_weight(w.cuda())
    Yv = lm.int8_matmul(x.cuda(), Wq, s, threshold=float("inf"))
    assert torch.equal(Y.view(torch.int16), Yv.view(torch.int16))


def test_group_zero_groups_and_zero_rows():
    # a row group that is all zero has scale 0 and codes 0; a zero weight group likewise
    x, w = _case(70, 512, 64, "bf16", seed=6)
    x[3, :] = 0
    x[5, 128:256] = 0
    w[256:384, 7] = 0
    w[:, 9] = 0
    _run(x, w, "bf16", 128)


def test_group_empty_shapes():
    X = torch.zeros((0, 256), dtype=torch.float16, device="cuda")
    Wq = torch.zeros((16, 256), dtype=torch.int8, device="cuda")
    s = torch.zeros((16, 2), dtype=torch.float32, device="cuda")
    assert lm.int8_matmul_group(X, Wq, s, 128).shape == (0, 16)
    # K = 0: the empty sum, Y = 0 (any group size is accepted)
    X0 = torch.zeros((5, 0), dtype=torch.bfloat16, device="cuda")
    Y = torch.full((5, 16), 3.0, dtype=torch.bfloat16, device="cuda")
    lm.lib().int8_matmul_group(X0.data_ptr() or None, 5, 0, 1, 128, None, None, 16, Y.data_ptr(), None, 0, None)
    torch.cuda.synchronize()
    assert not Y.float().any()


def test_group_rejects_bad_group_sizes():
    x, w = _case(8, 384, 16, "fp16", seed=7)
    with pytest.raises(lm.LLMInt8Error):
        lm.int8_quantize_weight_group(w.cuda(), 192)
    Wq, s = lm.int8_quantize_weight_group(w.cuda(), 128)
    with pytest.raises(ValueError):
        lm.int8_matmul_group(x.cuda(), Wq, s, 256)


def test_group_full_size_qkv_175b_sampled():
    # the benchmarked configuration: 4096 x 12288 x 36864 fp16, G = 1024; weight and X pass
    # compared in full, Y on sampled rows (first and last tile rows included)
    x, w, _, wl = workloads.make_workload("qkv_175b")
    print(f"\n[case] group full size qkv_175b {wl.M}x{wl.K}x{wl.N} G=1024", flush=True)
    rng = np.random.default_rng(12)
    rows = np.unique(np.concatenate([[0, 255, 256, wl.M - 1], rng.integers(0, wl.M, 4)]))
    _run(x, w, wl.dtype, 1024, rows=rows)


def test_group_two_stage_calls_equal_the_one_call():
    # one X pass serves two weights of the same K and group size
    x, w = _case(300, 2048, 264, "bf16", seed=8)
    _, w2 = _case(300, 2048, 136, "bf16", seed=9)
    Xd = x.cuda()
    Wq, s = lm.int8_quantize_weight_group(w.cuda(), 256)
    Wq2, s2 = lm.int8_quantize_weight_group(w2.cuda(), 256)
    ws = torch.empty(lm.int8_matmul_group_workspace_bytes(300, 2048, 256), dtype=torch.uint8, device="cuda")
    lm.int8_matmul_group_prepare(Xd, 256, ws)
    Ya = lm.int8_matmul_group_products(300, 2048, Xd.dtype, 256, Wq, s, ws)
    Yb = lm.int8_matmul_group_products(300, 2048, Xd.dtype, 256, Wq2, s2, ws)
    assert torch.equal(Ya.view(torch.int16), lm.int8_matmul_group(Xd, Wq, s, 256).view(torch.int16))
    assert torch.equal(Yb.view(torch.int16), lm.int8_matmul_group(Xd, Wq2, s2, 256).view(torch.int16))


def _group_draw(i):
    # seeded: G a power of two in [128, 4096], K a multiple of it, ragged M and N (N % 8 = 0)
    rng = np.random.default_rng(2000 + i)
    while True:
        G = int(2 ** rng.integers(7, 13))
        K = G * int(rng.integers(1, max(2, 16384 // G) + 1))
        M = int(rng.integers(1, 65)) if i % 2 == 0 else int(rng.integers(65, 600))
        N = 8 * int(rng.integers(1, 400))
        if M * N * K <= 3e9 and K <= 16384:
            return M, K, N, G, ("fp16" if rng.integers(2) else "bf16"), int(rng.integers(0, 6))


@pytest.mark.parametrize("i", range(24))
def test_group_seeded_shape_sweep(i):
    """Seeded shapes over both group-wise product kernels (small batches on even draws),
    Y compared bit for bit with the oracle."""
    M, K, N, G, dt, n_out = _group_draw(i)
    route = "small-batch" if lm.int8_matmul_group_small_batch(M, K, N, G) else "tiled"
    print(f"\n[case] group sweep {i}: {M}x{K}x{N} G={G} {dt} injected={n_out} -> {route}", flush=True)
    x, w = _case(M, K, N, dt, seed=100 + i, n_outliers=n_out)
    _run(x, w, dt, G)
