"""Parity of the fixed-outlier path (caller-supplied outlier dimensions, exact 16-bit W
rows) with the CPU oracle, through the C ABI: the weight conversion and the X pass bit
for bit, Y within the tolerance of the dynamic path (row-normwise 2e-3 and the a-priori
fp32 bound elementwise; bitwise when the set is empty)."""
import numpy as np
import pytest
import torch

import int8_quantized_matmul_rowwise_amd as lm
import oracle
import workloads
from tests.indep import f32_of, ulp16

pytestmark = pytest.mark.gpu


def _run(X, W, O, dt, rows=None):
    Od = torch.as_tensor(np.asarray(O, np.int32)).cuda()
    Xd, Wd = X.cuda(), W.cuda()
    Wq, s_w, WO = lm.int8_quantize_weight_fixed(Wd, Od)
    M, K = X.shape
    N = W.shape[1]
    ws = torch.empty(lm.int8_matmul_workspace_bytes(M, K, N), dtype=torch.uint8, device="cuda")
    Y = lm.int8_matmul_fixed(Xd, Od, Wq, s_w, WO, workspace=ws)
    torch.cuda.synchronize()
    Xb, Wb = workloads.bits(X), workloads.bits(W)
    Ou = np.unique(np.asarray(O, np.int32))  # the oracle takes the set ascending
    Wq_o, s_w_o, WO_o = oracle.quantize_weight_fixed(Wb, dt, Ou)
    assert np.array_equal(s_w.cpu().numpy().view(np.uint32), s_w_o.view(np.uint32)), "s_w differs"
    assert np.array_equal(Wq.cpu().numpy(), Wq_o), "Wq differs"
    wo = workloads.bits(WO.cpu())
    assert np.array_equal(wo[:, :Ou.size], WO_o) and not wo[:, Ou.size:].any(), "W_O differs"
    v = lm.workspace_views(ws, M, K, N, X.dtype)
    assert v["n_outliers"] == Ou.size and np.array_equal(v["outliers"].cpu().numpy(), Ou)
    Xq_o, s_x_o, XO_o = oracle.quantize_rows(Xb, dt, Ou)
    assert np.array_equal(v["s_x"].cpu().numpy().view(np.uint32), s_x_o.view(np.uint32)), "s_x differs"
    assert np.array_equal(v["Xq"].cpu().numpy(), Xq_o), "Xq differs"
    assert np.array_equal(workloads.bits(v["XO"].cpu())[:, :Ou.size], XO_o), "X[:,O] differs"
    res = oracle.matmul_fixed(Xb, dt, Wq_o, s_w_o, WO_o, Ou, rows)
    r = res["rows"]
    Yg = workloads.bits(Y.cpu())[r]
    if Ou.size == 0:
        assert np.array_equal(Yg, res["Y"]), "not bitwise with an empty set"
    yg, yo = f32_of(Yg, dt).astype(np.float64), f32_of(res["Y"], dt).astype(np.float64)
    d = np.abs(yg - yo)
    bound = ulp16(yo, dt) + 2 * (Ou.size + 2) * 2.0**-23 * (np.abs(res["y"].astype(np.float64)) + res["A"])
    assert np.all(d <= bound + 1e-30), f"T2: max excess {np.max(d - bound)}"
    nrm = np.linalg.norm(yo, axis=1)
    t1 = np.where(nrm > 0, np.linalg.norm(yg - yo, axis=1) / np.where(nrm > 0, nrm, 1), np.linalg.norm(yg - yo, axis=1))
    assert np.all(t1 <= 2e-3), f"T1 {t1.max()}"
    return {"n_outliers": int(Ou.size), "t1": float(t1.max())}


def _case(M, K, N, dt, seed):
    x, cols = workloads.make_x(M, K, dt, n_outliers=4, outlier_range=(8.0, 30.0), seed=seed, wid=62)
    w = workloads.make_w(K, N, dt, sigma=0.03, seed=seed, wid=62)
    return x, w, np.asarray(cols, np.int32)


@pytest.mark.parametrize("dt", ["fp16", "bf16"])
@pytest.mark.parametrize("M,K,N", [(300, 1040, 520), (40, 1040, 264), (1, 16, 8), (257, 272, 264), (16, 8192, 512)])
def test_fixed_parity(dt, M, K, N):
    print(f"\n[case] fixed {dt} {M}x{K}x{N}", flush=True)
    x, w, cols = _case(M, K, N, dt, seed=M + K)
    _run(x, w, cols, dt)


@pytest.mark.parametrize("dt", ["fp16", "bf16"])
def test_fixed_empty_and_full_sets(dt):
    x, w, _ = _case(130, 64, 40, dt, seed=3)
    _run(x, w, np.zeros(0, np.int32), dt)           # bitwise
    _run(x, w, np.arange(64, dtype=np.int32), dt)   # the whole product in 16 bits
    xs, ws_, _ = _case(20, 64, 40, dt, seed=4)
    _run(xs, ws_, np.arange(64, dtype=np.int32), dt)  # small-batch path


def test_fixed_unsorted_list_is_taken_as_a_set():
    # the X pass and the weight conversion each build the bitmap of the list, so the order of
    # the list does not matter for them (W_O follows the list, so the product needs it sorted)
    x, w, cols = _case(70, 256, 64, "fp16", seed=5)
    O = np.array([200, 7, 90], np.int32)
    Od = torch.as_tensor(O).cuda()
    Wq, s_w, WO = lm.int8_quantize_weight_fixed(w.cuda(), Od)
    Wq_o, s_w_o, _ = oracle.quantize_weight_fixed(workloads.bits(w), "fp16", np.sort(O))
    assert np.array_equal(Wq.cpu().numpy(), Wq_o)


@pytest.mark.parametrize("name", ["qkv_175b", "decode"])
def test_fixed_full_size_sampled(name):
    """The benchmarked shape, the workload's injected outlier columns as the fixed set."""
    x, w, cols, wl = workloads.make_workload(name)
    print(f"\n[case] fixed full size {name}", flush=True)
    rng = np.random.default_rng(12)
    rows = np.unique(np.concatenate([[0, wl.M - 1], rng.integers(0, wl.M, 6)])) if wl.M > 16 else None
    st = _run(x, w, np.sort(np.asarray(cols, np.int32)), wl.dtype, rows)
    print(f"[stats] {name}: {st}", flush=True)


def test_fixed_set_larger_than_one_launch_dimension():
    # n_O > 65535: the W_O gather covers the set with a capped grid (rows of W_O in a loop)
    M, K, N = 4, 66048, 8
    x, w, _ = _case(M, K, N, "fp16", seed=11)
    cols = np.arange(0, 65600, dtype=np.int32)
    print(f"\n[case] fixed {M}x{K}x{N} with {cols.size} outlier columns", flush=True)
    _run(x, w, cols, "fp16")


def _fixed_draw(i):
    # seeded: ragged M, K (% 16), N (% 8); a random ascending set of 0..80 columns, which need
    # not hold the injected large columns (those are then quantized like any other)
    rng = np.random.default_rng(3000 + i)
    while True:
        M = int(rng.integers(1, 129)) if i % 2 == 0 else int(rng.integers(129, 600))
        K = 16 * int(rng.integers(1, 500))
        N = 8 * int(rng.integers(1, 250))
        if M * K * N <= 3e9:
            break
    O = np.sort(rng.choice(K, size=int(rng.integers(0, min(K, 80) + 1)), replace=False)).astype(np.int32)
    return M, K, N, ("fp16" if rng.integers(2) else "bf16"), O


@pytest.mark.parametrize("i", range(16))
def test_fixed_seeded_shape_sweep(i):
    M, K, N, dt, O = _fixed_draw(i)
    route = "small-batch" if lm.int8_matmul_workspace_layout(M, K, N)["small_batch"] else "tiled"
    print(f"\n[case] fixed sweep {i}: {M}x{K}x{N} {dt} |O|={O.size} -> {route}", flush=True)
    x, w, _ = _case(M, K, N, dt, seed=200 + i)
    _run(x, w, O, dt)
