"""Parity of the HIP path with the CPU oracle (through the C-ABI), on seeded inputs.

Small and medium cases compare every element; the full-size workloads compare the
whole X pass and sampled rows of the products, in the same launch configuration the
benchmark times.  See tests/parity.py for the bars."""
import numpy as np
import pytest
import torch

import int8_quantized_matmul_rowwise_amd as lm
import oracle
import workloads
from tests import parity
from tests.indep import bits_of, f32_of
from tests.test_oracle_pipeline import _lattice_case

pytestmark = pytest.mark.gpu


def _case(M, K, N, dt, n_out=3, seed=0, rng=(6.5, 40.0), w_sigma=0.02):
    x, _ = workloads.make_x(M, K, dt, n_outliers=min(n_out, K), outlier_range=rng, seed=seed, wid=60)
    w = workloads.make_w(K, N, dt, sigma=w_sigma, seed=seed, wid=60)
    return x, w


def _banner(msg):
    print(f"\n[case] {msg}", flush=True)


def test_tiny_workload():
    x, w, cols, wl = workloads.make_workload("tiny")
    _banner("tiny 32x256x128 fp16")
    st = parity.run_case(x, w, wl.tau)
    assert st["n_outliers"] == 2


@pytest.mark.parametrize("dt", ["fp16", "bf16"])
def test_ragged_medium(dt):
    # several 256x256 tiles and a ragged tail in M, N and K (K = 8 * 128 + 16)
    _banner(f"ragged 300x1040x520 {dt}")
    x, w = _case(300, 1040, 520, dt, n_out=5, seed=1)
    st = parity.run_case(x, w, 6.0)
    assert st["n_outliers"] >= 5


@pytest.mark.parametrize("M,K,N,dt", [(1, 16, 8, "fp16"), (1, 4096, 264, "bf16"), (16, 8192, 512, "bf16"),
                                      (64, 1040, 264, "fp16"), (65, 1040, 264, "bf16"), (33, 32784, 24, "fp16"),
                                      (257, 272, 264, "fp16"), (513, 128, 8, "bf16"), (7, 32, 1032, "fp16")])
def test_edge_shapes(M, K, N, dt):
    _banner(f"edge {M}x{K}x{N} {dt}")
    x, w = _case(M, K, N, dt, n_out=2, seed=M + K + N)
    parity.run_case(x, w, 6.0)


@pytest.mark.parametrize("dt", ["fp16", "bf16"])
def test_threshold_exactly_tau_is_not_an_outlier(dt):
    _banner(f"x == tau {dt}")
    x, w = _case(64, 256, 136, dt, n_out=0, seed=3)
    x[5, 17] = 6.0
    x[9, 200] = -6.0
    x[11, 33] = 7.5
    st = parity.run_case(x, w, 6.0)
    assert st["n_outliers"] == 1


@pytest.mark.parametrize("dt", ["fp16", "bf16"])
@pytest.mark.parametrize("M", [40, 130])  # small-batch path and tiled path
def test_tau_zero_every_column_is_an_outlier(dt, M):
    # the degenerate 16-bit path: n_O = K (nine 32-wide chunks), C = 0, s_x = 0
    _banner(f"tau=0 {dt} M={M}")
    x, w = _case(M, 272, 72, dt, n_out=0, seed=4)
    st = parity.run_case(x, w, 0.0)
    assert st["n_outliers"] == 272


@pytest.mark.parametrize("dt", ["fp16", "bf16"])
def test_tau_inf_pure_vectorwise_is_bitwise(dt):
    _banner(f"tau=inf {dt}")
    x, w = _case(96, 512, 264, dt, n_out=4, seed=5)
    st = parity.run_case(x, w, float("inf"))
    assert st["n_outliers"] == 0 and st["n_ulp_flips"] == 0


def test_zero_rows_and_zero_weight_columns():
    _banner("zero rows / columns")
    x, w = _case(50, 320, 80, "fp16", n_out=2, seed=6)
    x[3] = 0
    x[10, :] = 0
    w[:, 7] = 0
    w[:, 64] = 0
    parity.run_case(x, w, 6.0)


@pytest.mark.parametrize("dt", ["fp16", "bf16"])
@pytest.mark.parametrize("M", [13, 70])  # small-batch path and tiled path
def test_lattice_closed_form_exact_on_gpu(dt, M):
    # power-of-two lattice: every step is exact, so Y must equal RN_T(exact) bitwise,
    # outlier part included (its sums are exact integers in any order)
    _banner(f"lattice {dt} M={M}")
    for seed in range(4):
        xl, wl_, tau, exact, cols = _lattice_case(dt, seed, M=M, K=320, N=136, out_cols=(3, 20, 41, 300))
        X = workloads.from_bits(bits_of(xl, dt), dt)
        W = workloads.from_bits(bits_of(wl_, dt), dt)
        Wq, s_w = lm.int8_quantize_weight(W.cuda())
        Y = lm.int8_matmul(X.cuda(), Wq, s_w, tau)
        with np.errstate(over="ignore"):
            ref = bits_of(exact.astype(np.float32), dt)
        assert np.array_equal(parity.to_bits(Y), ref), seed


def test_empty_batch_and_empty_features():
    _banner("M=0, K=0, N=0")
    Wq = torch.zeros(8, 64, dtype=torch.int8, device="cuda")
    s_w = torch.ones(8, device="cuda")
    Y = lm.int8_matmul(torch.zeros(0, 64, dtype=torch.float16, device="cuda"), Wq, s_w, 6.0)
    assert Y.shape == (0, 8)
    X = torch.randn(5, 0).to(torch.bfloat16).cuda()
    W = torch.zeros(0, 16, dtype=torch.bfloat16, device="cuda")
    Wq0, s0 = lm.int8_quantize_weight(W)
    assert torch.all(s0 == 0)
    Y = lm.int8_matmul(X, Wq0, s0, 6.0, Y=torch.full((5, 16), 7.0, dtype=torch.bfloat16, device="cuda"))
    torch.cuda.synchronize()
    assert torch.all(Y == 0) and not torch.signbit(Y.float()).any()
    Y = lm.int8_matmul(torch.randn(4, 32).half().cuda(), torch.zeros(0, 32, dtype=torch.int8, device="cuda"),
                       torch.zeros(0, device="cuda"), 6.0)
    assert Y.shape == (4, 0)


def test_determinism_and_stats():
    _banner("determinism + stats")
    x, w = _case(200, 1024, 384, "bf16", n_out=6, seed=7)
    Xd, Wd = x.cuda(), w.cuda()
    Wq, s_w = lm.int8_quantize_weight(Wd)
    Y1 = lm.int8_matmul(Xd, Wq, s_w, 6.0)
    Y2 = lm.int8_matmul(Xd, Wq, s_w, 6.0)
    torch.cuda.synchronize()
    assert torch.equal(Y1.view(torch.int16), Y2.view(torch.int16))
    n, cols = lm.int8_matmul_stats(Xd, 6.0)
    O = oracle.outlier_columns(workloads.bits(x), "bf16", 6.0)
    assert n == O.size and np.array_equal(cols.cpu().numpy(), O)
    n0, _ = lm.int8_matmul_stats(Xd, float("inf"))
    assert n0 == 0


def test_outputs_outside_y_untouched():
    # canaries around Y: the kernels write exactly M x N elements
    _banner("canaries")
    x, w = _case(70, 256, 136, "fp16", n_out=2, seed=8)
    Wq, s_w = lm.int8_quantize_weight(w.cuda())
    buf = torch.full((70 * 136 + 2048,), 12345.0, dtype=torch.float16, device="cuda")
    Y = buf[1024:1024 + 70 * 136].view(70, 136)
    lm.int8_matmul(x.cuda(), Wq, s_w, 6.0, Y=Y)
    torch.cuda.synchronize()
    assert torch.all(buf[:1024] == 12345.0) and torch.all(buf[1024 + 70 * 136:] == 12345.0)


_FULL = {}


def _full_inputs(name):
    if name not in _FULL:
        _FULL.clear()
        _FULL[name] = workloads.make_workload(name)
    return _FULL[name]


@pytest.mark.parametrize("name", ["ffn_up", "decode", "qkv_175b", "ffn_down"])
def test_full_size_workload_sampled(name):
    x, w, cols, wl = _full_inputs(name)
    _banner(f"full size {name} {wl.M}x{wl.K}x{wl.N} {wl.dtype}")
    rng = np.random.default_rng(11)
    rows = np.unique(np.concatenate([[0, wl.M - 1], rng.integers(0, wl.M, 6)])) if wl.M > 16 else None
    st = parity.run_case(x, w, wl.tau, rows=rows)
    assert st["n_outliers"] >= len(cols)
    print(f"[stats] {name}: {st}", flush=True)


def test_two_stage_calls_equal_the_one_call():
    _banner("prepare + products == int8_matmul")
    x, w = _case(130, 512, 264, "bf16", n_out=3, seed=9)
    Xd = x.cuda()
    Wq, s_w = lm.int8_quantize_weight(w.cuda())
    Y1 = lm.int8_matmul(Xd, Wq, s_w, 6.0)
    ws = lm.int8_matmul_prepare(Xd, Wq, 6.0)
    Y2 = lm.int8_matmul_products(130, 512, torch.bfloat16, Wq, s_w, ws)
    Y3 = lm.int8_matmul_products(130, 512, torch.bfloat16, Wq, s_w, ws)  # the workspace is reusable
    torch.cuda.synchronize()
    assert torch.equal(Y1.view(torch.int16), Y2.view(torch.int16))
    assert torch.equal(Y1.view(torch.int16), Y3.view(torch.int16))
