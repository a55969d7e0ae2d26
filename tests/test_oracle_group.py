"""Pins of the oracle's group-wise variant (one scale per group of G consecutive input
features, for each row of X and each column of W; the int32 partial of every group is
dequantized and summed in fp32, groups ascending).  None re-types the variant: G = K must
reduce to the (pinned) vector-wise path at tau = inf, each group's codes must be the pinned
scalar quantizer's, exact lattices give a closed form, and fp32 summation stays within its
a-priori bound of the float64 sum."""
import numpy as np
import pytest

import oracle
import workloads
from tests.indep import bits_of, f32_of

DTS = ["fp16", "bf16"]


def _rand(dt, M, K, N, seed):
    x, _ = workloads.make_x(M, K, dt, n_outliers=2, outlier_range=(8.0, 30.0), seed=seed, wid=63)
    w = workloads.make_w(K, N, dt, sigma=0.05, seed=seed, wid=63)
    return workloads.bits(x), workloads.bits(w)


@pytest.mark.parametrize("dt", DTS)
def test_group_equal_to_k_is_vectorwise_at_tau_inf(dt):
    X, W = _rand(dt, 9, 256, 24, seed=1)
    Xq, s_x = oracle.group_quantize_rows(X, dt, 256)
    Wq, s_w = oracle.group_quantize_weight(W, dt, 256)
    Xq_v, s_x_v, _ = oracle.quantize_rows(X, dt, np.zeros(0, np.int32))
    Wq_v, s_w_v = oracle.quantize_weight(W, dt)
    assert np.array_equal(Xq, Xq_v) and np.array_equal(s_x[:, 0], s_x_v)
    assert np.array_equal(Wq, Wq_v) and np.array_equal(s_w[:, 0], s_w_v)
    _, Y = oracle.group_gemm(Xq, s_x, Wq, s_w, 256, dt)
    assert np.array_equal(Y, oracle.matmul(X, dt, Wq_v, s_w_v, float("inf"))["Y"])


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("G", [16, 64, 128])
def test_group_codes_use_the_scalar_quantizer(dt, G):
    X, W = _rand(dt, 5, 256, 12, seed=G)
    Xq, s_x = oracle.group_quantize_rows(X, dt, G)
    Wq, s_w = oracle.group_quantize_weight(W, dt, G)
    Xf, Wf = f32_of(X, dt), f32_of(W, dt)
    for g in range(256 // G):
        sl = slice(g * G, (g + 1) * G)
        for i in range(5):
            assert s_x[i, g] == np.abs(Xf[i, sl]).max()
            assert np.array_equal(Xq[i, sl], oracle.quantize(Xf[i, sl], float(s_x[i, g])))
        for n in range(12):
            assert s_w[n, g] == np.abs(Wf[sl, n]).max()
            assert np.array_equal(Wq[n, sl], oracle.quantize(Wf[sl, n], float(s_w[n, g])))


def _group_lattice(seed, M=5, K=96, N=7, G=32):
    """x[i,k] = q 2^(e_i + d_g), w[k,n] = p 2^(f_n - d_g), |q|, |p| <= 127 with 127 reached in
    every row group / column group.  Then r_ig = 2^(e_i + d_g), c_ng = 2^(f_n - d_g), every
    group term is (q_g . p_g) 2^(e_i + f_n) exactly, and so is their running fp32 sum."""
    rng = np.random.default_rng(seed)
    ng = K // G
    e = rng.integers(-3, 3, M)
    f = rng.integers(-10, -5, N)
    d = rng.integers(-4, 5, ng)
    q = rng.integers(-127, 128, (M, K))
    p = rng.integers(-127, 128, (K, N))
    for g in range(ng):
        q[:, g * G + rng.integers(0, G)] = 127
        p[g * G + rng.integers(0, G, N), np.arange(N)] = -127
    dk = np.repeat(d, G)
    x = (q * np.exp2(e[:, None] + dk[None, :])).astype(np.float32)
    w = (p * np.exp2(f[None, :] - dk[:, None])).astype(np.float32)
    exact = (q @ p).astype(np.float64) * np.exp2(e[:, None] + f[None, :])
    return x, w, exact, G


@pytest.mark.parametrize("dt", DTS)
def test_group_lattice_closed_form(dt):
    for seed in range(20):
        x, w, exact, G = _group_lattice(seed)
        X, W = bits_of(x, dt), bits_of(w, dt)
        assert np.array_equal(f32_of(X, dt), x) and np.array_equal(f32_of(W, dt), w)
        Xq, s_x = oracle.group_quantize_rows(X, dt, G)
        Wq, s_w = oracle.group_quantize_weight(W, dt, G)
        y, Y = oracle.group_gemm(Xq, s_x, Wq, s_w, G, dt)
        assert np.array_equal(y.astype(np.float64), exact), seed
        assert np.array_equal(Y, bits_of(exact.astype(np.float32), dt)), seed


@pytest.mark.parametrize("dt", DTS)
def test_group_fp32_sum_within_its_bound(dt):
    G, K = 32, 512
    X, W = _rand(dt, 6, K, 10, seed=9)
    Xq, s_x = oracle.group_quantize_rows(X, dt, G)
    Wq, s_w = oracle.group_quantize_weight(W, dt, G)
    y, _ = oracle.group_gemm(Xq, s_x, Wq, s_w, G, dt)
    # float64 sum of the per-group terms (each term: two fp32 roundings of an exact product)
    ng = K // G
    C = np.stack([Xq[:, g * G:(g + 1) * G].astype(np.int64) @ Wq[:, g * G:(g + 1) * G].T.astype(np.int64)
                  for g in range(ng)])
    r = (s_x / np.float32(127.0)).astype(np.float32)
    c = (s_w / np.float32(127.0)).astype(np.float32)
    terms = np.stack([(C[g].astype(np.float32) * r[:, g:g + 1]).astype(np.float32) * c[None, :, g]
                      for g in range(ng)]).astype(np.float64)
    exact = terms.sum(axis=0)
    bound = ng * 2.0**-24 * np.abs(terms).sum(axis=0) + 1e-30
    assert np.all(np.abs(y - exact) <= bound)
