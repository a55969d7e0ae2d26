"""Pins of the oracle's fixed-outlier variant (caller-supplied outlier dimensions; their
W rows kept exactly in 16 bits).  None re-types the variant: the empty set must reduce to
the (pinned) dynamic path at tau = inf, the full set to a float64 textbook product, exact
lattices to a closed form, and the weight conversion to the pinned scalar quantizer."""
import numpy as np
import pytest

import oracle
import workloads
from tests.indep import bits_of, f32_of

DTS = ["fp16", "bf16"]


def _rand(dt, M, K, N, seed):
    x, _ = workloads.make_x(M, K, dt, n_outliers=3, outlier_range=(8.0, 30.0), seed=seed, wid=61)
    w = workloads.make_w(K, N, dt, sigma=0.05, seed=seed, wid=61)
    return workloads.bits(x), workloads.bits(w)


@pytest.mark.parametrize("dt", DTS)
def test_fixed_empty_set_is_the_dynamic_path_at_tau_inf(dt):
    X, W = _rand(dt, 9, 64, 24, seed=1)
    O = np.zeros(0, np.int32)
    Wq, s_w, WO = oracle.quantize_weight_fixed(W, dt, O)
    Wq_d, s_w_d = oracle.quantize_weight(W, dt)
    assert np.array_equal(Wq, Wq_d) and np.array_equal(s_w.view(np.uint32), s_w_d.view(np.uint32))
    assert WO.shape == (24, 0)
    res = oracle.matmul_fixed(X, dt, Wq, s_w, WO, O)
    ref = oracle.matmul(X, dt, Wq_d, s_w_d, float("inf"))
    assert np.array_equal(res["Y"], ref["Y"])


@pytest.mark.parametrize("dt", DTS)
def test_fixed_all_columns_is_the_16bit_product(dt):
    M, K, N = 7, 48, 13
    X, W = _rand(dt, M, K, N, seed=2)
    O = np.arange(K, dtype=np.int32)
    Wq, s_w, WO = oracle.quantize_weight_fixed(W, dt, O)
    assert not Wq.any() and not s_w.any()
    assert np.array_equal(WO, W.T)
    res = oracle.matmul_fixed(X, dt, Wq, s_w, WO, O)
    assert not res["Xq"].any() and not res["s_x"].any() and not res["C"].any()
    exact = f32_of(X, dt).astype(np.float64) @ f32_of(W, dt).astype(np.float64)
    A = np.abs(f32_of(X, dt).astype(np.float64)) @ np.abs(f32_of(W, dt).astype(np.float64))
    assert np.all(np.abs(res["F"] - exact) <= K * 2.0**-23 * A + 1e-30)
    # with C = 0 the epilogue is the 16-bit rounding of F itself
    assert np.array_equal(res["Y"], bits_of(res["F"], dt))


def _fixed_lattice(seed, M=6, K=40, N=9, out=(2, 17, 33)):
    """x = q 2^e_i, w = p 2^f_n: |q| <= 127 off O with row max 127, |q| in [129, 199] on O;
    |p| <= 127 off O with column max 127 off O, |p| <= 255 on O (all exact in fp16 and bf16).
    Then Xq = q off O, Wq = p off O, r_i = 2^e_i, c_n = 2^f_n, the int8 part is
    2^(e+f) q_off p_off and the exact 16-bit part 2^(e+f) q_O p_O, each fp32 step exact:
    y = 2^(e_i + f_n) (q @ p)[i, n]."""
    rng = np.random.default_rng(seed)
    O = np.array(out)
    off = np.setdiff1d(np.arange(K), O)
    e = rng.integers(-4, 3, M)
    f = rng.integers(-12, -6, N)
    q = rng.integers(-127, 128, (M, K))
    q[:, off[0]] = 127 * rng.choice([-1, 1], M)
    q[:, O] = rng.integers(129, 200, (M, O.size)) * rng.choice([-1, 1], (M, O.size))
    p = rng.integers(-127, 128, (K, N))
    p[off[rng.integers(0, off.size, N)], np.arange(N)] = 127 * rng.choice([-1, 1], N)
    p[O, :] = rng.integers(-255, 256, (O.size, N))
    x = (q * np.exp2(e)[:, None]).astype(np.float32)
    w = (p * np.exp2(f)[None, :]).astype(np.float32)
    exact = (q @ p).astype(np.float64) * np.exp2(e[:, None] + f[None, :])
    return x, w, O.astype(np.int32), exact


@pytest.mark.parametrize("dt", DTS)
def test_fixed_lattice_closed_form(dt):
    for seed in range(20):
        x, w, O, exact = _fixed_lattice(seed)
        X, W = bits_of(x, dt), bits_of(w, dt)
        assert np.array_equal(f32_of(X, dt), x) and np.array_equal(f32_of(W, dt), w)
        assert np.array_equal(exact.astype(np.float32).astype(np.float64), exact)
        Wq, s_w, WO = oracle.quantize_weight_fixed(W, dt, O)
        res = oracle.matmul_fixed(X, dt, Wq, s_w, WO, O)
        assert np.array_equal(res["Y"], bits_of(exact.astype(np.float32), dt)), seed


@pytest.mark.parametrize("dt", DTS)
def test_fixed_weight_conversion_uses_the_scalar_quantizer(dt):
    X, W = _rand(dt, 4, 96, 20, seed=4)
    O = np.array([5, 6, 40, 95], np.int32)
    Wq, s_w, WO = oracle.quantize_weight_fixed(W, dt, O)
    off = np.setdiff1d(np.arange(96), O)
    Wf = f32_of(W, dt)
    for n in range(20):
        assert s_w[n] == np.abs(Wf[off, n]).max()
        assert np.array_equal(Wq[n, off], oracle.quantize(Wf[off, n], float(s_w[n])))
        assert not Wq[n, O].any()
    assert np.array_equal(WO, W[O, :].T)


@pytest.mark.parametrize("dt", DTS)
def test_fixed_negation_symmetry(dt):
    X, W = _rand(dt, 5, 64, 16, seed=6)
    O = np.array([3, 30], np.int32)
    Wn = W ^ np.uint16(0x8000)
    r1 = oracle.matmul_fixed(X, dt, *oracle.quantize_weight_fixed(W, dt, O), O)
    r2 = oracle.matmul_fixed(X, dt, *oracle.quantize_weight_fixed(Wn, dt, O), O)
    a, b = f32_of(r1["Y"], dt), f32_of(r2["Y"], dt)
    assert np.array_equal(a, -b)
