"""Pins of the oracle's whole LLM.int8() path against brute force, closed forms and symmetries.

What is pinned and by what (none of these re-types the oracle's code):
  outlier set O      numpy brute force over independently converted X; x == tau edge
  s_x, Xq, X_O       numpy absmax over the non-outlier columns; Xq[:, O] == 0; the
                     quantizer against exact rounding; fancy-index gather
  C (int8 part)      numpy int64 matmul; K-permutation invariance
  F (16-bit part)    float64 numpy matmul; exact on integer lattices
  Y (epilogue)       closed form on power-of-two lattices: Y == RN_T(exact integer
                     product x 2^(e_i + f_n)), bitwise, with distinct row and column
                     exponents (a swapped or dropped scale fails), outliers included
  reductions         tau = +inf: pure vector-wise quantization; tau = 0: the 16-bit
                     product X @ W_hat; both against float64 within one output ulp
  symmetries         negation, power-of-two scaling, batch invariance with O fixed
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.indep import bits_of, f32_of, ulp16

DTS = ["fp16", "bf16"]


def _rand_case(seed, M, K, N, dt, n_out=2, tau=6.0):
    x, cols = workloads.make_x(M, K, dt, n_outliers=n_out, outlier_range=(6.5, 30.0), seed=seed, wid=50)
    w = workloads.make_w(K, N, dt, sigma=0.05, seed=seed, wid=50)
    return workloads.bits(x), workloads.bits(w), cols


# ----------------------------------------------------------------- outlier set

@pytest.mark.parametrize("dt", DTS)
def test_outlier_set_brute_force(dt):
    for seed in range(40):
        rng = np.random.default_rng(seed)
        M, K = int(rng.integers(1, 9)), int(rng.integers(1, 70))
        X, _, _ = _rand_case(seed, M, K, 3, dt, n_out=int(rng.integers(0, 4)))
        for tau in [0.0, 1.5, 6.0, float(np.inf)]:
            ref = np.nonzero((np.abs(f32_of(X, dt)) > tau).any(axis=0))[0]
            assert np.array_equal(oracle.outlier_columns(X, dt, tau), ref)


@pytest.mark.parametrize("dt", DTS)
def test_outlier_threshold_is_strict(dt):
    X = bits_of(np.array([[6.0, -6.0, 6.004, 0.0], [1.0, 2.0, -1.0, -7.0]], np.float32), dt)
    assert oracle.outlier_columns(X, dt, 6.0).tolist() == ([2, 3] if dt == "fp16" else [3])
    # 6.004 is 6 + 1/256 in fp16 but rounds to 6.0 in bf16, so only the -7 column exceeds there
    assert oracle.outlier_columns(X, dt, 0.0).tolist() == [0, 1, 2, 3]
    assert oracle.outlier_columns(X, dt, float("inf")).tolist() == []


# --------------------------------------------------------------- quantize rows

@pytest.mark.parametrize("dt", DTS)
def test_row_quantization_brute_force(dt):
    for seed in range(30):
        rng = np.random.default_rng(100 + seed)
        M, K = int(rng.integers(1, 12)), int(rng.integers(1, 300))
        X, _, _ = _rand_case(seed, M, K, 3, dt, n_out=int(rng.integers(0, 5)))
        O = oracle.outlier_columns(X, dt, 6.0)
        Xq, s_x, XO = oracle.quantize_rows(X, dt, O)
        Xf = f32_of(X, dt)
        keep = np.ones(K, bool)
        keep[O] = False
        s_ref = np.abs(Xf[:, keep]).max(axis=1) if keep.any() else np.zeros(M, np.float32)
        assert np.array_equal(s_x, s_ref.astype(np.float32))
        assert np.all(Xq[:, O] == 0)
        assert np.array_equal(XO, X[:, O])
        for i in range(M):
            e = 127.0 * Xf[i, keep].astype(np.float64) / s_x[i] if s_x[i] > 0 else np.zeros(keep.sum())
            q = Xq[i, keep].astype(np.int64)
            d = q != np.rint(e)
            frac = np.abs(e[d] - np.floor(e[d]) - 0.5)
            assert np.all(frac <= 2e-5 * np.maximum(1, np.abs(e[d])))
            if s_x[i] > 0:
                assert np.max(np.abs(q)) == 127


def test_row_scale_excludes_outlier_columns_not_just_large_values():
    # column 1 is an outlier dimension because of row 0; row 1 holds only 5.0 there,
    # which does not exceed tau, yet must not set row 1's scale (2.0)
    X = bits_of(np.array([[1.0, 10.0, -0.5], [2.0, 5.0, -1.0]], np.float32), "fp16")
    O = oracle.outlier_columns(X, "fp16", 6.0)
    assert O.tolist() == [1]
    Xq, s_x, XO = oracle.quantize_rows(X, "fp16", O)
    assert s_x.tolist() == [1.0, 2.0]
    assert Xq.tolist() == [[127, 0, -64], [127, 0, -64]]  # -0.5*127 = -63.5 -> -64 (ties to even)
    assert f32_of(XO, "fp16").ravel().tolist() == [10.0, 5.0]


def test_all_columns_outliers_and_zero_rows():
    X = bits_of(np.array([[7.0, -8.0], [0.0, 9.0], [0.0, 0.0]], np.float32), "fp16")
    O = oracle.outlier_columns(X, "fp16", 6.0)
    Xq, s_x, _ = oracle.quantize_rows(X, "fp16", O)
    assert O.tolist() == [0, 1] and np.all(Xq == 0) and np.all(s_x == 0)
    X2 = bits_of(np.zeros((2, 5), np.float32), "bf16")
    Xq2, s2, _ = oracle.quantize_rows(X2, "bf16", oracle.outlier_columns(X2, "bf16", 6.0))
    assert np.all(Xq2 == 0) and np.all(s2 == 0)


# ------------------------------------------------------------- weight

@pytest.mark.parametrize("dt", DTS)
def test_weight_quantization_brute_force(dt):
    for seed in range(10):
        rng = np.random.default_rng(200 + seed)
        K, N = int(rng.integers(1, 200)), int(rng.integers(1, 150))
        W = workloads.bits(workloads.make_w(K, N, dt, sigma=0.03, seed=seed, wid=51))
        Wq, s_w = oracle.quantize_weight(W, dt)
        Wf = f32_of(W, dt)
        assert np.array_equal(s_w, np.abs(Wf).max(axis=0))
        assert Wq.shape == (N, K)
        e = 127.0 * Wf.T.astype(np.float64) / np.where(s_w > 0, s_w, 1)[:, None]
        d = Wq.astype(np.int64) != np.rint(e)
        assert np.all(np.abs(e[d] - np.floor(e[d]) - 0.5) <= 2e-5 * np.maximum(1, np.abs(e[d])))
        assert np.all(np.abs(Wq).max(axis=1)[s_w > 0] == 127)


# ------------------------------------------------------------- products

@pytest.mark.parametrize("dt", DTS)
def test_int_gemm_against_numpy_int64(dt):
    rng = np.random.default_rng(3)
    for _ in range(10):
        M, K, N = (int(v) for v in rng.integers(1, 90, 3))
        Xq = rng.integers(-127, 128, (M, K)).astype(np.int8)
        Wq = rng.integers(-127, 128, (N, K)).astype(np.int8)
        rows = rng.choice(M, min(M, 5), replace=False)
        C = oracle.int_gemm(Xq, Wq, rows)
        ref = Xq[rows].astype(np.int64) @ Wq.T.astype(np.int64)
        assert np.array_equal(C, ref)
    # extreme values: every product is 127*127 (or -127*127); K large
    K = 20000
    Xq = np.full((1, K), -127, np.int8)
    Wq = np.full((2, K), 127, np.int8)
    Wq[1, ::2] = -127
    assert oracle.int_gemm(Xq, Wq).tolist() == [[-127 * 127 * K, 0]]


@pytest.mark.parametrize("dt", DTS)
def test_outlier_gemm_exact_on_integers_and_close_to_float64(dt):
    rng = np.random.default_rng(4)
    M, K, N = 6, 40, 9
    O = np.array([1, 5, 17, 33], np.int32)
    Wq = rng.integers(-127, 128, (N, K)).astype(np.int8)
    XOi = rng.integers(-100, 101, (M, O.size)).astype(np.float32)  # integers: every partial sum exact
    F, F64, A = oracle.outlier_gemm(bits_of(XOi, dt), O, dt, Wq)
    ref = XOi.astype(np.int64) @ Wq[:, O].T.astype(np.int64)
    assert np.array_equal(F, ref.astype(np.float32)) and np.array_equal(F64, ref.astype(np.float64))
    XOr = rng.standard_normal((M, O.size)).astype(np.float32) * 20
    XOb = bits_of(XOr, dt)
    F, F64, A = oracle.outlier_gemm(XOb, O, dt, Wq)
    ref64 = f32_of(XOb, dt).astype(np.float64) @ Wq[:, O].T.astype(np.float64)
    assert np.allclose(F64, ref64, rtol=1e-12, atol=1e-9)
    assert np.all(np.abs(F - ref64) <= O.size * 2.0**-24 * A + 1e-30)
    assert np.allclose(A, np.abs(f32_of(XOb, dt).astype(np.float64)) @ np.abs(Wq[:, O].T.astype(np.float64)))


# ------------------------------------------------------ closed form on lattices

def _lattice_case(dt, seed, M=7, K=48, N=11, out_cols=(3, 20, 41)):
    """x[i,j] = q[i,j] * 2^e_i, w[k,n] = p[k,n] * 2^f_n with |q| <= 127 outside the outlier
    columns, |q| in [129, 199] inside them (exact in both 16-bit types), each row's
    non-outlier absmax and each column's absmax exactly 127.  With tau = 127 * 2^max(e),
    O is exactly the outlier columns, Xq = q, Wq = p^T, r_i = 2^e_i, c_n = 2^f_n, every fp32
    step is exact, and y = 2^(e_i+f_n) * (q @ p)[i,n] exactly."""
    rng = np.random.default_rng(seed)
    e = rng.integers(-4, 3, M)
    f = rng.integers(-12, -6, N)
    q = rng.integers(-127, 128, (M, K))
    q[:, 0] = 127 * rng.choice([-1, 1], M)           # row absmax 127 in a non-outlier column
    cols = np.array(out_cols)
    q[:, cols] = rng.integers(129, 200, (M, cols.size)) * rng.choice([-1, 1], (M, cols.size))
    p = rng.integers(-127, 128, (K, N))
    p[rng.integers(0, K, N), np.arange(N)] = 127 * rng.choice([-1, 1], N)
    x = (q * np.exp2(e)[:, None]).astype(np.float32)
    w = (p * np.exp2(f)[None, :]).astype(np.float32)
    tau = float(127 * 2.0 ** e.max())
    exact = (q @ p).astype(np.float64) * np.exp2(e[:, None] + f[None, :])
    return x, w, tau, exact, cols


@pytest.mark.parametrize("dt", DTS)
def test_epilogue_closed_form_on_lattice(dt):
    for seed in range(25):
        x, w, tau, exact, cols = _lattice_case(dt, seed)
        X, W = bits_of(x, dt), bits_of(w, dt)
        assert np.array_equal(f32_of(X, dt), x) and np.array_equal(f32_of(W, dt), w)
        Wq, s_w = oracle.quantize_weight(W, dt)
        res = oracle.matmul(X, dt, Wq, s_w, tau)
        assert np.array_equal(res["O"], cols)
        assert np.array_equal(exact.astype(np.float32).astype(np.float64), exact)  # exact in fp32
        with np.errstate(over="ignore"):
            ref = bits_of(exact.astype(np.float32), dt)
        assert np.array_equal(res["Y"], ref), seed


@pytest.mark.parametrize("dt,cs,expect", [
    ("fp16", [2049, 2051, 2053], [2048.0, 2052.0, 2052.0]),   # spacing 2 in [2048, 4096)
    ("bf16", [257, 259, 261], [256.0, 260.0, 260.0]),         # spacing 2 in [256, 512)
])
def test_epilogue_output_rounding_ties_to_even(dt, cs, expect):
    # x = [127, 1, 0] and w columns [a, b, 127] give scales 127 (r = c = 1) and y = 127a + b,
    # an exact tie between two neighbours of the 16-bit format
    base = cs[0] - 1 - 127 * ((cs[0] - 1) // 127)
    a = (cs[0] - 1) // 127
    x = np.array([[127.0, 1.0, 0.0]], np.float32)
    w = np.array([[a, a, a], [c - 127 * a for c in cs], [127.0, 127.0, 127.0]], np.float32)
    assert base >= 0 and np.all(np.abs(w) <= 127)
    X, W = bits_of(x, dt), bits_of(w, dt)
    Wq, s_w = oracle.quantize_weight(W, dt)
    res = oracle.matmul(X, dt, Wq, s_w, float("inf"))
    assert res["C"].tolist() == [cs]
    assert f32_of(res["Y"], dt).tolist() == [expect]
    assert np.array_equal(res["Y"], bits_of(np.array([cs], np.float64), dt))


# ----------------------------------------------------------- special cases

@pytest.mark.parametrize("dt", DTS)
def test_tau_inf_is_pure_vectorwise_quantization(dt):
    X, W, _ = _rand_case(7, 24, 160, 40, dt, n_out=3)
    Wq, s_w = oracle.quantize_weight(W, dt)
    res = oracle.matmul(X, dt, Wq, s_w, float("inf"))
    assert res["O"].size == 0 and np.all(res["F"] == 0)
    Xq, s_x = res["Xq"], res["s_x"]
    s_ref = np.abs(f32_of(X, dt)).max(axis=1)
    assert np.array_equal(s_x, s_ref)
    exact = (Xq.astype(np.float64) * s_x[:, None].astype(np.float64) / 127.0) @ \
            (Wq.astype(np.float64) * s_w[:, None].astype(np.float64) / 127.0).T
    Yf = f32_of(res["Y"], dt).astype(np.float64)
    assert np.all(np.abs(Yf - exact) <= ulp16(exact, dt) * 0.5 + 8 * 2.0**-24 * np.abs(exact) + 1e-30)


@pytest.mark.parametrize("dt", DTS)
def test_tau_zero_is_the_16bit_product(dt):
    X, W, _ = _rand_case(8, 20, 96, 30, dt, n_out=2)
    Wq, s_w = oracle.quantize_weight(W, dt)
    res = oracle.matmul(X, dt, Wq, s_w, 0.0)
    Xf = f32_of(X, dt).astype(np.float64)
    nz = np.nonzero((Xf != 0).any(axis=0))[0]
    assert np.array_equal(res["O"], nz) and np.all(res["C"] == 0) and np.all(res["s_x"] == 0)
    What = Wq.T.astype(np.float64) * (s_w.astype(np.float64) / 127.0)[None, :]
    exact = Xf @ What
    A = np.abs(Xf) @ np.abs(What)
    Yf = f32_of(res["Y"], dt).astype(np.float64)
    bound = ulp16(exact, dt) * 0.5 + (X.shape[1] + 4) * 2.0**-24 * A + 1e-30
    assert np.all(np.abs(Yf - exact) <= bound)


# ------------------------------------------------------------- symmetries

@pytest.mark.parametrize("dt", DTS)
def test_negation_symmetry(dt):
    X, W, _ = _rand_case(9, 16, 128, 24, dt, n_out=3)
    Wq, s_w = oracle.quantize_weight(W, dt)
    a = oracle.matmul(X, dt, Wq, s_w, 6.0)
    b = oracle.matmul(X ^ np.uint16(0x8000), dt, Wq, s_w, 6.0)
    assert np.array_equal(a["O"], b["O"]) and np.array_equal(a["Xq"], -b["Xq"])
    assert np.array_equal(f32_of(a["Y"], dt), -f32_of(b["Y"], dt))


@pytest.mark.parametrize("dt", DTS)
def test_power_of_two_scaling(dt):
    X, W, _ = _rand_case(10, 16, 128, 24, dt, n_out=3)
    Wq, s_w = oracle.quantize_weight(W, dt)
    a = oracle.matmul(X, dt, Wq, s_w, 6.0)
    X2 = bits_of(f32_of(X, dt) * 2, dt)
    b = oracle.matmul(X2, dt, Wq, s_w, 12.0)
    assert np.array_equal(a["O"], b["O"]) and np.array_equal(a["Xq"], b["Xq"])
    assert np.array_equal(a["s_x"] * 2, b["s_x"]) and np.array_equal(a["C"], b["C"])
    assert np.array_equal(f32_of(a["Y"], dt) * 2, f32_of(b["Y"], dt))


@pytest.mark.parametrize("dt", DTS)
def test_k_permutation_leaves_integer_part_unchanged(dt):
    X, W, _ = _rand_case(11, 12, 200, 16, dt, n_out=4)
    perm = np.random.default_rng(5).permutation(200)
    Wq, s_w = oracle.quantize_weight(W, dt)
    a = oracle.matmul(X, dt, Wq, s_w, 6.0)
    Wq2, s_w2 = oracle.quantize_weight(W[perm], dt)
    b = oracle.matmul(X[:, perm], dt, Wq2, s_w2, 6.0)
    assert np.array_equal(np.sort(perm[b["O"]]), a["O"])
    assert np.array_equal(a["C"], b["C"]) and np.array_equal(a["s_x"], b["s_x"])
    assert np.array_equal(a["Xq"][:, perm], b["Xq"]) and np.array_equal(s_w, s_w2)


@pytest.mark.parametrize("dt", DTS)
def test_batch_invariance_with_outlier_set_fixed(dt):
    X, W, _ = _rand_case(12, 10, 128, 20, dt, n_out=2)
    Wq, s_w = oracle.quantize_weight(W, dt)
    a = oracle.matmul(X, dt, Wq, s_w, 6.0)
    extra = bits_of(np.clip(f32_of(X[:3], dt) * 0.5, -5, 5), dt)  # creates no new outlier column
    b = oracle.matmul(np.concatenate([X, extra]), dt, Wq, s_w, 6.0)
    assert np.array_equal(a["O"], b["O"])
    assert np.array_equal(a["Y"], b["Y"][: X.shape[0]])


def test_tiny_workload_statistics():
    x, w, cols, wl = workloads.make_workload("tiny")
    X, W = workloads.bits(x), workloads.bits(w)
    Wq, s_w = oracle.quantize_weight(W, "fp16")
    res = oracle.matmul(X, "fp16", Wq, s_w, wl.tau)
    assert res["O"].tolist() == [7, 131]
    assert np.array_equal(cols, [7, 131])
