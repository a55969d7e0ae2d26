"""GPU path vs the CPU oracle, element by element (test infrastructure).

Bars (the oracle is the reference; both sides get the same seeded inputs):
  bit-exact   Wq, s_w, the outlier set O and n_O, s_x, Xq (and its zero padding), the
              gathered outlier operands X[:,O] and Wq[:,O] (and their zero padding), and
              the int32 accumulators C.
  F           the 16-bit outlier product is summed in a different order on the GPU
              (inside the MFMA), so |F_gpu - F_exact| <= n_O * 2^-23 * A, A = sum |terms|.
  Y           T3: n_O == 0 -> bitwise equal (every step is a fixed sequence of
              correctly rounded fp32 ops);
              T2: every element within one output ulp plus the propagated fp32 bound
                  2 (n_O + 2) 2^-23 (|y| + c_n A);
              T1: per token row, ||Y_gpu - Y_orc||_2 / ||Y_orc||_2 <= 2e-3.
A legitimate difference in F's summation order can flip one rounding of y to the
16-bit output, so an element-wise relative bound cannot be used for bf16 (one bf16 ulp
is up to 7.8e-3 relative); the max element-wise relative error is reported instead.
"""
from __future__ import annotations

import numpy as np
import torch

import int8_quantized_matmul_rowwise_amd as lm
import oracle
from tests.indep import bits_of, f32_of, ulp16

T1_TOL = 2e-3


def to_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def dt_name(t: torch.Tensor) -> str:
    return "fp16" if t.dtype == torch.float16 else "bf16"


def check_weight(W: torch.Tensor, Wq_g: torch.Tensor, s_w_g: torch.Tensor):
    dt = dt_name(W)
    Wq_o, s_w_o = oracle.quantize_weight(to_bits(W.cpu()), dt)
    assert np.array_equal(s_w_g.cpu().numpy().view(np.uint32), s_w_o.view(np.uint32)), "s_w differs"
    wq = Wq_g.cpu().numpy()
    bad = np.argwhere(wq != Wq_o)
    assert bad.size == 0, f"Wq differs at {bad[:5].tolist()} (of {len(bad)})"
    return Wq_o, s_w_o


def check_y(Yg: np.ndarray, res: dict, s_w: np.ndarray, dt: str, n_o: int) -> dict:
    """Y bars T1-T3 for the oracle rows in `res`; returns the error statistics."""
    Yo = res["Y"]
    if n_o == 0:
        bad = np.argwhere(Yg != Yo)
        assert bad.size == 0, f"T3: Y not bitwise equal with no outliers at {bad[:5].tolist()}"
    yg = f32_of(Yg, dt).astype(np.float64)
    yo = f32_of(Yo, dt).astype(np.float64)
    same = Yg == Yo
    c = s_w.astype(np.float64) / 127.0
    with np.errstate(invalid="ignore", over="ignore"):
        bound = ulp16(yo, dt) + 2 * (n_o + 2) * 2.0**-23 * (np.abs(res["y"].astype(np.float64)) + c[None, :] * res["A"])
        diff = np.abs(yg - yo)
    bad = ~same & ~(diff <= bound)
    assert not bad.any(), f"T2: Y outside the bound at {np.argwhere(bad)[:5].tolist()}"
    fin = np.isfinite(yo) & np.isfinite(yg)
    num = np.sqrt(np.sum(np.where(fin, (yg - yo) ** 2, 0.0), axis=1))
    den = np.sqrt(np.sum(np.where(fin, yo ** 2, 0.0), axis=1))
    rel = np.where(den > 0, num / np.where(den > 0, den, 1.0), 0.0)
    assert np.all(num[den == 0] == 0), "T1: nonzero output on a row whose oracle output is zero"
    assert rel.max(initial=0.0) <= T1_TOL, f"T1: row-wise relative error {rel.max()}"
    floor = 1e-3 * np.sqrt(np.mean(yo[fin] ** 2)) if fin.any() else 0.0
    m = fin & (np.abs(yo) > floor)
    elem = np.max(np.abs(yg[m] - yo[m]) / np.abs(yo[m]), initial=0.0)
    return {"t1_max": float(rel.max(initial=0.0)), "elem_rel_max": float(elem), "n_ulp_flips": int((~same).sum())}


def run_case(X: torch.Tensor, W: torch.Tensor, tau: float, rows=None, device="cuda", check_acc=True,
             Wq_s=None) -> dict:
    """Run the HIP path on (X, W, tau) and compare everything with the oracle.

    X, W: CPU 16-bit tensors.  rows: oracle rows to compare for the products (None: all).
    Returns statistics; raises AssertionError on any parity failure."""
    dt = dt_name(X)
    M, K = X.shape
    N = W.shape[1]
    Xd = X.to(device)
    if Wq_s is None:
        Wd = W.to(device)
        Wq, s_w = lm.int8_quantize_weight(Wd)
        torch.cuda.synchronize()
        Wq_o, s_w_o = check_weight(W, Wq, s_w)
        del Wd
    else:
        Wq, s_w, Wq_o, s_w_o = Wq_s
    ws = torch.empty(max(lm.int8_matmul_workspace_bytes(M, K, N), 1), dtype=torch.uint8, device=device)
    Y = lm.int8_matmul(Xd, Wq, s_w, tau, workspace=ws)
    torch.cuda.synchronize()

    Xb = to_bits(X)
    O = oracle.outlier_columns(Xb, dt, tau)
    Xq_o, s_x_o, XO_o = oracle.quantize_rows(Xb, dt, O)
    n_o = int(O.size)
    v = lm.workspace_views(ws, M, K, N, X.dtype)
    assert v["n_outliers"] == n_o, f"n_O {v['n_outliers']} != {n_o}"
    assert np.array_equal(v["outliers"].cpu().numpy(), O), "outlier set differs"
    assert np.array_equal(v["s_x"].cpu().numpy().view(np.uint32), s_x_o.view(np.uint32)), "s_x differs"
    if K > 0:
        xq = v["Xq"].cpu().numpy()
        bad = np.argwhere(xq != Xq_o)
        assert bad.size == 0, f"Xq differs at {bad[:5].tolist()} (of {len(bad)})"
        assert not v["Xq_pad"].cpu().numpy().any(), "Xq padding not zero"
        P = v["XO"].shape[1]
        xo = to_bits(v["XO"])
        assert np.array_equal(xo[:, :n_o], XO_o) and not xo[:, n_o:].any(), "X[:,O] gather differs"
        # the small-batch path gathers Wq[:,O] inside its product kernel
        if N > 0 and not lm.int8_matmul_workspace_layout(M, K, N)["small_batch"]:
            wo = to_bits(v["WO"])
            ref = bits_of(Wq_o[:, O].astype(np.float32), dt)
            assert np.array_equal(wo[:, :n_o], ref) and not wo[:, n_o:].any(), "Wq[:,O] gather differs"
        assert P == (n_o + 31) // 32 * 32

    r = np.arange(M) if rows is None else np.asarray(rows, np.int64)
    stats = {"n_outliers": n_o, "rows_compared": int(r.size)}
    if N == 0 or M == 0:
        return stats
    C_o = oracle.int_gemm(Xq_o, Wq_o, r)
    F_o, F64, A = oracle.outlier_gemm(XO_o, O, dt, Wq_o, r)
    y_o, Y_o = oracle.dequant(C_o, F_o, s_x_o[r], s_w_o, dt)
    res = {"Y": Y_o, "y": y_o, "A": A}
    rt = torch.as_tensor(r, device=Y.device)
    Yg = to_bits(Y[rt])
    stats.update(check_y(Yg, res, s_w_o, dt, n_o))

    if check_acc:
        C, F, _ = lm.int8_matmul_accumulators(Xd, Wq, tau)
        torch.cuda.synchronize()
        Cg = C[rt].cpu().numpy()
        bad = np.argwhere(Cg != C_o)
        assert bad.size == 0, f"C differs at {bad[:5].tolist()} (of {len(bad)})"
        Fg = F[rt].cpu().numpy().astype(np.float64)
        fb = n_o * 2.0**-23 * A + 1e-30
        assert np.all(np.abs(Fg - F64) <= fb), "F outside its summation bound"
        if n_o == 0:
            assert not Fg.any()
        del C, F
    return stats
