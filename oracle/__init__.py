"""CPU oracle for the LLM.int8() matmul -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The GPU library never does, and the two share no code.  The arithmetic
lives in ``oracle.c`` (plain C, fp32 scales, round-to-nearest-even, exact integer dot
products); this file only builds it and marshals numpy arrays through ctypes.
16-bit tensors cross this interface as their raw uint16 bit patterns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liborc.so")
# LLMINT8_ORACLE_LIB: a prebuilt copy of the oracle (the sanitized test build); used as is
ALT_LIB = os.environ.get("LLMINT8_ORACLE_LIB")
DT = {"fp16": 0, "bf16": 1}

_lock = threading.Lock()
_lib = None
_SIGS = {}


def build(out: str = LIB, sanitize: bool = False) -> str:
    """Compile the oracle (gcc, no fast-math, no contraction).  Returns the library path.
    sanitize: AddressSanitizer + UndefinedBehaviorSanitizer (test build; load it with the
    sanitizer runtime preloaded and LLMINT8_ORACLE_LIB pointing at it)."""
    tmp = out + ".tmp%d" % os.getpid()
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"] \
        if sanitize else []
    subprocess.check_call(["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
                           "-fPIC", "-shared", "-Wall", "-Wextra", *san, "-o", tmp, SRC, "-lm"])
    os.replace(tmp, out)
    return out


_P = ctypes.c_void_p
_I64 = ctypes.c_int64


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if ALT_LIB:
            lib = ctypes.CDLL(ALT_LIB)
        else:
            if not os.path.exists(LIB) or os.path.getmtime(LIB) < max(os.path.getmtime(SRC),
                                                                       os.path.getmtime(os.path.join(HERE, "oracle.h"))):
                build()
            lib = ctypes.CDLL(LIB)
        sig = {
            "orc_set_threads": (ctypes.c_int, [ctypes.c_int]),
            "orc_to_f32_n": (None, [_P, _I64, ctypes.c_int, _P]),
            "orc_from_f32_n": (None, [_P, _I64, ctypes.c_int, _P]),
            "orc_inv_scale": (ctypes.c_float, [ctypes.c_float]),
            "orc_quantize_n": (None, [_P, _I64, ctypes.c_float, _P]),
            "orc_quantize_weight": (None, [_P, _I64, _I64, ctypes.c_int, _P, _P]),
            "orc_outlier_columns": (_I64, [_P, _I64, _I64, ctypes.c_int, ctypes.c_float, _P]),
            "orc_quantize_rows": (None, [_P, _I64, _I64, ctypes.c_int, _P, _I64, _P, _P, _P]),
            "orc_int_gemm": (ctypes.c_int, [_P, _P, _I64, _I64, _P, _I64, _P]),
            "orc_outlier_gemm": (None, [_P, _I64, ctypes.c_int, _P, _I64, _I64, _P, _P, _I64, _P, _P, _P]),
            "orc_dequant": (None, [_P, _P, _P, _P, _I64, _I64, ctypes.c_int, _P, _P]),
            "orc_quantize_weight_fixed": (None, [_P, _I64, _I64, ctypes.c_int, _P, _I64, _P, _P, _P]),
            "orc_outlier_gemm_exact": (None, [_P, _I64, ctypes.c_int, _P, _I64, _P, _I64, _P, _P, _P]),
            "orc_dequant_fixed": (None, [_P, _P, _P, _P, _I64, _I64, ctypes.c_int, _P, _P]),
            "orc_group_quantize_rows": (None, [_P, _I64, _I64, ctypes.c_int, _I64, _P, _P]),
            "orc_group_quantize_weight": (None, [_P, _I64, _I64, ctypes.c_int, _I64, _P, _P]),
            "orc_group_gemm": (None, [_P, _P, _P, _P, _I64, _I64, _I64, _P, _I64, ctypes.c_int, _P, _P]),
            "orc_block_quantize": (None, [_P, _I64, _I64, _P, _P]),
            "orc_block_dequantize": (None, [_P, _P, _I64, _I64, _P]),
        }
        _SIGS.update(sig)
        for name, (res, args) in sig.items():
            f = getattr(lib, name)
            f.restype = res
            f.argtypes = args
        _lib = lib
        return lib


class use_library:
    """Context manager: route every call through another build of the oracle (the
    mutation tests use it to check that the pins reject a planted mistake)."""

    def __init__(self, path: str):
        self.path = path

    def __enter__(self):
        global _lib
        _load()
        self.saved = _lib
        lib = ctypes.CDLL(self.path)
        for name, f in _SIGS.items():
            g = getattr(lib, name)
            g.restype, g.argtypes = f
        _lib = lib
        return lib

    def __exit__(self, *exc):
        global _lib
        _lib = self.saved
        return False


def _c(a: np.ndarray, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def set_threads(n: int = 0) -> int:
    """Threads for the row-parallel loops (0: all host cores).  Returns the count used."""
    return int(_load().orc_set_threads(int(n)))


def to_f32(h: np.ndarray, dt: str) -> np.ndarray:
    h = _c(h, np.uint16)
    out = np.empty(h.shape, np.float32)
    _load().orc_to_f32_n(_p(h), h.size, DT[dt], _p(out))
    return out


def from_f32(f: np.ndarray, dt: str) -> np.ndarray:
    f = _c(f, np.float32)
    out = np.empty(f.shape, np.uint16)
    _load().orc_from_f32_n(_p(f), f.size, DT[dt], _p(out))
    return out


def inv_scale(s: float) -> float:
    return float(_load().orc_inv_scale(ctypes.c_float(s)))


def quantize(x: np.ndarray, s: float) -> np.ndarray:
    """q = clamp(rne(x * RN32(127/s)), -127, 127) for fp32 x and one fp32 scale s."""
    x = _c(x, np.float32)
    q = np.empty(x.shape, np.int8)
    _load().orc_quantize_n(_p(x), x.size, ctypes.c_float(np.float32(s)), _p(q))
    return q


def quantize_weight(W: np.ndarray, dt: str):
    """W bits (K x N) -> (Wq int8 N x K, s_w fp32[N])."""
    W = _c(W, np.uint16)
    K, N = W.shape
    Wq = np.empty((N, K), np.int8)
    s_w = np.empty(N, np.float32)
    _load().orc_quantize_weight(_p(W), K, N, DT[dt], _p(Wq), _p(s_w))
    return Wq, s_w


def outlier_columns(X: np.ndarray, dt: str, tau: float) -> np.ndarray:
    X = _c(X, np.uint16)
    M, K = X.shape
    O = np.empty(max(K, 1), np.int32)
    n = _load().orc_outlier_columns(_p(X), M, K, DT[dt], ctypes.c_float(tau), _p(O))
    return O[:n].copy()


def quantize_rows(X: np.ndarray, dt: str, O: np.ndarray):
    """-> (Xq int8 M x K, s_x fp32[M], XO bits M x n_O)."""
    X = _c(X, np.uint16)
    O = _c(O, np.int32)
    M, K = X.shape
    Xq = np.empty((M, K), np.int8)
    s_x = np.empty(M, np.float32)
    XO = np.empty((M, O.size), np.uint16)
    _load().orc_quantize_rows(_p(X), M, K, DT[dt], _p(O), O.size, _p(Xq), _p(s_x), _p(XO))
    return Xq, s_x, XO


def _rows(rows, M):
    if rows is None:
        return None, M
    r = _c(rows, np.int64)
    assert r.size == 0 or (r.min() >= 0 and r.max() < M)
    return r, r.size


def int_gemm(Xq: np.ndarray, Wq: np.ndarray, rows=None) -> np.ndarray:
    Xq = _c(Xq, np.int8)
    Wq = _c(Wq, np.int8)
    M, K = Xq.shape
    N = Wq.shape[0]
    assert Wq.shape[1] == K
    r, nr = _rows(rows, M)
    C = np.empty((nr, N), np.int32)
    rc = _load().orc_int_gemm(_p(Xq), _p(Wq), K, N, _p(r), nr, _p(C))
    if rc != 0:
        raise OverflowError("int32 accumulator overflow in the oracle")
    return C


def outlier_gemm(XO: np.ndarray, O: np.ndarray, dt: str, Wq: np.ndarray, rows=None):
    """-> (F fp32, F64 float64, A float64), each nrows x N."""
    XO = _c(XO, np.uint16)
    O = _c(O, np.int32)
    Wq = _c(Wq, np.int8)
    M = XO.shape[0]
    N, K = Wq.shape
    r, nr = _rows(rows, M)
    F = np.empty((nr, N), np.float32)
    F64 = np.empty((nr, N), np.float64)
    A = np.empty((nr, N), np.float64)
    XO_ = XO if XO.size else np.zeros((M, 1), np.uint16)
    _load().orc_outlier_gemm(_p(XO_), O.size, DT[dt], _p(Wq), K, N, _p(O) if O.size else None,
                             _p(r), nr, _p(F), _p(F64), _p(A))
    return F, F64, A


def dequant(C: np.ndarray, F: np.ndarray, s_x_rows: np.ndarray, s_w: np.ndarray, dt: str):
    """-> (y fp32, Y bits), each nrows x N."""
    C = _c(C, np.int32)
    F = _c(F, np.float32)
    s_x_rows = _c(s_x_rows, np.float32)
    s_w = _c(s_w, np.float32)
    nr, N = C.shape
    y = np.empty((nr, N), np.float32)
    Y = np.empty((nr, N), np.uint16)
    _load().orc_dequant(_p(C), _p(F), _p(s_x_rows), _p(s_w), nr, N, DT[dt], _p(y), _p(Y))
    return y, Y


def matmul(X: np.ndarray, dt: str, Wq: np.ndarray, s_w: np.ndarray, tau: float, rows=None) -> dict:
    """The whole path: outlier columns, row quantization, int8 part, 16-bit part, epilogue.

    The X pass covers every row (the outlier set depends on all of them); the products
    and the epilogue cover ``rows`` only (all rows when None).  Returns every intermediate.
    """
    O = outlier_columns(X, dt, tau)
    Xq, s_x, XO = quantize_rows(X, dt, O)
    r = np.arange(X.shape[0]) if rows is None else np.asarray(rows, np.int64)
    C = int_gemm(Xq, Wq, r)
    F, F64, A = outlier_gemm(XO, O, dt, Wq, r)
    y, Y = dequant(C, F, s_x[r], s_w, dt)
    return dict(O=O, Xq=Xq, s_x=s_x, XO=XO, rows=r, C=C, F=F, F64=F64, A=A, y=y, Y=Y)


def block_quantize(x: np.ndarray, block: int):
    """Block-wise absmax int8 code of a flat fp32 array -> (q int8[n], absmax fp32[ceil(n/block)])."""
    x = _c(np.ravel(x), np.float32)
    n = x.size
    nb = -(-n // block) if n else 0
    q = np.zeros(n, np.int8)
    absmax = np.zeros(nb, np.float32)
    if n:
        _load().orc_block_quantize(_p(x), n, block, _p(q), _p(absmax))
    return q, absmax


def block_dequantize(q: np.ndarray, absmax: np.ndarray, block: int) -> np.ndarray:
    """Decode of block_quantize: x' = RN32(q * RN32(absmax / 127)) per block."""
    q = _c(np.ravel(q), np.int8)
    absmax = _c(absmax, np.float32)
    x = np.zeros(q.size, np.float32)
    if q.size:
        _load().orc_block_dequantize(_p(q), _p(absmax), q.size, block, _p(x))
    return x


# ---- fixed (caller-supplied) outlier dimensions

def quantize_weight_fixed(W: np.ndarray, dt: str, O: np.ndarray):
    """Weight conversion with the outlier set O fixed: (Wq N x K, s_w[N], WO N x nO exact 16-bit)."""
    W = _c(W, np.uint16)
    K, N = W.shape
    O = _c(O, np.int32)
    Wq = np.zeros((N, K), np.int8)
    s_w = np.zeros(N, np.float32)
    WO = np.zeros((N, O.size), np.uint16)
    _load().orc_quantize_weight_fixed(_p(W), K, N, DT[dt], _p(O), O.size, _p(Wq), _p(s_w), _p(WO))
    return Wq, s_w, WO


def outlier_gemm_exact(XO: np.ndarray, dt: str, WO: np.ndarray, rows=None):
    """F = X[:,O] W_O^T with the exact 16-bit W rows (fp32, t ascending); also F64 and A."""
    XO = _c(XO, np.uint16)
    WO = _c(WO, np.uint16)
    M, nO = XO.shape
    N = WO.shape[0]
    r, nr = _rows(rows, M)
    F = np.zeros((nr, N), np.float32)
    F64 = np.zeros((nr, N), np.float64)
    A = np.zeros((nr, N), np.float64)
    _load().orc_outlier_gemm_exact(_p(XO), nO, DT[dt], _p(WO), N, _p(r), nr, _p(F), _p(F64), _p(A))
    return F, F64, A


def dequant_fixed(C: np.ndarray, F: np.ndarray, s_x_rows: np.ndarray, s_w: np.ndarray, dt: str):
    """Epilogue of the fixed-outlier product: y = RN(RN(RN(C r) c) + F); returns (y, Y bits)."""
    C = _c(C, np.int32)
    F = _c(F, np.float32)
    nr, N = C.shape
    y = np.zeros((nr, N), np.float32)
    Y = np.zeros((nr, N), np.uint16)
    _load().orc_dequant_fixed(_p(C), _p(F), _p(_c(s_x_rows, np.float32)), _p(_c(s_w, np.float32)), nr, N, DT[dt],
                              _p(y), _p(Y))
    return y, Y


def matmul_fixed(X: np.ndarray, dt: str, Wq: np.ndarray, s_w: np.ndarray, WO: np.ndarray, O: np.ndarray,
                 rows=None) -> dict:
    """The whole fixed-outlier product of the oracle (X pass against O, int8 and exact 16-bit
    parts, epilogue) for the given rows (None: all)."""
    O = _c(O, np.int32)
    Xq, s_x, XO = quantize_rows(X, dt, O)
    rr = np.arange(X.shape[0]) if rows is None else np.asarray(rows, np.int64)
    C = int_gemm(Xq, Wq, rr)
    F, F64, A = outlier_gemm_exact(XO, dt, WO, rr)
    y, Y = dequant_fixed(C, F, s_x[rr], s_w, dt)
    return dict(O=O, Xq=Xq, s_x=s_x, XO=XO, rows=rr, C=C, F=F, F64=F64, A=A, y=y, Y=Y)


# ---- group-wise scales along K

def group_quantize_rows(X: np.ndarray, dt: str, G: int):
    """(Xq M x K, s_x M x K/G) with one scale per row and group of G features."""
    X = _c(X, np.uint16)
    M, K = X.shape
    assert G > 0 and K % G == 0
    Xq = np.zeros((M, K), np.int8)
    s_x = np.zeros((M, K // G), np.float32)
    _load().orc_group_quantize_rows(_p(X), M, K, DT[dt], G, _p(Xq), _p(s_x))
    return Xq, s_x


def group_quantize_weight(W: np.ndarray, dt: str, G: int):
    """(Wq N x K, s_w N x K/G) with one scale per output column and group."""
    W = _c(W, np.uint16)
    K, N = W.shape
    assert G > 0 and K % G == 0
    Wq = np.zeros((N, K), np.int8)
    s_w = np.zeros((N, K // G), np.float32)
    _load().orc_group_quantize_weight(_p(W), K, N, DT[dt], G, _p(Wq), _p(s_w))
    return Wq, s_w


def group_gemm(Xq: np.ndarray, s_x: np.ndarray, Wq: np.ndarray, s_w: np.ndarray, G: int, dt: str, rows=None):
    """(y fp32, Y bits) of the group-wise product for the given rows (None: all)."""
    Xq = _c(Xq, np.int8)
    Wq = _c(Wq, np.int8)
    M, K = Xq.shape
    N = Wq.shape[0]
    r, nr = _rows(rows, M)
    y = np.zeros((nr, N), np.float32)
    Y = np.zeros((nr, N), np.uint16)
    _load().orc_group_gemm(_p(Xq), _p(_c(s_x, np.float32)), _p(Wq), _p(_c(s_w, np.float32)), K, N, G, _p(r), nr,
                           DT[dt], _p(y), _p(Y))
    return y, Y
