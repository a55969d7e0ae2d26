"""LLM.int8() matmul for AMD Instinct MI355X: Python binding of the llmint8 C library.

The functions here carry the C-ABI names and only marshal arguments (torch tensors ->
device pointers, the current HIP stream, workspace allocation when the caller passes
none).  Every step of the computation runs in the HIP kernels of libllmint8.so; there
is no fallback, and importing fails loudly when the library has not been built
(``python -m int8_quantized_matmul_rowwise_amd.build``).

    Wq, s_w = int8_quantize_weight(W)                  # offline, W: K x N
    Y = int8_matmul(X, Wq, s_w, threshold=6.0)          # X: M x K -> Y: M x N
    n_outliers, cols = int8_matmul_stats(X, 6.0)
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
# LLMINT8_LIB: another build of the same sources (the host-sanitized test build)
LIB_PATH = os.environ.get("LLMINT8_LIB") or os.path.join(HERE, "libllmint8.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "llmint8.h")

F16, BF16 = 0, 1
_DT = {torch.float16: F16, torch.bfloat16: BF16}
OK, EINVAL, EWORKSPACE, EHIP, ERANGE = 0, -1, -2, -3, -4

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
_F = ctypes.c_float
_I = ctypes.c_int


class LLMInt8Error(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


class WorkspaceLayout(ctypes.Structure):
    _fields_ = [(n, _SZ) for n in ("xq", "xq_pitch", "s_x", "n_outliers", "outliers", "xo", "xo_pitch", "wo",
                                   "scratch", "total", "small_batch")]


_SIGNATURES = {
    "llmint8_status_string": (ctypes.c_char_p, [_I]),
    "int8_quantize_weight": (_I, [_P, _I64, _I64, _I, _P, _P, _P]),
    "int8_matmul_workspace_bytes": (_SZ, [_I64, _I64, _I64]),
    "int8_matmul": (_I, [_P, _I64, _I64, _I, _P, _P, _I64, _F, _P, _P, _SZ, _P]),
    "int8_matmul_noalloc": (_I, [_P, _I64, _I64, _I, _P, _P, _I64, _F, _P, _P]),
    "int8_matmul_stats": (_I, [_P, _I64, _I64, _I, _F, _P, _P, _P, _SZ, _P]),
    "int8_matmul_workspace_layout": (_I, [_I64, _I64, _I64, ctypes.POINTER(WorkspaceLayout)]),
    "int8_matmul_accumulators": (_I, [_P, _I64, _I64, _I, _P, _I64, _F, _P, _P, _P, _SZ, _P]),
    "int8_matmul_prepare": (_I, [_P, _I64, _I64, _I, _P, _I64, _F, _P, _SZ, _P]),
    "int8_matmul_products": (_I, [_I64, _I64, _I, _P, _P, _I64, _P, _P, _SZ, _P]),
    "int8_quantize_weight_fixed_workspace_bytes": (_SZ, [_I64]),
    "int8_quantize_weight_fixed": (_I, [_P, _I64, _I64, _I, _P, _I64, _P, _P, _P, _P, _SZ, _P]),
    "int8_matmul_fixed": (_I, [_P, _I64, _I64, _I, _P, _I64, _P, _P, _P, _I64, _P, _P, _SZ, _P]),
    "int8_blockwise_quantize": (_I, [_P, _I64, _I64, _P, _P, _P]),
    "int8_blockwise_dequantize": (_I, [_P, _P, _I64, _I64, _P, _P]),
    "int8_quantize_weight_group": (_I, [_P, _I64, _I64, _I, _I64, _P, _P, _P]),
    "int8_matmul_group_workspace_bytes": (_SZ, [_I64, _I64, _I64]),
    "int8_matmul_group_small_batch": (_I, [_I64, _I64, _I64, _I64]),
    "int8_matmul_group": (_I, [_P, _I64, _I64, _I, _I64, _P, _P, _I64, _P, _P, _SZ, _P]),
    "int8_matmul_group_prepare": (_I, [_P, _I64, _I64, _I, _I64, _P, _SZ, _P]),
    "int8_matmul_group_products": (_I, [_I64, _I64, _I, _I64, _P, _P, _I64, _P, _P, _SZ, _P]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libllmint8.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with python -m int8_quantized_matmul_rowwise_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().llmint8_status_string(int(status)).decode()


def _check(status: int, what: str) -> None:
    if status != OK:
        raise LLMInt8Error(status, f"{what}: {status_string(status)}")


def _stream(t: torch.Tensor, stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return int(getattr(stream, "cuda_stream", stream) or 0)


def _dev_tensor(t: torch.Tensor, name: str, dtype=None) -> torch.Tensor:
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must have dtype {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None or t.numel() == 0 else t.data_ptr()


def int8_matmul_workspace_bytes(M: int, K: int, N: int) -> int:
    return int(lib().int8_matmul_workspace_bytes(M, K, N))


def int8_matmul_workspace_layout(M: int, K: int, N: int) -> dict:
    out = WorkspaceLayout()
    _check(lib().int8_matmul_workspace_layout(M, K, N, ctypes.byref(out)), "int8_matmul_workspace_layout")
    return {n: int(getattr(out, n)) for n, _ in WorkspaceLayout._fields_}


def _workspace(ws: Optional[torch.Tensor], nbytes: int, device) -> torch.Tensor:
    if ws is None:
        return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
    return _dev_tensor(ws, "workspace")


def int8_quantize_weight(W: torch.Tensor, Wq: Optional[torch.Tensor] = None, w_scale: Optional[torch.Tensor] = None,
                         stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """W (K x N, fp16/bf16) -> (Wq N x K int8, w_scale fp32[N])."""
    _dev_tensor(W, "W")
    if W.dtype not in _DT or W.dim() != 2:
        raise TypeError("W must be a 2-D fp16 or bf16 tensor")
    K, N = W.shape
    if Wq is None:
        Wq = torch.empty((N, K), dtype=torch.int8, device=W.device)
    if w_scale is None:
        w_scale = torch.empty((N,), dtype=torch.float32, device=W.device)
    _dev_tensor(Wq, "Wq", torch.int8)
    _dev_tensor(w_scale, "w_scale", torch.float32)
    if tuple(Wq.shape) != (N, K) or tuple(w_scale.shape) != (N,):
        raise ValueError("Wq must be N x K and w_scale N")
    _check(lib().int8_quantize_weight(_ptr(W), K, N, _DT[W.dtype], _ptr(Wq), _ptr(w_scale), _stream(W, stream)),
           "int8_quantize_weight")
    return Wq, w_scale


def int8_matmul(X: torch.Tensor, Wq: torch.Tensor, w_scale: torch.Tensor, threshold: float = 6.0,
                Y: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Y = LLM.int8() product of X (M x K, fp16/bf16) with the converted weight (Wq, w_scale)."""
    _dev_tensor(X, "X")
    if X.dtype not in _DT or X.dim() != 2:
        raise TypeError("X must be a 2-D fp16 or bf16 tensor")
    M, K = X.shape
    _dev_tensor(Wq, "Wq", torch.int8)
    _dev_tensor(w_scale, "w_scale", torch.float32)
    N = Wq.shape[0]
    if Wq.dim() != 2 or Wq.shape[1] != K or tuple(w_scale.shape) != (N,):
        raise ValueError("Wq must be N x K and w_scale N")
    if Y is None:
        Y = torch.empty((M, N), dtype=X.dtype, device=X.device)
    _dev_tensor(Y, "Y", X.dtype)
    if tuple(Y.shape) != (M, N):
        raise ValueError("Y must be M x N")
    nbytes = int8_matmul_workspace_bytes(M, K, N)
    ws = _workspace(workspace, nbytes, X.device)
    _check(lib().int8_matmul(_ptr(X), M, K, _DT[X.dtype], _ptr(Wq), _ptr(w_scale), N, float(threshold), _ptr(Y),
                             _ptr(ws), ws.numel(), _stream(X, stream)), "int8_matmul")
    return Y


NOALLOC_SCRATCH_BYTES = 64 << 20  # LLMINT8_NOALLOC_SCRATCH_BYTES


def int8_matmul_noalloc(X: torch.Tensor, Wq: torch.Tensor, w_scale: torch.Tensor, threshold: float = 6.0,
                        Y: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """int8_matmul on the library's own device scratch (no workspace; the library call
    allocates nothing -- pass Y to keep the binding from allocating it either)."""
    _dev_tensor(X, "X")
    if X.dtype not in _DT or X.dim() != 2:
        raise TypeError("X must be a 2-D fp16 or bf16 tensor")
    M, K = X.shape
    _dev_tensor(Wq, "Wq", torch.int8)
    _dev_tensor(w_scale, "w_scale", torch.float32)
    N = Wq.shape[0]
    if Wq.dim() != 2 or Wq.shape[1] != K or tuple(w_scale.shape) != (N,):
        raise ValueError("Wq must be N x K and w_scale N")
    if Y is None:
        Y = torch.empty((M, N), dtype=X.dtype, device=X.device)
    _dev_tensor(Y, "Y", X.dtype)
    if tuple(Y.shape) != (M, N):
        raise ValueError("Y must be M x N")
    _check(lib().int8_matmul_noalloc(_ptr(X), M, K, _DT[X.dtype], _ptr(Wq), _ptr(w_scale), N, float(threshold),
                                     _ptr(Y), _stream(X, stream)), "int8_matmul_noalloc")
    return Y


def int8_matmul_prepare(X: torch.Tensor, Wq: torch.Tensor, threshold: float = 6.0,
                        workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Stage 1 of int8_matmul (the X pass) into a workspace, which is returned."""
    _dev_tensor(X, "X")
    if X.dtype not in _DT or X.dim() != 2:
        raise TypeError("X must be a 2-D fp16 or bf16 tensor")
    M, K = X.shape
    _dev_tensor(Wq, "Wq", torch.int8)
    N = Wq.shape[0]
    ws = _workspace(workspace, int8_matmul_workspace_bytes(M, K, N), X.device)
    _check(lib().int8_matmul_prepare(_ptr(X), M, K, _DT[X.dtype], _ptr(Wq), N, float(threshold), _ptr(ws),
                                     ws.numel(), _stream(X, stream)), "int8_matmul_prepare")
    return ws


def int8_matmul_products(M: int, K: int, dtype: torch.dtype, Wq: torch.Tensor, w_scale: torch.Tensor,
                         workspace: torch.Tensor, Y: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Stage 2 of int8_matmul: the products and the epilogue from a prepared workspace."""
    _dev_tensor(Wq, "Wq", torch.int8)
    _dev_tensor(w_scale, "w_scale", torch.float32)
    _dev_tensor(workspace, "workspace")
    N = Wq.shape[0]
    if Y is None:
        Y = torch.empty((M, N), dtype=dtype, device=Wq.device)
    _dev_tensor(Y, "Y", dtype)
    _check(lib().int8_matmul_products(M, K, _DT[dtype], _ptr(Wq), _ptr(w_scale), N, _ptr(Y), _ptr(workspace),
                                      workspace.numel(), _stream(Wq, stream)), "int8_matmul_products")
    return Y


def int8_matmul_stats(X: torch.Tensor, threshold: float = 6.0, outlier_cols: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None, stream=None) -> Tuple[int, torch.Tensor]:
    """(n_O, O[:n_O]) -- the outlier feature dimensions of X (synchronizes the stream)."""
    _dev_tensor(X, "X")
    if X.dtype not in _DT or X.dim() != 2:
        raise TypeError("X must be a 2-D fp16 or bf16 tensor")
    M, K = X.shape
    if outlier_cols is None:
        outlier_cols = torch.empty((max(K, 1),), dtype=torch.int32, device=X.device)
    _dev_tensor(outlier_cols, "outlier_cols", torch.int32)
    nbytes = int8_matmul_workspace_bytes(M, K, 0)
    ws = _workspace(workspace, nbytes, X.device)
    n = ctypes.c_int32(0)
    _check(lib().int8_matmul_stats(_ptr(X), M, K, _DT[X.dtype], float(threshold), ctypes.byref(n),
                                   outlier_cols.data_ptr(), _ptr(ws), ws.numel(), _stream(X, stream)),
           "int8_matmul_stats")
    return int(n.value), outlier_cols[: n.value]


def int8_matmul_accumulators(X: torch.Tensor, Wq: torch.Tensor, threshold: float = 6.0,
                             workspace: Optional[torch.Tensor] = None, stream=None):
    """Test hook: (C int32 M x N, F fp32 M x N, workspace) from the product kernels."""
    _dev_tensor(X, "X")
    M, K = X.shape
    N = Wq.shape[0]
    C = torch.empty((M, N), dtype=torch.int32, device=X.device)
    F = torch.empty((M, N), dtype=torch.float32, device=X.device)
    ws = _workspace(workspace, int8_matmul_workspace_bytes(M, K, N), X.device)
    _check(lib().int8_matmul_accumulators(_ptr(X), M, K, _DT[X.dtype], _ptr(Wq), N, float(threshold), _ptr(C),
                                          _ptr(F), _ptr(ws), ws.numel(), _stream(X, stream)),
           "int8_matmul_accumulators")
    return C, F, ws


def workspace_views(ws: torch.Tensor, M: int, K: int, N: int, dtype: torch.dtype) -> dict:
    """Views of the X pass's products left in an int8_matmul workspace (see the header)."""
    L = int8_matmul_workspace_layout(M, K, N)
    b = ws.view(torch.uint8)
    n_o = int(b[L["n_outliers"]: L["n_outliers"] + 4].view(torch.int32).item())
    P = int(math.ceil(n_o / 32) * 32)
    xq = b[L["xq"]: L["xq"] + M * L["xq_pitch"]].view(torch.int8).view(M, L["xq_pitch"]) if L["xq_pitch"] else None
    xo = b[L["xo"]: L["xo"] + 2 * M * L["xo_pitch"]].view(dtype).view(M, L["xo_pitch"]) if L["xo_pitch"] else None
    # the small-batch path has no W_O region (its product kernel gathers Wq[:,O] itself)
    wo = (b[L["wo"]: L["wo"] + 2 * N * L["xo_pitch"]].view(dtype).view(N, L["xo_pitch"])
          if L["xo_pitch"] and not L["small_batch"] else None)
    return {
        "n_outliers": n_o,
        "outliers": b[L["outliers"]: L["outliers"] + 4 * n_o].view(torch.int32),
        "Xq": None if xq is None else xq[:, :K],
        "Xq_pad": None if xq is None else xq[:, K:],
        "s_x": b[L["s_x"]: L["s_x"] + 4 * M].view(torch.float32),
        "XO": None if xo is None else xo[:, :P],
        "WO": None if wo is None else wo[:, :P],
    }


def _fixed_pitch(n_o: int) -> int:
    return (n_o + 31) // 32 * 32


def int8_quantize_weight_fixed(W: torch.Tensor, outlier_cols: torch.Tensor, stream=None):
    """Weight conversion with a fixed outlier set (device int32, ascending):
    (Wq N x K int8, w_scale fp32[N], W_O N x P 16-bit exact rows)."""
    _dev_tensor(W, "W")
    if W.dtype not in _DT or W.dim() != 2:
        raise TypeError("W must be a 2-D fp16 or bf16 tensor")
    _dev_tensor(outlier_cols, "outlier_cols", torch.int32)
    K, N = W.shape
    n_o = outlier_cols.numel()
    Wq = torch.empty((N, K), dtype=torch.int8, device=W.device)
    s_w = torch.empty(N, dtype=torch.float32, device=W.device)
    W_O = torch.empty((N, _fixed_pitch(n_o)), dtype=W.dtype, device=W.device)
    ws = torch.empty(max(int(lib().int8_quantize_weight_fixed_workspace_bytes(K)), 1), dtype=torch.uint8,
                     device=W.device)
    _check(lib().int8_quantize_weight_fixed(_ptr(W), K, N, _DT[W.dtype], _ptr(outlier_cols), n_o, _ptr(Wq), _ptr(s_w),
                                            _ptr(W_O), _ptr(ws), ws.numel(), _stream(W, stream)),
           "int8_quantize_weight_fixed")
    return Wq, s_w, W_O


def int8_matmul_fixed(X: torch.Tensor, outlier_cols: torch.Tensor, Wq: torch.Tensor, w_scale: torch.Tensor,
                      W_O: torch.Tensor, Y: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                      stream=None) -> torch.Tensor:
    """Y = X W with the fixed outlier set (no detection; exact 16-bit W rows on the set)."""
    _dev_tensor(X, "X")
    if X.dtype not in _DT or X.dim() != 2:
        raise TypeError("X must be a 2-D fp16 or bf16 tensor")
    _dev_tensor(outlier_cols, "outlier_cols", torch.int32)
    _dev_tensor(Wq, "Wq", torch.int8)
    _dev_tensor(w_scale, "w_scale", torch.float32)
    _dev_tensor(W_O, "W_O", X.dtype)
    M, K = X.shape
    N = Wq.shape[0]
    n_o = outlier_cols.numel()
    if W_O.shape != (N, _fixed_pitch(n_o)):
        raise ValueError("W_O must be N x (n_O rounded up to 32)")
    if Y is None:
        Y = torch.empty((M, N), dtype=X.dtype, device=X.device)
    ws = _workspace(workspace, int8_matmul_workspace_bytes(M, K, N), X.device)
    _check(lib().int8_matmul_fixed(_ptr(X), M, K, _DT[X.dtype], _ptr(outlier_cols), n_o, _ptr(Wq), _ptr(w_scale),
                                   _ptr(W_O), N, _ptr(Y), _ptr(ws), ws.numel(), _stream(X, stream)),
           "int8_matmul_fixed")
    return Y


def int8_blockwise_quantize(x: torch.Tensor, block: int = 2048, q: Optional[torch.Tensor] = None,
                            absmax: Optional[torch.Tensor] = None, stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Block-wise absmax int8 code of an fp32 tensor, taken flat: (q int8 of x's shape,
    absmax fp32[ceil(numel / block)])."""
    _dev_tensor(x, "x", torch.float32)
    n = x.numel()
    nb = -(-n // block) if block > 0 else 0
    if q is None:
        q = torch.empty(x.shape, dtype=torch.int8, device=x.device)
    if absmax is None:
        absmax = torch.empty(nb, dtype=torch.float32, device=x.device)
    _dev_tensor(q, "q", torch.int8)
    _dev_tensor(absmax, "absmax", torch.float32)
    if q.numel() != n or absmax.numel() != nb:
        raise ValueError("q must hold numel(x) codes and absmax ceil(numel / block) scales")
    _check(lib().int8_blockwise_quantize(_ptr(x), n, int(block), _ptr(q), _ptr(absmax), _stream(x, stream)),
           "int8_blockwise_quantize")
    return q, absmax


def int8_blockwise_dequantize(q: torch.Tensor, absmax: torch.Tensor, block: int = 2048,
                              x: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Decode of int8_blockwise_quantize: fp32 of q's shape."""
    _dev_tensor(q, "q", torch.int8)
    _dev_tensor(absmax, "absmax", torch.float32)
    n = q.numel()
    if x is None:
        x = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    _dev_tensor(x, "x", torch.float32)
    if x.numel() != n or absmax.numel() != (-(-n // block) if block > 0 else 0):
        raise ValueError("x must hold numel(q) values and absmax ceil(numel / block) scales")
    _check(lib().int8_blockwise_dequantize(_ptr(q), _ptr(absmax), n, int(block), _ptr(x), _stream(q, stream)),
           "int8_blockwise_dequantize")
    return x


def int8_quantize_weight_group(W: torch.Tensor, group: int = 1024, stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """W (K x N, fp16/bf16) -> (Wq N x K int8, w_scale fp32 N x K/group): one scale per
    output column and group of `group` consecutive rows of W."""
    _dev_tensor(W, "W")
    if W.dtype not in _DT or W.dim() != 2:
        raise TypeError("W must be a 2-D fp16 or bf16 tensor")
    K, N = W.shape
    if group <= 0 or K % group:
        raise ValueError("group must divide K")
    Wq = torch.empty((N, K), dtype=torch.int8, device=W.device)
    s_w = torch.empty((N, K // group), dtype=torch.float32, device=W.device)
    _check(lib().int8_quantize_weight_group(_ptr(W), K, N, _DT[W.dtype], int(group), _ptr(Wq), _ptr(s_w),
                                            _stream(W, stream)), "int8_quantize_weight_group")
    return Wq, s_w


def int8_matmul_group_workspace_bytes(M: int, K: int, group: int) -> int:
    return int(lib().int8_matmul_group_workspace_bytes(M, K, group))


def int8_matmul_group_small_batch(M: int, K: int, N: int, group: int) -> bool:
    """True when int8_matmul_group takes the small-batch product kernel for these sizes."""
    r = int(lib().int8_matmul_group_small_batch(M, K, N, group))
    _check(min(r, 0), "int8_matmul_group_small_batch")
    return r == 1


def int8_matmul_group(X: torch.Tensor, Wq: torch.Tensor, w_scale: torch.Tensor, group: int = 1024,
                      Y: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                      stream=None) -> torch.Tensor:
    """Y = X W with group-wise scales along K on both operands (no outlier decomposition)."""
    _dev_tensor(X, "X")
    if X.dtype not in _DT or X.dim() != 2:
        raise TypeError("X must be a 2-D fp16 or bf16 tensor")
    _dev_tensor(Wq, "Wq", torch.int8)
    _dev_tensor(w_scale, "w_scale", torch.float32)
    M, K = X.shape
    N = Wq.shape[0]
    if group <= 0 or K % group or Wq.dim() != 2 or Wq.shape[1] != K or tuple(w_scale.shape) != (N, K // group):
        raise ValueError("Wq must be N x K and w_scale N x K/group, with group dividing K")
    if Y is None:
        Y = torch.empty((M, N), dtype=X.dtype, device=X.device)
    _dev_tensor(Y, "Y", X.dtype)
    if tuple(Y.shape) != (M, N):
        raise ValueError("Y must be M x N")
    ws = _workspace(workspace, int8_matmul_group_workspace_bytes(M, K, group), X.device)
    _check(lib().int8_matmul_group(_ptr(X), M, K, _DT[X.dtype], int(group), _ptr(Wq), _ptr(w_scale), N, _ptr(Y),
                                   _ptr(ws), ws.numel(), _stream(X, stream)), "int8_matmul_group")
    return Y


def int8_matmul_group_prepare(X: torch.Tensor, group: int, workspace: torch.Tensor, stream=None) -> None:
    """The X pass of int8_matmul_group into `workspace`."""
    _dev_tensor(X, "X")
    if X.dtype not in _DT or X.dim() != 2:
        raise TypeError("X must be a 2-D fp16 or bf16 tensor")
    _dev_tensor(workspace, "workspace")
    M, K = X.shape
    _check(lib().int8_matmul_group_prepare(_ptr(X), M, K, _DT[X.dtype], int(group), _ptr(workspace),
                                           workspace.numel(), _stream(X, stream)), "int8_matmul_group_prepare")


def int8_matmul_group_products(M: int, K: int, dtype: torch.dtype, group: int, Wq: torch.Tensor,
                               w_scale: torch.Tensor, workspace: torch.Tensor, Y: Optional[torch.Tensor] = None,
                               stream=None) -> torch.Tensor:
    """The products of int8_matmul_group from a workspace filled by int8_matmul_group_prepare."""
    _dev_tensor(Wq, "Wq", torch.int8)
    _dev_tensor(w_scale, "w_scale", torch.float32)
    _dev_tensor(workspace, "workspace")
    N = Wq.shape[0]
    if group <= 0 or K % group or Wq.dim() != 2 or Wq.shape[1] != K or tuple(w_scale.shape) != (N, K // group):
        raise ValueError("Wq must be N x K and w_scale N x K/group, with group dividing K")
    if Y is None:
        Y = torch.empty((M, N), dtype=dtype, device=Wq.device)
    _dev_tensor(Y, "Y", dtype)
    if tuple(Y.shape) != (M, N):
        raise ValueError("Y must be M x N")
    _check(lib().int8_matmul_group_products(M, K, _DT[dtype], int(group), _ptr(Wq), _ptr(w_scale), N, _ptr(Y),
                                            _ptr(workspace), workspace.numel(), _stream(Wq, stream)),
           "int8_matmul_group_products")
    return Y


def group_workspace_views(ws: torch.Tensor, M: int, K: int, group: int) -> dict:
    """The X pass's products left in an int8_matmul_group workspace (see the header)."""
    ng = K // group
    b = ws.view(torch.uint8)
    o_s = (M * K + 255) // 256 * 256
    o_r = (o_s + 4 * M * ng + 255) // 256 * 256
    return {
        "Xq": b[: M * K].view(torch.int8).view(M, K),
        "s_x": b[o_s: o_s + 4 * M * ng].view(torch.float32).view(M, ng),
        "r": b[o_r: o_r + 4 * M * ng].view(torch.float32).view(ng, M),
    }


__all__ = [
    "int8_quantize_weight", "int8_matmul", "int8_matmul_noalloc", "int8_matmul_stats", "int8_matmul_prepare", "int8_matmul_products", "int8_matmul_workspace_bytes",
    "int8_matmul_workspace_layout", "int8_matmul_accumulators", "workspace_views", "LLMInt8Error", "lib",
    "int8_blockwise_quantize", "int8_blockwise_dequantize", "int8_quantize_weight_fixed", "int8_matmul_fixed",
    "status_string", "int8_quantize_weight_group", "int8_matmul_group", "int8_matmul_group_workspace_bytes",
    "group_workspace_views", "int8_matmul_group_small_batch", "int8_matmul_group_prepare", "int8_matmul_group_products",
]
