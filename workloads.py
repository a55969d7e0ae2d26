"""Seeded synthetic inputs for the LLM.int8() matmul (shared by the tests and the benchmark).

This module holds none of the method's arithmetic: it only draws X and W.  Shapes and
value distributions follow the five synthetic projection-layer workloads the build is
measured on (stand-ins for the models named on the "LLM.int8()" page's abstract and
the talk summary's outlier discussion; no model weights are available):

  tiny        X 32x256 fp16 ~N(0,1), columns {7,131} overwritten by +-U(8,20);
              W 256x128 fp16 ~N(0,0.02)
  ffn_up      X 2048x4096 fp16 ~N(0,1), 6 seeded columns at +-U(6,60) in every row;
              W 4096x16384 fp16 ~N(0,0.02)                       (6.7B-like FFN up-proj)
  decode      X 16x8192 bf16 ~N(0,1), 8 columns at +-U(10,40); W 8192x8192 bf16 ~N(0,0.015)
  qkv_175b    X 4096x12288 fp16 ~N(0,1), 7 columns at +-U(20,60); W 12288x36864 fp16 ~N(0,0.01)
  ffn_down    X 8192x28672 bf16 ~N(0,1), 64 columns at +-U(6,100); W 28672x8192 bf16 ~N(0,0.01)

Threshold 6.0 everywhere, seed 0 unless stated.

Recipe (identical on every machine with this torch build): a torch CPU generator per
tensor, seeded with ``(seed << 24) ^ (workload_id << 8) ^ tensor_id``; normals are drawn in
fp32 and scaled by sigma; an outlier value is an independent fair sign times an
independent U(a, b) magnitude, written into every row of each chosen column; the
chosen columns are the first n of a seeded random permutation of range(K), sorted
(fixed columns for ``tiny``).  The fp32 tensor is rounded once to the 16-bit dtype
(round to nearest even).
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass
from typing import Optional, Sequence, Tuple

import numpy as np
import torch

DTYPES = {"fp16": torch.float16, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class Workload:
    name: str
    wid: int
    M: int
    K: int
    N: int
    dtype: str
    x_sigma: float
    w_sigma: float
    n_outliers: int
    outlier_range: Tuple[float, float]
    fixed_cols: Optional[Tuple[int, ...]] = None
    tau: float = 6.0
    description: str = ""

    @property
    def flops(self) -> float:
        return 2.0 * self.M * self.N * self.K


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny", 0, 32, 256, 128, "fp16", 1.0, 0.02, 2, (8.0, 20.0), fixed_cols=(7, 131),
                 description="tiny check case"),
        Workload("ffn_up", 1, 2048, 4096, 16384, "fp16", 1.0, 0.02, 6, (6.0, 60.0),
                 description="FFN up-projection, 6.7B-like"),
        Workload("decode", 2, 16, 8192, 8192, "bf16", 1.0, 0.015, 8, (10.0, 40.0),
                 description="decode-shaped, memory-bound"),
        Workload("qkv_175b", 3, 4096, 12288, 36864, "fp16", 1.0, 0.01, 7, (20.0, 60.0),
                 description="QKV projection, 175B-like"),
        Workload("ffn_down", 4, 8192, 28672, 8192, "bf16", 1.0, 0.01, 64, (6.0, 100.0),
                 description="outlier stress, FFN down-projection"),
    ]
}


def _gen(seed: int, wid: int, tid: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed((int(seed) << 24) ^ (int(wid) << 8) ^ int(tid))
    return g


def make_x(M: int, K: int, dtype: str, *, sigma: float = 1.0, n_outliers: int = 0,
           outlier_range: Tuple[float, float] = (8.0, 20.0), fixed_cols: Optional[Sequence[int]] = None,
           seed: int = 0, wid: int = 99) -> Tuple[torch.Tensor, np.ndarray]:
    """X (M x K, 16-bit, CPU) and the sorted injected outlier columns."""
    x = torch.randn(M, K, generator=_gen(seed, wid, 1), dtype=torch.float32)
    if sigma != 1.0:
        x.mul_(sigma)
    if fixed_cols is not None:
        cols = np.array(sorted(int(c) for c in fixed_cols), dtype=np.int64)
    elif n_outliers > 0:
        perm = torch.randperm(K, generator=_gen(seed, wid, 2))
        cols = np.sort(perm[:n_outliers].numpy().astype(np.int64))
    else:
        cols = np.zeros(0, dtype=np.int64)
    if cols.size and M > 0:
        g = _gen(seed, wid, 3)
        a, b = outlier_range
        sign = torch.randint(0, 2, (M, cols.size), generator=g).to(torch.float32) * 2.0 - 1.0
        mag = a + (b - a) * torch.rand(M, cols.size, generator=g, dtype=torch.float32)
        x[:, torch.from_numpy(cols)] = sign * mag
    return x.to(DTYPES[dtype]), cols


def make_w(K: int, N: int, dtype: str, *, sigma: float = 0.02, seed: int = 0, wid: int = 99) -> torch.Tensor:
    """W (K x N, 16-bit, CPU), ~N(0, sigma)."""
    w = torch.randn(K, N, generator=_gen(seed, wid, 4), dtype=torch.float32)
    w.mul_(sigma)
    return w.to(DTYPES[dtype])


def with_rows(wl: Workload, rows: Optional[int]) -> Workload:
    """The workload with another number of rows of X (the same weight and X distribution)."""
    if rows is None or rows == wl.M:
        return wl
    return dataclasses.replace(wl, name=f"{wl.name}_m{rows}", M=int(rows))


def make_workload(name: str, seed: int = 0, rows: Optional[int] = None):
    """(X, W, injected_cols, workload) for a named workload; rows: another number of rows of X
    (the first rows of the same draw: the generators run in row-major order)."""
    wl = with_rows(WORKLOADS[name], rows)
    x, cols = make_x(wl.M, wl.K, wl.dtype, sigma=wl.x_sigma, n_outliers=wl.n_outliers,
                     outlier_range=wl.outlier_range, fixed_cols=wl.fixed_cols, seed=seed, wid=wl.wid)
    w = make_w(wl.K, wl.N, wl.dtype, sigma=wl.w_sigma, seed=seed, wid=wl.wid)
    return x, w, cols, wl


def bits(t: torch.Tensor) -> np.ndarray:
    """The raw 16-bit patterns of a CPU fp16/bf16 tensor as a numpy uint16 array (no copy)."""
    assert t.dtype in (torch.float16, torch.bfloat16) and t.device.type == "cpu"
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def from_bits(b: np.ndarray, dtype: str) -> torch.Tensor:
    """Inverse of bits(): a CPU tensor of the given 16-bit dtype over the same patterns."""
    return torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(DTYPES[dtype])


# ---- inputs of the block-wise codec: a flat fp32 optimizer-state-like tensor

CODEC_WORKLOAD = {"name": "adam_state", "n": 1 << 28, "block": 2048,
                  "description": "a 2^28-element fp32 optimizer state (1 GiB), blocks of 2048"}


def make_state(n: int, seed: int = 0, sigma: float = 1e-3, tail: float = 1e-3) -> torch.Tensor:
    """fp32 values ~ N(0, sigma) with a thin tail (a fraction `tail`) of entries of magnitude
    U(0.01, 0.5) and random sign: the spread of an Adam moment, whose rare large entries are
    what block-wise scaling is for.  Seeded torch CPU generator (tensor id 7)."""
    g = _gen(seed, 90, 7)
    x = torch.randn(n, generator=g, dtype=torch.float32) * sigma
    k = torch.rand(n, generator=g) < tail
    nk = int(k.sum())
    sign = torch.where(torch.rand(nk, generator=g) < 0.5, -1.0, 1.0)
    x[k] = sign * (0.01 + 0.49 * torch.rand(nk, generator=g))
    return x
