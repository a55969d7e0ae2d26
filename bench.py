#!/usr/bin/env python3
"""Benchmark of the LLM.int8() matmul on one MI355X.

A step is one int8_matmul call on resident inputs: the X pass (outlier columns, row
scales, int8 codes, outlier gather) and the products with the dequantizing epilogue.
The weight conversion is offline and not timed.  Default workload: the 175B-like QKV
projection, X 4096 x 12288 fp16 (7 outlier feature dimensions), W 12288 x 36864.

Printed: one JSON line with
  value            effective TOPS of the whole step, 2*M*N*K / step time
  pct_of_i8_peak   value / 5000 TOPS (MI355X dense int8 MFMA)
  roofline         the dominant kernel (the product kernel): 2*M*N*K per launch over its
                   average duration, from HIP events around back-to-back launches on
                   the library's stream; traffic = HBM bytes per launch from rocprofv3
                   FETCH_SIZE / WRITE_SIZE counters, when the stored measurement was
                   taken on the current kernel source (else null)
  cpu_baseline     the CPU oracle on a bounded sample of the same workload
  fp16_gemm        torch.matmul (hipBLASLt) of X and W in the 16-bit type, same shape
Progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

I8_PEAK_TOPS = 5000.0
KERNEL_SOURCES = ["int8_quantized_matmul_rowwise_amd/csrc/gemm.hip", "int8_quantized_matmul_rowwise_amd/csrc/common.hpp"]


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def stored_traffic(workload: str):
    """HBM bytes per launch of the product kernel from a committed rocprofv3 counter
    summary, if it was taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"gemm_kernel_traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def time_loop(fn, steps: int, torch) -> float:
    """Average ms per call of fn over `steps` back-to-back calls (HIP events on the current stream)."""
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s.record()
    for _ in range(steps):
        fn()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / steps


def cpu_baseline(x, w, wl, seconds: float) -> dict:
    import numpy as np

    import oracle
    import workloads

    cores = min(int(os.environ.get("OMP_NUM_THREADS") or os.cpu_count()), os.cpu_count())
    cores = oracle.set_threads(cores)
    X = workloads.bits(x)
    W = workloads.bits(w)
    log(f"cpu baseline: oracle weight conversion (untimed, offline) on {cores} threads")
    Wq, s_w = oracle.quantize_weight(W, wl.dtype)
    t0 = time.perf_counter()
    O = oracle.outlier_columns(X, wl.dtype, wl.tau)
    Xq, s_x, XO = oracle.quantize_rows(X, wl.dtype, O)
    t_xpass = time.perf_counter() - t0

    def products(rows):
        t = time.perf_counter()
        C = oracle.int_gemm(Xq, Wq, rows)
        F, _, _ = oracle.outlier_gemm(XO, O, wl.dtype, Wq, rows)
        oracle.dequant(C, F, s_x[rows], s_w, wl.dtype)
        return time.perf_counter() - t

    probe = np.arange(min(4, wl.M))
    t_probe = products(probe)
    R = int(max(1, min(wl.M, probe.size * max(0.0, seconds - t_xpass) / max(t_probe, 1e-9))))
    rows = np.arange(R)
    log(f"cpu baseline: X pass {t_xpass:.2f} s over {wl.M} rows; products for {R} rows")
    t_prod = products(rows)
    t = t_prod + t_xpass * R / wl.M
    return {
        "value": 2.0 * R * wl.N * wl.K / t / 1e12,
        "unit": "TOPS",
        "cores": cores,
        "kind": "oracle",
        "sample": f"X pass over all {wl.M} rows (time prorated to the sample) + int8 and 16-bit products and "
                  f"epilogue for rows 0..{R - 1} of {wl.M}; {t:.1f} s of CPU work",
    }


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="qkv_175b")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="CPU work budget of the oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fp16-gemm", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported "
              f"(the library has no multi-GPU path)", file=sys.stderr)
        return 2

    import torch

    import int8_quantized_matmul_rowwise_amd as lm
    import workloads

    lm.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = workloads.WORKLOADS[args.workload]
    log(f"workload {wl.name}: X {wl.M}x{wl.K} {wl.dtype}, W {wl.K}x{wl.N}, tau {wl.tau}")
    x, w, cols, _ = workloads.make_workload(wl.name)
    X = x.to(dev)
    W = w.to(dev)
    Wq, s_w = lm.int8_quantize_weight(W)
    ws = torch.empty(lm.int8_matmul_workspace_bytes(wl.M, wl.K, wl.N), dtype=torch.uint8, device=dev)
    Y = torch.empty((wl.M, wl.N), dtype=X.dtype, device=dev)
    torch.cuda.synchronize()

    def step():
        lm.int8_matmul(X, Wq, s_w, wl.tau, Y=Y, workspace=ws)

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    t_wall = time.perf_counter()
    ms_step = time_loop(step, args.steps, torch)
    t_wall = time.perf_counter() - t_wall
    n_out, _ = lm.int8_matmul_stats(X, wl.tau)
    ops = 2.0 * wl.M * wl.N * wl.K
    tops = ops / (ms_step * 1e-3) / 1e12

    # the dominant kernel alone: the product kernel, launched back to back on a prepared workspace
    lm.int8_matmul_prepare(X, Wq, wl.tau, workspace=ws)
    for _ in range(3):
        lm.int8_matmul_products(wl.M, wl.K, X.dtype, Wq, s_w, ws, Y=Y)
    ms_gemm = time_loop(lambda: lm.int8_matmul_products(wl.M, wl.K, X.dtype, Wq, s_w, ws, Y=Y), args.steps, torch)
    ms_xpass = time_loop(lambda: lm.int8_matmul_prepare(X, Wq, wl.tau, workspace=ws), args.steps, torch)
    gemm_tops = ops / (ms_gemm * 1e-3) / 1e12
    log(f"step {ms_step * 1e3:.1f} us = {tops:.0f} TOPS; product kernel {ms_gemm * 1e3:.1f} us = {gemm_tops:.0f} TOPS;"
        f" X pass {ms_xpass * 1e3:.1f} us; n_outliers {n_out}")

    fp16 = None
    if not args.no_fp16_gemm:
        for _ in range(3):
            torch.matmul(X, W)
        ms16 = time_loop(lambda: torch.matmul(X, W), max(5, args.steps // 2), torch)
        fp16 = {"ms": ms16, "tflops": ops / (ms16 * 1e-3) / 1e12,
                "pct_of_peak": ops / (ms16 * 1e-3) / 1e12 / 2500.0 * 100.0,
                "what": f"torch.matmul (hipBLASLt) {wl.dtype} X @ W at the same shape"}
        log(f"fp16 GEMM {ms16 * 1e3:.1f} us = {fp16['tflops']:.0f} TFLOP/s")
    del W
    torch.cuda.empty_cache()

    traffic = stored_traffic(wl.name)
    line = {
        "metric": "effective TOPS of int8 outlier-decomposed matmul; % i8 MFMA peak",
        "value": tops,
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic",
        "config": {"workload": wl.name, "M": wl.M, "K": wl.K, "N": wl.N, "x_dtype": wl.dtype,
                   "threshold": wl.tau, "n_outliers": n_out, "seed": 0},
        "pct_of_i8_peak": tops / I8_PEAK_TOPS * 100.0,
        "roofline": {"bound": "mfma", "achieved": gemm_tops, "peak": I8_PEAK_TOPS, "unit": "TFLOP/s",
                     "frac": gemm_tops / I8_PEAK_TOPS, "traffic": traffic,
                     "kernel": "gemm_kernel", "kernel_ms": ms_gemm, "xpass_ms": ms_xpass},
        "cpu_baseline": None,
        "fp16_gemm": fp16,
        "wall_s_timed": t_wall,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(x, w, wl, args.cpu_seconds)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
