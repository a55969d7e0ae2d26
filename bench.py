#!/usr/bin/env python3
"""Benchmark of the LLM.int8() matmul on one MI355X.

A step is one int8_matmul call on resident inputs: the X pass (outlier columns, row
scales, int8 codes, outlier gather) and the products with the dequantizing epilogue.
The weight conversion is offline and not timed.  Default workload: the 175B-like QKV
projection, X 4096 x 12288 fp16 (7 outlier feature dimensions), W 12288 x 36864.

Printed: one JSON line with
  value            effective TOPS of the whole step, 2*M*N*K / step time
  pct_of_i8_peak   value / 5000 TOPS (MI355X dense int8 MFMA)
  roofline         the dominant kernel (the product kernel, which also runs the outlier
                   product and the epilogue): per launch, the algorithmic work -- 2*M*N*K
                   ops for the tiled kernel (bound "mfma"), or the Wq + Xq + Y bytes for
                   the small-batch kernel (bound "hbm") -- over its average duration,
                   from HIP events around back-to-back launches on the library's stream;
                   traffic = HBM bytes per launch from rocprofv3 FETCH_SIZE and
                   WRITE_SIZE counters scaled by a copy calibration, when the stored
                   measurement was taken on the current kernel source (else null)
  cpu_baseline     the CPU oracle on a bounded sample of the same workload
  fp16_gemm        torch.matmul (hipBLASLt) of X and W in the 16-bit type, same shape
Progress goes to stderr.

Other modes, each with its own JSON line of the same shape:
  --fixed          the fixed-outlier path (the workload's injected columns as the set)
  --group G        the group-wise path, groups of G features along K (no outlier split);
                   the dominant kernel is the grouped product kernel
  --codec          the block-wise absmax int8 codec on a 2^28-element fp32 state (GB/s)
  --gpus N         N > 1 exits with a message: the library runs on one GPU

Counter measurement of `traffic` (one rocprofv3 run per counter, then on any host):
  rocprofv3 --pmc FETCH_SIZE --output-format csv -d DIR_F -o run -- \\
      python3 bench.py --steps 3 --warmup 1 --no-cpu-baseline --no-fp16-gemm --copy-mib 1024
  (the same with WRITE_SIZE into DIR_W), then
  python3 bench.py --traffic-summary DIR_F DIR_W [--workload NAME] [--group G]
which writes profiles/<kernel>_traffic_<workload>.json and .md.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

I8_PEAK_TOPS = 5000.0
HBM_PEAK_GBS = 8000.0
CSRC = "int8_quantized_matmul_rowwise_amd/csrc/"
# the product kernel of each batch path and the sources it is built from
KERNELS = {
    "gemm_kernel": [CSRC + "gemm.hip", CSRC + "common.hpp"],
    "gemm_small_kernel": [CSRC + "gemm_small.hip", CSRC + "common.hpp"],
    "gemm_group_kernel": [CSRC + "gemm_group.hip", CSRC + "common.hpp"],
}


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def product_kernel(M: int, K: int, N: int, group: int = 0) -> str:
    """The product kernel the library runs for these sizes (it reports its own choice)."""
    if group:
        return "gemm_group_kernel"
    import int8_quantized_matmul_rowwise_amd as lm
    return "gemm_small_kernel" if lm.int8_matmul_workspace_layout(M, K, N)["small_batch"] else "gemm_kernel"


def workload_tag(wl, group: int = 0) -> str:
    """The name of a timed configuration: the workload, with the group size for the group-wise path."""
    return f"{wl.name}_g{group}" if group else wl.name


def algorithmic_bytes(wl, group: int = 0) -> int:
    """Bytes the product kernel must move per launch: Xq, Wq, their scales (or factors), Y."""
    ng = wl.K // group if group else 1
    return wl.M * wl.K + wl.N * wl.K + 4 * ng * (wl.N + wl.M) + 2 * wl.M * wl.N


def kernel_source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for p in KERNELS[kernel]:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_path(kernel: str, workload: str, ext: str) -> str:
    return os.path.join(ROOT, "profiles", f"{kernel}_traffic_{workload}.{ext}")


def stored_traffic(kernel: str, workload: str):
    """HBM bytes per launch of the product kernel from the committed counter record, if it
    was taken on the current kernel source."""
    path = traffic_path(kernel, workload, "json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256") != kernel_source_hash(kernel):
        log(f"stored traffic for {kernel} was measured on another kernel source: traffic = null")
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

    # The oracle's products run one row per thread, so the probe takes one row per thread
    # and the sample is a whole number of such rounds.
    probe = np.arange(min(cores, wl.M))
    t_probe = products(probe)
    rounds = int(max(1.0, (seconds - t_xpass) / max(t_probe, 1e-9)))
    R = int(min(wl.M, probe.size * rounds))
    rows = np.arange(R)
    log(f"cpu baseline: X pass {t_xpass:.2f} s over {wl.M} rows; products for {R} rows")
    t_prod = products(rows)
    t = t_prod + t_xpass * R / wl.M
    reps = 1
    if R == wl.M and t < seconds / 4:
        # the whole workload is small: repeat the whole call (X pass + products) for a stable time
        reps = int(min(1000, max(2, seconds / 4 / max(t, 1e-6))))
        t0 = time.perf_counter()
        for _ in range(reps):
            O = oracle.outlier_columns(X, wl.dtype, wl.tau)
            Xq, s_x, XO = oracle.quantize_rows(X, wl.dtype, O)
            products(rows)
        t = (time.perf_counter() - t0) / reps
    sample = (f"X pass over all {wl.M} rows (time prorated to the sample) + int8 and 16-bit products and "
              f"epilogue for rows 0..{R - 1} of {wl.M}; {t:.1f} s of CPU work")
    if reps > 1:
        sample = f"the whole call (all {wl.M} rows) repeated {reps} times, {t * reps:.1f} s of CPU work"
    return {
        "value": 2.0 * R * wl.N * wl.K / t / 1e12,
        "unit": "TOPS",
        "cores": cores,
        "kind": "oracle",
        "sample": sample,
    }


# ---------------------------------------------------------------------------------------
# counter summary (host only)

def _counter_rows(d: str):
    files = sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True))
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    rows = []
    for f in files:
        with open(f, newline="") as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def _per_dispatch(rows, counter: str, match) -> list:
    """Counter value (KiB) of each dispatch whose kernel name satisfies match."""
    vals = {}
    for r in rows:
        if r["Counter_Name"] == counter and match(r["Kernel_Name"]):
            key = (r.get("Process_Id"), r["Dispatch_Id"])
            vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
    return list(vals.values())


def traffic_summary(fetch_dir: str, write_dir: str, wl, copy_mib: int, group: int = 0) -> int:
    kernel = product_kernel(wl.M, wl.K, wl.N, group)
    tag = workload_tag(wl, group)
    gflag = f" --group {group}" if group else ""
    copy_bytes = copy_mib * 1024 * 1024
    is_copy = lambda name: "elementwise_kernel" in name  # the calibration copy (torch add of 1 GiB)
    is_prod = lambda name: f"::{kernel}<" in name
    out = {"kernel": kernel, "workload": tag, "kernel_source_sha256": kernel_source_hash(kernel),
           "copy_calibration_bytes": copy_bytes}
    lines = [f"# {kernel} HBM traffic, workload {tag} ({wl.M}x{wl.K}x{wl.N} {wl.dtype})", ""]
    total = 0.0
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = _counter_rows(d)
        copies = _per_dispatch(rows, counter, is_copy)
        names = sorted({r["Kernel_Name"] for r in rows if is_copy(r["Kernel_Name"])})
        lines.append(f"- calibration kernel(s) for {counter}: " + "; ".join(n[:120] for n in names))
        prods = _per_dispatch(rows, counter, is_prod)
        if not copies or not prods:
            raise SystemExit(f"{counter}: {len(copies)} copy and {len(prods)} product dispatches found in {d}")
        copy_kib = sum(copies) / len(copies)
        factor = copy_bytes / (copy_kib * 1024.0)
        prod_kib = sum(prods) / len(prods)
        bytes_ = prod_kib * 1024.0 * factor
        total += bytes_
        key = counter.split("_")[0].lower()
        out[f"{key}_counter_kib_per_launch"] = prod_kib
        out[f"{key}_copy_counter_kib"] = copy_kib
        out[f"{key}_factor"] = factor
        out[f"{key}_bytes_per_launch"] = bytes_
        lines += [f"- {counter}: copy of {copy_mib} MiB reads {copy_kib:.0f} KiB per dispatch "
                  f"(factor {factor:.4f}); {kernel}: {prod_kib:.0f} KiB per launch over {len(prods)} launches "
                  f"-> {bytes_ / 1e9:.4f} GB"]
    out["hbm_bytes_per_launch"] = total
    alg = algorithmic_bytes(wl, group)
    out["algorithmic_bytes_per_launch"] = alg
    lines += [f"- HBM bytes per launch: {total / 1e9:.4f} GB; algorithmic (Xq + Wq + scales + Y): {alg / 1e9:.4f} GB "
              f"({total / alg:.2f}x)", "",
              "Commands (from the repository root on the GPU box, then on any host):", "",
              "    cd /tmp && export TMPDIR=/tmp; cd -",
              f"    rocprofv3 --pmc FETCH_SIZE --output-format csv -d {fetch_dir} -o run -- python3 bench.py "
              f"--workload {wl.name}{gflag} --steps 3 --warmup 1 --no-cpu-baseline --no-fp16-gemm --copy-mib {copy_mib}",
              f"    rocprofv3 --pmc WRITE_SIZE --output-format csv -d {write_dir} -o run -- python3 bench.py "
              f"--workload {wl.name}{gflag} --steps 3 --warmup 1 --no-cpu-baseline --no-fp16-gemm --copy-mib {copy_mib}",
              f"    python3 bench.py --traffic-summary {fetch_dir} {write_dir} --workload {wl.name}{gflag} "
              f"--copy-mib {copy_mib}", ""]
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(traffic_path(kernel, tag, "json"), "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    with open(traffic_path(kernel, tag, "md"), "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))
    return 0


def trace_summary(trace_dir: str, bench_json: str, wl, cmd: str, group: int = 0) -> int:
    """Kernel-trace statistics of a profiled bench run (rocprofv3 --kernel-trace --stats),
    beside the bench line of that same run."""
    files = sorted(glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True))
    if not files:
        raise SystemExit(f"no kernel_stats.csv under {trace_dir}")
    with open(files[0], newline="") as fh:
        rows = list(csv.DictReader(fh))
    kernel = product_kernel(wl.M, wl.K, wl.N, group)
    tag = workload_tag(wl, group)
    lines = [f"# Kernel trace, workload {tag} ({wl.M}x{wl.K}x{wl.N} {wl.dtype})", "",
             "| kernel | calls | average us | min us | max us | share of GPU time |", "|---|---|---|---|---|---|"]
    avg_prod = None
    for r in rows:
        name = r["Name"]
        short = name.replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "").replace("llmint8::", "")
        avg = float(r["AverageNs"]) / 1e3
        if f"::{kernel}<" in name:
            avg_prod = avg
        lines.append(f"| `{short[:90]}` | {r['Calls']} | {avg:.1f} | {float(r['MinNs']) / 1e3:.1f} | "
                     f"{float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.2f} % |")
    if bench_json and os.path.exists(bench_json):
        with open(bench_json) as f:
            line = json.loads([l for l in f if l.startswith("{")][-1])
        ms = line["roofline"]["kernel_ms"]
        lines += ["", f"bench line of the same run: step {line['ms_per_step'] * 1e3:.1f} us, {kernel} "
                  f"{ms * 1e3:.1f} us per launch (HIP events), value {line['value']:.1f} {line['unit']}, "
                  f"roofline achieved {line['roofline']['achieved']:.1f} {line['roofline']['unit']}"]
        if avg_prod:
            lines.append(f"trace average of {kernel}: {avg_prod:.1f} us ({(avg_prod / (ms * 1e3) - 1) * 100:+.1f} % "
                         f"vs the events)")
    lines += ["", "Command (repository root on the GPU box):", "", "    " + cmd, ""]
    out = os.path.join(ROOT, "profiles", f"kernel_trace_{tag}.md")
    with open(out, "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))
    return 0


def codec_bench(args) -> int:
    """The block-wise absmax int8 codec on a 2^28-element fp32 optimizer state (blocks of
    2048): quantize and dequantize timed back to back (HIP events on the current stream),
    algorithmic bytes 4n + n + 4 n/block (quantize) and n + 4n + 4 n/block (dequantize)."""
    import numpy as np
    import torch

    import int8_quantized_matmul_rowwise_amd as lm
    import oracle
    import workloads

    wl = workloads.CODEC_WORKLOAD
    n, block = wl["n"], wl["block"]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"codec workload {wl['name']}: n = {n}, block {block}")
    x = workloads.make_state(n, seed=0)
    xd = x.to(dev)
    q, a = lm.int8_blockwise_quantize(xd, block)
    xr = lm.int8_blockwise_dequantize(q, a, block)
    for _ in range(args.warmup):
        lm.int8_blockwise_quantize(xd, block, q=q, absmax=a)
        lm.int8_blockwise_dequantize(q, a, block, x=xr)
    ms_q = time_loop(lambda: lm.int8_blockwise_quantize(xd, block, q=q, absmax=a), args.steps, torch)
    ms_d = time_loop(lambda: lm.int8_blockwise_dequantize(q, a, block, x=xr), args.steps, torch)
    nb = -(-n // block)
    bq = 5.0 * n + 4.0 * nb
    gbs_q = bq / (ms_q * 1e-3) / 1e9
    gbs_d = bq / (ms_d * 1e-3) / 1e9
    log(f"quantize {ms_q * 1e3:.1f} us = {gbs_q:.0f} GB/s; dequantize {ms_d * 1e3:.1f} us = {gbs_d:.0f} GB/s")
    # the oracle on a bounded sample (2^24 elements), on all host threads
    cores = oracle.set_threads(min(int(os.environ.get("OMP_NUM_THREADS") or os.cpu_count()), os.cpu_count()))
    xs = x[: 1 << 24].numpy()
    t0 = time.perf_counter()
    reps = 0
    while time.perf_counter() - t0 < args.cpu_seconds / 2 or reps == 0:
        qs, as_ = oracle.block_quantize(xs, block)
        oracle.block_dequantize(qs, as_, block)
        reps += 1
    t_cpu = (time.perf_counter() - t0) / reps
    line = {
        "metric": "GB/s of the block-wise absmax int8 codec (quantize + dequantize of an fp32 tensor)",
        "value": 2 * bq / ((ms_q + ms_d) * 1e-3) / 1e9,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_q + ms_d,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl["name"], "n": n, "block": block},
        "roofline": {"bound": "hbm", "achieved": gbs_q, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs_q / HBM_PEAK_GBS, "traffic": None, "kernel": "block_quantize_kernel",
                     "kernel_ms": ms_q, "dequantize_ms": ms_d, "dequantize_gbs": gbs_d},
        "cpu_baseline": {"value": 2 * (5.0 * xs.size + 4.0 * (-(-xs.size // block))) / t_cpu / 1e9, "unit": "GB/s",
                         "cores": cores, "kind": "oracle",
                         "sample": f"quantize + dequantize of the first 2^24 elements, {reps} times"},
    }
    print(json.dumps(line), flush=True)
    return 0


def calibration_copy(copy_mib: int, dev, torch) -> None:
    """Counter calibration: an elementwise kernel that reads and writes copy_mib MiB once."""
    n = copy_mib * 1024 * 1024 // 4
    src = torch.empty(n, dtype=torch.int32, device=dev)  # no fill kernel: the add is the only elementwise one
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.add(src, 1, out=dst)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()


def group_bench(args, wl) -> int:
    """The group-wise path (groups of G features along K on both operands, no outlier
    decomposition) on the workload's shape: a step is one int8_matmul_group call (X pass +
    products); the dominant kernel is the grouped product kernel (bound "mfma")."""
    import numpy as np
    import torch

    import int8_quantized_matmul_rowwise_amd as lm
    import oracle
    import workloads

    G = args.group
    if wl.K % G:
        raise SystemExit(f"--group {G} does not divide K = {wl.K}")
    lm.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    kernel = product_kernel(wl.M, wl.K, wl.N, G)
    tag = workload_tag(wl, G)
    log(f"workload {tag}: X {wl.M}x{wl.K} {wl.dtype}, W {wl.K}x{wl.N}, groups of {G}; product kernel {kernel}")
    x, w, _, _ = workloads.make_workload(wl.name)
    X, W = x.to(dev), w.to(dev)
    Wq, s_w = lm.int8_quantize_weight_group(W, G)
    del W
    ws = torch.empty(lm.int8_matmul_group_workspace_bytes(wl.M, wl.K, G), dtype=torch.uint8, device=dev)
    Y = torch.empty((wl.M, wl.N), dtype=X.dtype, device=dev)
    torch.cuda.synchronize()
    if args.copy_mib > 0:
        calibration_copy(args.copy_mib, dev, torch)
    stream = torch.cuda.current_stream(dev)

    def step():
        lm.int8_matmul_group(X, Wq, s_w, G, Y=Y, workspace=ws, stream=stream)

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    t_wall = time.perf_counter()
    ms_step = time_loop(step, args.steps, torch)
    t_wall = time.perf_counter() - t_wall
    ops = 2.0 * wl.M * wl.N * wl.K
    tops = ops / (ms_step * 1e-3) / 1e12
    ms_gemm = time_loop(lambda: lm.int8_matmul_group_products(wl.M, wl.K, X.dtype, G, Wq, s_w, ws, Y=Y,
                                                              stream=stream), args.steps, torch)
    ms_xpass = time_loop(lambda: lm.int8_matmul_group_prepare(X, G, ws, stream=stream), args.steps, torch)
    achieved = ops / (ms_gemm * 1e-3) / 1e12
    log(f"step {ms_step * 1e3:.1f} us = {tops:.0f} TOPS; {kernel} {ms_gemm * 1e3:.1f} us = {achieved:.0f} TOPS; "
        f"X pass {ms_xpass * 1e3:.1f} us")
    roof = {"bound": "mfma", "achieved": achieved, "peak": I8_PEAK_TOPS, "unit": "TFLOP/s",
            "frac": achieved / I8_PEAK_TOPS, "traffic": stored_traffic(kernel, tag), "kernel": kernel,
            "kernel_ms": ms_gemm, "xpass_ms": ms_xpass}
    line = {
        "metric": "effective TOPS of int8 matmul with group-wise scales along K; % i8 MFMA peak",
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
        "config": {"workload": tag, "M": wl.M, "K": wl.K, "N": wl.N, "x_dtype": wl.dtype, "group": G, "seed": 0},
        "pct_of_i8_peak": tops / I8_PEAK_TOPS * 100.0,
        "roofline": roof,
        "cpu_baseline": None,
        "wall_s_timed": t_wall,
    }
    if not args.no_cpu_baseline:
        cores = oracle.set_threads(min(int(os.environ.get("OMP_NUM_THREADS") or os.cpu_count()), os.cpu_count()))
        Xb, Wb = workloads.bits(x), workloads.bits(w)
        log(f"cpu baseline: oracle group weight conversion (untimed, offline) on {cores} threads")
        Wq_o, s_w_o = oracle.group_quantize_weight(Wb, wl.dtype, G)
        t0 = time.perf_counter()
        Xq_o, s_x_o = oracle.group_quantize_rows(Xb, wl.dtype, G)
        t_xpass = time.perf_counter() - t0
        probe = np.arange(min(cores, wl.M))
        t0 = time.perf_counter()
        oracle.group_gemm(Xq_o, s_x_o, Wq_o, s_w_o, G, wl.dtype, probe)
        t_probe = time.perf_counter() - t0
        rounds = int(max(1.0, (args.cpu_seconds - t_xpass) / max(t_probe, 1e-9)))
        R = int(min(wl.M, probe.size * rounds))
        t0 = time.perf_counter()
        oracle.group_gemm(Xq_o, s_x_o, Wq_o, s_w_o, G, wl.dtype, np.arange(R))
        t = time.perf_counter() - t0 + t_xpass * R / wl.M
        line["cpu_baseline"] = {
            "value": 2.0 * R * wl.N * wl.K / t / 1e12, "unit": "TOPS", "cores": cores, "kind": "oracle",
            "sample": (f"group X pass over all {wl.M} rows (time prorated to the sample) + group-wise products for "
                       f"rows 0..{R - 1} of {wl.M}; {t:.1f} s of CPU work")}
    print(json.dumps(line), flush=True)
    return 0


# ---------------------------------------------------------------------------------------

def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="qkv_175b")
    ap.add_argument("--cpu-seconds", type=float, default=20.0, help="CPU work budget of the oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fp16-gemm", action="store_true")
    ap.add_argument("--cold", action="store_true", help="also time steps with L2 and the memory-side cache flushed")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="before the steps, run a plain copy-shaped kernel over this many MiB (counter calibration)")
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="summarize two rocprofv3 counter runs into the stored traffic record and exit")
    ap.add_argument("--fixed", action="store_true",
                    help="time the fixed-outlier path (the workload's injected columns as the set) instead")
    ap.add_argument("--group", type=int, default=0, metavar="G",
                    help="time the group-wise path with groups of G features along K instead (no outlier "
                         "decomposition)")
    ap.add_argument("--codec", action="store_true",
                    help="benchmark the block-wise int8 codec instead (its own JSON line)")
    ap.add_argument("--trace-summary", nargs=3, metavar=("TRACE_DIR", "BENCH_OUT", "COMMAND"),
                    help="summarize a rocprofv3 --kernel-trace --stats run of this script and exit")
    args = ap.parse_args()

    import workloads

    wl = workloads.WORKLOADS[args.workload]
    if args.trace_summary:
        return trace_summary(args.trace_summary[0], args.trace_summary[1], wl, args.trace_summary[2], args.group)
    if args.traffic_summary:
        return traffic_summary(args.traffic_summary[0], args.traffic_summary[1], wl, args.copy_mib or 1024,
                               args.group)
    if args.gpus != 1:
        print(f"bench.py: one GPU only; --gpus {args.gpus} is not supported (the library has no multi-GPU "
              f"path: each GPU would run the same kernels on its own column shard)", file=sys.stderr)
        return 2

    if args.codec:
        return codec_bench(args)
    if args.group:
        return group_bench(args, wl)

    import torch

    import int8_quantized_matmul_rowwise_amd as lm

    lm.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    kernel = product_kernel(wl.M, wl.K, wl.N)
    log(f"workload {wl.name}: X {wl.M}x{wl.K} {wl.dtype}, W {wl.K}x{wl.N}, tau {wl.tau}; product kernel {kernel}")
    x, w, cols, _ = workloads.make_workload(wl.name)
    X = x.to(dev)
    W = w.to(dev)
    Wq, s_w = lm.int8_quantize_weight(W)
    ws = torch.empty(lm.int8_matmul_workspace_bytes(wl.M, wl.K, wl.N), dtype=torch.uint8, device=dev)
    Y = torch.empty((wl.M, wl.N), dtype=X.dtype, device=dev)
    torch.cuda.synchronize()

    if args.copy_mib > 0:
        calibration_copy(args.copy_mib, dev, torch)

    if args.fixed:
        # the workload's injected outlier columns, fixed offline: no detection per call
        Ofix = torch.as_tensor(sorted(int(c) for c in cols), dtype=torch.int32, device=dev)
        Wq, s_w, W_O = lm.int8_quantize_weight_fixed(W, Ofix)
        torch.cuda.synchronize()

        def step():
            lm.int8_matmul_fixed(X, Ofix, Wq, s_w, W_O, Y=Y, workspace=ws)
    else:
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
    n_out = len(cols) if args.fixed else lm.int8_matmul_stats(X, wl.tau)[0]
    ops = 2.0 * wl.M * wl.N * wl.K
    tops = ops / (ms_step * 1e-3) / 1e12

    # The dominant kernel alone: the product launch (products + outlier product + epilogue)
    # back to back on a prepared workspace, HIP events around the loop on the stream it runs on.
    stream = torch.cuda.current_stream(dev)
    lm.int8_matmul_prepare(X, Wq, wl.tau, workspace=ws, stream=stream)
    for _ in range(3):
        lm.int8_matmul_products(wl.M, wl.K, X.dtype, Wq, s_w, ws, Y=Y, stream=stream)
    ms_gemm = time_loop(lambda: lm.int8_matmul_products(wl.M, wl.K, X.dtype, Wq, s_w, ws, Y=Y, stream=stream),
                        args.steps, torch)
    ms_xpass = time_loop(lambda: lm.int8_matmul_prepare(X, Wq, wl.tau, workspace=ws, stream=stream), args.steps, torch)
    if args.fixed:
        ms_xpass = ms_step - ms_gemm  # the fixed X pass (list bitmap, compaction, row coding) is the rest of a step
    cold = None
    if args.cold:
        # every step after a 512 MiB write that evicts L2 and the memory-side cache
        flush = torch.empty(512 * 1024 * 1024 // 4, dtype=torch.int32, device=dev)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        for s, e in evs:
            flush.add_(1)
            s.record(stream)
            step()
            e.record(stream)
        torch.cuda.synchronize()
        cold = sum(s.elapsed_time(e) for s, e in evs) / len(evs)
        log(f"cold step (caches flushed before each): {cold * 1e3:.1f} us")
        del flush
    if kernel == "gemm_kernel":
        achieved = ops / (ms_gemm * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": I8_PEAK_TOPS, "unit": "TFLOP/s",
                "frac": achieved / I8_PEAK_TOPS}
        log(f"step {ms_step * 1e3:.1f} us = {tops:.0f} TOPS; {kernel} {ms_gemm * 1e3:.1f} us = {achieved:.0f} TOPS;"
            f" X pass {ms_xpass * 1e3:.1f} us; n_outliers {n_out}")
    else:
        alg_bytes = algorithmic_bytes(wl)
        achieved = alg_bytes / (ms_gemm * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS}
        log(f"step {ms_step * 1e3:.1f} us = {tops:.1f} TOPS; {kernel} {ms_gemm * 1e3:.1f} us = {achieved:.0f} GB/s;"
            f" X pass {ms_xpass * 1e3:.1f} us; n_outliers {n_out}")
    roof["traffic"] = stored_traffic(kernel, wl.name)
    roof.update({"kernel": kernel, "kernel_ms": ms_gemm, "xpass_ms": ms_xpass})
    if cold is not None:
        roof["cold_ms_per_step"] = cold

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
                   "threshold": None if args.fixed else wl.tau, "n_outliers": n_out, "seed": 0,
                   **({"outliers": "fixed (caller-supplied)"} if args.fixed else {})},
        "pct_of_i8_peak": tops / I8_PEAK_TOPS * 100.0,
        "roofline": roof,
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
