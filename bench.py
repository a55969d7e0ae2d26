#!/usr/bin/env python3
"""Benchmark of the LLM.int8() matmul on one MI355X.

A step is one int8_matmul on resident inputs: the X pass (outlier columns, row scales,
int8 codes, outlier gather) and the products with the dequantizing epilogue, issued as
the two stages int8_matmul runs (int8_matmul_prepare, then int8_matmul_products) with a
HIP event between them (created without the system-scope fence, which would hold the next
kernel back by about 3 us).  The weight conversion is offline and not timed.  Default
workload: the 175B-like QKV projection, X 4096 x 12288 fp16 (7 outlier feature
dimensions), W 12288 x 36864.

Caches: the headline is cold.  Before every step (warmup and timed) 512 MiB are written
and then 512 MiB of a second buffer are read: no byte of the step's operands is left in L2
or the 256 MB memory-side cache, and no dirty line of the flush is left there either (a
write-only flush leaves up to 256 MB of dirty lines, whose write-back would share HBM with
the step's reads: a plain read of the 453 MB QKV weight takes about 140 us after a
write-only flush and about 85 us after this one, as long as warm).  Each step is timed by
its own events, so the flush is outside the step's time.  Warm steps (back to back) are
reported beside.

Printed: one JSON line with
  value            effective TOPS of the cold step, 2*M*N*K / step time
  pct_of_i8_peak   value / 5000 TOPS (MI355X dense int8 MFMA)
  roofline         the dominant kernel (the product kernel, which also runs the outlier
                   product and the epilogue): the algorithmic work per launch -- 2*M*N*K
                   ops for the tiled kernel (bound "mfma", unit TOPS), or the Wq + Xq + Y
                   bytes for the small-batch kernel (bound "hbm") -- over its average
                   duration inside the timed cold steps (HIP events on the library's
                   stream around its launch).  traffic = HBM bytes per launch from
                   rocprofv3 FETCH_SIZE and WRITE_SIZE scaled by a copy calibration;
                   clock_mhz and mfma_busy from GRBM_GUI_ACTIVE and
                   SQ_VALU_MFMA_BUSY_CYCLES -- each from its committed record under
                   profiles/ when that was measured on the current kernel source (else null)
  warm             the step back to back, one int8_matmul per step (caches warm), and the
                   product kernel and the X pass each back to back
  ceilings         measured on this machine in this run: the int8 MFMA rate and shader clock
                   of a register-only MFMA loop (zero operands, and random operands that
                   change from one MFMA to the next), the HBM stream-read rate (2 GiB,
                   back to back), and a plain read of as many bytes as the weight after
                   the same flush as the cold steps
  cpu_baseline     the CPU oracle on a bounded sample of the same workload, with the host's
                   core count and CPU model
  fp16_gemm        torch.matmul (hipBLASLt) of X and W in the 16-bit type, same shape
Progress goes to stderr.

Other modes, each with its own JSON line of the same shape:
  --fixed          the fixed-outlier path (the workload's injected columns as the set)
  --group G        the group-wise path, groups of G features along K (no outlier split)
  --codec          the block-wise absmax int8 codec on a 2^28-element fp32 state (GB/s)
  --gpus N         N > 1 exits with a message: the library runs on one GPU

Counter records (one rocprofv3 run per counter set, then on any host):
  rocprofv3 --pmc FETCH_SIZE --output-format csv -d DIR_F -o run -- \\
      python3 bench.py --steps 3 --warmup 1 --no-cpu-baseline --no-fp16-gemm --no-warm --copy-mib 1024
  (the same with WRITE_SIZE into DIR_W), then
  python3 bench.py --traffic-summary DIR_F DIR_W [--workload NAME] [--group G]
which writes profiles/<kernel>_traffic_<workload>.json and .md; and
  rocprofv3 --kernel-trace --pmc GRBM_GUI_ACTIVE SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_I8 \\
      --output-format csv -d DIR_C -o run -- python3 bench.py --steps 3 --warmup 1 ... --no-warm
  python3 bench.py --counter-summary DIR_C [--workload NAME] [--group G]
which writes profiles/<kernel>_counters_<workload>.json and .md (clock under load, MFMA busy).
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

I8_PEAK_TOPS = 5000.0
HBM_PEAK_GBS = 8000.0
FLUSH_MIB = 512
CSRC = "int8_quantized_matmul_rowwise_amd/csrc/"
# the product kernel of each path and the sources it is built from
KERNELS = {
    "gemm_kernel": [CSRC + "gemm.hip", CSRC + "common.hpp"],
    "gemm_small_kernel": [CSRC + "gemm_small.hip", CSRC + "common.hpp"],
    "gemm_group_kernel": [CSRC + "gemm_group.hip", CSRC + "common.hpp"],
    "gemm_group_small_kernel": [CSRC + "gemm_group_small.hip", CSRC + "common.hpp"],
}
HBM_BOUND = {"gemm_small_kernel", "gemm_group_small_kernel"}


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def product_kernel(M: int, K: int, N: int, group: int = 0) -> str:
    """The product kernel the library runs for these sizes (the library reports its own choice)."""
    import int8_quantized_matmul_rowwise_amd as lm
    if group:
        return "gemm_group_small_kernel" if lm.int8_matmul_group_small_batch(M, K, N, group) else "gemm_group_kernel"
    return "gemm_small_kernel" if lm.int8_matmul_workspace_layout(M, K, N)["small_batch"] else "gemm_kernel"


def workload_args(wl, group: int = 0) -> str:
    """The bench.py arguments that select the configuration wl (and group) names."""
    import re

    import workloads
    base, rows = wl.name, None
    m = re.match(r"(.+)_m(\d+)$", wl.name)
    if m and m.group(1) in workloads.WORKLOADS:
        base, rows = m.group(1), int(m.group(2))
    return f"--workload {base}" + (f" --rows {rows}" if rows else "") + (f" --group {group}" if group else "")


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


def record_path(kernel: str, what: str, workload: str, ext: str) -> str:
    return os.path.join(ROOT, "profiles", f"{kernel}_{what}_{workload}.{ext}")


def stored_record(kernel: str, what: str, workload: str):
    """A committed counter record of the product kernel, if it was taken on the current kernel source."""
    path = record_path(kernel, what, workload, "json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256") != kernel_source_hash(kernel):
        log(f"stored {what} record for {kernel} was measured on another kernel source: not used")
        return None
    return rec


def roofline(kernel: str, wl, tag: str, kernel_ms: float, group: int = 0) -> dict:
    if kernel in HBM_BOUND:
        achieved = algorithmic_bytes(wl, group) / (kernel_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS}
    else:
        achieved = 2.0 * wl.M * wl.N * wl.K / (kernel_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": I8_PEAK_TOPS, "unit": "TOPS",
                "frac": achieved / I8_PEAK_TOPS}
    tr = stored_record(kernel, "traffic", tag)
    ct = stored_record(kernel, "counters", tag)
    roof["traffic"] = tr["hbm_bytes_per_launch"] if tr else None
    roof["clock_mhz"] = ct["clock_mhz"] if ct else None
    roof["mfma_busy"] = ct["mfma_busy"] if ct else None
    roof["kernel"] = kernel
    roof["kernel_ms"] = kernel_ms
    return roof


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


class HipEvent:
    """A timing event recorded without the system-scope fence: HIP's default event record
    releases to system scope, which delays the next kernel on the stream by about 3 us (an
    event between the X pass and the products of a decode step added that much to the
    step); without the fence the stage events cost nothing measurable."""
    DISABLE_SYSTEM_FENCE = 0x20000000
    _hip = None

    def __init__(self):
        import ctypes
        if HipEvent._hip is None:
            h = ctypes.CDLL("libamdhip64.so")
            h.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            h.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            h.hipEventDestroy.argtypes = [ctypes.c_void_p]
            HipEvent._hip = h
        self._ct = ctypes
        self.ev = ctypes.c_void_p()
        if HipEvent._hip.hipEventCreateWithFlags(ctypes.byref(self.ev), self.DISABLE_SYSTEM_FENCE):
            raise RuntimeError("hipEventCreateWithFlags failed")

    def record(self, stream):
        if HipEvent._hip.hipEventRecord(self.ev, self._ct.c_void_p(int(stream.cuda_stream))):
            raise RuntimeError("hipEventRecord failed")

    def elapsed_time(self, end) -> float:
        ms = self._ct.c_float()
        if HipEvent._hip.hipEventElapsedTime(self._ct.byref(ms), self.ev, end.ev):
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def __del__(self):
        if HipEvent._hip is not None and self.ev:
            HipEvent._hip.hipEventDestroy(self.ev)


def timed_steps(stages, steps: int, warmup: int, torch, stream, flush=None):
    """Run warmup + `steps` steps, each the callables in `stages` in order, with an event on
    `stream` before, between and after them (HipEvent: no system fence); flush (if given)
    runs before every step, outside its events.  Returns (mean ms of the whole step, mean
    ms of each stage, wall s of the timed steps)."""
    def run(evs):
        if flush is not None:
            flush()
        for i, f in enumerate(stages):
            if evs:
                evs[i].record(stream)
            f()
        if evs:
            evs[-1].record(stream)

    for _ in range(warmup):
        run(None)
    torch.cuda.synchronize()
    evs = [[HipEvent() for _ in range(len(stages) + 1)] for _ in range(steps)]
    t0 = time.perf_counter()
    for ev in evs:
        run(ev)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    whole = sum(ev[0].elapsed_time(ev[-1]) for ev in evs) / steps
    parts = [sum(ev[i].elapsed_time(ev[i + 1]) for ev in evs) / steps for i in range(len(stages))]
    return whole, parts, wall


def make_flush(dev, torch):
    """The cold-step flush: FLUSH_MIB MiB written (an in-place add), then FLUSH_MIB MiB of a
    second buffer read (a sum), which leaves clean lines of that buffer in the caches."""
    n = FLUSH_MIB * 1024 * 1024 // 4
    wr = torch.empty(n, dtype=torch.int32, device=dev)
    rd = torch.zeros(n, dtype=torch.float32, device=dev)
    sink = torch.empty((), dtype=torch.float32, device=dev)

    def flush():
        wr.add_(1)
        torch.sum(rd, dim=0, out=sink)
    return (wr, rd, sink), flush


# ---------------------------------------------------------------------------------------
# host and device facts

def host_facts() -> dict:
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count()
    model = platform.processor() or ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"nproc": affinity, "cpu_count": os.cpu_count(), "cpu_model": model}


def oracle_threads() -> int:
    """All the host cores this process may use, capped by OMP_NUM_THREADS when it is set (the
    CPU share of a one-GPU machine)."""
    n = host_facts()["nproc"]
    env = os.environ.get("OMP_NUM_THREADS")
    return min(int(env), n) if env else n


def measured_ceilings(dev, torch, cold_bytes: int = 0) -> dict:
    """The int8 MFMA rate and shader clock of a register-only MFMA loop (zero and changing
    random operands) and the HBM stream-read rate, measured now on this device; with
    cold_bytes, also a plain read of that many bytes after the cold-step flush."""
    import ctypes

    import numpy as np

    from int8_quantized_matmul_rowwise_amd import build
    if not os.path.exists(build.PROBE_LIB):
        log("probe library missing (build it): no measured ceilings")
        return None
    P = ctypes.CDLL(build.PROBE_LIB)
    P.llmint8_probe_mfma_i8.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_void_p]
    P.llmint8_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p,
                                            ctypes.c_void_p]
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    stream = torch.cuda.current_stream(dev)
    sp = int(stream.cuda_stream)
    out = torch.empty(cus * 512, dtype=torch.int32, device=dev)
    clk = torch.empty(cus * 4, dtype=torch.int64, device=dev)
    iters = 20000
    res = {"cus": cus}
    for mode, name in ((1, "random_operands"), (0, "zero_operands")):
        rc = P.llmint8_probe_mfma_i8(cus, iters, mode, out.data_ptr(), clk.data_ptr(), sp)
        if rc:
            raise RuntimeError(f"mfma probe launch failed ({rc})")
        ms = time_loop(lambda: P.llmint8_probe_mfma_i8(cus, iters, mode, out.data_ptr(), clk.data_ptr(), sp), 3,
                       torch)
        c = clk.view(-1, 4).cpu().numpy().astype(np.float64)
        mhz = float(np.median((c[:, 1] - c[:, 0]) / np.maximum(c[:, 3] - c[:, 2], 1) * 100.0))
        tops = cus * 8 * iters * 8 * 65536 / (ms * 1e-3) / 1e12
        res[f"i8_mfma_tops_{name}"] = tops
        res[f"clock_mhz_{name}"] = mhz
        log(f"MFMA probe ({name}): {tops:.0f} TOPS at {mhz:.0f} MHz shader clock")
    del out, clk
    nbytes = 2 << 30
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
    grid = cus * 8
    part = torch.empty(grid * 256, dtype=torch.int32, device=dev)
    fn = lambda: P.llmint8_probe_stream_read(buf.data_ptr(), nbytes, grid, part.data_ptr(), sp)
    fn()
    ms = time_loop(fn, 10, torch)
    res["stream_read_gbs"] = nbytes / (ms * 1e-3) / 1e9
    log(f"stream read: {res['stream_read_gbs']:.0f} GB/s")
    del buf
    if cold_bytes > 0:
        nb = (cold_bytes + 15) // 16 * 16
        buf = torch.ones(nb // 4, dtype=torch.int32, device=dev)
        fbuf, flush = make_flush(dev, torch)
        st = torch.cuda.current_stream(dev)
        fn = lambda: P.llmint8_probe_stream_read(buf.data_ptr(), nb, grid, part.data_ptr(), sp)
        _, (ms_c,), _ = timed_steps([fn], 7, 2, torch, st, flush)
        res["cold_read_bytes"] = nb
        res["cold_read_us"] = ms_c * 1e3
        res["cold_read_gbs"] = nb / (ms_c * 1e-3) / 1e9
        log(f"plain read of {nb / 1e6:.1f} MB after the flush: {ms_c * 1e3:.1f} us = {res['cold_read_gbs']:.0f} GB/s")
        del buf, fbuf
    del part
    torch.cuda.empty_cache()
    return res


# ---------------------------------------------------------------------------------------
# CPU baseline

def cpu_baseline(x, w, wl, seconds: float) -> dict:
    import numpy as np

    import oracle
    import workloads

    cores = oracle.set_threads(oracle_threads())
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
    hf = host_facts()
    return {
        "value": 2.0 * R * wl.N * wl.K / t / 1e12,
        "unit": "TOPS",
        "cores": cores,
        "kind": "oracle",
        "sample": sample,
        "nproc": hf["nproc"],
        "cpu_model": hf["cpu_model"],
    }


# ---------------------------------------------------------------------------------------
# counter summaries (host only)

def _counter_rows(d: str):
    files = sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True))
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    rows = []
    for f in files:
        with open(f, newline="") as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def _per_dispatch(rows, counter: str, match) -> dict:
    """Counter value of each dispatch whose kernel name satisfies match, keyed by dispatch."""
    vals = {}
    for r in rows:
        if r["Counter_Name"] == counter and match(r["Kernel_Name"]):
            key = (r.get("Process_Id"), r["Dispatch_Id"])
            vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
    return vals


def traffic_summary(fetch_dir: str, write_dir: str, wl, copy_mib: int, group: int = 0) -> int:
    kernel = product_kernel(wl.M, wl.K, wl.N, group)
    tag = workload_tag(wl, group)
    copy_bytes = copy_mib * 1024 * 1024
    is_copy = lambda name: "elementwise_kernel" in name  # the calibration copy (torch add of 1 GiB)
    is_prod = lambda name: f"::{kernel}<" in name
    out = {"kernel": kernel, "workload": tag, "kernel_source_sha256": kernel_source_hash(kernel),
           "copy_calibration_bytes": copy_bytes}
    lines = [f"# {kernel} HBM traffic, workload {tag} ({wl.M}x{wl.K}x{wl.N} {wl.dtype})", ""]
    total = 0.0
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = _counter_rows(d)
        copies = list(_per_dispatch(rows, counter, is_copy).values())
        names = sorted({r["Kernel_Name"] for r in rows if is_copy(r["Kernel_Name"])})
        lines.append(f"- calibration kernel(s) for {counter}: " + "; ".join(n[:120] for n in names))
        prods = list(_per_dispatch(rows, counter, is_prod).values())
        if not copies or not prods:
            raise SystemExit(f"{counter}: {len(copies)} copy and {len(prods)} product dispatches found in {d}")
        # the calibration copy is the first elementwise dispatch group (the cache flushes of
        # the cold steps are elementwise too, but 512 MiB): take those of the copy's size
        copy_kib = max(copies)
        copies = [c for c in copies if c > 0.75 * copy_kib]
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
              f"{workload_args(wl, group)} --steps 3 --warmup 1 --no-cpu-baseline --no-fp16-gemm --no-warm "
              f"--no-ceilings --copy-mib {copy_mib}",
              f"    rocprofv3 --pmc WRITE_SIZE --output-format csv -d {write_dir} -o run -- python3 bench.py "
              f"{workload_args(wl, group)} --steps 3 --warmup 1 --no-cpu-baseline --no-fp16-gemm --no-warm "
              f"--no-ceilings --copy-mib {copy_mib}",
              f"    python3 bench.py --traffic-summary {fetch_dir} {write_dir} {workload_args(wl, group)} "
              f"--copy-mib {copy_mib}", ""]
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(record_path(kernel, "traffic", tag, "json"), "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    with open(record_path(kernel, "traffic", tag, "md"), "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))
    return 0


def _durations(rows, match) -> dict:
    """Duration (ns) of each dispatch of a matching kernel, from the counter rows' timestamps."""
    out = {}
    for r in rows:
        if match(r["Kernel_Name"]) and r.get("Start_Timestamp") and r.get("End_Timestamp"):
            out[(r.get("Process_Id"), r["Dispatch_Id"])] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
    return out


def counter_summary(d: str, wl, group: int = 0) -> int:
    """Clock under load and MFMA busy fraction of the product kernel from one rocprofv3 run
    with --kernel-trace and --pmc GRBM_GUI_ACTIVE SQ_VALU_MFMA_BUSY_CYCLES (+ MFMA op counts)."""
    kernel = product_kernel(wl.M, wl.K, wl.N, group)
    tag = workload_tag(wl, group)
    is_prod = lambda name: f"::{kernel}<" in name
    rows = _counter_rows(d)
    dur = _durations(rows, is_prod)
    counters = sorted({r["Counter_Name"] for r in rows})
    per = {c: _per_dispatch(rows, c, is_prod) for c in counters}
    keys = sorted(set(per.get("GRBM_GUI_ACTIVE", {})) & set(dur))
    if not keys:
        raise SystemExit(f"no {kernel} dispatch with both GRBM_GUI_ACTIVE and timestamps under {d}")
    import torch
    xcds = 8
    simds = 4 * (torch.cuda.get_device_properties(0).multi_processor_count if torch.cuda.is_available() else 256)
    mean = lambda c: sum(per[c][k] for k in keys) / len(keys)
    ns = sum(dur[k] for k in keys) / len(keys)
    cycles = mean("GRBM_GUI_ACTIVE") / xcds  # the counter is summed over the XCDs
    out = {"kernel": kernel, "workload": tag, "kernel_source_sha256": kernel_source_hash(kernel),
           "dispatches": len(keys), "duration_ns": ns, "grbm_gui_active_per_xcd": cycles,
           "clock_mhz": cycles / ns * 1e3}
    lines = [f"# {kernel} clock and MFMA activity, workload {tag} ({wl.M}x{wl.K}x{wl.N} {wl.dtype})", "",
             f"Per dispatch, averaged over {len(keys)} dispatches of the product kernel:", "",
             "| quantity | value |", "|---|---|",
             f"| duration (kernel trace) | {ns / 1e3:.1f} us |",
             f"| GRBM_GUI_ACTIVE per XCD (sum / 8) | {cycles:.4g} cycles |",
             f"| clock under this kernel (cycles / duration) | {out['clock_mhz']:.0f} MHz |"]
    if "SQ_VALU_MFMA_BUSY_CYCLES" in per:
        busy = mean("SQ_VALU_MFMA_BUSY_CYCLES") / simds
        out["mfma_busy_cycles_per_simd"] = busy
        out["mfma_busy"] = busy / cycles
        lines.append(f"| SQ_VALU_MFMA_BUSY_CYCLES per SIMD (sum / {simds}) | {busy:.4g} cycles |")
        lines.append(f"| matrix units busy (busy / active cycles) | {out['mfma_busy'] * 100:.1f} % |")
        if not kernel.endswith("small_kernel"):
            peak_at_clock = 8192 * simds / 4 * out["clock_mhz"] * 1e6 / 1e12
            out["i8_peak_tops_at_clock"] = peak_at_clock
            lines.append(f"| int8 peak at that clock (8192 ops/clk/CU) | {peak_at_clock:.0f} TOPS |")
    if "SQ_INSTS_VALU_MFMA_MOPS_I8" in per:
        ops = mean("SQ_INSTS_VALU_MFMA_MOPS_I8") * 512
        out["i8_mfma_ops"] = ops
        lines.append(f"| int8 MFMA ops (SQ_INSTS_VALU_MFMA_MOPS_I8 x 512) | {ops:.6g} (2MNK = "
                     f"{2.0 * wl.M * wl.N * wl.K:.6g}) |")
    tops = 2.0 * wl.M * wl.N * wl.K / ns * 1e-3
    lines.append(f"| effective rate over the traced duration | {tops:.0f} TOPS |")
    lines += ["", "Command (repository root on the GPU box, then on any host):", "",
              "    cd /tmp && export TMPDIR=/tmp; cd -",
              f"    rocprofv3 --kernel-trace --pmc {' '.join(counters)} --output-format csv -d {d} -o run -- "
              f"python3 bench.py {workload_args(wl, group)} --steps 3 --warmup 1 --no-cpu-baseline --no-fp16-gemm "
              f"--no-warm --no-ceilings",
              f"    python3 bench.py --counter-summary {d} {workload_args(wl, group)}", ""]
    with open(record_path(kernel, "counters", tag, "json"), "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    with open(record_path(kernel, "counters", tag, "md"), "w") as f:
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
        roof = line["roofline"]
        lines += ["", f"bench line of the same run: step {line['ms_per_step'] * 1e3:.1f} us, {kernel} "
                  f"{ms * 1e3:.1f} us per launch inside the step (HIP events), value {line['value']:.1f} "
                  f"{line['unit']}, roofline achieved {roof['achieved']:.1f} {roof['unit']} (frac {roof['frac']:.4f})"]
        # the timed steps' dispatches: the last `steps` of the product kernel in the per-dispatch
        # trace of a --no-warm run (the warmup steps before them include the part's clock
        # settling under load; with warm steps the last dispatches would be theirs)
        timed = None
        traces = sorted(glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True))
        if traces:
            with open(traces[0], newline="") as fh:
                durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in csv.DictReader(fh)
                        if f"::{kernel}<" in r["Kernel_Name"]]
            if len(durs) >= line["steps"]:
                timed = durs[-line["steps"]:]
                lines.append(f"trace of {kernel}, the {len(durs)} dispatches in order (us): "
                             + ", ".join(f"{d:.1f}" for d in durs))
        if avg_prod:
            def frac_of(us):
                if roof["bound"] == "mfma":
                    return 2.0 * wl.M * wl.N * wl.K / (us * 1e-6) / 1e12 / roof["peak"]
                return algorithmic_bytes(wl, group) / (us * 1e-6) / 1e9 / roof["peak"]
            lines.append(f"trace average of {kernel} over all its dispatches: {avg_prod:.1f} us "
                         f"({(avg_prod / (ms * 1e3) - 1) * 100:+.1f} % vs the events): roofline frac {frac_of(avg_prod):.4f}")
            if timed:
                avg_t = sum(timed) / len(timed)
                lines.append(f"trace average of {kernel} over the {len(timed)} timed steps' dispatches: {avg_t:.1f} us "
                             f"({(avg_t / (ms * 1e3) - 1) * 100:+.1f} % vs the events): roofline frac {frac_of(avg_t):.4f}")
            if avg_prod < 0.95 * ms * 1e3:
                lines.append("(the events bracket the product stage from the end of the X pass: under the profiler "
                             "the dispatch gap before the kernel, which lands inside that bracket, grows by a few "
                             "us, a large share of a short kernel; without the profiler the two agree more closely)")
    lines += ["", "Command (repository root on the GPU box):", "", "    " + cmd, ""]
    out = os.path.join(ROOT, "profiles", f"kernel_trace_{tag}.md")
    with open(out, "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))
    return 0


# ---------------------------------------------------------------------------------------
# the next rows

def codec_bench(args) -> int:
    """The block-wise absmax int8 codec on a 2^28-element fp32 optimizer state (blocks of
    2048): quantize and dequantize timed back to back (HIP events on the current stream),
    algorithmic bytes 4n + n + 4 n/block (quantize) and n + 4n + 4 n/block (dequantize).
    The state (1 GiB) is four times the memory-side cache, so every pass streams from HBM."""
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
    cores = oracle.set_threads(oracle_threads())
    xs = x[: 1 << 24].numpy()
    t0 = time.perf_counter()
    reps = 0
    while time.perf_counter() - t0 < args.cpu_seconds / 2 or reps == 0:
        qs, as_ = oracle.block_quantize(xs, block)
        oracle.block_dequantize(qs, as_, block)
        reps += 1
    t_cpu = (time.perf_counter() - t0) / reps
    hf = host_facts()
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
                         "sample": f"quantize + dequantize of the first 2^24 elements, {reps} times",
                         "nproc": hf["nproc"], "cpu_model": hf["cpu_model"]},
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
    decomposition) on the workload's shape: a step is one int8_matmul_group, issued as its
    two stages (X pass, products) with an event between them, caches cold like the headline."""
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
    x, w, _, _ = workloads.make_workload(args.workload, rows=args.rows)
    X, W = x.to(dev), w.to(dev)
    Wq, s_w = lm.int8_quantize_weight_group(W, G)
    del W
    ws = torch.empty(lm.int8_matmul_group_workspace_bytes(wl.M, wl.K, G), dtype=torch.uint8, device=dev)
    Y = torch.empty((wl.M, wl.N), dtype=X.dtype, device=dev)
    torch.cuda.synchronize()
    if args.copy_mib > 0:
        calibration_copy(args.copy_mib, dev, torch)
    stream = torch.cuda.current_stream(dev)
    stages = [lambda: lm.int8_matmul_group_prepare(X, G, ws, stream=stream),
              lambda: lm.int8_matmul_group_products(wl.M, wl.K, X.dtype, G, Wq, s_w, ws, Y=Y, stream=stream)]
    flush_buf, flush = make_flush(dev, torch)
    log(f"cold: warmup {args.warmup} steps, timing {args.steps} steps")
    ms_step, (ms_xpass, ms_gemm), t_wall = timed_steps(stages, args.steps, args.warmup, torch, stream, flush)
    del flush_buf
    ops = 2.0 * wl.M * wl.N * wl.K
    tops = ops / (ms_step * 1e-3) / 1e12
    log(f"step {ms_step * 1e3:.1f} us = {tops:.0f} TOPS; {kernel} {ms_gemm * 1e3:.1f} us; X pass {ms_xpass * 1e3:.1f} us")
    roof = roofline(kernel, wl, tag, ms_gemm, G)
    roof["xpass_ms"] = ms_xpass
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
        "config": {"workload": tag, "M": wl.M, "K": wl.K, "N": wl.N, "x_dtype": wl.dtype, "group": G, "seed": 0,
                   "caches": f"cold ({FLUSH_MIB} MiB written, then {FLUSH_MIB} MiB of another buffer read, before each step)"},
        "pct_of_i8_peak": tops / I8_PEAK_TOPS * 100.0,
        "roofline": roof,
        "cpu_baseline": None,
        "wall_s_timed": t_wall,
    }
    if not args.no_warm:
        one = lambda: lm.int8_matmul_group(X, Wq, s_w, G, Y=Y, workspace=ws, stream=stream)
        for _ in range(3):
            one()
        w_step = time_loop(one, args.steps, torch)
        w_g = time_loop(stages[1], args.steps, torch)
        w_x = time_loop(stages[0], args.steps, torch)
        line["warm"] = {"ms_per_step": w_step, "value": ops / (w_step * 1e-3) / 1e12, "kernel_ms": w_g,
                        "xpass_ms": w_x}
        log(f"warm step {w_step * 1e3:.1f} us; {kernel} {w_g * 1e3:.1f} us, X pass {w_x * 1e3:.1f} us (back to back)")
    if not args.no_cpu_baseline:
        cores = oracle.set_threads(oracle_threads())
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
        hf = host_facts()
        line["cpu_baseline"] = {
            "value": 2.0 * R * wl.N * wl.K / t / 1e12, "unit": "TOPS", "cores": cores, "kind": "oracle",
            "sample": (f"group X pass over all {wl.M} rows (time prorated to the sample) + group-wise products for "
                       f"rows 0..{R - 1} of {wl.M}; {t:.1f} s of CPU work"),
            "nproc": hf["nproc"], "cpu_model": hf["cpu_model"]}
    print(json.dumps(line), flush=True)
    return 0


# ---------------------------------------------------------------------------------------

def vector_bench(args, wl) -> int:
    """The LLM.int8() matmul (the headline), or with --fixed its fixed-outlier-set variant."""
    import torch

    import int8_quantized_matmul_rowwise_amd as lm

    lm.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    kernel = product_kernel(wl.M, wl.K, wl.N)
    log(f"workload {wl.name}: X {wl.M}x{wl.K} {wl.dtype}, W {wl.K}x{wl.N}, tau {wl.tau}; product kernel {kernel}")
    import workloads
    x, w, cols, _ = workloads.make_workload(args.workload, rows=args.rows)
    X = x.to(dev)
    W = w.to(dev)
    Wq, s_w = lm.int8_quantize_weight(W)
    ws = torch.empty(lm.int8_matmul_workspace_bytes(wl.M, wl.K, wl.N), dtype=torch.uint8, device=dev)
    Y = torch.empty((wl.M, wl.N), dtype=X.dtype, device=dev)
    torch.cuda.synchronize()
    if args.copy_mib > 0:
        calibration_copy(args.copy_mib, dev, torch)
    stream = torch.cuda.current_stream(dev)

    if args.fixed:
        # the workload's injected outlier columns, fixed offline: no detection per call.  The
        # fixed path has one entry point: the step is one call, and the product kernel's time
        # is taken from back-to-back launches on its prepared workspace.
        Ofix = torch.as_tensor(sorted(int(c) for c in cols), dtype=torch.int32, device=dev)
        Wq, s_w, W_O = lm.int8_quantize_weight_fixed(W, Ofix)
        torch.cuda.synchronize()
        stages = [lambda: lm.int8_matmul_fixed(X, Ofix, Wq, s_w, W_O, Y=Y, workspace=ws, stream=stream)]
    else:
        stages = [lambda: lm.int8_matmul_prepare(X, Wq, wl.tau, workspace=ws, stream=stream),
                  lambda: lm.int8_matmul_products(wl.M, wl.K, X.dtype, Wq, s_w, ws, Y=Y, stream=stream)]

    flush_buf, flush = make_flush(dev, torch)
    log(f"cold steps ({FLUSH_MIB} MiB written, {FLUSH_MIB} MiB read before each): warmup {args.warmup}, "
        f"timing {args.steps}")
    ms_step, parts, t_wall = timed_steps(stages, args.steps, args.warmup, torch, stream, flush)
    del flush_buf
    torch.cuda.empty_cache()
    if args.fixed:
        ms_gemm = time_loop(lambda: lm.int8_matmul_products(wl.M, wl.K, X.dtype, Wq, s_w, ws, Y=Y, stream=stream),
                            args.steps, torch)  # not valid for the fixed set's W_O: time only
        ms_xpass = ms_step - ms_gemm
    else:
        ms_xpass, ms_gemm = parts
    n_out = len(cols) if args.fixed else lm.int8_matmul_stats(X, wl.tau)[0]
    ops = 2.0 * wl.M * wl.N * wl.K
    tops = ops / (ms_step * 1e-3) / 1e12
    roof = roofline(kernel, wl, wl.name, ms_gemm)
    roof["xpass_ms"] = ms_xpass
    where, rest = ("back to back", "the rest of the step") if args.fixed else ("in the step", "X pass")
    log(f"cold step {ms_step * 1e3:.1f} us = {tops:.0f} TOPS; {kernel} {ms_gemm * 1e3:.1f} us {where} = "
        f"{roof['achieved']:.0f} {roof['unit']}; {rest} {ms_xpass * 1e3:.1f} us; n_outliers {n_out}")

    warm = None
    if not args.no_warm:
        # back to back, one call per step and events only around the loop, so that the host's
        # per-call cost hides behind the GPU (small workloads); the product kernel alone, back
        # to back on the prepared workspace
        if args.fixed:
            one = stages[0]
        else:
            one = lambda: lm.int8_matmul(X, Wq, s_w, wl.tau, Y=Y, workspace=ws, stream=stream)
        for _ in range(3):
            one()
        w_step = time_loop(one, args.steps, torch)
        warm = {"ms_per_step": w_step, "value": ops / (w_step * 1e-3) / 1e12}
        if not args.fixed:
            warm["kernel_ms"] = time_loop(stages[1], args.steps, torch)
            warm["xpass_ms"] = time_loop(stages[0], args.steps, torch)
        log(f"warm step {w_step * 1e3:.1f} us = {warm['value']:.0f} TOPS" +
            (f"; {kernel} {warm['kernel_ms'] * 1e3:.1f} us, X pass {warm['xpass_ms'] * 1e3:.1f} us (each back to back)"
             if not args.fixed else ""))

    fp16 = None
    if not args.no_fp16_gemm:
        for _ in range(3):
            torch.matmul(X, W)
        ms16 = time_loop(lambda: torch.matmul(X, W), max(5, args.steps // 2), torch)
        fp16 = {"ms": ms16, "tflops": ops / (ms16 * 1e-3) / 1e12,
                "pct_of_peak": ops / (ms16 * 1e-3) / 1e12 / 2500.0 * 100.0,
                "what": f"torch.matmul (hipBLASLt) {wl.dtype} X @ W at the same shape, warm"}
        log(f"fp16 GEMM {ms16 * 1e3:.1f} us = {fp16['tflops']:.0f} TFLOP/s")
    del W
    torch.cuda.empty_cache()
    ceilings = None if args.no_ceilings else measured_ceilings(dev, torch, cold_bytes=wl.N * wl.K)
    if ceilings and roof["bound"] == "hbm" and ceilings.get("cold_read_gbs"):
        # the product kernel's byte rate against a plain read of the weight in the same state
        roof["frac_of_cold_read"] = roof["achieved"] / ceilings["cold_read_gbs"]
    if ceilings and roof["bound"] == "mfma" and ceilings.get("i8_mfma_tops_random_operands"):
        # the product kernel's rate against this part's own int8 MFMA rate on changing
        # operands (its power limit), measured in the same run: boxes differ in that ceiling
        roof["frac_of_random_operand_mfma"] = roof["achieved"] / ceilings["i8_mfma_tops_random_operands"]

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
                   "caches": f"cold ({FLUSH_MIB} MiB written, then {FLUSH_MIB} MiB of another buffer read, before each step)",
                   **({"outliers": "fixed (caller-supplied)"} if args.fixed else {})},
        "pct_of_i8_peak": tops / I8_PEAK_TOPS * 100.0,
        "roofline": roof,
        "warm": warm,
        "ceilings": ceilings,
        "cpu_baseline": None,
        "fp16_gemm": fp16,
        "wall_s_timed": t_wall,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(x, w, wl, args.cpu_seconds)
    print(json.dumps(line), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="qkv_175b")
    ap.add_argument("--rows", type=int, default=None, metavar="M",
                    help="another number of rows of X on the workload's weight (a mid-size or small batch)")
    ap.add_argument("--cpu-seconds", type=float, default=20.0, help="CPU work budget of the oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fp16-gemm", action="store_true")
    ap.add_argument("--no-warm", action="store_true", help="skip the warm (back-to-back) steps")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the MFMA and stream-read probes")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="before the steps, run a plain copy-shaped kernel over this many MiB (counter calibration)")
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="summarize two rocprofv3 counter runs into the stored traffic record and exit")
    ap.add_argument("--counter-summary", metavar="DIR",
                    help="summarize a rocprofv3 --kernel-trace --pmc GRBM_GUI_ACTIVE ... run into the stored "
                         "clock / MFMA-busy record and exit")
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

    wl = workloads.with_rows(workloads.WORKLOADS[args.workload], args.rows)
    if args.trace_summary:
        return trace_summary(args.trace_summary[0], args.trace_summary[1], wl, args.trace_summary[2], args.group)
    if args.traffic_summary:
        return traffic_summary(args.traffic_summary[0], args.traffic_summary[1], wl, args.copy_mib or 1024,
                               args.group)
    if args.counter_summary:
        return counter_summary(args.counter_summary, wl, args.group)
    if args.gpus != 1:
        print(f"bench.py: one GPU only; --gpus {args.gpus} is not supported (the library has no multi-GPU "
              f"path: each GPU would run the same kernels on its own column shard)", file=sys.stderr)
        return 2

    if args.codec:
        return codec_bench(args)
    if args.group:
        return group_bench(args, wl)
    return vector_bench(args, wl)


if __name__ == "__main__":
    sys.exit(main())
