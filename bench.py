"""Benchmark of the FP8 NT GEMM (1x128 / 128x128 float32 scales, BF16 out).

One step = one call of the GEMM on one batch of synthetic input already in
HBM. The headline workload is the dense 4096x7168x2048 GEMM; the grouped
contiguous, masked-decode, no-padding, UE8M0-scale, K-grouped and small dense
workloads are measured after it and reported under "workloads". Prints ONE
JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--only INDEX]
                    [--no-cpu-baseline] [--no-extra] [--copy-calibration]

--only INDEX times a single workload (0..12), for profiling runs.
Before the W warm-up steps, about 0.25 s of untimed calls let the GPU
clocks settle (a GEMM on random data runs the part below its nominal clock).
Besides the back-to-back timing, every workload is also timed cold: before
each of --cold-iters calls a 1 GiB scratch buffer is read, which evicts the
L2 caches and the 256 MB Infinity Cache, and each call is timed on its own
with HIP events (median and minimum reported under "cold").
--copy-calibration runs a plain 1 GiB device copy (for scaling HBM traffic
counters) and exits.
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

METRIC = "TFLOPS & % FP8 MFMA peak: dense, m-grouped contiguous, masked FP8 NT GEMM"
FP8_PEAK_TFLOPS = 5000.0     # MI355X dense FP8 MFMA, published
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
HEADLINE = 1                 # dense 4096x7168x2048
CSRC = os.path.join(ROOT, "moe_grouped_gemm_amd", "csrc")
# The device code and launch set-up behind each kernel; a traffic figure is
# valid only for the code it was counted on.
KERNEL_SOURCES = {
    "fp8_gemm_nt_kernel": ("dg_internal.h", "dg_device.h", "dg_kernel.hip", "dg_kernel_deep.hip"),
    "k_grouped_kernel": ("dg_internal.h", "dg_device.h", "dg_kernel_kgrouped.hip"),
    "fp8_fp4_gemm_kernel": ("dg_internal.h", "dg_device.h", "dg_kernel_fp4.hip"),
}
PROFILES = os.path.join(ROOT, "profiles")


def parse_args():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    # Enough untimed launches (about 0.1 s of GPU work on the headline
    # workload) for the clocks to settle before timing.
    p.add_argument("--warmup", type=int, default=1000)
    p.add_argument("--only", type=int, default=None)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extra", action="store_true")
    p.add_argument("--copy-calibration", action="store_true")
    p.add_argument("--cold-iters", type=int, default=30)
    p.add_argument("--no-ceiling", action="store_true")
    return p.parse_args()


def kernel_of(spec) -> str:
    """Name of the kernel that runs a workload."""
    if spec.kind == "k_grouped":
        return "k_grouped_kernel"
    return "fp8_fp4_gemm_kernel" if spec.extra.get("fp4") else "fp8_gemm_nt_kernel"


def kernel_source_sha(kernel: str) -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(spec):
    """HBM bytes per launch from the committed counter summary of this
    workload, or None if there is none or its kernel's source changed since."""
    path = os.path.join(PROFILES, f"traffic_{spec.name}.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                key, val = line.split(":", 1)
                fields[key.strip()] = val.strip()
    if fields.get("kernel_source_sha256_16") != kernel_source_sha(kernel_of(spec)):
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


SETTLE_S = 0.25   # untimed GPU work before the warm-up steps


def settle(w, d):
    """Untimed calls for about SETTLE_S seconds of GPU time, so that the
    clocks have ramped before the timed steps."""
    import torch
    from moe_grouped_gemm_amd import dg

    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < SETTLE_S:
        for _ in range(20):
            dg.run_workload(w, d)
        torch.cuda.synchronize()
        n += 20
    return n


def time_workload(w, steps: int, warmup: int):
    import torch
    from moe_grouped_gemm_amd import dg

    d = w.new_output()
    settle(w, d)
    for _ in range(warmup):
        dg.run_workload(w, d)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(steps):
        dg.run_workload(w, d)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kernel_ms = start.elapsed_time(end) / steps
    return wall * 1e3 / steps, kernel_ms


FLUSH_BYTES = 1 << 30  # beyond every cache on the path (L2 4 MB per XCD, Infinity Cache 256 MB)


def time_cold(w, iters: int, flush):
    """Per-call kernel times with the caches flushed before each call: the
    inputs are in HBM only. Returns (median_ms, min_ms)."""
    import statistics
    import torch
    from moe_grouped_gemm_amd import dg

    d = w.new_output()
    for _ in range(3):
        dg.run_workload(w, d)
    stream = torch.cuda.current_stream()
    events = []
    for _ in range(iters):
        flush.view(torch.int64).sum()  # reads 1 GiB: every cache now holds other (clean) lines
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record(stream)
        dg.run_workload(w, d)
        end.record(stream)
        events.append((start, end))
    torch.cuda.synchronize()
    times = [s.elapsed_time(e) for s, e in events]
    return statistics.median(times), min(times)


def copy_ceiling_gbs(buf) -> float:
    """Bytes moved (read + written) per second by a device-to-device copy of
    a 1 GiB buffer: the HBM rate a plain streaming kernel reaches here."""
    import statistics
    import torch
    dst = torch.empty_like(buf)
    for _ in range(3):
        dst.copy_(buf)
    times = []
    for _ in range(10):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        dst.copy_(buf)
        e.record()
        times.append((s, e))
    torch.cuda.synchronize()
    ms = statistics.median([a.elapsed_time(b) for a, b in times])
    del dst
    return 2 * buf.numel() * buf.element_size() / (ms * 1e-3) / 1e9


def mfma_ceiling_tflops(variant: int, iters: int = 4096) -> float:
    """FP8 dense TFLOP/s of the matrix-core loop alone (dg_mfma_fp8_ceiling:
    the GEMM kernels' launch shape and MFMA on random E4M3 operands, nothing
    else), median of 5 timed launches after 3 untimed ones."""
    import ctypes
    import statistics
    import torch
    from moe_grouped_gemm_amd import dg

    g = torch.Generator(device="cuda")
    g.manual_seed(12345)
    frag = torch.randint(0, 256, (4096,), dtype=torch.uint8, device="cuda", generator=g)
    frag[(frag & 0x7F) == 0x7F] = 0x3C          # no NaN codes
    sink = torch.empty(512 * max(dg.get_num_cus(), 1), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    flops = ctypes.c_longlong(0)

    def launch():
        st = dg.lib().dg_mfma_fp8_ceiling(frag.data_ptr(), sink.data_ptr(), iters, variant,
                                          ctypes.byref(flops), ctypes.c_void_p(stream.cuda_stream))
        if st != 0:
            raise RuntimeError(f"dg_mfma_fp8_ceiling: status {st}")
    for _ in range(3):
        launch()
    times = []
    for _ in range(5):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        launch()
        b.record(stream)
        times.append((a, b))
    torch.cuda.synchronize()
    ms = statistics.median(x.elapsed_time(y) for x, y in times)
    return flops.value / (ms * 1e-3) / 1e12


def inputs_sha256(w) -> str:
    """SHA-256 (first 16 hex digits) of a workload's quantised operand and
    scale bytes, so that runs on different machines can be matched."""
    from moe_grouped_gemm_amd import synth
    h = hashlib.sha256()
    for t in (w.a, w.sfa, w.b, w.sfb):
        h.update(synth.to_numpy_bytes(t).tobytes())
    return h.hexdigest()[:16]


def blas_threads_to_use() -> tuple:
    """(affinity-mask cores, BLAS threads to use): the threads are the cores
    of the process affinity mask, but no more than OMP_NUM_THREADS when the
    environment sets it (a host shared between GPUs gives each its share)."""
    affinity = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS")
    threads = min(affinity, int(env)) if env and env.isdigit() and int(env) > 0 else affinity
    return affinity, threads


def cpu_baseline(w, budget_s: float = 20.0):
    """The oracle timed on this host on the same bytes (full workload,
    repeated while within the time budget), with the BLAS thread count set
    explicitly; plus the exact-rational brute force timed once on a tiny
    shape on one core."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits
    from moe_grouped_gemm_amd import synth
    from oracle import dg_oracle as O

    affinity, threads = blas_threads_to_use()
    a, sfa, b, sfb = (synth.to_numpy_bytes(t) for t in (w.a, w.sfa, w.b, w.sfb))
    with threadpool_limits(limits=threads, user_api="blas"):
        blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        used = int(blas[0]["num_threads"]) if blas else threads
        vendor = (f"{blas[0].get('internal_api')} {blas[0].get('version')}" if blas else "unknown")
        # About 10 s of CPU work: repeat the full workload while under half the budget.
        runs, t_total = 0, 0.0
        while runs == 0 or (t_total < budget_s / 2 and runs < 40):
            t0 = time.perf_counter()
            O.fp8_gemm_nt(a, sfa, b, sfb)
            t_total += time.perf_counter() - t0
            runs += 1
    sec = t_total / runs
    # exact rationals, single core, on 2 x 128 x 256 of the same workload's bytes
    tm, tn, tk = 2, 128, 256
    t0 = time.perf_counter()
    O.gemm_nt_exact(a[:tm, :tk], sfa[:tk // 128, :tm], b[:tn, :tk], sfb[:1, :tk // 128])
    exact_s = time.perf_counter() - t0
    return {
        "value": round(w.flops() / sec / 1e12, 6),
        "unit": "TFLOPS",
        "cores": used,
        "kind": "oracle",
        "sample": f"full {w.m}x{w.n}x{w.k} dense workload, {runs} run(s) of the float64 numpy oracle "
                  f"(dequantise, fp64 GEMM, BF16 rounding), {sec:.2f} s each",
        "affinity_cores": affinity,
        "blas": vendor,
        "exact_rational_brute_force": {"shape": f"{tm}x{tn}x{tk}", "seconds": round(exact_s, 3), "cores": 1,
                                       "flops_per_s": round(2 * tm * tn * tk / exact_s, 1)},
    }


def copy_calibration():
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_each_way": n, "launches": 3}), flush=True)


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the GEMM has no cross-GPU step: sharded by expert or by N, each GPU runs its own "
              "share as an independent single-GPU call).", file=sys.stderr)
        sys.exit(2)

    import torch
    from moe_grouped_gemm_amd import dg, synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        copy_calibration()
        return
    dg.lib()
    dev = torch.device("cuda:0")

    headline = args.only if args.only is not None else HEADLINE
    spec = synth.workload_spec(headline)
    w = synth.make_workload(spec, seed=0, device=dev)
    torch.cuda.synchronize()
    ms_step, kernel_ms = time_workload(w, args.steps, args.warmup)
    flush = torch.ones(FLUSH_BYTES, dtype=torch.uint8, device=dev) if args.cold_iters > 0 else None

    def cold_entry(wx):
        if flush is None:
            return None
        med, mn = time_cold(wx, args.cold_iters, flush)
        return {"median_ms": round(med, 5), "min_ms": round(mn, 5), "iters": args.cold_iters,
                "tflops_median": round(wx.flops() / (med * 1e-3) / 1e12, 2),
                "algorithmic_gbs_median": round(wx.algorithmic_bytes() / (med * 1e-3) / 1e9, 1)}
    flops = w.flops()
    value = flops / (ms_step * 1e-3) / 1e12
    achieved = flops / (kernel_ms * 1e-3) / 1e12
    traffic = read_traffic(spec)
    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3",
        "data": "synthetic",
        "inputs_sha256_16": inputs_sha256(w),
        "torch": torch.__version__,
        "numpy": __import__("numpy").__version__,
        "config": {"workload": spec.name, "kind": spec.kind, "n": spec.n, "k": spec.k,
                   **({"m": spec.m} if spec.kind in ("dense", "k_grouped") else {}),
                   "accumulate": ("fp32, E8M0 block scales applied by the MFMA"
                                  if spec.extra.get("ue8m0") or spec.extra.get("fp4")
                                  else "fp32 with per-128-K promotion"),
                   "output": "fp32, accumulated into D in place" if spec.kind == "k_grouped" else "bf16",
                   "seed": 0},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": FP8_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / FP8_PEAK_TFLOPS, 4), "traffic": traffic,
                     "kernel": kernel_of(spec),
                     "kernel_ms": round(kernel_ms, 5),
                     "algorithmic_bytes": w.algorithmic_bytes()},
    }
    out["roofline"]["timing"] = (f"HIP events on the launch stream around {args.steps} back-to-back calls, after "
                                 f"{args.warmup} untimed warm-up calls and {SETTLE_S} s of untimed calls that let the "
                                 "clocks settle; achieved = algorithmic work / (event time / calls)")
    if spec.kind == "masked":
        gbs = w.algorithmic_bytes() / (kernel_ms * 1e-3) / 1e9
        out["roofline"].update({"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                "frac": round(gbs / HBM_PEAK_GBS, 4)})
    out["cold"] = cold_entry(w)
    if out["cold"] is not None:
        cold_ms = out["cold"]["median_ms"]
        if spec.kind == "masked":
            out["roofline"]["frac_cold"] = round(w.algorithmic_bytes() / (cold_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
        else:
            out["roofline"]["frac_cold"] = round(flops / (cold_ms * 1e-3) / 1e12 / FP8_PEAK_TFLOPS, 4)
        out["roofline"]["frac_cold_timing"] = ("median of per-call HIP event times, each call after a 1 GiB read "
                                               "that evicts the L2 caches and the Infinity Cache")
    if flush is not None:
        out["hbm_copy_gbs"] = round(copy_ceiling_gbs(flush), 1)
    if not args.no_ceiling:
        ceil, ceil_promote, ceil32, ceil32_promote, ceil_col = (mfma_ceiling_tflops(v) for v in range(5))
        out["mfma_ceiling"] = {"tflops": round(ceil, 1), "tflops_with_fp32_promotion": round(ceil_promote, 1),
                               "tflops_with_per_column_promotion": round(ceil_col, 1),
                               "tflops_32x32x64": round(ceil32, 1),
                               "tflops_32x32x64_with_fp32_promotion": round(ceil32_promote, 1),
                               "what": "FP8 MFMA loop alone (16x16x128, the GEMMs' instruction; 32x32x64 for "
                                       "comparison), the GEMM's launch shape, random operands; with the "
                                       "float32 promotion of the float32-scale GEMMs (per-column: the "
                                       "K-grouped GEMM's)"}
        if spec.kind != "masked":
            # Against the loop alone, and against the loop with the same
            # promotion work as this workload's kernel.
            e8 = bool(spec.extra.get("ue8m0", False) or spec.extra.get("fp4", False))  # no promotion
            same = ceil if e8 else (ceil_col if spec.kind == "k_grouped" else ceil_promote)
            out["roofline"]["frac_of_measured_mfma_ceiling"] = round(achieved / ceil, 4)
            out["roofline"]["frac_of_measured_ceiling_with_same_promotion"] = round(achieved / same, 4)
    out["context"] = {
        "note": "claims for other hardware, quoted as context only (not targets, not baselines)",
        "ascend_950_dense_gemm": "up to 99.8% of theoretical TFLOPS (BF16/FP8/FP4, shapes not given)",
        "ascend_950_m_grouped_gemm": "above 800 TFLOPS on realistic expert-token patterns",
        "source": "third-party summary of the DeepGEMM-Ascend README",
    }

    if args.only is None and not args.no_extra:
        extra = {}
        for idx in (i for i in range(synth.NUM_WORKLOADS) if i != HEADLINE):
            s = synth.workload_spec(idx)
            wx = synth.make_workload(s, seed=0, device=dev)
            torch.cuda.synchronize()
            # time_workload lets the clocks settle first; at least 50 timed
            # calls whatever --steps is, so that short runs still average
            # over many launches
            steps = max(50, args.steps // 4)
            ms, kms = time_workload(wx, steps, max(10, args.warmup // 3))
            tf = wx.flops() / (kms * 1e-3) / 1e12
            gbs = wx.algorithmic_bytes() / (kms * 1e-3) / 1e9
            extra[s.name] = {"kernel_ms": round(kms, 5), "tflops": round(tf, 2),
                             "fp8_peak_frac": round(tf / FP8_PEAK_TFLOPS, 4),
                             "algorithmic_gbs": round(gbs, 1), "hbm_peak_frac": round(gbs / HBM_PEAK_GBS, 4),
                             "valid_rows": getattr(wx, "valid_rows", lambda: s.m)(),
                             "cold": cold_entry(wx)}
            del wx
            torch.cuda.empty_cache()
        out["workloads"] = extra

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w) if spec.kind == "dense" else None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
