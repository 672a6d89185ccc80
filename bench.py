"""Throughput of the single-precision product C = A x B on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--variant V] [--no-cpu-baseline] [--no-secondary]
    python bench.py --table | --general | --small | --shards | --ladder
                    | --vector-add | --bf16x3 | --bf16x3-general | --copy-calibration

One step is one call of sgemm_run on the 8192^3 workload (uniform[-1, 1)
inputs from seed 4, already resident in HBM).  W untimed calls, then exactly
K calls between two synchronisations, timed with HIP events recorded on the
stream the kernels run on.  Prints one JSON line.  The 2048^3 workload is
timed the same way (200 calls, after 0.3 s of untimed calls so that the
clocks have settled) and reported under "secondary".

The other modes print one JSON line per case: every workload with oracle
times (--table), the general form and strided batches (--general), small
products with sgemm_run's tile and every forced tile (--small), one
GPU's share of 8192^3 split by rows over 1-8 GPUs (--shards), the pages'
progression (--ladder), the vector add (--vector-add), the bfloat16 split
path (--bf16x3, --bf16x3-general), and the copy that calibrates the HBM
counters (--copy-calibration).

The CPU baseline is the oracle (double-precision triple loop) timed on the
host cores on a bounded sample of the same workload: the first R rows of C,
with R chosen so the sample takes roughly 10-20 s; its rate is scaled to the
same unit (TFLOP/s of the single-precision product it checks).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "FP32 SGEMM TFLOPS at 2048³ and 8192³ on 1 MI355X; % of FP32 MFMA peak"
PEAK_TFLOPS = 157.3    # MI355X dense FP32 matrix-core peak (published)
HEADLINE = "sgemm_8192x8192x8192_uniform_seed4"
SECONDARY = "sgemm_2048x2048x2048_uniform_seed2"
COUNTERS = os.path.join(ROOT, "profiles", "mfma_gemm_8192_hbm_counters.json")
COPY_BYTES = 256 << 20  # bytes read (and written) by the copy-calibration kernel


# Sources that define the kernel sgemm_run launches for aligned operands (its
# template, its shared helpers, its configurations, the file that
# instantiates them and the one that picks the configuration).
HOT_KERNEL_SOURCES = ("common.hpp", "mfma_dma.hpp", "mfma_configs.hpp", "mfma_layout_nn.hip",
                      "mfma_kernels.hip")


def kernel_source_digest() -> str:
    """Digest of the hot kernel's sources; HBM counters are valid only for it."""
    csrc = os.path.join(ROOT, "dense_fp32_matrix_03_amd", "csrc")
    h = hashlib.sha256()
    for name in HOT_KERNEL_SOURCES:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def measured_traffic(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when there is none for this workload or the kernels changed since."""
    try:
        with open(COUNTERS) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("workload") != workload or c.get("source_sha256") != kernel_source_digest():
        return None
    return c.get("hbm_bytes_per_launch")


# Library calls made by this process, in order, and the range of them that
# the last time_gpu() timed: (index of its first timed call, number of timed
# calls).  Each sgemm_run launches one kernel, so with --trace-summary these
# index the library's dispatches in a rocprofv3 kernel trace of the run.
_CALLS = [0]
LAST_TIMED = [(0, 0)]


def trace_fields() -> dict:
    first, n = LAST_TIMED[0]
    return {"trace_first": first, "trace_calls": n}


def write_hbm_counters(fetch_csv: str, write_csv: str, copy_fetch_csv: str,
                       copy_write_csv: str, out: str = COUNTERS) -> dict:
    """Host only: turn four rocprofv3 counter CSVs into the HBM-traffic
    summary the headline line quotes.  FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch) of the product kernel's dispatches in a run of the headline
    command, each scaled by what the same counter reads for the runtime's
    256 MiB device copy (COPY_BYTES read and written, from a run of
    --copy-calibration): scale = COPY_BYTES / (KiB x 1024).  Stamped with the
    digest of the hot kernel's sources."""
    import csv

    def values(path, counter, kernel):
        with open(path, newline="") as f:
            return [float(r["Counter_Value"]) for r in csv.DictReader(f)
                    if r["Counter_Name"] == counter and kernel in r["Kernel_Name"]]

    fetch = values(fetch_csv, "FETCH_SIZE", "mfma_gemm_dma_kernel")
    write = values(write_csv, "WRITE_SIZE", "mfma_gemm_dma_kernel")
    cfetch = values(copy_fetch_csv, "FETCH_SIZE", "copyBuffer")
    cwrite = values(copy_write_csv, "WRITE_SIZE", "copyBuffer")
    if not (fetch and write and cfetch and cwrite):
        raise ValueError("a counter CSV holds no dispatch of the expected kernel")
    with open(fetch_csv, newline="") as f:
        kernel = next(r["Kernel_Name"] for r in csv.DictReader(f)
                      if "mfma_gemm_dma_kernel" in r["Kernel_Name"])
    fscale = COPY_BYTES / (sum(cfetch) / len(cfetch) * 1024)
    wscale = COPY_BYTES / (sum(cwrite) / len(cwrite) * 1024)
    hbm = (sum(fetch) / len(fetch) * fscale + sum(write) / len(write) * wscale) * 1024
    from dense_fp32_matrix_03_amd import inputs
    cmd = "cd /tmp && TMPDIR=/tmp rocprofv3 --pmc {} --output-format csv -d <out> -o run -- "
    c = {"kernel": kernel, "workload": HEADLINE,
         "commands": {"FETCH_SIZE": cmd.format("FETCH_SIZE") + "python3 <repo>/bench.py "
                      "--steps 3 --warmup 1 --no-cpu-baseline --no-secondary",
                      "WRITE_SIZE": cmd.format("WRITE_SIZE") + "python3 <repo>/bench.py "
                      "--steps 3 --warmup 1 --no-cpu-baseline --no-secondary",
                      "copy_FETCH_SIZE": cmd.format("FETCH_SIZE") + "python3 <repo>/bench.py "
                      "--copy-calibration",
                      "copy_WRITE_SIZE": cmd.format("WRITE_SIZE") + "python3 <repo>/bench.py "
                      "--copy-calibration",
                      "summary": "python3 bench.py --write-hbm-counters FETCH WRITE COPY_FETCH "
                                 "COPY_WRITE (run_counter_collection.csv of each)"},
         "fetch_kib_per_dispatch": fetch, "write_kib_per_dispatch": write,
         "copy_kernel": "__amd_rocclr_copyBuffer, 256 MiB read + 256 MiB written",
         "copy_fetch_kib_per_dispatch": cfetch, "copy_write_kib_per_dispatch": cwrite,
         "fetch_scale": round(fscale, 4), "write_scale": round(wscale, 4),
         "hbm_bytes_per_launch": int(round(hbm)),
         "algorithmic_bytes_per_launch": inputs.BY_NAME[HEADLINE].min_bytes,
         "source_files": list(HOT_KERNEL_SOURCES), "source_sha256": kernel_source_digest()}
    with open(out, "w") as f:
        json.dump(c, f, indent=1)
        f.write("\n")
    return c


def time_gpu(w, variant: str, steps: int, warmup: int, warm_seconds: float = 0.0,
             trials: int = 1):
    import torch

    import dense_fp32_matrix_03_amd as sg
    from dense_fp32_matrix_03_amd import inputs

    A, B = inputs.make_inputs(w)
    dA = torch.from_numpy(A).cuda()
    dB = torch.from_numpy(B).cuda()
    del A, B
    dC = torch.empty((w.M, w.ldc), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    h = stream.cuda_stream

    # Device addresses as ints: the binding's tensor checks would add host
    # time per call that a product of a few microseconds cannot hide.
    pa, pb, pc = dA.data_ptr(), dB.data_ptr(), dC.data_ptr()

    def step():
        sg.sgemm_run_variant(variant, w.M, w.N, w.K, pa, w.lda, pb, w.ldb, pc, w.ldc, h)
        _CALLS[0] += 1

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # Optionally keep the device busy a little longer before timing, so that
    # short kernels are not timed while the clocks are still ramping up.
    t_end = time.perf_counter() + warm_seconds
    while time.perf_counter() < t_end:
        for _ in range(50):
            step()
        torch.cuda.synchronize()
    per_trial = []
    LAST_TIMED[0] = (_CALLS[0], steps * trials)
    for _ in range(trials):
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for _ in range(steps):
            step()
        t1.record(stream)
        torch.cuda.synchronize()
        per_trial.append(t0.elapsed_time(t1) / steps)
    finite = bool(torch.isfinite(dC[:, :w.N]).all().item())
    del dA, dB, dC
    torch.cuda.empty_cache()
    if trials == 1:
        return per_trial[0], finite
    return per_trial, finite


def time_graph(w, variant: str, calls: int = 50, replays: int = 20) -> float:
    """Per-call GPU time (ms) of `calls` sgemm_run launches captured in one
    HIP graph and replayed: the kernels run back to back with no host launch
    cost between them, which is what a short product costs inside a
    captured sequence."""
    import torch

    import dense_fp32_matrix_03_amd as sg
    from dense_fp32_matrix_03_amd import inputs

    A, B = inputs.make_inputs(w)
    dA = torch.from_numpy(A).cuda()
    dB = torch.from_numpy(B).cuda()
    del A, B
    dC = torch.empty((w.M, w.ldc), dtype=torch.float32, device="cuda")

    def body():
        for _ in range(calls):
            sg.sgemm_run_variant(variant, w.M, w.N, w.K, dA, w.lda, dB, w.ldb, dC, w.ldc)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        body()  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        body()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(replays):
        g.replay()
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / (calls * replays)
    del g, dA, dB, dC
    torch.cuda.empty_cache()
    return ms


def mfma_ceiling(which: int = 0, iters: int = 20000) -> float:
    """TFLOP/s of the library's register-only matrix-core loop (which = 0:
    FP32 32x32x2, 1: bfloat16 32x32x16), best of 5 launches after 2."""
    import torch

    import dense_fp32_matrix_03_amd as sg

    out = torch.empty(1024 * torch.cuda.get_device_properties(0).multi_processor_count,
                      dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    best = 0.0
    for i in range(7):
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        flops = sg.sgemm_mfma_ceiling(which, iters, out, out.numel(), stream.cuda_stream)
        t1.record(stream)
        torch.cuda.synchronize()
        if i >= 2:
            best = max(best, flops / (t0.elapsed_time(t1) * 1e-3) / 1e12)
    if not bool(torch.isfinite(out).all().item()):
        raise RuntimeError("matrix-core ceiling loop produced non-finite sums")
    return best


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, target_s: float = 12.0):
    """Time the oracle on the first R rows of the workload (no GPU involved)."""
    import numpy as np

    import oracle
    from dense_fp32_matrix_03_amd import inputs

    A, B = inputs.make_inputs(w)
    threads = oracle.max_threads()
    rows = 8
    while True:
        t = time.perf_counter()
        oracle.sgemm_f64(np.ascontiguousarray(A[:rows]), B, K=w.K, N=w.N, want_sabs=False,
                         threads=threads)
        dt = time.perf_counter() - t
        if dt >= target_s or rows >= w.M:
            break
        rows = min(w.M, max(rows * 2, int(rows * target_s / max(dt, 1e-3) * 1.05)))
    flops = 2.0 * rows * w.N * w.K
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"first {rows} of {w.M} rows of C (= {rows}x{w.N}x{w.K}), double "
                      f"accumulation, {dt:.1f} s on {threads} threads"}


def oracle_seconds(w, threads: int, rows: int | None = None) -> tuple[float, int]:
    """Wall time of the oracle's C pass (no abs-sum) on the first `rows` rows."""
    import numpy as np

    import oracle
    from dense_fp32_matrix_03_amd import inputs

    A, B = inputs.make_inputs(w)
    rows = w.M if rows is None else rows
    A = np.ascontiguousarray(A[:rows])
    t = time.perf_counter()
    oracle.sgemm_f64(A, B, K=w.K, N=w.N, want_sabs=False, threads=threads)
    return time.perf_counter() - t, rows


def workload_table(variant) -> list[dict]:
    """GPU time of sgemm_run (10 trials of R back-to-back calls, R = max(10,
    200 ms / t); median and min) and oracle times, for every workload, with
    the rate as a fraction of the published peak and of the measured
    matrix-core ceiling.  Products under 1e11 flops are also timed inside a
    captured graph (time_graph), where no host launch cost separates the
    calls."""
    import statistics

    import oracle
    from dense_fp32_matrix_03_amd import inputs

    cores = oracle.max_threads()
    ceiling = mfma_ceiling(0)
    print(json.dumps({"mfma_ceiling_tflops": round(ceiling, 2),
                      "pct_of_peak": round(100 * ceiling / PEAK_TFLOPS, 1),
                      "host_cpu": cpu_model(), "host_threads": cores}), flush=True)
    rows = []
    rate1 = None
    for w in inputs.WORKLOADS:
        ms0, _ = time_gpu(w, variant, 5, 3, warm_seconds=0.3)
        reps = max(10, int(math.ceil(200.0 / ms0)))
        trials, finite = time_gpu(w, variant, reps, 3, warm_seconds=0.3, trials=10)
        med, best = statistics.median(trials), min(trials)
        tf = w.flops / (med * 1e-3) / 1e12
        r = {"workload": w.name, "trials": 10, "calls_per_trial": reps,
             "gpu_ms_median": round(med, 5), "gpu_ms_min": round(best, 5),
             "gpu_tflops": round(tf, 2), "gpu_tflops_best": round(w.flops / (best * 1e-3) / 1e12, 2),
             "pct_of_peak": round(100 * tf / PEAK_TFLOPS, 1),
             "pct_of_mfma_ceiling": round(100 * tf / ceiling, 1), "output_finite": finite,
             "cores": cores}
        if w.flops < 1e11:
            # Short products: also the per-call time inside a captured graph.
            mg = time_graph(w, variant)
            r.update(gpu_ms_graph=round(mg, 5),
                     gpu_tflops_graph=round(w.flops / (mg * 1e-3) / 1e12, 2))
        if w.check == "full":
            t1, _ = oracle_seconds(w, 1)
            tn, _ = oracle_seconds(w, cores)
            rate1 = w.flops / t1
            r.update(oracle_1core_s=round(t1, 3), oracle_allcore_s=round(tn, 3))
        else:
            tn, _ = oracle_seconds(w, cores)
            r.update(oracle_allcore_s=round(tn, 3),
                     oracle_1core_s_extrapolated=round(w.flops / rate1, 1) if rate1 else None)
        print(json.dumps(r), flush=True)
        rows.append(r)
    return rows


LADDER = ("naive", "lds", "reg", "dbuf", "mfma_unpadded", "mfma_staged", "mfma_dword",
          "mfma_serial", "mfma")


def ladder(w, steps: int, warmup: int, settle: float) -> list[dict]:
    """Time the pages' progression and the matrix-core steps on one workload."""
    import dense_fp32_matrix_03_amd as sg

    rows = []
    for name in LADDER:
        v = sg.VARIANTS[name]
        ms, finite = time_gpu(w, v, steps, warmup, warm_seconds=settle)
        tf = w.flops / (ms * 1e-3) / 1e12
        r = {"case": sg.sgemm_variant_name(v), "workload": w.name, "M": w.M, "N": w.N,
             "K": w.K, "variant": sg.sgemm_variant_name(v), "ms": round(ms, 5),
             "tflops": round(tf, 3), "pct_of_peak": round(100 * tf / PEAK_TFLOPS, 2),
             "output_finite": finite, **trace_fields()}
        print(json.dumps(r), flush=True)
        rows.append(r)
    print(json.dumps({"trace_total_calls": _CALLS[0]}), flush=True)
    return rows


# General-form cases: (name, transA, transB, M, N, K, alpha, beta, batch).
GENERAL = (
    ("nn_2048", 0, 0, 2048, 2048, 2048, 1.0, 0.0, 1),
    ("nt_2048", 0, 1, 2048, 2048, 2048, 1.0, 0.0, 1),
    ("tn_2048", 1, 0, 2048, 2048, 2048, 1.0, 0.0, 1),
    ("tt_2048", 1, 1, 2048, 2048, 2048, 1.0, 0.0, 1),
    ("nn_2048_alpha_beta", 0, 0, 2048, 2048, 2048, 1.5, 0.5, 1),
    ("nn_8192", 0, 0, 8192, 8192, 8192, 1.0, 0.0, 1),
    ("nt_8192", 0, 1, 8192, 8192, 8192, 1.0, 0.0, 1),
    ("tn_8192", 1, 0, 8192, 8192, 8192, 1.0, 0.0, 1),
    ("tt_8192", 1, 1, 8192, 8192, 8192, 1.0, 0.0, 1),
    ("nn_8192_alpha_beta", 0, 0, 8192, 8192, 8192, 1.5, 0.5, 1),
    ("batched_64x512", 0, 0, 512, 512, 512, 1.0, 0.0, 64),
    ("batched_16x1024_nt", 0, 1, 1024, 1024, 1024, 1.0, 0.0, 16),
    ("batched_1024x64", 0, 0, 64, 64, 64, 1.0, 0.0, 1024),
)


def general_table(settle: float) -> list[dict]:
    """Time sgemm_run_strided_batched on the GENERAL cases (uniform inputs,
    packed operands), one JSON line each."""
    import numpy as np
    import torch

    import dense_fp32_matrix_03_amd as sg
    from dense_fp32_matrix_03_amd import inputs

    rows = []
    stream = torch.cuda.current_stream()
    h = stream.cuda_stream
    for name, ta, tb, M, N, K, alpha, beta, batch in GENERAL:
        g = np.random.default_rng(7)
        ar, ac = (K, M) if ta else (M, K)
        br, bc = (N, K) if tb else (K, N)
        dA = torch.from_numpy(inputs.uniform(g, (batch, ar, ac))).cuda()
        dB = torch.from_numpy(inputs.uniform(g, (batch, br, bc))).cuda()
        dC = torch.from_numpy(inputs.uniform(g, (batch, M, N))).cuda()

        def step():
            sg.sgemm_run_strided_batched(ta, tb, M, N, K, alpha, dA, ac, ar * ac, dB, bc,
                                         br * bc, beta, dC, N, M * N, batch, h)

        flops = 2.0 * M * N * K * batch
        for _ in range(3):
            step()
        torch.cuda.synchronize()
        t_end = time.perf_counter() + settle
        while time.perf_counter() < t_end:
            for _ in range(20):
                step()
            torch.cuda.synchronize()
        steps = max(10, min(200, int(4e12 / flops)))
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for _ in range(steps):
            step()
        t1.record(stream)
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / steps
        tf = flops / (ms * 1e-3) / 1e12
        r = {"case": name, "transA": ta, "transB": tb, "M": M, "N": N, "K": K, "alpha": alpha,
             "beta": beta, "batch": batch, "ms": round(ms, 5), "tflops": round(tf, 2),
             "pct_of_peak": round(100 * tf / PEAK_TFLOPS, 1),
             "output_finite": bool(torch.isfinite(dC).all().item())}
        print(json.dumps(r), flush=True)
        rows.append(r)
        del dA, dB, dC
        torch.cuda.empty_cache()
    return rows


# Tile sweep: (M, N, K, lda).  Small products, where the count of tiles
# decides, and medium ones on either side of each switch of sgemm_run's tile
# rule; 1000 x 1500 x 777 is the ragged workload (A rows not 16-byte aligned).
SMALL = ((256, 256, 256, 256), (300, 260, 100, 100), (128, 128, 128, 128), (256, 256, 32, 32),
         (768, 256, 256, 256), (256, 256, 1024, 1024), (512, 512, 64, 64), (512, 512, 128, 128),
         (384, 384, 256, 256), (100, 3000, 64, 64), (640, 640, 64, 64), (640, 640, 128, 128),
         (1000, 130, 256, 256), (512, 512, 256, 256),
         (384, 384, 512, 512), (1000, 130, 1024, 1024), (512, 512, 512, 512),
         (768, 768, 768, 768), (640, 640, 2048, 2048), (1000, 130, 2048, 2048),
         (768, 1024, 512, 512), (832, 1024, 512, 512), (1024, 1024, 1024, 1024),
         (1000, 1500, 776, 776), (1000, 1500, 777, 777), (960, 1600, 777, 777),
         (1000, 1700, 777, 777), (1024, 1536, 1024, 1024), (1200, 1200, 1200, 1200),
         (1536, 1536, 1536, 1536),
         (2048, 2048, 2048, 2048), (3072, 3072, 1024, 1024), (4096, 4096, 1024, 1024))
SMALL_TILES = ("mfma", "mfma_256", "mfma_128", "mfma_64x96", "mfma_64", "mfma_32x64", "mfma_32",
               "mfma_16")


def small_table(steps: int, settle: float) -> list[dict]:
    """sgemm_run and every forced tile on the SMALL shapes: HIP-event time
    per call over `steps` back-to-back calls after `settle` seconds of
    untimed calls (for the shortest this includes the host's launch cost; a
    kernel trace of the run gives the kernels' own durations through
    --trace-summary).  One JSON line per shape and tile."""
    from dense_fp32_matrix_03_amd import inputs

    import dense_fp32_matrix_03_amd as sg

    rows = []
    for M, N, K, lda in SMALL:
        w = inputs.Workload(f"sgemm_{M}x{N}x{K}_uniform_seed{M + N + K}", M, N, K, "uniform",
                            M + N + K, lda, N, N, "full")
        for variant in SMALL_TILES:
            v = sg.VARIANTS[variant]
            ms, finite = time_gpu(w, v, steps, 10, warm_seconds=settle)
            r = {"case": sg.sgemm_variant_name(v), "M": M, "N": N, "K": K, "lda": lda,
                 "variant": sg.sgemm_variant_name(v), "us": round(ms * 1e3, 3),
                 "tflops": round(w.flops / (ms * 1e-3) / 1e12, 2), "output_finite": finite,
                 **trace_fields()}
            print(json.dumps(r), flush=True)
            rows.append(r)
    print(json.dumps({"trace_total_calls": _CALLS[0]}), flush=True)
    return rows


# Fixed cost and per-k cost of one launch: M = N in KSCAN_MN, K in KSCAN_K
# (t = a + b K per shape), after two floor cases, then the five workloads.
KSCAN_MN = (256, 1024)
KSCAN_K = (32, 64, 128, 256, 512, 1024, 2048, 4096)


def kscan_cases():
    """(label, Workload) in the order --kscan runs them."""
    from dense_fp32_matrix_03_amd import inputs

    def w(M, N, K, seed=11):
        return inputs.Workload(f"sgemm_{M}x{N}x{K}_uniform_seed{seed}", M, N, K, "uniform",
                               seed, max(K, 1), N, N, "full")

    cases = [("floor: K = 0 (zero fill, no operand read)", w(256, 256, 0)),
             ("floor: one 32x32 tile", w(32, 32, 32))]
    for mn in KSCAN_MN:
        for k in KSCAN_K:
            cases.append((f"kscan M=N={mn}", w(mn, mn, k)))
    for wl in inputs.WORKLOADS:
        cases.append(("workload", wl))
    return cases


def kscan_table(variant, calls: int) -> list[dict]:
    """HIP-event time per call of sgemm_run on every kscan case (`calls`
    back-to-back calls after 20 untimed ones and 0.1 s of settling; 20 calls
    for 8192^3), one JSON line each with the range of library dispatches it
    timed (trace_first, trace_calls) for --trace-summary."""
    rows = []
    for label, w in kscan_cases():
        n = calls if w.flops < 1e12 else 20
        ms, finite = time_gpu(w, variant, n, 20 if n == calls else 3, warm_seconds=0.1)
        r = {"case": label, "workload": w.name, "M": w.M, "N": w.N, "K": w.K,
             "us": round(ms * 1e3, 3),
             "tflops": round(w.flops / (ms * 1e-3) / 1e12, 2) if w.K else 0.0,
             "output_finite": finite, **trace_fields()}
        print(json.dumps(r), flush=True)
        rows.append(r)
    print(json.dumps({"trace_total_calls": _CALLS[0]}), flush=True)
    return rows


# Products whose phases --phases reports: the five workloads and the ends of
# the K-scan.
PHASE_SHAPES = ((256, 256, 256), (1024, 1024, 1024), (2048, 2048, 2048), (1000, 1500, 777),
                (8192, 8192, 8192), (256, 256, 32), (256, 256, 4096), (1024, 1024, 32),
                (1024, 1024, 4096))
REALTIME_MHZ = 100.0  # s_memrealtime's reference clock on MI355X


def phase_table(settle: float) -> list[dict]:
    """Where a call's time goes: sgemm_phase_times on each PHASE_SHAPES
    product (A row-major with lda = K unless the workload says otherwise),
    after `settle` seconds of untimed calls, next to sgemm_run's own HIP-event
    time per call.  Per work-group, from the timestamps of the last of 20
    back-to-back calls: first-slice latency, main loop, k-set reduction,
    stores; across work-groups the spread of their starts and the span from
    the first start to the last end; the shader clock; and the main loop's
    matrix-core time at that clock (32 multiply-adds per cycle per SIMD)."""
    import numpy as np
    import torch

    import dense_fp32_matrix_03_amd as sg
    from dense_fp32_matrix_03_amd import inputs

    rows = []
    stream = torch.cuda.current_stream()
    h = stream.cuda_stream
    for M, N, K in PHASE_SHAPES:
        lda = 777 if (M, N, K) == (1000, 1500, 777) else K
        w = inputs.Workload(f"sgemm_{M}x{N}x{K}_uniform_seed{M + N + K}", M, N, K, "uniform",
                            M + N + K, lda, N, N, "full")
        ms, _ = time_gpu(w, sg.VARIANTS["mfma"], 20 if w.flops > 1e12 else 200, 5,
                         warm_seconds=settle)
        A, B = inputs.make_inputs(w)
        dA, dB = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
        dC = torch.empty((M, N), dtype=torch.float32, device="cuda")
        wgs = sg.sgemm_phase_times(M, N, K, dA, lda, dB, N, dC, N, None, 0, h)
        t = torch.zeros(8 * wgs, dtype=torch.int64, device="cuda")
        calls = 20
        t_end = time.perf_counter() + settle
        while True:
            for _ in range(calls):
                sg.sgemm_phase_times(M, N, K, dA, lda, dB, N, dC, N, t, t.numel(), h)
            torch.cuda.synchronize()
            if time.perf_counter() >= t_end:
                break
        q = t.cpu().numpy().astype(np.int64).reshape(wgs, 8)
        tile = int(q[0, 7])
        bm, bn, bk, ks = tile & 0xffff, (tile >> 16) & 0xffff, (tile >> 32) & 0xffff, tile >> 48
        us = 1.0 / REALTIME_MHZ

        def mean(a):
            return float(np.mean(a)) * us

        clock = float(np.mean((q[:, 6] - q[:, 5]) / np.maximum(q[:, 4] - q[:, 0], 1))) * REALTIME_MHZ
        kp = -(-K // bk) * bk
        # 32 multiply-adds per cycle per SIMD on either instruction (32x32x2
        # in 64 cycles, 16x16x4 in 32); the tile's four SIMDs share the work.
        loop_mfma_us = bm * bn * kp / 32 / 4 / clock
        r = {"M": M, "N": N, "K": K, "lda": lda, "tile": f"{bm}x{bn}x{bk}", "k_sets": ks,
             "workgroups": wgs, "call_us": round(ms * 1e3, 3),
             "span_us": round(float(q[:, 4].max() - q[:, 0].min()) * us, 3),
             "start_spread_us": round(float(q[:, 0].max() - q[:, 0].min()) * us, 3),
             "first_slice_us": round(mean(q[:, 1] - q[:, 0]), 3),
             "loop_us": round(mean(q[:, 2] - q[:, 1]), 3),
             "reduce_us": round(mean(q[:, 3] - q[:, 2]), 3),
             "store_us": round(mean(q[:, 4] - q[:, 3]), 3),
             "workgroup_us": round(mean(q[:, 4] - q[:, 0]), 3),
             "clock_mhz": round(clock, 0), "loop_mfma_us": round(loop_mfma_us, 3)}
        # Work-group w runs on XCD w % 8 (the dispatcher deals work-groups
        # to the eight XCDs in turn): per-XCD shader clock, main loop in
        # cycles at that clock, and the last end of a work-group.
        xcd = np.arange(wgs) % 8
        wg_clock = (q[:, 6] - q[:, 5]) / np.maximum(q[:, 4] - q[:, 0], 1) * REALTIME_MHZ
        loop_cyc = (q[:, 2] - q[:, 1]) * us * wg_clock
        xs = [x for x in range(8) if (xcd == x).any()]
        r["xcd_clock_mhz"] = [round(float(wg_clock[xcd == x].mean()), 0) for x in xs]
        r["xcd_loop_kcycles"] = [round(float(loop_cyc[xcd == x].mean()) / 1e3, 2) for x in xs]
        r["xcd_end_us"] = [round(float(q[xcd == x, 4].max() - q[:, 0].min()) * us, 2) for x in xs]
        print(json.dumps(r), flush=True)
        rows.append(r)
        del dA, dB, dC, t
        torch.cuda.empty_cache()
    return rows


def _read_csv(path):
    import csv
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def trace_summary(trace_csv: str, cases_jsonl: str, counters_csv: str | None = None) -> str:
    """Markdown table of kernel-trace durations (and, given a counter CSV of
    the same command, per-dispatch counter means) for every case line of a
    bench run's output that carries trace_first / trace_calls.  The
    library's dispatches are those whose kernel lives in namespace sgemm::,
    taken in dispatch order; their count must equal the run's
    trace_total_calls.  A counter CSV may also be given alone, in place of
    the trace.  Runs on the host, no GPU."""
    import statistics

    cases, total = [], None
    with open(cases_jsonl) as f:
        for line in f:
            line = line.strip()
            if not line.startswith("{"):
                continue
            d = json.loads(line)
            if "trace_total_calls" in d:
                total = d["trace_total_calls"]
            elif "trace_first" in d:
                cases.append(d)

    def ours(name):
        return "sgemm::" in name

    rows0 = _read_csv(trace_csv)
    if rows0 and "Counter_Name" in rows0[0]:
        # A counter CSV given alone: one row per dispatch and counter; its
        # timestamps (taken under counter collection) stand in for the trace.
        counters_csv, seen, kept = trace_csv, set(), []
        for r in rows0:
            if ours(r["Kernel_Name"]) and r["Dispatch_Id"] not in seen:
                seen.add(r["Dispatch_Id"])
                kept.append(r)
        rows0 = kept
    disp = sorted((r for r in rows0 if ours(r["Kernel_Name"])),
                  key=lambda r: int(r["Dispatch_Id"]))
    if total is not None and len(disp) != total:
        raise ValueError(f"{len(disp)} library dispatches in the trace, run made {total} calls")
    counters = {}
    if counters_csv:
        per = {}
        for r in _read_csv(counters_csv):
            if ours(r["Kernel_Name"]):
                per.setdefault(int(r["Dispatch_Id"]), {})[r["Counter_Name"]] = \
                    float(r["Counter_Value"])
        order = sorted(per)
        if total is not None and len(order) != total:
            raise ValueError(f"{len(order)} library dispatches in the counters, run made "
                             f"{total} calls")
        counters = {i: per[d] for i, d in enumerate(order)}
    names = sorted({k for v in counters.values() for k in v})
    head = ["case", "M x N x K", "kernel", "dispatches", "mean us", "median us", "min us",
            "TFLOP/s (mean)"] + names
    out = ["| " + " | ".join(head) + " |", "|" + "---|" * len(head)]
    for c in cases:
        i0, n = c["trace_first"], c["trace_calls"]
        rows = disp[i0:i0 + n]
        us = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3 for r in rows]
        kern = rows[0]["Kernel_Name"].split("(")[0].replace("void ", "").replace("sgemm::", "")
        mean = statistics.mean(us)
        fl = 2.0 * c["M"] * c["N"] * c["K"]
        cells = [c.get("case", ""), f'{c["M"]}x{c["N"]}x{c["K"]}', f"`{kern}`", str(n),
                 f"{mean:.3f}", f"{statistics.median(us):.3f}", f"{min(us):.3f}",
                 f"{fl / (mean * 1e-6) / 1e12:.2f}" if fl else "-"]
        for k in names:
            vals = [counters[i][k] for i in range(i0, i0 + n) if k in counters.get(i, {})]
            cells.append(f"{statistics.mean(vals):.4g}" if vals else "-")
        out.append("| " + " | ".join(cells) + " |")
    return "\n".join(out)


def shard_table(steps: int, warmup: int, settle: float) -> list[dict]:
    """One GPU's share of the 8192^3 product when C is split by rows over
    1, 2, 4 or 8 GPUs (M = 8192 / n, N = K = 8192, B whole): time sgemm_run
    on that shape.  Measures one GPU only; nothing here runs on several."""
    import dense_fp32_matrix_03_amd as sg
    from dense_fp32_matrix_03_amd import inputs

    rows = []
    for n in (1, 2, 4, 8):
        M = 8192 // n
        w = inputs.Workload(f"sgemm_{M}x8192x8192_uniform_seed4", M, 8192, 8192, "uniform", 4,
                            8192, 8192, 8192, "sampled")
        ms, finite = time_gpu(w, sg.VARIANTS["mfma"], steps, warmup, warm_seconds=settle)
        tf = w.flops / (ms * 1e-3) / 1e12
        r = {"share_of_gpus": n, "workload": w.name, "ms": round(ms, 5), "tflops": round(tf, 2),
             "pct_of_peak": round(100 * tf / PEAK_TFLOPS, 1), "output_finite": finite}
        print(json.dumps(r), flush=True)
        rows.append(r)
    return rows


HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bfloat16 matrix peak, published


def bf16x3_table(steps: int, warmup: int, settle: float, general: bool = False) -> list[dict]:
    """Time sgemm_run_bf16x3 (split + product, one call) on the square
    workloads and report single-precision-equivalent TFLOP/s (2 M N K per
    call) next to the bfloat16 matrix-core rate of its six piece products
    (6 * 2 M N K per call, whole call).  general: instead, at 2048^3 and
    8192^3, sgemm_run_bf16x3_ex with stored transposes (alpha = 1, beta = 0)
    and with alpha / beta (no transposes)."""
    import torch

    import dense_fp32_matrix_03_amd as sg
    from dense_fp32_matrix_03_amd import inputs

    rows = []
    stream = torch.cuda.current_stream()
    h = stream.cuda_stream
    ceiling = mfma_ceiling(1)
    print(json.dumps({"bf16_mfma_ceiling_tflops": round(ceiling, 1),
                      "pct_of_bf16_peak": round(100 * ceiling / BF16_PEAK_TFLOPS, 1)}), flush=True)

    def timed(step, w):
        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        t_end = time.perf_counter() + settle
        while time.perf_counter() < t_end:
            for _ in range(10):
                step()
            torch.cuda.synchronize()
        n = steps if w.flops > 1e12 else max(steps, 100)
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for _ in range(n):
            step()
        t1.record(stream)
        torch.cuda.synchronize()
        return n, t0.elapsed_time(t1) / n

    def report(w, n, ms, extra, dC, nbytes):
        tf = w.flops / (ms * 1e-3) / 1e12
        r = {"kernel": "bf16x3", "workload": w.name, **extra, "steps": n, "ms": round(ms, 5),
             "tflops_fp32_equivalent": round(tf, 2),
             "pct_of_fp32_peak": round(100 * tf / PEAK_TFLOPS, 1),
             "bf16_tflops": round(6 * tf, 1),
             "pct_of_bf16_peak": round(100 * 6 * tf / BF16_PEAK_TFLOPS, 1),
             "pct_of_bf16_ceiling": round(100 * 6 * tf / ceiling, 1),
             "workspace_bytes": nbytes,
             "output_finite": bool(torch.isfinite(dC[:, :w.N]).all().item())}
        print(json.dumps(r), flush=True)
        rows.append(r)

    names = (SECONDARY, HEADLINE) if general else ("sgemm_1024x1024x1024_uniform_seed1",
                                                   SECONDARY, HEADLINE)
    for name in names:
        w = inputs.BY_NAME[name]
        A, B = inputs.make_inputs(w)
        dA = torch.from_numpy(A).cuda()
        dB = torch.from_numpy(B).cuda()
        del A, B
        dC = torch.empty((w.M, w.ldc), dtype=torch.float32, device="cuda")
        nbytes = sg.sgemm_bf16x3_workspace_size(w.M, w.N, w.K)
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")

        def step():
            sg.sgemm_run_bf16x3(w.M, w.N, w.K, dA, w.lda, dB, w.ldb, dC, w.ldc, ws, nbytes, h)

        if not general:
            n, ms = timed(step, w)
            report(w, n, ms, {}, dC, nbytes)
            del dA, dB, dC, ws
            torch.cuda.empty_cache()
            continue
        # Square workloads: the stored transposes are the same arrays read
        # the other way (uniform entries either way).
        for ta, tb, alpha, beta in ((0, 1, 1.0, 0.0), (1, 1, 1.0, 0.0), (1, 0, 1.0, 0.0),
                                    (0, 0, 1.5, 0.5)):
            def step_ex(ta=ta, tb=tb, alpha=alpha, beta=beta):
                sg.sgemm_run_bf16x3_ex(ta, tb, w.M, w.N, w.K, alpha, dA, w.lda, dB, w.ldb,
                                       beta, dC, w.ldc, ws, nbytes, h)

            dC.fill_(0.0)
            n, ms = timed(step_ex, w)
            layout = ("T" if ta else "N") + ("T" if tb else "N")
            report(w, n, ms, {"entry": "sgemm_run_bf16x3_ex", "layout": layout,
                              "alpha": alpha, "beta": beta}, dC, nbytes)
        del dA, dB, dC, ws
        torch.cuda.empty_cache()
    return rows


def vector_add_table(steps: int, settle: float) -> list[dict]:
    """Effective bandwidth of vector_add, 3 * 4 * n bytes per call (A and B
    read, C written), as the blog counts it.  "resident": the same three
    arrays every call (at n = 2^24 they fit the 256 MB Infinity Cache, so
    this can exceed HBM); "rotating": four sets of arrays used in turn, so
    each call's operands were last touched four calls ago."""
    import torch

    import dense_fp32_matrix_03_amd as sg
    from dense_fp32_matrix_03_amd import inputs

    rows = []
    stream = torch.cuda.current_stream()
    h = stream.cuda_stream
    for n, mode in ((inputs.VECTOR_ADD_N, "resident"), (inputs.VECTOR_ADD_N, "rotating"),
                    (1 << 28, "resident")):
        nsets = 4 if mode == "rotating" else 1
        if n == inputs.VECTOR_ADD_N:
            A, B = inputs.vector_add_inputs(n)
        else:
            A, B = inputs.vector_add_inputs(n, "uniform", seed=1)
        sets = [(torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda(),
                 torch.empty(n, dtype=torch.float32, device="cuda")) for _ in range(nsets)]
        del A, B
        calls = [0]

        def step():
            a, b, c = sets[calls[0] % nsets]
            calls[0] += 1
            sg.vector_add(n, a, b, c, h)

        for _ in range(4):
            step()
        torch.cuda.synchronize()
        t_end = time.perf_counter() + settle
        while time.perf_counter() < t_end:
            for _ in range(20):
                step()
            torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for _ in range(steps):
            step()
        t1.record(stream)
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / steps
        gbs = 12.0 * n / (ms * 1e-3) / 1e9
        ok = bool(torch.isfinite(sets[0][2]).all().item())
        r = {"kernel": "vector_add", "n": n, "mode": mode, "sets": nsets, "steps": steps,
             "us": round(ms * 1e3, 3), "GB/s": round(gbs, 1),
             "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 1), "output_finite": ok}
        print(json.dumps(r), flush=True)
        rows.append(r)
        del sets
        torch.cuda.empty_cache()
    return rows


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description="single-precision GEMM throughput on MI355X")
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--variant", default="mfma", help="kernel variant (default: sgemm_run's)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--ladder", action="store_true",
                    help="time every rung of the vector-FMA ladder and the matrix-core "
                         "variants on --workload (default here: 2048^3), one JSON line each")
    ap.add_argument("--settle", type=float, default=0.3,
                    help="seconds of untimed calls before each --ladder timing")
    ap.add_argument("--table", action="store_true",
                    help="time every workload on the GPU and the oracle on the host (1 thread "
                         "and all threads; 8192^3 single-thread extrapolated from the "
                         "2048^3 rate) and print one JSON line per workload")
    ap.add_argument("--small", action="store_true",
                    help="time sgemm_run and every forced tile on small and medium products "
                         "(one JSON line each)")
    ap.add_argument("--shards", action="store_true",
                    help="time one GPU's share of 8192^3 split by rows of C over 1, 2, 4 "
                         "and 8 GPUs (single GPU; one JSON line each)")
    ap.add_argument("--general", action="store_true",
                    help="time the general form (transposes, alpha/beta, strided batches) "
                         "on a fixed set of cases, one JSON line each")
    ap.add_argument("--vector-add", action="store_true",
                    help="time vector_add (n = 2^24 with resident and rotating arrays, "
                         "n = 2^28) and print its effective bandwidth, one JSON line each")
    ap.add_argument("--bf16x3", action="store_true",
                    help="time sgemm_run_bf16x3 (single precision on the bfloat16 matrix "
                         "cores) at 1024^3, 2048^3 and 8192^3, one JSON line each")
    ap.add_argument("--bf16x3-general", action="store_true",
                    help="time sgemm_run_bf16x3_ex (stored transposes; alpha/beta) at "
                         "2048^3 and 8192^3, one JSON line each")
    ap.add_argument("--kscan", action="store_true",
                    help="time sgemm_run at M = N = 256 and 1024 over K = 32 .. 4096, two "
                         "floor cases and the five workloads, one JSON line each (with the "
                         "dispatch range each case timed, for --trace-summary)")
    ap.add_argument("--phases", action="store_true",
                    help="where a call's time goes: per-work-group phase timestamps "
                         "(sgemm_phase_times) on the workloads and the K-scan ends")
    ap.add_argument("--trace-summary", nargs="+", metavar=("TRACE_CSV", "CASES_JSONL"),
                    help="host only: summarise a rocprofv3 kernel trace (and optionally a "
                         "counter CSV) of a bench run per case: TRACE_CSV CASES_JSONL "
                         "[COUNTERS_CSV]")
    ap.add_argument("--write-hbm-counters", nargs=4,
                    metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="host only: write the HBM-traffic summary of the headline kernel "
                         "from four rocprofv3 counter CSVs (see profiles/)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device copy three times (the reference "
                         "kernel for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    a = ap.parse_args(argv)

    if a.write_hbm_counters:
        c = write_hbm_counters(*a.write_hbm_counters)
        print(json.dumps({k: c[k] for k in ("hbm_bytes_per_launch", "fetch_scale",
                                            "write_scale")}))
        return 0
    if a.trace_summary:
        if len(a.trace_summary) not in (2, 3):
            ap.error("--trace-summary takes TRACE_CSV CASES_JSONL [COUNTERS_CSV]")
        print(trace_summary(*a.trace_summary))
        return 0

    if a.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {a.gpus} is not supported "
              "(the product shards by rows of C with B replicated; not built here)",
              file=sys.stderr)
        return 2

    import torch

    import dense_fp32_matrix_03_amd as sg
    from dense_fp32_matrix_03_amd import inputs

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    torch.cuda.set_device(0)
    if a.copy_calibration:
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": COPY_BYTES, "launches": 3}), flush=True)
        return 0
    sg.sgemm_create()
    w = inputs.BY_NAME[a.workload]
    variant = sg.VARIANTS[a.variant] if a.variant in sg.VARIANTS else int(a.variant)
    if a.table:
        workload_table(variant)
        sg.sgemm_destroy()
        return 0
    if a.bf16x3 or a.bf16x3_general:
        bf16x3_table(a.steps, a.warmup, a.settle, general=a.bf16x3_general)
        sg.sgemm_destroy()
        return 0
    if a.vector_add:
        vector_add_table(a.steps, a.settle)
        sg.sgemm_destroy()
        return 0
    if a.phases:
        phase_table(a.settle)
        sg.sgemm_destroy()
        return 0
    if a.kscan:
        kscan_table(variant, max(a.steps, 200))
        sg.sgemm_destroy()
        return 0
    if a.small:
        small_table(max(a.steps, 100), min(a.settle, 0.1))
        sg.sgemm_destroy()
        return 0
    if a.shards:
        shard_table(a.steps, a.warmup, a.settle)
        sg.sgemm_destroy()
        return 0
    if a.general:
        general_table(a.settle)
        sg.sgemm_destroy()
        return 0
    if a.ladder:
        wl = w if a.workload != HEADLINE else inputs.BY_NAME[SECONDARY]
        ladder(wl, a.steps, a.warmup, a.settle)
        sg.sgemm_destroy()
        return 0

    ms, finite = time_gpu(w, variant, a.steps, a.warmup)
    tflops = w.flops / (ms * 1e-3) / 1e12
    out = {
        "metric": METRIC, "value": round(tflops, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "M": w.M, "N": w.N, "K": w.K, "lda": w.lda,
                   "ldb": w.ldb, "ldc": w.ldc, "dist": w.dist, "seed": w.seed,
                   "variant": sg.sgemm_variant_name(variant)},
        "pct_of_peak": round(100 * tflops / PEAK_TFLOPS, 2),
        "output_finite": finite,
    }
    traffic = measured_traffic(w.name)
    out["roofline"] = {"bound": "mfma", "achieved": round(tflops, 3), "peak": PEAK_TFLOPS,
                       "unit": "TFLOP/s", "frac": round(tflops / PEAK_TFLOPS, 4),
                       "traffic": traffic}
    if not a.no_secondary and w.name != SECONDARY:
        w2 = inputs.BY_NAME[SECONDARY]
        ms2, finite2 = time_gpu(w2, variant, 200, a.warmup, warm_seconds=0.3)
        t2 = w2.flops / (ms2 * 1e-3) / 1e12
        out["secondary"] = {"workload": w2.name, "value": round(t2, 3), "unit": "TFLOP/s",
                            "ms_per_step": round(ms2, 5),
                            "pct_of_peak": round(100 * t2 / PEAK_TFLOPS, 2),
                            "output_finite": finite2}
    sg.sgemm_destroy()
    out["cpu_baseline"] = None if a.no_cpu_baseline else cpu_baseline(w)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
