#!/usr/bin/env python3
"""Benchmark of the CSR SpMV hot path on one MI355X.

One step = one spmv_exec (y = alpha*A*x + beta*y, the whole hot path: the
merge-path kernel and, where rows cross partitions, its carry fix-up, or the
fused binned kernel) over the workload resident in HBM. The headline
workload (``--workload``, default: the 32M-row banded decay matrix, the
largest of the five) gives the JSON line's ``value``; the same steps are then
run on the other four workloads, each reported under ``per_config`` with its
own timing, roofline fraction, parity and CPU-oracle figures
(``--no-per-config`` skips them). Before every step
the caches are flushed on the same stream: a 1 GiB buffer is zero-filled,
then another 1 GiB buffer is summed with ordinary (cached) loads. The fill
alone would leave up to 256 MiB of dirty lines in the Infinity Cache whose
write-back then lands inside the timed call (measured: +6 to +12% on the
regular workloads); the cached read evicts them before it. Either way no
byte of the matrix is left in L2 or the Infinity Cache, so every step reads
it from HBM (``--no-flush`` times warm steps instead).

Timed region: K steps, each exec bracketed by a pair of HIP events (torch
events on the stream the library launches on) -> ``value`` and
``ms_per_step``. A second pass of K steps records HIP events that the
library places around its dominant kernel alone (spmv_exec_events) ->
``roofline.achieved``; keeping them out of the first pass keeps their
overhead out of ``value``.

Prints ONE JSON line. ``value`` is GFLOP/s (2 * nnz per step) over the mean
event-timed exec duration; ``roofline`` prices the dominant kernel against
MI355X's 8 TB/s HBM peak with the compulsory bytes (row_ptr, col_idx,
values, x, y) per launch; ``cpu_baseline`` times the CPU oracle on the host.
"""
import argparse
import ctypes
import hashlib
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "CSR SpMV GFLOP/s and achieved HBM GB/s (% of peak) on 1 MI355X"
WORKLOADS = {
    "tiny": "tiny fp32 CSR, 2,000 x 2,000, 5..15 entries per row",
    "laplacian": "fp64 5-point 2-D Laplacian, 2048 x 2048 grid (4,194,304 rows)",
    "powerlaw": "fp32 power-law rows (exponent 2.1, 1..100,000), 4,000,000^2, alpha 1.5 beta 0.5",
    "bimodal": "fp32 bimodal rows, 1,000,000^2: 1,000 x 50,000 + 5% empty + 3 per row",
    "banded": "fp32 banded decay matrix, 32,000,000 rows, 24..40 entries within |i-j| <= 1000",
}
KERNEL_SOURCES = ["merge_kernels.hip", "tile_exec.hpp", "binned_kernels.hip", "device_common.hpp",
                  "internal.hpp", "slab_kernels.hip"]
SPMM_SOURCES = ["spmm_kernels.hip", "device_common.hpp", "internal.hpp"]


def kernel_source_hash(files=KERNEL_SOURCES) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "load_balanced_csr_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


class HipEvents:
    """hipEvent_t handles from the HIP runtime torch has loaded."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self) -> int:
        e = ctypes.c_void_p()
        assert self.hip.hipEventCreate(ctypes.byref(e)) == 0
        return e.value

    def elapsed_ms(self, a: int, b: int) -> float:
        ms = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return ms.value

    def destroy(self, e: int):
        self.hip.hipEventDestroy(e)


def compulsory_bytes(w) -> int:
    s = w.values.dtype.itemsize
    b = 4 * (w.M + 1) + w.nnz * (4 + s) + w.N * s + w.M * s
    if w.beta != 0.0:
        b += w.M * s          # y is read as well as written
    return b


def load_traffic(workload: str, kernel: str, files=KERNEL_SOURCES):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken with the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        table = json.load(f)
    rec = table.get("%s/%s" % (workload, kernel))
    if not rec or rec.get("kernel_source_hash") != kernel_source_hash(files):
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(w, budget_s: float, y_gpu, fmt: str = "csr", allcores: bool = True):
    """The oracle as it stands, on one host core, repeated on the whole
    workload until the time budget is spent (at least once; the budget, 10 s
    by default, bounds the sample). Its result also checks the GPU's first
    exec (every row, the acceptance bound)."""
    import oracle
    try:
        all_cpus = os.sched_getaffinity(0)
        os.sched_setaffinity(0, {sorted(all_cpus)[0]})
    except (AttributeError, OSError):
        all_cpus = None
    times = []
    rows = (np.repeat(np.arange(w.M, dtype=np.int32), np.diff(w.row_ptr))
            if fmt == "coo" else None)
    t_end = time.perf_counter() + budget_s
    while True:
        t0 = time.perf_counter()
        if fmt == "coo":
            ref, scale = oracle.spmv_coo(w.M, rows, w.col_idx, w.values, w.x, w.alpha, w.beta,
                                         w.y0)
        elif fmt == "transpose":
            ref, scale = oracle.spmv_t(w.N, w.row_ptr, w.col_idx, w.values, w.x, w.alpha,
                                       w.beta, w.y0)
        else:
            ref, scale = oracle.spmv(w.row_ptr, w.col_idx, w.values, w.x, w.alpha, w.beta, w.y0)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() > t_end or len(times) >= 2000:
            break
    t = statistics.median(times)
    ok, worst, _ = oracle.within_tolerance(y_gpu, ref, scale, w.alpha, w.beta, w.y0,
                                           row_ptr=w.row_ptr if fmt != "transpose" else None)
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    res = {"value": round(2.0 * w.nnz / t / 1e9, 4), "unit": "GFLOP/s", "cores": 1,
           "kind": "oracle", "cpu": cpu, "host_cpus": os.cpu_count(),
           "sample": "whole workload (%d nnz), %d runs, median %.1f ms, fp64 accumulation"
                     % (w.nnz, len(times), t * 1e3),
           "GBps": round(compulsory_bytes(w) / t / 1e9, 3)}
    if fmt == "csr" and all_cpus and allcores:
        res["allcores"] = cpu_allcores(w, all_cpus)
    elif all_cpus:
        os.sched_setaffinity(0, all_cpus)
    return res, bool(ok), worst


def cpu_allcores(w, cpus, budget_s: float = 3.0):
    """A separately labelled figure, not the baseline: the same oracle loop
    run on disjoint row ranges (balanced by nonzeros) in one thread per core
    (the C calls release the interpreter lock)."""
    import concurrent.futures
    import oracle
    os.sched_setaffinity(0, cpus)
    n = len(cpus)
    rp = np.ascontiguousarray(w.row_ptr, dtype=np.int32)
    col = np.ascontiguousarray(w.col_idx, dtype=np.int32)
    cuts = np.searchsorted(rp.astype(np.int64), np.linspace(0, int(rp[-1]), n + 1), side="left")
    cuts[0], cuts[-1] = 0, w.M
    chunks = [np.arange(cuts[i], cuts[i + 1], dtype=np.int64) for i in range(n)
              if cuts[i + 1] > cuts[i]]
    y0 = w.y0 if w.beta != 0.0 else None
    run = lambda rows: oracle.spmv_rows(rows, rp, col, w.values, w.x, w.alpha, w.beta, y0)
    times = []
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(chunks)) as pool:
        t_end = time.perf_counter() + budget_s
        while True:
            t0 = time.perf_counter()
            list(pool.map(run, chunks))
            times.append(time.perf_counter() - t0)
            if time.perf_counter() > t_end or len(times) >= 200:
                break
    t = statistics.median(times)
    return {"value": round(2.0 * w.nnz / t / 1e9, 4), "unit": "GFLOP/s", "cores": n,
            "kind": "oracle rows split over threads (not the baseline)",
            "sample": "whole workload, %d runs, median %.2f ms" % (len(times), t * 1e3)}


class CacheFlush:
    """Evicts L2 and the 256 MiB Infinity Cache: zero-fill 1 GiB, then sum
    another 1 GiB with cached loads (which also writes back the fill's dirty
    lines before the next timed call rather than during it)."""

    def __init__(self, torch, dev):
        self.torch = torch
        self.wbuf = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        self.rbuf = torch.ones(1 << 28, dtype=torch.int32, device=dev)
        self.out = torch.zeros((), dtype=torch.int64, device=dev)

    def __call__(self):
        self.wbuf.zero_()
        self.torch.sum(self.rbuf, dim=(0,), dtype=self.torch.int64, out=self.out)


def read_ceiling(lb, torch, flush, gib: int = 2, reps: int = 10):
    """GB/s of the library's streaming-read probe over a 2 GiB buffer (each
    wavefront reads 4 KiB once), flushed and event-timed like the steps:
    the achievable read bandwidth to put beside the SpMV's."""
    buf = torch.ones(gib << 28, dtype=torch.int32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    ts = []
    for r in range(reps + 2):
        if flush is not None:
            flush()
        a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a_.record()
        lb.spmv_read_probe(buf, sink)
        b_.record()
        torch.cuda.synchronize()
        if r >= 2:
            ts.append(a_.elapsed_time(b_))
    nbytes = buf.numel() * 4
    del buf
    return round(nbytes / (statistics.median(ts) * 1e-3) / 1e9, 1)


def gather_sweep(reps: int = 10):
    """The x-gather ceiling of each layout the x slabs choose between: the
    library's gather probe (col_idx read once, x gathered at every column,
    nothing else) over 31M seeded uniform columns drawn from arrays of
    16 / 8 / 4 / 2 MB of fp32, and from 16 MB where the columns of
    workgroup b (4,096 consecutive entries) lie in slab b mod S of S
    slabs; flushed and event-timed like the steps. One JSON line."""
    import torch
    import load_balanced_csr_amd as lb
    dev = torch.device("cuda:0")
    flush = CacheFlush(torch, dev)
    nnz, N = 31 * 1024 * 1024, 4_000_000
    g = torch.Generator(device="cuda")
    g.manual_seed(1)
    x = torch.rand(N, device=dev, dtype=torch.float32, generator=g)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    rows = []

    def one(name, col):
        ms = timed_median(torch, flush, reps, lambda: lb.spmv_gather_probe(col, x, sink))
        rows.append({"x": name, "ms": round(ms, 4), "Ggathers_per_s": round(nnz / ms / 1e6, 1)})

    for nx in (N, N // 2, N // 4, N // 8):
        col = torch.randint(0, nx, (nnz,), device=dev, dtype=torch.int32, generator=g)
        one("uniform over %.0f MB" % (4 * nx / 1e6), col)
    blk = torch.arange(nnz, device=dev, dtype=torch.int64) // 4096
    for S in (8, 4, 16):
        slab = N // S
        col = (torch.randint(0, slab, (nnz,), device=dev, dtype=torch.int64, generator=g)
               + (blk % S) * slab).to(torch.int32)
        one("workgroup b in slab b mod %d (%.1f MB)" % (S, 4 * slab / 1e6), col)
    print(json.dumps({"gather_sweep": rows, "gathers": nnz,
                      "probe": "spmv_gather_probe, flushed, median of %d" % reps}), flush=True)


def slab_sweep(reps: int = 15):
    """x slabs on, off and auto (strategy merge) on seeded matrices whose x
    is wider than one XCD's L2 (power-law, uniform short rows with long
    spikes, skewed rows, random short rows in stream plans, and a stencil
    and a band, whose gathers stay near the row) or of 2..4 MB (random rows
    of 5..80 entries); flushed and event-timed like the steps. One JSON
    line."""
    import numpy as np
    import torch
    import synth
    import load_balanced_csr_amd as lb
    dev = torch.device("cuda:0")
    flush = CacheFlush(torch, dev)
    rng = np.random.default_rng(3)

    def mats():
        yield "powerlaw (4M rows, fp32)", synth.powerlaw()
        yield "powerlaw (2M rows, max 50,000)", synth.powerlaw(M=2_000_000, max_len=50_000)
        L = rng.integers(1, 16, 4_000_000)
        L[rng.choice(4_000_000, 2000, replace=False)] = 3000
        yield "uniform 1..15 + 2,000 rows of 3,000 (4M rows)", synth.random_csr(4_000_000, 4_000_000, L, 7)
        L = np.minimum((rng.pareto(1.5, 4_000_000) * 20 + 1).astype(np.int64), 5000)
        yield "skewed, Pareto 1.5, mean 58 (4M rows)", synth.random_csr(4_000_000, 4_000_000, L, 8)
        yield "uniform 5..15, stream plan (4M rows)", synth.random_csr(
            4_000_000, 4_000_000, rng.integers(5, 16, 4_000_000), 11)
        yield "uniform 20..40, stream plan (2M rows)", synth.random_csr(
            2_000_000, 2_000_000, rng.integers(20, 41, 2_000_000), 12)
        yield "uniform 40..80, x of 3 MB (750K rows)", synth.random_csr(
            750_000, 750_000, rng.integers(40, 81, 750_000), 13)
        yield "uniform 24..40, x of 2 MB (500K rows)", synth.random_csr(
            500_000, 500_000, rng.integers(24, 41, 500_000), 14)
        yield "uniform 5..15, x of 4 MB (1M rows)", synth.random_csr(
            1_000_000, 1_000_000, rng.integers(5, 16, 1_000_000), 15)
        yield "laplacian (fp64, 2048^2 grid)", synth.laplacian()
        yield "banded (4M rows)", synth.banded(M=4_000_000)

    rows = []
    for name, w in mats():
        rp, col, val, x = (torch.from_numpy(a).to(dev) for a in (w.row_ptr, w.col_idx, w.values, w.x))
        y = torch.zeros(w.M, device=dev, dtype=val.dtype)
        r = {"matrix": name, "nnz": w.nnz}
        for mode in ("auto", "off", "on"):
            p = lb.Plan(rp, col, val, (w.M, w.N), x_slabs=mode, strategy="merge",
                        static_matrix=True)
            info = p.info
            ms = timed_median(torch, flush, reps, lambda: p(x, y, 1.0, 0.0))
            r[mode + "_ms"] = round(ms, 4)
            if mode == "auto":
                r["auto_takes_slabs"] = info["x_slabs"]
                r["reduce"] = info["merge_reduce"]
            p.destroy()
        print("[bench] slab sweep %s" % json.dumps(r), file=sys.stderr, flush=True)
        rows.append(r)
        del rp, col, val, x, y
        torch.cuda.empty_cache()
    print(json.dumps({"slab_sweep": rows}), flush=True)


def read_sweep(reps: int = 10):
    """The streaming-read ceiling against buffer size (the library's read
    probe, each wavefront reading 4 KiB once, over 64 MiB .. 8 GiB) and a
    plain device copy (read + write) at three sizes; flushed and event-timed
    like the steps. One JSON line: the ceiling a kernel of a given size can
    reach, e.g. the 320 MiB of the laplacian workload."""
    import torch
    import load_balanced_csr_amd as lb
    dev = torch.device("cuda:0")
    flush = CacheFlush(torch, dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    rows = []
    for mib in (64, 128, 256, 320, 512, 1024, 2048, 8192):
        buf = torch.ones(mib << 18, dtype=torch.int32, device=dev)
        ms = timed_median(torch, flush, reps, lambda: lb.spmv_read_probe(buf, sink))
        rows.append({"read_MiB": mib, "us": round(ms * 1e3, 2),
                     "GBps": round(buf.numel() * 4 / ms / 1e6, 1)})
        del buf
    for mib in (32, 160, 320):
        a = torch.ones(mib << 18, dtype=torch.int32, device=dev)
        b = torch.empty_like(a)
        ms = timed_median(torch, flush, reps, lambda: b.copy_(a))
        rows.append({"copy_MiB": mib, "us": round(ms * 1e3, 2),
                     "GBps_read_plus_write": round(2 * a.numel() * 4 / ms / 1e6, 1)})
        del a, b
    print(json.dumps({"read_sweep": rows}), flush=True)


def calibrate_copy(mib: int, steps: int):
    """A plain copy kernel of known size (torch's device copy): reads and
    writes exactly mib MiB per launch. Under rocprofv3 --pmc FETCH_SIZE /
    WRITE_SIZE its per-dispatch counter values give the factor that turns
    those counters into bytes."""
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": n, "launches": steps}), flush=True)


METRIC_SPMM = "CSR SpMM (k right-hand sides) GFLOP/s and achieved HBM GB/s (% of peak) on 1 MI355X"


def spmm_bytes(w, k: int) -> int:
    """Compulsory bytes of Y = alpha*A*X + beta*Y: the matrix once, X (N x k)
    and Y (M x k) once each (Y twice when beta != 0)."""
    s = w.values.dtype.itemsize
    b = 4 * (w.M + 1) + w.nnz * (4 + s) + w.N * k * s + w.M * k * s
    if w.beta != 0.0:
        b += w.M * k * s
    return b


def run_spmm(args, w, torch, lb, dev):
    """SpMM mode (--rhs K > 1): one step = one spmv_exec_multi over the
    workload with K dense right-hand sides, flushed and event-timed like the
    SpMV steps. Prints one JSON line of its own metric."""
    import synth
    k = args.rhs
    dt = torch.float32 if w.values.dtype == np.float32 else torch.float64
    npdt = w.values.dtype
    rp = torch.from_numpy(w.row_ptr).to(dev)
    col = torch.from_numpy(w.col_idx).to(dev)
    val = torch.from_numpy(w.values).to(dev)
    Xh = synth.uniform(w.N * k, w.seed, synth.S_X, npdt).reshape(w.N, k)
    Y0h = (synth.uniform(w.M * k, w.seed, synth.S_Y, npdt).reshape(w.M, k)
           if w.beta != 0.0 else None)
    X = torch.from_numpy(Xh).to(dev)
    Y = torch.empty((w.M, k), dtype=dt, device=dev)
    Y0 = torch.from_numpy(Y0h).to(dev) if Y0h is not None else None
    plan = lb.Plan(rp, col, val, (w.M, w.N), strategy=args.strategy,
                   items_per_thread=args.items_per_thread)
    info = plan.info
    need = lb.spmv_spmm_workspace_size(plan.handle, k)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev) if need else None

    def step(ev0=None, ev1=None):
        lb.spmv_exec_multi(plan.handle, X, Y, w.alpha, w.beta, ws, None, ev0, ev1)

    if Y0 is not None:
        Y.copy_(Y0)
    else:
        Y.fill_(float("nan"))
    step()
    torch.cuda.synchronize()
    Y_first = Y.cpu().numpy()
    flush = None if args.no_flush else CacheFlush(torch, dev)
    hip = HipEvents()
    K, W = args.steps, args.warmup
    if Y0 is not None:
        Y.copy_(Y0)
    for _ in range(W):
        if flush is not None:
            flush()
        step()
    kb = [hip.create() for _ in range(K)]
    ke = [hip.create() for _ in range(K)]
    xb = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    xe = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    # timed region: K steps, events around each exec (every launch of it)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        if flush is not None:
            flush()
        xb[i].record()
        step()
        xe[i].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = [xb[i].elapsed_time(xe[i]) for i in range(K)]
    # second pass: the library's events, recorded by the main kernel's dispatch
    for i in range(K):
        if flush is not None:
            flush()
        step(kb[i], ke[i])
    torch.cuda.synchronize()
    kern_ms = [hip.elapsed_ms(kb[i], ke[i]) for i in range(K)]
    for e in kb + ke:
        hip.destroy(e)
    # every call must reproduce the first one bit for bit (beta != 0: one
    # more call from Y0)
    if w.beta != 0.0:
        Y.copy_(Y0)
        step()
        torch.cuda.synchronize()
    deterministic = bool(np.array_equal(Y.cpu().numpy().view(np.uint8),
                                        Y_first.view(np.uint8)))
    mean_ms = statistics.fmean(ms)
    mean_kern = statistics.fmean(kern_ms)
    Bc = spmm_bytes(w, k)
    # stream plans (partitions own whole rows) run the row-slot kernel, walk
    # plans the merge-slot kernel followed by the carry fix-up; walk plans
    # with long-row tiles also run the SpMM tiles when X rows are whole
    # 16-byte lanes of at most 32 bytes (the library's rule), and then the
    # library's events bracket the whole call
    s_el = X.element_size()
    tiled = (info["tile_rows"] > 0 and k % (16 // s_el) == 0 and k * s_el <= 32)
    kern = ("spmm_rows_kernel" if info["merge_reduce"] == "stream" else
            "spmm_tile_kernel + spmm_merge_kernel" if tiled else "spmm_merge_kernel")
    timed = ("events recorded by the main kernel's dispatch" if info["merge_reduce"] == "stream"
             else "events around the whole call (tiles, merge walk, carry fix-up, tile "
                  "reduction)" if tiled else
             "events recorded by the main kernel's dispatch (the carry fix-up after it is "
             "outside)")
    gbps = Bc / (mean_ms * 1e-3) / 1e9
    kern_gbps = Bc / (mean_kern * 1e-3) / 1e9
    out = {
        "metric": METRIC_SPMM,
        "value": round(2.0 * w.nnz * k / (mean_ms * 1e-3) / 1e9, 3),
        "unit": "GFLOP/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(mean_ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32" if dt == torch.float32 else "f64",
        "data": "synthetic",
        "config": {"workload": args.workload, "description": WORKLOADS[args.workload],
                   "rhs": k, "M": w.M, "N": w.N, "nnz": w.nnz, "alpha": w.alpha,
                   "beta": w.beta, "seed": w.seed, "merge_reduce": info["merge_reduce"],
                   "items_per_wave": info["items_per_wave"],
                   "cache": "warm" if flush is None else
                   "flushed before every step (1 GiB fill + 1 GiB cached read)"},
        "achieved_GBps": round(gbps, 2),
        "pct_hbm_peak": round(100.0 * gbps / HBM_PEAK_GBPS, 2),
        "compulsory_bytes": Bc,
        "roofline": {"bound": "hbm", "kernel": kern, "achieved": round(kern_gbps, 2),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(kern_gbps / HBM_PEAK_GBPS, 4),
                     "kernel_ms": round(mean_kern, 5),
                     "traffic": load_traffic("%s_k%d" % (args.workload, k), kern,
                                             SPMM_SOURCES),
                     "timed": timed},
        "exec_ms_median": round(statistics.median(ms), 5),
        "deterministic": deterministic,
        "wall_ms_per_step": round(wall * 1e3 / K, 5),
        "workspace_bytes": need,
        "kernel_source_hash": kernel_source_hash(SPMM_SOURCES),
    }
    # the X-row gathers alone (each nonzero's row of X, nothing else), in the
    # kernels' lane grouping, flushed and timed like the steps
    row_bytes = k * X.element_size()
    if row_bytes in (16, 32, 64, 128, 256) and X.is_contiguous() and w.nnz > 0:
        sink = torch.zeros(1, dtype=torch.int32, device=dev)
        g_ms = timed_median(torch, flush, min(K, 10),
                            lambda: lb.spmv_gather_rows_probe(col, X, sink))
        out["gather_rows_probe_ms"] = round(g_ms, 5)
        out["gather_rows_probe_G_per_s"] = round(w.nnz / (g_ms * 1e-3) / 1e9, 2)
    plan.destroy()
    ok = True
    if not args.no_cpu:
        import oracle
        print("[bench] cpu oracle baseline (spmm)", file=sys.stderr, flush=True)
        times = []
        t_end = time.perf_counter() + args.cpu_seconds
        while True:
            t1 = time.perf_counter()
            ref, scale = oracle.spmm(w.row_ptr, w.col_idx, w.values, Xh, w.alpha, w.beta, Y0h)
            times.append(time.perf_counter() - t1)
            if time.perf_counter() > t_end or len(times) >= 20:
                break
        t = statistics.median(times)
        ok, worst, _ = oracle.within_tolerance(Y_first, ref, scale, w.alpha, w.beta, Y0h,
                                               row_ptr=w.row_ptr)
        out["cpu_baseline"] = {"value": round(2.0 * w.nnz * k / t / 1e9, 4), "unit": "GFLOP/s",
                               "cores": 1, "kind": "oracle",
                               "sample": "whole workload with %d right-hand sides, %d runs, "
                                         "median %.1f ms" % (k, len(times), t * 1e3)}
        out["parity"] = {"ok": bool(ok), "worst_over_bound": round(worst, 5),
                         "checked": "first exec vs the oracle, every element"}
    print(json.dumps(out), flush=True)
    if not ok or deterministic is False:
        sys.exit(3)


TARGET_FRAC = {"laplacian": 0.70, "banded": 0.70, "powerlaw": 0.50, "bimodal": 0.50}


def kernel_of(info) -> str:
    if info["strategy"] == "binned":
        return "binned_spmv_kernel"
    if info["strategy"] == "rgcsr":
        return "rg_spmv_kernel"
    if info["strategy"] == "group":
        return "group_spmv_kernel"
    if info["merge_reduce"] == "stream":
        return "merge_stream_kernel"
    # long rows in column-blocked tiles: one grid walks the other partitions
    # and runs the tiles
    return "walk_tile_kernel" if info["tile_rows"] > 0 else "merge_spmv_kernel"


def timed_median(torch, flush, reps, fn):
    """Median ms of fn() over reps calls, each flushed and event-timed."""
    ts = []
    for r in range(reps + 2):
        if flush is not None:
            flush()
        a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a_.record()
        fn()
        b_.record()
        torch.cuda.synchronize()
        if r >= 2:
            ts.append(a_.elapsed_time(b_))
    return statistics.median(ts)


def probes(lb, torch, flush, w, tensors, ipt, reps):
    """The two measurement aids on this workload's own arrays: the gather
    probe (col_idx read once, x gathered at every column) and the stream
    probe (row_ptr, col_idx, values streamed in partitions of 64 * ipt units,
    y written; no x), flushed and event-timed like the steps."""
    rp, col, val, x = tensors
    s = w.values.dtype.itemsize
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    y = torch.empty(w.M, dtype=val.dtype, device="cuda")
    g_ms = timed_median(torch, flush, reps, lambda: lb.spmv_gather_probe(col, x, sink))
    ipt = ipt if ipt in (4, 8, 16) else 8
    s_ms = timed_median(torch, flush, reps,
                        lambda: lb.spmv_stream_probe(rp, col, val, y, ipt))
    s_bytes = 4 * (w.M + 1) + w.nnz * (4 + s) + w.M * s
    del y, sink
    return {"gather_probe_ms": round(g_ms, 5),
            "gather_probe_Ggathers_per_s": round(w.nnz / (g_ms * 1e-3) / 1e9, 2),
            "stream_probe_ms": round(s_ms, 5),
            "stream_probe_GBps": round(s_bytes / (s_ms * 1e-3) / 1e9, 1),
            "stream_probe_items_per_wave": 64 * ipt,
            "probes": "gather: col_idx read once and x gathered at every column in storage "
                      "order, nothing else; stream: row_ptr/col_idx/values streamed in the "
                      "plan's partition size and y written, no x (bytes: the compulsory ones "
                      "minus x)"}


def spmv_leg(args, w, torch, lb, dev, flush, K, W, cpu_seconds, headline):
    """Plan, parity, K flushed event-timed steps, the library's kernel events,
    determinism, the probes and the CPU oracle for one workload. Returns the
    full record (the headline's JSON line) and the per-config summary."""
    dt = torch.float32 if w.values.dtype == np.float32 else torch.float64
    rp = torch.from_numpy(w.row_ptr).to(dev)
    col = torch.from_numpy(w.col_idx).to(dev)
    val = torch.from_numpy(w.values).to(dev)
    x = torch.from_numpy(w.x).to(dev)
    y0 = torch.from_numpy(w.y0).to(dev) if w.y0 is not None else None
    y = torch.empty(w.M, dtype=dt, device=dev)
    torch.cuda.synchronize()

    # the benchmark's matrices never change after planning: it declares them
    # static, which lets the plan keep a copy of A (x slabs) where it pays
    popts = dict(strategy=args.strategy, items_per_thread=args.items_per_thread,
                 bin_streams=args.bin_streams, static_matrix=not args.mutable_matrix)
    if args.strategy == "rgcsr":
        assert args.format == "csr", "the row-grouped copy is built from CSR"

        def make_plan():
            return lb.Plan.rgcsr(rp, col, val, (w.M, w.N), group_rows=args.rg_group)
    elif args.format == "coo":
        rows = torch.from_numpy(np.repeat(np.arange(w.M, dtype=np.int32),
                                          np.diff(w.row_ptr))).to(dev)

        def make_plan():
            return lb.Plan.coo(rows, col, val, (w.M, w.N), **popts)
    elif args.format == "transpose":
        assert w.M == w.N, "the transposed benchmark uses square workloads"

        def make_plan():
            return lb.Plan.transpose(rp, col, val, (w.M, w.N), **popts)
    else:
        def make_plan():
            return lb.Plan(rp, col, val, (w.M, w.N), **popts)
    # planning cost (separate from the steps): median of 5 plan/destroy cycles
    plan_ms = []
    for _ in range(5):
        t0 = time.perf_counter()
        p_ = make_plan()
        plan_ms.append((time.perf_counter() - t0) * 1e3)
        p_.destroy()
    plan = make_plan()
    info = plan.info

    # first exec on fresh inputs; checked against the oracle below
    if y0 is not None:
        y.copy_(y0)
    else:
        y.fill_(float("nan"))
    plan(x, y, w.alpha, w.beta)
    torch.cuda.synchronize()
    y_first = y.cpu().numpy()

    hip = HipEvents()
    kb = [hip.create() for _ in range(K)]
    ke = [hip.create() for _ in range(K)]
    xb = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    xe = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    if y0 is not None:
        y.copy_(y0)
    for _ in range(W):
        if flush is not None:
            flush()
        plan(x, y, w.alpha, w.beta)
    # timed region: K steps, events around each exec only
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        if flush is not None:
            flush()
        xb[i].record()
        plan(x, y, w.alpha, w.beta)
        xe[i].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    exec_ms = [xb[i].elapsed_time(xe[i]) for i in range(K)]
    # second pass: the library's events around its dominant kernel
    for i in range(K):
        if flush is not None:
            flush()
        lb.spmv_exec_events(plan.handle, x, y, w.alpha, w.beta, kb[i], ke[i])
    torch.cuda.synchronize()
    kern_ms = [hip.elapsed_ms(kb[i], ke[i]) for i in range(K)]
    for e in kb + ke:
        hip.destroy(e)
    # every call must reproduce the first one bit for bit: beta = 0, the
    # last step's y; beta != 0 (y accumulates), one more call from y0
    if w.beta == 0.0:
        deterministic = bool(np.array_equal(y.cpu().numpy().view(np.uint8),
                                            y_first.view(np.uint8)))
    else:
        y.copy_(y0)
        plan(x, y, w.alpha, w.beta)
        torch.cuda.synchronize()
        deterministic = bool(np.array_equal(y.cpu().numpy().view(np.uint8),
                                            y_first.view(np.uint8)))
    # secondary figure: warm steps (no flush), events around each exec
    warm = []
    for i in range(min(K, 20)):
        a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a_.record()
        plan(x, y, w.alpha, w.beta)
        b_.record()
        warm.append((a_, b_))
    torch.cuda.synchronize()
    warm_ms = [a_.elapsed_time(b_) for a_, b_ in warm]
    plan.destroy()
    pr = probes(lb, torch, flush, w, (rp, col, val, x), info["items_per_thread"], min(K, 10)) \
        if args.format == "csr" and w.nnz > 0 else {}
    del rp, col, val, x, y0, y
    torch.cuda.empty_cache()

    mean_exec = statistics.fmean(exec_ms)
    mean_kern = statistics.fmean(kern_ms)
    Bc = compulsory_bytes(w)
    gflops = 2.0 * w.nnz / (mean_exec * 1e-3) / 1e9
    gbps_exec = Bc / (mean_exec * 1e-3) / 1e9
    kernel = kernel_of(info)
    achieved = Bc / (mean_kern * 1e-3) / 1e9
    traffic = load_traffic(args.workload if headline else w.name, kernel) \
        if args.format in ("csr", "coo") else None
    out = {
        "metric": METRIC,
        "value": round(gflops, 3),
        "unit": "GFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(mean_exec, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if dt == torch.float32 else "f64",
        "data": "synthetic",
        "config": {"workload": w.name, "description": WORKLOADS[w.name],
                   "M": w.M, "N": w.N, "nnz": w.nnz, "alpha": w.alpha, "beta": w.beta,
                   "seed": w.seed, "format": args.format, "strategy": info["strategy"],
                   "merge_reduce": info["merge_reduce"], "stream_lanes": info["stream_lanes"],
                   "items_per_wave": info["items_per_wave"],
                   "bin_streams": info["bin_streams"],
                   "dispatch_order": info["dispatch_order"],
                   # 1: the walk runs over the plan's slab-major copy of A
                   # (one column slab of x per XCD), then the combine
                   "static_matrix": not args.mutable_matrix,
                   "x_slabs": info["x_slabs"], "slab_segments": info["slab_segments"],
                   "cache": "warm" if flush is None else
                   "flushed before every step (1 GiB fill + 1 GiB cached read)"},
        "achieved_GBps": round(gbps_exec, 2),
        "pct_hbm_peak": round(100.0 * gbps_exec / HBM_PEAK_GBPS, 2),
        "compulsory_bytes": Bc,
        "roofline": {"bound": "hbm", "kernel": kernel, "achieved": round(achieved, 2),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "kernel_ms": round(mean_kern, 5),
                     # counters were taken on the CSR plan; a COO plan runs the
                     # same kernels on the same matrix, a transposed one on A^T
                     "traffic": traffic},
        "exec_ms_median": round(statistics.median(exec_ms), 5),
        "exec_ms_min": round(min(exec_ms), 5),
        "exec_ms_max": round(max(exec_ms), 5),
        "warm_exec_ms_median": round(statistics.median(warm_ms), 5),
        "warm_pct_hbm_peak": round(100.0 * Bc / (statistics.median(warm_ms) * 1e-3) / 1e9
                                   / HBM_PEAK_GBPS, 2),
        "deterministic": deterministic,
        "wall_ms_per_step": round(wall * 1e3 / K, 5),
        "plan_ms": round(statistics.median(plan_ms), 3),
        "plan_allocs": info["plan_allocs"],
        "plan_syncs": info["plan_syncs"],
        "kernel_source_hash": kernel_source_hash(),
    }
    out.update(pr)
    if info["strategy"] == "rgcsr":
        s_ = w.values.dtype.itemsize
        G = info["rgcsr_group"]
        out["config"]["rgcsr_group"] = G
        out["rgcsr_stored"] = info["rgcsr_stored"]
        # bytes the row-grouped layout itself moves: padded entries, row
        # lengths, group bases, x and y (the metric keeps the CSR bytes)
        out["format_bytes"] = (info["rgcsr_stored"] * (4 + s_) + 4 * w.M + 8 * (w.M // G + 2)
                               + (w.N + w.M) * s_ + (w.M * s_ if w.beta != 0.0 else 0))
    ok = True
    if not args.no_cpu:
        print("[bench] cpu oracle baseline: %s" % w.name, file=sys.stderr, flush=True)
        out["cpu_baseline"], ok, worst = cpu_baseline(w, cpu_seconds, y_first, args.format,
                                                      allcores=headline)
        out["cpu_baseline"]["gpu_speedup"] = round(out["value"] / out["cpu_baseline"]["value"], 1)
        out["parity"] = {"ok": ok, "worst_over_bound": round(worst, 5),
                         "checked": "first exec vs the oracle, every row"}
    summary = {k: out[k] for k in ("dtype", "ms_per_step", "exec_ms_median", "achieved_GBps",
                                   "pct_hbm_peak", "deterministic", "plan_ms", "plan_allocs",
                                   "plan_syncs")}
    summary.update({"M": w.M, "nnz": w.nnz, "GFLOPs": out["value"],
                    "strategy": info["strategy"], "merge_reduce": info["merge_reduce"],
                    "items_per_wave": info["items_per_wave"],
                    "dispatch_order": info["dispatch_order"], "x_slabs": info["x_slabs"],
                    "kernel": kernel,
                    "kernel_ms": out["roofline"]["kernel_ms"],
                    "roofline_frac": out["roofline"]["frac"],
                    "target_frac": TARGET_FRAC.get(w.name),
                    "traffic": traffic,
                    "traffic_over_bytes": round(traffic / Bc, 3) if traffic else None})
    for k in ("gather_probe_ms", "gather_probe_Ggathers_per_s", "stream_probe_ms",
              "stream_probe_GBps"):
        if k in out:
            summary[k] = out[k]
    if "parity" in out:
        summary["parity_ok"] = out["parity"]["ok"]
        summary["worst_over_bound"] = out["parity"]["worst_over_bound"]
        summary["cpu_oracle_GFLOPs"] = out["cpu_baseline"]["value"]
    return out, summary, ok and deterministic is not False


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="banded", choices=list(WORKLOADS))
    ap.add_argument("--no-per-config", action="store_true",
                    help="time the headline workload only")
    ap.add_argument("--strategy", default="auto",
                    choices=["auto", "merge", "binned", "rgcsr", "group"])
    ap.add_argument("--rg-group", type=int, default=0,
                    help="rows per group of the row-grouped CSR copy (--strategy rgcsr; 0 = 64)")
    ap.add_argument("--items-per-thread", type=int, default=0)
    ap.add_argument("--bin-streams", type=int, default=0,
                    help="binned schedule: one launch per bin over N streams (0 = one grid)")
    ap.add_argument("--no-flush", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--format", default="csr", choices=["csr", "coo", "transpose"],
                    help="coo: plan from row-sorted COO entries (row offsets derived on the "
                         "device); transpose: y = alpha A^T x + beta y (plan-time transpose)")
    ap.add_argument("--rhs", type=int, default=1, metavar="K",
                    help="K > 1: time the multi-vector form (SpMM) with K right-hand sides")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (counter calibration)")
    ap.add_argument("--gather-sweep", action="store_true",
                    help="only run the x-gather probe over the layouts x slabs choose between")
    ap.add_argument("--read-sweep", action="store_true",
                    help="only run the streaming-read probe over buffer sizes (and a copy)")
    ap.add_argument("--mutable-matrix", action="store_true",
                    help="plan without declaring the matrix static (no plan-time copy of A)")
    ap.add_argument("--slab-sweep", action="store_true",
                    help="only time x slabs on / off / auto on matrices with a wide x")
    args = ap.parse_args()

    if args.slab_sweep:
        return slab_sweep()
    if args.read_sweep:
        return read_sweep()
    if args.calibrate_copy:
        return calibrate_copy(args.calibrate_copy, args.steps)
    if args.gather_sweep:
        return gather_sweep()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import load_balanced_csr_amd as lb

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.init()
    dev = torch.device("cuda:0")
    print("[bench] generating %s" % args.workload, file=sys.stderr, flush=True)
    w = synth.CONFIGS[args.workload]()
    if args.rhs > 1:
        return run_spmm(args, w, torch, lb, dev)
    flush = None if args.no_flush else CacheFlush(torch, dev)
    K, W = args.steps, args.warmup
    print("[bench] %s: %d rows, %d nonzeros" % (w.name, w.M, w.nnz), file=sys.stderr, flush=True)
    out, summary, ok = spmv_leg(args, w, torch, lb, dev, flush, K, W, args.cpu_seconds, True)
    del w
    # achievable streaming-read bandwidth on this GPU, same flush and timing
    ceiling = read_ceiling(lb, torch, flush)
    out["read_ceiling_GBps"] = ceiling
    out["pct_of_read_ceiling"] = round(100.0 * out["achieved_GBps"] / ceiling, 2) if ceiling else None
    per = {args.workload: summary}
    if not args.no_per_config and args.format == "csr" and args.strategy == "auto":
        for name in WORKLOADS:
            if name == args.workload:
                continue
            print("[bench] per-config leg: %s" % name, file=sys.stderr, flush=True)
            try:
                wk = synth.CONFIGS[name]()
                _, summ, ok_k = spmv_leg(args, wk, torch, lb, dev, flush, K, W,
                                         min(args.cpu_seconds, 2.0), False)
                del wk
                ok = ok and ok_k
            except Exception as e:  # reported, and the run fails below
                summ = {"error": "%s: %s" % (type(e).__name__, e)}
                ok = False
            per[name] = summ
    out["per_config"] = {k: per[k] for k in WORKLOADS if k in per}
    print(json.dumps(out), flush=True)
    if not ok:
        sys.exit(3)


if __name__ == "__main__":
    main()
