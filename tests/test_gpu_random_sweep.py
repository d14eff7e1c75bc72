"""Seeded random sweep across features: for each seed a matrix of random
shape and row-length mix (uniform, Zipf tail, a few very long rows, many
empty rows; duplicate and unsorted columns in some), random dtype, alpha and
beta, run through every schedule and input form the library has -- auto,
merge-path walk in both dispatch orders, stream where it applies, x slabs,
binned as one grid and per bin on streams, group-mapped, row-grouped, COO,
transposed -- and SpMM with a random k, each against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import synth
import load_balanced_csr_amd as lb
from gpu_util import check, dev, log

pytestmark = pytest.mark.gpu

SEEDS = list(range(48))


def _matrix(seed):
    rng = np.random.default_rng(1000 + seed)
    kind = ["uniform", "zipf", "long", "empty"][seed % 4]
    M = int(rng.choice([1, 7, 300, 5000, 40000, 90000], p=[.05, .1, .15, .25, .3, .15]))
    if kind in ("zipf", "long"):              # room for long rows
        N = int(rng.choice([30000, 120000, 1_500_000]))
    else:
        N = int(rng.choice([1, 13, 2000, 30000, 120000], p=[.1, .1, .3, .3, .2]))
    if kind == "uniform":
        L = rng.integers(0, 40, M)
    elif kind == "zipf":
        L = np.minimum(rng.zipf(1.6, M), 5000)
    elif kind == "long":
        L = rng.integers(0, 5, M)
        L[rng.integers(0, M, max(1, M // 500))] = rng.integers(2000, 20000)
    else:
        L = np.where(rng.random(M) < 0.7, 0, rng.integers(1, 60, M))
    L = np.minimum(L, N).astype(np.int64)
    dt = np.float64 if seed % 3 == 0 else np.float32
    w = synth.random_csr(M, N, L, 77 + seed, dt)
    col = w.col_idx.copy()
    if seed % 5 == 1 and col.size:            # duplicates: repeat a neighbour's column
        dup = rng.random(col.size) < 0.1
        col[1:][dup[1:]] = col[:-1][dup[1:]]
    if seed % 5 == 2 and col.size:            # unsorted within rows
        for r in range(M):
            a, b = w.row_ptr[r], w.row_ptr[r + 1]
            if b - a > 1:
                col[a:b] = rng.permutation(col[a:b])
    alpha = float(rng.choice([1.0, -0.5, 2.25]))
    beta = float(rng.choice([0.0, 0.0, 0.5, -1.0]))
    y0 = synth.uniform(M, seed, synth.S_Y, dt)
    return w.row_ptr, col, w.values, w.x, y0, M, N, dt, alpha, beta, rng


def _variants(rng):
    v = {
        "auto": dict(),
        "walk_partition": dict(strategy="merge", merge_reduce="walk", dispatch_order="partition",
                               items_per_thread=int(rng.choice([4, 8, 16]))),
        "walk_column": dict(strategy="merge", merge_reduce="walk", dispatch_order="column",
                            items_per_thread=int(rng.choice([4, 7, 8, 16]))),
        "binned": dict(strategy="binned"),
        "binned_streams": dict(strategy="binned", bin_streams=int(rng.integers(1, 5))),
        "group": dict(strategy="group"),
        # x slabs forced on: the slab-major copy, its walk and the combine,
        # whatever the column order (duplicates, unsorted rows)
        "x_slabs": dict(strategy="merge", x_slabs="on"),
    }
    return v


@pytest.mark.parametrize("seed", SEEDS)
def test_random_sweep(seed):
    rp, col, val, x, y0, M, N, dt, alpha, beta, rng = _matrix(seed)
    tdt = torch.float32 if dt == np.float32 else torch.float64
    d_rp, d_col, d_val, d_x = dev(rp), dev(col), dev(val), dev(x)
    ref_y0 = y0 if beta != 0 else None

    def run_and_check(plan, what, transpose=False):
        n_out = N if transpose else M
        yin = y0 if not transpose else synth.uniform(N, seed, synth.S_Y, dt)
        y = dev(yin) if beta != 0 else torch.full((n_out,), float("nan"), dtype=tdt,
                                                  device="cuda")
        xin = x if not transpose else synth.uniform(M, seed + 1, synth.S_X, dt)
        plan(dev(xin), y, alpha, beta)
        torch.cuda.synchronize()
        yh = y.cpu().numpy()
        if transpose:
            ref, scale = oracle.spmv_t(N, rp, col, val, xin, alpha, beta,
                                       yin if beta != 0 else None)
            ok, worst, idx = oracle.within_tolerance(yh, ref, scale, alpha, beta,
                                                     yin if beta != 0 else None)
            assert ok, "%s: col %d y=%r ref=%r worst=%.3g" % (what, idx, yh[idx], ref[idx], worst)
        else:
            check(yh, rp, col, val, x, alpha, beta, ref_y0, what)

    log("sweep seed", seed, "M=%d N=%d nnz=%d %s alpha=%g beta=%g" % (M, N, col.size, dt.__name__,
                                                                       alpha, beta))
    for name, opts in _variants(rng).items():
        plan = lb.Plan(d_rp, d_col, d_val, (M, N), **opts)
        run_and_check(plan, "seed %d %s" % (seed, name))
        if name in ("auto", "walk_column"):
            k = int(rng.integers(1, 20))
            X = rng.uniform(-1, 1, (N, k)).astype(dt)
            Y0 = rng.uniform(-1, 1, (M, k)).astype(dt)
            Y = dev(Y0) if beta != 0 else torch.full((M, k), float("nan"), dtype=tdt,
                                                     device="cuda")
            plan.exec_multi(dev(X), Y, alpha, beta)
            torch.cuda.synchronize()
            Yh = Y.cpu().numpy()
            for c in {0, k - 1}:
                check(Yh[:, c].copy(), rp, col, val, X[:, c].copy(), alpha, beta,
                      Y0[:, c].copy() if beta != 0 else None, "seed %d %s spmm k=%d col %d"
                      % (seed, name, k, c))
        plan.destroy()
    # row-grouped copy, COO and transposed plans
    plan = lb.Plan.rgcsr(d_rp, d_col, d_val, (M, N), group_rows=int(rng.choice([1, 8, 64])))
    run_and_check(plan, "seed %d rgcsr" % seed)
    plan.destroy()
    rows = dev(np.repeat(np.arange(M, dtype=np.int32), np.diff(rp)))
    plan = lb.Plan.coo(rows, d_col, d_val, (M, N))
    run_and_check(plan, "seed %d coo" % seed)
    plan.destroy()
    plan = lb.Plan.transpose(d_rp, d_col, d_val, (M, N))
    run_and_check(plan, "seed %d transpose" % seed, transpose=True)
    plan.destroy()
