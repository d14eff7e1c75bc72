"""COO input (entries sorted by row) on the GPU vs the COO oracle: the plan
derives the row offsets on the device and runs the CSR path; SpMV and SpMM
over such a plan, empty and trailing empty rows, no entries, and the order
check."""
import numpy as np
import pytest
import torch

import oracle
import synth
import load_balanced_csr_amd as lb
from gpu_util import dev, log, run

pytestmark = pytest.mark.gpu


def _coo_of(w):
    rows = np.repeat(np.arange(w.M, dtype=np.int32), np.diff(w.row_ptr))
    return rows, w.col_idx, w.values


def _check_coo(y, M, rows, cols, vals, x, alpha, beta, y0, what):
    ref, scale = oracle.spmv_coo(M, rows, cols, vals, x, alpha, beta, y0 if beta != 0 else None)
    counts = np.bincount(rows, minlength=M) if rows.size else np.zeros(M, np.int64)
    rp = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)   # only marks empty rows
    ok, worst, idx = oracle.within_tolerance(y, ref, scale, alpha, beta,
                                             y0 if beta != 0 else None, row_ptr=rp)
    assert ok, "%s: row %d y=%r ref=%r worst=%.3g" % (what, idx, y[idx], ref[idx], worst)


OPTS = {"auto": dict(), "merge8_walk": dict(strategy="merge", items_per_thread=8,
                                            merge_reduce="walk"),
        "binned": dict(strategy="binned")}


@pytest.mark.parametrize("opt", list(OPTS))
def test_coo_workloads(opt):
    for name, w in (("tiny", synth.tiny()), ("laplacian", synth.laplacian(n=120)),
                    ("powerlaw", synth.powerlaw(M=30_000, max_len=10_000)),
                    ("bimodal", synth.bimodal(M=20_000, n_long=8, long_len=5000))):
        rows, cols, vals = _coo_of(w)
        plan = lb.Plan.coo(dev(rows), dev(cols), dev(vals), (w.M, w.N), **OPTS[opt])
        y0 = synth.uniform(w.M, 77, synth.S_Y, vals.dtype.type)
        for alpha, beta in ((1.0, 0.0), (1.5, 0.5)):
            log("coo", name, opt, alpha, beta)
            y = run(plan, w.x, alpha, beta, y0 if beta != 0 else None, vals.dtype.type)
            _check_coo(y, w.M, rows, cols, vals, w.x, alpha, beta, y0, "%s/%s" % (name, opt))
        plan.destroy()


def test_coo_edges():
    # trailing and leading empty rows, a row spanning several partitions,
    # repeated positions (they add), no entries at all
    rng = np.random.default_rng(3)
    M, N = 5000, 700
    rows = np.sort(np.concatenate([rng.integers(10, 4000, 20_000), np.full(3000, 2500)]))
    cols = rng.integers(0, N, rows.size).astype(np.int32)
    cols[:50] = 5                                   # repeated (row, col) pairs
    rows = rows.astype(np.int32)
    for dt in (np.float32, np.float64):
        vals = rng.uniform(-1, 1, rows.size).astype(dt)
        x = rng.uniform(-1, 1, N).astype(dt)
        y0 = rng.uniform(-1, 1, M).astype(dt)
        plan = lb.Plan.coo(dev(rows), dev(cols), dev(vals), (M, N))
        for alpha, beta in ((1.0, 0.0), (-2.0, 1.0)):
            y = run(plan, x, alpha, beta, y0 if beta != 0 else None, dt)
            _check_coo(y, M, rows, cols, vals, x, alpha, beta, y0, "edges")
        # SpMM over the same plan
        X = rng.uniform(-1, 1, (N, 4)).astype(dt)
        Y = torch.full((M, 4), float("nan"), dtype=torch.float32 if dt == np.float32
                       else torch.float64, device="cuda")
        plan.exec_multi(dev(X), Y, 1.0, 0.0)
        torch.cuda.synchronize()
        for c in range(4):
            _check_coo(Y[:, c].cpu().numpy(), M, rows, cols, vals, X[:, c].copy(), 1.0, 0.0, None,
                       "edges spmm col %d" % c)
        plan.destroy()
    e32 = torch.empty(0, dtype=torch.int32, device="cuda")
    plan = lb.Plan.coo(e32, e32, torch.empty(0, device="cuda"), (7, 3))
    y = run(plan, np.ones(3, np.float32), 1.0, 0.0)
    assert np.array_equal(y, np.zeros(7, np.float32))
    plan.destroy()


def test_coo_order_check():
    rows = dev(np.array([0, 2, 1, 3], np.int32))     # out of order
    cols = dev(np.array([0, 1, 2, 3], np.int32))
    vals = dev(np.ones(4, np.float32))
    with pytest.raises(lb.SpmvError) as e:
        lb.Plan.coo(rows, cols, vals, (4, 4))
    assert e.value.status == 6
    with pytest.raises(lb.SpmvError) as e:           # a row index >= M
        lb.Plan.coo(dev(np.array([0, 1, 2, 4], np.int32)), cols, vals, (4, 4))
    assert e.value.status == 6
