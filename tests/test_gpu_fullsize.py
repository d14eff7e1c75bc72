"""The five workloads at full size, planned with the defaults bench.py times,
through both schedules: every row against the oracle, bitwise
reproducibility, and exact results on inputs whose answer is known."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import DevMatrix, check, dev, log, run

pytestmark = pytest.mark.gpu

FULL = ["tiny", "laplacian", "powerlaw", "bimodal", "banded"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_parity(name):
    log("generate", name)
    w = synth.CONFIGS[name]()
    dt = w.values.dtype.type
    ref, scale = oracle.spmv(w.row_ptr, w.col_idx, w.values, w.x, w.alpha, w.beta, w.y0)
    m = DevMatrix.of(w)
    for variant in (None, "static", "merge8", "merge8_walk", "merge8_xwin", "merge7", "binned"):
        log("run", name, variant or "auto", "M=%d nnz=%d" % (w.M, w.nnz))
        plan = m.plan(variant)
        y = run(plan, w.x, w.alpha, w.beta, w.y0, dt)
        ok, worst, idx = oracle.within_tolerance(y, ref, scale, w.alpha, w.beta, w.y0,
                                                 row_ptr=w.row_ptr)
        assert ok, (name, variant, idx, y[idx], ref[idx], scale[idx], worst)
        y2 = run(plan, w.x, w.alpha, w.beta, w.y0, dt)
        assert np.array_equal(y, y2), (name, variant, "not reproducible")
        plan.destroy()
        log("ok", name, variant or "auto", "worst/bound = %.3g" % worst)
    del m
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["powerlaw", "bimodal", "banded"])
def test_full_size_row_lengths_exact(name):
    """values = 1 and x = 1 give y = row length exactly (< 2^24): pins the row
    assignment, the segmented reduction, the carries and the fix-up."""
    w = synth.CONFIGS[name]()
    L = np.diff(w.row_ptr).astype(np.float32)
    m = DevMatrix(w.row_ptr, w.col_idx, np.ones(w.nnz, np.float32), w.M, w.N)
    # "static": the plan bench.py times (power-law: x slabs)
    for variant in (None, "static", "merge8", "merge8_walk", "binned"):
        log("lengths", name, variant)
        plan = m.plan(variant)
        y = run(plan, np.ones(w.N, np.float32), 1.0, 0.0)
        assert np.array_equal(y, L), (name, variant)
        plan.destroy()
    del m
    torch.cuda.empty_cache()


def test_full_size_laplacian_closed_forms():
    w = synth.laplacian()
    n = w.params["grid"]
    r, c = np.divmod(np.arange(w.M, dtype=np.int64), n)
    inner = (r > 0) & (r < n - 1) & (c > 0) & (c < n - 1)
    nbrs = 4 - (r == 0) - (r == n - 1) - (c == 0) - (c == n - 1)
    m = DevMatrix.of(w)
    for variant in ("merge8", "merge8_walk", "binned"):
        log("laplacian closed forms", variant)
        plan = m.plan(variant)
        y = run(plan, np.ones(w.M), 1.0, 0.0, dtype=np.float64)
        assert np.array_equal(y, (4 - nbrs).astype(np.float64))
        y = run(plan, (r * r + c * c).astype(np.float64), 1.0, 0.0, dtype=np.float64)
        assert np.all(y[inner] == -4.0)
        y = run(plan, r.astype(np.float64), 1.0, 0.0, dtype=np.float64)
        assert np.all(y[inner] == 0.0)
        plan.destroy()
