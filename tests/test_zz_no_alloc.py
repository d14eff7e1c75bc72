"""spmv_exec_noalloc (no plan, no device allocation: the library's own
scratch array) against the entry points it stands in for, spmv_plan_ex +
spmv_exec on a merge-path walk plan at the same partition size in partition
order without long-row tiles: the same partitions, kernels and fix-up, so y
must be equal bit for bit; and within the oracle's bound. Two calls in a row, the second on a
smaller input (the scratch keeps the first call's contents)."""
import numpy as np
import pytest
import torch

import oracle
import synth
import load_balanced_csr_amd as lb
from gpu_util import DevMatrix, dev, log

pytestmark = pytest.mark.gpu


def _as(w, dt):
    if w.values.dtype == dt:
        return w
    return synth.Workload(w.name, w.M, w.N, w.row_ptr, w.col_idx, w.values.astype(dt),
                          w.x.astype(dt), None if w.y0 is None else w.y0.astype(dt), w.alpha,
                          w.beta, w.seed)


def _y_start(w, beta, y0, tdt):
    if beta != 0.0:
        return dev(y0)
    return torch.full((w.M,), float("nan"), dtype=tdt, device="cuda")


def _both(w, alpha, beta, y0):
    tdt = torch.float32 if w.values.dtype == np.float32 else torch.float64
    m = DevMatrix.of(w)
    x = dev(w.x)
    ipt = 16 if w.values.dtype == np.float32 else 8
    plan = m.plan(None, strategy="merge", merge_reduce="walk", items_per_thread=ipt,
                  dispatch_order="partition", long_row_tiles="off")
    y_plan = _y_start(w, beta, y0, tdt)
    plan(x, y_plan, alpha, beta)
    y_na = _y_start(w, beta, y0, tdt)
    lb.spmv_exec_noalloc(m.rp, m.col, m.val, w.M, w.N, x, y_na, alpha, beta)
    torch.cuda.synchronize()
    plan.destroy()
    return y_plan.cpu().numpy(), y_na.cpu().numpy()


@pytest.mark.parametrize("dt", [np.float32, np.float64])
def test_noalloc_matches_the_plan_path_two_calls(dt):
    first = _as(synth.CONFIGS["powerlaw"](), dt)                  # full size
    second = _as(synth.bimodal(M=30_000, n_long=30, long_len=4000), dt)   # smaller
    for w in (first, second):
        y0 = synth.uniform(w.M, 5, synth.S_Y, dt)
        for alpha, beta in ((1.0, 0.0), (1.5, 0.5)):
            log("noalloc", w.name, np.dtype(dt).name, "M=%d nnz=%d" % (w.M, w.nnz), alpha, beta)
            y_plan, y_na = _both(w, alpha, beta, y0)
            assert np.array_equal(y_plan.view(np.uint8), y_na.view(np.uint8)), (w.name, alpha)
            yo = y0 if beta != 0.0 else None
            ref, scale = oracle.spmv(w.row_ptr, w.col_idx, w.values, w.x, alpha, beta, yo)
            ok, worst, idx = oracle.within_tolerance(y_na, ref, scale, alpha, beta, yo,
                                                     row_ptr=w.row_ptr)
            assert ok, (w.name, idx, worst)


def test_noalloc_empty_matrix_and_banded_size():
    # no entries: y = beta * y exactly
    rp = torch.zeros(9, dtype=torch.int32, device="cuda")
    e32 = torch.empty(0, dtype=torch.int32, device="cuda")
    ef = torch.empty(0, dtype=torch.float32, device="cuda")
    y = torch.arange(8, dtype=torch.float32, device="cuda")
    lb.spmv_exec_noalloc(rp, e32, ef, 8, 4, torch.ones(4, device="cuda"), y, 1.0, 0.5)
    torch.cuda.synchronize()
    assert torch.equal(y.cpu(), torch.arange(8, dtype=torch.float32) * 0.5)
    # the largest workload fits the scratch (1.03M partitions at T = 1024)
    w = synth.CONFIGS["banded"]()
    y_plan, y_na = _both(w, 1.0, 0.0, None)
    assert np.array_equal(y_plan.view(np.uint8), y_na.view(np.uint8))
    del w
    torch.cuda.empty_cache()
