"""Inf and NaN in x (or X) where no stored entry reads them must not reach y
(or Y). y_i sums a_ij x_j over row i's stored entries only (the RgCSR page,
Section 3, row loop; the PPoPP'23 page, Section 4.3), so every schedule's
padding, masked edge entries and clamped re-reads must add exactly nothing,
not 0 * x. The matrices below use odd columns only and x holds NaN, +Inf and
-Inf at every even index (column 0 included: masked entries of a walk that
leaves long rows to the tiles once read X row 0). Every row is compared with
the oracle, which reads x only at stored entries."""
import numpy as np
import pytest
import torch

import oracle
import synth
import load_balanced_csr_amd as lb
from gpu_util import DevMatrix, check, dev, log

pytestmark = pytest.mark.gpu

_BAD = np.array([np.nan, np.inf, -np.inf])


def _odd_columns(w):
    """The same rows on columns 2c + 1 of a matrix twice as wide; x at the
    odd indices is w's x, at the even ones NaN / +Inf / -Inf in turn."""
    N = 2 * w.N
    x = np.empty(N, w.x.dtype)
    x[1::2] = w.x
    x[0::2] = np.resize(_BAD, w.N).astype(w.x.dtype)
    col = (2 * w.col_idx.astype(np.int64) + 1).astype(np.int32)
    return synth.Workload(w.name + "_odd", w.M, N, w.row_ptr, col, w.values, x, None, 1.0,
                          0.0, w.seed)


CASES = {
    # long rows: the walk + tile grid, masked edge partitions, tile reduce
    "bimodal": lambda: _odd_columns(synth.bimodal(M=40_000, n_long=40, long_len=8000)),
    # stream plan with the x window (fp64)
    "laplacian": lambda: _odd_columns(synth.laplacian(n=150)),
    # walk plan, rows cut between partitions
    "powerlaw": lambda: _odd_columns(synth.powerlaw(M=50_000, max_len=15_000)),
}

SPMV_VARIANTS = {
    "auto": dict(strategy="merge"),
    "walk": dict(strategy="merge", merge_reduce="walk"),
    "walk_no_tiles": dict(strategy="merge", merge_reduce="walk", long_row_tiles="off"),
    "binned": dict(strategy="binned"),
    "group": dict(strategy="group"),
}


@pytest.mark.parametrize("case", list(CASES))
def test_spmv_ignores_unread_nonfinite_x(case):
    w = CASES[case]()
    assert np.isnan(w.x[0]) and np.all(np.isfinite(w.x[1::2]))
    dt = w.values.dtype
    m = DevMatrix.of(w)
    y0 = synth.uniform(w.M, 5, synth.S_Y, dt.type)
    plans = [(name, m.plan(None, **opts)) for name, opts in SPMV_VARIANTS.items()]
    plans.append(("rgcsr", lb.Plan.rgcsr(m.rp, m.col, m.val, (w.M, w.N))))
    for name, plan in plans:
        for alpha, beta in ((1.0, 0.0), (-0.5, 2.0)):
            log("nonfinite spmv", case, name, alpha, beta)
            x = dev(w.x)
            y = dev(y0.copy()) if beta != 0 else torch.full(
                (w.M,), float("nan"), dtype=x.dtype, device="cuda")
            plan(x, y, alpha, beta)
            torch.cuda.synchronize()
            check(y.cpu().numpy(), w.row_ptr, w.col_idx, w.values, w.x, alpha, beta,
                  y0 if beta != 0 else None, "%s %s" % (case, name))
        plan.destroy()


@pytest.mark.parametrize("case", list(CASES))
def test_spmm_ignores_unread_nonfinite_x(case):
    w = CASES[case]()
    dt = w.values.dtype
    m = DevMatrix.of(w)
    plan = m.plan(None, strategy="merge")
    ks = (1, 4, 8, 16) if dt == np.float32 else (2, 4, 8)
    rng = np.random.default_rng(3)
    for k in ks:
        X = rng.uniform(-1, 1, (w.N, k)).astype(dt)
        X[0::2] = np.resize(_BAD, (w.N // 2, k)).astype(dt)
        Y0 = rng.uniform(-1, 1, (w.M, k)).astype(dt)
        need = lb.spmv_spmm_workspace_size(plan.handle, k)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
        for beta in (0.0, 0.5):
            log("nonfinite spmm", case, "k", k, "beta", beta, "tiles", plan.info["tile_rows"])
            Y = dev(Y0.copy())
            lb.spmv_exec_multi(plan.handle, dev(X), Y, 1.25, beta, ws if need else None)
            torch.cuda.synchronize()
            ref, scale = oracle.spmm(w.row_ptr, w.col_idx, w.values, X, 1.25, beta,
                                     Y0 if beta != 0 else None)
            ok, worst, idx = oracle.within_tolerance(Y.cpu().numpy(), ref, scale, 1.25, beta,
                                                     Y0 if beta != 0 else None,
                                                     row_ptr=w.row_ptr)
            assert ok, (case, k, beta, divmod(idx, k), worst)
    plan.destroy()
