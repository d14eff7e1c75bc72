"""Transposed SpMV (y = alpha * A^T x + beta * y from A in CSR) and CSC
input on the GPU vs the transposed oracle: rectangular matrices, empty rows
and columns, long rows (which become long columns), SpMM over the same
plan, and the checks on malformed input."""
import numpy as np
import pytest
import torch

import oracle
import synth
import load_balanced_csr_amd as lb
from gpu_util import dev, log, run

pytestmark = pytest.mark.gpu

OPTS = {"auto": dict(), "merge8_walk": dict(strategy="merge", items_per_thread=8,
                                            merge_reduce="walk"),
        "binned": dict(strategy="binned")}


def _check_t(y, w_rp, w_col, w_val, N, x, alpha, beta, y0, what):
    ref, scale = oracle.spmv_t(N, w_rp, w_col, w_val, x, alpha, beta, y0 if beta != 0 else None)
    ok, worst, idx = oracle.within_tolerance(y, ref, scale, alpha, beta,
                                             y0 if beta != 0 else None)
    assert ok, "%s: col %d y=%r ref=%r worst=%.3g" % (what, idx, y[idx], ref[idx], worst)
    # columns of A with no entries: exactly beta * y0
    empty = np.bincount(w_col, minlength=N) == 0
    want = (y0 * y0.dtype.type(beta)) if beta != 0 else np.zeros(N, y.dtype)
    assert np.array_equal(y[empty], want[empty]), what + ": empty columns"


def _rect(M, N, L, seed, dtype=np.float32):
    return synth.random_csr(M, N, np.minimum(L, N), seed, dtype)


@pytest.mark.parametrize("opt", list(OPTS))
def test_transpose_workloads(opt):
    rng = np.random.default_rng(8)
    cases = [("tiny", synth.tiny()), ("laplacian", synth.laplacian(n=100)),
             ("powerlaw", synth.powerlaw(M=20_000, max_len=6_000)),
             ("bimodal", synth.bimodal(M=20_000, n_long=6, long_len=5000)),
             ("wide", _rect(300, 9000, rng.integers(0, 80, 300), 5)),
             ("tall", _rect(9000, 300, rng.integers(0, 12, 9000), 6, np.float64))]
    for name, w in cases:
        plan = lb.Plan.transpose(dev(w.row_ptr), dev(w.col_idx), dev(w.values), (w.M, w.N),
                                 **OPTS[opt])
        assert plan.M == w.N and plan.N == w.M
        dt = w.values.dtype.type
        x = synth.uniform(w.M, 5, synth.S_X, dt)
        y0 = synth.uniform(w.N, 6, synth.S_Y, dt)
        for alpha, beta in ((1.0, 0.0), (-1.5, 0.5)):
            log("transpose", name, opt, "M=%d N=%d nnz=%d" % (w.M, w.N, w.nnz), alpha, beta)
            y = run(plan, x, alpha, beta, y0 if beta != 0 else None, dt)
            _check_t(y, w.row_ptr, w.col_idx, w.values, w.N, x, alpha, beta, y0, name + "/" + opt)
        plan.destroy()


def test_csc_input_and_spmm():
    # A (M x N) in CSC is the CSR of an N x M matrix B = A^T: A x = B^T x
    rng = np.random.default_rng(9)
    M, N = 4000, 2500
    B = _rect(N, M, rng.integers(0, 30, N), 11)          # CSR of A^T
    plan = lb.Plan.csc(dev(B.row_ptr), dev(B.col_idx), dev(B.values), (M, N))
    assert plan.M == M and plan.N == N
    x = rng.uniform(-1, 1, N).astype(np.float32)
    y = run(plan, x, 2.0, 0.0)
    _check_t(y, B.row_ptr, B.col_idx, B.values, M, x, 2.0, 0.0, None, "csc")
    X = rng.uniform(-1, 1, (N, 3)).astype(np.float32)
    Y = torch.full((M, 3), float("nan"), device="cuda")
    plan.exec_multi(dev(X), Y)
    torch.cuda.synchronize()
    for c in range(3):
        _check_t(Y[:, c].cpu().numpy(), B.row_ptr, B.col_idx, B.values, M, X[:, c].copy(), 1.0,
                 0.0, None, "csc spmm col %d" % c)
    plan.destroy()


def test_transpose_checks_and_empty():
    rp = dev(np.array([0, 2, 1, 3], np.int32))          # decreasing row_ptr
    col = dev(np.array([0, 1, 2], np.int32))
    val = dev(np.ones(3, np.float32))
    with pytest.raises(lb.SpmvError) as e:
        lb.Plan.transpose(rp, col, val, (3, 4))
    assert e.value.status == 6
    with pytest.raises(lb.SpmvError) as e:              # a column index >= N
        lb.Plan.transpose(dev(np.array([0, 1, 2, 3], np.int32)),
                          dev(np.array([0, 5, 1], np.int32)), val, (3, 4))
    assert e.value.status == 6
    # no entries: y = beta * y0 exactly, y not read when beta = 0
    e32 = torch.empty(0, dtype=torch.int32, device="cuda")
    plan = lb.Plan.transpose(dev(np.zeros(6, np.int32)), e32,
                             torch.empty(0, device="cuda"), (5, 9))
    y = run(plan, np.ones(5, np.float32), 1.0, 0.0)
    assert np.array_equal(y, np.zeros(9, np.float32))
    plan.destroy()


def test_transpose_long_columns_take_tiles():
    """A with 40 columns of 8,000 entries: A^T has long rows, so the
    transposed plan takes the long-row tiles (SpMV and SpMM). A is built
    from B = A^T (a bimodal matrix) on the host; y = A^T x = B x."""
    Bw = synth.bimodal(M=20_000, n_long=40, long_len=8000)
    rows = np.repeat(np.arange(Bw.M, dtype=np.int64), np.diff(Bw.row_ptr))
    order = np.lexsort((rows, Bw.col_idx))
    a_col = rows[order].astype(np.int32)
    a_val = Bw.values[order]
    a_rp = np.zeros(Bw.N + 1, np.int32)
    a_rp[1:] = np.cumsum(np.bincount(Bw.col_idx, minlength=Bw.N))
    plan = lb.Plan.transpose(dev(a_rp), dev(a_col), dev(a_val), (Bw.N, Bw.M),
                             strategy="merge", merge_reduce="walk")
    assert plan.M == Bw.M and plan.N == Bw.N
    assert plan.info["tile_rows"] > 0, plan.info
    y0 = synth.uniform(Bw.M, 6, synth.S_Y, np.float32)
    for alpha, beta in ((1.0, 0.0), (-1.5, 0.5)):
        log("transpose tiles", alpha, beta)
        y = run(plan, Bw.x, alpha, beta, y0 if beta != 0 else None)
        _check_t(y, a_rp, a_col, a_val, Bw.M, Bw.x, alpha, beta, y0, "transpose tiles")
    rng = np.random.default_rng(12)
    for k in (4, 8):
        X = rng.uniform(-1, 1, (Bw.N, k)).astype(np.float32)
        Y = torch.full((Bw.M, k), float("nan"), device="cuda")
        log("transpose tiles spmm k", k)
        plan.exec_multi(dev(X), Y)
        torch.cuda.synchronize()
        ref, scale = oracle.spmm(Bw.row_ptr, Bw.col_idx, Bw.values, X, 1.0, 0.0, None)
        ok, worst, idx = oracle.within_tolerance(Y.cpu().numpy(), ref, scale, 1.0, 0.0, None,
                                                 row_ptr=Bw.row_ptr)
        assert ok, (k, divmod(idx, k), worst)
    plan.destroy()
