"""Multi-vector SpMV (Y = alpha * A X + beta * Y) on the GPU vs the oracle:
every plan layout (partitions that end at row ends, and partitions that cut
rows and leave k-wide carries), k from 1 to beyond one 64-column block,
strided X and Y, empty and long rows, and the argument checks."""
import numpy as np
import pytest
import torch

import oracle
import synth
import load_balanced_csr_amd as lb
from gpu_util import DevMatrix, dev, log

pytestmark = pytest.mark.gpu

# plan options: stream layout (rows never cut) where rows allow it, and the
# walk layout (rows cut between partitions, carries) forced
PLANS = {
    "auto": dict(),
    "merge4": dict(strategy="merge", items_per_thread=4),
    "merge16": dict(strategy="merge", items_per_thread=16),
    "merge8_walk": dict(strategy="merge", items_per_thread=8, merge_reduce="walk"),
    "merge4_walk": dict(strategy="merge", items_per_thread=4, merge_reduce="walk"),
}


def _run(m, plan, X_h, alpha, beta, Y0_h=None, ldx=None, ldy=None):
    """One exec_multi with X, Y embedded in wider row-major buffers when
    ldx / ldy exceed k. Y starts as Y0 (beta != 0) or NaN (must not be read)."""
    dt = torch.float32 if X_h.dtype == np.float32 else torch.float64
    k = X_h.shape[1]
    ldx, ldy = ldx or k, ldy or k
    Xb = torch.full((m.N, ldx), float("nan"), dtype=dt, device="cuda")
    Xb[:, :k] = dev(X_h)
    Yb = torch.full((m.M, ldy), float("nan"), dtype=dt, device="cuda")
    if beta != 0:
        Yb[:, :k] = dev(Y0_h)
    X, Y = Xb[:, :k], Yb[:, :k]
    plan.exec_multi(X, Y, alpha, beta)
    torch.cuda.synchronize()
    out = Yb.cpu().numpy()
    assert np.all(np.isnan(out[:, k:])), "columns past k written"
    return out[:, :k]


def _check(Y, m, X_h, alpha, beta, Y0_h=None, what=""):
    ref, scale = oracle.spmm(m.row_ptr_h, m.col_h, m.val_h, X_h, alpha, beta,
                             Y0_h if beta != 0 else None)
    ok, worst, idx = oracle.within_tolerance(Y, ref, scale, alpha, beta,
                                             Y0_h if beta != 0 else None, row_ptr=m.row_ptr_h)
    if not ok:
        i, c = divmod(idx, Y.shape[1])
        raise AssertionError("%s: row %d col %d y=%r ref=%r scale=%r worst=%.3g" % (
            what, i, c, Y[i, c], ref[i, c], scale[i, c], worst))
    return worst


def _case(w, plan_name, ks, dtype=None, ld_extra=0, seed=3):
    dtype = dtype or w.values.dtype.type
    m = DevMatrix(w.row_ptr, w.col_idx, w.values.astype(dtype), w.M, w.N)
    plan = lb.Plan(m.rp, m.col, m.val, (m.M, m.N), **PLANS[plan_name])
    info = plan.info
    rng = np.random.default_rng(seed)
    for k in ks:
        X = rng.uniform(-1, 1, (m.N, k)).astype(dtype)
        Y0 = rng.uniform(-1, 1, (m.M, k)).astype(dtype)
        for alpha, beta in ((1.0, 0.0), (1.5, -0.5)):
            log("spmm", plan_name, info["merge_reduce"], "T=%d" % info["items_per_wave"],
                "M=%d N=%d nnz=%d k=%d ld+%d" % (m.M, m.N, len(m.col_h), k, ld_extra), alpha, beta)
            Y = _run(m, plan, X, alpha, beta, Y0, ldx=k + ld_extra if ld_extra else None,
                     ldy=k + 2 * ld_extra if ld_extra else None)
            _check(Y, m, X, alpha, beta, Y0, what="%s/%s/k%d" % (plan_name, info["merge_reduce"], k))
    plan.destroy()


@pytest.mark.parametrize("plan_name", list(PLANS))
@pytest.mark.parametrize("dtype", [np.float32, np.float64], ids=["f32", "f64"])
def test_random_shapes(plan_name, dtype):
    rng = np.random.default_rng(40)
    for trial in range(6):
        M = int(rng.choice([1, 7, 64, 65, 300, 2000]))
        N = int(rng.integers(1, 3000))
        kind = trial % 3
        if kind == 0:
            L = rng.integers(0, 12, M)
        elif kind == 1:
            L = np.minimum(rng.zipf(1.8, M), 3000)
        else:
            L = rng.integers(0, 3, M) * rng.integers(0, 60, M)
        L = np.minimum(L, N)
        w = synth.random_csr(M, N, L, 100 + trial, dtype)
        _case(w, plan_name, (1, 3, 8), dtype, seed=trial)


@pytest.mark.parametrize("plan_name", list(PLANS))
def test_scaled_workloads(plan_name):
    for name, w in (("laplacian", synth.laplacian(n=150)),
                    ("powerlaw", synth.powerlaw(M=20_000, max_len=8_000)),
                    ("bimodal", synth.bimodal(M=20_000, n_long=8, long_len=5000))):
        log("workload", name)
        _case(w, plan_name, (4, 16))


@pytest.mark.parametrize("plan_name", ["auto", "merge8_walk"])
def test_wide_and_strided(plan_name):
    """k beyond one 64-column block (65, 130), odd k, row strides > k."""
    w = synth.random_csr(3000, 2500, np.random.default_rng(5).integers(0, 20, 3000), 7)
    _case(w, plan_name, (5, 64, 65, 130))
    _case(w, plan_name, (1, 7, 33), ld_extra=3)


@pytest.mark.parametrize("plan_name", ["auto", "merge8_walk"])
def test_long_rows_and_empty(plan_name):
    # a row spanning many partitions; rows of T-1; all-empty stretches
    for lengths, N in (([100_000], 120_000), ([511] * 40, 600),
                       ([0] * 700 + [5000] + [0] * 300, 6000), ([0] * 50, 10)):
        L = np.asarray(lengths)
        w = synth.random_csr(len(L), N, L, len(L))
        _case(w, plan_name, (2, 9))


def test_deterministic():
    w = synth.powerlaw(M=30_000, max_len=10_000)
    m = DevMatrix.of(w)
    plan = lb.Plan(m.rp, m.col, m.val, (m.M, m.N), **PLANS["merge8_walk"])
    X = dev(synth.uniform(m.N * 8, 2, synth.S_X, np.float32).reshape(m.N, 8))
    Y1 = torch.empty((m.M, 8), dtype=torch.float32, device="cuda")
    Y2 = torch.empty_like(Y1)
    plan.exec_multi(X, Y1)
    plan.exec_multi(X, Y2)
    torch.cuda.synchronize()
    assert torch.equal(Y1, Y2)
    plan.destroy()


def test_argument_checks():
    w = synth.random_csr(100, 80, np.full(100, 5), 9)
    m = DevMatrix.of(w)
    plan = lb.Plan(m.rp, m.col, m.val, (m.M, m.N), **PLANS["merge4_walk"])
    X = torch.zeros((m.N, 4), device="cuda")
    Y = torch.zeros((m.M, 4), device="cuda")
    need = lb.spmv_spmm_workspace_size(plan.handle, 4)
    assert need > 0
    with pytest.raises(lb.SpmvError) as e:        # workspace missing
        lb.spmv_exec_multi(plan.handle, X, Y)
    assert e.value.status == 1
    short = torch.empty(need - 1, dtype=torch.uint8, device="cuda")
    with pytest.raises(lb.SpmvError) as e:
        lb.spmv_exec_multi(plan.handle, X, Y, workspace=short)
    assert e.value.status == 1
    big = torch.zeros((m.N + m.M, 4), device="cuda")   # X and Y overlap
    with pytest.raises(lb.SpmvError) as e:
        plan.exec_multi(big[: m.N], big[m.N - 1: m.N - 1 + m.M])
    assert e.value.status == 1
    lib = lb.load()                               # k < 0 an error, k = 0 a no-op
    assert lib.spmv_exec_multi(plan.handle, -1, X.data_ptr(), 4, Y.data_ptr(), 4, 1.0, 0.0,
                               None, 0, None) == 1
    assert lib.spmv_exec_multi(plan.handle, 0, X.data_ptr(), 4, Y.data_ptr(), 4, 1.0, 0.0,
                               None, 0, None) == 0
    assert lib.spmv_exec_multi(plan.handle, 4, X.data_ptr(), 3, Y.data_ptr(), 4, 1.0, 0.0,
                               None, 0, None) == 1    # ldx < k
    sp = lb.Plan(m.rp, m.col, m.val, (m.M, m.N), **PLANS["merge4"])
    assert sp.info["merge_reduce"] == "stream"
    assert lb.spmv_spmm_workspace_size(sp.handle, 64) == 0
    sp.destroy()
    plan.destroy()


def test_full_size_laplacian_k8():
    """fp64 Laplacian on the 2048 x 2048 grid with 8 right-hand sides, the
    launch the SpMM benchmark times, against the oracle on every row."""
    w = synth.laplacian()
    _case(w, "auto", (8,))


@pytest.mark.parametrize("name", ["powerlaw", "bimodal", "banded"])
def test_full_size_k8(name):
    """The full-size power-law (walk layout, column order), bimodal (walk
    layout, long-row tiles in its SpMV plan) and banded (stream layout, one
    workgroup per partition) matrices with 8 right-hand sides and the default
    plan, the launch the SpMM benchmark times: every row against the oracle."""
    log("generate", name)
    w = synth.CONFIGS[name]()
    _case(w, "auto", (8,))
    torch.cuda.empty_cache()


@pytest.mark.parametrize("kind", ["binned", "binned_streams", "group", "rgcsr"])
def test_spmm_on_other_schedules(kind):
    # spmv_exec_multi runs on the plan's merge-path partitions whatever
    # schedule spmv_exec uses: the SpMV schedule must not change the result
    w = synth.bimodal(M=20_000, n_long=15, long_len=4000)
    m = DevMatrix.of(w)
    if kind == "rgcsr":
        plan = lb.Plan.rgcsr(m.rp, m.col, m.val, (w.M, w.N), group_rows=32)
    elif kind == "binned_streams":
        plan = m.plan(None, strategy="binned", bin_streams=3)
    else:
        plan = m.plan(None, strategy=kind)
    rng = np.random.default_rng(11)
    for k, beta in ((1, 0.0), (6, 0.5), (40, -1.0)):
        X = rng.uniform(-1, 1, (w.N, k)).astype(np.float32)
        Y0 = rng.uniform(-1, 1, (w.M, k)).astype(np.float32)
        log("spmm on", kind, "k", k)
        Y = _run(m, plan, X, 1.5, beta, Y0)
        _check(Y, m, X, 1.5, beta, Y0, "%s k=%d" % (kind, k))
    plan.destroy()


def test_carry_chains_around_step_sizes():
    """Walk plan, rows whose carries run over n partitions for n just below,
    at and above the fix-up's step sizes (8 slices of 64 / kl partitions,
    kl the power of two covering k): chains that end inside a step, at its
    last partition and one past it, for k = 1, 8, 33, 64."""
    T = 512                                   # items_per_thread 8
    Ls = []
    for n in (7, 8, 9, 63, 64, 65, 511, 512, 513):
        for d in (-1, 0, 1):
            Ls += [T * n + d, 3, 0, 3]
    L = np.asarray(Ls)
    w = synth.random_csr(len(L), 300_000, L, 11)
    _case(w, "merge8_walk", (1, 8, 33, 64))
