"""x slabs: merge-path walk over a slab-major copy of A (one column slab of x
per XCD), then the combine of each row's slab sums. Every row against the
oracle, bitwise reproducibility, exact row lengths, the auto choice on a
wide-x power-law matrix, the cases the slabs must survive (empty rows, rows
in every slab, N smaller than the slab count, fp64, beta != 0), the plans
that must decline them (columns not sorted within a row), the values
refresh, and the other entry points over a slab plan (SpMM, other
schedules)."""
import numpy as np
import pytest
import torch

import oracle
import load_balanced_csr_amd as lb
import synth
from gpu_util import DevMatrix, check, dev, log, run

pytestmark = pytest.mark.gpu


def _random(M, N, L, seed, dt=np.float32):
    w = synth.random_csr(M, N, np.asarray(L), seed)
    if dt != np.float32:
        w = synth.Workload("random_f64", M, N, w.row_ptr, w.col_idx, w.values.astype(dt),
                           w.x.astype(dt), None, 1.0, 0.0, seed)
    return w


def _mixed_lengths(M, N, seed, long_len):
    rng = np.random.default_rng(seed)
    L = rng.integers(0, 12, M)
    L[rng.choice(M, M // 10, replace=False)] = 0
    L[rng.choice(M, 12, replace=False)] = long_len   # rows over every slab
    L[-1] = 0
    return np.minimum(L, N)


CASES = {
    "powerlaw": lambda: synth.powerlaw(M=30_000, max_len=8_000),
    "wide_x": lambda: _random(20_000, 3_000_000, _mixed_lengths(20_000, 3_000_000, 1, 4_000), 2),
    "f64": lambda: _random(25_000, 400_000, _mixed_lengths(25_000, 400_000, 3, 9_000), 4,
                           np.float64),
    "narrow_N": lambda: _random(3_000, 5, np.random.default_rng(5).integers(0, 6, 3_000), 6),
    "one_column": lambda: _random(2_000, 1, np.random.default_rng(7).integers(0, 2, 2_000), 8),
    "last_row_long": lambda: _random(4_097, 70_001,
                                     np.r_[np.random.default_rng(9).integers(1, 9, 4_096),
                                           [50_001]], 10),
}


def _slab_plan(m, **kw):
    return m.plan(None, strategy="merge", x_slabs="on", **kw)


# cases whose long rows the long-row tiles would take (tiles win over slabs)
NO_TILES = {"last_row_long"}


@pytest.mark.parametrize("case", list(CASES))
def test_slab_plans_match_the_oracle(case):
    w = CASES[case]()
    dt = w.values.dtype.type
    m = DevMatrix.of(w)
    plan = _slab_plan(m, long_row_tiles="off") if case in NO_TILES else _slab_plan(m)
    info = plan.info
    assert info["x_slabs"] == 1 and info["slab_segments"] > 0, info
    assert info["slab_segments"] <= w.nnz
    assert info["plan_allocs"] == 2 and info["plan_syncs"] == 1, info
    y0 = synth.uniform(w.M, 11, synth.S_Y, dt)
    for alpha, beta in ((1.0, 0.0), (-1.5, 0.5)):
        log("slabs", case, info["slab_segments"], alpha, beta)
        yo = y0 if beta != 0 else None
        y = run(plan, w.x, alpha, beta, yo, dt)
        check(y, w.row_ptr, w.col_idx, w.values, w.x, alpha, beta, yo, "slabs %s" % case)
        y2 = run(plan, w.x, alpha, beta, yo, dt)
        assert np.array_equal(y.view(np.uint8), y2.view(np.uint8)), "not reproducible"
    plan.destroy()


def test_tiles_take_precedence():
    """A plan whose long rows the column-blocked tiles take keeps no slabs,
    even when asked for them."""
    w = CASES["last_row_long"]()
    m = DevMatrix.of(w)
    plan = _slab_plan(m, merge_reduce="walk")
    info = plan.info
    assert info["tile_rows"] > 0 and info["x_slabs"] == 0 and info["plan_allocs"] == 1, info
    y = run(plan, w.x, 1.0, 0.0)
    check(y, w.row_ptr, w.col_idx, w.values, w.x, 1.0, 0.0, None, "tiles over slabs")
    plan.destroy()


def test_failed_slab_allocation_leaves_a_plain_plan(monkeypatch):
    """When the slab copy cannot be allocated the plan is made without it:
    one allocation, no slabs, and the result of the plain walk, bitwise."""
    w = CASES["wide_x"]()
    m = DevMatrix.of(w)
    monkeypatch.setenv("SPMV_TEST_FAIL_ALLOC", "2")
    plan = _slab_plan(m)
    monkeypatch.delenv("SPMV_TEST_FAIL_ALLOC")
    info = plan.info
    assert info["x_slabs"] == 0 and info["slab_segments"] == 0, info
    assert info["plan_allocs"] == 1 and info["plan_syncs"] == 1, info
    plain = m.plan(None, strategy="merge", x_slabs="off")
    for key in ("items_per_wave", "n_partitions", "merge_reduce", "dispatch_order"):
        assert plain.info[key] == info[key], key
    log("slabs", "failed allocation", info["items_per_wave"], info["n_partitions"])
    y = run(plan, w.x, 1.0, 0.0)
    check(y, w.row_ptr, w.col_idx, w.values, w.x, 1.0, 0.0, None, "no slab allocation")
    yp = run(plain, w.x, 1.0, 0.0)
    assert np.array_equal(y.view(np.uint8), yp.view(np.uint8))
    plan.destroy()
    plain.destroy()


def test_slab_segment_count():
    """A row has one segment per slab its columns reach: the count the plan
    reports equals the count from the columns (slab of column c: 8c // N)."""
    w = CASES["wide_x"]()
    m = DevMatrix.of(w)
    plan = _slab_plan(m)
    slab = (w.col_idx.astype(np.int64) * 8) // w.N
    row = np.repeat(np.arange(w.M), np.diff(w.row_ptr))
    expect = len(np.unique(row * 8 + slab))
    assert plan.info["slab_segments"] == expect
    plan.destroy()


def test_slab_row_lengths_exact():
    w = CASES["wide_x"]()
    m = DevMatrix(w.row_ptr, w.col_idx, np.ones(w.nnz, np.float32), w.M, w.N)
    plan = _slab_plan(m)
    assert plan.info["x_slabs"] == 1
    y = run(plan, np.ones(w.N, np.float32), 1.0, 0.0)
    assert np.array_equal(y, np.diff(w.row_ptr).astype(np.float32))
    plan.destroy()


def test_auto_takes_slabs_on_wide_powerlaw():
    """A power-law matrix whose x (6 MB) is wider than one XCD's L2, declared
    static: the automatic plan walks at T = 256 and takes slabs; off when
    asked, and never when the matrix is not declared static."""
    w = synth.powerlaw(M=1_500_000, max_len=20_000)
    m = DevMatrix.of(w)
    plan = m.plan(None, static_matrix=True)
    info = plan.info
    log("auto slabs", info["x_slabs"], info["items_per_wave"], info["merge_reduce"],
        info["slab_segments"], info["plan_allocs"], info["plan_syncs"])
    assert info["strategy"] == "merge" and info["merge_reduce"] == "walk", info
    assert info["x_slabs"] == 1 and info["plan_allocs"] == 2 and info["plan_syncs"] == 1, info
    y0 = w.y0
    y = run(plan, w.x, w.alpha, w.beta, y0)
    check(y, w.row_ptr, w.col_idx, w.values, w.x, w.alpha, w.beta, y0, "auto slabs")
    off = m.plan(None, x_slabs="off", static_matrix=True)
    assert off.info["x_slabs"] == 0 and off.info["plan_allocs"] == 1
    # not declared static: no copy of A, whatever the gathers
    borrowed = m.plan(None)
    assert borrowed.info["x_slabs"] == 0 and borrowed.info["plan_allocs"] == 1
    borrowed.destroy()
    y = run(off, w.x, w.alpha, w.beta, y0)
    check(y, w.row_ptr, w.col_idx, w.values, w.x, w.alpha, w.beta, y0, "slabs off")
    off.destroy()
    plan.destroy()


def test_auto_takes_slabs_on_wide_random_stream_plan():
    """Short rows (a stream plan) with uniform columns over a 4.8 MB x: no
    workgroup's columns fit an x window, so the automatic plan takes slabs;
    a stencil keeps its window and no slabs (the five workloads' choices
    are pinned in test_gpu_plan.py)."""
    M = 1_200_000
    w = synth.random_csr(M, M, np.random.default_rng(18).integers(5, 16, M), 19,
                         beta=0.25)
    m = DevMatrix.of(w)
    plan = m.plan(None, static_matrix=True)
    info = plan.info
    log("auto slabs, stream", info["x_slabs"], info["merge_reduce"], info["items_per_wave"],
        info["slab_segments"])
    assert info["merge_reduce"] == "stream" and info["x_slabs"] == 1, info
    y = run(plan, w.x, 1.0, 0.25, w.y0)
    check(y, w.row_ptr, w.col_idx, w.values, w.x, 1.0, 0.25, w.y0, "auto slabs, stream")
    y2 = run(plan, w.x, 1.0, 0.25, w.y0)
    assert np.array_equal(y.view(np.uint8), y2.view(np.uint8))
    plan.destroy()


def test_auto_slabs_for_mid_x_and_long_rows():
    """x of 1.1 MB, rows of 100..199 (mean length x x bytes >= 1e8): the
    automatic plan takes slabs; the same rows over 2 MB but of 5..15
    entries do not."""
    M = 280_000
    w = synth.random_csr(M, M, np.random.default_rng(20).integers(100, 200, M), 21)
    m = DevMatrix.of(w)
    plan = m.plan(None, static_matrix=True)
    info = plan.info
    log("auto slabs, mid x", info["x_slabs"], info["merge_reduce"], info["slab_segments"])
    assert info["x_slabs"] == 1, info
    y = run(plan, w.x, 1.0, 0.0)
    check(y, w.row_ptr, w.col_idx, w.values, w.x, 1.0, 0.0, None, "auto slabs, mid x")
    plan.destroy()
    M = 500_000
    w = synth.random_csr(M, M, np.random.default_rng(22).integers(5, 16, M), 23)
    plan = DevMatrix.of(w).plan(None, static_matrix=True)
    assert plan.info["x_slabs"] == 0, plan.info
    plan.destroy()


def test_unsorted_columns():
    """Columns out of order inside some rows: the automatic choice keeps no
    slabs (a run's end columns stray from its slab); forced on, the runs
    still partition every row, so the result is right."""
    w = CASES["wide_x"]()
    rng = np.random.default_rng(12)
    col = w.col_idx.copy()
    for r in np.nonzero(np.diff(w.row_ptr) > 100)[0][:5]:
        a, b = w.row_ptr[r], w.row_ptr[r + 1]
        col[a:b] = rng.permutation(col[a:b])
    sorted_auto = DevMatrix.of(w).plan(None, strategy="merge", static_matrix=True)
    assert sorted_auto.info["x_slabs"] == 1, sorted_auto.info
    sorted_auto.destroy()
    m = DevMatrix(w.row_ptr, col, w.values, w.M, w.N)
    auto = m.plan(None, strategy="merge", static_matrix=True)
    info = auto.info
    assert info["x_slabs"] == 0 and info["plan_allocs"] == 1, info
    y = run(auto, w.x, 1.0, 0.0)
    check(y, w.row_ptr, col, w.values, w.x, 1.0, 0.0, None, "unsorted, auto")
    auto.destroy()
    forced = _slab_plan(m)
    assert forced.info["x_slabs"] == 1
    y0 = synth.uniform(w.M, 17, synth.S_Y, np.float32)
    y = run(forced, w.x, -0.5, 2.0, y0)
    check(y, w.row_ptr, col, w.values, w.x, -0.5, 2.0, y0, "unsorted, slabs on")
    forced.destroy()


def test_repeated_columns_keep_slabs():
    """Equal neighbouring columns are sorted (non-decreasing): slabs stay on
    and the repeats add."""
    M, N = 2_000, 100_000
    rng = np.random.default_rng(13)
    L = rng.integers(1, 10, M)
    rp = synth.row_ptr_from_lengths(L.astype(np.int32))
    col = np.sort(rng.integers(0, N, int(rp[-1])).astype(np.int32))   # placeholder order
    for r in range(M):
        a, b = rp[r], rp[r + 1]
        c = np.sort(rng.integers(0, N, b - a))
        if b - a > 1:
            c[1] = c[0]
        col[a:b] = c
    val = rng.uniform(-1, 1, int(rp[-1])).astype(np.float32)
    x = rng.uniform(-1, 1, N).astype(np.float32)
    m = DevMatrix(rp, col, val, M, N)
    plan = _slab_plan(m)
    assert plan.info["x_slabs"] == 1
    y = run(plan, x, 1.0, 0.0)
    check(y, rp, col, val, x, 1.0, 0.0, None, "repeats")
    plan.destroy()


def test_update_values():
    """The slab copy holds the values of plan time until
    spmv_plan_update_values; then the new ones, bitwise as a fresh plan."""
    w = CASES["powerlaw"]()
    m = DevMatrix.of(w)
    plan = _slab_plan(m)
    assert plan.info["x_slabs"] == 1
    v2 = synth.uniform(w.nnz, 14, synth.S_VAL, np.float32)
    m.val.copy_(dev(v2))
    y = run(plan, w.x, 1.0, 0.0)
    check(y, w.row_ptr, w.col_idx, w.values, w.x, 1.0, 0.0, None, "before the refresh")
    plan.update_values(m.val)
    y = run(plan, w.x, 1.0, 0.0)
    check(y, w.row_ptr, w.col_idx, v2, w.x, 1.0, 0.0, None, "after the refresh")
    fresh = _slab_plan(m)
    y2 = run(fresh, w.x, 1.0, 0.0)
    assert np.array_equal(y.view(np.uint8), y2.view(np.uint8))
    # another array, on a plan without slabs too
    v3 = dev(synth.uniform(w.nnz, 15, synth.S_VAL, np.float32))
    for p in (plan, m.plan(None, strategy="merge", x_slabs="off")):
        p.update_values(v3)
        y = run(p, w.x, 1.0, 0.0)
        check(y, w.row_ptr, w.col_idx, v3.cpu().numpy(), w.x, 1.0, 0.0, None, "other array")
        p.destroy()
    fresh.destroy()


def test_update_values_refused_for_copies_in_other_layouts():
    w = CASES["narrow_N"]()
    m = DevMatrix.of(w)
    t = lb.Plan.transpose(m.rp, m.col, m.val, (w.M, w.N))
    with pytest.raises(Exception):
        t.update_values(m.val)
    t.destroy()


def test_other_entry_points_over_a_slab_plan():
    """SpMM and the other schedules run on the plan's own arrays: right
    whether or not the plan took slabs."""
    w = CASES["powerlaw"]()
    m = DevMatrix.of(w)
    plan = _slab_plan(m)
    assert plan.info["x_slabs"] == 1
    rng = np.random.default_rng(16)
    k = 4
    X = rng.uniform(-1, 1, (w.N, k)).astype(np.float32)
    Y = torch.full((w.M, k), float("nan"), device="cuda")
    plan.exec_multi(dev(X), Y, 1.0, 0.0)
    torch.cuda.synchronize()
    ref, scale = oracle.spmm(w.row_ptr, w.col_idx, w.values, X, 1.0, 0.0, None)
    ok, worst, idx = oracle.within_tolerance(Y.cpu().numpy(), ref, scale, 1.0, 0.0, None,
                                             row_ptr=w.row_ptr)
    assert ok, ("spmm over slabs", idx, worst)
    for s in ("binned", "group", "merge"):
        plan.set_strategy(s)
        y = run(plan, w.x, 1.0, 0.0)
        check(y, w.row_ptr, w.col_idx, w.values, w.x, 1.0, 0.0, None, "slab plan as " + s)
    plan.destroy()


def test_slabs_in_the_other_input_forms():
    """COO and transposed / CSC plans build through the same planning and
    take slabs the same way: forced on, each against its oracle."""
    w = CASES["powerlaw"]()
    rows = np.repeat(np.arange(w.M, dtype=np.int32), np.diff(w.row_ptr))
    m = DevMatrix.of(w)
    coo = lb.Plan.coo(dev(rows), m.col, m.val, (w.M, w.N), strategy="merge", x_slabs="on")
    assert coo.info["x_slabs"] == 1, coo.info
    y = run(coo, w.x, 1.0, 0.0)
    ref, scale = oracle.spmv_coo(w.M, rows, w.col_idx, w.values, w.x, 1.0, 0.0, None)
    ok, worst, idx = oracle.within_tolerance(y, ref, scale, 1.0, 0.0, None, row_ptr=w.row_ptr)
    assert ok, ("coo over slabs", idx, worst)
    coo.destroy()
    for kind in ("transpose", "csc"):
        if kind == "transpose":
            p = lb.Plan.transpose(m.rp, m.col, m.val, (w.M, w.N), strategy="merge",
                                  x_slabs="on")
        else:
            # A's CSR arrays are the CSC arrays of A^T (N x M)
            p = lb.Plan.csc(m.rp, m.col, m.val, (w.N, w.M), strategy="merge", x_slabs="on")
        assert p.info["x_slabs"] == 1, (kind, p.info)
        x = synth.uniform(w.M, 24, synth.S_X, np.float32)
        y0 = synth.uniform(w.N, 25, synth.S_Y, np.float32)
        y = run(p, x, 0.75, -0.5, y0)
        ref, scale = oracle.spmv_t(w.N, w.row_ptr, w.col_idx, w.values, x, 0.75, -0.5, y0)
        ok, worst, idx = oracle.within_tolerance(y, ref, scale, 0.75, -0.5, y0)
        assert ok, (kind, "over slabs", idx, worst)
        p.destroy()


def test_spmm_with_one_contiguous_column_is_the_spmv():
    """exec_multi with k = 1 and unit strides runs as spmv_exec, so on a
    slab plan it is bitwise the SpMV over the slab copy; a strided column
    (ldx = 3) takes the SpMM kernels and stays within the bound."""
    w = CASES["powerlaw"]()
    m = DevMatrix.of(w)
    plan = _slab_plan(m)
    assert plan.info["x_slabs"] == 1
    y = run(plan, w.x, 1.0, 0.0)
    Y = torch.full((w.M, 1), float("nan"), device="cuda")
    plan.exec_multi(dev(w.x).view(w.N, 1), Y, 1.0, 0.0)
    torch.cuda.synchronize()
    assert np.array_equal(Y.cpu().numpy()[:, 0].view(np.uint8), y.view(np.uint8))
    Xb = torch.full((w.N, 3), float("nan"), device="cuda")
    Xb[:, 0] = dev(w.x)
    Y2 = torch.full((w.M, 1), float("nan"), device="cuda")
    plan.exec_multi(Xb[:, :1], Y2, 1.0, 0.0)
    torch.cuda.synchronize()
    check(Y2.cpu().numpy()[:, 0].copy(), w.row_ptr, w.col_idx, w.values, w.x, 1.0, 0.0, None,
          "strided column")
    plan.destroy()
