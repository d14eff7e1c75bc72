"""Column-blocked tiles of long rows in merge-path walk plans: the interior
nonzeros of long rows are summed per block of x by the tile kernel, the
rest by the walk kernel, and the block partials added after the fix-up.
Every row against the oracle, bitwise reproducibility, exact row lengths,
and the cases the tiles must survive: unsorted columns, a misaligned x, an
entry count that is not a multiple of four, fp64, beta != 0, SpMM over the
same plan, and tiles switched off."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import DevMatrix, check, dev, log, run

pytestmark = pytest.mark.gpu


def _long_rows(M, N, n_long, long_len, seed, dt=np.float32, short=3, last_long=False):
    rng = np.random.default_rng(seed)
    L = np.full(M, short, np.int64)
    L[rng.choice(M, n_long, replace=False)] = long_len
    L[rng.choice(M, M // 20, replace=False)] = 0
    if last_long:
        L[-1] = long_len     # the array's last (partial) quad in a tile row
    w = synth.random_csr(M, N, L, seed + 1)
    if dt != np.float32:
        w = synth.Workload("long_f64", M, N, w.row_ptr, w.col_idx, w.values.astype(dt),
                           w.x.astype(dt), None, 1.0, 0.0, seed)
    return w


CASES = {
    # (M, N, long rows, their length): several blocks, ragged last block
    "small": lambda: _long_rows(6000, 30_001, 40, 9000, 1),
    "many_blocks": lambda: _long_rows(20_000, 200_000, 30, 60_000, 2),
    "odd_nnz": lambda: _long_rows(5001, 50_003, 11, 24_001, 3, short=5),
    "f64": lambda: _long_rows(8000, 24_000, 25, 15_000, 4, np.float64),
    # more tile rows than one workgroup's group, the last row among them,
    # an odd entry count
    "two_groups_last_row": lambda: _long_rows(4003, 40_000, 70, 12_345, 6, last_long=True),
    "f64_last_row": lambda: _long_rows(3001, 9_001, 9, 7_001, 7, np.float64, last_long=True),
}


@pytest.mark.parametrize("case", list(CASES))
def test_tiled_plans_match_the_oracle(case):
    w = CASES[case]()
    dt = w.values.dtype.type
    m = DevMatrix.of(w)
    plan = m.plan(None, strategy="merge", merge_reduce="walk")
    info = plan.info
    assert info["tile_rows"] > 0 and info["walk_partitions"] < info["n_partitions"], info
    y0 = synth.uniform(w.M, 9, synth.S_Y, dt)
    for alpha, beta in ((1.0, 0.0), (-1.5, 0.5)):
        log("tiles", case, info["tile_rows"], info["tile_blocks"], alpha, beta)
        yo = y0 if beta != 0 else None
        y = run(plan, w.x, alpha, beta, yo, dt)
        check(y, w.row_ptr, w.col_idx, w.values, w.x, alpha, beta, yo, "tiles %s" % case)
        y2 = run(plan, w.x, alpha, beta, yo, dt)
        assert np.array_equal(y.view(np.uint8), y2.view(np.uint8)), "not reproducible"
    # the same matrix without tiles: also within the bound
    off = m.plan(None, strategy="merge", merge_reduce="walk", long_row_tiles="off")
    assert off.info["tile_rows"] == 0
    y = run(off, w.x, 1.0, 0.0, None, dt)
    check(y, w.row_ptr, w.col_idx, w.values, w.x, 1.0, 0.0, None, "tiles off %s" % case)
    off.destroy()
    plan.destroy()


def test_tiled_row_lengths_exact():
    w = CASES["many_blocks"]()
    L = np.diff(w.row_ptr).astype(np.float32)
    m = DevMatrix(w.row_ptr, w.col_idx, np.ones(w.nnz, np.float32), w.M, w.N)
    plan = m.plan(None, strategy="merge", merge_reduce="walk")
    assert plan.info["tile_rows"] > 0
    y = run(plan, np.ones(w.N, np.float32), 1.0, 0.0)
    assert np.array_equal(y, L)
    plan.destroy()


def test_tiles_with_unsorted_columns_and_misaligned_x():
    w = CASES["small"]()
    rng = np.random.default_rng(5)
    col = w.col_idx.copy()
    for r in np.nonzero(np.diff(w.row_ptr) > 1000)[0]:
        a, b = w.row_ptr[r], w.row_ptr[r + 1]
        col[a:b] = rng.permutation(col[a:b])
    m = DevMatrix(w.row_ptr, col, w.values, w.M, w.N)
    plan = m.plan(None, strategy="merge", merge_reduce="walk")
    assert plan.info["tile_rows"] > 0
    y = run(plan, w.x, 1.0, 0.0)
    check(y, w.row_ptr, col, w.values, w.x, 1.0, 0.0, None, "unsorted")
    # x at a 4-byte offset: the x block is staged with plain loads
    buf = torch.zeros(w.N + 1, dtype=torch.float32, device="cuda")
    buf[1:] = dev(w.x)
    x = buf[1:]
    yd = torch.full((w.M,), float("nan"), device="cuda")
    plan(x, yd, 1.0, 0.0)
    torch.cuda.synchronize()
    check(yd.cpu().numpy(), w.row_ptr, col, w.values, w.x, 1.0, 0.0, None, "misaligned x")
    # SpMM tiles over the unsorted rows (columns outside a tile's X block
    # come from global X) and with X at a 4-byte offset (no tiles then)
    X = rng.uniform(-1, 1, (w.N, 8)).astype(np.float32)
    for off in (0, 1):
        Xb = torch.zeros(w.N * 8 + off, dtype=torch.float32, device="cuda")
        Xb[off:] = dev(X.reshape(-1))
        Xd = Xb[off:].view(w.N, 8)
        Y = torch.full((w.M, 8), float("nan"), device="cuda")
        plan.exec_multi(Xd, Y, 1.0, 0.0)
        torch.cuda.synchronize()
        ref, scale = oracle.spmm(w.row_ptr, col, w.values, X, 1.0, 0.0, None)
        ok, worst, idx = oracle.within_tolerance(Y.cpu().numpy(), ref, scale, 1.0, 0.0, None,
                                                 row_ptr=w.row_ptr)
        assert ok, ("unsorted spmm", off, divmod(idx, 8), worst)
    plan.destroy()


@pytest.mark.parametrize("case", list(CASES))
def test_spmm_over_a_tiled_plan(case):
    """SpMM on a plan with long-row tiles: k where the tiles run (16-byte
    lanes, X rows of at most 32 bytes) and where they do not, row strides
    past k, beta != 0, against the oracle on every element; then the SpMV of
    the same plan still right."""
    w = CASES[case]()
    dt = w.values.dtype.type
    m = DevMatrix.of(w)
    plan = m.plan(None, strategy="merge", merge_reduce="walk")
    assert plan.info["tile_rows"] > 0
    ks = (1, 3, 4, 8, 12, 16, 20) if dt == np.float32 else (1, 2, 4, 6, 8, 10)
    rng = np.random.default_rng(7)
    for k in ks:
        for ld_extra, beta in ((0, 0.0), (4, 0.5)):
            X = rng.uniform(-1, 1, (w.N, k)).astype(dt)
            Y0 = rng.uniform(-1, 1, (w.M, k)).astype(dt)
            tdt = torch.float32 if dt == np.float32 else torch.float64
            Xb = torch.full((w.N, k + ld_extra), float("nan"), dtype=tdt, device="cuda")
            Xb[:, :k] = dev(X)
            Yb = torch.full((w.M, k + ld_extra), float("nan"), dtype=tdt, device="cuda")
            if beta != 0:
                Yb[:, :k] = dev(Y0)
            log("spmm tiles", case, "k", k, "ld+", ld_extra, "beta", beta)
            plan.exec_multi(Xb[:, :k], Yb[:, :k], 1.5, beta)
            torch.cuda.synchronize()
            out = Yb.cpu().numpy()
            assert np.all(np.isnan(out[:, k:])), "columns past k written"
            ref, scale = oracle.spmm(w.row_ptr, w.col_idx, w.values, X, 1.5, beta,
                                     Y0 if beta != 0 else None)
            ok, worst, idx = oracle.within_tolerance(out[:, :k], ref, scale, 1.5, beta,
                                                     Y0 if beta != 0 else None,
                                                     row_ptr=w.row_ptr)
            assert ok, (case, k, ld_extra, beta, divmod(idx, k), worst)
    # and the SpMV after it still right (the SpMM rewrote the carry rows)
    y = run(plan, w.x, 1.0, 0.0, None, dt)
    check(y, w.row_ptr, w.col_idx, w.values, w.x, 1.0, 0.0, None, "spmv after spmm")
    plan.destroy()


@pytest.mark.parametrize("case", ["small", "two_groups_last_row"])
def test_spmv_unchanged_by_an_untiled_spmm(case):
    """The fix-up and the tiles' reduction share one launch and must write
    different rows; an SpMM without tiles (X rows of 12 bytes) walks every
    partition and rewrites the carry rows of the tile rows' interior
    partitions. The SpMV after it is bitwise the SpMV before it, every
    time, and right."""
    w = CASES[case]()
    m = DevMatrix.of(w)
    plan = m.plan(None, strategy="merge", merge_reduce="walk")
    assert plan.info["tile_rows"] > 0
    y0 = synth.uniform(w.M, 13, synth.S_Y, np.float32)
    y_before = run(plan, w.x, -1.25, 0.5, y0)
    check(y_before, w.row_ptr, w.col_idx, w.values, w.x, -1.25, 0.5, y0, "tiles before spmm")
    rng = np.random.default_rng(3)
    X = rng.uniform(-1, 1, (w.N, 3)).astype(np.float32)
    Y = torch.zeros((w.M, 3), dtype=torch.float32, device="cuda")
    log("tiles", case, "untiled spmm k 3, then spmv")
    plan.exec_multi(dev(X), Y, 1.0, 0.0)
    torch.cuda.synchronize()
    for _ in range(3):
        y = run(plan, w.x, -1.25, 0.5, y0)
        assert np.array_equal(y.view(np.uint8), y_before.view(np.uint8))
    plan.destroy()


def test_spmm_tile_row_groups():
    """The SpMM tile kernel takes 8, 16 or 32 rows a wave (the most that
    still leaves 1024 tiles). The cases above have few tiles (8 a wave); a
    matrix of ~190 long rows over 2.2M columns takes 16 at k = 4 (one
    sub-block a column block) and 32 at k = 8 (two), each against the
    oracle on every element, beta zero and not."""
    w = _long_rows(20_000, 2_200_000, 200, 45_000, 8)
    m = DevMatrix.of(w)
    plan = m.plan(None, strategy="merge", merge_reduce="walk")
    info = plan.info
    n, nb = info["tile_rows"], info["tile_blocks"]
    assert 128 < n <= 200, info   # some long rows fall among the empty ones

    def rows_per_wave(sub):
        for rw in (32, 16):
            if -(-n // (8 * rw)) * nb * sub >= 1024:
                return rw
        return 8

    assert (rows_per_wave(1), rows_per_wave(2)) == (16, 32), (n, nb)
    rng = np.random.default_rng(11)
    for k in (4, 8):
        X = rng.uniform(-1, 1, (w.N, k)).astype(np.float32)
        Y0 = rng.uniform(-1, 1, (w.M, k)).astype(np.float32)
        for beta in (0.0, 0.5):
            Y = dev(Y0.copy())
            log("spmm tile groups k", k, "beta", beta)
            plan.exec_multi(dev(X), Y, -0.75, beta)
            torch.cuda.synchronize()
            ref, scale = oracle.spmm(w.row_ptr, w.col_idx, w.values, X, -0.75, beta,
                                     Y0 if beta != 0 else None)
            ok, worst, idx = oracle.within_tolerance(Y.cpu().numpy(), ref, scale, -0.75, beta,
                                                     Y0 if beta != 0 else None,
                                                     row_ptr=w.row_ptr)
            assert ok, (k, beta, divmod(idx, k), worst)
    plan.destroy()
