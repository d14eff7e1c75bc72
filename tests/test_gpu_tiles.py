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
    plan.destroy()


def test_spmm_over_a_tiled_plan():
    w = CASES["small"]()
    m = DevMatrix.of(w)
    plan = m.plan(None, strategy="merge", merge_reduce="walk")
    assert plan.info["tile_rows"] > 0
    X = synth.uniform(w.N * 4, 3, synth.S_X, np.float32).reshape(w.N, 4)
    Y = torch.full((w.M, 4), float("nan"), device="cuda")
    plan.exec_multi(dev(X), Y, 1.0, 0.0)
    torch.cuda.synchronize()
    Yh = Y.cpu().numpy()
    for c in range(4):
        check(Yh[:, c].copy(), w.row_ptr, w.col_idx, w.values, X[:, c].copy(), 1.0, 0.0, None,
              "spmm col %d" % c)
    # and the SpMV after it still right (the SpMM rewrote the carry rows)
    y = run(plan, w.x, 1.0, 0.0)
    check(y, w.row_ptr, w.col_idx, w.values, w.x, 1.0, 0.0, None, "spmv after spmm")
    plan.destroy()
