"""HIP path vs the CPU oracle on small and scaled workloads, every schedule
variant, plus the plan's splits and bins vs the oracle's (exact)."""
import numpy as np
import pytest
import torch

import oracle
import synth
import load_balanced_csr_amd as lb
from gpu_util import VARIANTS, DevMatrix, check, dev, log, run

pytestmark = pytest.mark.gpu
ALL = list(VARIANTS)


def _csr(lengths, N, seed, dtype=np.float32):
    return synth.random_csr(len(lengths), N, np.asarray(lengths), seed, dtype)


def _case(w, variant, alpha, beta, dtype=None, what=""):
    dtype = dtype or w.values.dtype.type
    y0 = w.y0 if w.y0 is not None else synth.uniform(w.M, w.seed, synth.S_Y, dtype)
    m = DevMatrix.of(w)
    log("case", what, variant, "M=%d N=%d nnz=%d" % (w.M, w.N, w.nnz), alpha, beta)
    plan = m.plan(variant)
    y = run(plan, w.x, alpha, beta, y0 if beta != 0 else None, dtype)
    plan.destroy()
    return check(y, w.row_ptr, w.col_idx, w.values, w.x, alpha, beta,
                 y0 if beta != 0 else None, what="%s/%s" % (what, variant))


@pytest.mark.parametrize("variant", ALL)
def test_worked_example(variant, golden):
    rp = np.array(golden("rgcsr_worked_example.txt")["row_ptr"], dtype=np.int32)
    w = synth.random_csr(8, 8, np.diff(rp), 11)
    assert np.array_equal(w.row_ptr, rp)
    for alpha, beta in ((1.0, 0.0), (1.5, 0.5), (-2.0, 1.0)):
        _case(w, variant, alpha, beta, what="worked")


@pytest.mark.parametrize("variant", ALL)
def test_empty_first_and_last_rows(variant, golden):
    rp = np.array(golden("loadbalance_fig1_tiles.txt")["row_ptr"], dtype=np.int32)
    w = synth.random_csr(4, 6, np.diff(rp), 12)
    _case(w, variant, 1.0, 0.0, what="fig1")
    _case(w, variant, 1.5, 0.5, what="fig1")


@pytest.mark.parametrize("variant", ALL)
@pytest.mark.parametrize("dtype", [np.float32, np.float64], ids=["f32", "f64"])
def test_random_shapes(variant, dtype):
    rng = np.random.default_rng(100)
    for trial in range(10):
        M = int(rng.choice([1, 2, 7, 63, 64, 65, 257, 1000, 3000]))
        N = int(rng.integers(1, 5000))
        kind = trial % 4
        if kind == 0:
            L = rng.integers(0, 12, M)
        elif kind == 1:
            L = np.minimum(rng.zipf(1.8, M), 4000)
        elif kind == 2:
            L = np.where(rng.random(M) < 0.03, rng.integers(500, 5000, M), rng.integers(0, 4, M))
        else:
            L = rng.integers(0, 60, M) * (rng.random(M) < 0.5)
        L = np.minimum(L, N)
        w = synth.random_csr(M, N, L, 200 + trial, dtype)
        a, b = [(1.0, 0.0), (1.5, 0.5), (-0.75, 2.0), (0.0, 1.0)][trial % 4]
        y0 = synth.uniform(M, 300 + trial, synth.S_Y, dtype)
        w.y0 = y0
        _case(w, variant, a, b, dtype, what="random%d" % trial)


@pytest.mark.parametrize("variant", ALL)
def test_tiny_workload(variant):
    _case(synth.tiny(), variant, 1.0, 0.0, what="tiny")


SCALED = {
    "laplacian": lambda: synth.laplacian(n=200),
    "powerlaw": lambda: synth.powerlaw(M=60_000, max_len=20_000),
    "bimodal": lambda: synth.bimodal(M=60_000, n_long=20, long_len=6000),
    "banded": lambda: synth.banded(M=120_000, half_band=1000),
}


@pytest.mark.parametrize("variant", ALL)
@pytest.mark.parametrize("name", list(SCALED))
def test_scaled_workloads(variant, name):
    w = SCALED[name]()
    _case(w, variant, w.alpha, w.beta, what=name)


@pytest.mark.parametrize("variant", ALL)
def test_long_rows_and_partition_edges(variant):
    # one row of 100,000 nonzeros spans ~100 partitions; rows of T-1 put row
    # ends exactly on partition boundaries; a row of exactly T nonzeros too
    for lengths, N in (([100_000], 120_000), ([511] * 50, 600), ([1023] * 20 + [0, 1024, 0], 2000),
                       ([255] * 33 + [256, 257], 300), ([0] * 700 + [5000] + [0] * 300, 6000)):
        w = _csr(lengths, N, len(lengths))
        _case(w, variant, 1.0, 0.0, what="edges%d" % len(lengths))
        w.y0 = synth.uniform(w.M, 5, synth.S_Y, np.float32)
        _case(w, variant, 1.5, 0.5, what="edges%d" % len(lengths))


def _jumping_bands(M, N, dtype, seed):
    """Rows i hold columns c(i) + {-40, -20, -5, 0, 3, 17, 31} (inside [0, N)),
    where c(i) follows i, jumps forward by N/2, back below the start, then
    returns: column spans of workgroups that straddle a jump do not fit the
    x window, so those gather from global x."""
    offs = np.array([-40, -20, -5, 0, 3, 17, 31])
    i = np.arange(M)
    c = np.where(i < M // 4, i, np.where(i < M // 2, i + N // 2,
                 np.where(i < 3 * M // 4, i // 8, i)))
    cols = c[:, None] + offs[None, :]
    ok = (cols >= 0) & (cols < N)
    L = ok.sum(1)
    row_ptr = np.zeros(M + 1, dtype=np.int32)
    np.cumsum(L, out=row_ptr[1:])
    col_idx = cols[ok].astype(np.int32)
    values = synth.uniform(int(row_ptr[-1]), seed, synth.S_VAL, dtype)
    x = synth.uniform(N, seed, synth.S_X, dtype)
    return row_ptr, col_idx, values, x


@pytest.mark.parametrize("variant", ["merge7_xwin", "merge8_xwin", "merge4_xwin", "merge16_xwin"])
@pytest.mark.parametrize("dtype", [np.float32, np.float64], ids=["f32", "f64"])
def test_window_with_jumping_bands(variant, dtype):
    M, N = 400_000, 900_000
    rp, ci, va, x = _jumping_bands(M, N, dtype, 31)
    m = DevMatrix(rp, ci, va, M, N)
    plan = m.plan(variant)
    info = plan.info
    log("case jumps", variant, info["merge_reduce"], info["x_window"])
    # every (dtype, T) used here leaves LDS for a window beside the staging buffers
    room = True
    assert info["merge_reduce"] == "stream" and info["x_window"] == room, info
    y0 = synth.uniform(M, 32, synth.S_Y, dtype)
    for a, b in ((1.0, 0.0), (-1.5, 0.5)):
        y = run(plan, x, a, b, y0 if b != 0 else None, dtype)
        check(y, rp, ci, va, x, a, b, y0 if b != 0 else None, what="jumps/%s" % variant)
    plan.destroy()


@pytest.mark.parametrize("dtype,variant", [(np.float32, None), (np.float32, "merge7_xwin"),
                                           (np.float32, "merge8_xwin"), (np.float64, None),
                                           (np.float64, "merge8_xwin")],
                         ids=["f32-auto", "f32-merge7", "f32-merge8", "f64-auto", "f64-merge8"])
def test_window_three_bands(variant, dtype):
    """5-point stencil on a 2048 x 2048 grid: a workgroup's columns sit in
    three bands (rows above, own, below) 2048 apart, too wide together for one
    window interval but short each: the three-interval window is chosen."""
    w = synth.laplacian(n=2048)
    va, x = w.values.astype(dtype), w.x.astype(dtype)
    m = DevMatrix(w.row_ptr, w.col_idx, va, w.M, w.N)
    plan = m.plan(variant)
    info = plan.info
    log("case bands", variant, info["items_per_thread"], info["x_window_intervals"])
    assert info["merge_reduce"] == "stream" and info["x_window_intervals"] == 3, info
    y0 = synth.uniform(w.M, 33, synth.S_Y, dtype)
    for a, b in ((1.0, 0.0), (-1.5, 0.5)):
        y = run(plan, x, a, b, y0 if b != 0 else None, dtype)
        check(y, w.row_ptr, w.col_idx, va, x, a, b, y0 if b != 0 else None,
              what="bands/%s" % variant)
    plan.destroy()


@pytest.mark.parametrize("variant", ALL)
def test_no_entries(variant):
    # every row empty: y = beta * y exactly (0 with beta = 0, y not read)
    for M in (1, 5, 5000):
        w = _csr([0] * M, 10, 1)
        y0 = synth.uniform(M, 9, synth.S_Y, np.float32)
        m = DevMatrix.of(w)
        plan = m.plan(variant)
        y = run(plan, w.x, 1.0, 0.0)
        assert np.array_equal(y, np.zeros(M, np.float32))
        y = run(plan, w.x, 1.0, 2.5, y0)
        assert np.array_equal(y, y0 * np.float32(2.5))
        plan.destroy()


def test_zero_rows_is_noop():
    rp = dev(np.zeros(1, np.int32))
    e32 = torch.empty(0, dtype=torch.int32, device="cuda")
    ef = torch.empty(0, dtype=torch.float32, device="cuda")
    plan = lb.Plan(rp, e32, ef, (0, 7))
    x = torch.ones(7, device="cuda")
    y = torch.empty(0, device="cuda")
    plan(x, y, 1.0, 0.0)
    torch.cuda.synchronize()
    plan.destroy()


def test_reduction_mode_choice():
    """stream where every row fits a quarter partition, walk otherwise; a
    forced stream on a matrix with a longer row is refused."""
    w = synth.laplacian(n=64)
    m = DevMatrix.of(w)
    info = m.plan("merge8").info
    assert info["merge_reduce"] == "stream" and info["stream_lanes"] == 1
    assert m.plan("merge8_walk").info["merge_reduce"] == "walk"
    m = DevMatrix.of(synth.banded(M=50_000, half_band=500))
    info = m.plan("merge8").info
    assert info["merge_reduce"] == "stream" and info["x_window"]
    assert not m.plan("merge8_noxwin").info["x_window"]
    m = DevMatrix.of(synth.powerlaw(M=50_000, max_len=60))
    info = m.plan("merge8").info
    assert info["merge_reduce"] == "stream" and not info["x_window"]
    w = _csr([3] * 50 + [65] + [3] * 50, 200, 3)        # 65 > 512 / 8
    m = DevMatrix.of(w)
    assert m.plan("merge8").info["merge_reduce"] == "walk"
    with pytest.raises(lb.SpmvError) as e:
        m.plan("merge8", merge_reduce="stream")
    assert e.value.status == 1


@pytest.mark.parametrize("variant", ["merge8", "merge8_walk", "binned"])
def test_deterministic_and_alpha_scaling(variant):
    w = synth.powerlaw(M=40_000, max_len=20_000)
    m = DevMatrix.of(w)
    plan = m.plan(variant)
    y1 = run(plan, w.x, 1.0, 0.0)
    y2 = run(plan, w.x, 1.0, 0.0)
    assert np.array_equal(y1, y2), "bitwise reproducible"
    y4 = run(plan, w.x, 4.0, 0.0)
    assert np.array_equal(y4, np.float32(4) * y1), "power-of-two alpha is exact"
    yh = run(plan, w.x, 0.5, 0.0)
    assert np.array_equal(yh, np.float32(0.5) * y1)
    plan.destroy()


@pytest.mark.parametrize("variant", ALL)
def test_identity_and_diagonal_bitwise(variant):
    n = 70_000
    rng = np.random.default_rng(5)
    for dt in (np.float32, np.float64):
        x = synth.uniform(n, 1, synth.S_X, dt)
        d = (rng.uniform(-4, 4, n)).astype(dt)
        rp = np.arange(n + 1, dtype=np.int32)
        col = np.arange(n, dtype=np.int32)
        m = DevMatrix(rp, col, np.ones(n, dt), n, n)
        plan = m.plan(variant)
        assert np.array_equal(run(plan, x, 1.0, 0.0, dtype=dt), x), "identity"
        plan.destroy()
        m = DevMatrix(rp, col, d, n, n)
        plan = m.plan(variant)
        assert np.array_equal(run(plan, x, 1.0, 0.0, dtype=dt), d * x), "diagonal"
        plan.destroy()


@pytest.mark.parametrize("variant", ALL)
def test_integer_row_sums_exact(variant):
    # row structures of the scaled workloads, values in {-1, 1, 2, 4}, x = 1:
    # every partial sum is an integer < 2^24, so y must equal the row sums
    for name in ("powerlaw", "bimodal", "banded"):
        w = SCALED[name]()
        ints = np.random.default_rng(1).choice(np.array([-1, 1, 2, 4], np.float32), w.nnz)
        m = DevMatrix(w.row_ptr, w.col_idx, ints, w.M, w.N)
        plan = m.plan(variant)
        y = run(plan, np.ones(w.N, np.float32), 1.0, 0.0)
        cs = np.concatenate([[0], np.cumsum(ints.astype(np.int64))])
        want = (cs[w.row_ptr[1:]] - cs[w.row_ptr[:-1]]).astype(np.float64)
        assert np.array_equal(y.astype(np.float64), want), name
        plan.destroy()


def _split_cases(golden):
    yield "worked", np.array(golden("rgcsr_worked_example.txt")["row_ptr"], dtype=np.int32)
    yield "fig1", np.array(golden("loadbalance_fig1_tiles.txt")["row_ptr"], dtype=np.int32)
    yield "empty", np.zeros(40, dtype=np.int32)
    yield "dense_row", np.array([0, 100_000], dtype=np.int32)
    for name in SCALED:
        yield name, SCALED[name]().row_ptr


@pytest.mark.parametrize("ipt", [4, 8, 16])
def test_splits_match_oracle(ipt, golden):
    for name, rp in _split_cases(golden):
        M, nnz = rp.size - 1, int(rp[-1])
        N = 100_000 if name == "dense_row" else max(M, 1)
        m = DevMatrix(rp, np.zeros(nnz, np.int32), np.zeros(nnz, np.float32), M, N)
        plan = m.plan("merge%d" % ipt)
        sr, sn = plan.splits()
        orr, onz = oracle.merge_splits(rp, 64 * ipt)
        assert np.array_equal(sr, orr) and np.array_equal(sn, onz), name
        plan.destroy()


@pytest.mark.parametrize("variant", ["binned", "binned_alt", "binned_one"])
def test_bins_match_oracle(variant, golden):
    for name, rp in _split_cases(golden):
        M, nnz = rp.size - 1, int(rp[-1])
        m = DevMatrix(rp, np.zeros(nnz, np.int32), np.zeros(nnz, np.float32), M,
                      100_000 if name == "dense_row" else max(M, 1))
        plan = m.plan(variant)
        info = plan.info
        edges = info["bin_max_len"][:-1]
        ob, ooff, ocnt = oracle.bins(rp, edges)
        b, off = plan.bins()
        assert np.array_equal(off, ooff), name
        assert np.array_equal(b, ob), name
        assert info["bin_count"] == list(ocnt)
        assert info["max_row_len"] == int(np.diff(rp).max(initial=0))
        assert info["n_empty_rows"] == int((np.diff(rp) == 0).sum())
        assert info["bin_identity"] == (int((ocnt > 0).sum()) <= 1)
        plan.destroy()


def test_malformed_inputs_are_rejected():
    def plan_status(rp, nnz, N=10, validate=False, col=None):
        col = col if col is not None else np.zeros(nnz, np.int32)
        m = DevMatrix(np.asarray(rp, np.int32), col, np.ones(nnz, np.float32), len(rp) - 1, N)
        try:
            m.plan("merge8", validate_columns=validate).destroy()
            return 0
        except lb.SpmvError as e:
            return e.status
    assert plan_status([0, 2, 1, 3], 3) == 6          # decreasing
    assert plan_status([1, 2, 3], 3) == 6             # row_ptr[0] != 0
    assert plan_status([0, 2, 3], 4) == 6             # row_ptr[M] != nnz
    assert plan_status([0, 2, 3], 3, validate=True, col=np.array([0, 10, 1], np.int32)) == 6
    assert plan_status([0, 2, 3], 3, validate=True, col=np.array([0, 9, 1], np.int32)) == 0

    w = synth.tiny()
    m = DevMatrix.of(w)
    plan = m.plan("merge8")
    x = dev(w.x)
    with pytest.raises(lb.SpmvError) as e:
        lb.spmv_exec(plan.handle, x, x, 1.0, 0.0)
    assert e.value.status == 1
    h = plan.handle
    plan.destroy()
    with pytest.raises(lb.SpmvError) as e:
        lb.spmv_exec(h, x, torch.empty(w.M, device="cuda"), 1.0, 0.0)
    assert e.value.status == 5


def test_read_probe_runs_and_leaves_the_sink():
    buf = torch.ones(1 << 22, dtype=torch.int32, device="cuda")   # 16 MiB
    sink = torch.full((1,), 7, dtype=torch.int32, device="cuda")
    lb.spmv_read_probe(buf, sink)
    torch.cuda.synchronize()
    assert int(sink.item()) == 7
    with pytest.raises(lb.SpmvError):
        lb.spmv_read_probe(buf[1:], sink)       # 4-byte offset: misaligned


@pytest.mark.parametrize("order", ["partition", "column"])
def test_walk_carry_chains_around_step_sizes(order):
    """Walk plan at T = 512: rows whose carries run over n partitions for n
    just below, at and above 64 (one fix-up wave's chunk) and 64 + 512 (one
    chunk and one continuation step of eight 64-partition windows), so a
    row's chain ends inside a step, at its last partition and one past it."""
    T = 512
    Ls = []
    for n in (63, 64, 65, 575, 576, 577, 1087, 1088, 1089):
        for d in (-1, 0, 1):
            Ls += [T * n + d, 2, 0, 5]
    L = np.asarray(Ls)
    w = synth.random_csr(len(L), 700_000, L, 13)
    m = DevMatrix.of(w)
    plan = m.plan(None, strategy="merge", merge_reduce="walk", items_per_thread=8,
                  dispatch_order=order)
    assert plan.info["items_per_wave"] == T
    for alpha, beta in ((1.0, 0.0), (-0.5, 2.0)):
        y0 = synth.uniform(w.M, 3, synth.S_Y, np.float32)
        log("chains", order, "nnz=%d" % len(w.col_idx), alpha, beta)
        y = run(plan, w.x, alpha, beta, y0)
        check(y, w.row_ptr, w.col_idx, w.values, w.x, alpha, beta,
              y0 if beta != 0 else None, "chains %s" % order)
    plan.destroy()
