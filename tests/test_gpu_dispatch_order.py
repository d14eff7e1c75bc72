"""Column dispatch order of the merge-path walk kernel
(options.dispatch_order = column): the same partitions, carries and fix-up
in another workgroup order, so y must be bitwise equal to the partition
order and within the bound of the oracle; plans that do not walk keep the
partition order; bad values are rejected."""
import numpy as np
import pytest
import torch

import synth
import load_balanced_csr_amd as lb
from gpu_util import DevMatrix, check, dev, log

pytestmark = pytest.mark.gpu


def _unsorted(M, N, seed):
    # long rows with their columns shuffled (the order helps less, results
    # must not change)
    rng = np.random.default_rng(seed)
    L = np.where(rng.random(M) < 0.01, 3000, rng.integers(0, 6, M))
    w = synth.random_csr(M, N, L, seed + 1)
    col = w.col_idx.copy()
    for r in range(M):
        a, b = w.row_ptr[r], w.row_ptr[r + 1]
        col[a:b] = rng.permutation(col[a:b])
    return synth.Workload("unsorted", M, N, w.row_ptr, col, w.values, w.x, None, 1.0, 0.0, seed)


def _f64(w):
    return synth.Workload(w.name, w.M, w.N, w.row_ptr, w.col_idx, w.values.astype(np.float64),
                          w.x.astype(np.float64), None, 1.0, 0.0, w.seed)


CASES = {
    "powerlaw": lambda: synth.powerlaw(M=60_000, max_len=20_000),
    "bimodal": lambda: synth.bimodal(M=40_000, n_long=40, long_len=8000),
    "bimodal_f64": lambda: _f64(synth.bimodal(M=20_000, n_long=10, long_len=6000)),
    "laplacian_walk": lambda: synth.laplacian(n=150),
    "unsorted": lambda: _unsorted(20_000, 50_000, 7),
    "tiny": lambda: synth.tiny(),
}


@pytest.mark.parametrize("case", list(CASES))
@pytest.mark.parametrize("ipt", [4, 8, 16])
def test_column_order_bitwise_equal(case, ipt):
    w = CASES[case]()
    m = DevMatrix.of(w)
    dt = w.values.dtype.type
    x = dev(w.x)
    y0 = dev(synth.uniform(w.M, 4, synth.S_Y, dt))
    # long-row tiles change the summation order, so they stay off here: this
    # compares the two dispatch orders of the same partitions
    base = m.plan(None, strategy="merge", items_per_thread=ipt, merge_reduce="walk",
                  dispatch_order="partition", long_row_tiles="off")
    col = m.plan(None, strategy="merge", items_per_thread=ipt, merge_reduce="walk",
                 dispatch_order="column")
    assert base.info["dispatch_order"] == "partition"
    assert col.info["dispatch_order"] == "column"
    for alpha, beta in ((1.0, 0.0), (-1.5, 0.5)):
        log("dispatch order", case, "ipt", ipt, alpha, beta)
        ys = []
        for plan in (base, col):
            y = y0.clone() if beta != 0 else torch.full_like(y0, float("nan"))
            plan(x, y, alpha, beta)
            ys.append(y)
        torch.cuda.synchronize()
        a, b = ys[1].cpu().numpy(), ys[0].cpu().numpy()
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), case
        check(a, w.row_ptr, w.col_idx, w.values, w.x, alpha, beta,
              y0.cpu().numpy() if beta != 0 else None, "%s ipt %d" % (case, ipt))
    base.destroy()
    col.destroy()


def test_column_order_only_for_walk_plans():
    w = synth.laplacian(n=100)
    m = DevMatrix.of(w)
    p = m.plan(None, strategy="merge", items_per_thread=8, merge_reduce="stream",
               dispatch_order="column")
    assert p.info["dispatch_order"] == "partition"
    p.destroy()
    e32 = torch.empty(0, dtype=torch.int32, device="cuda")
    p = lb.Plan(dev(np.zeros(6, np.int32)), e32, torch.empty(0, device="cuda"), (5, 9),
                strategy="merge", merge_reduce="walk", dispatch_order="column")
    assert p.info["dispatch_order"] == "partition"
    y = torch.full((5,), float("nan"), device="cuda")
    p(torch.ones(9, device="cuda"), y, 1.0, 0.0)
    torch.cuda.synchronize()
    assert torch.equal(y.cpu(), torch.zeros(5))
    p.destroy()


def test_auto_order():
    # long sparse rows fill most partitions: column order; short rows: not
    w = CASES["bimodal"]()
    m = DevMatrix.of(w)
    # by default these long rows go to column-blocked tiles (partition order)
    p = m.plan(None, strategy="merge", merge_reduce="walk")
    assert p.info["tile_rows"] > 0 and p.info["dispatch_order"] == "partition"
    p.destroy()
    p = m.plan(None, strategy="merge", merge_reduce="walk", long_row_tiles="off")
    assert p.info["dispatch_order"] == "column"
    x = dev(w.x)
    y = torch.full((w.M,), float("nan"), device="cuda")
    p(x, y, 1.0, 0.0)
    torch.cuda.synchronize()
    check(y.cpu().numpy(), w.row_ptr, w.col_idx, w.values, w.x, 1.0, 0.0, None, "auto column")
    p.destroy()
    w = synth.laplacian(n=150)
    p = DevMatrix.of(w).plan(None, strategy="merge", merge_reduce="walk")
    assert p.info["dispatch_order"] == "partition"
    p.destroy()


def test_dispatch_order_option_check():
    w = synth.tiny()
    o = lb.make_options(strategy="merge")
    o.dispatch_order = 3
    with pytest.raises(lb.SpmvError) as e:
        lb.spmv_plan(dev(w.row_ptr), dev(w.col_idx), dev(w.values), w.M, w.N, o, None)
    assert e.value.status == 1


@pytest.mark.parametrize("k", [3, 8, 16])
def test_column_order_spmm(k):
    # SpMM over walk plans takes the same order: bitwise equal to the
    # partition order, within the bound of the oracle column by column
    # (long-row tiles off in both: with them the sums of the long rows
    # take another order)
    w = CASES["bimodal"]()
    m = DevMatrix.of(w)
    rng = np.random.default_rng(k)
    X_h = rng.uniform(-1, 1, (w.N, k)).astype(np.float32)
    Y0_h = rng.uniform(-1, 1, (w.M, k)).astype(np.float32)
    X = dev(X_h)
    outs = []
    for order in ("partition", "column"):
        p = m.plan(None, strategy="merge", merge_reduce="walk", dispatch_order=order,
                   long_row_tiles="off")
        assert p.info["dispatch_order"] == order and p.info["tile_rows"] == 0
        # most partitions lie inside the long rows, so SpMM takes the order too
        assert 2 * p.info["interior_partitions"] >= p.info["n_partitions"]
        Y = dev(Y0_h)
        p.exec_multi(X, Y, 1.5, 0.5)
        torch.cuda.synchronize()
        outs.append(Y.cpu().numpy())
        p.destroy()
    assert np.array_equal(outs[0].view(np.uint8), outs[1].view(np.uint8))
    for c in (0, k - 1):
        check(outs[1][:, c].copy(), w.row_ptr, w.col_idx, w.values, X_h[:, c].copy(), 1.5, 0.5,
              Y0_h[:, c].copy(), "spmm col %d" % c)


@pytest.mark.parametrize("case", ["powerlaw", "bimodal", "tiny", "laplacian_walk"])
def test_interior_partition_count(case):
    # partitions with the same split row at both ends, from the merge-path
    # split computed on the host
    w = CASES[case]()
    m = DevMatrix.of(w)
    p = m.plan(None, strategy="merge", merge_reduce="walk", items_per_thread=8)
    T, P = p.info["items_per_wave"], p.info["n_partitions"]
    rp = w.row_ptr.astype(np.int64)
    W = w.M + int(rp[-1])
    d = np.minimum(np.arange(P + 1, dtype=np.int64) * T, W)
    i = np.searchsorted(rp + np.arange(w.M + 1), d, side="right") - 1
    want = int(np.count_nonzero(i[:-1] == i[1:]))
    assert p.info["interior_partitions"] == want, (case, p.info["interior_partitions"], want)
    p.destroy()


def test_auto_partition_size_for_wide_x():
    # rows crossing partitions, x of 6 MB (> one XCD's L2), few interior
    # partitions: the plan splits again at T = 256; its interior count is
    # that of the final split
    w = synth.powerlaw(M=1_500_000, max_len=50_000)
    m = DevMatrix.of(w)
    p = m.plan(None, strategy="merge")
    assert p.info["merge_reduce"] == "walk"
    assert p.info["items_per_wave"] == 256, p.info["items_per_wave"]
    T, P = 256, p.info["n_partitions"]
    rp = w.row_ptr.astype(np.int64)
    assert P == (w.M + int(rp[-1]) + T - 1) // T
    d = np.minimum(np.arange(P + 1, dtype=np.int64) * T, w.M + int(rp[-1]))
    i = np.searchsorted(rp + np.arange(w.M + 1), d, side="right") - 1
    assert p.info["interior_partitions"] == int(np.count_nonzero(i[:-1] == i[1:]))
    x = dev(w.x)
    y0 = dev(w.y0)
    y = y0.clone()
    p(x, y, w.alpha, w.beta)
    torch.cuda.synchronize()
    check(y.cpu().numpy(), w.row_ptr, w.col_idx, w.values, w.x, w.alpha, w.beta, w.y0, "T=256")
    p.destroy()
    # x within one L2: the default partition size stays
    w = CASES["bimodal"]()
    p = DevMatrix.of(w).plan(None, strategy="merge")
    assert p.info["items_per_wave"] == 1024
    p.destroy()
