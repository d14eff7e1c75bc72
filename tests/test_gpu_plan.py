"""Planning contract and the binding's argument checks.

* A plan is built with one device allocation for its metadata and one host
  synchronisation (the OpSparse page, Section 5.1: all metadata in one
  allocation, no synchronisation mid-pipeline); a plan that takes x slabs
  makes one more allocation, for its slab-major copy of the matrix, and no
  further synchronisation. The choices the device takes from the counted
  rows (partition size, stream or walk, column dispatch order, tiles,
  slabs) are the ones the five workloads are benchmarked with.
* The Python binding rejects, before any launch, tensors too short or of the
  wrong type for the plan; the C ABI rejects x and y whose bytes overlap.
* The measurement aids run, touch only their own outputs, and keep the sink.
"""
import numpy as np
import pytest
import torch

import synth
import load_balanced_csr_amd as lb
from gpu_util import DevMatrix, dev, log

pytestmark = pytest.mark.gpu

# workload -> (items per wave, reduction, dispatch order, x slabs) of the
# default plan
EXPECTED = {
    "tiny": (256, "stream", "partition", 0),
    "laplacian": (256, "stream", "partition", 0),
    "powerlaw": (256, "walk", "column", 1),   # x of 16 MB: slabs
    "bimodal": (1024, "walk", "partition", 0),   # its long rows go to tiles
    "banded": (1024, "stream", "partition", 0),
}


@pytest.mark.parametrize("name", list(EXPECTED))
def test_one_allocation_one_sync(name):
    log("plan contract", name)
    w = synth.CONFIGS[name]()
    m = DevMatrix.of(w)
    # planned as bench.py plans it: the matrix declared static
    plan = m.plan(None, static_matrix=True)
    info = plan.info
    assert info["plan_allocs"] == 1 + info["x_slabs"] and info["plan_syncs"] == 1, info
    assert (info["items_per_wave"], info["merge_reduce"], info["dispatch_order"],
            info["x_slabs"]) == EXPECTED[name], info
    assert info["n_partitions"] == -(-(w.M + w.nnz) // info["items_per_wave"])
    assert (info["tile_rows"] > 0) == (name == "bimodal"), info
    plan.destroy()
    # not declared static, the plan borrows A and keeps no copy of it
    plan = m.plan(None)
    assert plan.info["x_slabs"] == 0 and plan.info["plan_allocs"] == 1, plan.info
    plan.destroy()
    del m
    torch.cuda.empty_cache()


def test_coo_plan_one_allocation_one_sync():
    w = synth.powerlaw(M=50_000, max_len=20_000)
    rows = dev(np.repeat(np.arange(w.M, dtype=np.int32), np.diff(w.row_ptr)))
    col, val = dev(w.col_idx), dev(w.values)
    plan = lb.Plan.coo(rows, col, val, (w.M, w.N))
    info = plan.info
    assert info["plan_allocs"] == 1 and info["plan_syncs"] == 1, info
    plan.destroy()


def test_forced_sizes_keep_the_contract():
    w = synth.bimodal(M=40_000, n_long=40, long_len=8000)
    m = DevMatrix.of(w)
    for ipt in (4, 7, 8, 16):
        for order in ("partition", "column"):
            plan = m.plan(None, strategy="merge", items_per_thread=ipt, merge_reduce="walk",
                          dispatch_order=order)
            info = plan.info
            assert info["items_per_thread"] == ipt and info["dispatch_order"] == order
            assert info["plan_allocs"] == 1 and info["plan_syncs"] == 1
            plan.destroy()


def _untouched(y, fill):
    torch.cuda.synchronize()
    return bool(torch.all(y == fill).item())


def test_binding_rejects_short_and_mistyped_tensors():
    w = synth.random_csr(300, 200, np.full(300, 4), 5)
    m = DevMatrix.of(w)
    plan = m.plan(None)
    x = dev(w.x)
    y = torch.full((w.M,), 7.0, dtype=torch.float32, device="cuda")
    bad = [
        (x[:-1], y, ValueError),                                   # x short
        (x, y[:-1], ValueError),                                   # y short
        (x.double(), y, TypeError),                                # x of another dtype
        (x, y.double(), TypeError),                                # y of another dtype
    ]
    for xx, yy, exc in bad:
        with pytest.raises(exc):
            plan(xx, yy, 1.0, 0.0)
        assert _untouched(y, 7.0)
    X = torch.zeros((w.N - 1, 4), device="cuda")
    Y = torch.full((w.M, 4), 7.0, device="cuda")
    with pytest.raises(ValueError):
        plan.exec_multi(X, Y)
    with pytest.raises(TypeError):
        plan.exec_multi(torch.zeros((w.N, 4), device="cuda", dtype=torch.float64), Y)
    assert _untouched(Y, 7.0)
    plan.destroy()
    # shapes given at plan time
    with pytest.raises(ValueError):
        lb.Plan(m.rp[:-1], m.col, m.val, (m.M, m.N))               # row_ptr short
    with pytest.raises(ValueError):
        lb.Plan(m.rp, m.col, m.val[:-1], (m.M, m.N))               # values short


def test_partially_overlapping_x_and_y_rejected():
    w = synth.random_csr(256, 256, np.full(256, 3), 8)
    m = DevMatrix.of(w)
    plan = m.plan(None)
    buf = torch.zeros(400, dtype=torch.float32, device="cuda")
    with pytest.raises(lb.SpmvError) as e:
        plan(buf[100:356], buf[0:256], 1.0, 0.0)                   # x starts inside y
    assert e.value.status == 1
    with pytest.raises(lb.SpmvError) as e:
        plan(buf[0:256], buf[144:400], 1.0, 0.0)                   # y starts inside x
    assert e.value.status == 1
    plan(buf[0:256], torch.empty(256, device="cuda"), 1.0, 0.0)    # disjoint: fine
    torch.cuda.synchronize()
    plan.destroy()


def test_probes_run_and_keep_their_sink():
    w = synth.powerlaw(M=20_000, max_len=2_000)
    rp, col, val, x = dev(w.row_ptr), dev(w.col_idx), dev(w.values), dev(w.x)
    sink = torch.full((1,), 7, dtype=torch.int32, device="cuda")
    lb.spmv_gather_probe(col, x, sink)
    y = torch.full((w.M,), float("nan"), device="cuda")
    for ipt in (4, 8, 16):
        lb.spmv_stream_probe(rp, col, val, y, ipt)
    torch.cuda.synchronize()
    assert int(sink.item()) == 7
    assert bool(torch.isfinite(y).all().item())      # every row of y written
    with pytest.raises(lb.SpmvError):
        lb.spmv_stream_probe(rp, col, val, y, 7)      # items per thread 4, 8 or 16
    for k, dt in ((4, torch.float32), (8, torch.float32), (8, torch.float64), (64, torch.float32)):
        X = torch.ones((w.N, k), dtype=dt, device="cuda")
        lb.spmv_gather_rows_probe(col, X, sink)
    torch.cuda.synchronize()
    assert int(sink.item()) == 7
    with pytest.raises(lb.SpmvError):                 # 12-byte rows
        lb.spmv_gather_rows_probe(col, torch.ones((w.N, 3), device="cuda"), sink)
