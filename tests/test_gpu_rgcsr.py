"""Row-grouped CSR plans on the GPU: SpMV on the column-interleaved copy vs
the CSR oracle for several group sizes, the stored-entry count vs the
oracle's (and the page's worked example), strategy switching, and the copy
semantics (values changed after planning reach MERGE, not RGCSR)."""
import numpy as np
import pytest
import torch

import oracle
import synth
import load_balanced_csr_amd as lb
from gpu_util import DevMatrix, check, dev, log, run

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("G", [0, 1, 4, 32, 100, 1024])
def test_rgcsr_workloads(G):
    for name, w in (("tiny", synth.tiny()), ("laplacian", synth.laplacian(n=120)),
                    ("powerlaw", synth.powerlaw(M=20_000, max_len=5_000)),
                    ("banded", synth.banded(M=30_000, half_band=300)),
                    ("empty", synth.random_csr(500, 40, np.zeros(500, np.int64), 3))):
        m = DevMatrix.of(w)
        plan = lb.Plan.rgcsr(m.rp, m.col, m.val, (w.M, w.N), group_rows=G)
        info = plan.info
        assert info["strategy"] == "rgcsr" and info["rgcsr_group"] == (G or 64)
        assert info["rgcsr_stored"] == oracle.rgcsr_stored(w.row_ptr, G or 64), name
        y0 = synth.uniform(w.M, 9, synth.S_Y, w.values.dtype.type)
        for alpha, beta in ((1.0, 0.0), (1.5, 0.5)):
            log("rgcsr", name, G, alpha, beta)
            y = run(plan, w.x, alpha, beta, y0 if beta != 0 else None, w.values.dtype.type)
            check(y, w.row_ptr, w.col_idx, w.values, w.x, alpha, beta,
                  y0 if beta != 0 else None, what="rgcsr %s G=%d" % (name, G))
        plan.destroy()


def test_rgcsr_worked_example(golden):
    g = golden("rgcsr_worked_example.txt")
    rp = np.array(g["row_ptr"], dtype=np.int32)
    w = synth.random_csr(8, 8, np.diff(rp), 11)
    m = DevMatrix.of(w)
    for G, zeros in ((int(g["rgcsr_group_size"][0]), int(g["rgcsr_artificial_zeros"][0])),
                     (8, int(g["ellpack_artificial_zeros"][0]))):
        plan = lb.Plan.rgcsr(m.rp, m.col, m.val, (8, 8), group_rows=G)
        assert plan.info["rgcsr_stored"] - int(g["nnz"][0]) == zeros
        y = run(plan, w.x, 1.0, 0.0)
        check(y, w.row_ptr, w.col_idx, w.values, w.x, 1.0, 0.0, what="worked G=%d" % G)
        plan.destroy()


def test_rgcsr_switch_and_copy():
    w = synth.powerlaw(M=10_000, max_len=2_000)
    m = DevMatrix.of(w)
    plan = lb.Plan.rgcsr(m.rp, m.col, m.val, (w.M, w.N))
    y_rg = run(plan, w.x, 1.0, 0.0)
    m.val.mul_(2.0)                                  # change A's values on the device
    torch.cuda.synchronize()
    y_rg2 = run(plan, w.x, 1.0, 0.0)
    assert np.array_equal(y_rg, y_rg2)               # the copy is unaffected
    plan.set_strategy("merge")
    y_m = run(plan, w.x, 1.0, 0.0)
    check(y_m, w.row_ptr, w.col_idx, w.values * 2, w.x, 1.0, 0.0, what="merge after switch")
    plan.set_strategy("rgcsr")
    assert np.array_equal(run(plan, w.x, 1.0, 0.0), y_rg)
    plan.destroy()
    p2 = lb.Plan(m.rp, m.col, m.val, (w.M, w.N))
    with pytest.raises(lb.SpmvError):
        p2.set_strategy("rgcsr")
    p2.destroy()
