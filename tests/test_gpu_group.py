"""Group-mapped schedule (groups of 1, 2 or 4 wavefronts over equal shares of
rows, LDS prefix sum, get_tile search) on the GPU vs the oracle, across group
sizes, rows per group, long and empty rows."""
import numpy as np
import pytest

import synth
import load_balanced_csr_amd as lb
from gpu_util import DevMatrix, check, log, run

pytestmark = pytest.mark.gpu


def _case(w, waves, rows, what):
    m = DevMatrix.of(w)
    plan = lb.Plan(m.rp, m.col, m.val, (w.M, w.N))
    plan.set_group(waves, rows)
    info = plan.info
    assert info["strategy"] == "group" and info["group_waves"] == (waves or 4)
    y0 = synth.uniform(w.M, 13, synth.S_Y, w.values.dtype.type)
    for alpha, beta in ((1.0, 0.0), (-1.5, 0.5)):
        log("group", what, waves, info["group_rows"], alpha, beta)
        y = run(plan, w.x, alpha, beta, y0 if beta != 0 else None, w.values.dtype.type)
        check(y, w.row_ptr, w.col_idx, w.values, w.x, alpha, beta, y0 if beta != 0 else None,
              what="group %s w%d r%d" % (what, waves, info["group_rows"]))
    plan.destroy()


@pytest.mark.parametrize("waves", [0, 1, 2, 4])
@pytest.mark.parametrize("rows", [0, 1, 7, 256])
def test_group_workloads(waves, rows):
    for name, w in (("tiny", synth.tiny()), ("laplacian", synth.laplacian(n=90)),
                    ("powerlaw", synth.powerlaw(M=20_000, max_len=6_000)),
                    ("bimodal", synth.bimodal(M=20_000, n_long=6, long_len=5000))):
        _case(w, waves, rows, name)


def test_group_edges_and_option():
    for lengths, N in (([100_000], 120_000), ([0] * 700 + [5000] + [0] * 300, 6000),
                       ([0] * 50, 10), ([3] * 1000 + [0] * 9, 50)):
        w = synth.random_csr(len(lengths), N, np.asarray(lengths), len(lengths))
        _case(w, 4, 0, "edges%d" % len(lengths))
        _case(w, 1, 256, "edges%d" % len(lengths))
    w = synth.random_csr(3000, 900, np.random.default_rng(2).integers(0, 40, 3000), 4,
                         np.float64)
    m = DevMatrix.of(w)
    plan = lb.Plan(m.rp, m.col, m.val, (w.M, w.N), strategy="group")
    assert plan.info["strategy"] == "group"
    y = run(plan, w.x, 2.0, 0.0, dtype=np.float64)
    check(y, w.row_ptr, w.col_idx, w.values, w.x, 2.0, 0.0, what="group option f64")
    with pytest.raises(lb.SpmvError):
        plan.set_group(3, 0)
    with pytest.raises(lb.SpmvError):
        plan.set_group(1, 257)
    plan.destroy()
