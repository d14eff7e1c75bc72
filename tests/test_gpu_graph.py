"""spmv_exec and spmv_exec_multi captured into a HIP graph (torch.cuda.graph
on a side stream) and replayed: every schedule, with beta != 0 so each
replay must continue the eager sequence y <- alpha A x + beta y bitwise,
with eager work and synchronisations between the replays."""
import numpy as np
import pytest
import torch

import synth
import load_balanced_csr_amd as lb
from gpu_util import DevMatrix, dev, log

pytestmark = pytest.mark.gpu

STEPS = 4


def _spmv_cases():
    lap = synth.laplacian(n=200)
    pw = synth.powerlaw(M=50_000, max_len=15_000)
    bi = synth.bimodal(M=40_000, n_long=40, long_len=8000)
    return {
        "merge_stream_window": (lap, dict(strategy="merge")),
        "merge_walk_partition": (pw, dict(strategy="merge", merge_reduce="walk",
                                          dispatch_order="partition")),
        "merge_walk_column": (bi, dict(strategy="merge", merge_reduce="walk",
                                       dispatch_order="column")),
        # long rows in column-blocked tiles: the walk+tile grid, then the
        # fix-up and the tile reduction in one grid, two launches per exec
        "merge_walk_tiles": (bi, dict(strategy="merge", merge_reduce="walk")),
        # x slabs: the walk over the slab-major copy, its fix-up and the
        # combine, three launches per exec
        "merge_x_slabs": (pw, dict(strategy="merge", x_slabs="on")),
        "binned": (pw, dict(strategy="binned")),
        "group": (pw, dict(strategy="group")),
        "rgcsr": (lap, None),
    }


def _plan(w, opts):
    m = DevMatrix.of(w)
    if opts is None:
        return m, lb.Plan.rgcsr(m.rp, m.col, m.val, (w.M, w.N))
    return m, m.plan(None, **opts)


def _capture(fn):
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("case", list(_spmv_cases()))
def test_spmv_graph_replays(case):
    w, opts = _spmv_cases()[case]
    m, plan = _plan(w, opts)
    if case == "merge_walk_tiles":
        assert plan.info["tile_rows"] > 0, plan.info
    if case == "merge_x_slabs":
        assert plan.info["x_slabs"] == 1, plan.info
    dt = w.values.dtype.type
    x = dev(w.x)
    y0 = dev(synth.uniform(w.M, 12, synth.S_Y, dt))
    alpha, beta = 1.25, 0.5
    # eager sequence
    y = y0.clone()
    eager = []
    for _ in range(STEPS):
        plan(x, y, alpha, beta)
        eager.append(y.clone())
    torch.cuda.synchronize()
    # captured: one exec, replayed STEPS times on the same y
    y.copy_(y0)
    torch.cuda.synchronize()
    g = _capture(lambda: plan(x, y, alpha, beta))
    y.copy_(y0)
    scratch = torch.empty(1 << 20, device="cuda")
    for i in range(STEPS):
        log("graph", case, "replay", i)
        g.replay()
        scratch.uniform_()                    # unrelated eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(y, eager[i]), "%s replay %d" % (case, i)
    del g
    plan.destroy()


@pytest.mark.parametrize("case", ["stream", "walk", "walk_tiles_k8"])
def test_spmm_graph_replays(case):
    # the walk cases run the SpMM long-row tiles too (X rows of 16 and 32
    # bytes): tiles, merge walk, then fix-up and tile reduction in one grid,
    # three launches
    if case == "stream":
        w = synth.laplacian(n=150)
        opts = dict(strategy="merge")
        k = 8
    else:
        w = synth.bimodal(M=30_000, n_long=20, long_len=6000)
        opts = dict(strategy="merge", merge_reduce="walk")
        k = 4 if case == "walk" else 8
    m = DevMatrix.of(w)
    plan = m.plan(None, **opts)
    if case != "stream":
        assert plan.info["tile_rows"] > 0, plan.info
    dt = w.values.dtype
    rng = np.random.default_rng(5)
    X = dev(rng.uniform(-1, 1, (w.N, k)).astype(dt))
    Y0 = dev(rng.uniform(-1, 1, (w.M, k)).astype(dt))
    need = lb.spmv_spmm_workspace_size(plan.handle, k)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    alpha, beta = -0.75, 0.5
    Y = Y0.clone()
    eager = []
    for _ in range(STEPS):
        lb.spmv_exec_multi(plan.handle, X, Y, alpha, beta, ws if need else None)
        eager.append(Y.clone())
    torch.cuda.synchronize()
    g = _capture(lambda: lb.spmv_exec_multi(plan.handle, X, Y, alpha, beta, ws if need else None))
    Y.copy_(Y0)
    for i in range(STEPS):
        log("graph spmm", case, "replay", i)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(Y, eager[i]), "%s replay %d" % (case, i)
    del g
    plan.destroy()
