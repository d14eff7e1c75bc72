"""spmv_exec_events and spmv_exec_multi_events: the result is bitwise the
one of the plain call on the same plan, the events' interval is positive
and lies inside events recorded on the stream around the call, and either
event may be NULL. SpMV on every schedule (the events come from the
dominant kernel's dispatch, or bracket the fork and join of per-bin
streams); SpMM with k <= 64 (main kernel's dispatch) and k > 64 (the whole
call)."""
import ctypes

import numpy as np
import pytest
import torch

import synth
import load_balanced_csr_amd as lb
from gpu_util import DevMatrix, dev, log

pytestmark = pytest.mark.gpu


class _Events:
    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                 ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.made = []

    def create(self):
        e = ctypes.c_void_p()
        assert self.hip.hipEventCreate(ctypes.byref(e)) == 0
        self.made.append(e.value)
        return e.value

    def elapsed(self, a, b):
        ms = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return ms.value

    def close(self):
        for e in self.made:
            self.hip.hipEventDestroy(e)


def _plans():
    lap = synth.laplacian(n=300)
    pw = synth.powerlaw(M=60_000, max_len=20_000)
    return {
        "merge_stream": (lap, dict(strategy="merge")),
        "merge_walk": (pw, dict(strategy="merge", merge_reduce="walk")),
        "binned": (pw, dict(strategy="binned")),
        "binned_streams": (pw, dict(strategy="binned", bin_streams=3)),
        "group": (pw, dict(strategy="group")),
        "rgcsr": (lap, None),
    }


def _inside(ev, e0, e1, run):
    """Runs run(e0, e1) between two torch events; returns (inner, outer) ms."""
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    run(e0, e1)
    b.record()
    torch.cuda.synchronize()
    return ev.elapsed(e0, e1), a.elapsed_time(b)


@pytest.mark.parametrize("case", list(_plans()))
def test_spmv_events(case):
    w, opts = _plans()[case]
    m = DevMatrix.of(w)
    plan = (lb.Plan.rgcsr(m.rp, m.col, m.val, (w.M, w.N)) if opts is None
            else m.plan(None, **opts))
    x = dev(w.x)
    ref = torch.empty(w.M, dtype=x.dtype, device="cuda")
    plan(x, ref, 1.5, 0.0)
    torch.cuda.synchronize()
    ev = _Events()
    try:
        e0, e1 = ev.create(), ev.create()
        y = torch.full_like(ref, float("nan"))
        for i in range(3):
            inner, outer = _inside(ev, e0, e1, lambda a_, b_: lb.spmv_exec_events(
                plan.handle, x, y, 1.5, 0.0, a_, b_))
            log("events", case, plan.info["strategy"], "inner %.4f outer %.4f ms" % (inner,
                                                                                  outer))
            assert torch.equal(y, ref), case
            assert 0.0 < inner <= outer + 1e-3, (case, inner, outer)
        for a_, b_ in ((e0, 0), (0, e1), (0, 0)):
            y.fill_(float("nan"))
            lb.spmv_exec_events(plan.handle, x, y, 1.5, 0.0, a_, b_)
            torch.cuda.synchronize()
            assert torch.equal(y, ref), (case, a_, b_)
    finally:
        ev.close()
        plan.destroy()


@pytest.mark.parametrize("k", [8, 70])
@pytest.mark.parametrize("layout", ["stream", "walk"])
def test_spmm_events(layout, k):
    if layout == "stream":
        w, opts = synth.laplacian(n=200), dict(strategy="merge")
    else:
        w, opts = synth.bimodal(M=30_000, n_long=20, long_len=6000), dict(
            strategy="merge", merge_reduce="walk")
    m = DevMatrix.of(w)
    plan = m.plan(None, **opts)
    assert plan.info["merge_reduce"] == layout
    dt = w.values.dtype
    rng = np.random.default_rng(k)
    X = dev(rng.uniform(-1, 1, (w.N, k)).astype(dt))
    need = lb.spmv_spmm_workspace_size(plan.handle, k)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda") if need else None
    ref = torch.empty((w.M, k), dtype=X.dtype, device="cuda")
    lb.spmv_exec_multi(plan.handle, X, ref, 0.75, 0.0, ws)
    torch.cuda.synchronize()
    ev = _Events()
    try:
        e0, e1 = ev.create(), ev.create()
        Y = torch.full_like(ref, float("nan"))
        for i in range(3):
            inner, outer = _inside(ev, e0, e1, lambda a_, b_: lb.spmv_exec_multi(
                plan.handle, X, Y, 0.75, 0.0, ws, None, a_, b_))
            log("spmm events", layout, "k=%d" % k, "inner %.4f outer %.4f ms" % (inner, outer))
            assert torch.equal(Y, ref), (layout, k)
            assert 0.0 < inner <= outer + 1e-3, (layout, k, inner, outer)
        for a_, b_ in ((e0, None), (None, e1)):
            Y.fill_(float("nan"))
            lb.spmv_exec_multi(plan.handle, X, Y, 0.75, 0.0, ws, None, a_, b_)
            torch.cuda.synchronize()
            assert torch.equal(Y, ref), (layout, k, a_, b_)
    finally:
        ev.close()
        plan.destroy()
