"""Binned schedule with one launch per bin on concurrent streams
(options.bin_streams): the same per-row arithmetic as the single grid, so y
must be bitwise equal to it, and within the bound of the oracle; the call
must order like one launch on the caller's stream (work queued before it is
seen, work queued after it sees y), on a non-default stream too, and must
capture into a graph whose replays match the eager result."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import DevMatrix, check, dev, log

pytestmark = pytest.mark.gpu


def _skewed(M, seed, dtype=np.float32):
    # lengths 0..3000 with a heavy tail: every default bin gets rows
    rng = np.random.default_rng(seed)
    L = np.minimum(3000, (rng.pareto(1.2, M) * 3).astype(np.int64))
    L[rng.integers(0, M, M // 20)] = 0
    return synth.random_csr(M, 6000, L, seed + 1, dtype)


CASES = {
    "tiny": lambda: synth.tiny(),
    "powerlaw": lambda: synth.powerlaw(M=40_000, max_len=12_000),
    "bimodal": lambda: synth.bimodal(M=30_000, n_long=12, long_len=6000),
    "skewed_f64": lambda: _skewed(25_000, 41, np.float64),
}


def _exec(plan, x, y0, alpha, beta, dt, stream=None):
    y = y0.clone() if beta != 0 else torch.full_like(y0, float("nan"))
    plan(x, y, alpha, beta, stream=stream)
    return y


@pytest.mark.parametrize("case", list(CASES))
def test_bin_streams_bitwise_equal_to_one_grid(case):
    w = CASES[case]()
    m = DevMatrix.of(w)
    dt = w.values.dtype.type
    tdt = torch.float32 if dt == np.float32 else torch.float64
    x = dev(w.x)
    y0 = dev(synth.uniform(w.M, 9, synth.S_Y, dt))
    bins_alt = [(1, 1), (6, 4), (40, 16), (900, 64), (None, 256)]
    for bins in (None, bins_alt):
        ref_plan = m.plan(None, strategy="binned", bins=bins)
        for n in (1, 2, 3, 8):
            plan = m.plan(None, strategy="binned", bins=bins, bin_streams=n)
            assert plan.info["bin_streams"] == n
            for alpha, beta in ((1.0, 0.0), (1.5, 0.5)):
                log("bin_streams", case, "bins", "alt" if bins else "default", "n", n, alpha, beta)
                y_ref = _exec(ref_plan, x, y0, alpha, beta, dt)
                y = _exec(plan, x, y0, alpha, beta, dt)
                torch.cuda.synchronize()
                a, b = y.cpu().numpy(), y_ref.cpu().numpy()
                assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), \
                    "%s n=%d: differs from the single grid" % (case, n)
                check(a, w.row_ptr, w.col_idx, w.values, w.x, alpha, beta,
                      y0.cpu().numpy() if beta != 0 else None, "%s n=%d" % (case, n))
            plan.destroy()
        ref_plan.destroy()
    assert tdt in (torch.float32, torch.float64)


def test_bin_streams_order_on_caller_stream():
    # a side stream as the caller: x is written just before the call and y
    # consumed just after it, with no host synchronisation in between
    w = synth.bimodal(M=20_000, n_long=10, long_len=5000)
    m = DevMatrix.of(w)
    plan = m.plan(None, strategy="binned", bin_streams=4)
    ref = m.plan(None, strategy="binned")
    x_h = w.x
    x = torch.zeros(w.N, device="cuda")
    y = torch.empty(w.M, device="cuda")
    out = torch.empty(w.M, device="cuda")
    y_ref = torch.empty(w.M, device="cuda")
    s = torch.cuda.Stream()
    xs = dev(x_h)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        for it in range(5):
            x.copy_(xs * (it + 1))           # queued before the exec on s
            plan(x, y, 1.0, 0.0)              # current stream: s
            out.copy_(y * 2.0)                # queued after the exec on s
            ref(x, y_ref, 1.0, 0.0)
            y_ref.mul_(2.0)
            s.synchronize()
            assert torch.equal(out, y_ref), "iteration %d" % it
    plan.destroy()
    ref.destroy()


def test_bin_streams_graph_capture():
    w = synth.powerlaw(M=30_000, max_len=8000)
    m = DevMatrix.of(w)
    plan = m.plan(None, strategy="binned", bin_streams=3)
    x = dev(w.x)
    y = torch.empty(w.M, device="cuda")
    y_eager = torch.empty(w.M, device="cuda")
    plan(x, y_eager, 2.0, 0.0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            plan(x, y, 2.0, 0.0)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(4):
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_eager), "replay %d" % rep
        plan(x, y_eager, 2.0, 0.0)           # eager work between the replays
        torch.cuda.synchronize()
    del g
    plan.destroy()


def test_bin_streams_option_checks():
    import load_balanced_csr_amd as lb
    w = synth.tiny()
    m = DevMatrix.of(w)
    with pytest.raises(lb.SpmvError) as e:
        m.plan(None, strategy="binned", bin_streams=9)
    assert e.value.status == 1
    # one bin: nothing to split, the single launch runs
    p = m.plan(None, strategy="binned", bins=[(None, 8)], bin_streams=4)
    x = dev(w.x)
    y = torch.full((w.M,), float("nan"), device="cuda")
    p(x, y, 1.0, 0.0)
    torch.cuda.synchronize()
    check(y.cpu().numpy(), w.row_ptr, w.col_idx, w.values, w.x, 1.0, 0.0, None, "one bin")
    p.destroy()
