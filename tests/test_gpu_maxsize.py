"""The largest matrix the library accepts: M + nnz = 2^31 - 65 work items
(M = 2^20 rows, ~2.15e9 nonzeros, 17 GB of column indices and values),
built on the device. With values 1 every partial sum is an integer below
2^24, so y is exact in any summation order: y = row length for x = 1, and a
closed-form count for x = (column mod 2). Sampled rows, among them rows of
16M entries, are also checked against the oracle with random x. Every
schedule that fits in memory runs, and SpMM with two right-hand sides."""
import numpy as np
import pytest
import torch

import oracle
import load_balanced_csr_amd as lb
from gpu_util import log

pytestmark = pytest.mark.gpu

M = 1 << 20
N = 1 << 20
NNZ = (1 << 31) - 1 - M - 64
N_LONG = 16
LONG = 16_000_000          # < 2^24: fp32 sums stay exact
A_MUL, K_MUL = 7919, 13    # col(r, k) = (7919 r + 13 k) mod N; parity = (r + k) mod 2


def _lengths():
    rng = np.random.default_rng(31)
    L = np.zeros(M, np.int64)
    long_rows = rng.choice(M, N_LONG, replace=False)
    L[long_rows] = LONG
    rest = NNZ - N_LONG * LONG
    short = np.setdiff1d(np.arange(M), long_rows)
    base, extra = divmod(rest, short.size)
    L[short] = base
    L[short[rng.choice(short.size, extra, replace=False)]] += 1
    # a few empty rows, their entries moved to neighbours
    empties = short[rng.choice(short.size, 1000, replace=False)]
    moved = int(L[empties].sum())
    L[empties] = 0
    keep = np.setdiff1d(short, empties)
    q, rem = divmod(moved, keep.size)
    L[keep] += q
    L[keep[:rem]] += 1
    assert int(L.sum()) == NNZ and L.max() < (1 << 24)
    return L, long_rows


@pytest.fixture(scope="module")
def big():
    free = torch.cuda.mem_get_info()[0]
    if free < 40 << 30:
        pytest.skip("needs ~40 GB of free device memory")
    L, long_rows = _lengths()
    rp_h = np.concatenate([[0], np.cumsum(L)]).astype(np.int64)
    rp64 = torch.from_numpy(rp_h).cuda()
    col = torch.empty(NNZ, dtype=torch.int32, device="cuda")
    chunk = 1 << 27
    log("maxsize: generating", NNZ, "entries")
    for e0 in range(0, NNZ, chunk):
        e = torch.arange(e0, min(NNZ, e0 + chunk), dtype=torch.int64, device="cuda")
        r = torch.searchsorted(rp64, e, right=True) - 1
        k = e - rp64[r]
        col[e0:e0 + e.numel()] = ((r * A_MUL + k * K_MUL) % N).to(torch.int32)
        del e, r, k
    val = torch.ones(NNZ, dtype=torch.float32, device="cuda")
    rp = rp64.to(torch.int32)
    del rp64
    torch.cuda.synchronize()
    yield dict(L=L, rp_h=rp_h, rp=rp, col=col, val=val, long_rows=long_rows)
    del col, val, rp
    torch.cuda.empty_cache()


def _expected_odd(L):
    r = np.arange(M)
    # k in [0, L) with (r + k) odd
    return np.where(r % 2 == 0, L // 2, (L + 1) // 2).astype(np.float32)


def _sample_check(b, y, x_h, what):
    rows = list(b["long_rows"][:2]) + [0, 1, 12345, M // 2, M - 2, M - 1]
    for r in rows:
        a, e = int(b["rp_h"][r]), int(b["rp_h"][r + 1])
        cols = b["col"][a:e].cpu().numpy()
        ref, scale = oracle.spmv(np.array([0, e - a], np.int64), cols,
                                 np.ones(e - a, np.float32), x_h, 1.0, 0.0, None)
        ok, worst, _ = oracle.within_tolerance(y[r:r + 1], ref, scale, 1.0, 0.0, None)
        assert ok, "%s: row %d (len %d) y=%r ref=%r worst=%.3g" % (what, r, e - a, y[r], ref[0],
                                                                  worst)


@pytest.mark.parametrize("opts", [
    dict(),                                                   # auto: merge-path, walk
    dict(strategy="merge", dispatch_order="column"),
    dict(strategy="binned"),
    dict(strategy="group"),
], ids=["auto", "merge_column", "binned", "group"])
def test_max_size_exact(big, opts):
    b = big
    log("maxsize: plan", opts)
    plan = lb.Plan(b["rp"], b["col"], b["val"], (M, N), **opts)
    assert plan.info["nnz"] == NNZ
    L = b["L"].astype(np.float32)
    ones = torch.ones(N, device="cuda")
    y = torch.full((M,), float("nan"), device="cuda")
    log("maxsize: exec x = 1", plan.info["strategy"], plan.info["merge_reduce"])
    plan(ones, y, 1.0, 0.0)
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy(), L), "row lengths"
    odd = (torch.arange(N, device="cuda") % 2).to(torch.float32)
    plan(odd, y, 1.0, 0.0)
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy(), _expected_odd(b["L"])), "odd columns"
    x_h = np.random.default_rng(7).uniform(-1, 1, N).astype(np.float32)
    plan(torch.from_numpy(x_h).cuda(), y, 1.0, 0.0)
    torch.cuda.synchronize()
    _sample_check(b, y.cpu().numpy(), x_h, str(opts))
    plan.destroy()


def test_max_size_spmm(big):
    b = big
    plan = lb.Plan(b["rp"], b["col"], b["val"], (M, N))
    X = torch.stack([torch.ones(N, device="cuda"),
                     (torch.arange(N, device="cuda") % 2).to(torch.float32)], 1).contiguous()
    Y = torch.full((M, 2), float("nan"), device="cuda")
    log("maxsize: spmm k = 2")
    plan.exec_multi(X, Y, 1.0, 0.0)
    torch.cuda.synchronize()
    Yh = Y.cpu().numpy()
    assert np.array_equal(Yh[:, 0], b["L"].astype(np.float32))
    assert np.array_equal(Yh[:, 1], _expected_odd(b["L"]))
    plan.destroy()
