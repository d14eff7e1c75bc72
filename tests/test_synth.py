"""Seeded generators: shapes, distributions and determinism (CPU only)."""
import hashlib
import os
import subprocess
import sys

import numpy as np

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _check_csr(w, distinct_sorted=True):
    rp, col = w.row_ptr, w.col_idx
    assert rp.dtype == np.int32 and col.dtype == np.int32
    assert rp[0] == 0 and np.all(np.diff(rp) >= 0) and rp[-1] == col.size == w.values.size
    assert col.size == 0 or (col.min() >= 0 and col.max() < w.N)
    if distinct_sorted:
        d = np.diff(col.astype(np.int64))
        starts = rp[1:-1]
        inside = np.ones(d.size, dtype=bool)
        inside[starts[(starts > 0) & (starts < col.size)] - 1] = False
        assert np.all(d[inside] > 0), "columns strictly increasing within each row"


def test_uniform_exact_and_in_range():
    a = synth.uniform(100000, 5, 1, np.float32)
    assert a.min() >= -1 and a.max() < 1 and abs(a.mean()) < 0.01
    assert np.all(a * np.float32(2 ** 23) == np.round(a * np.float32(2 ** 23)))
    b = synth.uniform(100000, 5, 1, np.float64)
    assert b.min() >= -1 and b.max() < 1 and abs(b.mean()) < 0.01


def test_tiny():
    w = synth.tiny()
    L = np.diff(w.row_ptr)
    assert w.M == w.N == 2000 and L.min() == 5 and L.max() == 15
    assert abs(L.mean() - 10) < 0.2
    _check_csr(w)
    assert w.values.dtype == np.float32 and w.alpha == 1.0 and w.beta == 0.0


def test_laplacian_full_size_counts():
    w = synth.laplacian()
    n = 2048
    assert w.M == n * n and w.nnz == 5 * n * n - 4 * n == 20_963_328
    L = np.diff(w.row_ptr)
    assert (L == 3).sum() == 4 and (L == 4).sum() == 4 * (n - 2) and (L == 5).sum() == (n - 2) ** 2
    _check_csr(w)
    assert w.values.dtype == np.float64


def test_powerlaw_tail():
    M = 4_000_000
    L = synth.rowlen_powerlaw(M, 2.1, 100_000, 1003)
    assert L.min() == 1 and L.max() <= 100_000
    k = np.arange(2, 100_001, dtype=np.float64)
    mean = 1.0 + np.sum((k - 0.5) ** -1.1)                 # E[L] = sum_k P(L >= k)
    second = 1.0 + np.sum((2 * k - 1) * (k - 0.5) ** -1.1)  # E[L^2]
    sd = np.sqrt((second - mean ** 2) / M)
    assert abs(L.mean() - mean) < 6 * sd, (L.mean(), mean, sd)
    assert 7.5 < mean < 8.1
    p1 = 1 - 1.5 ** -1.1
    assert abs((L == 1).mean() - p1) < 0.002
    for kk in (2, 8, 64, 1024):
        assert abs((L >= kk).mean() - (kk - 0.5) ** -1.1) < 0.002


def test_powerlaw_small_matrix():
    w = synth.powerlaw(M=20000, max_len=2000)
    _check_csr(w)
    assert w.alpha == 1.5 and w.beta == 0.5 and w.y0 is not None


def test_bimodal_full_size_counts():
    L = synth.rowlen_bimodal(1_000_000, 1000, 50_000, 50_000, 3, 1004)
    assert (L == 50_000).sum() == 1000 and (L == 0).sum() == 50_000 and (L == 3).sum() == 949_000
    assert L.sum() == 52_847_000


def test_banded_small():
    w = synth.banded(M=30000, half_band=1000)
    _check_csr(w)
    L = np.diff(w.row_ptr)
    assert L.min() >= 24 and L.max() <= 40
    i = np.repeat(np.arange(w.M), L)
    d = np.abs(w.col_idx.astype(np.int64) - i)
    assert d.max() <= 1000
    want = (0.9 ** d.astype(np.float64)).astype(np.float32)
    assert np.array_equal(np.abs(w.values), want)
    neg = (w.values < 0).mean()
    assert 0.45 < neg < 0.55


def _digest(w):
    h = hashlib.sha256()
    for a in (w.row_ptr, w.col_idx, w.values, w.x):
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def test_thread_count_does_not_change_inputs():
    code = ("import sys; sys.path.insert(0, %r); import synth, hashlib, numpy as np;"
            "w = synth.powerlaw(M=50000, max_len=5000);"
            "h = hashlib.sha256();"
            "[h.update(np.ascontiguousarray(a).tobytes()) for a in (w.row_ptr, w.col_idx, w.values, w.x)];"
            "print(h.hexdigest())") % ROOT
    outs = []
    for t in ("1", "3"):
        env = dict(os.environ, OMP_NUM_THREADS=t)
        outs.append(subprocess.check_output([sys.executable, "-c", code], env=env).decode().strip())
    assert outs[0] == outs[1] == _digest(synth.powerlaw(M=50000, max_len=5000))
