"""Seeded synthetic CSR workloads (inputs only).

This module generates the CSR arrays, x and the initial y that both the GPU
path and the CPU oracle consume. It computes nothing of the SpMV, its
merge-path partition or its binning. Every array is a pure function of
(seed, stream, index), so results do not depend on the host thread count.

The five workloads follow the shapes the pages measure on (sparse matrices of
regular, banded and heavy-tailed row-length mixes), built synthetically:

``tiny``        2,000 x 2,000 fp32, row lengths uniform in [5, 15].
``laplacian``   fp64 5-point 2-D Laplacian on an n x n grid (n = 2048 by
                default); neighbours outside the grid are dropped.
``powerlaw``    4,000,000^2 fp32, row lengths from a discrete power law with
                exponent 2.1 clipped to [1, 100000], alpha = 1.5, beta = 0.5.
``bimodal``     1,000,000^2 fp32: 1,000 rows of 50,000 entries, 5% of the rows
                empty, the rest 3 entries.
``banded``      32,000,000 rows fp32, 24..40 entries per row within |i-j| <=
                1000, values +-0.9^|i-j| (exponential decay matrix, c = 1).

Each generator takes a ``scale`` so tests can build the same structure at a
size the oracle finishes in seconds.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gen.c")
_LIB = os.path.join(_HERE, "libsynth.so")
_lib = None

# stream ids: which random array a draw belongs to
S_LEN, S_COL, S_VAL, S_X, S_Y, S_SIGN = 1, 2, 3, 4, 5, 6


def build(force: bool = False) -> str:
    """Compile gen.c into libsynth.so (gcc, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall",
                               _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    """libsynth.so, or the copy SYNTH_LIB names (a sanitizer build of the
    same gen.c, made by tests/test_sanitizers.py)."""
    global _lib
    if _lib is None:
        alt = os.environ.get("SYNTH_LIB")
        if not alt:
            build()
        lib = ctypes.CDLL(alt or _LIB)
        i64, u64, i32 = ctypes.c_int64, ctypes.c_uint64, ctypes.c_int32
        p = ctypes.c_void_p
        lib.synth_hash.argtypes = [u64, u64, u64, u64]
        lib.synth_hash.restype = u64
        lib.synth_uniform_f32.argtypes = [i64, u64, u64, p]
        lib.synth_uniform_f64.argtypes = [i64, u64, u64, p]
        lib.synth_rowlen_uniform.argtypes = [i64, i32, i32, u64, u64, p]
        lib.synth_rowlen_powerlaw.argtypes = [i64, ctypes.c_double, i32, u64, u64, p]
        lib.synth_rowlen_bimodal.argtypes = [i64, i64, i32, i64, i32, u64, u64, p]
        lib.synth_rowlen_bimodal.restype = ctypes.c_int
        lib.synth_row_ptr.argtypes = [i64, p, p]
        lib.synth_row_ptr.restype = i64
        lib.synth_cols_distinct.argtypes = [i64, i64, p, i64, u64, u64, p]
        lib.synth_cols_distinct.restype = ctypes.c_int
        lib.synth_values_decay_f32.argtypes = [i64, p, p, ctypes.c_double, ctypes.c_double,
                                               u64, u64, p]
        lib.synth_laplacian_2d.argtypes = [i64, p, p, p]
        lib.synth_laplacian_2d.restype = i64
        _lib = lib
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


@dataclass
class Workload:
    name: str
    M: int
    N: int
    row_ptr: np.ndarray
    col_idx: np.ndarray
    values: np.ndarray
    x: np.ndarray
    y0: Optional[np.ndarray]
    alpha: float
    beta: float
    seed: int
    params: dict = field(default_factory=dict)

    @property
    def nnz(self) -> int:
        return int(self.row_ptr[-1])

    @property
    def dtype(self):
        return self.values.dtype

    def compulsory_bytes(self) -> int:
        """row_ptr + col_idx + values + x + y (y counted once)."""
        s = self.values.dtype.itemsize
        return 4 * (self.M + 1) + self.nnz * (4 + s) + self.N * s + self.M * s


# ---- primitive draws --------------------------------------------------------

def uniform(n: int, seed: int, stream: int, dtype=np.float32) -> np.ndarray:
    """U[-1, 1): 24 random bits (fp32) or 53 (fp64), exactly representable."""
    lib = _load()
    out = np.empty(n, dtype=dtype)
    if dtype == np.float32:
        lib.synth_uniform_f32(n, seed, stream, _ptr(out))
    else:
        lib.synth_uniform_f64(n, seed, stream, _ptr(out))
    return out


def rowlen_uniform(M: int, lo: int, hi: int, seed: int) -> np.ndarray:
    L = np.empty(M, dtype=np.int32)
    _load().synth_rowlen_uniform(M, lo, hi, seed, S_LEN, _ptr(L))
    return L


def rowlen_powerlaw(M: int, exponent: float, max_len: int, seed: int) -> np.ndarray:
    L = np.empty(M, dtype=np.int32)
    _load().synth_rowlen_powerlaw(M, exponent - 1.0, max_len, seed, S_LEN, _ptr(L))
    return L


def rowlen_bimodal(M: int, n_long: int, long_len: int, n_empty: int, short_len: int,
                   seed: int) -> np.ndarray:
    L = np.empty(M, dtype=np.int32)
    rc = _load().synth_rowlen_bimodal(M, n_long, long_len, n_empty, short_len, seed, S_LEN,
                                      _ptr(L))
    if rc:
        raise ValueError("bimodal row lengths: bad counts")
    return L


def row_ptr_from_lengths(L: np.ndarray) -> np.ndarray:
    L = np.ascontiguousarray(L, dtype=np.int32)
    rp = np.empty(L.size + 1, dtype=np.int32)
    if _load().synth_row_ptr(L.size, _ptr(L), _ptr(rp)) < 0:
        raise ValueError("nnz does not fit in int32")
    return rp


def columns_distinct(M: int, N: int, row_ptr: np.ndarray, seed: int,
                     half_window: int = -1) -> np.ndarray:
    nnz = int(row_ptr[-1])
    col = np.empty(max(nnz, 1), dtype=np.int32)[:nnz]
    if nnz and _load().synth_cols_distinct(M, N, _ptr(row_ptr), half_window, seed, S_COL,
                                           _ptr(col)):
        raise ValueError("a row asks for more distinct columns than its range holds")
    return col


# ---- the workloads -------------------------------------------------------------

def tiny(seed: int = 1001, M: int = 2000, N: Optional[int] = None) -> Workload:
    N = M if N is None else N
    L = rowlen_uniform(M, 5, 15, seed)
    rp = row_ptr_from_lengths(L)
    col = columns_distinct(M, N, rp, seed)
    val = uniform(int(rp[-1]), seed, S_VAL, np.float32)
    x = uniform(N, seed, S_X, np.float32)
    return Workload("tiny", M, N, rp, col, val, x, None, 1.0, 0.0, seed,
                    {"row_len": [5, 15]})


def laplacian(seed: int = 1002, n: int = 2048) -> Workload:
    M = n * n
    nnz = 5 * n * n - 4 * n if n > 1 else 1
    rp = np.empty(M + 1, dtype=np.int32)
    col = np.empty(nnz, dtype=np.int32)
    val = np.empty(nnz, dtype=np.float64)
    got = _load().synth_laplacian_2d(n, _ptr(rp), _ptr(col), _ptr(val))
    assert got == nnz, (got, nnz)
    x = uniform(M, seed, S_X, np.float64)
    return Workload("laplacian", M, M, rp, col, val, x, None, 1.0, 0.0, seed, {"grid": n})


def powerlaw(seed: int = 1003, M: int = 4_000_000, max_len: int = 100_000,
             exponent: float = 2.1) -> Workload:
    L = rowlen_powerlaw(M, exponent, min(max_len, M), seed)
    rp = row_ptr_from_lengths(L)
    col = columns_distinct(M, M, rp, seed)
    val = uniform(int(rp[-1]), seed, S_VAL, np.float32)
    x = uniform(M, seed, S_X, np.float32)
    y0 = uniform(M, seed, S_Y, np.float32)
    return Workload("powerlaw", M, M, rp, col, val, x, y0, 1.5, 0.5, seed,
                    {"exponent": exponent, "max_len": max_len})


def bimodal(seed: int = 1004, M: int = 1_000_000, n_long: int = 1000,
            long_len: int = 50_000, empty_frac: float = 0.05,
            short_len: int = 3) -> Workload:
    n_empty = int(round(empty_frac * M))
    L = rowlen_bimodal(M, n_long, long_len, n_empty, short_len, seed)
    rp = row_ptr_from_lengths(L)
    col = columns_distinct(M, M, rp, seed)
    val = uniform(int(rp[-1]), seed, S_VAL, np.float32)
    x = uniform(M, seed, S_X, np.float32)
    return Workload("bimodal", M, M, rp, col, val, x, None, 1.0, 0.0, seed,
                    {"n_long": n_long, "long_len": long_len, "n_empty": n_empty,
                     "short_len": short_len})


def banded(seed: int = 1005, M: int = 32_000_000, half_band: int = 1000,
           lo: int = 24, hi: int = 40, decay: float = 0.9) -> Workload:
    L = rowlen_uniform(M, lo, hi, seed)
    rp = row_ptr_from_lengths(L)
    col = columns_distinct(M, M, rp, seed, half_window=half_band)
    nnz = int(rp[-1])
    val = np.empty(nnz, dtype=np.float32)
    _load().synth_values_decay_f32(M, _ptr(rp), _ptr(col), decay, 1.0, seed, S_SIGN,
                                   _ptr(val))
    x = uniform(M, seed, S_X, np.float32)
    return Workload("banded", M, M, rp, col, val, x, None, 1.0, 0.0, seed,
                    {"half_band": half_band, "row_len": [lo, hi], "decay": decay})


def random_csr(M: int, N: int, lengths: np.ndarray, seed: int, dtype=np.float32,
               alpha: float = 1.0, beta: float = 0.0) -> Workload:
    """Distinct sorted uniform columns for the given row lengths (each <= N)."""
    rp = row_ptr_from_lengths(np.asarray(lengths, dtype=np.int32))
    col = columns_distinct(M, N, rp, seed)
    val = uniform(int(rp[-1]), seed, S_VAL, dtype)
    x = uniform(N, seed, S_X, dtype)
    y0 = uniform(M, seed, S_Y, dtype) if beta != 0.0 else None
    return Workload("random", M, N, rp, col, val, x, y0, alpha, beta, seed)


# The five workloads at full size, by name, with their seeds.
CONFIGS = {
    "tiny": lambda: tiny(),
    "laplacian": lambda: laplacian(),
    "powerlaw": lambda: powerlaw(),
    "bimodal": lambda: bimodal(),
    "banded": lambda: banded(),
}
