"""CPU oracle for the CSR SpMV path -- TEST INFRASTRUCTURE ONLY.

Only tests/, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
bench.py may import this package. The product library never calls it; the
two share no code.

What each function computes and which passage it follows is stated in
oracle.c. Every function here is pinned by tests/test_oracle.py against facts
that do not come from the oracle itself (dense brute force, closed forms,
invariants, a hand-worked split table).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

# Acceptance rule: per row |y - ref| <= RTOL * (|alpha| * scale + |beta| * |y_old|).
RTOL = {np.dtype(np.float32): 1e-5, np.dtype(np.float64): 1e-13}


def build(force: bool = False) -> str:
    """Compile oracle.c with strict IEEE arithmetic (no contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
                               "-shared", "-Wall", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class OracleLib:
    """ctypes view of one compiled copy of oracle.c."""

    def __init__(self, so_path: str):
        lib = ctypes.CDLL(so_path)
        i64, i32, d, p = ctypes.c_int64, ctypes.c_int32, ctypes.c_double, ctypes.c_void_p
        for name in ("oracle_spmv_f32", "oracle_spmv_f64"):
            f = getattr(lib, name)
            f.argtypes = [i64, p, p, p, p, d, d, p, p, p]
            f.restype = ctypes.c_int
        for name in ("oracle_spmv_rows_f32", "oracle_spmv_rows_f64"):
            f = getattr(lib, name)
            f.argtypes = [p, p, p, p, d, d, p, p, i64, p, p]
            f.restype = ctypes.c_int
        for name in ("oracle_spmm_f32", "oracle_spmm_f64"):
            f = getattr(lib, name)
            f.argtypes = [i64, p, p, p, i64, p, i64, d, d, p, i64, p, p]
            f.restype = ctypes.c_int
        for name in ("oracle_spmv_coo_f32", "oracle_spmv_coo_f64"):
            f = getattr(lib, name)
            f.argtypes = [i64, i64, p, p, p, p, d, d, p, p, p]
            f.restype = ctypes.c_int
        for name in ("oracle_spmv_t_f32", "oracle_spmv_t_f64"):
            f = getattr(lib, name)
            f.argtypes = [i64, i64, p, p, p, p, d, d, p, p, p]
            f.restype = ctypes.c_int
        lib.oracle_rgcsr_stored.argtypes = [i64, p, i64]
        lib.oracle_rgcsr_stored.restype = i64
        lib.oracle_merge_splits.argtypes = [i64, i64, p, i64, p, p]
        lib.oracle_merge_splits.restype = i64
        lib.oracle_bins.argtypes = [i64, p, i32, p, p, p, p]
        lib.oracle_bins.restype = ctypes.c_int
        self.lib = lib

    def spmv(self, row_ptr, col_idx, values, x, alpha: float = 1.0, beta: float = 0.0,
             y_old=None) -> Tuple[np.ndarray, np.ndarray]:
        """ref = alpha*A*x + beta*y_old in fp64, and scale = sum_k |a_ik x_k|.

        The dtype of ``values`` (fp32 or fp64) selects the input precision; x
        and y_old must have the same dtype. y_old is not read when beta == 0."""
        values = np.asarray(values)
        dt = values.dtype
        if dt not in (np.float32, np.float64):
            raise TypeError("values must be float32 or float64")
        if beta != 0.0 and y_old is None:
            raise ValueError("beta != 0 needs y_old")
        rp, col = _c(row_ptr, np.int32), _c(col_idx, np.int32)
        val, xx = _c(values, dt), _c(x, dt)
        yo = _c(y_old, dt) if beta != 0.0 else None
        M = rp.size - 1
        ref = np.empty(M, dtype=np.float64)
        scale = np.empty(M, dtype=np.float64)
        f = self.lib.oracle_spmv_f32 if dt == np.float32 else self.lib.oracle_spmv_f64
        rc = f(M, _ptr(rp), _ptr(col), _ptr(val), _ptr(xx), float(alpha), float(beta),
               _ptr(yo), _ptr(ref), _ptr(scale))
        assert rc == 0
        return ref, scale

    def spmv_rows(self, rows, row_ptr, col_idx, values, x, alpha: float = 1.0,
                  beta: float = 0.0, y_old=None) -> Tuple[np.ndarray, np.ndarray]:
        """The same definition on the listed rows only (for sampled checks)."""
        values = np.asarray(values)
        dt = values.dtype
        if beta != 0.0 and y_old is None:
            raise ValueError("beta != 0 needs y_old")
        rows = _c(rows, np.int64)
        rp, col = _c(row_ptr, np.int32), _c(col_idx, np.int32)
        val, xx = _c(values, dt), _c(x, dt)
        yo = _c(y_old, dt) if beta != 0.0 else None
        ref = np.empty(rows.size, dtype=np.float64)
        scale = np.empty(rows.size, dtype=np.float64)
        f = self.lib.oracle_spmv_rows_f32 if dt == np.float32 else self.lib.oracle_spmv_rows_f64
        rc = f(_ptr(rp), _ptr(col), _ptr(val), _ptr(xx), float(alpha), float(beta), _ptr(yo),
               _ptr(rows), rows.size, _ptr(ref), _ptr(scale))
        assert rc == 0
        return ref, scale

    def spmm(self, row_ptr, col_idx, values, X, alpha: float = 1.0, beta: float = 0.0,
             Y_old=None) -> Tuple[np.ndarray, np.ndarray]:
        """ref = alpha*A*X + beta*Y_old (M x k) in fp64, and scale[i, c] =
        sum_e |a_ie * X[col_e, c]|. X is N x k, Y_old M x k (row-major, any
        row stride); their dtype must match ``values``."""
        values = np.asarray(values)
        dt = values.dtype
        if dt not in (np.float32, np.float64):
            raise TypeError("values must be float32 or float64")
        if beta != 0.0 and Y_old is None:
            raise ValueError("beta != 0 needs Y_old")
        rp, col, val = _c(row_ptr, np.int32), _c(col_idx, np.int32), _c(values, dt)
        XX = _c(X, dt)
        if XX.ndim != 2:
            raise ValueError("X must be 2-D")
        k = XX.shape[1]
        yo = _c(Y_old, dt) if beta != 0.0 else None
        if yo is not None and yo.shape[1] != k:
            raise ValueError("Y_old must have k columns")
        M = rp.size - 1
        ref = np.empty((M, k), dtype=np.float64)
        scale = np.empty((M, k), dtype=np.float64)
        f = self.lib.oracle_spmm_f32 if dt == np.float32 else self.lib.oracle_spmm_f64
        rc = f(M, _ptr(rp), _ptr(col), _ptr(val), k, _ptr(XX), k, float(alpha), float(beta),
               _ptr(yo), k, _ptr(ref), _ptr(scale))
        assert rc == 0
        return ref, scale

    def spmv_coo(self, M: int, row_idx, col_idx, values, x, alpha: float = 1.0,
                 beta: float = 0.0, y_old=None) -> Tuple[np.ndarray, np.ndarray]:
        """The SpMV of an M-row matrix given as COO entries (any order)."""
        values = np.asarray(values)
        dt = values.dtype
        if dt not in (np.float32, np.float64):
            raise TypeError("values must be float32 or float64")
        if beta != 0.0 and y_old is None:
            raise ValueError("beta != 0 needs y_old")
        ri, col = _c(row_idx, np.int32), _c(col_idx, np.int32)
        val, xx = _c(values, dt), _c(x, dt)
        yo = _c(y_old, dt) if beta != 0.0 else None
        ref = np.empty(M, dtype=np.float64)
        scale = np.empty(M, dtype=np.float64)
        f = self.lib.oracle_spmv_coo_f32 if dt == np.float32 else self.lib.oracle_spmv_coo_f64
        rc = f(M, ri.size, _ptr(ri), _ptr(col), _ptr(val), _ptr(xx), float(alpha), float(beta),
               _ptr(yo), _ptr(ref), _ptr(scale))
        assert rc == 0, rc
        return ref, scale

    def spmv_t(self, N: int, row_ptr, col_idx, values, x, alpha: float = 1.0,
               beta: float = 0.0, y_old=None) -> Tuple[np.ndarray, np.ndarray]:
        """y = alpha * A^T x + beta * y_old for the CSR matrix A (M x N):
        x has M entries, the result N."""
        values = np.asarray(values)
        dt = values.dtype
        if dt not in (np.float32, np.float64):
            raise TypeError("values must be float32 or float64")
        if beta != 0.0 and y_old is None:
            raise ValueError("beta != 0 needs y_old")
        rp, col = _c(row_ptr, np.int32), _c(col_idx, np.int32)
        val, xx = _c(values, dt), _c(x, dt)
        yo = _c(y_old, dt) if beta != 0.0 else None
        M = rp.size - 1
        ref = np.empty(N, dtype=np.float64)
        scale = np.empty(N, dtype=np.float64)
        f = self.lib.oracle_spmv_t_f32 if dt == np.float32 else self.lib.oracle_spmv_t_f64
        rc = f(M, N, _ptr(rp), _ptr(col), _ptr(val), _ptr(xx), float(alpha), float(beta),
               _ptr(yo), _ptr(ref), _ptr(scale))
        assert rc == 0
        return ref, scale

    def rgcsr_stored(self, row_ptr, G: int) -> int:
        """Entries a row-grouped CSR layout with groups of G rows stores."""
        rp = _c(row_ptr, np.int32)
        return int(self.lib.oracle_rgcsr_stored(rp.size - 1, _ptr(rp), int(G)))

    def merge_splits(self, row_ptr, T: int) -> Tuple[np.ndarray, np.ndarray]:
        """Merge-path split coordinates (rows ended, nonzeros consumed) at
        every multiple of T items and at the end, by walking the items."""
        rp = _c(row_ptr, np.int32)
        M = rp.size - 1
        nnz = int(rp[-1]) if M >= 0 else 0
        W = M + nnz
        P = (W + T - 1) // T
        sr = np.empty(P + 1, dtype=np.int32)
        sn = np.empty(P + 1, dtype=np.int32)
        got = self.lib.oracle_merge_splits(M, nnz, _ptr(rp), T, _ptr(sr), _ptr(sn))
        assert got == P, (got, P)
        return sr, sn

    def bins(self, row_ptr, max_len) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
        """Rows grouped by length bin: (bins[M], offsets[B+1], counts[B]).
        ``max_len`` lists the inclusive upper length of bins 0..B-2."""
        rp = _c(row_ptr, np.int32)
        M = rp.size - 1
        ml = _c(list(max_len) + [0], np.int64)
        B = len(max_len) + 1
        counts = np.empty(B, dtype=np.int64)
        offsets = np.empty(B + 1, dtype=np.int64)
        out = np.empty(max(M, 1), dtype=np.int32)[:M]
        rc = self.lib.oracle_bins(M, _ptr(rp), B, _ptr(ml), _ptr(counts), _ptr(offsets),
                                  _ptr(out))
        assert rc == 0
        return out, offsets, counts


def _c(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def _default() -> OracleLib:
    """The oracle library: liboracle.so, or the copy ORACLE_LIB names (a
    sanitizer build of the same oracle.c, made by tests/test_sanitizers.py)."""
    global _lib
    if _lib is None:
        alt = os.environ.get("ORACLE_LIB")
        if alt:
            _lib = OracleLib(alt)
        else:
            build()
            _lib = OracleLib(_LIB)
    return _lib


def spmv(*args, **kw):
    return _default().spmv(*args, **kw)


def spmv_rows(*args, **kw):
    return _default().spmv_rows(*args, **kw)


def spmm(*args, **kw):
    return _default().spmm(*args, **kw)


def spmv_coo(*args, **kw):
    return _default().spmv_coo(*args, **kw)


def spmv_t(*args, **kw):
    return _default().spmv_t(*args, **kw)


def rgcsr_stored(*args, **kw):
    return _default().rgcsr_stored(*args, **kw)


def merge_splits(*args, **kw):
    return _default().merge_splits(*args, **kw)


def bins(*args, **kw):
    return _default().bins(*args, **kw)


def compile_variant(source_text: str, out_path: str) -> OracleLib:
    """Compile a (test-modified) copy of oracle.c the same way as build()."""
    src = out_path + ".c"
    with open(src, "w") as f:
        f.write(source_text)
    subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
                           "-shared", "-w", src, "-o", out_path, "-lm"])
    return OracleLib(out_path)


def source_text() -> str:
    with open(_SRC) as f:
        return f.read()


def within_tolerance(y, ref, scale, alpha: float, beta: float, y_old=None,
                     rtol: Optional[float] = None, row_ptr=None):
    """Acceptance rule. Returns (ok, worst_ratio, index_of_worst).

    |y_i - ref_i| <= rtol * (|alpha| * scale_i + |beta| * |y_old_i|) for every
    row, and rows with no entries (when row_ptr is given) must equal
    fl(beta * y_old_i) exactly (0 when beta == 0). y may also be M x k (one
    column per right-hand side); the rule then holds per element. Values compare as values,
    so -0 equals +0. NaN in y is a failure unless ref is NaN there."""
    y = np.asarray(y)
    if rtol is None:
        rtol = RTOL[y.dtype]
    yd = y.astype(np.float64)
    bound = abs(alpha) * scale
    if beta != 0.0:
        bound = bound + abs(beta) * np.abs(np.asarray(y_old, dtype=np.float64))
    err = np.abs(yd - ref)
    nan_ok = np.isnan(yd) & np.isnan(ref)
    lim = rtol * bound
    bad = ~((err <= lim) | nan_ok)
    if row_ptr is not None:
        rp = np.asarray(row_ptr)
        empty = (rp[1:] - rp[:-1]) == 0
        if y.ndim == 2:                      # M x k (multi-vector): per row
            empty = empty[:, None]
        if beta != 0.0:
            want = (np.asarray(y_old, dtype=y.dtype) * y.dtype.type(beta)).astype(np.float64)
        else:
            want = np.zeros(y.shape, dtype=np.float64)
        bad |= empty & (yd != want)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(lim > 0, err / np.where(lim > 0, lim, 1.0), np.where(err > 0, np.inf, 0.0))
    ratio = np.where(nan_ok, 0.0, ratio).ravel()   # worst: flat index
    worst = int(np.argmax(ratio)) if ratio.size else -1
    return (not bool(bad.any())), (float(ratio[worst]) if worst >= 0 else 0.0), worst
