"""ctypes binding of libspmv.so (the C ABI in include/spmv.h).

Argument marshalling only: tensors become device pointers and sizes, the
current torch stream becomes the hipStream_t, statuses become exceptions.
Every step of planning and execution runs in the library's HIP kernels.
There is no fallback: if libspmv.so cannot be built or loaded, the calls
raise.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch  # loads the HIP runtime libspmv.so binds to (same soname)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libspmv.so")

SPMV_SUCCESS = 0
STATUS_NAMES = {0: "SUCCESS", 1: "INVALID_ARG", 2: "UNSUPPORTED", 3: "ALLOC", 4: "HIP",
                5: "INVALID_PLAN", 6: "INVALID_MATRIX"}
SPMV_F32, SPMV_F64 = 0, 1
STRATEGY = {"auto": 0, "merge": 1, "binned": 2, "rgcsr": 3, "group": 4}
STRATEGY_NAME = {v: k for k, v in STRATEGY.items()}
MAX_BINS = 8

EXPORTED = ("spmv_plan", "spmv_plan_ex", "spmv_plan_coo", "spmv_plan_transpose",
            "spmv_plan_csc", "spmv_plan_rgcsr", "spmv_exec", "spmv_exec_events", "spmv_destroy",
            "spmv_plan_set_strategy", "spmv_plan_set_group", "spmv_plan_update_values",
            "spmv_plan_info",
            "spmv_plan_copy_splits",
            "spmv_plan_copy_bins", "spmv_read_probe", "spmv_gather_probe",
            "spmv_gather_rows_probe",
            "spmv_stream_probe", "spmv_spmm_workspace_size",
            "spmv_exec_multi", "spmv_exec_multi_events", "spmv_exec_noalloc",
            "spmv_status_string", "spmv_last_error")


class SpmvError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__("%s: %s (%s)" % (where, STATUS_NAMES.get(status, status), detail))


class PlanOptions(ctypes.Structure):
    _fields_ = [("strategy", ctypes.c_int32), ("items_per_thread", ctypes.c_int32),
                ("n_bins", ctypes.c_int32), ("validate_columns", ctypes.c_int32),
                ("merge_reduce", ctypes.c_int32), ("stream_lanes", ctypes.c_int32),
                ("x_window", ctypes.c_int32), ("bin_streams", ctypes.c_int32),
                ("bin_max_len", ctypes.c_int64 * MAX_BINS),
                ("bin_lanes", ctypes.c_int32 * MAX_BINS),
                ("dispatch_order", ctypes.c_int32), ("long_row_tiles", ctypes.c_int32),
                ("x_slabs", ctypes.c_int32), ("static_matrix", ctypes.c_int32)]


class PlanInfo(ctypes.Structure):
    _fields_ = [("M", ctypes.c_int64), ("N", ctypes.c_int64), ("nnz", ctypes.c_int64),
                ("dtype", ctypes.c_int32), ("strategy", ctypes.c_int32),
                ("items_per_thread", ctypes.c_int32), ("items_per_wave", ctypes.c_int32),
                ("n_partitions", ctypes.c_int64), ("merge_reduce", ctypes.c_int32),
                ("stream_lanes", ctypes.c_int32), ("x_window", ctypes.c_int32),
                ("bin_streams", ctypes.c_int32), ("n_bins", ctypes.c_int32),
                ("bin_identity", ctypes.c_int32), ("bin_max_len", ctypes.c_int64 * MAX_BINS),
                ("bin_lanes", ctypes.c_int32 * MAX_BINS),
                ("bin_count", ctypes.c_int64 * MAX_BINS), ("max_row_len", ctypes.c_int64),
                ("n_empty_rows", ctypes.c_int64), ("workspace_bytes", ctypes.c_int64),
                ("rgcsr_group", ctypes.c_int32), ("pad1", ctypes.c_int32),
                ("rgcsr_stored", ctypes.c_int64), ("group_waves", ctypes.c_int32),
                ("group_rows", ctypes.c_int32), ("dispatch_order", ctypes.c_int32),
                ("interior_partitions", ctypes.c_int32), ("plan_allocs", ctypes.c_int32),
                ("plan_syncs", ctypes.c_int32), ("tile_rows", ctypes.c_int32),
                ("tile_blocks", ctypes.c_int32), ("walk_partitions", ctypes.c_int32),
                ("x_slabs", ctypes.c_int32), ("slab_segments", ctypes.c_int64),
                ("slab_bytes", ctypes.c_int64)]


_lib = None


def load(build_if_missing: bool = True):
    """Load libspmv.so (building it with hipcc first if it is not there)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        if not build_if_missing:
            raise OSError("libspmv.so is not built: " + LIB_PATH)
        from . import build as _build
        _build.build(force=False)
    lib = ctypes.CDLL(LIB_PATH)
    i64, i32, p, d = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_double
    st = ctypes.c_int
    lib.spmv_plan.argtypes = [ctypes.POINTER(p), i64, i64, i64, p, p, p, i32, p]
    lib.spmv_plan_ex.argtypes = [ctypes.POINTER(p), i64, i64, i64, p, p, p, i32,
                                 ctypes.POINTER(PlanOptions), p]
    lib.spmv_plan_coo.argtypes = [ctypes.POINTER(p), i64, i64, i64, p, p, p, i32, p, p]
    lib.spmv_plan_transpose.argtypes = [ctypes.POINTER(p), i64, i64, i64, p, p, p, i32, p, p]
    lib.spmv_plan_csc.argtypes = [ctypes.POINTER(p), i64, i64, i64, p, p, p, i32, p, p]
    lib.spmv_plan_rgcsr.argtypes = [ctypes.POINTER(p), i64, i64, i64, p, p, p, i32, i32, p]
    lib.spmv_exec.argtypes = [p, p, p, d, d, p]
    lib.spmv_exec_events.argtypes = [p, p, p, d, d, p, p, p]
    lib.spmv_destroy.argtypes = [p]
    lib.spmv_plan_set_strategy.argtypes = [p, i32]
    lib.spmv_plan_update_values.argtypes = [p, p, p]
    lib.spmv_plan_set_group.argtypes = [p, i32, i32]
    lib.spmv_plan_info.argtypes = [p, ctypes.POINTER(PlanInfo)]
    lib.spmv_plan_copy_splits.argtypes = [p, p, p, i64]
    lib.spmv_plan_copy_bins.argtypes = [p, p, i64, p]
    lib.spmv_read_probe.argtypes = [p, i64, p, p]
    lib.spmv_gather_probe.argtypes = [p, i64, p, i64, i32, p, p]
    lib.spmv_gather_rows_probe.argtypes = [p, i64, p, i64, i32, p, p]
    lib.spmv_stream_probe.argtypes = [p, p, p, i64, i64, i32, i32, p, p]
    lib.spmv_exec_noalloc.argtypes = [i64, i64, i64, p, p, p, i32, p, p, d, d, p]
    lib.spmv_spmm_workspace_size.argtypes = [p, i64, ctypes.POINTER(ctypes.c_size_t)]
    lib.spmv_exec_multi.argtypes = [p, i64, p, i64, p, i64, d, d, p, ctypes.c_size_t, p]
    lib.spmv_exec_multi_events.argtypes = [p, i64, p, i64, p, i64, d, d, p, ctypes.c_size_t, p,
                                           p, p]
    for name in EXPORTED:
        if name not in ("spmv_status_string", "spmv_last_error"):
            getattr(lib, name).restype = st
    lib.spmv_status_string.argtypes = [st]
    lib.spmv_status_string.restype = ctypes.c_char_p
    lib.spmv_last_error.argtypes = []
    lib.spmv_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status: int, where: str):
    if status != SPMV_SUCCESS:
        raise SpmvError(status, where, load().spmv_last_error().decode(errors="replace"))


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _dev_ptr(t: Optional[torch.Tensor], name: str, dtypes,
             contiguous: bool = True) -> Optional[int]:
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch tensor" % name)
    if t.dtype not in dtypes:
        raise TypeError("%s has dtype %s, expected one of %s" % (name, t.dtype, dtypes))
    if not t.is_cuda:
        raise ValueError("%s must be a device (cuda) tensor" % name)
    if contiguous and not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t.data_ptr() if t.numel() else None


def _dtype_code(values: torch.Tensor) -> int:
    return SPMV_F32 if values.dtype == torch.float32 else SPMV_F64


# Shape and value type of every plan made through this module (handle ->
# (M, N, torch dtype)): the C ABI takes bare pointers and cannot see a
# tensor's length, so the sizes are checked here, before any call that
# would read or write past a short tensor.
_plans: dict = {}
_TORCH_DTYPE = {SPMV_F32: torch.float32, SPMV_F64: torch.float64}


def _register(handle: int, M: int, N: int, dtype_code: int) -> int:
    _plans[handle] = (int(M), int(N), _TORCH_DTYPE[dtype_code])
    return handle


def _plan_shape(plan: int):
    """(M, N, dtype) of a plan; asks the library for handles made elsewhere
    (an invalid handle raises there)."""
    got = _plans.get(plan)
    if got is not None:
        return got
    info = PlanInfo()
    _check(load().spmv_plan_info(plan, ctypes.byref(info)), "spmv_plan_info")
    return int(info.M), int(info.N), _TORCH_DTYPE[info.dtype]


def _check_vec(t: torch.Tensor, name: str, n: int, dtype) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s has dtype %s, the plan's values are %s" % (name, t.dtype, dtype))
    if t.numel() < n:
        raise ValueError("%s has %d elements, the plan needs %d" % (name, t.numel(), n))


def _check_csr(row_ptr, col_idx, values, M: int, N: int) -> None:
    if int(M) < 0 or int(N) < 0:
        raise ValueError("negative shape (%d, %d)" % (M, N))
    if row_ptr is not None and int(row_ptr.numel()) != int(M) + 1 and int(M) > 0:
        raise ValueError("row_ptr has %d entries, M + 1 = %d" % (row_ptr.numel(), int(M) + 1))
    if int(values.numel()) != int(col_idx.numel()):
        raise ValueError("values (%d) and col_idx (%d) differ in length"
                         % (values.numel(), col_idx.numel()))


MERGE_REDUCE = {"auto": 0, "walk": 1, "stream": 2}
DISPATCH_ORDER = {"auto": 0, "partition": 1, "column": 2}
DISPATCH_ORDER_NAME = {1: "partition", 2: "column"}
MERGE_REDUCE_NAME = {1: "walk", 2: "stream"}


def make_options(strategy: str = "auto", items_per_thread: int = 0, bins=None,
                 validate_columns: bool = False, merge_reduce: str = "auto",
                 stream_lanes: int = 0, x_window: str = "auto",
                 bin_streams: int = 0, dispatch_order: str = "auto",
                 long_row_tiles: str = "auto", x_slabs: str = "auto",
                 static_matrix: bool = False) -> PlanOptions:
    """bins: optional list of (max_len, lanes) pairs; the last max_len is ignored.
    bin_streams: 0 runs the binned schedule as one grid; n >= 1 launches each
    bin on its own, dealt over the caller's stream and n - 1 plan streams.
    dispatch_order: "partition" or "column" (walk plans: workgroups sorted by
    the column of their middle nonzero), "auto" the library's choice."""
    o = PlanOptions()
    o.strategy = STRATEGY[strategy]
    o.items_per_thread = items_per_thread
    o.validate_columns = int(bool(validate_columns))
    o.merge_reduce = MERGE_REDUCE[merge_reduce]
    o.stream_lanes = stream_lanes
    o.x_window = {"auto": 0, "off": 1, "on": 2}[x_window]
    o.bin_streams = bin_streams
    o.dispatch_order = DISPATCH_ORDER[dispatch_order]
    o.long_row_tiles = {"auto": 0, "off": 1}[long_row_tiles]
    o.x_slabs = {"auto": 0, "off": 1, "on": 2}[x_slabs]
    o.static_matrix = int(bool(static_matrix))
    if bins:
        o.n_bins = len(bins)
        for k, (ml, lanes) in enumerate(bins):
            o.bin_max_len[k] = ml if ml is not None else 0
            o.bin_lanes[k] = lanes
    return o


def spmv_plan(row_ptr: torch.Tensor, col_idx: torch.Tensor, values: torch.Tensor, M: int,
              N: int, options: Optional[PlanOptions] = None, stream=None) -> int:
    """Plan handle for the CSR matrix (device int32 row_ptr/col_idx, fp32/fp64
    values). The tensors are borrowed: keep them alive until spmv_destroy."""
    lib = load()
    _check_csr(row_ptr, col_idx, values, M, N)
    nnz = int(col_idx.numel())
    h = ctypes.c_void_p()
    args = (ctypes.byref(h), M, N, nnz, _dev_ptr(row_ptr, "row_ptr", (torch.int32,)),
            _dev_ptr(col_idx, "col_idx", (torch.int32,)),
            _dev_ptr(values, "values", (torch.float32, torch.float64)), _dtype_code(values))
    if options is None:
        _check(lib.spmv_plan(*args, _stream(stream)), "spmv_plan")
    else:
        _check(lib.spmv_plan_ex(*args, ctypes.byref(options), _stream(stream)), "spmv_plan_ex")
    return _register(h.value, M, N, _dtype_code(values))


def spmv_plan_coo(row_idx: torch.Tensor, col_idx: torch.Tensor, values: torch.Tensor, M: int,
                  N: int, options: Optional[PlanOptions] = None, stream=None) -> int:
    """Plan handle for a COO matrix sorted by row (device int32 row_idx /
    col_idx, fp32/fp64 values). col_idx and values are borrowed; row_idx is
    read only during the call."""
    lib = load()
    nnz = int(col_idx.numel())
    if int(row_idx.numel()) != nnz:
        raise ValueError("row_idx and col_idx must have the same length")
    _check_csr(None, col_idx, values, M, N)
    h = ctypes.c_void_p()
    _check(lib.spmv_plan_coo(ctypes.byref(h), M, N, nnz,
                             _dev_ptr(row_idx, "row_idx", (torch.int32,)),
                             _dev_ptr(col_idx, "col_idx", (torch.int32,)),
                             _dev_ptr(values, "values", (torch.float32, torch.float64)),
                             _dtype_code(values),
                             ctypes.byref(options) if options is not None else None,
                             _stream(stream)), "spmv_plan_coo")
    return _register(h.value, M, N, _dtype_code(values))


def _plan_other(fn: str, ptr: torch.Tensor, idx: torch.Tensor, values: torch.Tensor, M: int,
                N: int, options: Optional[PlanOptions], stream) -> int:
    lib = load()
    h = ctypes.c_void_p()
    # fn's offsets cover the rows of the stored matrix: M for a transpose
    # (A is M x N in CSR), N for CSC (A^T is N x M)
    _check_csr(ptr, idx, values, M if fn == "spmv_plan_transpose" else N,
               N if fn == "spmv_plan_transpose" else M)
    _check(getattr(lib, fn)(ctypes.byref(h), M, N, int(idx.numel()),
                            _dev_ptr(ptr, "offsets", (torch.int32,)),
                            _dev_ptr(idx, "indices", (torch.int32,)),
                            _dev_ptr(values, "values", (torch.float32, torch.float64)),
                            _dtype_code(values),
                            ctypes.byref(options) if options is not None else None,
                            _stream(stream)), fn)
    # the plan computes with A^T for a transpose (shape N x M), with A for CSC
    if fn == "spmv_plan_transpose":
        return _register(h.value, N, M, _dtype_code(values))
    return _register(h.value, M, N, _dtype_code(values))


def spmv_plan_transpose(row_ptr, col_idx, values, M: int, N: int,
                        options: Optional[PlanOptions] = None, stream=None) -> int:
    """Plan computing y = alpha * A^T x + beta * y for the CSR matrix A (M x N);
    the plan keeps its own copy of A^T (A's tensors are read only here)."""
    return _plan_other("spmv_plan_transpose", row_ptr, col_idx, values, M, N, options, stream)


def spmv_plan_csc(col_ptr, row_idx, values, M: int, N: int,
                  options: Optional[PlanOptions] = None, stream=None) -> int:
    """Plan computing y = alpha * A x + beta * y for A (M x N) in CSC form."""
    return _plan_other("spmv_plan_csc", col_ptr, row_idx, values, M, N, options, stream)


def spmv_plan_rgcsr(row_ptr, col_idx, values, M: int, N: int, group_rows: int = 0,
                    stream=None) -> int:
    """Plan whose spmv_exec runs on a row-grouped CSR copy of A (groups of
    group_rows rows, 0 = 64); the copy is taken here."""
    lib = load()
    _check_csr(row_ptr, col_idx, values, M, N)
    h = ctypes.c_void_p()
    _check(lib.spmv_plan_rgcsr(ctypes.byref(h), M, N, int(col_idx.numel()),
                               _dev_ptr(row_ptr, "row_ptr", (torch.int32,)),
                               _dev_ptr(col_idx, "col_idx", (torch.int32,)),
                               _dev_ptr(values, "values", (torch.float32, torch.float64)),
                               _dtype_code(values), int(group_rows), _stream(stream)),
           "spmv_plan_rgcsr")
    return _register(h.value, M, N, _dtype_code(values))


def spmv_exec(plan: int, x: torch.Tensor, y: torch.Tensor, alpha: float = 1.0,
              beta: float = 0.0, stream=None) -> None:
    """y = alpha * A x + beta * y, enqueued on the stream (asynchronous)."""
    dts = (torch.float32, torch.float64)
    M, N, dt = _plan_shape(plan)
    _check_vec(x, "x", N, dt)
    _check_vec(y, "y", M, dt)
    _check(load().spmv_exec(plan, _dev_ptr(x, "x", dts), _dev_ptr(y, "y", dts), float(alpha),
                            float(beta), _stream(stream)), "spmv_exec")


def spmv_exec_events(plan: int, x: torch.Tensor, y: torch.Tensor, alpha: float, beta: float,
                     ev_begin: int, ev_end: int, stream=None) -> None:
    """spmv_exec recording two hipEvent_t handles around the dominant kernel."""
    dts = (torch.float32, torch.float64)
    M, N, dt = _plan_shape(plan)
    _check_vec(x, "x", N, dt)
    _check_vec(y, "y", M, dt)
    _check(load().spmv_exec_events(plan, _dev_ptr(x, "x", dts), _dev_ptr(y, "y", dts),
                                   float(alpha), float(beta), _stream(stream), ev_begin, ev_end),
           "spmv_exec_events")


def spmv_exec_noalloc(row_ptr: torch.Tensor, col_idx: torch.Tensor, values: torch.Tensor,
                      M: int, N: int, x: torch.Tensor, y: torch.Tensor, alpha: float = 1.0,
                      beta: float = 0.0, stream=None) -> None:
    """One y = alpha * A x + beta * y with no plan and no device allocation
    (the library's own scratch array holds the partition data)."""
    _check_csr(row_ptr, col_idx, values, M, N)
    _check_vec(x, "x", N, values.dtype)
    _check_vec(y, "y", M, values.dtype)
    dts = (torch.float32, torch.float64)
    _check(load().spmv_exec_noalloc(int(M), int(N), int(col_idx.numel()),
                                    _dev_ptr(row_ptr, "row_ptr", (torch.int32,)),
                                    _dev_ptr(col_idx, "col_idx", (torch.int32,)),
                                    _dev_ptr(values, "values", dts), _dtype_code(values),
                                    _dev_ptr(x, "x", dts), _dev_ptr(y, "y", dts), float(alpha),
                                    float(beta), _stream(stream)), "spmv_exec_noalloc")


def spmv_spmm_workspace_size(plan: int, k: int) -> int:
    """Bytes of device workspace spmv_exec_multi needs for k right-hand sides."""
    n = ctypes.c_size_t(0)
    _check(load().spmv_spmm_workspace_size(plan, int(k), ctypes.byref(n)),
           "spmv_spmm_workspace_size")
    return int(n.value)


def _row_major(t: torch.Tensor, name: str):
    if t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1):
        raise ValueError("%s must be a 2-D row-major tensor (unit column stride)" % name)
    return max(int(t.stride(0)), int(t.shape[1]))


def spmv_exec_multi(plan: int, X: torch.Tensor, Y: torch.Tensor, alpha: float = 1.0,
                    beta: float = 0.0, workspace: Optional[torch.Tensor] = None,
                    stream=None, ev_begin: Optional[int] = None,
                    ev_end: Optional[int] = None) -> None:
    """Y = alpha * A X + beta * Y for the k = X.shape[1] columns of X (N x k)
    and Y (M x k), both row-major; ``workspace`` is a device tensor of at
    least spmv_spmm_workspace_size(plan, k) bytes (None when that is 0).
    ev_begin / ev_end: optional hipEvent_t handles, recorded by the main
    kernel's dispatch for k <= 64 and around every launch for k > 64."""
    dts = (torch.float32, torch.float64)
    M, N, dt = _plan_shape(plan)
    for t, name, rows in ((X, "X", N), (Y, "Y", M)):
        if not isinstance(t, torch.Tensor):
            raise TypeError("%s must be a torch tensor" % name)
        if t.dtype != dt:
            raise TypeError("%s has dtype %s, the plan's values are %s" % (name, t.dtype, dt))
        if t.dim() != 2 or t.shape[0] < rows:
            raise ValueError("%s must be 2-D with at least %d rows" % (name, rows))
    if X.shape[1] != Y.shape[1]:
        raise ValueError("X and Y must have the same number of columns")
    ldx, ldy = _row_major(X, "X"), _row_major(Y, "Y")
    ws, wsb = None, 0
    if workspace is not None:
        if not workspace.is_cuda:
            raise ValueError("workspace must be a device tensor")
        ws, wsb = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    _check(load().spmv_exec_multi_events(plan, int(X.shape[1]), _dev_ptr(X, "X", dts, False),
                                         ldx, _dev_ptr(Y, "Y", dts, False), ldy, float(alpha),
                                         float(beta), ws, wsb, _stream(stream), ev_begin,
                                         ev_end), "spmv_exec_multi")


def spmv_read_probe(data: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """One streaming read of the whole (16-byte multiple) device tensor `data`;
    `sink` is a device int32 tensor (measurement aid, see the header)."""
    if not (data.is_cuda and sink.is_cuda and sink.dtype == torch.int32):
        raise ValueError("spmv_read_probe needs device tensors and an int32 sink")
    _check(load().spmv_read_probe(data.data_ptr(), data.numel() * data.element_size(),
                                  sink.data_ptr(), _stream(stream)), "spmv_read_probe")


def spmv_gather_probe(col_idx: torch.Tensor, x: torch.Tensor, sink: torch.Tensor,
                      stream=None) -> None:
    """Read col_idx once and gather x at every column, nothing else
    (measurement aid, see the header)."""
    if not (col_idx.is_cuda and x.is_cuda and sink.is_cuda and sink.dtype == torch.int32
            and col_idx.dtype == torch.int32 and x.dtype in (torch.float32, torch.float64)):
        raise ValueError("spmv_gather_probe needs device tensors: int32 col_idx, fp32/fp64 x, "
                         "int32 sink")
    _check(load().spmv_gather_probe(col_idx.data_ptr(), col_idx.numel(), x.data_ptr(), x.numel(),
                                    _dtype_code(x), sink.data_ptr(), _stream(stream)),
           "spmv_gather_probe")


def spmv_gather_rows_probe(col_idx: torch.Tensor, X: torch.Tensor, sink: torch.Tensor,
                           stream=None) -> None:
    """Read col_idx once and gather the row of X (2-D, contiguous) at every
    column, nothing else (measurement aid, see the header)."""
    if not (col_idx.is_cuda and X.is_cuda and sink.is_cuda and sink.dtype == torch.int32
            and col_idx.dtype == torch.int32 and X.dim() == 2 and X.is_contiguous()):
        raise ValueError("spmv_gather_rows_probe needs device tensors: int32 col_idx, a "
                         "contiguous 2-D X, int32 sink")
    _check(load().spmv_gather_rows_probe(col_idx.data_ptr(), col_idx.numel(), X.data_ptr(),
                                         X.shape[0], X.shape[1] * X.element_size(),
                                         sink.data_ptr(), _stream(stream)),
           "spmv_gather_rows_probe")


def spmv_stream_probe(row_ptr: torch.Tensor, col_idx: torch.Tensor, values: torch.Tensor,
                      y: torch.Tensor, items_per_thread: int, stream=None) -> None:
    """Stream the CSR arrays in partitions of 64 * items_per_thread units and
    write y, with no x and no arithmetic (measurement aid, see the header)."""
    M = int(row_ptr.numel()) - 1
    _check_csr(row_ptr, col_idx, values, M, 1)
    _check_vec(y, "y", M, values.dtype)
    _check(load().spmv_stream_probe(_dev_ptr(row_ptr, "row_ptr", (torch.int32,)),
                                    _dev_ptr(col_idx, "col_idx", (torch.int32,)),
                                    _dev_ptr(values, "values", (torch.float32, torch.float64)),
                                    M, int(col_idx.numel()), _dtype_code(values),
                                    int(items_per_thread), y.data_ptr(), _stream(stream)),
           "spmv_stream_probe")


def spmv_destroy(plan: Optional[int]) -> None:
    _check(load().spmv_destroy(plan), "spmv_destroy")
    _plans.pop(plan, None)


def spmv_plan_set_strategy(plan: int, strategy: str) -> None:
    _check(load().spmv_plan_set_strategy(plan, STRATEGY[strategy]), "spmv_plan_set_strategy")


def spmv_plan_update_values(plan: int, values: torch.Tensor, stream=None) -> None:
    """Make the plan use `values` (nnz entries, the planned layout and dtype)
    from the next exec on; a plan with x slabs rewrites its copy on `stream`."""
    info = spmv_plan_info(plan)
    _check_vec(values, "values", int(info["nnz"]),
               torch.float32 if info["dtype"] == "f32" else torch.float64)
    _check(load().spmv_plan_update_values(
        plan, _dev_ptr(values, "values", (torch.float32, torch.float64)), _stream(stream)),
        "spmv_plan_update_values")


def spmv_plan_set_group(plan: int, group_waves: int = 0, rows_per_group: int = 0) -> None:
    """Select the group-mapped schedule (0 = defaults)."""
    _check(load().spmv_plan_set_group(plan, int(group_waves), int(rows_per_group)),
           "spmv_plan_set_group")


def spmv_plan_info(plan: int) -> dict:
    info = PlanInfo()
    _check(load().spmv_plan_info(plan, ctypes.byref(info)), "spmv_plan_info")
    nb = info.n_bins
    return {"M": info.M, "N": info.N, "nnz": info.nnz,
            "dtype": "f32" if info.dtype == SPMV_F32 else "f64",
            "strategy": STRATEGY_NAME[info.strategy], "items_per_thread": info.items_per_thread,
            "items_per_wave": info.items_per_wave, "n_partitions": info.n_partitions,
            "merge_reduce": MERGE_REDUCE_NAME.get(info.merge_reduce, "none"),
            "stream_lanes": info.stream_lanes, "x_window": bool(info.x_window),
            "x_window_intervals": info.x_window, "bin_streams": info.bin_streams,
            "dispatch_order": DISPATCH_ORDER_NAME.get(info.dispatch_order, "partition"),
            "interior_partitions": info.interior_partitions,
            "n_bins": nb, "bin_identity": bool(info.bin_identity),
            "bin_max_len": list(info.bin_max_len[:nb]), "bin_lanes": list(info.bin_lanes[:nb]),
            "bin_count": list(info.bin_count[:nb]), "max_row_len": info.max_row_len,
            "n_empty_rows": info.n_empty_rows, "workspace_bytes": info.workspace_bytes,
            "rgcsr_group": info.rgcsr_group, "rgcsr_stored": info.rgcsr_stored,
            "group_waves": info.group_waves, "group_rows": info.group_rows,
            "plan_allocs": info.plan_allocs, "plan_syncs": info.plan_syncs,
            "tile_rows": info.tile_rows, "tile_blocks": info.tile_blocks,
            "walk_partitions": info.walk_partitions, "x_slabs": info.x_slabs,
            "slab_segments": info.slab_segments, "slab_bytes": info.slab_bytes}


def spmv_plan_copy_splits(plan: int):
    import numpy as np
    P = spmv_plan_info(plan)["n_partitions"]
    rows = np.empty(P + 1, dtype=np.int32)
    nz = np.empty(P + 1, dtype=np.int32)
    _check(load().spmv_plan_copy_splits(plan, rows.ctypes.data, nz.ctypes.data, P + 1),
           "spmv_plan_copy_splits")
    return rows, nz


def spmv_plan_copy_bins(plan: int):
    import numpy as np
    info = spmv_plan_info(plan)
    M = info["M"]
    bins = np.empty(max(M, 1), dtype=np.int32)
    offsets = np.empty(info["n_bins"] + 1, dtype=np.int64)
    _check(load().spmv_plan_copy_bins(plan, bins.ctypes.data, M, offsets.ctypes.data),
           "spmv_plan_copy_bins")
    return bins[:M], offsets


def spmv_status_string(status: int) -> str:
    return load().spmv_status_string(status).decode()


def spmv_last_error() -> str:
    return load().spmv_last_error().decode(errors="replace")


class Plan:
    """A planned CSR matrix: ``Plan(row_ptr, col_idx, values, (M, N))``, then
    ``plan(x, y, alpha, beta)``. Holds references to the borrowed tensors."""

    def __init__(self, row_ptr, col_idx, values, shape, strategy: str = "auto",
                 items_per_thread: int = 0, bins=None, validate_columns: bool = False,
                 merge_reduce: str = "auto", stream_lanes: int = 0, x_window: str = "auto",
                 bin_streams: int = 0, dispatch_order: str = "auto",
                 long_row_tiles: str = "auto", x_slabs: str = "auto",
                 static_matrix: bool = False, stream=None):
        self.M, self.N = int(shape[0]), int(shape[1])
        self._keep = (row_ptr, col_idx, values)
        opts = None
        if (strategy != "auto" or items_per_thread or bins or validate_columns
                or merge_reduce != "auto" or stream_lanes or x_window != "auto" or bin_streams
                or dispatch_order != "auto" or long_row_tiles != "auto" or x_slabs != "auto"
                or static_matrix):
            opts = make_options(strategy, items_per_thread, bins, validate_columns,
                                merge_reduce, stream_lanes, x_window, bin_streams,
                                dispatch_order, long_row_tiles, x_slabs, static_matrix)
        self.handle = spmv_plan(row_ptr, col_idx, values, self.M, self.N, opts, stream)

    @classmethod
    def coo(cls, row_idx, col_idx, values, shape, stream=None, **opts):
        """Plan for a COO matrix sorted by row (see spmv_plan_coo); the same
        options as the CSR constructor."""
        self = cls.__new__(cls)
        self.M, self.N = int(shape[0]), int(shape[1])
        self._keep = (col_idx, values)
        o = make_options(**opts) if opts else None
        self.handle = spmv_plan_coo(row_idx, col_idx, values, self.M, self.N, o, stream)
        return self

    @classmethod
    def transpose(cls, row_ptr, col_idx, values, shape, stream=None, **opts):
        """Plan for y = alpha * A^T x + beta * y, A (shape = (M, N)) in CSR;
        the plan's own shape is (N, M)."""
        self = cls.__new__(cls)
        self.M, self.N = int(shape[1]), int(shape[0])
        self._keep = ()
        o = make_options(**opts) if opts else None
        self.handle = spmv_plan_transpose(row_ptr, col_idx, values, int(shape[0]),
                                          int(shape[1]), o, stream)
        return self

    @classmethod
    def csc(cls, col_ptr, row_idx, values, shape, stream=None, **opts):
        """Plan for y = alpha * A x + beta * y, A (shape = (M, N)) in CSC."""
        self = cls.__new__(cls)
        self.M, self.N = int(shape[0]), int(shape[1])
        self._keep = ()
        o = make_options(**opts) if opts else None
        self.handle = spmv_plan_csc(col_ptr, row_idx, values, self.M, self.N, o, stream)
        return self

    @classmethod
    def rgcsr(cls, row_ptr, col_idx, values, shape, group_rows: int = 0, stream=None):
        """Plan running on a row-grouped CSR copy of A (groups of group_rows
        rows, 0 = 64)."""
        self = cls.__new__(cls)
        self.M, self.N = int(shape[0]), int(shape[1])
        self._keep = (row_ptr, col_idx, values)
        self.handle = spmv_plan_rgcsr(row_ptr, col_idx, values, self.M, self.N, group_rows,
                                      stream)
        return self

    def __call__(self, x, y, alpha: float = 1.0, beta: float = 0.0, stream=None):
        spmv_exec(self.handle, x, y, alpha, beta, stream)
        return y

    def exec_multi(self, X, Y, alpha: float = 1.0, beta: float = 0.0, workspace=None,
                   stream=None):
        """Y = alpha * A X + beta * Y (X: N x k, Y: M x k, row-major). Without
        a workspace the plan keeps one of the needed size (a torch tensor)."""
        if workspace is None:
            need = spmv_spmm_workspace_size(self.handle, int(X.shape[1]))
            if need > 0:
                ws = getattr(self, "_ws", None)
                if ws is None or ws.numel() < need or ws.device != Y.device:
                    self._ws = torch.empty(need, dtype=torch.uint8, device=Y.device)
                workspace = self._ws
        spmv_exec_multi(self.handle, X, Y, alpha, beta, workspace, stream)
        return Y

    def set_strategy(self, strategy: str):
        spmv_plan_set_strategy(self.handle, strategy)

    def update_values(self, values, stream=None):
        """Use `values` from the next call on (see spmv_plan_update_values)."""
        spmv_plan_update_values(self.handle, values, stream)
        if self._keep:
            self._keep = self._keep[:-1] + (values,)

    def set_group(self, group_waves: int = 0, rows_per_group: int = 0):
        spmv_plan_set_group(self.handle, group_waves, rows_per_group)

    @property
    def info(self) -> dict:
        return spmv_plan_info(self.handle)

    def splits(self):
        return spmv_plan_copy_splits(self.handle)

    def bins(self):
        return spmv_plan_copy_bins(self.handle)

    def destroy(self):
        if self.handle:
            h, self.handle = self.handle, None
            spmv_destroy(h)

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass
