"""Load-balanced CSR sparse matrix-vector multiplication for AMD MI355X.

y = alpha * A x + beta * y with A in CSR (int32 row_ptr/col_idx, fp32 or fp64
values), computed by hand-written gfx950 HIP kernels in libspmv.so: a
merge-path schedule over rows + nonzeros with a carry fix-up, and a binned
schedule (thread / lane-group / wavefront / workgroup per row); and the
multi-vector form Y = alpha * A X + beta * Y over the same plan. This package
is a thin ctypes binding over the C ABI declared in include/spmv.h.
"""
from .binding import (EXPORTED, LIB_PATH, Plan, PlanOptions, SpmvError, load, make_options,
                      spmv_destroy, spmv_exec, spmv_exec_events, spmv_last_error, spmv_plan,
                      spmv_plan_copy_bins, spmv_plan_copy_splits, spmv_plan_info,
                      spmv_plan_set_strategy, spmv_read_probe, spmv_status_string,
                      spmv_exec_multi, spmv_spmm_workspace_size, spmv_plan_coo,
                      spmv_plan_transpose, spmv_plan_csc, spmv_plan_rgcsr,
                      spmv_plan_set_group, spmv_gather_probe, spmv_gather_rows_probe,
                      spmv_stream_probe, spmv_exec_noalloc)

__all__ = ["EXPORTED", "LIB_PATH", "Plan", "PlanOptions", "SpmvError", "load", "make_options",
           "spmv_destroy", "spmv_exec", "spmv_exec_events", "spmv_last_error", "spmv_plan",
           "spmv_plan_copy_bins", "spmv_plan_copy_splits", "spmv_plan_info",
           "spmv_plan_set_strategy", "spmv_read_probe", "spmv_status_string",
           "spmv_exec_multi", "spmv_spmm_workspace_size", "spmv_plan_coo",
           "spmv_plan_transpose", "spmv_plan_csc", "spmv_plan_rgcsr",
           "spmv_plan_set_group", "spmv_gather_probe", "spmv_gather_rows_probe",
           "spmv_stream_probe", "spmv_exec_noalloc"]
