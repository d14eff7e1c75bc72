"""Helpers for the GPU tests: move a workload to the device, run the C ABI
through the binding, compare with the oracle."""
import sys

import numpy as np
import torch

import oracle
import load_balanced_csr_amd as lb

# plan options of the schedule variants every parity case runs through
VARIANTS = {
    # merge-path; the reduction is "stream" where every row fits T/8, else "walk"
    "merge4": dict(strategy="merge", items_per_thread=4),
    "merge8": dict(strategy="merge", items_per_thread=8),
    "merge16": dict(strategy="merge", items_per_thread=16),
    # merge-path with the exact split and per-lane walk on every matrix
    "merge8_walk": dict(strategy="merge", items_per_thread=8, merge_reduce="walk"),
    # stream reduction with other lane-group widths (ignored when walk applies)
    "merge8_g1": dict(strategy="merge", items_per_thread=8, stream_lanes=1),
    "merge16_g16": dict(strategy="merge", items_per_thread=16, stream_lanes=16),
    "merge8_g64": dict(strategy="merge", items_per_thread=8, stream_lanes=64),
    "merge4_g8": dict(strategy="merge", items_per_thread=4, stream_lanes=8),
    # stream reduction with the workgroup's x window forced on / off (a block
    # whose column span does not fit still gathers from HBM)
    "merge8_xwin": dict(strategy="merge", items_per_thread=8, x_window="on"),
    "merge4_xwin": dict(strategy="merge", items_per_thread=4, x_window="on", stream_lanes=2),
    "merge8_noxwin": dict(strategy="merge", items_per_thread=8, x_window="off"),
    "merge7": dict(strategy="merge", items_per_thread=7),
    "merge7_xwin": dict(strategy="merge", items_per_thread=7, x_window="on", stream_lanes=4),
    "merge16_xwin": dict(strategy="merge", items_per_thread=16, x_window="on", stream_lanes=8),
    # declared static: the plan may keep a copy of A (x slabs where they pay)
    "static": dict(static_matrix=True),
    "binned": dict(strategy="binned"),
    # other bin edges: correctness must not depend on them
    "binned_alt": dict(strategy="binned",
                       bins=[(1, 1), (6, 4), (40, 16), (900, 64), (None, 256)]),
    "binned_one": dict(strategy="binned", bins=[(None, 8)]),
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


class DevMatrix:
    def __init__(self, row_ptr, col_idx, values, M, N):
        self.M, self.N = M, N
        self.row_ptr_h, self.col_h, self.val_h = row_ptr, col_idx, values
        self.rp, self.col, self.val = dev(row_ptr), dev(col_idx), dev(values)

    @classmethod
    def of(cls, w):
        return cls(w.row_ptr, w.col_idx, w.values, w.M, w.N)

    def plan(self, variant="merge8", **kw):
        opts = dict(VARIANTS[variant]) if variant else {}
        opts.update(kw)
        return lb.Plan(self.rp, self.col, self.val, (self.M, self.N), **opts)


def run(plan, x_h, alpha, beta, y0_h=None, dtype=np.float32):
    """One exec; y starts as y0 (beta != 0) or NaN (beta == 0, must not be read)."""
    x = dev(x_h)
    M = plan.M
    if beta != 0.0:
        y = dev(y0_h)
    else:
        y = torch.full((M,), float("nan"), dtype=torch.float32 if dtype == np.float32
                       else torch.float64, device="cuda")
    plan(x, y, alpha, beta)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def check(y, row_ptr, col_idx, values, x, alpha, beta, y0=None, what=""):
    ref, scale = oracle.spmv(row_ptr, col_idx, values, x, alpha, beta, y0)
    ok, worst, idx = oracle.within_tolerance(y, ref, scale, alpha, beta, y0, row_ptr=row_ptr)
    if not ok:
        L = int(row_ptr[idx + 1] - row_ptr[idx]) if idx >= 0 else -1
        raise AssertionError("%s: row %d (len %d) y=%r ref=%r scale=%r worst=%.3g" %
                             (what, idx, L, y[idx], ref[idx], scale[idx], worst))
    return worst
