"""The C ABI library loads, exports every declared symbol and rejects bad
arguments before touching the device (CPU only: no GPU call is made)."""
import ctypes
import os
import re

import pytest

import load_balanced_csr_amd as lb
from load_balanced_csr_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "spmv.h")).read()
    return sorted(set(re.findall(r"SPMV_API\s+[\w\s\*]+?\b(spmv_\w+)\s*\(", src)))


def test_header_and_binding_agree():
    assert declared_functions() == sorted(binding.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = lb.load()
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings():
    for s, text in [(0, "success"), (1, "invalid argument"), (5, "invalid plan handle"),
                    (6, "malformed CSR matrix")]:
        assert lb.spmv_status_string(s) == text


def _plan_raw(M, N, nnz, rp=0x1000, col=0x2000, val=0x3000, dtype=0, out=True):
    lib = lb.load()
    h = ctypes.c_void_p(0xdead)
    st = lib.spmv_plan(ctypes.byref(h) if out else None, M, N, nnz, rp, col, val, dtype, None)
    return st, h.value


@pytest.mark.parametrize("args,status", [
    (dict(M=-1, N=5, nnz=0), 1),
    (dict(M=5, N=-1, nnz=0), 1),
    (dict(M=5, N=5, nnz=-3), 1),
    (dict(M=5, N=5, nnz=3, dtype=7), 1),
    (dict(M=5, N=5, nnz=3, rp=None), 1),
    (dict(M=5, N=5, nnz=3, col=None), 1),
    (dict(M=5, N=5, nnz=3, val=None), 1),
    (dict(M=0, N=5, nnz=3), 1),
    (dict(M=5, N=0, nnz=3), 1),
    (dict(M=5, N=5, nnz=3, out=False), 1),
    (dict(M=2 ** 31, N=5, nnz=3), 2),
    (dict(M=2 ** 30, N=5, nnz=2 ** 30 + 5), 2),
    (dict(M=5, N=5, nnz=2 ** 31), 1),          # nnz beyond int32 indices
    (dict(M=5, N=5, nnz=2 ** 31 - 64 - 5), 2),  # M + nnz = 2^31 - 64: past the limit
])
def test_plan_rejects_bad_arguments(args, status):
    st, h = _plan_raw(**args)
    assert st == status, lb.spmv_last_error()
    if args.get("out", True):
        assert h is None  # *out set to NULL on failure


def test_plan_alloc_failure_is_reported(monkeypatch):
    monkeypatch.setenv("SPMV_TEST_FAIL_ALLOC", "1")
    st, h = _plan_raw(M=10, N=10, nnz=20)
    assert st == 3 and h is None
    assert "SPMV_TEST_FAIL_ALLOC" in lb.spmv_last_error()


def test_bad_options_rejected():
    lib = lb.load()
    h = ctypes.c_void_p()
    for kw in (dict(items_per_thread=5), dict(strategy="merge", bins=[(4, 3), (0, 64)]),
               dict(bins=[(8, 1), (4, 2), (0, 64)])):
        o = lb.make_options(**kw)
        st = lib.spmv_plan_ex(ctypes.byref(h), 10, 10, 20, 0x1000, 0x2000, 0x3000, 0,
                              ctypes.byref(o), None)
        assert st == 1, kw
    # per-bin streams beyond the bin count, dispatch orders that do not exist
    for field, bad in (("bin_streams", 9), ("bin_streams", -1), ("dispatch_order", 3),
                       ("dispatch_order", -1), ("x_slabs", 3), ("x_slabs", -1),
                       ("static_matrix", 2)):
        o = lb.make_options()
        setattr(o, field, bad)
        st = lib.spmv_plan_ex(ctypes.byref(h), 10, 10, 20, 0x1000, 0x2000, 0x3000, 0,
                              ctypes.byref(o), None)
        assert st == 1, (field, bad)
        assert field in lb.spmv_last_error()


def test_exec_and_destroy_reject_foreign_handles():
    lib = lb.load()
    assert lib.spmv_exec(None, 0x10, 0x20, 1.0, 0.0, None) == 5
    assert lib.spmv_exec(0x12345678, 0x10, 0x20, 1.0, 0.0, None) == 5
    assert lib.spmv_destroy(0x12345678) == 5
    assert lib.spmv_destroy(None) == 0
    assert lib.spmv_plan_update_values(None, 0x1000, None) == 5
    assert lib.spmv_plan_update_values(0x12345678, 0x1000, None) == 5
    info = binding.PlanInfo()
    assert lib.spmv_plan_info(0x12345678, ctypes.byref(info)) == 5
    with pytest.raises(lb.SpmvError) as e:
        lb.spmv_plan_info(0x12345678)
    assert e.value.status == 5


def test_library_has_no_undefined_symbols_of_its_own():
    """Every kernel the library launches has its host stub linked in (a
    device-only builtin in a kernel body once made the host pass drop them)."""
    import subprocess
    out = subprocess.check_output(["nm", "-D", "--undefined-only", lb.LIB_PATH]).decode()
    own = [l for l in out.splitlines() if "spmv" in l]
    assert not own, own[:5]


def test_struct_layouts_match_the_header(tmp_path):
    # sizes and field offsets of the option and info structs as the C
    # compiler lays them out, against the binding's ctypes mirrors
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("no C compiler or ROCm headers")
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "spmv.h"', 'int main(void) {']
    for cname, py in (("spmv_plan_options_t", binding.PlanOptions),
                      ("spmv_plan_info_t", binding.PlanInfo)):
        lines.append('printf("%s size %%zu\\n", sizeof(%s));' % (cname, cname))
        for fname, _ in py._fields_:
            lines.append('printf("%s %s %%zu\\n", offsetof(%s, %s));' % (cname, fname, cname, fname))
    lines += ["return 0; }"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    r = subprocess.run([cc, "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                        "-I", "/opt/rocm/include", str(src), "-o", str(exe)],
                       capture_output=True, text=True)
    if r.returncode != 0:
        pytest.skip("header does not compile as C here: " + r.stderr[:200])
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split("\n")
    got = {tuple(l.split()[:2]): int(l.split()[2]) for l in out if l}
    for cname, py in (("spmv_plan_options_t", binding.PlanOptions),
                      ("spmv_plan_info_t", binding.PlanInfo)):
        assert got[(cname, "size")] == ctypes.sizeof(py), cname
        for fname, _ in py._fields_:
            assert got[(cname, fname)] == getattr(py, fname).offset, (cname, fname)


def _noalloc_raw(M, N, nnz, dtype=0, rp=0x1000, col=0x2000, val=0x3000, x=0x4000, y=0x8000):
    lib = lb.load()
    return lib.spmv_exec_noalloc(M, N, nnz, rp, col, val, dtype, x, y, 1.0, 0.0, None)


@pytest.mark.parametrize("args,status", [
    (dict(M=-1, N=5, nnz=0), 1),
    (dict(M=5, N=5, nnz=3, dtype=9), 1),
    (dict(M=5, N=5, nnz=2 ** 31), 1),
    (dict(M=5, N=5, nnz=3, rp=None), 1),
    (dict(M=5, N=5, nnz=3, rp=0x1004), 1),                 # misaligned
    (dict(M=5, N=5, nnz=3, x=0x8008), 1),                  # x overlaps y
    (dict(M=2 ** 31 - 100, N=5, nnz=0), 2),                # beyond the scratch (fp32)
    (dict(M=700_000_000, N=5, nnz=0, dtype=1), 2),         # beyond the scratch (fp64)
])
def test_noalloc_rejects_before_any_device_call(args, status):
    """Sizes and pointers are checked on the host first; none of these
    reaches a HIP call (this container has no GPU)."""
    assert _noalloc_raw(**args) == status, lb.spmv_last_error()
