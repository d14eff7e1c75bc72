"""The CPU oracle against facts that do not come from it (CPU only)."""
import numpy as np
import pytest

import oracle
import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(oracle._default())


def test_worked_example_structure(golden):
    """The worked CSR example: the row pointers read off the page reproduce
    every count the page prints about that matrix."""
    g = golden("rgcsr_worked_example.txt")
    rp = np.array(g["first_entry_positions"] + g["nnz"])
    assert list(rp) == g["row_ptr"]
    L = np.diff(rp)
    M = L.size
    assert L.sum() == g["nnz"][0] == 13
    assert M * L.max() - L.sum() == g["ellpack_artificial_zeros"][0]
    gs = g["rgcsr_group_size"][0]
    pad = sum(gs * L[k:k + gs].max() - L[k:k + gs].sum() for k in range(0, M, gs))
    assert pad == g["rgcsr_artificial_zeros"][0]
    assert g["bcsr_stored"][0] - g["nnz"][0] == g["bcsr_artificial_zeros"][0]


def test_fig1_tiles_fixture(golden):
    g = golden("loadbalance_fig1_tiles.txt")
    assert list(np.concatenate([[0], np.cumsum(g["atoms_per_tile"])])) == g["row_ptr"]


def test_acceptance_rule_rejects_planted_errors():
    """The acceptance rule itself: a result off by 2*rtol*scale in one row,
    a wrong empty row, or a NaN must each be rejected."""
    rp, col, val, x, y0 = pins._small_random(11)
    ref, scale = oracle.spmv(rp, col, val, x, 1.5, 0.5, y0)
    y = ref.astype(np.float32)
    ok, worst, _ = oracle.within_tolerance(y, ref, scale, 1.5, 0.5, y0, row_ptr=rp)
    assert ok and worst <= 1.0
    full = np.flatnonzero(np.diff(rp) > 3)[0]
    bad = y.copy()
    bad[full] = np.float32(ref[full] + 2e-5 * (1.5 * scale[full] + 0.5 * abs(y0[full])) * 1.01)
    assert not oracle.within_tolerance(bad, ref, scale, 1.5, 0.5, y0, row_ptr=rp)[0]
    empty = np.flatnonzero(np.diff(rp) == 0)[0]
    bad = y.copy()
    bad[empty] = np.nextafter(bad[empty], np.float32(np.inf))
    assert not oracle.within_tolerance(bad, ref, scale, 1.5, 0.5, y0, row_ptr=rp)[0]
    bad = y.copy()
    bad[full] = np.nan
    assert not oracle.within_tolerance(bad, ref, scale, 1.5, 0.5, y0, row_ptr=rp)[0]
