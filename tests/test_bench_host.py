"""Host-side checks of bench.py's byte accounting (no GPU): the slots of the
slice-offset SELL form it assumes when it reports the bytes a product
physically streams, against a brute-force count per 64-row slice."""
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402
from preconditioned_cg_solver_amd import inputs as I  # noqa: E402


def brute_slots(M):
    """Slots of the slice-offset form by definition: per 64-row slice, the
    number of distinct column offsets (col - row) of its rows, times 64."""
    rows = M.row_of_entry()
    total = 0
    for s in range((M.n + 63) // 64):
        sel = (rows >= 64 * s) & (rows < 64 * s + 64)
        offs = set((M.col_idx[sel].astype(np.int64) - rows[sel]).tolist())
        if len(offs) > 8:
            return None
        total += 64 * len(offs)
    return total


@pytest.mark.parametrize("make", [lambda: I.poisson2d(37), lambda: I.poisson3d(13),
                                  lambda: I.heat2d(40)])
def test_slice_offset_slots_match_brute_force(make, monkeypatch):
    monkeypatch.delenv("SLA_SELL_OFS", raising=False)
    M = make()
    got = bench.slice_offset_slots(M)
    assert got is not None
    assert got == (brute_slots(M), (M.n + 63) // 64)


def test_slice_offset_form_rejects_unsorted_and_wide_rows(monkeypatch):
    monkeypatch.delenv("SLA_SELL_OFS", raising=False)
    A = I.poisson2d(24)
    ci, v = A.col_idx.copy(), A.vals.copy()
    a, b = A.row_ptr[100], A.row_ptr[101]
    ci[a:b], v[a:b] = ci[a:b][::-1].copy(), v[a:b][::-1].copy()
    assert bench.slice_offset_slots(I.SparseMatrix(A.n, 1, A.row_ptr, ci, v)) is None
    # a random matrix: far more than 8 distinct offsets per slice
    R = I.random_spd_csr(3000, np.random.default_rng(1), max_deg=12)
    assert brute_slots(R) is None and bench.slice_offset_slots(R) is None
    monkeypatch.setenv("SLA_SELL_OFS", "0")
    assert bench.slice_offset_slots(I.poisson3d(13)) is None


def test_moved_bytes_of_the_slice_offset_form(monkeypatch):
    """Values + one 4-byte offset per slot + one mask byte per row + slice
    starts + six vectors, 26 MB below the per-entry int16 form on 128^3."""
    monkeypatch.delenv("SLA_SELL_OFS", raising=False)
    A = I.poisson3d(128)
    slots, ns = bench.slice_offset_slots(A)
    n = A.n
    assert bench.moved_bytes_a_step(A, n) == slots * 8 + slots // 64 * 4 + ns * 64 \
        + 4 * (ns + 1) + 6 * 8 * n
    monkeypatch.setenv("SLA_SELL_OFS", "0")
    assert bench.moved_bytes_a_step(A, n) - (slots * 8 + slots // 64 * 4 + ns * 64
                                             + 4 * (ns + 1) + 6 * 8 * n) > 25e6
