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


def _fake_counter_run(d, counter, rows):
    """A rocprofv3 counter_collection.csv with the given (kernel, value) rows."""
    import csv
    os.makedirs(d / "host", exist_ok=True)
    with open(d / "host" / "pmc_counter_collection.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"])
        for i, (k, v) in enumerate(rows):
            w.writerow([i, k, 256, counter, v])


def test_counter_summary_calibrates_by_the_copy(tmp_path):
    """Per-kernel bytes = mean counter KiB per dispatch x 1024 x the factor that
    makes the 256 MiB copy read and write 256 MiB; the L2 hit rate is
    HIT / (HIT + MISS) summed over the dispatches."""
    copy = "void at::native::copyBuffer<double>(...)"
    step = "void sla::(anonymous namespace)::sell_step<double, 2, true, true, 8, true>(...)"
    fetch, write, l2 = tmp_path / "f", tmp_path / "w", tmp_path / "l2"
    # the copy reads 2x and writes 3x what the counters report; the step's two
    # dispatches report 1000 and 3000 KiB fetched, 10 and 30 KiB written
    _fake_counter_run(fetch, "FETCH_SIZE", [(copy, 128 * 1024.0), (step, 1000.0), (step, 3000.0)])
    _fake_counter_run(write, "WRITE_SIZE", [(copy, 256 * 1024.0 / 3), (step, 10.0), (step, 30.0)])
    import csv
    os.makedirs(l2 / "host")
    with open(l2 / "host" / "pmc_counter_collection.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"])
        w.writerows([[0, step, 256, "TCC_HIT_sum", 30], [0, step, 256, "TCC_MISS_sum", 70],
                     [1, step, 256, "TCC_HIT_sum", 10], [1, step, 256, "TCC_MISS_sum", 90]])
    bench.summarize_counters(str(fetch), str(write), str(l2), workload="fake", out_dir=tmp_path)
    import json
    rec = json.load(open(tmp_path / "traffic_fake.json"))
    assert rec["fetch_scale"] == pytest.approx(2.0) and rec["write_scale"] == pytest.approx(3.0)
    k = rec["kernels"]["sell_step<double, 2, true, true, 8, true>"]
    assert k["dispatches"] == 2
    assert k["fetch_bytes"] == pytest.approx(2000.0 * 1024 * 2.0)
    assert k["write_bytes"] == pytest.approx(20.0 * 1024 * 3.0)
    assert k["l2_hit_rate"] == pytest.approx(0.2)
    assert k["source"] == "solver.hip"
    assert bench.kernel_bytes(rec, r"sell_step<\w+, 2[,>]") == pytest.approx(k["bytes"])
    assert bench.kernel_bytes(rec, r"sell_step<\w+, 4[,>]") is None
    assert "A step" in open(tmp_path / "traffic_fake.md").read()


def test_column_block_launches_take_their_reduction_mode():
    """The column-block pass is one kernel for every step; the summaries name
    each launch by the reduction launched after it."""
    keys = ["vec_p_update<double, 2>", "csr_blk_step<double, true>", "blk_reduce<double, 8>",
            "vec_r_update<double>", "csr_blk_step<double, true>", "blk_reduce<double, 9>",
            "csr_blk_step<double, false>", "blk_reduce<double, 6>", "csr_blk_step<double, true>"]
    out = bench._pair_blocks(keys)
    assert out[1] == "csr_blk_step<double, 8>"
    assert out[4] == "csr_blk_step<double, 9>"
    assert out[6] == "csr_blk_step<double, 6>"
    assert out[8] == "csr_blk_step<double, true>"  # no reduction after it: unchanged
    assert out[0] == keys[0] and out[2] == keys[2]
    assert bench._describe("csr_blk_step<double, 8>").startswith("column blocks of the A product")
    assert "G step" in bench._describe("blk_reduce<double, 6>")
