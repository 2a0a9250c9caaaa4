"""The whole-pass counter summary (``profiling.pass_summary``) on small
hand-made counter files: calibration by the last plain copy, only the
dispatches after it counted, per-kernel sums.  CPU only."""

import csv

import pytest

from depth_wise_attention_block_amd import profiling as P

T, D = 4, 8
ROW_KIB = 2 * T * D / 1024          # one bf16 row of T x D, in KiB


def _write(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for i, (name, value) in enumerate(rows):
            w.writerow([i + 1, name, counter, value])


def test_pass_summary_counts_only_after_the_last_copy(tmp_path):
    copy = f"void attnres::{P.COPY_KERNEL}(args)"
    # FETCH_SIZE reads half the bytes a copy moves, WRITE_SIZE all of them
    fetch = [("setup()", 50.0), (copy, ROW_KIB / 2), ("stale()", 9.0), (copy, ROW_KIB / 2),
             ("k_a(x)", 3 * ROW_KIB / 2), ("k_b(y)", ROW_KIB / 2), ("k_a(x)", ROW_KIB / 2)]
    write = [("setup()", 50.0), (copy, ROW_KIB), ("stale()", 9.0), (copy, ROW_KIB),
             ("k_a(x)", ROW_KIB), ("k_b(y)", 2 * ROW_KIB), ("k_a(x)", 0.0)]
    _write(tmp_path / "f.csv", "FETCH_SIZE", fetch)
    _write(tmp_path / "w.csv", "WRITE_SIZE", write)
    row = 2 * T * D
    s = P.pass_summary(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), "cf", "cw", T, D,
                       algorithmic=8 * row, label="x")
    assert s["copy_calibration"]["fetch_scale"] == pytest.approx(2.0)
    assert s["copy_calibration"]["write_scale"] == pytest.approx(1.0)
    assert s["pass"]["fetch_bytes"] == pytest.approx(5 * row)
    assert s["pass"]["write_bytes"] == pytest.approx(3 * row)
    assert s["pass"]["traffic_over_algorithmic"] == pytest.approx(1.0)
    assert s["pass"]["launches"] == 3
    assert s["kernels"]["k_a"]["launches"] == 2
    assert s["kernels"]["k_a"]["fetch_bytes"] == pytest.approx(4 * row)
    assert s["kernels"]["k_b"]["write_bytes"] == pytest.approx(2 * row)
    assert "stale" not in s["kernels"] and "setup" not in s["kernels"]


def test_pass_summary_needs_a_copy(tmp_path):
    _write(tmp_path / "f.csv", "FETCH_SIZE", [("k_a(x)", 1.0)])
    _write(tmp_path / "w.csv", "WRITE_SIZE", [("k_a(x)", 1.0)])
    with pytest.raises(SystemExit):
        P.pass_summary(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), "", "", T, D, 1, "x")
