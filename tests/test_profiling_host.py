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


@pytest.mark.parametrize("label", ["schedule_93_t32768_two_phase", "schedule_93_t32768_backward",
                                   "many_sources_s94_t32768"])
def test_bench_reports_pass_traffic_only_on_the_sources_it_was_taken_on(label):
    """``bench.pass_traffic``: the committed summary's bytes while the sources
    its kernels are built from are unchanged (their SHA-256 is recorded), else
    None; never at another T."""
    import json
    import os

    import bench
    with open(os.path.join(os.path.dirname(bench.__file__), "profiles", f"{label}_counters.json")) as f:
        c = json.load(f)
    current = c["source_sha256"] == P.pass_source_digest(label)
    expected = c["pass"]["traffic_bytes"] if current else None
    assert bench.pass_traffic(label, 32768) == expected
    assert bench.pass_traffic(label, 4096) is None
