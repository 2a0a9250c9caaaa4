"""Host-side contract of bench.py (no GPU): the one-GPU guard and the rule that
counter traffic is reported only for the kernel source it was measured on."""

import json
import os
import subprocess
import sys

import pytest

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, REPO)

import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(REPO, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_counter_traffic_requires_the_measured_source(tmp_path, monkeypatch):
    from depth_wise_attention_block_amd.profiling import aggregate_source_digest

    kernel = "aggregate_kernel<true, 2, 2, 9>"
    summary = {"workload": {"T": 262144, "d": 7168, "S": 9}, "aggregate_source_sha256": aggregate_source_digest(),
               "kernels": {kernel: {"traffic_bytes_per_launch": 123.0}}}
    path = tmp_path / "counters.json"
    path.write_text(json.dumps(summary))
    monkeypatch.setattr(bench, "COUNTERS_FILE", str(path))
    assert bench.counter_traffic(kernel, 262144) == 123.0
    assert bench.counter_traffic(kernel, 4096) is None                 # another workload size
    assert bench.counter_traffic("accumulate_kernel<true, false>", 262144) is None
    summary["aggregate_source_sha256"] = "0" * 64                       # taken on other source
    path.write_text(json.dumps(summary))
    assert bench.counter_traffic(kernel, 262144) is None
    monkeypatch.setattr(bench, "COUNTERS_FILE", str(tmp_path / "missing.json"))
    assert bench.counter_traffic(kernel, 262144) is None


@pytest.mark.parametrize("name", ["aggregate_prefill_t262144_counters.json"])
def test_committed_counter_summary_is_well_formed(name):
    """The committed summary names its commands, its copy calibration and, for
    every kernel, traffic within 1% of the algorithmic bytes."""
    with open(os.path.join(REPO, "profiles", name)) as f:
        c = json.load(f)
    assert c["commands"] and all("rocprofv3 --pmc" in v for run in c["commands"].values() for v in run.values())
    for cal in c["copy_calibration"].values():
        assert abs(cal["fetch_scale"] - 2.0) < 0.01 and abs(cal["write_scale"] - 1.0) < 0.01
    for k, v in c["kernels"].items():
        assert abs(v["traffic_over_algorithmic"] - 1.0) < 0.01, k
