"""Turn rocprofv3 output into the short summaries kept under ``profiles/``.

    python -m depth_wise_attention_block_amd.profiling trace  --csv KERNEL_STATS.csv --cmd "..." --out X.txt
    python -m depth_wise_attention_block_amd.profiling trace  --db RESULTS.db       --cmd "..." --out X.txt
    python -m depth_wise_attention_block_amd.profiling counters --fetch FETCH.csv --write WRITE.csv \
        --cmd-fetch "..." --cmd-write "..." --out X.json

``counters`` calibrates each counter with the plain-copy kernel that
``bench.py --with-copy`` launches (it moves a known T*d bf16 in and out), and
records the HBM bytes per aggregation launch together with the SHA-256 of the
kernel source it was taken on; ``bench.py`` reports that traffic only while the
source is unchanged.
"""

from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import json
import os
import sqlite3

HERE = os.path.dirname(os.path.abspath(__file__))
AGG_SOURCE = os.path.join(HERE, "csrc", "aggregate.hip")

COPY_KERNEL = "accumulate_kernel<true, true>"
RMW_KERNEL = "accumulate_kernel<true, false>"
AGG_KERNEL = "aggregate_kernel<true, 2>"


def _short(name: str) -> str:
    for prefix in ("void ", "attnres::", "(anonymous namespace)::"):
        name = name.replace(prefix, "")
    return name.split("(")[0].strip()


def kernel_stats_from_db(db_path: str):
    db = sqlite3.connect(db_path)
    rows = db.execute("select name, total_calls, total_duration, average from top_kernels").fetchall()
    return [(n, int(c), float(tot), float(avg)) for n, c, tot, avg in rows]  # the view reports microseconds


def kernel_stats_from_csv(csv_path: str):
    out = []
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            out.append((r["Name"], int(r["Calls"]), float(r["TotalDurationNs"]) / 1e3, float(r["AverageNs"]) / 1e3))
    return out


def write_trace_summary(stats, cmd: str, out_path: str, top: int = 8) -> None:
    lines = [f"# rocprofv3 kernel-trace summary", f"# command: {cmd}", "#",
             f"# {'kernel':<60} {'calls':>6} {'total_us':>12} {'avg_us':>10}"]
    for name, calls, tot, avg in sorted(stats, key=lambda r: -r[2])[:top]:
        lines.append(f"  {_short(name)[:60]:<60} {calls:>6} {tot:>12.1f} {avg:>10.1f}")
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")


def _per_kernel(csv_path: str, counter: str):
    vals = collections.defaultdict(list)
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter:
                vals[_short(r["Kernel_Name"])].append(float(r["Counter_Value"]))
    return vals


def counters_summary(fetch_csv: str, write_csv: str, T: int, d: int, S: int, cmd_fetch: str, cmd_write: str):
    fetch = _per_kernel(fetch_csv, "FETCH_SIZE")
    write = _per_kernel(write_csv, "WRITE_SIZE")
    kib = 1024.0
    copy_bytes = 2 * T * d                       # the copy reads and writes T*d bf16
    f_copy = sum(fetch[COPY_KERNEL]) / len(fetch[COPY_KERNEL]) * kib
    w_copy = sum(write[COPY_KERNEL]) / len(write[COPY_KERNEL]) * kib
    f_scale, w_scale = copy_bytes / f_copy, copy_bytes / w_copy
    agg_f = sum(fetch[AGG_KERNEL]) / len(fetch[AGG_KERNEL]) * kib * f_scale
    agg_w = sum(write[AGG_KERNEL]) / len(write[AGG_KERNEL]) * kib * w_scale
    alg_read = 2 * S * T * d + 4 * d
    alg_write = 2 * T * d + 4 * T * S
    out = {
        "kernel": AGG_KERNEL, "workload": {"T": T, "d": d, "S": S},
        "commands": {"FETCH_SIZE": cmd_fetch, "WRITE_SIZE": cmd_write},
        "copy_calibration": {"bytes_moved_each_way": copy_bytes, "fetch_kib": f_copy / kib, "write_kib": w_copy / kib,
                             "fetch_scale": f_scale, "write_scale": w_scale},
        "fetch_kib_per_launch_raw": agg_f / kib / f_scale, "write_kib_per_launch_raw": agg_w / kib / w_scale,
        "fetch_bytes_per_launch": agg_f, "write_bytes_per_launch": agg_w,
        "traffic_bytes_per_launch": agg_f + agg_w,
        "algorithmic_read_bytes": alg_read, "algorithmic_write_bytes": alg_write,
        "traffic_over_algorithmic": (agg_f + agg_w) / (alg_read + alg_write),
        "aggregate_source_sha256": hashlib.sha256(open(AGG_SOURCE, "rb").read()).hexdigest(),
    }
    if RMW_KERNEL in fetch and RMW_KERNEL in write:
        out["accumulate_rmw_bytes_per_launch"] = (sum(fetch[RMW_KERNEL]) / len(fetch[RMW_KERNEL]) * kib * f_scale
                                                  + sum(write[RMW_KERNEL]) / len(write[RMW_KERNEL]) * kib * w_scale)
    return out


def main():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = p.add_subparsers(dest="what", required=True)
    t = sub.add_parser("trace")
    t.add_argument("--db")
    t.add_argument("--csv")
    t.add_argument("--cmd", required=True)
    t.add_argument("--out", required=True)
    c = sub.add_parser("counters")
    c.add_argument("--fetch", required=True)
    c.add_argument("--write", required=True)
    c.add_argument("--cmd-fetch", required=True)
    c.add_argument("--cmd-write", required=True)
    c.add_argument("--T", type=int, default=262144)
    c.add_argument("--d", type=int, default=7168)
    c.add_argument("--S", type=int, default=9)
    c.add_argument("--out", required=True)
    a = p.parse_args()
    if a.what == "trace":
        stats = kernel_stats_from_db(a.db) if a.db else kernel_stats_from_csv(a.csv)
        write_trace_summary(stats, a.cmd, a.out)
    else:
        s = counters_summary(a.fetch, a.write, a.T, a.d, a.S, a.cmd_fetch, a.cmd_write)
        with open(a.out, "w") as f:
            json.dump(s, f, indent=1)
            f.write("\n")


if __name__ == "__main__":
    main()
