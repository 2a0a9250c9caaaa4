"""Turn rocprofv3 output into the short summaries kept under ``profiles/``.

    python -m depth_wise_attention_block_amd.profiling trace  --csv KERNEL_STATS.csv --cmd "..." --out X.txt
    python -m depth_wise_attention_block_amd.profiling trace  --db RESULTS.db       --cmd "..." --out X.txt
    python -m depth_wise_attention_block_amd.profiling counters \
        --run LABEL FETCH.csv WRITE.csv "fetch command" "write command" [--run ...] --out X.json

    python -m depth_wise_attention_block_amd.profiling pass \
        --fetch FETCH.csv --write WRITE.csv --fetch-cmd "..." --write-cmd "..." \
        --T T --d D --algorithmic BYTES --label NAME --out X.json
    python -m depth_wise_attention_block_amd.profiling markers --csv MARKER_API_TRACE.csv --cmd "..." --out X.txt

``counters`` calibrates each counter with the plain-copy kernel that
``bench.py --with-copy`` launches in every run (it moves a known T*d bf16 in and
out), and records the HBM bytes per launch of each kernel together with the
SHA-256 of the sources the aggregation kernel is compiled from;
``bench.py`` reports that traffic only while those sources are unchanged.
``pass`` does the same for a whole multi-launch pass (a schedule forward or
backward run once after one copy): it sums the calibrated bytes of every
dispatch after the last copy and sets them against the pass's algorithmic
bytes, with a per-kernel breakdown.
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
# every file the aggregation kernels are compiled from, and launch_policy.h,
# which picks their launch shape (threads, grid, token order): a change to any
# of them makes committed counter bytes stale
AGG_SOURCES = tuple(os.path.join(HERE, "csrc", f)
                    for f in ("aggregate.hip", "device_common.h", "internal.h", "launch_policy.h"))


# every file the kernels of one whole pass are compiled from, plus the launch
# policy (capi.cpp sizes the backward's grids and workspaces itself)
PASS_SOURCES = {
    "schedule_93_t32768_two_phase": ("aggregate.hip", "twophase.hip", "device_common.h", "internal.h",
                                     "launch_policy.h"),
    "schedule_93_t32768_backward": ("backward.hip", "device_common.h", "internal.h", "launch_policy.h",
                                    "capi.cpp"),
    "many_sources_s94_t32768": ("aggregate.hip", "device_common.h", "internal.h", "launch_policy.h"),
}


def source_digest(paths) -> str:
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def aggregate_source_digest() -> str:
    return source_digest(AGG_SOURCES)


def pass_source_digest(label: str):
    """SHA-256 of the sources of the pass ``label``, or None for an unknown pass."""
    files = PASS_SOURCES.get(label)
    return None if files is None else source_digest(os.path.join(HERE, "csrc", f) for f in files)

COPY_KERNEL = "accumulate_kernel<true, true>"


def algorithmic_bytes(kernel: str, T: int, d: int, S: int):
    """(read, write) bytes each kernel must move at S sources, bf16, or None."""
    row = 2 * T * d
    table = {
        "aggregate_kernel<true, 2, 0, 9>": (S * row + 4 * d, row + 4 * T * S),
        "aggregate_kernel<true, 2, 1, 9>": ((S - 1) * row + row + 4 * d, 2 * row + 4 * T * S),
        "aggregate_kernel<true, 2, 2, 9>": ((S - 1) * row + 2 * row + 4 * d, 2 * row + 4 * T * S),
        "accumulate_kernel<true, false>": (2 * row, row),
        "accumulate_kernel<true, true>": (row, row),
    }
    return table.get(kernel)


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


def dispatch_durations(trace_csv: str, match: str, last: int):
    """Durations (us) of the last ``last`` dispatches whose kernel name contains
    ``match``, in launch order, from a ``*_kernel_trace.csv``."""
    rows = []
    with open(trace_csv) as f:
        for r in csv.DictReader(f):
            if match in r["Kernel_Name"]:
                rows.append((int(r["Start_Timestamp"]), _short(r["Kernel_Name"]),
                             (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3))
    rows.sort()
    return [(n, d) for _, n, d in rows[-last:]]


def write_trace_summary(stats, cmd: str, out_path: str, top: int = 8, dispatches=None) -> None:
    lines = [f"# rocprofv3 kernel-trace summary", f"# command: {cmd}", "#",
             f"# {'kernel':<60} {'calls':>6} {'total_us':>12} {'avg_us':>10}"]
    for name, calls, tot, avg in sorted(stats, key=lambda r: -r[2])[:top]:
        lines.append(f"  {_short(name)[:60]:<60} {calls:>6} {tot:>12.1f} {avg:>10.1f}")
    if dispatches:
        lines += ["#", "# last dispatches in launch order (us):"]
        lines += [f"  {n[:60]:<60} {d:>10.1f}" for n, d in dispatches]
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")


def _per_kernel(csv_path: str, counter: str):
    vals = collections.defaultdict(list)
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter:
                vals[_short(r["Kernel_Name"])].append(float(r["Counter_Value"]))
    return vals


def counters_summary(runs, T: int, d: int, S: int):
    """``runs``: list of (label, fetch_csv, write_csv, fetch_cmd, write_cmd).
    Each run is calibrated by its own copy kernel; kernels seen in several runs
    keep the first run's figures."""
    kib = 1024.0
    mean = lambda v: sum(v) / len(v)
    copy_bytes = 2 * T * d                       # the copy reads and writes T*d bf16
    commands, calibration, kernels = {}, {}, {}
    for label, fetch_csv, write_csv, cmd_fetch, cmd_write in runs:
        fetch = _per_kernel(fetch_csv, "FETCH_SIZE")
        write = _per_kernel(write_csv, "WRITE_SIZE")
        f_scale = copy_bytes / (mean(fetch[COPY_KERNEL]) * kib)
        w_scale = copy_bytes / (mean(write[COPY_KERNEL]) * kib)
        commands[label] = {"FETCH_SIZE": cmd_fetch, "WRITE_SIZE": cmd_write}
        calibration[label] = {"kernel": COPY_KERNEL, "bytes_moved_each_way": copy_bytes,
                              "fetch_scale": f_scale, "write_scale": w_scale}
        for name in sorted(set(fetch) & set(write)):
            if name in kernels or not name.startswith(("aggregate_kernel", "accumulate_kernel")):
                continue
            fb = mean(fetch[name]) * kib * f_scale
            wb = mean(write[name]) * kib * w_scale
            entry = {"run": label, "fetch_kib_raw": mean(fetch[name]), "write_kib_raw": mean(write[name]),
                     "fetch_bytes_per_launch": fb, "write_bytes_per_launch": wb,
                     "traffic_bytes_per_launch": fb + wb, "launches": len(fetch[name])}
            alg = algorithmic_bytes(name, T, d, S)
            if alg is not None:
                entry.update({"algorithmic_read_bytes": alg[0], "algorithmic_write_bytes": alg[1],
                              "traffic_over_algorithmic": (fb + wb) / (alg[0] + alg[1])})
            kernels[name] = entry
    return {
        "workload": {"T": T, "d": d, "S": S},
        "commands": commands,
        "copy_calibration": calibration,
        "kernels": kernels,
        "aggregate_sources": [os.path.relpath(p, os.path.dirname(HERE)) for p in AGG_SOURCES],
        "aggregate_source_sha256": aggregate_source_digest(),
    }


def _per_dispatch(csv_path: str, counter: str):
    """[(dispatch id, short kernel name, value)] in dispatch order."""
    rows = {}
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter:
                rows[int(r["Dispatch_Id"])] = (_short(r["Kernel_Name"]), float(r["Counter_Value"]))
    return [(i, n, v) for i, (n, v) in sorted(rows.items())]


def pass_summary(fetch_csv: str, write_csv: str, fetch_cmd: str, write_cmd: str, T: int, d: int,
                 algorithmic: int, label: str):
    """Counter bytes of every dispatch after the last plain copy (one pass of a
    multi-launch workload), calibrated by that copy, against ``algorithmic``."""
    kib = 1024.0
    copy_bytes = 2 * T * d
    per_kernel, calib = collections.OrderedDict(), {}
    total = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        disp = _per_dispatch(path, counter)
        copies = [k for k, (_, n, _) in enumerate(disp) if n == COPY_KERNEL]
        if not copies:
            raise SystemExit(f"{path}: no {COPY_KERNEL} dispatch to calibrate {counter} with")
        scale = copy_bytes / (disp[copies[-1]][2] * kib)
        calib[counter] = scale
        after = disp[copies[-1] + 1:]
        total[counter] = sum(v for _, _, v in after) * kib * scale
        for _, name, v in after:
            e = per_kernel.setdefault(name, {"launches": 0, "FETCH_SIZE": 0.0, "WRITE_SIZE": 0.0})
            e[counter] += v * kib * scale
            if counter == "FETCH_SIZE":
                e["launches"] += 1
    traffic = total["FETCH_SIZE"] + total["WRITE_SIZE"]
    return {
        "workload": label, "T": T, "d": d,
        "sources": [f"depth_wise_attention_block_amd/csrc/{f}" for f in PASS_SOURCES.get(label, ())],
        "source_sha256": pass_source_digest(label),
        "commands": {"FETCH_SIZE": fetch_cmd, "WRITE_SIZE": write_cmd},
        "copy_calibration": {"kernel": COPY_KERNEL, "bytes_moved_each_way": copy_bytes,
                             "fetch_scale": calib["FETCH_SIZE"], "write_scale": calib["WRITE_SIZE"]},
        "pass": {"fetch_bytes": total["FETCH_SIZE"], "write_bytes": total["WRITE_SIZE"], "traffic_bytes": traffic,
                 "algorithmic_bytes": algorithmic, "traffic_over_algorithmic": traffic / algorithmic,
                 "launches": sum(e["launches"] for e in per_kernel.values())},
        "kernels": {n: {"launches": e["launches"], "fetch_bytes": e["FETCH_SIZE"], "write_bytes": e["WRITE_SIZE"]}
                    for n, e in sorted(per_kernel.items(), key=lambda kv: -(kv[1]["FETCH_SIZE"] +
                                                                            kv[1]["WRITE_SIZE"]))},
    }


def marker_summary(csv_path: str, cmd: str, out_path: str) -> None:
    """Tally the roctx ranges of a ``rocprofv3 --marker-trace`` run by kind (the
    range name without its trailing number): count and host time."""
    import re
    kinds = {}
    order = []
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            kind = re.sub(r" \d+$", "", r["Function"])
            us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
            if kind not in kinds:
                kinds[kind] = [0, 0.0]
                order.append(kind)
            kinds[kind][0] += 1
            kinds[kind][1] += us
    lines = ["# roctx ranges (host enqueue time of each schedule step), by kind", f"# command: {cmd}", "#",
             f"# {'range':<40} {'count':>6} {'total_us':>12} {'avg_us':>10}"]
    for k in order:
        n, tot = kinds[k]
        lines.append(f"  {k[:40]:<40} {n:>6} {tot:>12.1f} {tot / n:>10.1f}")
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")


def main():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = p.add_subparsers(dest="what", required=True)
    t = sub.add_parser("trace")
    t.add_argument("--db")
    t.add_argument("--csv")
    t.add_argument("--cmd", required=True)
    t.add_argument("--out", required=True)
    t.add_argument("--dispatches", nargs=3, metavar=("TRACE_CSV", "NAME_SUBSTRING", "LAST"),
                   help="also list the last LAST dispatches of matching kernels")
    c = sub.add_parser("counters")
    c.add_argument("--run", nargs=5, action="append", required=True,
                   metavar=("LABEL", "FETCH_CSV", "WRITE_CSV", "FETCH_CMD", "WRITE_CMD"))
    c.add_argument("--T", type=int, default=262144)
    c.add_argument("--d", type=int, default=7168)
    c.add_argument("--S", type=int, default=9)
    c.add_argument("--out", required=True)
    q = sub.add_parser("pass")
    for flag in ("--fetch", "--write", "--fetch-cmd", "--write-cmd", "--label", "--out"):
        q.add_argument(flag, required=True)
    q.add_argument("--T", type=int, required=True)
    q.add_argument("--d", type=int, default=7168)
    q.add_argument("--algorithmic", type=int, required=True, help="algorithmic bytes of one pass")
    mk = sub.add_parser("markers")
    mk.add_argument("--csv", required=True)
    mk.add_argument("--cmd", required=True)
    mk.add_argument("--out", required=True)
    a = p.parse_args()
    if a.what == "markers":
        marker_summary(a.csv, a.cmd, a.out)
        return
    if a.what == "pass":
        s = pass_summary(a.fetch, a.write, a.fetch_cmd, a.write_cmd, a.T, a.d, a.algorithmic, a.label)
        with open(a.out, "w") as f:
            json.dump(s, f, indent=1)
            f.write("\n")
        return
    if a.what == "trace":
        stats = kernel_stats_from_db(a.db) if a.db else kernel_stats_from_csv(a.csv)
        disp = dispatch_durations(a.dispatches[0], a.dispatches[1], int(a.dispatches[2])) if a.dispatches else None
        write_trace_summary(stats, a.cmd, a.out, dispatches=disp)
    else:
        s = counters_summary(a.run, a.T, a.d, a.S)
        with open(a.out, "w") as f:
            json.dump(s, f, indent=1)
            f.write("\n")


if __name__ == "__main__":
    main()
