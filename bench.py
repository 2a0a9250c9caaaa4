#!/usr/bin/env python3
"""Throughput of the Block AttnRes hot path on one MI355X.

Default workload: the long-context prefill chunk, T = 262144 tokens, d = 7168,
S = 9 bf16 sources (~34 GB resident in HBM).  One step = one layer of the hot
path: the previous layer's output is added into the current block's partial
sum (read-modify-write) and the nine sources are aggregated into the residual
and the depth weights -- one ``attnres_accumulate_aggregate`` launch (or, with
``--unfused``, ``attnres_accumulate`` then ``attnres_aggregate``).

Prints one JSON line: tokens/s for the whole step, plus a ``roofline`` object
for the dominant kernel (algorithmic bytes per launch over its average launch
time, timed with HIP events on the stream it runs on) and a ``cpu_baseline``
object (the float64 CPU oracle on a bounded token sample of the same step).

Other workloads (``--workload``) are for measurement notes, not bench lines.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

REPO = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, REPO)

METRIC = "Block AttnRes tokens/s and achieved HBM GB/s (% peak), d=7168, S=9, bf16"
PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E, AMD's published peak
COUNTERS_FILE = os.path.join(REPO, "profiles", "aggregate_prefill_t262144_counters.json")


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="prefill_t262144",
                   choices=["prefill_t262144", "layer_t4096", "decode", "decode_93", "schedule_93", "full_s94",
                            "backward_t32768", "schedule_93_backward"])
    p.add_argument("--decode-T", type=int, default=64)
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--cpu-seconds", type=float, default=10.0, help="bounded oracle timing budget")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-pattern-probe", action="store_true",
                   help="skip the trivial-arithmetic probe of the same HBM access pattern")
    p.add_argument("--schedule-mode", default="two_phase", choices=["two_phase", "fused", "unfused"],
                   help="schedule_93 only: per-layer launches (unfused / fused) or the two-phase schedule")
    p.add_argument("--unfused", action="store_true",
                   help="time attnres_accumulate + attnres_aggregate as two launches instead of the fused one")
    p.add_argument("--rotate", type=int, default=0,
                   help="input sets to cycle through (default: 3 for layer_t4096 -- 1.76 GB, beyond the 256 MB "
                        "Infinity Cache -- else 1)")
    p.add_argument("--with-copy", action="store_true",
                   help="also run one plain copy of T*d bf16 before each step, outside the timed region "
                        "(reference kernel for the HBM byte counters)")
    return p.parse_args()


def counter_traffic(kernel: str, T: int):
    """HBM bytes per launch of ``kernel`` from the committed counter summary, if
    it was taken on the current kernel source at this T; else None."""
    try:
        with open(COUNTERS_FILE) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    from depth_wise_attention_block_amd.profiling import aggregate_source_digest
    if c.get("aggregate_source_sha256") != aggregate_source_digest() or c.get("workload", {}).get("T") != T:
        return None
    k = c.get("kernels", {}).get(kernel)
    return None if k is None else k.get("traffic_bytes_per_launch")


def pass_traffic(label: str, T: int):
    """HBM bytes of one whole pass from its committed counter summary
    (``profiles/<label>_counters.json``), if it was taken on the current
    sources at this T; else None."""
    from depth_wise_attention_block_amd.profiling import pass_source_digest
    try:
        with open(os.path.join(REPO, "profiles", f"{label}_counters.json")) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("source_sha256") is None or c.get("source_sha256") != pass_source_digest(label) or c.get("T") != T:
        return None
    return c.get("pass", {}).get("traffic_bytes")


# ---- the oracle's baseline on the host cores ---------------------------------
#
# The CPU oracle is plain float64 NumPy on one thread.  The baseline runs it in
# a pool of single-threaded worker processes, one per host core the process
# may use (at most MAX_ORACLE_WORKERS, the CPU share of one GPU on a shared
# host), over a token sample of the same step held in shared memory.  The pool
# is started before anything touches the GPU: the workers are started fresh
# (spawn), never forked from a process with GPU state.

MAX_ORACLE_WORKERS = 16
ORACLE_CHUNK = 128          # tokens per oracle call, as in the one-thread timing


def usable_cpus() -> int:
    """Host CPUs this process may run on (its affinity set, where the OS has one)."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def oracle_workers() -> int:
    return max(1, min(MAX_ORACLE_WORKERS, usable_cpus()))


def _single_thread_env():
    """Worker initializer: one BLAS/OpenMP thread, and the oracle imported up
    front so that the timed tasks start computing at once."""
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS", "BLIS_NUM_THREADS"):
        os.environ[var] = "1"
    import numpy  # noqa: F401
    import threadpoolctl  # noqa: F401

    from oracle import attnres_oracle  # noqa: F401


def _noop(_):
    return os.getpid()


def _oracle_worker(args):
    """One worker: the fused step's oracle (accumulate, then the 9-source
    aggregation) over its share of the shared token sample, repeated until
    ``budget_s`` of wall time has passed.  Returns (tokens, seconds)."""
    shm_name, n_tok, d, rank, nworkers, budget_s = args
    from multiprocessing import shared_memory

    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import attnres_oracle as orc

    shm = shared_memory.SharedMemory(name=shm_name)
    try:
        H_all = np.ndarray((10, n_tok, d), dtype=np.float32, buffer=shm.buf)   # 9 sources + layer output
        w = np.ndarray((d,), dtype=np.float32, buffer=shm.buf, offset=10 * n_tok * d * 4)
        starts = list(range(rank * ORACLE_CHUNK, n_tok, nworkers * ORACLE_CHUNK))
        done, t0 = 0, time.perf_counter()
        with threadpool_limits(limits=1):
            while time.perf_counter() - t0 < budget_s and starts:
                for a in starts:
                    H = np.array(H_all[:9, a:a + ORACLE_CHUNK])
                    F = np.array(H_all[9, a:a + ORACLE_CHUNK])
                    H[8] = orc.accumulate(H[8], F, "bf16")
                    orc.depth_attention(H, w)
                    done += H.shape[1]
                    if time.perf_counter() - t0 >= budget_s:
                        break
        return done, time.perf_counter() - t0
    finally:
        del H_all, w
        shm.close()


def start_oracle_pool():
    """The worker pool, started before the GPU is touched (and checked alive)."""
    import multiprocessing as mp

    n = oracle_workers()
    pool = mp.get_context("spawn").Pool(n, initializer=_single_thread_env)
    pool.map(_noop, range(n))
    return pool, n


def cpu_baseline(wl, budget_s: float, seed: int, pool=None, nworkers: int = 1):
    """The oracle, as it is, on a bounded token sample of the same step: one
    thread for ~budget_s/3 (the per-core figure), then the pool of single-
    threaded workers over a shared sample for ~budget_s."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits

    from depth_wise_attention_block_amd import synth
    from oracle import attnres_oracle as orc

    T, d = wl.T, wl.d
    rows = synth.token_sample(T, 65536, 0, seed=seed + 17)
    rows = rows[torch.randperm(rows.numel(), generator=torch.Generator().manual_seed(seed))]
    w = wl.w.float().cpu().numpy()
    # one thread
    done, elapsed, k = 0, 0.0, 0
    with threadpool_limits(limits=1):
        torch.set_num_threads(1)
        while elapsed < budget_s / 3 and k * ORACLE_CHUNK < rows.numel():
            idx = rows[k * ORACLE_CHUNK:(k + 1) * ORACLE_CHUNK].to(wl.out.device)
            k += 1
            H = wl.store.slots.index_select(1, idx).float().cpu().numpy()
            F = wl.F.index_select(0, idx).float().cpu().numpy()
            t0 = time.perf_counter()
            H[8] = orc.accumulate(H[8], F, "bf16")
            orc.depth_attention(H, w)
            elapsed += time.perf_counter() - t0
            done += idx.numel()
    one = done / elapsed
    result = {"value": one, "unit": "tokens/s", "cores": 1, "kind": "oracle",
              "sample": f"{done} tokens of the same step (accumulate + 9-source aggregate), float64 NumPy, "
                        f"one thread, {elapsed:.1f} s"}
    if pool is None:
        return result
    # the pool: a shared sample of n_tok tokens (same step's rows, float32 = the bf16 values exactly)
    from multiprocessing import shared_memory

    n_tok = min(rows.numel(), 32 * ORACLE_CHUNK)
    shm = shared_memory.SharedMemory(create=True, size=(10 * n_tok * d + d) * 4)
    try:
        H_all = np.ndarray((10, n_tok, d), dtype=np.float32, buffer=shm.buf)
        for a in range(0, n_tok, 1024):
            idx = rows[a:a + 1024][: n_tok - a].to(wl.out.device)
            H_all[:9, a:a + idx.numel()] = wl.store.slots.index_select(1, idx).float().cpu().numpy()
            H_all[9, a:a + idx.numel()] = wl.F.index_select(0, idx).float().cpu().numpy()
        np.ndarray((d,), dtype=np.float32, buffer=shm.buf, offset=10 * n_tok * d * 4)[:] = w
        t0 = time.perf_counter()
        parts = pool.map(_oracle_worker, [(shm.name, n_tok, d, r, nworkers, budget_s) for r in range(nworkers)])
        wall = time.perf_counter() - t0
        del H_all
    finally:
        shm.close()
        shm.unlink()
    total = sum(p[0] for p in parts)
    result.update({
        "value": total / wall, "cores": nworkers,
        "sample": f"{total} token-steps over a {n_tok}-token sample of the same step (accumulate + 9-source "
                  f"aggregate), float64 NumPy, {nworkers} single-threaded worker processes, {wall:.1f} s wall",
        "single_thread_tokens_per_s": round(one, 1),
        "host_cpus": os.cpu_count(), "usable_cpus": usable_cpus(),
    })
    return result


def pattern_ceiling(T: int, d: int):
    """Run the access-pattern probe (trivial arithmetic, same reads and writes)
    in a child process; None if it is not built or fails."""
    import subprocess

    exe = os.path.join(REPO, "depth_wise_attention_block_amd", "pattern_bench")
    if not os.path.exists(exe):
        return None
    try:
        proc = subprocess.run([exe, str(T), str(d), "5"], stdout=subprocess.PIPE, stderr=subprocess.PIPE,
                              text=True, timeout=120)
    except subprocess.TimeoutExpired:
        return None
    if proc.returncode != 0:
        print(f"# pattern probe failed: {proc.stderr.strip()}", file=sys.stderr)
        return None
    return json.loads(proc.stdout.strip().splitlines()[-1])


def cpu_baseline_backward(wl, budget_s: float, seed: int):
    """The oracle's backward, as it is, on a bounded token sample."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits

    from depth_wise_attention_block_amd import synth
    from oracle import attnres_oracle as orc

    rows = synth.token_sample(wl.T, 8192, 0, seed=seed + 19)
    chunk = 64
    w = wl.w.float().cpu().numpy()
    done, elapsed, k = 0, 0.0, 0
    with threadpool_limits(limits=1):
        torch.set_num_threads(1)
        while elapsed < budget_s and k * chunk < rows.numel():
            idx = rows[k * chunk:(k + 1) * chunk].to(wl.H.device)
            k += 1
            H = wl.H.index_select(1, idx).float().cpu().numpy()
            g = wl.g.index_select(0, idx).float().cpu().numpy()
            t0 = time.perf_counter()
            orc.depth_attention_backward(H, w, g)
            elapsed += time.perf_counter() - t0
            done += idx.numel()
    return {"value": done / elapsed, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} tokens of the same step (9-source aggregation backward), float64 NumPy, "
                      f"one thread, {elapsed:.1f} s"}


def bench_decode_93(args, dev):
    """The whole 93-layer depth path for a decode batch (T = --decode-T tokens):
    one pass = the 93 layers' aggregations and the output layer's, in the
    schedule mode --schedule-mode (two-phase by default: from block 3 one
    inter-block pass per block and one merge per later layer; fused: one update
    + aggregate launch per layer), launched eagerly from Python or replayed as
    one HIP graph."""
    import torch

    from depth_wise_attention_block_amd import workloads

    wl = workloads.Schedule(args.decode_T, seed=args.seed, device=dev)
    T = wl.T
    stream = torch.cuda.current_stream(dev)

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    mode = args.schedule_mode
    eager_ms = timed(lambda: wl.step(mode=mode))
    graph = wl.capture(mode)
    graph_ms = timed(graph.replay)
    step_bytes = wl.step_bytes(mode)
    achieved = step_bytes / (graph_ms * 1e-3) / 1e9
    return {
        "metric": METRIC, "value": round(T / (graph_ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(graph_ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "decode_93", "T": T, "d": wl.d, "layers": wl.layers, "block_size": wl.block_size,
                   "mode": mode,
                   "step": "one decode pass through the 93-layer depth path (94 aggregations), replayed as a "
                           "HIP graph"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": None,
                     "kernel": "whole pass (launch-bound at this size)", "bytes_per_launch": step_bytes},
        "cpu_baseline": None,
        "detail": {"eager_ms_per_pass": round(eager_ms, 4), "graph_ms_per_pass": round(graph_ms, 4),
                   "aggregations_per_pass": len(wl.source_counts()),
                   "graph_us_per_aggregation": round(graph_ms * 1e3 / len(wl.source_counts()), 2)},
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the hot path shards over "
              "tokens with no communication, so N GPUs would each run this same single-GPU step.",
              file=sys.stderr)
        sys.exit(2)

    pool = nworkers = None
    if not args.no_cpu_baseline and args.workload in ("prefill_t262144", "layer_t4096", "decode"):
        pool, nworkers = start_oracle_pool()   # before anything touches the GPU

    ceiling = None
    if args.workload in ("prefill_t262144", "layer_t4096", "decode") and not args.no_pattern_probe:
        T_probe = {"prefill_t262144": 262144, "layer_t4096": 4096, "decode": args.decode_T}[args.workload]
        ceiling = pattern_ceiling(T_probe, 7168)

    import torch

    from depth_wise_attention_block_amd import binding, workloads

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    binding.lib()
    if args.workload == "decode_93":
        print(json.dumps(bench_decode_93(args, dev)), flush=True)
        return

    fused = not args.unfused
    t_setup = time.perf_counter()
    if args.workload == "backward_t32768":
        wl = workloads.LayerBackward(32768, seed=args.seed, device=dev)
        T = wl.T
        step_bytes = wl.step_bytes()
        cfg = {"workload": "backward_t32768", "T": T, "d": wl.d, "S": wl.S,
               "step": "one aggregation backward: recompute, float32 source gradients accumulated, "
                       "last source's gradient handed out (bf16), dL/dw reduced over tokens"}
    elif args.workload == "schedule_93_backward":
        wl = workloads.ScheduleBackward(32768, seed=args.seed, device=dev)
        T = wl.T
        step_bytes = wl.step_bytes()
        cfg = {"workload": "schedule_93_backward", "T": T, "d": wl.d, "layers": wl.layers,
               "block_size": wl.block_size,
               "step": "output-layer + 93 aggregation backwards in reverse, partial sums recomputed per block, "
                       "float32 source gradients, each layer output's gradient handed out"}
    elif args.workload == "full_s94":
        wl = workloads.ManySources(32768, 94, seed=args.seed, device=dev)
        T = wl.T
        step_bytes = wl.step_bytes()
        cfg = {"workload": "full_s94", "T": T, "d": wl.d, "S": wl.S,
               "step": "one aggregation over 94 sources (batched online softmax)"}
    elif args.workload == "schedule_93":
        wl = workloads.Schedule(32768, seed=args.seed, device=dev)
        T = wl.T
        sched_mode = "unfused" if args.unfused else args.schedule_mode
        step_bytes = wl.step_bytes(sched_mode)
        cfg = {"workload": "schedule_93", "T": T, "d": wl.d, "layers": wl.layers, "block_size": wl.block_size,
               "mode": sched_mode,
               "step": {"two_phase": "blocks 1-2 one launch per layer; blocks 3-8 one inter-block pass per block "
                                     "+ one merge per later layer; output-layer aggregate",
                        "fused": "layer 1 aggregate + 93 fused (partial update + next aggregate) launches",
                        "unfused": "93 x (aggregate + partial update) + output-layer aggregate"}[sched_mode]}
    else:
        T = {"prefill_t262144": 262144, "layer_t4096": 4096, "decode": args.decode_T}[args.workload]
        rotate = args.rotate or (3 if args.workload == "layer_t4096" else 1)
        wls = [workloads.LayerStep(T, seed=args.seed + k, device=dev) for k in range(rotate)]
        wl = wls[0]
        step_bytes = wl.step_bytes(fused)
        cfg = {"workload": args.workload, "T": T, "d": wl.d, "S": 9, "input_sets": rotate,
               "step": ("one fused launch: partial += layer output, then aggregate over 9 sources" if fused else
                        "attnres_accumulate (partial += layer output), then attnres_aggregate over 9 sources")}
    copy_store = copy_src = None
    if args.with_copy:
        copy_store = binding.SourceStore(T, wl.d, s_max=2, dtype=torch.bfloat16, device=dev)
        copy_src = {"schedule_93": lambda: wl.F[0], "schedule_93_backward": lambda: wl.fwd.F[0],
                    "backward_t32768": lambda: wl.g, "full_s94": lambda: wl.H[0]}.get(args.workload, lambda: wl.F)()
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t_setup
    print(f"# setup {setup_s:.1f} s: workload {cfg['workload']} T={T} fused={fused}", file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream(dev)
    dom_events, acc_events = [], []   # dominant kernel; stand-alone update (unfused only)
    step_no = [0]

    def one_step(timed: bool):
        nonlocal wl
        if args.workload in ("prefill_t262144", "layer_t4096", "decode"):
            wl = wls[step_no[0] % len(wls)]
            step_no[0] += 1
        if copy_store is not None:
            copy_store.reset()
            copy_store.accumulate(copy_src)   # plain copy of T*d bf16 (first layer of a block)
        if args.workload in ("schedule_93", "schedule_93_backward"):
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)] if timed else None
            if ev:
                ev[0].record(stream)
            wl.step(mode=sched_mode) if args.workload == "schedule_93" else wl.step()
            if ev:
                ev[1].record(stream)
                dom_events.append((ev[0], ev[1]))
            return
        if args.workload in ("full_s94", "backward_t32768"):
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)] if timed else None
            if ev:
                ev[0].record(stream)
            wl.step()
            if ev:
                ev[1].record(stream)
                dom_events.append((ev[0], ev[1]))
            return
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)] if timed else None
        if ev:
            ev[0].record(stream)
        if fused:
            wl.fused()
            if ev:
                ev[1].record(stream)
                dom_events.append((ev[0], ev[1]))
            return
        wl.accumulate()
        if ev:
            ev[1].record(stream)
        wl.aggregate()
        if ev:
            ev[2].record(stream)
            acc_events.append((ev[0], ev[1]))
            dom_events.append((ev[1], ev[2]))

    for _ in range(args.warmup):
        one_step(False)
    torch.cuda.synchronize()

    t0 = time.perf_counter()
    for _ in range(args.steps):
        one_step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    detail = {"setup_s": round(setup_s, 1), "fused": fused}
    if args.workload in ("schedule_93", "schedule_93_backward"):
        # with the copy in the loop, the events around each pass time the pass alone
        ms_step = (sum(a.elapsed_time(b) for a, b in dom_events) / len(dom_events) if copy_store is not None
                   else wall * 1e3 / args.steps)
        achieved = step_bytes / (ms_step * 1e-3) / 1e9
        label = {"schedule_93": "schedule_93_t32768_two_phase",
                 "schedule_93_backward": "schedule_93_t32768_backward"}[args.workload]
        counted = args.workload == "schedule_93_backward" or sched_mode == "two_phase"
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": pass_traffic(label, T) if counted else None,
                "kernel": "whole schedule (all launches of one pass)", "bytes_per_launch": step_bytes}
        detail["step_gb"] = step_bytes / 1e9
    elif args.workload in ("full_s94", "backward_t32768"):
        dom_ms = sum(a.elapsed_time(b) for a, b in dom_events) / len(dom_events)
        ms_step = dom_ms if copy_store is not None else wall * 1e3 / args.steps
        achieved = step_bytes / (dom_ms * 1e-3) / 1e9
        kernel = {"full_s94": "aggregate_many_kernel<true, 2>",
                  "backward_t32768": "aggregate_backward_kernel<true, 2> + reduce_rows_kernel"}[args.workload]
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBPS, 4),
                "traffic": pass_traffic("many_sources_s94_t32768", T) if args.workload == "full_s94" else None,
                "kernel": kernel, "bytes_per_launch": step_bytes, "avg_launch_ms": round(dom_ms, 4)}
    else:
        dom_ms = sum(a.elapsed_time(b) for a, b in dom_events) / len(dom_events)
        if copy_store is not None:
            # the copy sits between the timed launches: count the step's kernels only
            ms_step = dom_ms + (sum(a.elapsed_time(b) for a, b in acc_events) / len(acc_events) if acc_events else 0)
        else:
            ms_step = wall * 1e3 / args.steps
        dom_bytes = wl.fused_bytes() if fused else wl.aggregate_bytes()
        kernel = "aggregate_kernel<true, 2, 2, 9>" if fused else "aggregate_kernel<true, 2, 0, 9>"
        achieved = dom_bytes / (dom_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": counter_traffic(kernel, T),
                "kernel": kernel, "bytes_per_launch": dom_bytes, "avg_launch_ms": round(dom_ms, 4)}
        if ceiling is not None:
            # the step's traffic in the kernel's own structure (token per workgroup, XCD runs) ...
            key = "fused_pattern_10r2w_gbps" if fused else "token_pattern_9r1w_gbps"
            roof["pattern_ceiling"] = ceiling[key]
            roof["frac_of_pattern_ceiling"] = round(achieved / ceiling[key], 4)
            # ... and the fastest structure probed for the same traffic
            mix = "10r2w" if fused else "9r1w"
            probes = {k: v for k, v in ceiling.items() if k.endswith(f"{mix}_gbps")}
            best = max(probes, key=probes.get)
            roof["best_probe"] = best[:-len("_gbps")]
            roof["best_probe_gbps"] = probes[best]
            roof["frac_of_best_probe"] = round(achieved / probes[best], 4)
            detail["pattern_probe"] = ceiling
        detail.update({"dominant_ms": round(dom_ms, 4), "dominant_tokens_per_s": round(T / (dom_ms * 1e-3)),
                       "step_gbps": round(step_bytes / (ms_step * 1e-3) / 1e9, 1)})
        if acc_events:
            acc_ms = sum(a.elapsed_time(b) for a, b in acc_events) / len(acc_events)
            detail.update({"accumulate_ms": round(acc_ms, 4),
                           "accumulate_gbps": round(wl.accumulate_bytes() / (acc_ms * 1e-3) / 1e9, 1)})

    if args.workload == "decode":
        # latency per fused call: hot (inputs still in the caches) and cold (a
        # 512 MB write between calls evicts the 256 MB Infinity Cache)
        flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        lat = {"hot": [], "cold": []}
        for mode in ("hot", "cold"):
            for _ in range(200):
                if mode == "cold":
                    flush.fill_(1)
                ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
                ev[0].record(stream)
                wl.fused()
                ev[1].record(stream)
                lat[mode].append(ev)
        torch.cuda.synchronize()
        for mode, evs in lat.items():
            us = sorted(a.elapsed_time(b) * 1e3 for a, b in evs)
            detail[f"latency_us_{mode}_median"] = round(us[len(us) // 2], 2)
            detail[f"latency_us_{mode}_min"] = round(us[0], 2)
        del flush

    cpu = None
    if not args.no_cpu_baseline and args.workload in ("prefill_t262144", "layer_t4096", "decode"):
        cpu = cpu_baseline(wl, args.cpu_seconds, args.seed, pool, nworkers)
    elif not args.no_cpu_baseline and args.workload == "backward_t32768":
        cpu = cpu_baseline_backward(wl, args.cpu_seconds, args.seed)

    line = {
        "metric": METRIC, "value": round(T / (ms_step * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic", "config": cfg, "roofline": roof, "cpu_baseline": cpu, "detail": detail,
    }
    print(json.dumps(line), flush=True)
    if pool is not None:
        pool.close()
        pool.join()


if __name__ == "__main__":
    main()
