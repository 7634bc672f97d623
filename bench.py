#!/usr/bin/env python3
"""Benchmark of the DSA lightning-indexer hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config decode|prefill|long|
                     tiny|index_cache] [--rotate R] [--no-cpu-baseline]
                     [--only]

One step = one pass of the whole hot path over one batch: IndexCache mask
(host), q quantisation, paged FP8 logits, per-row top-k into the shared index
buffer, each through the C ABI of libdsa_indexer.so.  The headline workload
(``value``) is the decode batch: 64 requests with contexts uniform in
[1024, 8192], one query each at the last position, 64 heads, head_dim 128,
index_topk 2048, FP8 e4m3 K with one fp32 scale per token, 64-token pages
drawn from a shuffled 16384-page pool (synthetic, seeded).  The default run
adds one record per other workload of the metric: ``prefill`` (8192 queries
against a 40960-token cache: the FP8-MFMA-bound chunk), ``long`` (16 rows
at the end of a 1M-token cache) and ``index_cache`` (61-layer stacks at
freq 4, a seeded pattern and freq 1); ``--only`` measures the chosen
``--config`` alone.  The tiled workloads (prefill, long) also time the fused
forward (dsa_indexer_forward_fused: no logits buffer), after checking that
its top-k equals the forward's bit for bit.

Timing: inputs are resident in HBM before the timed region.  R copies of the
K cache (and of q / weights) rotate across steps so that consecutive steps do
not hit the 256 MB Infinity Cache.  W eager warm-up steps, then one HIP graph
holding exactly K steps (step i uses copy i mod R) is captured, checked
bit-exactly against the eager result, and its replay is the timed region
(bracketed by device synchronisation).  Per-kernel durations come from HIP
events on the launch stream around 64 back-to-back launches of each kernel,
queued behind a GPU sleep so that no host gap falls inside a bracket.

Prints ONE JSON line.  ``roofline`` is for the dominant kernel (the logits
kernel): achieved = algorithmic bytes (or FLOPs) per launch / its average
duration, against the published peaks and against the rates this box
measures in the same run (a 1 GiB device copy; the library's pure FP8 MFMA
loop); ``ms_per_step_quantiles`` are over the timed replay and 16 more;
``cpu_baseline`` times the CPU oracle (numpy) on a bounded sample of the same
workload on this host (every workload's record has one).
"""

import argparse
import csv
import glob
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense FP8 MFMA, TFLOP/s

METRIC = ("indexer query-rows/sec (logits+top-k), HBM GB/s & FP8 MFMA util "
          "vs peak")

WORKLOADS = {
    "decode": "decode batch: 64 requests, context U[1024,8192] (seed 1), 1 "
              "query each at the last position, H=64, head_dim 128, "
              "index_topk 2048, FP8 e4m3 K + fp32 scale per token (132 B), "
              "64-token pages from a shuffled 16384-page pool",
    "prefill": "prefill chunk: 1 request, 32768-token cached prefix + 8192 "
               "new queries at positions 32768..40959, causal, H=64, "
               "head_dim 128, index_topk 2048, FP8 K, shuffled 64-token pages",
    "long": "long context: 1 request, 1048576-token FP8 K cache (16384 "
            "shuffled pages, 1% of tokens x4), 16 decode rows at the tail, "
            "H=64, head_dim 128, index_topk 2048",
    "tiny": "tiny: 1 request, 256 cached tokens, 8 queries at 248..255, H=4, "
            "index_topk 32",
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="decode",
                    choices=sorted(WORKLOADS) + ["index_cache"])
    ap.add_argument("--only", action="store_true",
                    help="measure --config alone (no other workload records)")
    ap.add_argument("--rotate", type=int, default=8,
                    help="K-cache copies rotated across steps (cold cache)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device copy (for scaling "
                         "hardware byte counters)")
    ap.add_argument("--opt", action="append", default=[],
                    help="library tuning knob key=value (dsa_set_option)")
    ap.add_argument("--trace-summary", metavar="DIR",
                    help="summarise a rocprofv3 --kernel-trace --stats CSV "
                         "directory as markdown (no GPU)")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="per-dispatch FETCH_SIZE / WRITE_SIZE of the logits "
                         "kernel from two rocprofv3 --pmc CSV directories, "
                         "scaled by the 256 MiB calibration copy (no GPU)")
    ap.add_argument("--mfma-summary", metavar="DIR",
                    help="per-dispatch MFMA counters (SQ_VALU_MFMA_BUSY_"
                         "CYCLES, SQ_INSTS_VALU_MFMA_MOPS_F8, ..., "
                         "GRBM_GUI_ACTIVE) of the logits kernel from one "
                         "rocprofv3 --pmc CSV directory (no GPU)")
    ap.add_argument("--bench-log", help="bench JSON line of the profiled run")
    ap.add_argument("--command", action="append", default=[],
                    help="command line(s) that produced the profile")
    return ap.parse_args()


def make_batch(name):
    from dsa_lightning_indexer_amd import synth
    return {"decode": synth.decode, "prefill": synth.prefill,
            "long": synth.long_context, "tiny": synth.tiny}[name]()


def logits_work(b):
    """Algorithmic bytes and FLOPs of one step, charged to its logits launch
    (the dominant kernel).

    Bytes: 132 B of K (128 FP8 key bytes + 4 B fp32 scale) per key read --
    every visible (row, key) pair for rows that are one per request (each
    key is used by one row), every cached key once for a request whose rows
    share the keys (prefill, long context: a tile reads a key once for all
    of its rows) -- plus H * (128 + 4 + 4) B of FP8 q, q scales and weights
    per row, plus the k int32 indices written per row.  The logits written
    by the logits kernel and read back by the top-k are a round trip inside
    the step, not counted.  FLOPs: 2 * H * 128 per visible (row, key) pair.
    """
    H = b.H
    pairs = b.visible_pairs
    flops = 2.0 * H * 128 * pairs
    per_row = b.T * H * (128 + 4 + 4) + 4 * b.k * b.T
    if b.T == b.R:                                 # one row per request
        kbytes = 132 * pairs
    else:                                          # keys shared by a request
        kbytes = 132 * sum(int(c) for c in b.contexts)
    return kbytes + per_row, flops


def dominant_kernel(b):
    """(Name prefix, name part) of the step's logits kernel as the profiler
    prints it: a decode batch's forward scores with its page schedule (the
    instance whose last template argument is true); a tiled batch's forward
    with the tile kernel that writes logits (last template argument false:
    true is the fused forward's candidate pass)."""
    if b.T <= 128 and b.T <= 2 * b.R:
        return "logits_balanced_kernel<", ", true>"
    if b.T <= 2 * b.R:
        return "logits_row_prefetch_kernel<", ""
    return "logits_tile16_kernel<", ", false>"


def host_cpu():
    """(CPU model name, usable cores) of this host."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model, len(os.sched_getaffinity(0))


# Rows of the oracle's CPU sample per workload (evenly spaced; the whole batch
# when absent): the prefill chunk's 8192 rows and the 1M-token tail's 16 rows
# of 1M columns would take minutes to hours in numpy.
CPU_SAMPLE_ROWS = {"prefill": 256, "long": 1}


def cpu_baseline(b, seconds, max_rows=None):
    """Time the CPU oracle on the same workload: quantise q, logits and the
    sort-based top-k of a declared sample of rows (the whole batch, or
    ``max_rows`` evenly spaced rows), passes repeated until ``seconds`` of
    work; BLAS threads = the usable cores."""
    from oracle import indexer as oi
    model, cores = host_cpu()
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=cores)
    except Exception:                                   # pragma: no cover
        limiter = None
    rows = np.arange(b.T)
    sample = "whole batch"
    if max_rows is not None and b.T > max_rows:
        rows = np.linspace(0, b.T - 1, max_rows).round().astype(np.int64)
        sample = f"{len(rows)} evenly spaced rows of {b.T}"
    try:
        t0 = time.perf_counter()
        done = 0
        reps = 0
        while True:
            q = b.q_bf16[rows].float().numpy()
            codes = np.zeros((b.T, b.H, 128), np.uint8)
            sc = np.ones((b.T, b.H), np.float32)
            codes[rows], sc[rows] = oi.quantize_q(q)
            lg = oi.indexer_logits(codes, sc, b.weights, b.k_cache,
                                   b.block_table, b.query_start_loc,
                                   b.positions, b.ld, rows=rows)
            oi.indexer_topk(lg, b.positions, b.k, rows=rows)
            done += len(rows)
            reps += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
    finally:
        if limiter is not None:
            limiter.unregister()
    return {"value": done / el, "unit": "query-rows/s", "cores": int(cores),
            "kind": "oracle", "cpu_model": model,
            "sample": f"{sample}, {reps} pass(es), {done} rows in {el:.1f} s "
                      "(numpy fp64 oracle: quantise q, logits, sort-based "
                      "top-k)"}



# ----------------------------------------------------------------------------
# Profile summaries (run on the host over rocprofv3 CSV output).
# ----------------------------------------------------------------------------
LOGITS_SOURCES = ("dsa_lightning_indexer_amd/csrc/kernels_logits.hip",
                  "dsa_lightning_indexer_amd/csrc/dsa_common.h",
                  "dsa_lightning_indexer_amd/csrc/dsa_launch.h",
                  "dsa_lightning_indexer_amd/csrc/dsa_score.h")
CALIBRATION_BYTES = 1 << 28


def logits_sources_digest():
    """Digest of the sources the logits kernels are built from: byte counters
    taken for another version of the kernel are not reported."""
    h = hashlib.sha256()
    for rel in LOGITS_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def counters_path(config):
    return os.path.join(ROOT, "profiles", f"{config}_dominant_kernel_counters.json")


def traffic_from_counters(config):
    """HBM bytes per logits launch from the committed counter summary of this
    workload, or None when there is none or the kernel has changed since."""
    try:
        with open(counters_path(config)) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("sources_digest") != logits_sources_digest():
        return None
    return int(d["traffic_bytes_per_launch"])


def _csv_rows(directory, suffix):
    rows = []
    for path in sorted(glob.glob(os.path.join(directory, f"*{suffix}"))):
        with open(path, newline="") as f:
            rows.extend(csv.DictReader(f))
    if not rows:
        raise SystemExit(f"no *{suffix} under {directory}")
    return rows


def _base_name(name):
    """Kernel name without its template arguments (the instances of one
    kernel chosen per launch shape count as one kernel)."""
    return name.split("<")[0]


def _per_dispatch(rows):
    """{dispatch id: (kernel name, summed counter value in KiB)}; only the
    dispatches at the largest grid of their kernel instance are kept (the
    workload's own launch: the chunked leg and the fused forward's sample
    pass launch the same instance on smaller grids)."""
    out, grid = {}, {}
    for r in rows:
        key = r["Dispatch_Id"]
        name, v, g = out.get(key, (r["Kernel_Name"], 0.0, int(r["Grid_Size"])))
        out[key] = (name, v + float(r["Counter_Value"]), g)
        grid[name] = max(grid.get(name, 0), g)
    return {k: (n, v, g) for k, (n, v, g) in out.items() if g == grid[n]}


def _matcher(config):
    head, tail = dominant_kernel(make_batch(config))
    return lambda name: f"dsa::{head}" in name and tail in name


def pmc_summary(args):
    fetch = _per_dispatch(_csv_rows(args.pmc_summary[0],
                                    "counter_collection.csv"))
    write = _per_dispatch(_csv_rows(args.pmc_summary[1],
                                    "counter_collection.csv"))

    def calib(d):
        # the calibration copies are the largest copy dispatches
        v = sorted((x for n, x, _ in d.values() if "copyBuffer" in n),
                   reverse=True)[:3]
        if not v:
            raise SystemExit("no calibration copy in the counter run")
        if max(v) > 1.05 * min(v):
            raise SystemExit("the largest copies of the counter run differ: "
                             "not the three calibration copies")
        return sum(v) / len(v)

    is_dom = _matcher(args.config)

    def logits(d):
        # the matching instance at the largest grid: the workload's own
        # logits launch (a fused sample pass is a smaller launch)
        top = max((g for n, _, g in d.values() if is_dom(n)), default=0)
        v = [x for n, x, g in d.values() if is_dom(n) and g == top]
        names = sorted({n for n, _, g in d.values() if is_dom(n) and g == top})
        if not v:
            raise SystemExit("no logits dispatch in the counter run")
        return sum(v) / len(v), len(v), names

    f_cal, w_cal = calib(fetch), calib(write)
    f_ff = CALIBRATION_BYTES / (f_cal * 1024.0)
    w_ff = CALIBRATION_BYTES / (w_cal * 1024.0)

    def every_kernel(directory):
        # per (kernel, grid): dispatches and average KiB per dispatch
        acc = {}
        per = {}
        for r in _csv_rows(directory, "counter_collection.csv"):
            k = (r["Dispatch_Id"], r["Kernel_Name"], int(r["Grid_Size"]))
            per[k] = per.get(k, 0.0) + float(r["Counter_Value"])
        for (_, name, g), v in per.items():
            if "dsa::" not in name:
                continue
            a = acc.setdefault((name, g), [0, 0.0])
            a[0] += 1
            a[1] += v
        return {k: (n, v / n) for k, (n, v) in acc.items()}

    ef, ew = every_kernel(args.pmc_summary[0]), every_kernel(args.pmc_summary[1])
    kernels_kib = []
    for (name, g) in sorted(ef, key=lambda x: -ef[x][1]):
        n, fk = ef[(name, g)]
        wk = ew.get((name, g), (0, 0.0))[1]
        kernels_kib.append({
            "kernel": name, "grid": g, "dispatches": n, "fetch_kib": round(fk, 1),
            "write_kib": round(wk, 1),
            "hbm_bytes": int(round(fk * 1024 * f_ff + wk * 1024 * w_ff))})
    f_kib, nf, names = logits(fetch)
    w_kib, nw, _ = logits(write)
    bench = None
    if args.bench_log:
        with open(args.bench_log) as f:
            for line in f:
                if line.startswith("{") and '"metric"' in line:
                    bench = json.loads(line)
    out = {
        "config": args.config,
        "kernel": names,
        "sources_digest": logits_sources_digest(),
        "fetch_kib_per_dispatch": round(f_kib, 1),
        "write_kib_per_dispatch": round(w_kib, 1),
        "dispatches": [nf, nw],
        "calibration_copy_bytes": CALIBRATION_BYTES,
        "calibration_fetch_kib": round(f_cal, 1),
        "calibration_write_kib": round(w_cal, 1),
        "fetch_scale": round(f_ff, 4),
        "write_scale": round(w_ff, 4),
        "traffic_bytes_per_launch": int(round(f_kib * 1024 * f_ff +
                                              w_kib * 1024 * w_ff)),
        "algorithmic_bytes_per_launch":
            bench["roofline"]["algorithmic_bytes"] if bench else None,
        "every_kernel_per_dispatch": kernels_kib,
        "commands": args.command,
    }
    print(json.dumps(out, indent=1))


SIMDS = 4 * 256               # MI355X: 256 compute units x 4 SIMDs


def mfma_summary(args):
    """Average per dispatch of each counter of a multi-counter --pmc run,
    for the workload's logits kernel at its largest grid (the workload's own
    launch), with the MFMA busy fraction SQ_VALU_MFMA_BUSY_CYCLES /
    (GRBM_GUI_ACTIVE x SIMDs) and the FP8 MFMA work the counters saw
    (SQ_INSTS_VALU_MFMA_MOPS_F8 x 512 FLOP) beside the algorithmic FLOPs."""
    rows = _csv_rows(args.mfma_summary, "counter_collection.csv")
    # GRBM_GUI_ACTIVE comes summed over the XCDs (each counts the cycles
    # the GPU is busy): per XCD it is the dispatch's active cycles
    xcc = 8
    for a in glob.glob(os.path.join(args.mfma_summary, "*agent_info.csv")):
        with open(a, newline="") as f:
            for r in csv.DictReader(f):
                if r.get("Agent_Type") == "GPU" and r.get("Num_Xcc"):
                    xcc = int(r["Num_Xcc"])
    per, grid = {}, {}
    for r in rows:
        key = r["Dispatch_Id"]
        d = per.setdefault(key, {"name": r["Kernel_Name"],
                                 "grid": int(r["Grid_Size"]), "c": {},
                                 "ns": None})
        c = r["Counter_Name"]
        d["c"][c] = d["c"].get(c, 0.0) + float(r["Counter_Value"])
        if r.get("End_Timestamp") and r.get("Start_Timestamp"):
            d["ns"] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        grid[d["name"]] = max(grid.get(d["name"], 0), d["grid"])
    is_dom = _matcher(args.config)
    top = max((d["grid"] for d in per.values() if is_dom(d["name"])),
              default=0)
    dom = [d for d in per.values() if is_dom(d["name"]) and d["grid"] == top]
    if not dom:
        raise SystemExit("no logits dispatch in the counter run")
    names = sorted({c for d in dom for c in d["c"]})
    avg = {c: sum(d["c"].get(c, 0.0) for d in dom) / len(dom) for c in names}
    b = make_batch(args.config)
    _, flops = logits_work(b)
    out = {"config": args.config,
           "kernel": sorted({d["name"] for d in dom}),
           "sources_digest": logits_sources_digest(),
           "dispatches": len(dom),
           "counters_per_dispatch": {c: round(v, 1) for c, v in avg.items()},
           "simds": SIMDS,
           "algorithmic_fp8_flops": flops,
           "commands": args.command}
    out["xcds"] = xcc
    if "SQ_VALU_MFMA_BUSY_CYCLES" in avg and avg.get("GRBM_GUI_ACTIVE"):
        active = avg["GRBM_GUI_ACTIVE"] / xcc
        out["active_cycles_per_dispatch"] = round(active, 1)
        out["mfma_busy_frac"] = round(avg["SQ_VALU_MFMA_BUSY_CYCLES"] /
                                      (active * SIMDS), 4)
        ns = [d["ns"] for d in dom if d["ns"]]
        if ns:
            dur = sorted(ns)[len(ns) // 2] * 1e-9
            out["median_dispatch_ms"] = round(dur * 1e3, 4)
            out["clock_ghz"] = round(active / dur / 1e9, 3)
    if "SQ_INSTS_VALU_MFMA_MOPS_F8" in avg:
        out["counted_fp8_flops"] = avg["SQ_INSTS_VALU_MFMA_MOPS_F8"] * 512
        out["counted_over_algorithmic"] = round(
            out["counted_fp8_flops"] / flops, 4)
    if args.bench_log:
        with open(args.bench_log) as f:
            for line in f:
                if line.startswith("{") and '"metric"' in line:
                    bl = json.loads(line)
                    out["bench_logits_ms"] = bl["kernels_ms"]["logits"]
                    out["bench_roofline_frac"] = bl["roofline"]["frac"]
    print(json.dumps(out, indent=1))


def trace_summary(args):
    stats = _csv_rows(args.trace_summary, "kernel_stats.csv")
    trace = _csv_rows(args.trace_summary, "kernel_trace.csv")
    durs, by_grid = {}, {}
    for r in trace:
        d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        g = (int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) *
             int(r["Grid_Size_Z"]))
        durs.setdefault(r["Kernel_Name"], []).append(d)
        by_grid.setdefault(r["Kernel_Name"], {}).setdefault(g, []).append(d)
    is_dom = _matcher(args.config)
    dom = [n for n in by_grid if is_dom(n)]
    lines = [f"# Kernel trace: {WORKLOADS.get(args.config, args.config)}", "",
             "Commands (from the repository root):", "", "```"]
    lines += args.command + ["```", "",
                             "Durations are per dispatch over every dispatch "
                             "of the run (warm-up, graph replays and the "
                             "per-kernel event loops).", "",
                             "| kernel | calls | average (us) | median (us) "
                             "| min (us) | max (us) | % |",
                             "|---|---|---|---|---|---|---|"]
    for r in stats:
        name = r["Name"]
        d = sorted(durs.get(name, [0.0]))
        nm = name if len(name) <= 90 else name[:87] + "..."
        lines.append(f"| `{nm}` | {r['Calls']} | "
                     f"{float(r['AverageNs']) / 1e3:.3f} | "
                     f"{d[len(d) // 2]:.3f} | {d[0]:.3f} | {d[-1]:.3f} | "
                     f"{float(r['Percentage']):.2f} |")
    top = {}
    for n in dom:
        b = _base_name(n)
        top[b] = max(top.get(b, 0), max(by_grid[n]))
    for n in dom:
        g = max(by_grid[n])
        if g != top[_base_name(n)]:
            continue                  # a smaller instance: the chunked leg
        d = sorted(by_grid[n][g])
        lines += ["", f"Dominant kernel at the workload's own launch (its "
                  f"largest grid, {g} threads; dispatches of the same "
                  f"kernel on smaller grids, if any, are the chunked-forward "
                  f"leg): `{n}`, "
                  f"{len(d)} dispatches, average {sum(d) / len(d):.3f} us, "
                  f"median {d[len(d) // 2]:.3f} us."]
    # back-to-back dispatches of the dominant kernel (the per-kernel event
    # loop): the idle time from one's end to the next one's start, which a
    # HIP-event average over the loop includes and a dispatch duration not
    seq = sorted(trace, key=lambda r: int(r["Start_Timestamp"]))

    def grid_of(r):
        return (int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) *
                int(r["Grid_Size_Z"]))

    pairs = []
    for a_, b_ in zip(seq, seq[1:]):
        if (is_dom(a_["Kernel_Name"]) and a_["Kernel_Name"] == b_["Kernel_Name"]
                and grid_of(a_) == grid_of(b_) ==
                top.get(_base_name(a_["Kernel_Name"]), -1)):
            dur = (int(a_["End_Timestamp"]) - int(a_["Start_Timestamp"])) / 1e3
            gap = (int(b_["Start_Timestamp"]) - int(a_["End_Timestamp"])) / 1e3
            pairs.append((dur, gap))
    if pairs:
        gaps = sorted(g for _, g in pairs)
        per = sorted(d + g for d, g in pairs)
        lines += ["", f"Back-to-back dispatches of the dominant kernel at its "
                  f"largest grid: {len(pairs)} pairs; gap from one dispatch's "
                  f"end to the next one's start: median "
                  f"{gaps[len(gaps) // 2]:.3f} us (min {gaps[0]:.3f}, max "
                  f"{gaps[-1]:.3f}); duration + gap: median "
                  f"{per[len(per) // 2]:.3f} us (what a HIP-event average "
                  f"over back-to-back launches measures)."]
    if args.bench_log:
        with open(args.bench_log) as f:
            for line in f:
                if line.startswith("{") and '"metric"' in line:
                    b = json.loads(line)
                    lines += ["", "Bench line of the same (profiled) run: "
                              f"ms/step {b['ms_per_step']}, per-kernel HIP-"
                              f"event averages (ms) {b['kernels_ms']}, "
                              f"roofline {b['roofline']['achieved']} "
                              f"{b['roofline']['unit']} (frac "
                              f"{b['roofline']['frac']})."]
    print("\n".join(lines))


def _events(torch):
    return (torch.cuda.Event(enable_timing=True),
            torch.cuda.Event(enable_timing=True))


def _timed(torch, fn, launches, rotate):
    """Average duration (ms) of ``launches`` back-to-back calls fn(i %
    rotate) between two HIP events on the launch stream, queued behind a
    GPU sleep so that the host has enqueued them all first."""
    a, z = _events(torch)
    torch.cuda.synchronize()
    torch.cuda._sleep(int(20e6))
    a.record()
    for i in range(launches):
        fn(i % rotate)
    z.record()
    torch.cuda.synchronize()
    return a.elapsed_time(z) / launches


def _in_step(torch, before, kernel, after, K, R, warmup):
    """Average duration (ms) of ``kernel`` inside eager steps: before(r),
    event, kernel(r), event, after(r) for K steps (after ``warmup`` steps),
    so that the kernel runs between the step's other kernels as it does in
    the timed graph rather than back to back with itself."""
    for i in range(warmup):
        before(i % R); kernel(i % R); after(i % R)
    torch.cuda.synchronize()
    ev = [_events(torch) for _ in range(K)]
    for i in range(K):
        before(i % R)
        ev[i][0].record()
        kernel(i % R)
        ev[i][1].record()
        after(i % R)
    torch.cuda.synchronize()
    return sum(a.elapsed_time(z) for a, z in ev) / K


def _graph_steps(torch, step, K, R, warmup, check_buf, ref_step):
    """W eager warm-up steps, then a HIP graph of exactly K steps (step i on
    copy i mod R), checked bit-exactly against the eager result of its last
    step, replayed once for the timed region.  Returns (ms per step, [ms per
    step of 16 more replays])."""
    for i in range(warmup):
        step(i % R)
    last = (K - 1) % R
    step(last)
    torch.cuda.synchronize()
    ref = check_buf.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(K):
            step(i % R)
    torch.cuda.synchronize()
    check_buf.fill_(-7)
    graph.replay()
    torch.cuda.synchronize()
    if not torch.equal(check_buf, ref):
        raise SystemExit("graph replay differs from the eager result")
    ref_step(last)                              # eager work between replays
    torch.cuda.synchronize()
    a, z = _events(torch)
    torch.cuda.synchronize()
    a.record()
    graph.replay()
    z.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(z) / K
    again = []
    for _ in range(16):
        a, z = _events(torch)
        a.record()
        graph.replay()
        z.record()
        torch.cuda.synchronize()
        again.append(round(a.elapsed_time(z) / K, 5))
    if not torch.equal(check_buf, ref):
        raise SystemExit("graph replay differs from the eager result")
    del graph
    return ms, again


def _quantiles(vals):
    """p10 / p50 / p90 (nearest rank) of per-replay step times."""
    v = sorted(vals)
    pick = lambda q: v[min(len(v) - 1, int(round(q * (len(v) - 1))))]
    return {"p10": pick(0.1), "p50": pick(0.5), "p90": pick(0.9),
            "replays": len(v)}


def measure_workload(args, name, K, W, extras=False, cpu=True,
                     cpu_rows=None):
    """One workload: step time over a graph of K steps, per-kernel times and
    the logits kernel's roofline (and, with ``extras``, the kernels around
    the hot path).  Returns the record (a dict)."""
    import torch
    from dsa_lightning_indexer_amd import binding

    dev = torch.device("cuda", 0)
    b = make_batch(name)
    R = max(1, args.rotate if name in ("decode", "long") else 1)
    bt = torch.from_numpy(b.block_table).to(dev)
    qsl = torch.from_numpy(b.query_start_loc).to(dev)
    pos = torch.from_numpy(b.positions).to(dev)
    kcs = [torch.from_numpy(b.k_cache).to(dev) for _ in range(R)]
    qs_in = [b.q_bf16.to(dev) for _ in range(R)]
    ws_in = [torch.from_numpy(b.weights).to(dev) for _ in range(R)]
    T, H, ld, k = b.T, b.H, b.ld, b.k
    q8 = torch.empty((T, H, 128), dtype=torch.uint8, device=dev)
    qsc = torch.empty((T, H), dtype=torch.float32, device=dev)
    logits = torch.empty((T, ld), dtype=torch.float32, device=dev)
    buf = torch.empty((T, k), dtype=torch.int32, device=dev)
    tws_n = binding.dsa_topk_workspace_size(T, ld, k)
    tws = torch.empty(max(tws_n, 1), dtype=torch.uint8, device=dev)
    fws = torch.empty(binding.dsa_forward_workspace_size(T, H, ld, k),
                      dtype=torch.uint8, device=dev)

    def forward(r):
        binding.dsa_indexer_forward(qs_in[r], ws_in[r], kcs[r], bt, qsl, pos,
                                    ld, k, logits=logits, out=buf,
                                    workspace=fws)

    def step(r):
        binding.dsa_index_cache_mask(1)                       # one F layer
        forward(r)

    torch.cuda.synchronize()
    binding.dsa_device_error_flags(reset=True)
    ms_step, again = _graph_steps(torch, step, K, R, W, buf, step)
    NK = 64
    kq = _timed(torch, lambda r: binding.dsa_quantize_q(qs_in[r], q8, qsc),
                NK, R)
    kl = _timed(torch, lambda r: binding.dsa_indexer_logits(
        q8, qsc, ws_in[r], kcs[r], bt, qsl, pos, ld, logits), NK, R)
    # decode batches: the step scores with the page schedule its
    # quantisation launch builds; time that kernel (one schedule, built
    # once: it depends only on the batch's metadata)
    sched = binding.dsa_logits_schedule(bt, qsl, pos, ld) \
        if b.T <= 128 and b.T <= 2 * b.R else None
    kl_plain = kl
    if sched is not None:
        kl = _timed(torch, lambda r: binding.dsa_indexer_logits_scheduled(
            q8, qsc, ws_in[r], kcs[r], bt, qsl, pos, ld, sched, logits),
            NK, R)
    kt = _timed(torch, lambda r: binding.dsa_indexer_topk(
        logits, pos, k, buf, tws), NK, R)
    # the logits kernel between the step's quantisation and top-k (as in the
    # timed graph; back to back with itself the chip runs it at a lower
    # clock: see the kernel traces).  Tiled batches only: a decode kernel
    # is about as short as the launch latency the event pair then includes.
    kl_step = None if T <= 2 * b.R else _in_step(
        torch, lambda r: binding.dsa_quantize_q(qs_in[r], q8, qsc),
        (lambda r: binding.dsa_indexer_logits_scheduled(
            q8, qsc, ws_in[r], kcs[r], bt, qsl, pos, ld, sched, logits))
        if sched is not None else
        (lambda r: binding.dsa_indexer_logits(
            q8, qsc, ws_in[r], kcs[r], bt, qsl, pos, ld, logits)),
        lambda r: binding.dsa_indexer_topk(logits, pos, k, buf, tws),
        NK, R, 4)
    kf = _timed(torch, forward, NK, R)
    kernels = {"quantize_q": round(kq, 5), "logits": round(kl, 5),
               "topk": round(kt, 5), "forward": round(kf, 5)}
    if kl_step is not None:
        kernels["logits_in_step"] = round(kl_step, 5)
    if sched is not None:
        kernels["logits_without_schedule"] = round(kl_plain, 5)
    rec = {}
    if extras:
        # Row-chunked forward under a 256 MiB logits budget.
        ch_rows = binding.dsa_logits_chunk_rows(T, ld, 256 << 20)
        ch_ws = torch.empty(max(1, binding.dsa_forward_chunked_workspace_size(
            T, b.R, H, ld, k, ch_rows)), dtype=torch.uint8, device=dev)
        ch_out = torch.empty((T, k), dtype=torch.int32, device=dev)
        kernels["forward_chunked_256MiB"] = round(_timed(
            torch, lambda r: binding.dsa_indexer_forward_chunked(
                qs_in[r], ws_in[r], kcs[r], bt, qsl, pos, ld, k,
                rows_per_chunk=ch_rows, out=ch_out, workspace=ch_ws),
            NK, R), 5)
        del ch_ws
        rec["chunked_rows_per_chunk"] = int(ch_rows)
        # The indexer-K write path (the rows' own tokens as new keys, into
        # a copy of the cache), the compressed slots, the hand-off.
        new_k = torch.randn((T, 128), dtype=torch.bfloat16, device=dev)
        slots = binding.dsa_slot_mapping(bt, qsl, pos)
        c_slots = torch.empty((T,), dtype=torch.int64, device=dev)
        c_pos = torch.empty((T,), dtype=torch.int32, device=dev)
        kernels["compressed_slot_mapping"] = round(_timed(
            torch, lambda r: binding.dsa_compressed_slot_mapping(
                bt, qsl, pos, 4, 64, slots=c_slots, positions_c=c_pos),
            NK, R), 5)
        kw_cache = kcs[0].clone()
        kkw = _timed(torch, lambda r: binding.dsa_indexer_k_write(
            new_k, slots, kw_cache), NK, R)
        kernels["k_write"] = round(kkw, 5)
        del kw_cache
        ho_slots = torch.empty((T, k), dtype=torch.int64, device=dev)
        kernels["topk_to_slots"] = round(_timed(
            torch, lambda r: binding.dsa_topk_to_slots(buf, bt, qsl,
                                                       slots=ho_slots),
            NK, R), 5)
        ho_mask = torch.empty((T, ld), dtype=torch.float32, device=dev)
        kmask = _timed(torch, lambda r: binding.dsa_topk_mask(
            buf, ld, mask=ho_mask), NK, R)
        kernels["topk_mask"] = round(kmask, 5)
        del ho_mask
        rec["topk_mask_gbs"] = round(T * ld * 4 / (kmask * 1e-3) / 1e9, 1)
        rec["k_write_gbs"] = round(T * (2 * 128 + 8 + 132) /
                                   (kkw * 1e-3) / 1e9, 1)
    if T > 2 * b.R:
        # The fused forward (no logits buffer) on the same batch: its top-k
        # must equal the forward's bit for bit; then a graph of K fused
        # steps, timed like the forward's.
        fu_ws = torch.empty(binding.dsa_forward_fused_workspace_size(
            T, b.R, H, ld, k), dtype=torch.uint8, device=dev)
        fu_out = torch.empty((T, k), dtype=torch.int32, device=dev)

        def fused(r):
            binding.dsa_indexer_forward_fused(
                qs_in[r], ws_in[r], kcs[r], bt, qsl, pos, ld, k, out=fu_out,
                workspace=fu_ws)

        def fused_step(r):
            binding.dsa_index_cache_mask(1)
            fused(r)

        forward(0)
        fused(0)
        torch.cuda.synchronize()
        if not torch.equal(fu_out, buf):
            raise SystemExit("fused forward differs from the forward")
        ms_fused, again_fused = _graph_steps(torch, fused_step, K, R, W,
                                             fu_out, fused_step)
        kernels["forward_fused"] = round(_timed(torch, fused, NK, R), 5)
        rec["fused"] = {
            "ms_per_step": round(ms_fused, 5),
            "ms_per_step_more_replays": again_fused,
            "ms_per_step_quantiles": _quantiles([round(ms_fused, 5)] +
                                                again_fused),
            "value": round(T / (ms_fused * 1e-3), 1),
            "unit": "query-rows/s",
            "speedup_vs_forward": round(ms_step / ms_fused, 4),
            "topk_equal_to_forward": True,
            "workspace_bytes": int(fu_ws.numel()),
            "logits_bytes_not_written": int(T * ld * 4)}
        del fu_ws
    assert binding.dsa_device_error_flags(reset=True) == 0

    alg_bytes, flops = logits_work(b)
    gbs = alg_bytes / (kl * 1e-3) / 1e9
    tfl = flops / (kl * 1e-3) / 1e12
    if T > 2 * b.R:                       # rows share the keys: MFMA-bound
        roof = {"bound": "mfma", "achieved": round(tfl, 2),
                "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(tfl / FP8_PEAK_TFLOPS, 4)}
    else:
        roof = {"bound": "hbm", "achieved": round(gbs, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4)}
    roof["traffic"] = traffic_from_counters(name)
    roof["kernel"] = dominant_kernel(b)[0].rstrip("<")
    roof["algorithmic_bytes"] = int(alg_bytes)
    roof["algorithmic_flops"] = flops
    roof["kernel_ms"] = round(kl, 5)
    if kl_step is not None:
        # the same kernel timed between the step's other kernels
        roof["kernel_ms_in_step"] = round(kl_step, 5)
        roof["frac_in_step"] = round(
            flops / (kl_step * 1e-3) / 1e12 / FP8_PEAK_TFLOPS, 4)
    roof["hbm_gbs"] = round(gbs, 1)
    roof["fp8_tflops"] = round(tfl, 2)
    if roof["bound"] == "hbm":
        # the attainable floor on this machine: a bare read of exactly the K
        # pages the batch's rows reach (the library's page-read helper: no
        # metadata lookups, no compute), timed like the logits kernel
        ids = torch.from_numpy(visible_page_ids(b)).to(dev)
        kr = _timed(torch, lambda r: binding.dsa_page_read_probe(kcs[r], ids),
                    NK, R)
        rb = int(ids.numel()) * 8448
        roof["bare_read_ms"] = round(kr, 5)
        roof["bare_read_bytes"] = rb
        roof["bare_read_gbs"] = round(rb / (kr * 1e-3) / 1e9, 1)
        roof["frac_of_bare_read"] = round(kr / kl, 4)
    rec.update({
        "workload": WORKLOADS[name],
        "value": round(T / (ms_step * 1e-3), 1), "unit": "query-rows/s",
        "ms_per_step": round(ms_step, 5), "ms_per_step_more_replays": again,
        "ms_per_step_quantiles": _quantiles([round(ms_step, 5)] + again),
        "rows": T, "heads": H, "index_topk": k,
        "visible_pairs": b.visible_pairs, "kcache_copies_rotated": R,
        "kernels_ms": kernels, "roofline": roof})
    del kcs, qs_in, ws_in, logits, fws, tws
    if cpu and not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(b, args.cpu_seconds, cpu_rows)
    torch.cuda.empty_cache()
    return rec


def visible_page_ids(b):
    """Physical ids of the K pages the batch's rows reach (page j of row t's
    request for j <= p_t / 64), row by row."""
    req = np.searchsorted(b.query_start_loc, np.arange(b.T), side="right") - 1
    ids = [b.block_table[int(req[t]), : int(b.positions[t]) // 64 + 1]
           for t in range(b.T)]
    return np.concatenate(ids).astype(np.int32)


def copy_rate(torch):
    """Attainable HBM rate on this machine: a 1 GiB device-to-device copy (read
    and write counted), GB/s."""
    dev = torch.device("cuda", 0)
    c_src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
    c_dst = torch.empty_like(c_src)
    c_dst.copy_(c_src)
    a, z = _events(torch)
    torch.cuda.synchronize()
    a.record()
    for _ in range(5):
        c_dst.copy_(c_src)
    z.record()
    torch.cuda.synchronize()
    del c_src, c_dst
    torch.cuda.empty_cache()
    return 2 * (1 << 30) * 5 / (a.elapsed_time(z) * 1e-3) / 1e9


def mfma_rate(torch):
    """Attainable FP8 MFMA rate on this machine: the library's pure MFMA loop
    (no memory traffic) at the clock the chip holds under it, TFLOP/s."""
    from dsa_lightning_indexer_amd import binding
    iters = 4000
    binding.dsa_fp8_mfma_rate_probe(iters)
    a, z = _events(torch)
    torch.cuda.synchronize()
    a.record()
    flops = sum(binding.dsa_fp8_mfma_rate_probe(iters) for _ in range(5))
    z.record()
    torch.cuda.synchronize()
    return flops / (a.elapsed_time(z) * 1e-3) / 1e12


def add_measured_peaks(roof, copy_gbs, mfma_tflops):
    """The roofline against the box's measured rates as well as the
    published peaks."""
    if copy_gbs is not None:
        roof["copy_gbs_measured"] = round(copy_gbs, 1)
        if roof["bound"] == "hbm":
            roof["frac_of_measured_copy"] = round(roof["achieved"] / copy_gbs,
                                                  4)
    if mfma_tflops is not None:
        roof["fp8_mfma_measured_tflops"] = round(mfma_tflops, 1)
        if roof["bound"] == "mfma":
            roof["frac_of_measured_mfma"] = round(
                roof["achieved"] / mfma_tflops, 4)
            if "kernel_ms_in_step" in roof:
                roof["frac_of_measured_mfma_in_step"] = round(
                    roof["algorithmic_flops"] / (roof["kernel_ms_in_step"] *
                                                 1e-3) / 1e12 / mfma_tflops, 4)


def main():
    args = parse()
    if args.trace_summary:
        return trace_summary(args)
    if args.pmc_summary:
        return pmc_summary(args)
    if args.mfma_summary:
        return mfma_summary(args)
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; "
                                   "--gpus N > 1 is not supported"}))
        sys.exit(2)
    K, W = max(1, args.steps), max(0, args.warmup)

    import torch
    from dsa_lightning_indexer_amd import binding

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    for kv in args.opt:
        key, val = kv.split("=")
        binding.dsa_set_option(key, int(val))

    if args.copy_calibration:
        src = torch.empty(1 << 28, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if args.config == "index_cache":
        out = bench_index_cache(args, K, W)
        print(json.dumps(out), flush=True)
        return

    head = args.config
    main_rec = measure_workload(args, head, K, W, extras=True, cpu=True,
                                cpu_rows=CPU_SAMPLE_ROWS.get(head))
    roof = main_rec.pop("roofline")
    # Not in counter runs: their scale comes from the largest copies, which
    # must be the 256 MiB calibration copies.
    cg = None if args.copy_calibration else copy_rate(torch)
    mt = mfma_rate(torch)
    add_measured_peaks(roof, cg, mt)
    out = {
        "metric": METRIC, "value": main_rec.pop("value"),
        "unit": main_rec.pop("unit"), "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": main_rec.pop("ms_per_step"),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8_e4m3 (fp32 accumulate)", "data": "synthetic",
        "config": {"workload": main_rec.pop("workload"),
                   "rows": main_rec.pop("rows"),
                   "heads": main_rec.pop("heads"),
                   "index_topk": main_rec.pop("index_topk"),
                   "visible_pairs": main_rec.pop("visible_pairs"),
                   "kcache_copies_rotated":
                       main_rec.pop("kcache_copies_rotated")},
        "roofline": roof,
    }
    cpu_rec = main_rec.pop("cpu_baseline", None)
    out.update(main_rec)
    if cpu_rec is not None:
        out["cpu_baseline"] = cpu_rec
    if not args.only:
        # the metric's other workloads: the FP8-MFMA-bound prefill chunk,
        # the 1M-token tail and the IndexCache stacks
        for name in ("prefill", "long"):
            if name == head:
                continue
            try:
                out[name] = measure_workload(
                    args, name, K, W, cpu=True,
                    cpu_rows=CPU_SAMPLE_ROWS.get(name))
                add_measured_peaks(out[name]["roofline"], cg, mt)
            except Exception as e:                    # pragma: no cover
                out[name] = {"error": repr(e)}
        try:
            out["index_cache"] = bench_index_cache(args, K, W)
        except Exception as e:                        # pragma: no cover
            out["index_cache"] = {"error": repr(e)}
    if args.opt:
        out["options"] = args.opt
    print(json.dumps(out), flush=True)


def bench_index_cache(args, K, W):
    """IndexCache stack: 61 layers, 32 decode requests x 16384 context,
    freq 4 / offset 2 (16 F layers), the seeded 61-character pattern and
    freq 1 (61 F layers), every layer with its own K cache, q and weights.
    Each run is captured once as a HIP graph (one dsa_index_cache_run over
    the whole stack), checked against the eager run, and replayed K times
    back to back for the timed region."""
    import torch
    from dsa_lightning_indexer_amd import binding, synth

    dev = torch.device("cuda", 0)
    L = 61
    layers_np = synth.index_cache_layers(list(range(L)))
    ref = layers_np[0]
    layers = []
    for l in range(L):
        b = layers_np[l]
        layers.append({"q_bf16": b.q_bf16.to(dev),
                       "weights": torch.from_numpy(b.weights).to(dev),
                       "k_cache": torch.from_numpy(b.k_cache).to(dev)})
    # host inputs of the freq-4 stack's F layers, for the CPU oracle's pass
    host_f4 = {l: layers_np[l] for l, sk in enumerate(
        binding.dsa_index_cache_mask(L, freq=4, offset=2)) if not sk}
    del layers_np
    bt = torch.from_numpy(ref.block_table).to(dev)
    qsl = torch.from_numpy(ref.query_start_loc).to(dev)
    pos = torch.from_numpy(ref.positions).to(dev)
    T, k, ld, H = ref.T, ref.k, ref.ld, ref.H
    buf = torch.empty((T, k), dtype=torch.int32, device=dev)
    ws = torch.empty(binding.dsa_run_workspace_size(T, ref.R, H, ld, k),
                     dtype=torch.uint8, device=dev)
    pattern = synth.index_cache_pattern(L)
    runs = {"freq4": dict(freq=4, offset=2), "pattern": dict(pattern=pattern),
            "freq1": dict(freq=1, offset=2)}
    n_full = {name: sum(1 for sk in binding.dsa_index_cache_mask(L, **kw)
                        if not sk) for name, kw in runs.items()}
    res = {}
    for name, kw in runs.items():
        def run():
            binding.dsa_index_cache_run(layers, bt, qsl, pos, ld, k, buf,
                                        workspace=ws, **kw)
        for _ in range(max(1, W)):
            run()
        torch.cuda.synchronize()
        ref_buf = buf.clone()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            run()
        torch.cuda.synchronize()
        buf.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        if not torch.equal(buf, ref_buf):
            raise SystemExit(f"IndexCache {name}: graph replay differs")
        a, z = _events(torch)
        torch.cuda._sleep(int(20e6))
        a.record()
        for _ in range(K):
            g.replay()
        z.record()
        torch.cuda.synchronize()
        res[name] = a.elapsed_time(z) / K
        del g
    # one F layer's logits kernel alone, rotating over the 16 freq-4 F
    # layers' inputs (each launch reads a cache the previous ones did not),
    # with the page schedule built once for all of them, as
    # dsa_index_cache_run builds it once per pass
    full4 = [l for l, sk in enumerate(binding.dsa_index_cache_mask(
        L, freq=4, offset=2)) if not sk]
    q8s = [binding.dsa_quantize_q(layers[l]["q_bf16"]) for l in full4]
    lg = torch.empty((T, ld), dtype=torch.float32, device=dev)
    sch = binding.dsa_logits_schedule(bt, qsl, pos, ld)
    kl = _timed(torch, lambda i: binding.dsa_indexer_logits_scheduled(
        q8s[i][0], q8s[i][1], layers[full4[i]]["weights"],
        layers[full4[i]]["k_cache"], bt, qsl, pos, ld, sch, lg), 64,
        len(full4))
    assert binding.dsa_device_error_flags(reset=True) == 0
    # algorithmic bytes of one F layer (as for decode): K pages, q fp8 +
    # scales + weights, top-k indices written; no logits round trip
    per_layer_bytes = 132 * T * 16384 + T * H * 136 + 4 * T * k
    del layers, ws, q8s, sch
    torch.cuda.empty_cache()
    cpu_rec = None
    if not args.no_cpu_baseline:
        cpu_rec = cpu_baseline_index_cache(host_f4, ref, L, args.cpu_seconds)
    del host_f4
    rec = {
        "metric": "IndexCache stack forward (61 DSA layers)",
        "value": round(T / (res["freq4"] * 1e-3), 1), "unit": "query-rows/s",
        "steps": K, "warmup": W, "ms_per_step": round(res["freq4"], 4),
        "workload": "IndexCache stack: 61 layers, freq 4 offset 2 "
                    f"({n_full['freq4']} F), a seeded 61-character pattern "
                    f"({n_full['pattern']} F) and freq 1 (61 F); 32 decode "
                    "requests x 16384 context, H=64, index_topk 2048, every "
                    "layer its own K cache, q and weights",
        "pattern": pattern,
        "ms": {name: round(v, 4) for name, v in res.items()},
        "full_layers": n_full,
        "speedup_vs_freq1": {name: round(res["freq1"] / v, 3)
                             for name, v in res.items()},
        "full_layer_ratio": {name: round(61 / f, 3)
                             for name, f in n_full.items()},
        "stack_hbm_gbs": {name: round(n_full[name] * per_layer_bytes /
                                      (v * 1e-3) / 1e9, 1)
                          for name, v in res.items()},
        "f_layer_logits_ms": round(kl, 5),
        "f_layer_logits_roofline": {
            "bound": "hbm", "achieved": round(per_layer_bytes /
                                              (kl * 1e-3) / 1e9, 1),
            "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(per_layer_bytes / (kl * 1e-3) / 1e9 / HBM_PEAK_GBS,
                          4),
            "algorithmic_bytes": per_layer_bytes},
    }
    if cpu_rec is not None:
        rec["cpu_baseline"] = cpu_rec
    return rec


def cpu_baseline_index_cache(host_layers, ref, L, seconds):
    """Time the CPU oracle's layer loop over the freq-4 / offset-2 stack of
    L layers (quantise q, logits and top-k on every F layer, the shared
    buffer kept on every S layer) for the whole batch, in whole passes
    repeated until ``seconds`` of work.  ``host_layers`` maps each F layer
    to its host inputs; BLAS threads = the usable cores."""
    from oracle import index_cache as oic
    model, cores = host_cpu()
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=cores)
    except Exception:                                   # pragma: no cover
        limiter = None
    mask = oic.skip_mask(L, freq=4, offset=2)
    layers = [None if mask[l] else
              {"q": host_layers[l].q_bf16.float().numpy(),
               "weights": host_layers[l].weights,
               "k_cache": host_layers[l].k_cache} for l in range(L)]
    buf = np.full((ref.T, ref.k), -1, np.int32)
    try:
        t0 = time.perf_counter()
        reps = 0
        while True:
            oic.run(layers, ref.block_table, ref.query_start_loc,
                    ref.positions, ref.ld, ref.k, buf, freq=4, offset=2)
            reps += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
    finally:
        if limiter is not None:
            limiter.unregister()
    n_f = int(sum(1 for m in mask if not m))
    return {"value": reps * ref.T / el, "unit": "query-rows/s",
            "cores": int(cores), "kind": "oracle", "cpu_model": model,
            "sample": f"whole batch ({ref.T} rows), the freq-4 stack of {L} "
                      f"layers ({n_f} F), {reps} pass(es) in {el:.1f} s "
                      "(numpy fp64 oracle layer loop: quantise q, logits, "
                      "sort-based top-k per F layer)"}


if __name__ == "__main__":
    main()
