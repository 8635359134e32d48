#!/usr/bin/env python3
"""Benchmark of the device-wide prefix scan on one MI355X.

Default workload (the headline metric): float32 inclusive add-scan of
n = 2^28 values uniform in [0, 1) (seed 2), input and output resident in HBM.
One step is one scan_inclusive call over the whole array (a single
multi-tile look-back kernel launch).  W untimed warm-up steps, then K timed
steps back to back between two device synchronisations; two HIP events on
the stream the launches run on, before the first and after the last, give
the kernel's average duration for the roofline entry (gaps between launches
included).

Before the warm-up steps the step runs untimed, back to back, for about
--settle-ms (default 200 ms): after the GPU has been idle, launches 6-40 of
this size run 3-9% slower than the first five and than every later one (a
transient of the GPU's clocks or power state: the kernel is the same, and
100 ms of load before the timed launches removes it).  With 5 warm-up steps
the timed region would otherwise sit inside the transient.  The JSON line
records the settle time and launch count.

Prints one JSON line.  value = Gelem/s (n * K / elapsed).  Effective HBM
traffic counts the minimal 1 read + 1 write per element (8 bytes).

Also reported:
  roofline      HBM-bound: algorithmic bytes per launch / average launch time
                against MI355X's 8 TB/s; `traffic` is the counter-measured HBM
                bytes per launch from the committed rocprofv3 summary, used only
                while the kernel sources still match the ones it was taken on.
  cpu_baseline  the sequential oracle on one host core over a bounded sample
                (the first 2^26 elements of the same input).
  copy_probe    a plain 16-byte copy of 1 GiB with streaming hints, for the
                achievable bandwidth of a one-read-one-write kernel.

--suite FILE additionally times every workload (int32 exclusive add at 2^20
and 2^28, int32 max, uint32 bitwise or, compaction, affine, segmented add, (maximum, count),
2x2 and 3x3 matrices, CSR row offsets, a 256-bin histogram, radix split passes and a
four-pass sort, the
max-scan size sweep with reduce-then-scan beside it) and writes one JSON line
per workload to FILE.

--latency FILE times the latency regime (config 1, int32 exclusive add at
2^20 on every path; the one-workgroup / one-tile crossover; the int32 max
sweep 4^5..4^13 with reduce-then-scan beside it): per-call medians with the
inputs cache-resident and after a 512 MiB flush, and back-to-back averages,
one JSON line per case; every case starts with a small copy-probe launch so
that a kernel trace of the same run splits into cases
(--summarize-latency).

--workloads-once K runs each full-size workload K times (for rocprofv3
passes); --summarize-rocprof, --summarize-traffic, --summarize-wl-trace and
--summarize-wl-insts, --summarize-latency and --summarize-dispatches turn
rocprofv3 CSV output into the summaries under profiles/.
"""
import argparse
import hashlib
import glob
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_GBPS = 8000.0
N_MAIN = 1 << 28
METRIC = "scan Gelem/s + effective HBM GB/s (% of peak), fp32/int32 n=2^28, 1 MI355X"
PROFILES = os.path.join(ROOT, "profiles")
TRAFFIC_FILE = os.path.join(PROFILES, "traffic_f32_inclusive_add_2p28.txt")
STATS_FILE = os.path.join(PROFILES, "kernel_stats_f32_inclusive_add_2p28.txt")
TRAFFIC_ALL_FILE = os.path.join(PROFILES, "traffic_all_workloads.txt")
SCAN_KERNEL = "tile_scan_persistent"
COPY_KERNEL = "copy_probe_kernel"
PROFILE_CMDS = {
    "trace": "rocprofv3 --kernel-trace --stats -f csv -d $OUT/prof_trace -o bench -- "
             "python3 bench.py --steps 200 --warmup 200 --no-cpu-baseline",
    "fetch": "rocprofv3 --pmc FETCH_SIZE -f csv -d $OUT/prof_fetch -o bench -- "
             "python3 bench.py --steps 3 --warmup 1 --no-cpu-baseline",
    "write": "rocprofv3 --pmc WRITE_SIZE -f csv -d $OUT/prof_write -o bench -- "
             "python3 bench.py --steps 3 --warmup 1 --no-cpu-baseline",
    "wl_fetch": "rocprofv3 --pmc FETCH_SIZE -f csv -d $OUT/prof_wl_fetch -o wl -- "
                "python3 bench.py --workloads-once 3",
    "wl_write": "rocprofv3 --pmc WRITE_SIZE -f csv -d $OUT/prof_wl_write -o wl -- "
                "python3 bench.py --workloads-once 3",
    "wl_trace": "rocprofv3 --kernel-trace -f csv -d $OUT/prof_wl_trace -o wl -- "
                "python3 bench.py --workloads-once 40 --settle-ms 200",
    "latency": "rocprofv3 --kernel-trace -f csv -d $OUT/prof_lat -o lat -- "
               "python3 bench.py --latency $OUT/latency_traced.jsonl",
    "driver": "rocprofv3 --kernel-trace --stats -f csv -d $OUT/prof_drv -o drv -- "
              "python3 bench.py --gpus 1 --steps 20 --warmup 5",
    "driver_nosettle": "rocprofv3 --kernel-trace --stats -f csv -d $OUT/prof_drv0 -o drv -- "
                       "python3 bench.py --gpus 1 --steps 20 --warmup 5 --settle-ms 0",
    "wl_insts": "rocprofv3 --pmc SQ_WAVES SQ_INSTS_VALU SQ_INSTS_SALU SQ_INSTS_LDS SQ_INSTS_VMEM_RD "
                "SQ_INSTS_VMEM_WR SQ_LDS_BANK_CONFLICT GRBM_GUI_ACTIVE -f csv -d $OUT/prof_wl_insts -o wl -- "
                "python3 bench.py --workloads-once 3",
}
WL_INSTS_FILE = os.path.join(ROOT, "profiles", "instructions_all_workloads.txt")
# one wave64 VALU instruction keeps a 16-lane SIMD busy for at least 4 cycles;
# MI355X: 256 CUs x 4 SIMDs at 2.4 GHz
VALU_ISSUE_PER_S = 256 * 4 * 2.4e9 / 4
WL_TRACE_FILE = os.path.join(ROOT, "profiles", "kernel_times_all_workloads.txt")
LATENCY_FILE = os.path.join(ROOT, "profiles", "kernel_times_latency_regime.txt")
DISPATCH_FILE = os.path.join(ROOT, "profiles", "dispatches_f32_inclusive_add_2p28_driver_command.txt")
MALL_BYTES = 256 << 20  # MI355X Infinity Cache (L2s: 4 MiB per XCD)
FLUSH_BYTES = 512 << 20

# Latency-regime cases: (label, op, exclusive, n, input, small_n_max, multi-tile mode).
# small_n_max None: the library default (one tile); 0 with mode 1: one workgroup per
# tile forced; 1 << 40: the single-workgroup kernel forced.
_SINGLE, _AUTO = 1 << 40, None
LATENCY_CASES = (
    [("int32 exclusive add 2^%d, %s" % (k, path), "add", True, 1 << k, "int32_0_15", lim, mode)
     for k in (10, 12, 13, 14, 15, 16)
     for path, lim, mode in (("one workgroup", _SINGLE, 0), ("one workgroup per tile", 0, 1))]
    + [("config 1: int32 exclusive add 2^20, %s" % path, "add", True, 1 << 20, "int32_0_15", lim, mode)
       for path, lim, mode in (("auto", _AUTO, 0), ("persistent", 0, 2), ("reduce-then-scan", 0, 3))]
    + [("int32 inclusive max 4^%d, auto" % k, "max", False, 4 ** k, "int32_full", _AUTO, 0) for k in range(5, 14)]
    + [("int32 inclusive max 4^%d, reduce-then-scan" % k, "max", False, 4 ** k, "int32_full", 0, 3)
       for k in range(9, 14)]
)

# Full-size workloads for per-kernel counter runs: (label, kernel-name fragment,
# n, algorithmic bytes per launch as a function of n and the kept count).
WORKLOADS = [
    ("float32 inclusive add 2^28", "tile_scan_persistent<dwpt::OpAdd<float>, false", 1 << 28,
     lambda n, kept: 8 * n),
    ("int32 exclusive add 2^28", "tile_scan_persistent<dwpt::OpAdd<int>, true", 1 << 28, lambda n, kept: 8 * n),
    ("int32 inclusive max 2^28", "tile_scan_persistent<dwpt::OpMax<int>, false", 1 << 28, lambda n, kept: 8 * n),
    ("compaction float32 N(0,1) 2^28 (read all, write kept)", "compact_persistent<float", 1 << 28,
     lambda n, kept: 4 * n + 4 * kept),
    ("uint32 affine inclusive 2^26 pairs", "tile_scan_persistent<dwpt::OpAffine, false", 1 << 26,
     lambda n, kept: 16 * n),
    ("segmented int32 inclusive add 2^27 (values, head bytes, out)",
     "tile_scan_persistent<dwpt::OpSeg<dwpt::OpAdd<int> >, false", 1 << 27, lambda n, kept: 9 * n),
    ("(maximum, count) inclusive 2^27 pairs", "tile_scan_persistent<dwpt::OpMaxCount, false", 1 << 27,
     lambda n, kept: 16 * n),
    ("2x2 matrix product inclusive 2^25 matrices", "tile_scan_persistent<dwpt::OpMat2, false", 1 << 25,
     lambda n, kept: 32 * n),
    ("3x3 matrix product inclusive 2^24 matrices", "tile_scan_persistent<dwpt::OpMat3, false", 1 << 24,
     lambda n, kept: 72 * n),
    ("CSR row counts, 2^27 sorted COO row indices (indices read once)", "csr_count_kernel", 1 << 27,
     lambda n, kept: 4 * n),
    ("histogram counts, 2^27 uniform indices over 256 bins (indices read once)", "csr_count_small_kernel", 1 << 27,
     lambda n, kept: 4 * n),
    ("radix split histogram pass, 2^28 uint32 keys (keys read once)", "radix_hist_kernel", 1 << 28,
     lambda n, kept: 4 * n),
    ("radix split scatter pass, 2^28 uint32 keys (keys read + written)", "radix_scatter_kernel<false>", 1 << 28,
     lambda n, kept: 8 * n),
]


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "device_wide_prefix_tile_amd", "csrc", "*"))):
        with open(p, "rb") as f:
            h.update(os.path.basename(p).encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def read_kv(path):
    rec = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, _, v = line.partition(":")
                rec[k.strip()] = v.strip()
    return rec


def counter_traffic():
    """HBM bytes per launch from the committed counter summary, if it matches the sources."""
    try:
        rec = read_kv(TRAFFIC_FILE)
    except OSError:
        return None
    if rec.get("source_hash") != kernel_source_hash():
        return None
    try:
        return int(float(rec["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def _csv_rows(directory, suffix):
    import csv
    rows = []
    for path in sorted(glob.glob(os.path.join(directory, "**", "*" + suffix), recursive=True)):
        with open(path, newline="") as f:
            rows.extend(csv.DictReader(f))
    return rows


def _short(name):
    name = name.replace("(anonymous namespace)::", "").split("(")[0]
    return name.replace("void dwpt::", "").replace("dwpt::", "")[:110]


def summarize_rocprof(trace_dir, fetch_dir, write_dir):
    """Write the kernel-time and HBM-traffic summaries under profiles/ from rocprofv3 CSV output."""
    stats = _csv_rows(trace_dir, "kernel_stats.csv")
    lines = ["# rocprofv3 kernel statistics, float32 inclusive add-scan n=2^28 (bench.py workload)",
             "# command: " + PROFILE_CMDS["trace"],
             "# kernel | calls | average us | min us | max us | share %"]
    scan_avg = None
    for r in stats:
        avg = float(r["AverageNs"]) / 1e3
        lines.append("%s | %s | %.2f | %.2f | %.2f | %.1f" % (_short(r["Name"]), r["Calls"], avg,
                                                           float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3,
                                                           float(r["Percentage"])))
        if SCAN_KERNEL in r["Name"] and "float" in r["Name"]:
            scan_avg = avg
    if scan_avg is not None:
        lines.append("scan_kernel_average_us: %.2f" % scan_avg)
        lines.append("scan_kernel_effective_GBps: %.1f" % (8 * N_MAIN / (scan_avg * 1e-6) / 1e9))
    with open(STATS_FILE, "w") as f:
        f.write("\n".join(lines) + "\n")

    def per_dispatch(directory, counter):
        vals = {"scan": [], "copy": []}
        for r in _csv_rows(directory, "counter_collection.csv"):
            if r.get("Counter_Name") != counter:
                continue
            name = r.get("Kernel_Name", "")
            v = float(r["Counter_Value"])
            if SCAN_KERNEL in name and "float" in name:
                vals["scan"].append(v)
            elif COPY_KERNEL in name:
                vals["copy"].append(v)
        return {k: (sum(v) / len(v) if v else None) for k, v in vals.items()}

    fetch = per_dispatch(fetch_dir, "FETCH_SIZE")
    write = per_dispatch(write_dir, "WRITE_SIZE")
    copy_kib = (1 << 30) / 1024.0  # the copy probe reads and writes 1 GiB per launch
    out = ["# HBM traffic of the float32 inclusive add-scan kernel, n=2^28, per launch",
           "# commands: " + PROFILE_CMDS["fetch"],
           "#           " + PROFILE_CMDS["write"],
           "# FETCH_SIZE / WRITE_SIZE are KiB per dispatch; each is scaled by what the same counter",
           "# reads for the 1 GiB copy probe (1048576 KiB each way) so the figure is in true bytes.",
           "source_hash: " + kernel_source_hash()]
    if None not in (fetch["scan"], fetch["copy"], write["scan"], write["copy"]):
        fs, ws = copy_kib / fetch["copy"], copy_kib / write["copy"]
        rd = fetch["scan"] * fs * 1024
        wr = write["scan"] * ws * 1024
        out += ["copy_fetch_kib: %.0f" % fetch["copy"], "copy_write_kib: %.0f" % write["copy"],
                "fetch_scale: %.4f" % fs, "write_scale: %.4f" % ws,
                "scan_fetch_kib: %.0f" % fetch["scan"], "scan_write_kib: %.0f" % write["scan"],
                "hbm_read_bytes_per_launch: %.0f" % rd, "hbm_write_bytes_per_launch: %.0f" % wr,
                "hbm_bytes_per_launch: %.0f" % (rd + wr),
                "algorithmic_bytes_per_launch: %d" % (8 * N_MAIN),
                "traffic_over_algorithmic: %.4f" % ((rd + wr) / (8 * N_MAIN))]
    else:
        out.append("# counters missing: fetch=%r write=%r" % (fetch, write))
    with open(TRAFFIC_FILE, "w") as f:
        f.write("\n".join(out) + "\n")
    print(open(STATS_FILE).read())
    print(open(TRAFFIC_FILE).read())


def _counter_means(directory, counter, fragments):
    """Mean counter value per dispatch for each kernel-name fragment (None if absent)."""
    vals = {f: [] for f in fragments}
    for r in _csv_rows(directory, "counter_collection.csv"):
        if r.get("Counter_Name") != counter:
            continue
        for f in fragments:
            if f in r.get("Kernel_Name", ""):
                vals[f].append(float(r["Counter_Value"]))
    return {f: (sum(v) / len(v) if v else None) for f, v in vals.items()}


def summarize_workload_traffic(fetch_dir, write_dir):
    """HBM bytes per launch of every full-size workload against its algorithmic bytes."""
    import numpy as np
    import seeded_inputs as si
    frags = [COPY_KERNEL] + [w[1] for w in WORKLOADS]
    fetch = _counter_means(fetch_dir, "FETCH_SIZE", frags)
    write = _counter_means(write_dir, "WRITE_SIZE", frags)
    kept = int(np.count_nonzero(si.float32_normal(3, 1 << 28) > 0))
    out = ["# HBM traffic per launch of each full-size workload (rocprofv3 counters)",
           "# commands: " + PROFILE_CMDS["wl_fetch"],
           "#           " + PROFILE_CMDS["wl_write"],
           "# FETCH_SIZE / WRITE_SIZE (KiB per dispatch) scaled by what the same counter reads for",
           "# the 1 GiB copy probe; algorithmic bytes = one read of every input byte + one write of",
           "# every output byte.",
           "source_hash: " + kernel_source_hash(),
           "compaction_kept: %d" % kept,
           "# workload | read MB | write MB | total MB | algorithmic MB | traffic / algorithmic"]
    if fetch[COPY_KERNEL] and write[COPY_KERNEL]:
        copy_kib = (1 << 30) / 1024.0
        fs, ws = copy_kib / fetch[COPY_KERNEL], copy_kib / write[COPY_KERNEL]
        out.append("fetch_scale: %.4f  write_scale: %.4f" % (fs, ws))
        for label, frag, n, alg in WORKLOADS:
            if fetch[frag] is None or write[frag] is None:
                out.append("%s | counters missing" % label)
                continue
            rd, wr, a = fetch[frag] * fs * 1024, write[frag] * ws * 1024, alg(n, kept)
            out.append("%s | %.1f | %.1f | %.1f | %.1f | %.4f" % (label, rd / 1e6, wr / 1e6, (rd + wr) / 1e6,
                                                                 a / 1e6, (rd + wr) / a))
    else:
        out.append("# copy probe counters missing")
    with open(TRAFFIC_ALL_FILE, "w") as f:
        f.write("\n".join(out) + "\n")
    print(open(TRAFFIC_ALL_FILE).read())


def summarize_workload_trace(trace_dir):
    """Kernel durations of every full-size workload's dominant kernel (kernel trace of
    --workloads-once K --settle-ms 200: the median over the last 20 of the kernel's dispatches,
    which follow 200 ms of untimed ones) against its algorithmic bytes."""
    import numpy as np
    import seeded_inputs as si
    durs = {w[1]: [] for w in WORKLOADS}
    rows = sorted(_csv_rows(trace_dir, "kernel_trace.csv"), key=lambda r: int(r["Start_Timestamp"]))
    for r in rows:
        for frag in durs:
            if frag in r.get("Kernel_Name", ""):
                durs[frag].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    kept = int(np.count_nonzero(si.float32_normal(3, 1 << 28) > 0))
    out = ["# Kernel duration per launch of each full-size workload's main kernel (rocprofv3 kernel trace)",
           "# command: " + PROFILE_CMDS["wl_trace"],
           "# median over the kernel's last 20 dispatches (after 200 ms of untimed ones); GB/s = algorithmic",
           "# bytes / duration",
           "source_hash: " + kernel_source_hash(),
           "# workload | kernel | dispatches | median us | algorithmic MB | GB/s | % of 8 TB/s"]
    for label, frag, n, alg in WORKLOADS:
        d = durs[frag]
        if not d:
            out.append("%s | %s | 0 | missing" % (label, frag))
            continue
        med = statistics.median(d[-20:])
        a = alg(n, kept)
        out.append("%s | %s | %d | %.2f | %.1f | %.1f | %.1f" % (label, frag, len(d), med, a / 1e6,
                                                                a / (med * 1e-6) / 1e9,
                                                                100 * a / (med * 1e-6) / 1e9 / PEAK_GBPS))
    with open(WL_TRACE_FILE, "w") as f:
        f.write("\n".join(out) + "\n")
    print(open(WL_TRACE_FILE).read())


def summarize_workload_insts(insts_dir, trace_summary=WL_TRACE_FILE):
    """Instruction counts per launch of every full-size workload's main kernel (SQ counters,
    summed over the chip), and the time the VALU instructions alone need at full issue rate,
    against the kernel's measured duration."""
    names = ("SQ_WAVES", "SQ_INSTS_VALU", "SQ_INSTS_SALU", "SQ_INSTS_LDS", "SQ_INSTS_VMEM_RD",
             "SQ_INSTS_VMEM_WR", "SQ_LDS_BANK_CONFLICT", "GRBM_GUI_ACTIVE")
    per = {}
    for name in names:
        per[name] = _counter_means(insts_dir, name, [w[1] for w in WORKLOADS])
    dur = {}
    if os.path.exists(trace_summary):
        for line in open(trace_summary):
            parts = [x.strip() for x in line.split("|")]
            if len(parts) >= 4 and not line.startswith("#"):
                try:
                    dur[parts[1]] = float(parts[3])
                except ValueError:
                    pass
    out = ["# Instructions per launch of each full-size workload's main kernel (rocprofv3 SQ counters)",
           "# command: " + PROFILE_CMDS["wl_insts"],
           "# mean over the kernel's dispatches; counters summed over the chip.  valu_us = VALU",
           "# instructions x 4 cycles / (1024 SIMDs x 2.4 GHz): the least time they need; kernel_us from",
           "# " + os.path.basename(trace_summary) + "; lds_conflict_share = LDS bank-conflict cycles / (256 CUs x",
           "# GRBM_GUI_ACTIVE / 8 XCDs), the share of each CU's time spent in bank conflicts.",
           "source_hash: " + kernel_source_hash(),
           "# workload | waves | VALU | SALU | LDS | VMEM rd | VMEM wr | valu_us | kernel_us | valu/kernel | "
           "lds_conflict_share"]
    for label, frag, n, alg in WORKLOADS:
        v = {k: per[k][frag] for k in names}
        if v["SQ_INSTS_VALU"] is None:
            out.append("%s | counters missing" % label)
            continue
        valu_us = v["SQ_INSTS_VALU"] / VALU_ISSUE_PER_S * 1e6
        k_us = dur.get(frag)
        gui = v["GRBM_GUI_ACTIVE"] / 8 if v["GRBM_GUI_ACTIVE"] else None
        conf = v["SQ_LDS_BANK_CONFLICT"] / (256 * gui) if gui and v["SQ_LDS_BANK_CONFLICT"] is not None else None
        out.append("%s | %.0f | %.4g | %.4g | %.4g | %.4g | %.4g | %.1f | %s | %s | %s" % (
            label, v["SQ_WAVES"], v["SQ_INSTS_VALU"], v["SQ_INSTS_SALU"], v["SQ_INSTS_LDS"], v["SQ_INSTS_VMEM_RD"],
            v["SQ_INSTS_VMEM_WR"], valu_us, "%.1f" % k_us if k_us else "-",
            "%.2f" % (valu_us / k_us) if k_us else "-", "%.2f" % conf if conf is not None else "-"))
    with open(WL_INSTS_FILE, "w") as f:
        f.write("\n".join(out) + "\n")
    print(open(WL_INSTS_FILE).read())


def _dispatches(trace_dir):
    """(name, start ns, end ns) of every dispatch in a kernel trace, in start order."""
    rows = sorted(_csv_rows(trace_dir, "kernel_trace.csv"), key=lambda r: int(r["Start_Timestamp"]))
    return [(r.get("Kernel_Name", ""), int(r["Start_Timestamp"]), int(r["End_Timestamp"])) for r in rows]


def _ours(name):
    return "dwpt::" in name or "zero_words_kernel" in name


def _calls(disp):
    """Groups a case's dispatches into calls: a call starts at each dispatch of the kernel
    that started the case (reduce-then-scan: tile totals, carries, seeded scan)."""
    disp = [d for d in disp if _ours(d[0]) and "zero_words_kernel" not in d[0]]
    calls = []
    for d in disp:
        if not calls or d[0] == disp[0][0]:
            calls.append([])
        calls[-1].append(d)
    return calls


def summarize_latency(trace_dir, jsonl_path):
    """Per-call kernel time of each latency-regime case from a kernel trace of --latency
    (split into cases at the copy-probe markers), beside the event timings of an unprofiled
    --latency run."""
    disp = _dispatches(trace_dir)
    segs, cur = [], None
    for d in disp:
        if COPY_KERNEL in d[0]:
            cur = []
            segs.append(cur)
        elif cur is not None:
            cur.append(d)
    events = {}
    if jsonl_path and os.path.exists(jsonl_path):
        for line in open(jsonl_path):
            rec = json.loads(line)
            events[rec["case"]] = rec
    out = ["# Latency regime: kernel time per call of each case (rocprofv3 kernel trace), beside the",
           "# event timings of the same cases in a run without the profiler",
           "# trace: " + PROFILE_CMDS["latency"],
           "# events: python3 bench.py --latency $OUT/latency.jsonl",
           "# kernel_us: the call's kernels' summed durations; span_us: first kernel start to last",
           "# kernel end (reduce-then-scan: three launches); medians over the last 200 cache-resident",
           "# calls and over 30 calls that each follow a 512 MiB flush (cold).  event_us: one call",
           "# between its own events (launch included); b2b_us: average of 200 calls back to back.",
           "source_hash: " + kernel_source_hash(),
           "# case | kernels | kernel_us | span_us | cold kernel_us | event_us | b2b_us | cold event_us"]
    if len(segs) != 2 * len(LATENCY_CASES):
        out.append("# trace holds %d marked segments, expected %d" % (len(segs), 2 * len(LATENCY_CASES)))
    for i, case in enumerate(LATENCY_CASES):
        label = case[0]
        if 2 * i + 1 >= len(segs):
            out.append("%s | missing" % label)
            continue
        hot, cold = _calls(segs[2 * i])[-200:], _calls(segs[2 * i + 1])
        names = " + ".join(_short(d[0]).split("<")[0] for d in (hot[-1] if hot else []))

        def med(calls, span):
            if not calls:
                return float("nan")
            if span:
                return statistics.median((c[-1][2] - c[0][1]) / 1e3 for c in calls)
            return statistics.median(sum(d[2] - d[1] for d in c) / 1e3 for c in calls)
        ev = events.get(label, {})
        out.append("%s | %s | %.2f | %.2f | %.2f | %s | %s | %s" % (
            label, names, med(hot, False), med(hot, True), med(cold, False), ev.get("median_us", "-"),
            ev.get("back_to_back_us", "-"), ev.get("cold_median_us", "-")))
    with open(LATENCY_FILE, "w") as f:
        f.write("\n".join(out) + "\n")
    print(open(LATENCY_FILE).read())


def summarize_dispatches(trace_dir, trace_dir_nosettle):
    """Per-dispatch durations of the headline scan kernel in traces of the driver's command
    (python3 bench.py --gpus 1 --steps 20 --warmup 5), with and without the settle phase."""
    out = ["# Per-dispatch durations of the float32 inclusive add-scan kernel, n=2^28, under the",
           "# benchmark driver's command, after the GPU was idle",
           "# with settle:    " + PROFILE_CMDS["driver"],
           "# without settle: " + PROFILE_CMDS["driver_nosettle"],
           "# The warm-up and timed launches are the last 25 scan dispatches before the first copy-probe",
           "# dispatch; the settle launches come before them.",
           "source_hash: " + kernel_source_hash()]
    for title, d in (("with settle", trace_dir), ("without settle (--settle-ms 0)", trace_dir_nosettle)):
        disp = _dispatches(d)
        first_copy = next((i for i, x in enumerate(disp) if COPY_KERNEL in x[0]), len(disp))
        scans = [(x[2] - x[1]) / 1e3 for x in disp[:first_copy] if SCAN_KERNEL in x[0] and "float" in x[0]]
        settle, main = scans[:-25], scans[-25:]
        out.append("")
        out.append("## " + title)
        out.append("settle_dispatches: %d" % len(settle))
        if settle:
            blocks = [settle[i:i + 50] for i in range(0, len(settle), 50)]
            out.append("settle_mean_us_per_50: " + " ".join("%.1f" % (sum(b) / len(b)) for b in blocks))
        out.append("warmup_us: " + " ".join("%.1f" % v for v in main[:5]))
        out.append("timed_us: " + " ".join("%.1f" % v for v in main[5:]))
        if len(main) == 25:
            out.append("timed_mean_us: %.2f" % (sum(main[5:]) / 20))
            out.append("timed_frac_of_8TBps: %.4f" % (8 * N_MAIN / (sum(main[5:]) / 20 * 1e-6) / 1e9 / PEAK_GBPS))
    with open(DISPATCH_FILE, "w") as f:
        f.write("\n".join(out) + "\n")
    print(open(DISPATCH_FILE).read())


def latency(dw, torch, si, out_path, steps=200):
    """Times each latency-regime case; one JSON line per case to out_path."""
    import numpy as np
    flush = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
    mark_a = torch.zeros(1024, dtype=torch.float32, device="cuda")
    mark_b = torch.empty_like(mark_a)
    lines = []
    for label, op, excl, n, gen, lim, mode in LATENCY_CASES:
        log("latency: " + label)
        x_host = getattr(si, gen)(7, n)
        x = torch.from_numpy(x_host).cuda()
        y = torch.empty_like(x)
        scan = dw.scan_exclusive if excl else dw.scan_inclusive
        fn = lambda: scan(x, op, out=y)  # noqa: E731
        old_lim = dw.scan_set_small_n_max(dw.SCAN_SMALL_N_AUTO if lim is None else lim)
        old_mode = dw.scan_set_multi_tile_mode(mode)
        try:
            torch.cuda.synchronize()
            dw.scan_copy_probe(mark_a, mark_b)  # marks the start of the case in a kernel trace
            _, ms = time_launches(fn, steps, 100, torch)
            _, t = time_back_to_back(fn, steps, 0, torch)
            torch.cuda.synchronize()
            dw.scan_copy_probe(mark_a, mark_b)  # the cold calls
            cold = time_cold(fn, 30, flush, torch)
        finally:
            dw.scan_set_small_n_max(old_lim)
            dw.scan_set_multi_tile_mode(old_mode)
        y_host = y.cpu().numpy()
        # the last output against a direct fold of the input
        if op == "add":
            v = x_host[:-1] if excl else x_host
            want = np.array([int(np.sum(v, dtype=np.int64)) & 0xFFFFFFFF], dtype=np.uint32).view(np.int32)[0]
        else:
            want = x_host.max()
        lines.append({"case": label, "n": n, "median_us": round(statistics.median(ms) * 1e3, 2),
                      "back_to_back_us": round(t * 1e6, 2), "cold_median_us": round(cold * 1e3, 2),
                      "last_ok": bool(y_host[-1] == want)})
    del flush
    torch.cuda.synchronize()
    assert dw.scan_get_device_error() == 0, "device reported a look-back timeout"
    with open(out_path, "w") as f:
        for l in lines:
            f.write(json.dumps(l) + "\n")
    print(json.dumps({"latency_cases": len(lines), "all_last_ok": all(l["last_ok"] for l in lines)}), flush=True)


def workloads_once(dw, torch, si, steps, settle_ms=0.0):
    """Each full-size workload `steps` times, one input resident at a time (for counter runs
    and kernel traces); with settle_ms, each workload first runs untimed for that long, so
    that the traced launches are past the clock transient that follows the input's upload."""
    import numpy as np

    def run(fn):
        if settle_ms > 0:
            settle_clocks(fn, settle_ms, torch)
        for _ in range(steps):
            fn()
    a = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1.0)
    run(lambda: dw.scan_copy_probe(a, b))
    del a, b
    x = torch.from_numpy(si.float32_01(2, 1 << 28)).cuda()
    y = torch.empty_like(x)
    run(lambda: dw.scan_inclusive(x, "add", out=y))
    del x, y
    x = torch.from_numpy(si.int32_0_15(1, 1 << 28)).cuda()
    y = torch.empty_like(x)
    run(lambda: dw.scan_exclusive(x, "add", out=y))
    run(lambda: dw.scan_inclusive(x, "max", out=y))
    del x, y
    x = torch.from_numpy(si.float32_normal(3, 1 << 28)).cuda()
    y = torch.empty_like(x)
    cnt = torch.zeros(1, dtype=torch.uint32, device="cuda")
    run(lambda: dw.compact(x, out=y, count=cnt))
    del x, y
    ab = torch.from_numpy(si.affine_pairs(4, 1 << 26)).cuda()
    yab = torch.empty_like(ab)
    run(lambda: dw.scan_inclusive(ab, "affine", out=yab))
    del ab, yab
    xs = torch.from_numpy(si.int32_pm100(5, 1 << 27)).cuda()
    hs = torch.from_numpy(si.segment_heads(5, 1 << 27, 1000.0)).cuda()
    ys = torch.empty_like(xs)
    run(lambda: dw.segmented_scan(xs, hs, "add", out=ys))
    del xs, hs, ys
    vc = torch.from_numpy(si.maxcount_pairs(8, 1 << 27)).cuda()
    yvc = torch.empty_like(vc)
    run(lambda: dw.scan_inclusive(vc, "maxcount", out=yvc))
    del vc, yvc
    m = torch.from_numpy(si.mat2_elems(9, 1 << 25)).cuda()
    ym = torch.empty_like(m)
    run(lambda: dw.scan_inclusive(m, "mat2", out=ym))
    del m, ym
    m3 = torch.from_numpy(si.mat3_elems(10, 1 << 24)).cuda()
    ym3 = torch.empty_like(m3)
    run(lambda: dw.scan_inclusive(m3, "mat3", out=ym3))
    del m3, ym3
    nnz, n_rows = 1 << 27, 1 << 23
    rows = torch.from_numpy(np.sort(si.uint32_full(10, nnz) % n_rows).astype(np.uint32)).cuda()
    rp = torch.empty(n_rows + 1, dtype=torch.uint32, device="cuda")
    run(lambda: dw.csr_row_offsets(rows, n_rows, out=rp))
    del rows, rp
    bins = torch.from_numpy((si.uint32_full(11, nnz) % 256).astype(np.uint32)).cuda()
    bp = torch.empty(257, dtype=torch.uint32, device="cuda")
    run(lambda: dw.csr_row_offsets(bins, 256, out=bp))
    del bins, bp
    k = torch.from_numpy(si.uint32_full(11, 1 << 28)).cuda()
    ko = torch.empty_like(k)
    run(lambda: dw.radix_split(k, 8, keys_out=ko))
    del k, ko
    torch.cuda.synchronize()
    err = dw.scan_get_device_error()
    print(json.dumps({"workloads_once": steps, "device_error": err}), flush=True)


def time_launches(fn, steps, warmup, torch):
    """Run fn() warmup times, then `steps` times between synchronisations.

    Returns (elapsed seconds of the timed region, list of per-launch event ms).
    """
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for a, b in evs:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    return elapsed, [a.elapsed_time(b) for a, b in evs]


def time_back_to_back(fn, steps, warmup, torch):
    """Run fn() warmup times, then `steps` times back to back between synchronisations.

    Returns (elapsed seconds of the timed region by the host clock, seconds per launch
    from HIP events recorded on the launches' stream before the first and after the
    last launch -- the launches' average duration, counting the short gaps between
    them).  No event sits between two launches, so the timed region is the plain
    job.
    """
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    a.record(stream)
    for _ in range(steps):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    return elapsed, a.elapsed_time(b) * 1e-3 / steps


def settle_clocks(fn, ms, torch):
    """Run fn back to back, untimed, for about `ms` milliseconds; returns the launch count."""
    launches = 0
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(8):
            fn()
        launches += 8
        torch.cuda.synchronize()
    return launches


def time_cold(fn, reps, flush, torch):
    """Median time of one call with nothing of its inputs in the caches: each call follows
    a write of `flush` (larger than the Infinity Cache) and sits between its own events."""
    stream = torch.cuda.current_stream()
    ms = []
    for _ in range(reps):
        flush.zero_()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        torch.cuda.synchronize()
        ms.append(a.elapsed_time(b))
    return statistics.median(ms)


def host_cpu():
    """CPU model and logical CPU count of the host the oracle runs on."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return "%s, %d logical CPUs (oracle uses 1)" % (model, os.cpu_count() or 0)


def cpu_baseline(x):
    import oracle
    sample = x[: 1 << 26]
    times = []
    t_start = time.perf_counter()
    while len(times) < 2 or (time.perf_counter() - t_start < 10.0 and len(times) < 20):
        t0 = time.perf_counter()
        y, s = oracle.scan("add", sample)
        times.append(time.perf_counter() - t0)
    med = statistics.median(times)
    return {"value": round(sample.shape[0] / med / 1e9, 4), "unit": "Gelem/s", "cores": 1, "kind": "oracle",
            "host": host_cpu(),
            "sample": "first 2^26 of the 2^28 float32 inputs, sequential double-accumulated inclusive add, "
                      "median of %d runs" % len(times)}, (y, s)


def copy_probe(dw, torch, nbytes=1 << 30, reps=20):
    a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1.0)
    _, per_launch = time_back_to_back(lambda: dw.scan_copy_probe(a, b), reps, 3, torch)
    del a, b
    return round(2 * nbytes / per_launch / 1e9, 1)


def suite(dw, torch, si, out_path, steps):
    """Time each workload at its full size; one JSON line per workload."""
    import numpy as np
    lines = []
    copy_gbps = copy_probe(dw, torch)
    flush = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")

    def rec(name, n, bytes_per_elem, fn):
        log("suite: " + name)
        # 100 launches warm the workload up; median_us: one call's time,
        # each launch between its own event pair (latency); the rates: the same number
        # of launches back to back (throughput, gaps between launches included)
        elapsed, ms = time_launches(fn, steps, 100, torch)
        _, t = time_back_to_back(fn, steps, 0, torch)
        line = {"workload": name, "n": n, "median_us": round(statistics.median(ms) * 1e3, 2),
                "back_to_back_us": round(t * 1e6, 2),
                "gelem_s": round(n / t / 1e9, 2),
                "effective_GBps": round(n * bytes_per_elem / t / 1e9, 1),
                "pct_of_peak": round(100 * n * bytes_per_elem / t / 1e9 / PEAK_GBPS, 1),
                "pct_of_copy": round(100 * n * bytes_per_elem / t / 1e9 / copy_gbps, 1)}
        if n * bytes_per_elem <= MALL_BYTES:
            # repeated calls find input and output in the Infinity Cache: the figures above
            # are cache-resident; cold_median_us is one call after a 512 MiB flush
            line["cache_resident"] = True
            line["cold_median_us"] = round(time_cold(fn, 30, flush, torch) * 1e3, 2)
        lines.append(line)

    x = torch.from_numpy(si.int32_0_15(1, 1 << 20)).cuda()
    y = torch.empty_like(x)
    rec("int32 exclusive add 2^20", 1 << 20, 8, lambda: dw.scan_exclusive(x, "add", out=y))
    x = torch.from_numpy(si.int32_0_15(1, 1 << 28)).cuda()
    y = torch.empty_like(x)
    rec("int32 exclusive add 2^28", 1 << 28, 8, lambda: dw.scan_exclusive(x, "add", out=y))
    rec("int32 inclusive max 2^28", 1 << 28, 8, lambda: dw.scan_inclusive(x, "max", out=y))
    del x, y
    xb = torch.from_numpy(si.uint32_full(12, 1 << 28)).cuda()
    yb = torch.empty_like(xb)
    rec("uint32 inclusive bitwise or 2^28", 1 << 28, 8, lambda: dw.scan_inclusive(xb, "or", out=yb))
    del xb, yb
    xc = torch.from_numpy(si.float32_normal(3, 1 << 28)).cuda()
    yc = torch.empty_like(xc)
    cnt = torch.zeros(1, dtype=torch.uint32, device="cuda")
    dw.compact(xc, out=yc, count=cnt)
    torch.cuda.synchronize()
    kept = int(cnt.cpu().numpy()[0])
    rec("compaction float32 N(0,1) 2^28 (bytes: read all + write kept)", 1 << 28, 4 + 4 * kept / (1 << 28),
        lambda: dw.compact(xc, out=yc, count=cnt))
    del xc, yc
    ab = torch.from_numpy(si.affine_pairs(4, 1 << 26)).cuda()
    yab = torch.empty_like(ab)
    rec("uint32 affine inclusive 2^26 pairs", 1 << 26, 16, lambda: dw.scan_inclusive(ab, "affine", out=yab))
    del ab, yab
    xs = torch.from_numpy(si.int32_pm100(5, 1 << 27)).cuda()
    hs = torch.from_numpy(si.segment_heads(5, 1 << 27, 1000.0)).cuda()
    ys = torch.empty_like(xs)
    rec("segmented int32 inclusive add 2^27", 1 << 27, 9, lambda: dw.segmented_scan(xs, hs, "add", out=ys))
    del xs, hs, ys
    vc = torch.from_numpy(si.maxcount_pairs(8, 1 << 27)).cuda()
    yvc = torch.empty_like(vc)
    rec("(maximum, count) inclusive 2^27 pairs, values in [-1000, 1000]", 1 << 27, 16,
        lambda: dw.scan_inclusive(vc, "maxcount", out=yvc))
    del vc, yvc
    m = torch.from_numpy(si.mat2_elems(9, 1 << 25)).cuda()
    ym = torch.empty_like(m)
    rec("2x2 uint32 matrix product inclusive 2^25 matrices", 1 << 25, 32, lambda: dw.scan_inclusive(m, "mat2", out=ym))
    del m, ym
    m3 = torch.from_numpy(si.mat3_elems(10, 1 << 24)).cuda()
    ym3 = torch.empty_like(m3)
    rec("3x3 uint32 matrix product inclusive 2^24 matrices", 1 << 24, 72,
        lambda: dw.scan_inclusive(m3, "mat3", out=ym3))
    del m3, ym3
    # CSR row offsets of 2^27 sorted COO row indices over 2^23 rows (16 per row on
    # average); per entry: the index read once, and 4 / 16 bytes of row_ptr written
    nnz, n_rows = 1 << 27, 1 << 23
    rows = torch.from_numpy(np.sort(si.uint32_full(10, nnz) % n_rows).astype(np.uint32)).cuda()
    rp = torch.empty(n_rows + 1, dtype=torch.uint32, device="cuda")
    rec("CSR row offsets, 2^27 sorted COO entries over 2^23 rows", nnz, 4 + 4 * (n_rows + 1) / nnz,
        lambda: dw.csr_row_offsets(rows, n_rows, out=rp))
    del rows, rp
    # histogram bin offsets of 2^27 uniform bin indices over 256 bins (per-workgroup LDS counts)
    bins = torch.from_numpy((si.uint32_full(11, nnz) % 256).astype(np.uint32)).cuda()
    bp = torch.empty(257, dtype=torch.uint32, device="cuda")
    rec("histogram bin offsets, 2^27 uniform indices over 256 bins", nnz, 4 + 4 * 257 / nnz,
        lambda: dw.csr_row_offsets(bins, 256, out=bp))
    del bins, bp
    # one radix-sort pass (stable split by the digit (key >> 8) & 255): algorithmic bytes are
    # one read and one write of every key (and value); the three launches move 12 B per key
    # plus the scan of 256 counts per 8192-key tile
    keys = torch.from_numpy(si.uint32_full(11, 1 << 28)).cuda()
    k1, k2 = torch.empty_like(keys), torch.empty_like(keys)
    rec("radix split pass, 2^28 uint32 keys", 1 << 28, 8, lambda: dw.radix_split(keys, 8, keys_out=k1))

    def four_passes():
        dw.radix_split(keys, 0, keys_out=k1)
        dw.radix_split(k1, 8, keys_out=k2)
        dw.radix_split(k2, 16, keys_out=k1)
        dw.radix_split(k1, 24, keys_out=k2)
    rec("radix sort (four 8-bit passes), 2^28 uint32 keys", 1 << 28, 32, four_passes)
    del keys, k1, k2
    keys = torch.from_numpy(si.uint32_full(12, 1 << 27)).cuda()
    vals = torch.from_numpy(si.uint32_full(13, 1 << 27)).cuda()
    ko, vo = torch.empty_like(keys), torch.empty_like(vals)
    rec("radix split pass, 2^27 uint32 key-value pairs", 1 << 27, 16,
        lambda: dw.radix_split(keys, 8, vals, keys_out=ko, vals_out=vo))
    del keys, vals, ko, vo
    for k in range(5, 16):
        n = 4 ** k
        xm = torch.from_numpy(si.int32_full(6, n)).cuda()
        ym = torch.empty_like(xm)
        rec("int32 inclusive max 4^%d" % k, n, 8, lambda: dw.scan_inclusive(xm, "max", out=ym))
        if 9 <= k <= 14:
            # the reduce-then-scan alternative at the same size (12 B/element of traffic; the
            # figure below still counts the algorithmic 8)
            old = dw.scan_set_multi_tile_mode(3)
            rec("int32 inclusive max 4^%d, reduce-then-scan" % k, n, 8, lambda: dw.scan_inclusive(xm, "max", out=ym))
            dw.scan_set_multi_tile_mode(old)
        del xm, ym
    xf = torch.from_numpy(si.float32_01(2, 1 << 28)).cuda()
    yf = torch.empty_like(xf)
    old = dw.scan_set_multi_tile_mode(3)
    rec("float32 inclusive add 2^28, reduce-then-scan", 1 << 28, 8, lambda: dw.scan_inclusive(xf, "add", out=yf))
    dw.scan_set_multi_tile_mode(old)
    del xf, yf, flush
    torch.cuda.empty_cache()
    with open(out_path, "w") as f:
        for l in lines:
            f.write(json.dumps(l) + "\n")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    # defaults: 200 warm-up and 200 timed launches (about 0.14 s of GPU time)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--settle-ms", type=float, default=200.0,
                    help="untimed back-to-back steps for about this long before the warm-up steps")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing")
    ap.add_argument("--latency", metavar="FILE", help="time the latency-regime cases, JSON lines to FILE, and exit")
    ap.add_argument("--summarize-latency", nargs=2, metavar=("TRACE_DIR", "JSONL"),
                    help="write the latency-regime summary under profiles/ and exit")
    ap.add_argument("--summarize-dispatches", nargs=2, metavar=("TRACE_DIR", "TRACE_DIR_NOSETTLE"),
                    help="write the per-dispatch summary of the driver-command traces and exit")
    ap.add_argument("--suite", metavar="FILE", help="also time every workload, JSON lines to FILE")
    ap.add_argument("--summarize-rocprof", nargs=3, metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/ summaries from rocprofv3 CSV output and exit")
    ap.add_argument("--workloads-once", type=int, metavar="K",
                    help="run every full-size workload K times (for counter runs) and exit")
    ap.add_argument("--summarize-wl-insts", metavar="PMC_DIR",
                    help="write the per-workload instruction summary from a --workloads-once SQ counter run")
    ap.add_argument("--summarize-wl-trace", metavar="TRACE_DIR",
                    help="write the per-workload kernel time summary from a --workloads-once trace")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the per-workload traffic summary under profiles/ and exit")
    args = ap.parse_args()
    args.settle_given = "--settle-ms" in sys.argv
    if args.summarize_rocprof:
        summarize_rocprof(*args.summarize_rocprof)
        return
    if args.summarize_wl_insts:
        summarize_workload_insts(args.summarize_wl_insts)
        return
    if args.summarize_wl_trace:
        summarize_workload_trace(args.summarize_wl_trace)
        return
    if args.summarize_traffic:
        summarize_workload_traffic(*args.summarize_traffic)
        return
    if args.summarize_latency:
        summarize_latency(*args.summarize_latency)
        return
    if args.summarize_dispatches:
        summarize_dispatches(*args.summarize_dispatches)
        return
    if args.gpus != 1:
        print("bench.py: the scan runs on one GPU; --gpus %d is not supported "
              "(the library does not shard a scan across GPUs)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import device_wide_prefix_tile_amd as dw
    import seeded_inputs as si

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dw.lib()
    if args.workloads_once:
        workloads_once(dw, torch, si, args.workloads_once, args.settle_ms if args.settle_given else 0.0)
        return
    if args.latency:
        latency(dw, torch, si, args.latency)
        return
    log("generating input")
    x_host = si.float32_01(2, N_MAIN)
    x = torch.from_numpy(x_host).cuda()
    y = torch.empty_like(x)
    torch.cuda.synchronize()

    step = lambda: dw.scan_inclusive(x, "add", out=y)  # noqa: E731
    settle_launches = settle_clocks(step, args.settle_ms, torch) if args.settle_ms > 0 else 0
    log("timing %d steps after %d warm-up steps (settle: %d launches)" % (args.steps, args.warmup, settle_launches))
    elapsed, avg_kernel_s = time_back_to_back(step, args.steps, args.warmup, torch)
    assert dw.scan_get_device_error() == 0, "device reported a look-back timeout"
    value = N_MAIN * args.steps / elapsed / 1e9
    bytes_per_launch = 8 * N_MAIN
    achieved = bytes_per_launch / avg_kernel_s / 1e9
    traffic = counter_traffic()

    result = {
        "metric": METRIC, "value": round(value, 2), "unit": "Gelem/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(elapsed / args.steps * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "float32 inclusive add-scan, n=2^28, values uniform in [0,1) (seed 2)",
                   "n": N_MAIN, "op": "add", "variant": "inclusive", "element": "float32",
                   "kernel": "persistent single-pass tile scan, streaming prefix resolver, 15360-element tiles"},
        "settle": {"ms": args.settle_ms, "launches": settle_launches},
        "effective_GBps": round(bytes_per_launch * args.steps / elapsed / 1e9, 1),
        "pct_of_peak": round(100 * bytes_per_launch * args.steps / elapsed / 1e9 / PEAK_GBPS, 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_GBPS, 4), "traffic": traffic,
                     "kernel_avg_us": round(avg_kernel_s * 1e6, 2),
                     "algorithmic_bytes_per_launch": bytes_per_launch},
    }
    log("copy probe")
    result["copy_probe_GBps"] = copy_probe(dw, torch)
    # the kernel's rate against what a plain one-read-one-write copy reaches here
    result["roofline"]["frac_of_copy"] = round(achieved / result["copy_probe_GBps"], 4)

    # output check on the oracle's sample, and the last element against a double sum
    y_host = y.cpu().numpy()
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        base, (ref, s) = cpu_baseline(x_host)
        result["cpu_baseline"] = base
        k = ref.shape[0]
        ok = bool(np.all(np.abs(y_host[:k] - ref) <= 1e-5 * s + 1e-6))
        result["parity_sample_ok"] = ok
    total = float(np.sum(x_host, dtype=np.float64))
    result["parity_last_ok"] = bool(abs(float(y_host[-1]) - total) <= 1e-5 * total + 1e-6)
    del x, y
    torch.cuda.empty_cache()
    if args.suite:
        suite(dw, torch, si, args.suite, max(10, args.steps // 2))
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
