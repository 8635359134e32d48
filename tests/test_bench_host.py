"""Host-side logic of bench.py on the CPU: the one-GPU guard and the rocprofv3 summaries."""
import csv
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
import seeded_inputs  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""  # no JSON line


def _write_counters(directory, counter, rows):
    os.makedirs(directory, exist_ok=True)
    with open(os.path.join(directory, "x_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (name, value) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_traffic_summary_scales_by_the_copy_probe(tmp_path, monkeypatch):
    """Counter values are scaled by what the counter reads for the 1 GiB copy probe, per dispatch."""
    out = tmp_path / "traffic.txt"
    monkeypatch.setattr(bench, "TRAFFIC_ALL_FILE", str(out))
    monkeypatch.setattr(seeded_inputs, "float32_normal", lambda seed, n: np.array([1.0, -1.0], np.float32))
    label, frag, n, alg = bench.WORKLOADS[0]
    kib = (1 << 30) / 1024
    # the copy probe's FETCH_SIZE reads twice the true bytes, WRITE_SIZE the true bytes
    _write_counters(tmp_path / "f", "FETCH_SIZE", [(bench.COPY_KERNEL + "(x)", 2 * kib),
                                                  (frag + ">(p)", 2 * 1.5 * kib), (frag + ">(p)", 2 * 0.5 * kib)])
    _write_counters(tmp_path / "w", "WRITE_SIZE", [(bench.COPY_KERNEL + "(x)", kib), (frag + ">(p)", kib)])
    bench.summarize_workload_traffic(str(tmp_path / "f"), str(tmp_path / "w"))
    text = out.read_text()
    assert "fetch_scale: 0.5000  write_scale: 1.0000" in text
    line = [l for l in text.splitlines() if l.startswith(label + " |")][0]
    rd, wr, total, a, ratio = [float(v) for v in line.split("|")[1:]]
    # mean read 1 GiB (two dispatches of 1.5 and 0.5 GiB), write 1 GiB
    assert abs(rd - (1 << 30) / 1e6) < 0.1 and abs(wr - (1 << 30) / 1e6) < 0.1
    assert abs(a - alg(n, 1) / 1e6) < 0.1
    assert abs(ratio - (2 * (1 << 30)) / alg(n, 1)) < 1e-3
    assert "counters missing" in text  # every other workload had no dispatches


def test_source_hash_is_stable_and_covers_the_kernels():
    h = bench.kernel_source_hash()
    assert h == bench.kernel_source_hash() and len(h) == 16


def _write_trace(directory, rows):
    os.makedirs(directory, exist_ok=True)
    with open(os.path.join(directory, "x_kernel_trace.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        t = 1000
        for name, dur_ns in rows:
            w.writerow({"Kernel_Name": name, "Start_Timestamp": t, "End_Timestamp": t + dur_ns})
            t += dur_ns + 500


def test_dispatch_summary_takes_the_last_25_scans_before_the_copy_probe(tmp_path, monkeypatch):
    out = tmp_path / "disp.txt"
    monkeypatch.setattr(bench, "DISPATCH_FILE", str(out))
    scan = "void dwpt::tile_scan_persistent<dwpt::OpAdd<float>, false, 1024, 16, 3>(dwpt::ScanParams)"
    # 60 settle launches at 400 us, 5 warm-up at 350, 20 timed at 300, then the copy probe
    # and a later scan launch that is not counted
    rows = [(scan, 400000)] * 60 + [(scan, 350000)] * 5 + [(scan, 300000)] * 20
    rows += [("(anonymous namespace)::copy_probe_kernel(x)", 1000), (scan, 1)]
    _write_trace(tmp_path / "a", rows)
    _write_trace(tmp_path / "b", rows[60:])
    bench.summarize_dispatches(str(tmp_path / "a"), str(tmp_path / "b"))
    text = out.read_text()
    a, b = text.split("## without settle")
    assert "settle_dispatches: 60" in a and "timed_mean_us: 300.00" in a
    assert "settle_dispatches: 0" in b and "timed_mean_us: 300.00" in b
    assert "warmup_us: 350.0 350.0 350.0 350.0 350.0" in b


def test_latency_summary_splits_cases_at_the_markers(tmp_path, monkeypatch):
    out = tmp_path / "lat.txt"
    monkeypatch.setattr(bench, "LATENCY_FILE", str(out))
    cases = [("case A", "add", True, 100, "int32_0_15", None, 0), ("case B", "max", False, 100, "int32_full", 0, 3)]
    monkeypatch.setattr(bench, "LATENCY_CASES", cases)
    mark = ("(anonymous namespace)::copy_probe_kernel(x)", 100)
    single = ("void dwpt::tile_scan_kernel<dwpt::OpAdd<int>, true, 1024, 16, true>(dwpt::ScanParams)", 3000)
    rts = [("void dwpt::tile_reduce_kernel<dwpt::OpMax<int>>(p)", 1000),
           ("void dwpt::carry_scan_kernel<dwpt::OpMax<int>>(p)", 2000),
           ("void dwpt::tile_scan_seeded_kernel<dwpt::OpMax<int>>(p)", 4000)]
    flush = ("void at::native::vectorized_elementwise_kernel<fill>(x)", 90000)
    rows = [single] * 3 + [mark] + [single] * 10 + [mark] + [flush, ("void dwpt::tile_scan_kernel<dwpt::OpAdd<int>, "
                                                                    "true, 1024, 16, true>(dwpt::ScanParams)", 5000)] * 4
    rows += [mark] + rts * 10 + [mark] + (([flush] + rts) * 3)
    _write_trace(tmp_path / "t", rows)
    jl = tmp_path / "lat.jsonl"
    jl.write_text('{"case": "case A", "median_us": 6.1, "back_to_back_us": 5.0, "cold_median_us": 7.0}\n')
    bench.summarize_latency(str(tmp_path / "t"), str(jl))
    lines = {l.split(" | ")[0]: l.split(" | ") for l in out.read_text().splitlines() if " | " in l}
    a, b = lines["case A"], lines["case B"]
    assert a[1] == "tile_scan_kernel" and float(a[2]) == 3.0 and float(a[4]) == 5.0 and a[5] == "6.1"
    assert b[1] == "tile_reduce_kernel + carry_scan_kernel + tile_scan_seeded_kernel"
    assert float(b[2]) == 7.0 and float(b[3]) == 8.0 and float(b[4]) == 7.0  # span: three kernels + two 0.5 us gaps
    assert b[5] == "-"
