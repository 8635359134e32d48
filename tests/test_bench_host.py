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
