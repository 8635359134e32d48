"""Reader for the worked examples under tests/golden/ (one cited example per file)."""
import glob
import os

import numpy as np

GOLDEN_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
_DTYPES = {"int32": np.int32, "uint32": np.uint32, "float32": np.float32}


def load(path):
    rec = {"path": path, "source": []}
    with open(path, encoding="utf-8") as f:
        for line in f:
            line = line.rstrip("\n")
            if not line.strip():
                continue
            if line.startswith("#"):
                rec["source"].append(line[1:].strip())
                continue
            key, _, val = line.partition(":")
            rec[key.strip()] = val.strip()
    dt = _DTYPES[rec["dtype"]]
    for key in ("input", "inclusive", "exclusive", "flags", "positions", "output"):
        if key in rec:
            rec[key] = np.array([float(v) if dt == np.float32 else int(v) for v in rec[key].split()],
                                dtype=dt if key not in ("flags", "positions") else np.uint32)
    rec["dtype"] = dt
    return rec


def all_examples(kind=None):
    recs = [load(p) for p in sorted(glob.glob(os.path.join(GOLDEN_DIR, "*.txt")))]
    return [r for r in recs if kind is None or r["kind"] == kind]
