"""Shared helpers of the GPU parity tests: device transfer and the float32 tolerance check."""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

# |y_gpu - y_ref| <= REL * sum_{k<=i} |x_k| + ABS, with y_ref accumulated in double
REL, ABS = 1e-5, 1e-6
_CHUNK = 1 << 22
_THREADS = max(1, min(16, os.cpu_count() or 1))


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def from_dev(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


def f32_error_ratio(y_gpu: np.ndarray, y_ref: np.ndarray, s: np.ndarray):
    """Largest |y_gpu - y_ref| / (REL*s + ABS) and where it occurs (threaded, chunked)."""
    n = y_gpu.shape[0]
    spans = [(c, min(n, c + _CHUNK)) for c in range(0, n, _CHUNK)]

    def work(span):
        c0, c1 = span
        r = np.abs(y_gpu[c0:c1].astype(np.float64) - y_ref[c0:c1]) / (REL * s[c0:c1] + ABS)
        if r.size == 0:
            return 0.0, 0
        k = int(np.argmax(r))
        return float(r[k]), c0 + k

    if not spans:
        return 0.0, 0
    with ThreadPoolExecutor(_THREADS) as ex:
        res = list(ex.map(work, spans))
    return max(res)


def assert_f32_close(y_gpu, y_ref, s, what=""):
    worst, at = f32_error_ratio(y_gpu, y_ref, s)
    assert worst <= 1.0, "%s: error/tolerance %.3f at index %d (gpu %r, ref %r, s %r)" % (
        what, worst, at, float(y_gpu[at]), float(y_ref[at]), float(s[at]))
    return worst


def assert_equal(y_gpu, y_ref, what=""):
    if not np.array_equal(y_gpu.view(np.uint8), np.ascontiguousarray(y_ref).view(np.uint8)):
        a = y_gpu.reshape(y_gpu.shape[0], -1).view(np.uint32) if y_gpu.dtype.itemsize >= 4 else y_gpu
        b = np.ascontiguousarray(y_ref).reshape(y_gpu.shape[0], -1).view(np.uint32) \
            if y_gpu.dtype.itemsize >= 4 else y_ref
        bad = np.flatnonzero(np.any(a.reshape(a.shape[0], -1) != b.reshape(b.shape[0], -1), axis=1))
        i = int(bad[0])
        raise AssertionError("%s: %d mismatches, first at %d: gpu %r ref %r" % (
            what, bad.size, i, y_gpu[i], y_ref[i]))
