"""scan_noalloc, the allocation-free plain scan, through the C ABI.

Its status words live in the library's static per-GPU array instead of a
per-stream workspace; the kernels are the same.  Checked against the
existing entry points (scan_inclusive / scan_exclusive) on the same inputs:
bit for bit for integer, max/min and affine scans, and both against the
oracle within 1e-5 * prefix|x| + 1e-6 for float add -- two calls in a row,
the second with a smaller input (the array keeps the first call's status
words, which must read as stale), on every kernel path.
"""
import ctypes

import numpy as np
import pytest
import torch

import device_wide_prefix_tile_amd as dw
import oracle
import seeded_inputs as si
from parity_helpers import assert_equal, assert_f32_close, from_dev, to_dev

pytestmark = pytest.mark.gpu

ADD, MAX, AFFINE, MAX_COUNT, MAT2, MAT3 = 0, 1, 3, 4, 5, 6
I32, U32, F32, U32X2, I32_U32, U32X4, U32X9 = 0, 1, 2, 3, 4, 5, 6


def noalloc(x, op, dt, exclusive):
    """One call of the C entry point on the current stream; returns the output tensor."""
    out = torch.empty_like(x)
    stream = torch.cuda.current_stream().cuda_stream
    st = dw.lib().scan_noalloc(op, dt, ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(out.data_ptr()),
                               x.shape[0], 1 if exclusive else 0, ctypes.c_void_p(stream))
    assert st == 0, dw.scan_status_string(st)
    return out


def existing(x, opname, exclusive):
    return (dw.scan_exclusive if exclusive else dw.scan_inclusive)(x, opname)


class Mode:
    def __init__(self, small, mode):
        self.small, self.mode = small, mode

    def __enter__(self):
        self.old_small = dw.scan_set_small_n_max(self.small)
        self.old_mode = dw.scan_set_multi_tile_mode(self.mode)

    def __exit__(self, *a):
        dw.scan_set_small_n_max(self.old_small)
        dw.scan_set_multi_tile_mode(self.old_mode)


# small-n bound and multi-tile mode: automatic, persistent forced, one tile per workgroup
# forced, single workgroup forced, and reduce-then-scan requested (not used without a buffer)
PATHS = {"auto": (dw.SCAN_SMALL_N_AUTO, 0), "multi": (0, 2), "fallback": (0, 1), "single": (1 << 40, 0), "rts": (0, 3)}


@pytest.mark.parametrize("path", list(PATHS))
def test_noalloc_matches_existing_entry_points(path):
    big, small = (1 << 24) + 999, 70001
    if path == "single":
        big, small = 200003, 5000
    with Mode(*PATHS[path]):
        for seed, n in ((1, big), (2, small)):  # two calls in a row, the second smaller
            print("noalloc path=%s n=%d" % (path, n), flush=True)
            x = si.int32_full(900 + seed, n)
            xd = to_dev(x)
            for op, opname in ((ADD, "add"), (MAX, "max")):
                for excl in (False, True):
                    y = from_dev(noalloc(xd, op, I32, excl))
                    assert_equal(y, from_dev(existing(xd, opname, excl)), "i32 %s excl=%s n=%d" % (opname, excl, n))
                    assert_equal(y, oracle.scan(opname, x, exclusive=excl), "i32 %s oracle n=%d" % (opname, n))
            f = si.float32_01(910 + seed, n)
            fd = to_dev(f)
            ref, s = oracle.scan("add", f)
            assert_f32_close(from_dev(noalloc(fd, ADD, F32, False)), ref, s, "f32 add noalloc n=%d" % n)
            assert_f32_close(from_dev(existing(fd, "add", False)), ref, s, "f32 add existing n=%d" % n)
            ab = si.affine_pairs(920 + seed, n // 2, odd_a=True)
            abd = to_dev(ab)
            y = from_dev(noalloc(abd, AFFINE, U32X2, False))
            assert_equal(y, from_dev(existing(abd, "affine", False)), "affine n=%d" % (n // 2))
            m = si.mat3_elems(930 + seed, n // 64)
            md = to_dev(m)
            y = from_dev(noalloc(md, MAT3, U32X9, True))
            assert_equal(y, from_dev(existing(md, "mat3", True)), "mat3 n=%d" % (n // 64))
            # the 512-thread classes: (maximum, count) pairs and 2x2 matrices
            vc = si.maxcount_pairs(950 + seed, n // 4, span=20, unit_counts=False)
            vd = to_dev(vc)
            y = from_dev(noalloc(vd, MAX_COUNT, I32_U32, False))
            assert_equal(y, from_dev(existing(vd, "maxcount", False)), "maxcount n=%d" % (n // 4))
            m2 = si.mat2_elems(960 + seed, n // 16)
            m2d = to_dev(m2)
            y = from_dev(noalloc(m2d, MAT2, U32X4, True))
            assert_equal(y, from_dev(existing(m2d, "mat2", True)), "mat2 n=%d" % (n // 16))
    assert dw.scan_get_device_error() == 0


def test_noalloc_in_place_and_binding():
    n = 3 * 15360 + 77
    x = si.int32_0_15(940, n)
    t = to_dev(x)
    dw.scan_noalloc(t, "add", exclusive=True, out=t)
    assert_equal(from_dev(t), oracle.scan("add", x, exclusive=True), "in place")
    assert dw.scan_get_device_error() == 0
