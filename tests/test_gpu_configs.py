"""The five scan workloads at full size, in the launch configuration the benchmark times.

Every output element is compared with the oracle (the C oracle finishes even
2^30 elements in seconds):
  1. int32 exclusive add, n = 2^20, values in [0, 15], plus the 8-element
     worked example of the pages;
  2. float32 inclusive add, n = 2^28, values in [0, 1), within
     1e-5 * prefix|x| + 1e-6 of the double-accumulated oracle;
  3. compaction of float32 N(0,1), n = 2^28, keep x > 0: count and contents
     bit-exact;
  4. uint32 affine-map composition, n = 2^26 pairs, inclusive, bit-exact
     (and the odd-multiplier variant, where no prefix collapses to zero);
  5. segmented int32 inclusive add, n = 2^27, values in [-100, 100], heads with
     geometric segment lengths of mean 1000; and an int32 max-scan over
     n = 2^10 .. 2^30 (powers of 4).
"""
import numpy as np
import pytest
import torch

import device_wide_prefix_tile_amd as dw
import oracle
import seeded_inputs as si
from parity_helpers import assert_equal, assert_f32_close, from_dev, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def fresh():
    yield
    torch.cuda.empty_cache()


class Mode:
    """Force a multi-tile kernel: 1 one workgroup per tile, 2 persistent, 3 reduce-then-scan; 0 by size."""

    def __init__(self, mode):
        self.mode = mode

    def __enter__(self):
        self.old = dw.scan_set_multi_tile_mode(self.mode)

    def __exit__(self, *a):
        dw.scan_set_multi_tile_mode(self.old)


def test_config1_int32_exclusive_add_2p20():
    n = 1 << 20
    x = si.int32_0_15(1, n)
    xd = to_dev(x)
    ref = oracle.scan("add", x, exclusive=True)
    for mode in (0, 1, 2, 3):
        with Mode(mode):
            y = from_dev(dw.scan_exclusive(xd, "add"))
        assert_equal(y, ref, "config1 mode=%d" % mode)
    ex = np.array([3, 1, 7, 0, 4, 1, 6, 3], np.int32)
    np.testing.assert_array_equal(from_dev(dw.scan_exclusive(to_dev(ex), "add")), [0, 3, 4, 11, 11, 15, 16, 22])
    np.testing.assert_array_equal(from_dev(dw.scan_inclusive(to_dev(ex), "add")), [3, 4, 11, 11, 15, 16, 22, 25])


def test_config2_f32_inclusive_add_2p28():
    n = 1 << 28
    x = si.float32_01(2, n)
    xd = to_dev(x)
    ys = {}
    for mode in (0, 3):  # the benchmarked kernel, and reduce-then-scan
        with Mode(mode):
            ys[mode] = from_dev(dw.scan_inclusive(xd, "add"))
    del xd
    ref, s = oracle.scan("add", x)
    for mode, y in ys.items():
        worst = assert_f32_close(y, ref, s, "config2 mode=%d" % mode)
        print("config2 mode=%d worst error/tolerance = %.4f" % (mode, worst))
    assert dw.scan_get_device_error() == 0


def test_f32_add_mixed_signs_2p28():
    """float32 add over values uniform in [-1, 1) and over N(0, 1): the running sums cancel,
    so the tolerance, scaled by the prefix of |x|, is far above the value itself; exclusive too."""
    n = 1 << 28
    for name, x in (("uniform[-1,1)", si.float32_sym(7, n)), ("normal", si.float32_normal(3, n))):
        xd = to_dev(x)
        yi = from_dev(dw.scan_inclusive(xd, "add"))
        ye = from_dev(dw.scan_exclusive(xd, "add"))
        del xd
        ref, s = oracle.scan("add", x)
        worst = assert_f32_close(yi, ref, s, "mixed signs inclusive " + name)
        print("%s inclusive worst error/tolerance = %.4f" % (name, worst))
        del ref
        ref_e, s_e = oracle.scan("add", x, exclusive=True)
        assert_f32_close(ye, ref_e, s_e, "mixed signs exclusive " + name)
        del yi, ye, ref_e, s_e, x
    assert dw.scan_get_device_error() == 0


def test_config3_compact_2p28():
    n = 1 << 28
    x = si.float32_normal(3, n)
    xd = to_dev(x)
    ref, rc, _ = oracle.compact(x)
    for mode in (0, 3):
        with Mode(mode):
            out, cnt = dw.compact(xd)
        out, cnt = from_dev(out), int(from_dev(cnt)[0])
        assert cnt == rc, "config3 mode=%d" % mode
        assert_equal(out[:cnt], ref, "config3 mode=%d" % mode)


@pytest.mark.parametrize("odd", [False, True], ids=["any_a", "odd_a"])
def test_config4_affine_2p26(odd):
    n = 1 << 26
    ab = si.affine_pairs(40 if odd else 4, n, odd_a=odd)
    abd = to_dev(ab)
    ref = oracle.scan_affine(ab)
    for mode in (0, 3):
        with Mode(mode):
            y = from_dev(dw.scan_inclusive(abd, "affine"))
        assert_equal(y, ref, "config4 odd=%s mode=%d" % (odd, mode))


def test_config5_segmented_add_2p27():
    n = 1 << 27
    x = si.int32_pm100(5, n)
    h = si.segment_heads(5, n, 1000.0)
    xd, hd = to_dev(x), to_dev(h)
    ref = oracle.segmented_scan("add", x, h)
    for mode in (0, 3):
        with Mode(mode):
            y = from_dev(dw.segmented_scan(xd, hd, "add"))
        assert_equal(y, ref, "config5 segmented mode=%d" % mode)


@pytest.mark.parametrize("k", range(5, 16))
def test_config5_max_sweep(k):
    n = 4 ** k
    x = si.int32_full(6, n)
    xd = to_dev(x)
    ref = oracle.scan("max", x)
    # the size-selected kernel, and below 2^30 every multi-tile path forced
    for mode in (0, 1, 2, 3) if k < 15 else (0,):
        with Mode(mode):
            y = from_dev(dw.scan_inclusive(xd, "max"))
        assert_equal(y, ref, "config5 max sweep n=4^%d mode=%d" % (k, mode))
