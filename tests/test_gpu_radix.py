"""One radix-sort pass (a stable split by an 8-bit digit) on the GPU against the oracle.

Radix sort is a split by digit plus a scan that places every element; 32-bit
keys take four 8-bit passes ("Lecture 7: 并行模式五 —— 前缀和 / 扫描", concept 2;
PMPP chapter 9 notes, §9.6).  The result of a stable split is unique, so keys
and values are compared bit for bit.  Tiles hold 8192 keys.
"""
import numpy as np
import pytest
import torch

import device_wide_prefix_tile_amd as dw
import oracle
import seeded_inputs as si
from parity_helpers import assert_equal, from_dev, to_dev

pytestmark = pytest.mark.gpu

TILE = 8192
SIZES = [1, 2, 63, 64, 65, 1000, TILE - 1, TILE, TILE + 1, 3 * TILE + 77, 100003, (1 << 20) + 13]


def check(keys, shift, vals=None, what=""):
    print("radix_split n=%d shift=%d vals=%s %s" % (keys.size, shift, vals is not None, what), flush=True)
    ko_ref, vo_ref = oracle.radix_split(keys, shift, vals)
    kd = to_dev(keys)
    vd = to_dev(vals) if vals is not None else None
    ko, vo = dw.radix_split(kd, shift, vd)
    assert_equal(from_dev(ko), ko_ref, "keys n=%d shift=%d %s" % (keys.size, shift, what))
    if vals is not None:
        assert_equal(from_dev(vo), vo_ref, "vals n=%d shift=%d %s" % (keys.size, shift, what))


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("shift", [0, 8, 16, 24])
def test_uniform_keys(n, shift):
    check(si.uint32_full(1000 + n % 1009, n), shift, what="uniform")


@pytest.mark.parametrize("n", [1, 65, TILE + 1, 3 * TILE + 77, (1 << 20) + 13])
@pytest.mark.parametrize("shift", [0, 24])
def test_pairs(n, shift):
    keys = si.uint32_full(2000 + n % 1013, n)
    vals = np.arange(n, dtype=np.uint32)  # values record the input position: the permutation is checked
    check(keys, shift, vals, "pairs")


@pytest.mark.parametrize("shift", [3, 13, 25, 31])
def test_unaligned_digits(shift):
    """Digits that straddle byte boundaries, and the short top digits (shift > 24)."""
    n = 5 * TILE + 999
    check(si.uint32_full(3000 + shift, n), shift, si.uint32_full(3100 + shift, n), "unaligned digit")


def test_skewed_digits():
    n = 7 * TILE + 4321
    check(np.full(n, 0xABCDEF12, np.uint32), 8, np.arange(n, dtype=np.uint32), "all keys equal")
    keys = si.uint32_full(41, n) & np.uint32(0x00000300)  # four digit values, bit-sparse
    check(keys, 8, np.arange(n, dtype=np.uint32), "four digits")
    keys = np.where(si.uint32_full(42, n) % 100 == 0, np.uint32(255), np.uint32(0)).astype(np.uint32)
    check(keys, 0, np.arange(n, dtype=np.uint32), "two digits, 1% high")
    check(np.arange(n, dtype=np.uint32), 0, what="ascending")
    check(np.arange(n, dtype=np.uint32)[::-1].copy(), 0, what="descending")
    check(np.arange(n, dtype=np.uint32)[::-1].copy() << np.uint32(24), 24, what="descending top digit")


def test_unaligned_keys():
    """Keys 4 bytes off 16-byte alignment (element loads in every kernel), with values."""
    n = 6 * TILE + 321
    keys, vals = si.uint32_full(45, n + 1), si.uint32_full(46, n + 1)
    ref_k, ref_v = oracle.radix_split(keys[1:], 16, vals[1:])
    kd, vd = to_dev(keys)[1:], to_dev(vals)[1:]
    assert kd.data_ptr() % 16 == 4
    ko, vo = dw.radix_split(kd, 16, vd)
    assert_equal(from_dev(ko), ref_k, "unaligned keys")
    assert_equal(from_dev(vo), ref_v, "unaligned values")


def test_four_passes_sort():
    """Four passes with shift = 0, 8, 16, 24 sort the keys, values following (stable)."""
    n = 3 * TILE * 7 + 5
    keys = si.uint32_full(55, n)
    keys[::11] = keys[7]  # equal keys: their values must stay in input order
    k, v = to_dev(keys), torch.arange(n, dtype=torch.int32, device="cuda").view(torch.uint32)
    for shift in (0, 8, 16, 24):
        k, v = dw.radix_split(k, shift, v)
    assert_equal(from_dev(k), np.sort(keys), "sorted keys")
    assert_equal(from_dev(v), np.argsort(keys, kind="stable").astype(np.uint32), "stable permutation")


def test_interleaved_with_scans_on_one_stream():
    """The histogram buffer, the scan workspace and the look-back status array
    serve alternating calls on one stream without interfering."""
    n = 40 * TILE + 3
    keys = si.uint32_full(61, n)
    x = si.int32_0_15(62, 3 << 20)
    xd = to_dev(x)
    ref_k, _ = oracle.radix_split(keys, 16)
    ref_s = oracle.scan("add", x)
    kd = to_dev(keys)
    for rep in range(3):
        ko, _ = dw.radix_split(kd, 16)
        y = dw.scan_inclusive(xd, "add")
        assert_equal(from_dev(ko), ref_k, "radix rep %d" % rep)
        assert_equal(from_dev(y), ref_s, "scan rep %d" % rep)
    small = si.uint32_full(63, 777)
    ko, _ = dw.radix_split(to_dev(small), 0)  # smaller after larger: histogram buffer reused
    assert_equal(from_dev(ko), oracle.radix_split(small, 0)[0], "small after large")


def test_given_outputs_and_side_stream():
    n = 9 * TILE + 1
    keys, vals = si.uint32_full(71, n), si.uint32_full(72, n)
    ref_k, ref_v = oracle.radix_split(keys, 8, vals)
    kd, vd = to_dev(keys), to_dev(vals)
    ko = torch.full((n,), 7, dtype=torch.int32, device="cuda")
    vo = torch.full((n,), 7, dtype=torch.int32, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        dw.radix_split(kd, 8, vd, keys_out=ko, vals_out=vo, stream=side)
    side.synchronize()
    assert_equal(ko.cpu().numpy().view(np.uint32), ref_k, "keys on a side stream")
    assert_equal(vo.cpu().numpy().view(np.uint32), ref_v, "vals on a side stream")


def test_binding_rejects_bad_arguments():
    kd = torch.zeros(100, dtype=torch.uint32, device="cuda")
    with pytest.raises(ValueError):
        dw.radix_split(kd, 32)
    with pytest.raises(dw.ScanError):
        dw.radix_split(kd, 0, keys_out=kd)  # in place: rejected by the library
    with pytest.raises(ValueError):
        dw.radix_split(kd, 0, vals_out=torch.zeros_like(kd))
    with pytest.raises(TypeError):
        dw.radix_split(torch.zeros(100, dtype=torch.float32, device="cuda"), 0)
    e = torch.empty(0, dtype=torch.uint32, device="cuda")
    ko, vo = dw.radix_split(e, 0, e.clone())
    assert ko.numel() == 0 and vo.numel() == 0


@pytest.mark.parametrize("with_vals", [False, True])
def test_full_size(with_vals):
    """The benchmarked size: 2^28 keys (2^27 key-value pairs), compared whole."""
    n = 1 << (27 if with_vals else 28)
    keys = si.uint32_full(81 + with_vals, n)
    vals = si.uint32_full(83, n) if with_vals else None
    check(keys, 8, vals, "full size")
