"""The C-ABI library loads and exports what include/*.h declares; host-side checks (no GPU).

Nothing here launches a kernel: only calls that are rejected (or are no-ops)
before the library touches the HIP runtime are made.
"""
import ctypes
import glob
import os
import re

import pytest

from device_wide_prefix_tile_amd import binding
from device_wide_prefix_tile_amd import build as dbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h, encoding="utf-8").read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^\s*[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M):
            if m.group(1) not in ("if", "while", "for", "return", "sizeof"):
                names.add(m.group(1))
    return names


def test_header_declares_the_scan_calls():
    names = declared_functions()
    for n in ("scan_inclusive", "scan_exclusive", "segmented_scan", "compact"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = binding.lib()
    names = declared_functions()
    assert names
    for n in sorted(names):
        assert hasattr(L, n), n
    assert set(binding.EXPORTS) == names


def test_library_is_built_for_gfx950():
    blob = open(dbuild.LIB_PATH, "rb").read()
    assert b"gfx950" in blob


def test_status_strings():
    for s in range(6):
        assert binding.status_string(s)
    assert binding.status_string(99) == "unknown status"


def test_argument_checks_before_any_launch():
    L = binding.lib()
    ADD, MAX, AFF = 0, 1, 3
    I32, U32, F32, PAIR = 0, 1, 2, 3
    # n == 0 is a no-op
    assert L.scan_inclusive(ADD, F32, None, None, 0, None) == 0
    assert L.scan_exclusive(MAX, I32, None, None, 0, None) == 0
    assert L.segmented_scan(ADD, I32, None, None, None, 0, 0, None) == 0
    # unsupported combinations
    assert L.scan_inclusive(AFF, F32, 1024, 2048, 10, None) == binding.SCAN_ERR_UNSUPPORTED
    assert L.scan_inclusive(ADD, PAIR, 1024, 2048, 10, None) == binding.SCAN_ERR_UNSUPPORTED
    assert L.scan_inclusive(9, I32, 1024, 2048, 10, None) == binding.SCAN_ERR_UNSUPPORTED
    assert L.segmented_scan(AFF, PAIR, 1024, 4096, 2048, 10, 0, None) == binding.SCAN_ERR_UNSUPPORTED
    assert L.compact(PAIR, 1024, 2048, 4096, 10, None) == binding.SCAN_ERR_UNSUPPORTED
    MC, MAT2, MCPAIR, MAT = 4, 5, 4, 5
    assert L.scan_inclusive(MC, I32, 1024, 2048, 10, None) == binding.SCAN_ERR_UNSUPPORTED
    assert L.scan_inclusive(MC, PAIR, 1024, 2048, 10, None) == binding.SCAN_ERR_UNSUPPORTED
    assert L.scan_inclusive(MAT2, PAIR, 1024, 2048, 10, None) == binding.SCAN_ERR_UNSUPPORTED
    assert L.scan_exclusive(ADD, MAT, 1024, 2048, 10, None) == binding.SCAN_ERR_UNSUPPORTED
    assert L.scan_inclusive(MAX, MCPAIR, 1024, 2048, 10, None) == binding.SCAN_ERR_UNSUPPORTED
    assert L.scan_inclusive(6, MAT, 1024, 2048, 10, None) == binding.SCAN_ERR_UNSUPPORTED
    assert L.scan_inclusive(MAT2, 6, 1024, 2048, 10, None) == binding.SCAN_ERR_UNSUPPORTED
    assert L.segmented_scan(MC, MCPAIR, 1024, 4096, 2048, 10, 0, None) == binding.SCAN_ERR_UNSUPPORTED
    MAT3, MAT9 = 6, 6
    AND, OR = 7, 8
    assert L.scan_inclusive(AND, F32, 1024, 2048, 10, None) == binding.SCAN_ERR_UNSUPPORTED
    assert L.scan_exclusive(OR, F32, 1024, 2048, 10, None) == binding.SCAN_ERR_UNSUPPORTED
    assert L.scan_inclusive(AND, PAIR, 1024, 2048, 10, None) == binding.SCAN_ERR_UNSUPPORTED
    assert L.scan_inclusive(9, U32, 1024, 2048, 10, None) == binding.SCAN_ERR_UNSUPPORTED
    assert L.segmented_scan(OR, U32, 1024, 4096, 2048, 10, 0, None) == binding.SCAN_ERR_UNSUPPORTED
    assert L.scan_inclusive(AND, U32, 1026, 2048, 10, None) == binding.SCAN_ERR_INVALID
    assert L.scan_inclusive(MAT3, MAT, 1024, 2048, 10, None) == binding.SCAN_ERR_UNSUPPORTED
    assert L.scan_inclusive(MAT2, MAT9, 1024, 2048, 10, None) == binding.SCAN_ERR_UNSUPPORTED
    assert L.scan_inclusive(ADD, MAT9, 1024, 2048, 10, None) == binding.SCAN_ERR_UNSUPPORTED
    assert L.scan_inclusive(7, MAT9, 1024, 2048, 10, None) == binding.SCAN_ERR_UNSUPPORTED
    assert L.scan_inclusive(MAT3, 7, 1024, 2048, 10, None) == binding.SCAN_ERR_UNSUPPORTED
    assert L.segmented_scan(MAT3, MAT9, 1024, 4096, 2048, 10, 0, None) == binding.SCAN_ERR_UNSUPPORTED
    # 3x3 matrices are arrays of uint32: 4-byte alignment suffices, 2 does not;
    # partial overlap is measured in 36-byte elements
    assert L.scan_inclusive(MAT3, MAT9, 1026, 8192, 10, None) == binding.SCAN_ERR_INVALID
    assert L.scan_inclusive(MAT3, MAT9, 1024, 8194, 10, None) == binding.SCAN_ERR_INVALID
    assert L.scan_inclusive(MAT3, MAT9, 1024, 1024 + 36 * 9, 10, None) == binding.SCAN_ERR_INVALID
    # a 2x2 matrix is one 16-byte vector: 16-byte alignment; a pair needs 8
    assert L.scan_inclusive(MAT2, MAT, 1032, 8192, 10, None) == binding.SCAN_ERR_INVALID
    assert L.scan_inclusive(MAT2, MAT, 1024, 8200, 10, None) == binding.SCAN_ERR_INVALID
    assert L.scan_inclusive(MC, MCPAIR, 1028, 8192, 10, None) == binding.SCAN_ERR_INVALID
    # in-place is allowed, partial overlap is not (n matrices of 16 bytes)
    assert L.scan_inclusive(MAT2, MAT, 1024, 1024 + 16 * 5, 10, None) == binding.SCAN_ERR_INVALID
    # invalid pointers, alignment and overlap
    assert L.scan_inclusive(ADD, I32, None, 2048, 10, None) == binding.SCAN_ERR_INVALID
    assert L.scan_inclusive(ADD, I32, 1025, 4096, 10, None) == binding.SCAN_ERR_INVALID
    assert L.scan_inclusive(AFF, PAIR, 1028, 8192, 10, None) == binding.SCAN_ERR_INVALID
    assert L.scan_inclusive(ADD, I32, 1024, 1028, 10, None) == binding.SCAN_ERR_INVALID
    assert L.segmented_scan(ADD, I32, 1024, None, 8192, 10, 0, None) == binding.SCAN_ERR_INVALID
    assert L.segmented_scan(ADD, I32, 1024, 8192, 8192, 10, 0, None) == binding.SCAN_ERR_INVALID
    assert L.compact(F32, 1024, 8192, None, 10, None) == binding.SCAN_ERR_INVALID
    assert L.compact(F32, 1024, 8192, 1 << 20, 1 << 32, None) == binding.SCAN_ERR_INVALID
    # the count may not overlap the input (nor the output): reduce-then-scan writes it
    # before its last pass reads the input again
    assert L.compact(F32, 1024, 8192, 1024 + 8, 10, None) == binding.SCAN_ERR_INVALID
    assert L.compact(F32, 1024, 8192, 1024, 10, None) == binding.SCAN_ERR_INVALID
    assert L.compact(F32, 1024, 8192, 8192 + 36, 10, None) == binding.SCAN_ERR_INVALID
    assert L.scan_copy_probe(1024, 2048, 10, None) == binding.SCAN_ERR_INVALID
    # the allocation-free scan: same checks, and inputs whose status words do not fit its
    # 16 MiB static array are rejected before anything is launched (fake, never-touched
    # addresses); float32 and int32 add have 1 status word per 15360-element tile, affine 2
    # per 7680 pairs
    NOALLOC_F32_MAX, NOALLOC_I32_MAX = 123357 * 15360, 123357 * 15360
    assert L.scan_noalloc(ADD, F32, None, None, 0, 0, None) == 0
    assert L.scan_noalloc(AFF, F32, 1024, 2048, 10, 0, None) == binding.SCAN_ERR_UNSUPPORTED
    assert L.scan_noalloc(ADD, I32, None, 2048, 10, 1, None) == binding.SCAN_ERR_INVALID
    assert L.scan_noalloc(ADD, I32, 1024, 1028, 10, 1, None) == binding.SCAN_ERR_INVALID
    assert L.scan_noalloc(ADD, F32, 1 << 20, 1 << 40, NOALLOC_F32_MAX + 1, 0, None) == binding.SCAN_ERR_INVALID
    assert L.scan_noalloc(ADD, I32, 1 << 20, 1 << 40, NOALLOC_I32_MAX + 1, 1, None) == binding.SCAN_ERR_INVALID
    assert L.scan_noalloc(6, 6, 1 << 20, 1 << 40, 13706 * 3584 + 1, 0, None) == binding.SCAN_ERR_INVALID
    assert L.scan_noalloc(AFF, PAIR, 1 << 20, 1 << 40, 61678 * 7680 + 1, 0, None) == binding.SCAN_ERR_INVALID
    # CSR row offsets: row_ptr required and aligned, indices required when nnz > 0,
    # no overlap at all, nnz below 2^32
    assert L.csr_row_offsets(1024, 10, 5, None, None) == binding.SCAN_ERR_INVALID
    assert L.csr_row_offsets(1024, 10, 5, 8194, None) == binding.SCAN_ERR_INVALID
    assert L.csr_row_offsets(None, 10, 5, 8192, None) == binding.SCAN_ERR_INVALID
    assert L.csr_row_offsets(1026, 10, 5, 8192, None) == binding.SCAN_ERR_INVALID
    assert L.csr_row_offsets(1024, 10, 5, 1024, None) == binding.SCAN_ERR_INVALID
    assert L.csr_row_offsets(1024, 10, 5, 1024 + 36, None) == binding.SCAN_ERR_INVALID
    assert L.csr_row_offsets(1024, 1 << 32, 5, 1 << 40, None) == binding.SCAN_ERR_INVALID


def test_radix_split_argument_checks():
    """Rejected on the host, before any device work (fake addresses are never touched)."""
    L = binding.lib()
    ok, bad = binding.SCAN_OK, binding.SCAN_ERR_INVALID
    assert L.radix_split(None, None, 0, 0, None, None, None) == ok  # nothing to do
    assert L.radix_split(1024, None, 10, 32, 1 << 20, None, None) == bad  # shift > 31
    assert L.radix_split(1024, 4096, 10, 0, 1 << 20, None, None) == bad  # vals without vals_out
    assert L.radix_split(1024, 4096, 0, 0, 1 << 20, None, None) == ok  # n == 0: nothing is read
    assert L.radix_split(1024, None, 10, 0, 1 << 20, 4096, None) == bad  # vals_out without vals
    assert L.radix_split(None, None, 10, 0, 1 << 20, None, None) == bad
    assert L.radix_split(1024, None, 10, 0, None, None, None) == bad
    assert L.radix_split(1026, None, 10, 0, 1 << 20, None, None) == bad  # misaligned
    assert L.radix_split(1024, 1 << 16, 10, 0, 1 << 20, (1 << 24) + 2, None) == bad
    assert L.radix_split(1024, None, 1 << 32, 0, 1 << 40, None, None) == bad  # n >= 2^32
    assert L.radix_split(1024, None, 10, 0, 1024, None, None) == bad  # in place
    assert L.radix_split(1024, None, 10, 0, 1024 + 36, None, None) == bad  # partial overlap
    assert L.radix_split(1024, 1 << 16, 10, 0, 1 << 20, 1 << 16, None) == bad  # vals_out is vals
    assert L.radix_split(1024, 1 << 16, 10, 0, 1 << 20, 1024 + 8, None) == bad  # vals_out over keys
    assert L.radix_split(1024, 1 << 16, 10, 0, 1 << 20, (1 << 20) + 4, None) == bad  # outputs overlap


def test_tuning_knobs_round_trip():
    old = binding.scan_set_small_n_max(12345)
    assert binding.scan_set_small_n_max(binding.SCAN_SMALL_N_AUTO) == 12345
    assert binding.scan_set_small_n_max(old) == binding.SCAN_SMALL_N_AUTO
    old = binding.scan_set_spin_limit(77)
    assert binding.scan_set_spin_limit(old) == 77
    old = binding.scan_set_multi_tile_mode(2)
    assert binding.scan_set_multi_tile_mode(3) == 2
    assert binding.scan_set_multi_tile_mode(1) == 3
    assert binding.scan_set_multi_tile_mode(7) == 1
    assert binding.scan_set_multi_tile_mode(old) == 0
