"""CSR row offsets from COO row indices on the GPU against the oracle.

row_ptr[r] = number of entries with row index < r (r = 0 .. n_rows): the
counts of every row followed by their exclusive scan.  Building the CSR
format is among the uses of a prefix sum listed in the introduction of
"CUDA编程并行前缀和扫描详解"; row_ptr has N + 1 entries ("UIUC ECE 408
应用并行编程", L09).  Results are integers: compared bit for bit.
"""
import numpy as np
import pytest
import torch

import device_wide_prefix_tile_amd as dw
import oracle
import seeded_inputs as si
from parity_helpers import assert_equal, from_dev, to_dev

pytestmark = pytest.mark.gpu


def sorted_rows(seed, nnz, n_rows):
    return np.sort(si.uint32_full(seed, nnz) % n_rows).astype(np.uint32)


def check(rows, n_rows, what):
    ref = oracle.csr_offsets(rows, n_rows)
    rd = to_dev(rows) if rows.size else torch.empty(0, dtype=torch.uint32, device="cuda")
    got = from_dev(dw.csr_row_offsets(rd, n_rows))
    assert_equal(got, ref, what)


@pytest.mark.parametrize("n_rows,nnz", [(1, 1), (7, 100), (1000, 8000), (4096, 4097), (100000, 800000),
                                        (1 << 20, 1 << 23)])
def test_sorted(n_rows, nnz):
    check(sorted_rows(800 + nnz % 97, nnz, n_rows), n_rows, "sorted n_rows=%d nnz=%d" % (n_rows, nnz))


@pytest.mark.parametrize("n_rows,nnz", [(3, 1000), (1000, 8000), (100000, 800000)])
def test_unsorted(n_rows, nnz):
    rows = (si.uint32_full(900 + n_rows % 89, nnz) % n_rows).astype(np.uint32)
    check(rows, n_rows, "unsorted n_rows=%d nnz=%d" % (n_rows, nnz))


@pytest.mark.parametrize("n_rows", [1, 2, 16, 256, 1023, 1024, 4096, 16383, 16384, 16385])
def test_few_bins(n_rows):
    """Histogram offsets of few bins (up to 1023 bins every index is counted in LDS, up
    to 16384 runs are, each workgroup with its own counts): uniform bin indices, sorted
    ones, and a skewed mix with most entries in one bin."""
    nnz = (1 << 22) + 77
    rows = (si.uint32_full(950 + n_rows % 83, nnz) % n_rows).astype(np.uint32)
    check(rows, n_rows, "uniform bins n_rows=%d" % n_rows)
    check(np.sort(rows), n_rows, "sorted bins n_rows=%d" % n_rows)
    skew = np.where(si.uint32_full(960, nnz) % 10 == 0, rows, np.uint32(n_rows - 1)).astype(np.uint32)
    check(skew, n_rows, "skewed bins n_rows=%d" % n_rows)


@pytest.mark.parametrize("nnz", [1, 2, 3, 4, 5, 4099, 1 << 20])
def test_few_bins_tails_and_alignment(nnz):
    """Counts of few bins from 16-byte loads: index counts that are not a multiple of
    four, and indices that start 4, 8 or 12 bytes past a 16-byte boundary (read one
    index at a time instead); indices past the last bin are not counted."""
    rows = (si.uint32_full(970 + nnz % 61, nnz + 3) % 300).astype(np.uint32)
    ref_all = {}
    dev = to_dev(rows)
    for off in range(4):
        part = rows[off:off + nnz]
        ref_all[off] = oracle.csr_offsets(part, 257)
        got = from_dev(dw.csr_row_offsets(dev[off:off + nnz], 257))
        assert_equal(got, ref_all[off], "nnz=%d starting %d bytes in" % (nnz, 4 * off))


def test_few_bins_full_size():
    """2^27 uniform indices over 256 bins, the benchmarked histogram."""
    nnz = 1 << 27
    rows = (si.uint32_full(11, nnz) % 256).astype(np.uint32)
    check(rows, 256, "2^27 entries over 256 bins")


def test_edge_cases():
    check(np.zeros(0, np.uint32), 5, "no entries")
    check(np.zeros(0, np.uint32), 0, "no rows, no entries")
    check(np.array([0, 1, 2], np.uint32), 0, "no rows")
    check(np.full(100000, 17, np.uint32), 50, "one row")
    rows = si.uint32_full(31, 50000)  # mostly past the last row: not counted
    check(rows, 1000, "indices past the last row")
    rows = np.arange(70000, dtype=np.uint32)[::-1].copy()  # strictly decreasing
    check(rows, 70000, "decreasing")
    check(np.repeat(np.arange(4000, dtype=np.uint32), 3)[:-1], 4000, "runs across window boundaries")


def test_repeated_calls_and_streams():
    rows = sorted_rows(77, 300000, 20000)
    ref = oracle.csr_offsets(rows, 20000)
    rd = to_dev(rows)
    side = torch.cuda.Stream()
    for k in range(6):
        with torch.cuda.stream(side if k % 2 else torch.cuda.current_stream()):
            out = dw.csr_row_offsets(rd, 20000)
        torch.cuda.synchronize()
        assert_equal(from_dev(out), ref, "call %d" % k)
