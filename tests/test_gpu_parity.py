"""GPU parity: the HIP library against the sequential oracle, element by element.

Integer, max/min, affine and compaction results must be bit-exact; float32
add results must satisfy |y_gpu - y_ref| <= 1e-5 * sum_{k<=i}|x_k| + 1e-6 with
y_ref accumulated in double.  Sizes span one or several tiles (15360
four-byte or 7680 eight-byte elements) with ragged tails; every size runs the
default path and the one-workgroup-per-tile fallback, and small sizes also
the single-workgroup path and the persistent kernel forced on (through the
small-n and mode knobs).
"""
import numpy as np
import pytest
import torch

import device_wide_prefix_tile_amd as dw
import golden_fixtures
import oracle
import seeded_inputs as si
from parity_helpers import assert_equal, assert_f32_close, from_dev, to_dev

pytestmark = pytest.mark.gpu

TILE = 15 * 64 * 16   # elements per tile of plain 4-byte scans (15 data wavefronts x 64 lanes x 16)
TILE_C = 15 * 64 * 20  # elements per tile of compaction
TILE_SEG = 15 * 64 * 16  # elements per tile of segmented scans (16 consecutive elements per lane in the
                         # persistent kernel, 1024 per wavefront)
TILE8 = 15 * 64 * 8   # pairs per tile of the 8-byte affine type
SIZES = [1, 2, 3, 63, 64, 65, 255, 256, 257, 1000, 4097, TILE8 - 1, TILE8, TILE8 + 1, TILE_C - 1, TILE_C,
         TILE_C + 1, TILE - 1, TILE, TILE + 1, 3 * TILE + 17, 65536 + 1, 250001, 1000003]
NP = {"i32": np.int32, "u32": np.uint32, "f32": np.float32}


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    dw.lib()
    old = dw.scan_set_small_n_max(dw.SCAN_SMALL_N_AUTO)
    yield
    dw.scan_set_small_n_max(old)


class Path:
    """Select a kernel path: 'single' (one workgroup walks all tiles), 'multi'
    (the persistent multi-tile kernel, forced even for small n), 'fallback'
    (one workgroup per tile, forced even for small n), 'rts' (reduce-then-scan,
    forced even for small n) or 'auto' (the default)."""

    def __init__(self, which):
        self.which = which

    def __enter__(self):
        lim = {"single": 1 << 40, "multi": 0, "fallback": 0, "rts": 0}.get(self.which)
        self.old = dw.scan_set_small_n_max(lim) if lim is not None else None
        self.old_mode = dw.scan_set_multi_tile_mode({"fallback": 1, "multi": 2, "rts": 3}.get(self.which, 0))

    def __exit__(self, *a):
        if self.old is not None:
            dw.scan_set_small_n_max(self.old)
        dw.scan_set_multi_tile_mode(self.old_mode)


def paths_for(n):
    # at these sizes 'auto' picks 'single' (at most one tile) or 'fallback' (the
    # persistent kernel starts at about 1.2e7 elements), both run here forced;
    # the full-size configurations cover 'auto' above that
    return ["multi", "single", "fallback", "rts"] if n <= 3 * TILE + 17 else ["auto", "multi", "rts"]


def values(dt, n, seed):
    if dt == "i32":
        return si.int32_full(seed, n)
    if dt == "u32":
        return si.uint32_full(seed, n)
    return si.float32_sym(seed, n)


def check_scan(op, x, y_gpu, exclusive, what):
    ref = oracle.scan(op, x, exclusive=exclusive)
    if isinstance(ref, tuple):
        return assert_f32_close(y_gpu, ref[0], ref[1], what)
    assert_equal(y_gpu, ref, what)


# ---------------------------------------------------------------- worked examples
@pytest.mark.parametrize("rec", golden_fixtures.all_examples("scan"), ids=lambda r: r["path"].split("/")[-1])
@pytest.mark.parametrize("path", ["single", "multi", "fallback"])
def test_golden_scan_on_gpu(rec, path):
    for dt in (rec["dtype"], np.int32, np.float32):
        x = rec["input"].astype(dt)
        with Path(path):
            if "inclusive" in rec:
                y = from_dev(dw.scan_inclusive(to_dev(x), rec["op"]))
                np.testing.assert_array_equal(y.astype(np.float64), rec["inclusive"].astype(np.float64))
            if "exclusive" in rec:
                y = from_dev(dw.scan_exclusive(to_dev(x), rec["op"]))
                np.testing.assert_array_equal(y.astype(np.float64), rec["exclusive"].astype(np.float64))


@pytest.mark.parametrize("rec", golden_fixtures.all_examples("compact"), ids=lambda r: r["path"].split("/")[-1])
@pytest.mark.parametrize("path", ["single", "multi", "fallback"])
def test_golden_compact_on_gpu(rec, path):
    for dt in (rec["dtype"], np.int32, np.float32):
        x = rec["input"].astype(dt)
        with Path(path):
            out, cnt = dw.compact(to_dev(x))
            out, cnt = from_dev(out), int(from_dev(cnt)[0])
        assert cnt == len(rec["output"])
        np.testing.assert_array_equal(out[:cnt].astype(np.float64), rec["output"].astype(np.float64))


# ---------------------------------------------------------------- plain scans
@pytest.mark.parametrize("dt", ["i32", "u32", "f32"])
@pytest.mark.parametrize("op", ["add", "max", "min"])
@pytest.mark.parametrize("exclusive", [False, True], ids=["incl", "excl"])
def test_scan_parity(op, dt, exclusive):
    fn = dw.scan_exclusive if exclusive else dw.scan_inclusive
    for k, n in enumerate(SIZES):
        x = values(dt, n, 100 + k)
        xd = to_dev(x)
        for path in paths_for(n):
            with Path(path):
                y = from_dev(fn(xd, op))
            check_scan(op, x, y, exclusive, "%s %s excl=%s n=%d path=%s" % (op, dt, exclusive, n, path))


def bitwise_input(seed, n, op, dt):
    """AND: all bits set except where rare events clear one; OR: no bits except where rare
    events set one -- about 16 events over the array, so the scan keeps changing late
    and every tile's carry matters (uniform words would saturate within a few elements)."""
    u = si.uint32_full(seed, n).astype(np.uint64)
    v = si.uint32_full(seed + 1, n)
    event = (u % np.uint64(max(64, n // 16))) == 0
    bit = (np.uint32(1) << (v % np.uint32(32))).astype(np.uint32)
    w = np.where(event, ~bit if op == "and" else bit,
                 np.uint32(0xFFFFFFFF) if op == "and" else np.uint32(0)).astype(np.uint32)
    return w.view(np.int32) if dt == "i32" else w


@pytest.mark.parametrize("dt", ["i32", "u32"])
@pytest.mark.parametrize("op", ["and", "or"])
@pytest.mark.parametrize("exclusive", [False, True], ids=["incl", "excl"])
def test_bitwise_parity(op, dt, exclusive):
    fn = dw.scan_exclusive if exclusive else dw.scan_inclusive
    for k, n in enumerate(SIZES + [(1 << 26) + 5]):
        x = bitwise_input(800 + k, n, op, dt)
        ref = oracle.scan(op, x, exclusive=exclusive)
        for path in paths_for(n):
            with Path(path):
                y = from_dev(fn(to_dev(x), op))
            assert_equal(y, ref, "%s %s excl=%s n=%d path=%s" % (op, dt, exclusive, n, path))


def test_bitwise_rejects_floats():
    with pytest.raises(TypeError):
        dw.scan_inclusive(torch.zeros(10, dtype=torch.float32, device="cuda"), "and")


@pytest.mark.parametrize("exclusive", [False, True], ids=["incl", "excl"])
@pytest.mark.parametrize("odd", [False, True], ids=["any_a", "odd_a"])
def test_affine_parity(exclusive, odd):
    fn = dw.scan_exclusive if exclusive else dw.scan_inclusive
    for k, n in enumerate(SIZES):
        ab = si.affine_pairs(200 + k, n, odd_a=odd)
        for path in paths_for(n):
            with Path(path):
                y = from_dev(fn(to_dev(ab), "affine"))
            assert_equal(y, oracle.scan_affine(ab, exclusive=exclusive),
                         "affine excl=%s odd=%s n=%d path=%s" % (exclusive, odd, n, path))


# ---------------------------------------------------------------- composite and matrix operators
TILE_MC = 7 * 64 * 16  # (value, count) pairs per tile (512-thread workgroups: 7 data wavefronts)
TILE_M2 = 7 * 64 * 8   # 2x2 matrices per tile
PAIR_SIZES = [1, 2, 63, 64, 65, 1000, 4097, TILE_M2 - 1, TILE_M2, TILE_M2 + 1, TILE_MC - 1, TILE_MC,
              TILE_MC + 1, 3 * TILE_MC + 17, 65537, 250001]


@pytest.mark.parametrize("exclusive", [False, True], ids=["incl", "excl"])
@pytest.mark.parametrize("counts", ["unit", "wrap"])
def test_maxcount_parity(exclusive, counts):
    fn = dw.scan_exclusive if exclusive else dw.scan_inclusive
    for k, n in enumerate(PAIR_SIZES):
        # values in [-20, 20]: the running maximum ties often
        vc = si.maxcount_pairs(600 + k, n, span=20, unit_counts=(counts == "unit"))
        ref = oracle.scan_maxcount(vc, exclusive=exclusive)
        for path in paths_for(n):
            with Path(path):
                y = from_dev(fn(to_dev(vc), "maxcount"))
            assert_equal(y, ref, "maxcount excl=%s counts=%s n=%d path=%s" % (exclusive, counts, n, path))


@pytest.mark.parametrize("exclusive", [False, True], ids=["incl", "excl"])
def test_mat2_parity(exclusive):
    fn = dw.scan_exclusive if exclusive else dw.scan_inclusive
    for k, n in enumerate(PAIR_SIZES):
        x = si.mat2_elems(700 + k, n)
        ref = oracle.scan_mat2(x, exclusive=exclusive)
        for path in paths_for(n):
            with Path(path):
                y = from_dev(fn(to_dev(x), "mat2"))
            assert_equal(y, ref, "mat2 excl=%s n=%d path=%s" % (exclusive, n, path))


def test_mat2_special_cases():
    n = 7 * TILE_M2 + 5
    # powers of [[1, 1], [1, 0]] (Fibonacci numbers mod 2^32)
    x = np.tile(np.array([1, 1, 1, 0], np.uint32), (n, 1))
    for path in ("multi", "fallback", "rts"):
        with Path(path):
            assert_equal(from_dev(dw.scan_inclusive(to_dev(x), "mat2")), oracle.scan_mat2(x), "fib " + path)
    # affine maps as [[a, b], [0, 1]]: the matrix scan's first row is the affine scan
    ab = si.affine_pairs(95, n)
    m = np.zeros((n, 4), np.uint32)
    m[:, 0], m[:, 1], m[:, 3] = ab[:, 0], ab[:, 1], 1
    y = from_dev(dw.scan_inclusive(to_dev(m), "mat2"))
    assert_equal(np.ascontiguousarray(y[:, :2]), from_dev(dw.scan_inclusive(to_dev(ab), "affine")), "mat2 vs affine")


TILE_M3 = 7 * 64 * 8   # 3x3 matrices per tile (512-thread workgroups: 7 data wavefronts x 64 lanes x 8)
MAT3_SIZES = [1, 2, 3, 63, 64, 65, 255, 256, 257, 767, 768, 769, TILE_M3 - 1, TILE_M3, TILE_M3 + 1,
              3 * TILE_M3 + 17, 5000, 65537, 250001]


@pytest.mark.parametrize("exclusive", [False, True], ids=["incl", "excl"])
def test_mat3_parity(exclusive):
    fn = dw.scan_exclusive if exclusive else dw.scan_inclusive
    for k, n in enumerate(MAT3_SIZES):
        x = si.mat3_elems(750 + k, n)
        ref = oracle.scan_mat3(x, exclusive=exclusive)
        for path in paths_for(n):
            with Path(path):
                y = from_dev(fn(to_dev(x), "mat3"))
            assert_equal(y, ref, "mat3 excl=%s n=%d path=%s" % (exclusive, n, path))


def test_mat3_special_cases():
    n = 9 * TILE_M3 + 5
    # powers of the tribonacci companion matrix
    x = np.tile(np.array([1, 1, 1, 1, 0, 0, 0, 1, 0], np.uint32), (n, 1))
    for path in ("multi", "fallback", "rts"):
        with Path(path):
            assert_equal(from_dev(dw.scan_inclusive(to_dev(x), "mat3")), oracle.scan_mat3(x), "tribonacci " + path)
    # 2x2 matrices A as [[A, 0], [0, 1]]: the upper-left block is the 2x2 scan
    a = si.mat2_elems(96, n)
    m = np.zeros((n, 9), np.uint32)
    m[:, 0], m[:, 1], m[:, 3], m[:, 4], m[:, 8] = a[:, 0], a[:, 1], a[:, 2], a[:, 3], 1
    y = from_dev(dw.scan_exclusive(to_dev(m), "mat3"))
    assert_equal(np.ascontiguousarray(y[:, [0, 1, 3, 4]]), from_dev(dw.scan_exclusive(to_dev(a), "mat2")),
                 "mat3 vs mat2")
    # (n, 3, 3) tensors are accepted as they are
    x3 = si.mat3_elems(97, 3000).reshape(-1, 3, 3)
    assert_equal(from_dev(dw.scan_inclusive(to_dev(x3), "mat3")), oracle.scan_mat3(x3), "(n, 3, 3)")


@pytest.mark.parametrize("path", ["auto", "multi", "fallback", "rts"])
def test_mat3_unaligned_and_in_place(path):
    """Views 4 bytes off 16-byte alignment take the word-wise path; in place is allowed."""
    for k, n in enumerate([1, 769, 3 * TILE_M3 + 17, 250001]):
        flat = si.mat3_elems(760 + k, n + 1).reshape(-1)
        x = flat[1:1 + 9 * n].reshape(n, 9)  # the matrices that start one word in
        ref = oracle.scan_mat3(x)
        with Path(path):
            xd = to_dev(flat)[1:1 + 9 * n].view(n, 9)  # 4 bytes off 16-byte alignment
            assert xd.data_ptr() % 16 == 4
            assert_equal(from_dev(dw.scan_inclusive(xd, "mat3")), ref, "unaligned n=%d path=%s" % (n, path))
            dw.scan_inclusive(xd, "mat3", out=xd)
            assert_equal(from_dev(xd), ref, "unaligned in place n=%d path=%s" % (n, path))
            t = to_dev(x)
            dw.scan_exclusive(t, "mat3", out=t)
            assert_equal(from_dev(t), oracle.scan_mat3(x, exclusive=True), "in place n=%d path=%s" % (n, path))


def odd_det_matrices(seed, n, k):
    """(n, k*k) uint32 matrices I + 2R: odd determinant, so invertible mod 2^32 -- their
    products never collapse to zero, unlike products of uniform matrices, and every
    output depends on the whole prefix (a wrong carry between tiles cannot go unseen)."""
    m = (si.uint32_full(seed, k * k * n).reshape(n, k * k) * np.uint32(2)).astype(np.uint32)
    for i in range(k):
        m[:, i * k + i] += np.uint32(1)
    return m


@pytest.mark.parametrize("op,k", [("mat2", 2), ("mat3", 3)])
def test_matrix_products_nondegenerate_large(op, k):
    """2^22 matrices with odd determinants: the persistent kernel's steady state (several
    tiles per workgroup), the one-tile kernel and reduce-then-scan, inclusive and exclusive."""
    n = (1 << 22) + 3
    x = odd_det_matrices(720 + k, n, k)
    ref_fn = oracle.scan_mat2 if k == 2 else oracle.scan_mat3
    xd = to_dev(x)
    for excl in (False, True):
        ref = ref_fn(x, exclusive=excl)
        for path in ("auto", "multi", "fallback", "rts"):
            print("%s excl=%s path=%s" % (op, excl, path), flush=True)
            with Path(path):
                y = from_dev((dw.scan_exclusive if excl else dw.scan_inclusive)(xd, op))
            assert_equal(y, ref, "%s excl=%s path=%s" % (op, excl, path))
    assert not np.any(np.all(ref_fn(x)[-5:] == 0, axis=1))  # nothing collapsed
    assert dw.scan_get_device_error() == 0


@pytest.mark.parametrize("op,logn", [("maxcount", 27), ("mat2", 25), ("mat3", 24)])
def test_composite_and_matrix_full_size(op, logn):
    """The benchmarked sizes of the composite and matrix operators, compared whole."""
    n = 1 << logn
    print("%s inclusive n=2^%d" % (op, logn), flush=True)
    if op == "maxcount":
        x, ref_fn = si.maxcount_pairs(8, n), oracle.scan_maxcount
    elif op == "mat2":
        x, ref_fn = si.mat2_elems(9, n), oracle.scan_mat2
    else:
        x, ref_fn = si.mat3_elems(10, n), oracle.scan_mat3
    xd = to_dev(x)
    y = from_dev(dw.scan_inclusive(xd, op))
    assert_equal(y, ref_fn(x), "%s full size" % op)
    del xd
    torch.cuda.empty_cache()


# ---------------------------------------------------------------- segmented scans
HEAD_MIXES = {
    "mean1000": lambda s, n: si.segment_heads(s, n, 1000.0),
    "mean3": lambda s, n: si.segment_heads(s, n, 3.0),
    "mean5000": lambda s, n: si.segment_heads(s, n, 5000.0),
    "all": lambda s, n: np.ones(n, np.uint8),
    "first_only": lambda s, n: np.zeros(n, np.uint8),
    "tile_starts": lambda s, n: (np.arange(n) % TILE_SEG == 0).astype(np.uint8) * 7,
    "tile_ends": lambda s, n: (np.arange(n) % TILE_SEG == TILE_SEG - 1).astype(np.uint8),
    "lane_starts": lambda s, n: (np.arange(n) % 16 == 0).astype(np.uint8),
    "wave_ends": lambda s, n: (np.arange(n) % 1024 == 1023).astype(np.uint8),
}


@pytest.mark.parametrize("dt", ["i32", "u32", "f32"])
@pytest.mark.parametrize("op", ["add", "max", "min"])
@pytest.mark.parametrize("exclusive", [False, True], ids=["incl", "excl"])
def test_segmented_parity(op, dt, exclusive):
    for k, n in enumerate([1, 2, 65, TILE_C - 1, TILE_C + 1, TILE_SEG - 1, TILE_SEG + 1, 3 * TILE_SEG + 17, 250001,
                           1000003]):
        x = values(dt, n, 300 + k) if dt != "i32" else si.int32_pm100(300 + k, n)
        for mix, gen in HEAD_MIXES.items():
            h = gen(400 + k, n)
            xd, hd = to_dev(x), to_dev(h)
            for path in paths_for(n):
                with Path(path):
                    y = from_dev(dw.segmented_scan(xd, hd, op, exclusive=exclusive))
                ref = oracle.segmented_scan(op, x, h, exclusive=exclusive)
                what = "seg %s %s excl=%s n=%d heads=%s path=%s" % (op, dt, exclusive, n, mix, path)
                if isinstance(ref, tuple):
                    assert_f32_close(y, ref[0], ref[1], what)
                else:
                    assert_equal(y, ref, what)


def test_segmented_head_zero_flag_ignored():
    x = np.arange(1, 10001, dtype=np.int32)
    h = np.zeros(x.size, np.uint8)
    h[5000] = 1
    for path in ("single", "multi", "fallback"):
        with Path(path):
            y = from_dev(dw.segmented_scan(to_dev(x), to_dev(h), "add"))
        assert_equal(y, oracle.segmented_scan("add", x, h), "head[0]=0 path=%s" % path)


# ---------------------------------------------------------------- compaction
def compact_inputs(dt, n, seed):
    if dt == "f32":
        return si.float32_normal(seed, n)
    if dt == "i32":
        return si.int32_full(seed, n)
    u = si.uint32_full(seed, n)
    u[si.segment_heads(seed, n, 2.0).astype(bool)] = 0
    return u


@pytest.mark.parametrize("dt", ["i32", "u32", "f32"])
def test_compact_parity(dt):
    for k, n in enumerate([0] + SIZES):
        x = compact_inputs(dt, n, 500 + k)
        xd = to_dev(x) if n else torch.empty(0, dtype={"i32": torch.int32, "u32": torch.uint32,
                                                         "f32": torch.float32}[dt], device="cuda")
        for path in paths_for(n):
            with Path(path):
                out, cnt = dw.compact(xd)
                out, cnt = from_dev(out), int(from_dev(cnt)[0])
            ref, rc, _ = oracle.compact(x)
            what = "compact %s n=%d path=%s" % (dt, n, path)
            assert cnt == rc, what
            assert_equal(out[:cnt], ref, what)


def test_compact_special_values():
    x = np.array([0.0, -0.0, np.nan, 1.0, -1.0, np.inf, -np.inf, 1e-45, -1e-45] * 1000, np.float32)
    for path in ("single", "multi", "fallback"):
        with Path(path):
            out, cnt = dw.compact(to_dev(x))
            out, cnt = from_dev(out), int(from_dev(cnt)[0])
        ref, rc, _ = oracle.compact(x)
        assert cnt == rc == 3000
        assert_equal(out[:cnt], ref, "special values path=%s" % path)


@pytest.mark.parametrize("path", ["multi", "fallback", "single"])
def test_compact_output_offsets(path):
    """Outputs that start 4, 8 or 12 bytes past a 16-byte boundary (the persistent kernel
    writes each tile's run in 16-byte chunks aligned in memory), with inputs aligned and not,
    over several tiles and a ragged tail; nothing outside [0, count) is written."""
    n = 5 * TILE_C + 333
    x = si.float32_normal(71, n)
    ref, rc, _ = oracle.compact(x)
    for k, (in_off, out_off) in enumerate([(0, 1), (0, 2), (0, 3), (1, 1), (3, 2)]):
        xd = to_dev(np.concatenate([np.zeros(in_off, np.float32), x]))[in_off:]
        buf = torch.full((n + 8,), 5.5, dtype=torch.float32, device="cuda")
        o = buf[out_off:out_off + n]
        with Path(path):
            _, cnt = dw.compact(xd, out=o)
            cnt = int(from_dev(cnt)[0])
        b = from_dev(buf)
        what = "compact offsets in=%d out=%d path=%s" % (in_off, out_off, path)
        assert cnt == rc, what
        assert_equal(b[out_off:out_off + cnt], ref, what)
        assert np.all(b[:out_off] == np.float32(5.5)) and np.all(b[out_off + cnt:] == np.float32(5.5)), what


def test_compact_leaves_tail_untouched():
    x = si.float32_normal(9, 20000)
    out = torch.full((20000,), 12345.0, device="cuda")
    o, cnt = dw.compact(to_dev(x), out=out)
    o, cnt = from_dev(o), int(from_dev(cnt)[0])
    assert np.all(o[cnt:] == 12345.0)


@pytest.mark.parametrize("kept", ["none", "all"])
@pytest.mark.parametrize("path", ["auto", "multi", "fallback", "rts"])
def test_compact_none_or_all_kept_large(kept, path):
    """Compaction that keeps nothing or everything at a size that runs the persistent kernel
    by default ([L7] concept 2 compaction figure: the count is the last exclusive flag
    position plus the last flag): count 0 with the output untouched, or count n with the
    output equal to the input."""
    n = (1 << 24) + 17
    base = np.abs(si.float32_normal(66, n))
    if kept == "none":
        x = -base
        x[::7] = -0.0
        x[3::11] = 0.0
    else:
        x = base + np.float32(1e-30)
        x[5::13] = np.float32(1e-45)  # the smallest subnormal is > 0 and kept
    xd = to_dev(x)
    out = torch.full((n,), 7.0, dtype=torch.float32, device="cuda")
    with Path(path):
        o, cnt = dw.compact(xd, out=out)
        o, cnt = from_dev(o), int(from_dev(cnt)[0])
    ref, rc, _ = oracle.compact(x)
    assert rc == (0 if kept == "none" else n)
    assert cnt == rc, "compact %s path=%s: count %d" % (kept, path, cnt)
    if kept == "none":
        assert np.all(o == np.float32(7.0)), "output written although nothing was kept"
    else:
        assert_equal(o, ref, "compact all path=%s" % path)
    assert dw.scan_get_device_error() == 0


# ---------------------------------------------------------------- float max/min ties
# The tie reading for float max and min: a later value replaces the running one only when
# strictly greater (smaller), so of +0 and -0 the earlier one stays ([PMPP9] §9.1 identity
# table; [L7] concept 1: the order of operands is fixed, commutativity is not assumed).
# +0 and -0 are the only distinct floats that compare equal, so they are the only inputs
# that can show an operand swap in a float max/min combine.  The arrays below put the first
# zero at positions on lane (4 elements), round (256), wavefront (1024) and tile (15360)
# boundaries and follow it with zeros of both signs, so that any level of the kernel that
# folded a later zero before an earlier one (lanes, DPP steps, wavefronts, tile totals, the
# carry between tiles) would change the sign of some output.
TIE_FIRSTS = [0, 1, 3, 4, 5, 255, 256, 1023, 1024, 1025, 4096, TILE - 1, TILE, TILE + 1, 2 * TILE - 3,
              3 * TILE + 1000]


def signed_zero_input(seed, n, first, op, sign):
    """Values that never win before `first`; a zero of the given sign at `first`; after it,
    zeros of both signs (3 of 4) mixed with values that never win."""
    u = si.uint32_full(seed, n)
    lose = np.float32(-1.0) if op == "max" else np.float32(1.0)
    x = np.where(u % 4 == 0, lose * (1 + (u >> 8) % 5).astype(np.float32),
                 np.where((u >> 2) % 2 == 0, np.float32(0.0), np.float32(-0.0))).astype(np.float32)
    x[:first] = lose * np.float32(3.0)
    x[first] = np.float32(0.0) if sign > 0 else np.float32(-0.0)
    return x


@pytest.mark.parametrize("op", ["max", "min"])
@pytest.mark.parametrize("exclusive", [False, True], ids=["incl", "excl"])
def test_float_minmax_signed_zero_ties(op, exclusive):
    fn = dw.scan_exclusive if exclusive else dw.scan_inclusive
    n = 4 * TILE + 17
    for k, first in enumerate(TIE_FIRSTS):
        for sign in (1, -1):
            x = signed_zero_input(1000 + 2 * k + (sign < 0), n, first, op, sign)
            ref = oracle.scan(op, x, exclusive=exclusive)
            assert np.signbit(ref[-1]) == (sign < 0)
            xd = to_dev(x)
            for path in ("single", "multi", "fallback", "rts", "auto"):
                with Path(path):
                    y = from_dev(fn(xd, op))
                assert_equal(y.view(np.uint32), ref.view(np.uint32),
                             "%s excl=%s first=%d sign=%d path=%s" % (op, exclusive, first, sign, path))


@pytest.mark.parametrize("op", ["max", "min"])
def test_float_minmax_signed_zero_ties_large(op):
    """The same at a size the persistent kernel takes by default, the first zero deep in the
    array (thousands of tiles of carry before and after it)."""
    n = (1 << 24) + 17
    first = (1 << 24) - 3 * TILE + 5
    for sign in (1, -1):
        x = signed_zero_input(1100 + (sign < 0), n, first, op, sign)
        xd = to_dev(x)
        for exclusive in (False, True):
            ref = oracle.scan(op, x, exclusive=exclusive)
            for path in ("auto", "multi", "fallback", "rts"):
                with Path(path):
                    y = from_dev((dw.scan_exclusive if exclusive else dw.scan_inclusive)(xd, op))
                assert_equal(y.view(np.uint32), ref.view(np.uint32),
                             "%s excl=%s sign=%d path=%s" % (op, exclusive, sign, path))
    assert dw.scan_get_device_error() == 0


@pytest.mark.parametrize("op", ["max", "min"])
@pytest.mark.parametrize("exclusive", [False, True], ids=["incl", "excl"])
def test_segmented_float_minmax_signed_zero_ties(op, exclusive):
    """Segmented float max/min: every segment restarts, so every segment's first zero is a
    tie decision -- thousands per array, at segment heads spread over lanes, wavefronts and
    tiles (mean segment length 37, plus heads at every tile start)."""
    for k, n in enumerate([TILE_SEG - 1, 3 * TILE_SEG + 17, 250001, (1 << 24) + 17]):
        u = si.uint32_full(1200 + k, n)
        lose = np.float32(-1.0) if op == "max" else np.float32(1.0)
        x = np.where(u % 3 == 0, lose, np.where((u >> 2) % 2 == 0, np.float32(0.0),
                                                np.float32(-0.0))).astype(np.float32)
        h = si.segment_heads(1300 + k, n, 37.0)
        h[::TILE_SEG] = 1
        ref = oracle.segmented_scan(op, x, h, exclusive=exclusive)
        xd, hd = to_dev(x), to_dev(h)
        for path in (paths_for(n) if n < (1 << 24) else ["auto", "multi", "rts"]):
            with Path(path):
                y = from_dev(dw.segmented_scan(xd, hd, op, exclusive=exclusive))
            assert_equal(y.view(np.uint32), ref.view(np.uint32),
                         "seg %s excl=%s n=%d path=%s" % (op, exclusive, n, path))


# ---------------------------------------------------------------- closed forms, layouts
def test_all_ones_float_is_bit_exact():
    # every prefix of ones is an integer <= 2^24: exact in float32 under any association
    n = 1 << 24
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    ye = from_dev(dw.scan_exclusive(x))
    yi = from_dev(dw.scan_inclusive(x))
    np.testing.assert_array_equal(ye, np.arange(n, dtype=np.float32))
    np.testing.assert_array_equal(yi, np.arange(1, n + 1, dtype=np.float32))


@pytest.mark.parametrize("path", ["auto", "single", "multi", "fallback", "rts"])
@pytest.mark.parametrize("n", [5000, 1000003])
def test_in_place(n, path):
    """out == in on every kernel path.  Reduce-then-scan compaction would write a tile's kept
    elements below the tile while earlier tiles of the same launch may not have read theirs
    yet, so in place it runs the single-pass kernel instead; the scans are safe there (each
    tile reads, then writes, only its own range)."""
    with Path(path):
        x = si.int32_full(61, n)
        t = to_dev(x)
        dw.scan_inclusive(t, "add", out=t)
        assert_equal(from_dev(t), oracle.scan("add", x), "in-place scan n=%d path=%s" % (n, path))
        h = si.segment_heads(62, n, 50.0)
        t = to_dev(x)
        dw.segmented_scan(t, to_dev(h), "max", exclusive=True, out=t)
        assert_equal(from_dev(t), oracle.segmented_scan("max", x, h, exclusive=True),
                     "in-place seg n=%d path=%s" % (n, path))
        for k, f in enumerate([si.float32_normal(63, n), np.abs(si.float32_normal(64, n)) + np.float32(1)]):
            t = to_dev(f)
            _, cnt = dw.compact(t, out=t)
            ref, rc, _ = oracle.compact(f)
            cnt = int(from_dev(cnt)[0])
            assert cnt == rc, "in-place compact %d n=%d path=%s" % (k, n, path)
            assert_equal(from_dev(t)[:cnt], ref, "in-place compact %d n=%d path=%s" % (k, n, path))


@pytest.mark.parametrize("n", [4097, 1000003])
def test_unaligned_views(n):
    # a view at a 4-byte offset takes the scalar path; results are the same
    x = si.float32_sym(71, n + 1)
    xd = to_dev(x)[1:]
    out = torch.empty(n + 1, dtype=torch.float32, device="cuda")[1:]
    y = from_dev(dw.scan_inclusive(xd, "add", out=out))
    ref, s = oracle.scan("add", x[1:])
    assert_f32_close(y, ref, s, "unaligned add n=%d" % n)
    xi = si.int32_full(72, n + 1)
    y = from_dev(dw.scan_exclusive(to_dev(xi)[1:], "min"))
    assert_equal(y, oracle.scan("min", xi[1:], exclusive=True), "unaligned min n=%d" % n)


def test_workspace_reuse_across_calls_and_streams():
    # status words of earlier calls (other ops, sizes, payload widths) must read as empty
    xs = [si.int32_full(80 + k, n) for k, n in enumerate([1000003, 70001, 4 * 1000003, 9000])]
    fs = si.float32_01(85, 2000003)
    s2 = torch.cuda.Stream()
    for rep in range(3):
        for x in xs:
            assert_equal(from_dev(dw.scan_inclusive(to_dev(x), "add")), oracle.scan("add", x), "reuse add")
            y, s = oracle.scan("add", fs)
            assert_f32_close(from_dev(dw.scan_inclusive(to_dev(fs), "add")), y, s, "reuse f32")
            with torch.cuda.stream(s2):
                yd = dw.scan_exclusive(to_dev(x), "max")
            s2.synchronize()
            assert_equal(from_dev(yd), oracle.scan("max", x, exclusive=True), "reuse max stream2")
    assert dw.scan_get_device_error() == 0


def test_concurrent_streams_share_the_gpu():
    """Persistent launches on two streams at once, each sized for the whole GPU: the second
    kernel's workgroups start only as the first one's retire, and neither may wait on a
    workgroup that has not started (tile numbers go out in start order)."""
    n = 1 << 25
    a, b = si.int32_full(91, n), si.float32_01(92, n)
    ra, (rb, sb) = oracle.scan("max", a), oracle.scan("add", b)
    xa, xb = to_dev(a), to_dev(b)
    ya, yb = torch.empty_like(xa), torch.empty_like(xb)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    with Path("multi"):
        for rep in range(4):
            with torch.cuda.stream(s1):
                dw.scan_inclusive(xa, "max", out=ya, stream=s1)
            with torch.cuda.stream(s2):
                dw.scan_inclusive(xb, "add", out=yb, stream=s2)
        torch.cuda.synchronize()
    assert_equal(from_dev(ya), ra, "stream 1")
    assert_f32_close(from_dev(yb), rb, sb, "stream 2")
    assert dw.scan_get_device_error() == 0


def test_host_threads_on_their_own_streams():
    """Two host threads call the library at the same time, each on its own stream (the
    library's calls release the interpreter lock): workspaces are per stream, and the
    settings and workspace table are guarded."""
    import threading
    n = (1 << 24) + 999
    a, b = si.int32_full(93, n), si.int32_0_15(94, n)
    ra, rb = oracle.scan("max", a, exclusive=True), oracle.scan("add", b)
    errors = []

    def work(x, ref, op, excl, name):
        try:
            st = torch.cuda.Stream()
            with torch.cuda.stream(st):
                xd = to_dev(x)
                yd = torch.empty_like(xd)
                for _ in range(20):
                    (dw.scan_exclusive if excl else dw.scan_inclusive)(xd, op, out=yd, stream=st)
                st.synchronize()
                if not np.array_equal(yd.cpu().numpy(), ref):
                    errors.append(name)
        except Exception as e:  # reported below, in the main thread
            errors.append("%s: %r" % (name, e))

    ts = [threading.Thread(target=work, args=(a, ra, "max", True, "max")),
          threading.Thread(target=work, args=(b, rb, "add", False, "add"))]
    for t in ts:
        t.start()
    for t in ts:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in ts), "a thread did not finish"
    assert not errors, errors
    assert dw.scan_get_device_error() == 0


def test_repeat_runs_bit_exact():
    # one passing run proves little for a protocol with races: repeat and compare
    n = (1 << 22) + 123
    x = si.int32_0_15(90, n)
    ab = si.affine_pairs(91, n // 2, odd_a=True)
    ref = oracle.scan("add", x, exclusive=True)
    ref_ab = oracle.scan_affine(ab)
    xd, abd = to_dev(x), to_dev(ab)
    for rep in range(20):
        assert_equal(from_dev(dw.scan_exclusive(xd, "add")), ref, "repeat %d add" % rep)
        if rep % 4 == 0:
            assert_equal(from_dev(dw.scan_inclusive(abd, "affine")), ref_ab, "repeat %d affine" % rep)
    assert dw.scan_get_device_error() == 0


def test_modes_alternate_on_one_stream():
    # Every kernel path on one stream, one after another, several rounds.
    # One 1 per tile makes the exclusive carries between tiles small integers
    # (t for tile t): the values that would pass for valid status words if
    # reduce-then-scan's plain carries ever shared memory with them.
    n = 300 * TILE + 77
    x = (np.arange(n) % TILE == 0).astype(np.int32)
    xd = to_dev(x)
    ref = oracle.scan("add", x, exclusive=True)
    for rnd in range(4):
        for path in ("rts", "multi", "fallback", "rts", "multi"):
            with Path(path):
                y = from_dev(dw.scan_exclusive(xd, "add"))
            assert_equal(y, ref, "round %d path=%s" % (rnd, path))
    assert dw.scan_get_device_error() == 0


def test_epoch_wrap_clears_status_words():
    """Status words carry the call number modulo 2^12 and the array is cleared when it
    wraps: more than 4095 multi-tile calls on one stream, alternating a float32 sum (one
    49-bit payload per tile) with an int32 maximum (one 32-bit payload) so that the words
    left by one layout must read as stale for the other, checked before, around and after
    the wrap."""
    n = 3 * TILE + 17
    f = si.float32_01(95, n)
    x = si.int32_full(96, n)
    rf, sf = oracle.scan("add", f)
    rx = oracle.scan("max", x)
    fd, xd = to_dev(f), to_dev(x)
    yf, yx = torch.empty_like(fd), torch.empty_like(xd)
    with Path("multi"):
        for k in range(2100):
            dw.scan_inclusive(fd, "add", out=yf)
            dw.scan_inclusive(xd, "max", out=yx)
            if k % 300 == 0 or 2040 <= k <= 2060:
                assert_f32_close(from_dev(yf), rf, sf, "f32 add call %d" % k)
                assert_equal(from_dev(yx), rx, "i32 max call %d" % k)
    with Path("fallback"):
        for k in range(2100):
            dw.scan_exclusive(xd, "max", out=yx)
            if k % 700 == 0:
                assert_equal(from_dev(yx), oracle.scan("max", x, exclusive=True), "fallback call %d" % k)
    assert dw.scan_get_device_error() == 0


def test_rts_float_sum_is_reproducible():
    # Reduce-then-scan fixes the association of a float sum by n alone (tile
    # totals, then one workgroup folding them in order): repeated calls, also
    # on another stream, give identical bits.
    n = 5 * TILE + 12345
    x = si.float32_sym(94, n)
    xd = to_dev(x)
    ref, s = oracle.scan("add", x)
    with Path("rts"):
        first = from_dev(dw.scan_inclusive(xd, "add"))
        assert_f32_close(first, ref, s, "rts float add")
        side = torch.cuda.Stream()
        for k in range(5):
            with torch.cuda.stream(side if k % 2 else torch.cuda.current_stream()):
                y = dw.scan_inclusive(xd, "add")
            torch.cuda.synchronize()
            assert np.array_equal(from_dev(y).view(np.uint32), first.view(np.uint32)), "run %d differs" % k


def test_bounded_waits_report_timeout_and_recover():
    # A tiny spin limit makes waits give up at once: the call must still
    # finish (every wave exits), report SCAN_ERR_TIMEOUT, clear it when read,
    # and leave later calls correct.
    n = (1 << 24) + 5
    x = si.float32_01(93, n)
    xd = to_dev(x)
    ref, s = oracle.scan("add", x)
    for mode in (2, 1):
        old_mode = dw.scan_set_multi_tile_mode(mode)
        old = dw.scan_set_spin_limit(0)
        try:
            for _ in range(3):
                dw.scan_inclusive(xd, "add")
            st = dw.scan_get_device_error()
        finally:
            dw.scan_set_spin_limit(old)
        assert st in (0, 5), st
        assert dw.scan_get_device_error() == 0
        y = from_dev(dw.scan_inclusive(xd, "add"))
        dw.scan_set_multi_tile_mode(old_mode)
        assert_f32_close(y, ref, s, "after timeout mode=%d" % mode)
        assert dw.scan_get_device_error() == 0


@pytest.mark.parametrize("op", ["mat3", "mat2", "affine"])
def test_bounded_waits_blocked_operators(op):
    """The same for the blocked-layout pipelines (3x3 matrices: the waiting tile held in
    LDS), persistent kernel forced."""
    n = (1 << 22) + 7
    x = {"mat3": lambda: odd_det_matrices(731, n, 3), "mat2": lambda: odd_det_matrices(732, n, 2),
         "affine": lambda: si.affine_pairs(733, n, odd_a=True)}[op]()
    ref = {"mat3": oracle.scan_mat3, "mat2": oracle.scan_mat2, "affine": oracle.scan_affine}[op](x)
    xd = to_dev(x)
    old_mode = dw.scan_set_multi_tile_mode(2)
    try:
        old = dw.scan_set_spin_limit(0)
        try:
            for _ in range(3):
                dw.scan_inclusive(xd, op)
            st = dw.scan_get_device_error()
        finally:
            dw.scan_set_spin_limit(old)
        assert st in (0, 5), st
        assert dw.scan_get_device_error() == 0
        assert_equal(from_dev(dw.scan_inclusive(xd, op)), ref, "%s after timeout" % op)
    finally:
        dw.scan_set_multi_tile_mode(old_mode)
    assert dw.scan_get_device_error() == 0


@pytest.mark.parametrize("path", ["multi", "auto"])
def test_blocked_layout_unaligned_and_in_place(path):
    """The persistent kernel's blocked lane layout (affine, (maximum, count), 2x2 matrices,
    segmented scans) on the element-wise path (views one element off 16-byte alignment), in
    place, and over ragged tails."""
    n = 3 * TILE_SEG + 4321
    with Path(path):
        ab = si.affine_pairs(81, n + 1)
        y = from_dev(dw.scan_inclusive(to_dev(ab)[1:], "affine"))
        assert_equal(y, oracle.scan_affine(ab[1:]), "unaligned affine")
        vc = si.maxcount_pairs(82, n + 1)
        y = from_dev(dw.scan_exclusive(to_dev(vc)[1:], "maxcount"))
        assert_equal(y, oracle.scan_maxcount(vc[1:], exclusive=True), "unaligned maxcount")
        x = si.int32_pm100(83, n + 1)
        h = si.segment_heads(84, n + 1, 37.0)
        y = from_dev(dw.segmented_scan(to_dev(x)[1:], to_dev(h)[1:], "add", exclusive=True))
        assert_equal(y, oracle.segmented_scan("add", x[1:], h[1:], exclusive=True), "unaligned segmented")
        m = si.mat2_elems(85, n)
        t = to_dev(m)
        dw.scan_inclusive(t, "mat2", out=t)
        assert_equal(from_dev(t), oracle.scan_mat2(m), "in-place mat2")
        t = to_dev(ab)
        dw.scan_exclusive(t, "affine", out=t)
        assert_equal(from_dev(t), oracle.scan_affine(ab, exclusive=True), "in-place affine")
