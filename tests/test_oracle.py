"""Pins for the CPU oracle (no GPU).

The oracle is checked against things other than itself:
  * worked examples printed on the pages (tests/golden/, each file cites its page);
  * closed forms (all-ones float sums are exact integers; the page's compaction
    program on x[i] = i % 10 - 5 keeps 400 values 1 2 3 4 ...);
  * brute force on tiny inputs: every y[i] recomputed from scratch with Python
    integers, math.fsum, builtin max/min, 2x2 matrix products and per-segment folds;
  * invariants (last inclusive element = total, exclusive = inclusive shifted
    right with the identity, compaction keeps order and count);
  * special cases that reduce to numpy routines (cumsum, maximum.accumulate,
    cumprod) at larger sizes.
"""
import math
import struct

import numpy as np
import pytest

import oracle
import seeded_inputs as si
import golden_fixtures

U32 = 1 << 32
IDENT = {
    ("add", np.int32): 0, ("max", np.int32): -(1 << 31), ("min", np.int32): (1 << 31) - 1,
    ("add", np.uint32): 0, ("max", np.uint32): 0, ("min", np.uint32): U32 - 1,
    ("max", np.float32): -math.inf, ("min", np.float32): math.inf,
}


# --------------------------------------------------------------------------
# worked examples from the pages
# --------------------------------------------------------------------------
@pytest.mark.parametrize("rec", golden_fixtures.all_examples("scan"), ids=lambda r: r["path"].split("/")[-1])
def test_golden_scan(rec):
    x = rec["input"]
    for dt in {rec["dtype"], np.int32, np.float32}:
        xx = x.astype(dt)
        if "inclusive" in rec:
            y = oracle.scan(rec["op"], xx)
            y = y[0] if isinstance(y, tuple) else y
            np.testing.assert_array_equal(np.asarray(y, np.float64), rec["inclusive"].astype(np.float64))
        if "exclusive" in rec:
            y = oracle.scan(rec["op"], xx, exclusive=True)
            y = y[0] if isinstance(y, tuple) else y
            np.testing.assert_array_equal(np.asarray(y, np.float64), rec["exclusive"].astype(np.float64))
    if "remaining" in rec:
        incl = oracle.scan("add", x.astype(np.int32))
        assert int(rec["total_length"]) - int(incl[-1]) == int(rec["remaining"])


@pytest.mark.parametrize("rec", golden_fixtures.all_examples("compact"), ids=lambda r: r["path"].split("/")[-1])
def test_golden_compact(rec):
    for dt in {rec["dtype"], np.int32, np.float32}:
        x = rec["input"].astype(dt)
        out, count, pos = oracle.compact(x)
        np.testing.assert_array_equal(pos, rec["positions"])
        np.testing.assert_array_equal(out.astype(np.float64), rec["output"].astype(np.float64))
        assert count == int(rec["flags"].sum()) == len(rec["output"])
        # the flag scan itself is an exclusive add-scan of the printed flags
        np.testing.assert_array_equal(oracle.scan("add", rec["flags"], exclusive=True), rec["positions"])


# --------------------------------------------------------------------------
# closed forms
# --------------------------------------------------------------------------
def test_all_ones_float_is_exact_index():
    # every partial sum of ones is an integer <= 2^24, exact in float and double
    n = 1 << 20
    x = np.ones(n, np.float32)
    y, s = oracle.scan("add", x, exclusive=True)
    np.testing.assert_array_equal(y, np.arange(n, dtype=np.float64))
    np.testing.assert_array_equal(s, np.arange(n, dtype=np.float64))
    y, s = oracle.scan("add", x)
    np.testing.assert_array_equal(y, np.arange(1, n + 1, dtype=np.float64))


def test_page_compaction_program_closed_form():
    # x[i] = i % 10 - 5 over 1000 elements, keep x > 0: i % 10 in {6,7,8,9}
    x = np.array([(i % 10) - 5 for i in range(1000)], np.float32)
    out, count, pos = oracle.compact(x)
    assert count == 400
    np.testing.assert_array_equal(out, np.tile(np.array([1, 2, 3, 4], np.float32), 100))
    assert pos[-1] + (1 if x[-1] > 0 else 0) == count


def test_int32_add_wraps():
    x = np.array([2**31 - 1, 1, -1, 5], np.int32)
    np.testing.assert_array_equal(oracle.scan("add", x),
                                  np.array([2**31 - 1, -(2**31), 2**31 - 1, -(2**31) + 4], np.int32))


def test_affine_known_recurrence():
    # y_i = a_i * y_{i-1} + b_i with y_{-1} = 0; a = 2, b = 1 gives 1, 3, 7, 15 (= 2^(i+1) - 1)
    ab = np.array([[2, 1]] * 6, np.uint32)
    y = oracle.scan_affine(ab)
    np.testing.assert_array_equal(y[:, 1], np.array([1, 3, 7, 15, 31, 63], np.uint32))
    np.testing.assert_array_equal(y[:, 0], np.array([2, 4, 8, 16, 32, 64], np.uint32))
    ye = oracle.scan_affine(ab, exclusive=True)
    np.testing.assert_array_equal(ye[0], [1, 0])
    np.testing.assert_array_equal(ye[1:], y[:-1])


def test_affine_non_commutative_order():
    # applying (3,5) after (2,7): x -> 3*(2x+7)+5 = 6x + 26, not 2*(3x+5)+7 = 6x + 17
    ab = np.array([[2, 7], [3, 5]], np.uint32)
    np.testing.assert_array_equal(oracle.scan_affine(ab)[1], [6, 26])


def test_float_max_ties_keep_earlier():
    # reading: a later value replaces the running one only when strictly greater
    x = np.array([0.0, -0.0, 1.0, 1.0], np.float32)
    y = oracle.scan("max", x)
    assert struct.pack("<f", y[1]) == struct.pack("<f", 0.0)  # +0 kept over -0
    y = oracle.scan("min", np.array([-0.0, 0.0], np.float32))
    assert struct.pack("<f", y[1]) == struct.pack("<f", -0.0)
    ye = oracle.scan("max", x, exclusive=True)
    assert ye[0] == -np.inf


# --------------------------------------------------------------------------
# brute force on tiny inputs: each y[i] from scratch
# --------------------------------------------------------------------------
def _tiny(dtype, n, rng):
    if dtype == np.int32:
        return rng.integers(-(2**31), 2**31, n, dtype=np.int64).astype(np.int32)
    if dtype == np.uint32:
        return rng.integers(0, 2**32, n, dtype=np.uint64).astype(np.uint32)
    return (rng.integers(-(2**23), 2**23, n) * 2.0**-23).astype(np.float32)


def _bf_fold(op, dtype, vals):
    """Fold a prefix from scratch with Python builtins."""
    vals = [v.item() for v in vals]
    if not vals:
        return IDENT[(op, dtype)] if (op, dtype) in IDENT else 0
    if op == "add":
        if dtype == np.float32:
            return math.fsum(vals)
        t = sum(vals) % U32
        return t - U32 if (dtype == np.int32 and t >= 2**31) else t
    return max(vals) if op == "max" else min(vals)


@pytest.mark.parametrize("dtype", [np.int32, np.uint32, np.float32])
@pytest.mark.parametrize("op", ["add", "max", "min"])
@pytest.mark.parametrize("exclusive", [False, True])
def test_bruteforce_scan(op, dtype, exclusive):
    rng = np.random.default_rng(11)
    for n in list(range(0, 34)) + [63, 64, 65]:
        x = _tiny(dtype, n, rng)
        y = oracle.scan(op, x, exclusive=exclusive)
        y = y[0] if isinstance(y, tuple) else y
        for i in range(n):
            want = _bf_fold(op, dtype, x[:i] if exclusive else x[:i + 1])
            assert float(y[i]) == float(want), (op, dtype, exclusive, n, i)


# Bitwise AND / OR scans ([L7] concept 1 lists them among scan operators):
# identities all bits set / no bits set.
@pytest.mark.parametrize("dtype", [np.int32, np.uint32])
@pytest.mark.parametrize("op", ["and", "or"])
@pytest.mark.parametrize("exclusive", [False, True])
def test_bruteforce_bitwise(op, dtype, exclusive):
    rng = np.random.default_rng(21)
    f = (lambda a, b: a & b) if op == "and" else (lambda a, b: a | b)
    ident = -1 if op == "and" else 0  # all bits / none, as a Python int
    for n in (1, 2, 3, 7, 33):
        # mostly-set words for AND, mostly-clear ones for OR, so prefixes stay varied
        r = rng.integers(0, 2**32, (3, n), dtype=np.uint64)
        w = (r[0] | r[1] | r[2]) if op == "and" else (r[0] & r[1] & r[2])
        x = w.astype(np.uint32).view(np.int32) if dtype == np.int32 else w.astype(np.uint32)
        y = oracle.scan(op, x, exclusive=exclusive)
        for i in range(n):
            acc = ident
            for k in range(i if exclusive else i + 1):
                acc = f(acc, int(x[k]))
            want = np.array(acc & 0xFFFFFFFF, dtype=np.uint64).astype(np.uint32)
            assert int(y.view(np.uint32)[i]) == int(want), (op, exclusive, n, i)


def test_bitwise_against_numpy_and_monotone():
    n = 100000
    u = si.uint32_full(22, 3 * n).reshape(3, n)
    xa = u[0] | u[1] | u[2] | (si.uint32_full(23, n) & np.uint32(0xFFFF0FFF))
    xo = u[0] & u[1] & u[2] & (si.uint32_full(24, n) >> np.uint32(3))
    ya, yo = oracle.scan("and", xa), oracle.scan("or", xo)
    np.testing.assert_array_equal(ya, np.bitwise_and.accumulate(xa))
    np.testing.assert_array_equal(yo, np.bitwise_or.accumulate(xo))
    assert np.all(ya[1:] & ~ya[:-1] == 0) and np.all(yo[:-1] & ~yo[1:] == 0)  # bits only leave / only join
    np.testing.assert_array_equal(oracle.scan("and", xa, exclusive=True)[1:], ya[:-1])
    assert oracle.scan("and", xa, exclusive=True)[0] == np.uint32(0xFFFFFFFF)
    assert oracle.scan("or", xo, exclusive=True)[0] == 0
    np.testing.assert_array_equal(oracle.scan("or", xo.view(np.int32)).view(np.uint32), yo)
    with pytest.raises(TypeError):
        oracle.scan("and", np.zeros(3, np.float32))


def test_bruteforce_exercise_input():
    # exercise array of the PMPP chapter-9 notes (§八 "Scan定义"); the page prints no answer
    x = np.array([3, 1, 4, 1, 5, 9, 2, 6], np.int32)
    want_incl = [sum(x[:i + 1].tolist()) for i in range(8)]
    want_excl = [sum(x[:i].tolist()) for i in range(8)]
    np.testing.assert_array_equal(oracle.scan("add", x), want_incl)
    np.testing.assert_array_equal(oracle.scan("add", x, exclusive=True), want_excl)
    assert want_incl == [3, 4, 8, 9, 14, 23, 25, 31]


def _mat_affine(pairs):
    """Compose x -> a x + b maps as 2x2 matrices [[a, b], [0, 1]], later on the left."""
    m = [[1, 0], [0, 1]]
    for a, b in pairs:
        a, b = int(a), int(b)
        m = [[(a * m[0][0]) % U32, (a * m[0][1] + b * m[1][1]) % U32], [0, 1]]
    return m[0][0], m[0][1]


def _closed_affine(pairs):
    """A_i = prod a_k; B_i = sum_j b_j * prod_{k>j} a_k (mod 2^32)."""
    A = 1
    for a, _ in pairs:
        A = (A * int(a)) % U32
    B = 0
    for j, (_, b) in enumerate(pairs):
        p = int(b)
        for a, _ in pairs[j + 1:]:
            p = (p * int(a)) % U32
        B = (B + p) % U32
    return A, B


@pytest.mark.parametrize("exclusive", [False, True])
def test_bruteforce_affine(exclusive):
    rng = np.random.default_rng(5)
    for n in list(range(0, 20)) + [40]:
        ab = rng.integers(0, 2**32, (n, 2), dtype=np.uint64).astype(np.uint32)
        y = oracle.scan_affine(ab, exclusive=exclusive)
        for i in range(n):
            pre = [tuple(p) for p in (ab[:i] if exclusive else ab[:i + 1])]
            assert tuple(int(v) for v in y[i]) == _mat_affine(pre) == _closed_affine(pre)


def _bf_segmented(op, dtype, x, heads, exclusive):
    out = []
    for i in range(len(x)):
        s = max(j for j in range(i + 1) if j == 0 or heads[j])
        out.append(_bf_fold(op, dtype, x[s:i] if exclusive else x[s:i + 1]))
    return out


@pytest.mark.parametrize("dtype", [np.int32, np.uint32, np.float32])
@pytest.mark.parametrize("op", ["add", "max", "min"])
@pytest.mark.parametrize("exclusive", [False, True])
def test_bruteforce_segmented(op, dtype, exclusive):
    rng = np.random.default_rng(7)
    for n in list(range(0, 24)) + [50]:
        x = _tiny(dtype, n, rng)
        heads = (rng.random(n) < 0.25).astype(np.uint8)
        if n > 1 and rng.random() < 0.5:
            heads[0] = 0  # index 0 is a head whatever its flag says
        y = oracle.segmented_scan(op, x, heads, exclusive=exclusive)
        y = y[0] if isinstance(y, tuple) else y
        want = _bf_segmented(op, dtype, x, heads, exclusive)
        for i in range(n):
            assert float(y[i]) == float(want[i]), (op, dtype, exclusive, n, i)


@pytest.mark.parametrize("dtype", [np.int32, np.uint32, np.float32])
def test_bruteforce_compact(dtype):
    rng = np.random.default_rng(9)
    for n in range(0, 40):
        x = _tiny(dtype, n, rng)
        if dtype == np.uint32:
            x[rng.random(n) < 0.4] = 0
        out, count, pos = oracle.compact(x)
        keep = [v for v in x.tolist() if v > 0]
        assert count == len(keep)
        assert out.tolist() == keep
        for i in range(n):
            assert pos[i] == sum(1 for v in x[:i].tolist() if v > 0)


# --------------------------------------------------------------------------
# invariants and special cases at larger sizes
# --------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", [np.int32, np.uint32, np.float32])
@pytest.mark.parametrize("op", ["add", "max", "min"])
def test_invariants(op, dtype):
    n = 100003
    x = {np.int32: si.int32_full, np.uint32: si.uint32_full, np.float32: si.float32_sym}[dtype](21, n)
    inc = oracle.scan(op, x)
    exc = oracle.scan(op, x, exclusive=True)
    if isinstance(inc, tuple):
        (inc, s_inc), (exc, s_exc) = inc, exc
        np.testing.assert_array_equal(s_exc[1:], s_inc[:-1])
        assert s_exc[0] == 0.0
        # values on the 2^-23 grid with |prefix| < 2^17: every double partial sum is exact
        assert inc[-1] == math.fsum(x.astype(np.float64).tolist())
        assert s_inc[-1] == math.fsum(np.abs(x.astype(np.float64)).tolist())
        ident = 0.0
    else:
        ident = IDENT[(op, dtype)]
        if op == "add":
            total = int(x.astype(np.int64).sum()) % U32
            assert int(inc[-1].astype(np.int64)) % U32 == total
        elif op == "max":
            assert inc[-1] == x.max()
            assert np.all(inc[1:] >= inc[:-1])
        else:
            assert inc[-1] == x.min()
            assert np.all(inc[1:] <= inc[:-1])
    # exclusive = inclusive shifted right by one with the identity at index 0
    assert float(exc[0]) == float(ident)
    np.testing.assert_array_equal(exc[1:], inc[:-1])


def test_reduces_to_numpy_routines():
    n = 200001
    xi = si.int32_full(3, n)
    np.testing.assert_array_equal(oracle.scan("add", xi),
                                  (np.cumsum(xi.astype(np.int64)) % U32).astype(np.uint32).view(np.int32))
    np.testing.assert_array_equal(oracle.scan("max", xi), np.maximum.accumulate(xi))
    np.testing.assert_array_equal(oracle.scan("min", xi), np.minimum.accumulate(xi))
    xu = si.uint32_full(4, n)
    np.testing.assert_array_equal(oracle.scan("max", xu), np.maximum.accumulate(xu))
    xf = si.float32_01(2, n)
    y, s = oracle.scan("add", xf)
    np.testing.assert_array_equal(y, np.cumsum(xf.astype(np.float64)))
    np.testing.assert_array_equal(s, np.cumsum(np.abs(xf.astype(np.float64))))
    np.testing.assert_array_equal(oracle.scan("max", xf), np.maximum.accumulate(xf))


def test_affine_special_cases():
    n = 100000
    ab = si.affine_pairs(4, n)
    # all a = 1: the b component is the wrapping add-scan of b
    ab1 = ab.copy()
    ab1[:, 0] = 1
    y = oracle.scan_affine(ab1)
    np.testing.assert_array_equal(y[:, 0], np.ones(n, np.uint32))
    np.testing.assert_array_equal(y[:, 1], (np.cumsum(ab1[:, 1].astype(np.uint64)) % U32).astype(np.uint32))
    # all b = 0: the a component is the running product, b stays 0
    ab0 = ab.copy()
    ab0[:, 1] = 0
    y = oracle.scan_affine(ab0)
    np.testing.assert_array_equal(y[:, 1], np.zeros(n, np.uint32))
    np.testing.assert_array_equal(y[:, 0], (np.cumprod(ab0[:, 0].astype(np.uint64)) % U32).astype(np.uint32))
    # the a component is always the running product of the multipliers
    y = oracle.scan_affine(ab)
    np.testing.assert_array_equal(y[:, 0], (np.cumprod(ab[:, 0].astype(np.uint64)) % U32).astype(np.uint32))


def test_segmented_special_cases():
    n = 50000
    x = si.int32_pm100(5, n)
    # every element a head: inclusive gives x, exclusive the identity
    h = np.ones(n, np.uint8)
    np.testing.assert_array_equal(oracle.segmented_scan("add", x, h), x)
    np.testing.assert_array_equal(oracle.segmented_scan("add", x, h, exclusive=True), np.zeros(n, np.int32))
    np.testing.assert_array_equal(oracle.segmented_scan("max", x, h, exclusive=True),
                                  np.full(n, -(2**31), np.int32))
    # a single head at 0: the plain scan
    h = np.zeros(n, np.uint8)
    for op in ("add", "max", "min"):
        np.testing.assert_array_equal(oracle.segmented_scan(op, x, h), oracle.scan(op, x))
        np.testing.assert_array_equal(oracle.segmented_scan(op, x, h, exclusive=True),
                                      oracle.scan(op, x, exclusive=True))
    # random heads: each segment's last value is the segment's own sum
    h = si.segment_heads(5, n, mean_len=100.0)
    y = oracle.segmented_scan("add", x, h)
    starts = np.flatnonzero(h)
    ends = np.append(starts[1:], n) - 1
    for a, b in zip(starts[:200], ends[:200]):
        assert y[b] == x[a:b + 1].astype(np.int64).sum()


def test_compaction_invariants_large():
    n = 300000
    x = si.float32_normal(3, n)
    out, count, pos = oracle.compact(x)
    flags = (x > 0)
    assert count == int(flags.sum())
    np.testing.assert_array_equal(out, x[flags])
    assert pos[-1] + int(flags[-1]) == count
    np.testing.assert_array_equal(pos, oracle.scan("add", flags.astype(np.uint32), exclusive=True))


# ---------------------------------------------------------------- (max, count) and 2x2 matrices
# The composite "(maximum, number of occurrences)" operator and matrix
# multiplication are the scan operators "Lecture 7: 并行模式五 —— 前缀和 / 扫描"
# names beside addition (concept 1); neither has a worked example on the
# pages, so both are pinned by brute force, closed forms and invariants.

def _maxcount_brute(vc, exclusive):
    out = []
    for i in range(len(vc)):
        pre = vc[:i] if exclusive else vc[:i + 1]
        if len(pre) == 0:
            out.append((-(2**31), 0))
            continue
        m = max(int(v) for v, _ in pre)
        c = sum(int(c) & 0xFFFFFFFF for v, c in pre if int(v) == m) % 2**32
        out.append((m, c))
    return out


@pytest.mark.parametrize("exclusive", [False, True], ids=["incl", "excl"])
def test_bruteforce_maxcount(exclusive):
    rng = np.random.default_rng(11)
    for n in (1, 2, 3, 7, 40, 97):
        v = rng.integers(-3, 4, n).astype(np.int32)  # few values: many ties
        c = rng.integers(0, 2**32, n, dtype=np.uint64).astype(np.uint32)  # counts that wrap
        vc = np.stack([v, c.view(np.int32)], axis=1)
        y = oracle.scan_maxcount(vc, exclusive=exclusive)
        want = _maxcount_brute(vc, exclusive)
        assert [(int(a), int(b) & 0xFFFFFFFF) for a, b in y] == want


def test_maxcount_closed_forms():
    n = 1000
    # all values equal: the count is the running sum of the counts
    vc = np.stack([np.full(n, 5, np.int32), np.arange(1, n + 1, dtype=np.int32)], axis=1)
    y = oracle.scan_maxcount(vc)
    np.testing.assert_array_equal(y[:, 0], 5)
    np.testing.assert_array_equal(y[:, 1].astype(np.int64), np.arange(1, n + 1) * np.arange(2, n + 2) // 2)
    # strictly increasing values with count 1: every element is a new maximum
    vc = np.stack([np.arange(-n, 0, dtype=np.int32), np.ones(n, np.int32)], axis=1)
    y = oracle.scan_maxcount(vc)
    np.testing.assert_array_equal(y, vc)
    # the empty fold heads every exclusive result
    y = oracle.scan_maxcount(vc, exclusive=True)
    assert tuple(y[0]) == (-(2**31), 0)
    np.testing.assert_array_equal(y[1:], oracle.scan_maxcount(vc)[:-1])


def test_maxcount_against_numpy():
    n = 3000
    v = (si.int32_full(71, n) % 50).astype(np.int32)
    vc = np.stack([v, np.ones(n, np.int32)], axis=1)
    y = oracle.scan_maxcount(vc)
    m = np.maximum.accumulate(v)
    np.testing.assert_array_equal(y[:, 0], m)
    counts = np.array([int((v[:i + 1] == m[i]).sum()) for i in range(n)])
    np.testing.assert_array_equal(y[:, 1], counts)


def _mat_mul(x, y):
    a, b, c, d = (int(t) for t in x)
    e, f, g, h = (int(t) for t in y)
    M = 2**32
    return ((a * e + b * g) % M, (a * f + b * h) % M, (c * e + d * g) % M, (c * f + d * h) % M)


@pytest.mark.parametrize("exclusive", [False, True], ids=["incl", "excl"])
def test_bruteforce_mat2(exclusive):
    rng = np.random.default_rng(12)
    for n in (1, 2, 3, 5, 33):
        x = rng.integers(0, 2**32, (n, 4), dtype=np.uint64).astype(np.uint32)
        y = oracle.scan_mat2(x, exclusive=exclusive)
        for i in range(n):
            P = (1, 0, 0, 1)
            for k in range(i if exclusive else i + 1):
                P = _mat_mul(x[k], P)  # the later factor on the left
            assert tuple(int(t) for t in y[i]) == P, i


def test_mat2_fibonacci_powers():
    # every element [[1, 1], [1, 0]]: the i-th inclusive product is its
    # (i+1)-th power [[F(i+2), F(i+1)], [F(i+1), F(i)]] (textbook identity),
    # with the Fibonacci numbers here from their defining recurrence
    n = 500
    x = np.tile(np.array([1, 1, 1, 0], np.uint32), (n, 1))
    y = oracle.scan_mat2(x)
    F = [0, 1]
    while len(F) < n + 3:
        F.append(F[-1] + F[-2])
    for i in range(n):
        want = [F[i + 2] % 2**32, F[i + 1] % 2**32, F[i + 1] % 2**32, F[i] % 2**32]
        assert [int(t) for t in y[i]] == want, i


def test_mat2_embeds_affine():
    # affine maps are the matrices [[a, b], [0, 1]]: the matrix scan must
    # reproduce the affine scan (pinned above) in its first row
    n = 2000
    ab = si.affine_pairs(13, n)
    x = np.zeros((n, 4), np.uint32)
    x[:, 0], x[:, 1], x[:, 3] = ab[:, 0], ab[:, 1], 1
    for exclusive in (False, True):
        y = oracle.scan_mat2(x, exclusive=exclusive)
        np.testing.assert_array_equal(y[:, :2], oracle.scan_affine(ab, exclusive=exclusive))
        np.testing.assert_array_equal(y[:, 2], 0)
        np.testing.assert_array_equal(y[:, 3], 1)


def test_mat2_determinant_is_multiplicative():
    n = 2000
    x = si.uint32_full(14, 4 * n).reshape(n, 4)
    y = oracle.scan_mat2(x)
    M = 2**32
    det = lambda t: (int(t[0]) * int(t[3]) - int(t[1]) * int(t[2])) % M
    acc = 1
    for i in range(n):
        acc = acc * det(x[i]) % M
        assert det(y[i]) == acc, i


def _mat3_mul(x, y):
    """3x3 product x * y mod 2^32 of two row-major 9-tuples, in Python ints."""
    M = 2**32
    return tuple(sum(int(x[3 * r + k]) * int(y[3 * k + c]) for k in range(3)) % M
                 for r in range(3) for c in range(3))


@pytest.mark.parametrize("exclusive", [False, True], ids=["incl", "excl"])
def test_bruteforce_mat3(exclusive):
    rng = np.random.default_rng(15)
    for n in (1, 2, 3, 5, 17):
        x = rng.integers(0, 2**32, (n, 9), dtype=np.uint64).astype(np.uint32)
        y = oracle.scan_mat3(x, exclusive=exclusive)
        for i in range(n):
            P = (1, 0, 0, 0, 1, 0, 0, 0, 1)
            for k in range(i if exclusive else i + 1):
                P = _mat3_mul(x[k], P)  # the later factor on the left
            assert tuple(int(t) for t in y[i]) == P, i
    assert oracle.scan_mat3(x.reshape(-1, 3, 3), exclusive=exclusive).shape == (17, 3, 3)


def test_mat3_tribonacci_powers():
    # every element the companion matrix T = [[1, 1, 1], [1, 0, 0], [0, 1, 0]]
    # of s(k+3) = s(k+2) + s(k+1) + s(k): T maps (s(k+2), s(k+1), s(k)) to
    # (s(k+3), s(k+2), s(k+1)), so column j of T^m is (s_j(m+2), s_j(m+1),
    # s_j(m)) for the sequence s_j started from the j-th unit vector
    # (s_j(2), s_j(1), s_j(0)) = e_j -- sequences from the recurrence alone
    n = 400
    x = np.tile(np.array([1, 1, 1, 1, 0, 0, 0, 1, 0], np.uint32), (n, 1))
    y = oracle.scan_mat3(x)
    cols = []
    for j in range(3):
        e = [0, 0, 0]
        e[j] = 1
        s = [e[2], e[1], e[0]]
        while len(s) < n + 4:
            s.append(s[-1] + s[-2] + s[-3])
        cols.append(s)
    for i in range(n):
        m = i + 1  # inclusive element i is T^(i+1)
        want = [cols[c][m + 2 - r] % 2**32 for r in range(3) for c in range(3)]
        assert [int(t) for t in y[i]] == want, i


def test_mat3_embeds_mat2():
    # [[A, 0], [0, 1]] multiplies like A: the upper-left block of the 3x3
    # scan must be the 2x2 scan (pinned above) and the rest stay [0, 0, 1]
    n = 2000
    a = si.mat2_elems(16, n)
    x = np.zeros((n, 9), np.uint32)
    x[:, 0], x[:, 1], x[:, 3], x[:, 4], x[:, 8] = a[:, 0], a[:, 1], a[:, 2], a[:, 3], 1
    for exclusive in (False, True):
        y = oracle.scan_mat3(x, exclusive=exclusive)
        np.testing.assert_array_equal(y[:, [0, 1, 3, 4]], oracle.scan_mat2(a, exclusive=exclusive))
        np.testing.assert_array_equal(y[:, [2, 5, 6, 7]], 0)
        np.testing.assert_array_equal(y[:, 8], 1)


def test_mat3_permutations_compose():
    # permutation matrices (column j has its 1 in row p[j]) multiply like the
    # permutations compose: X_i ... X_0 is the matrix of p_i o ... o p_0,
    # computed here by following indices, without any matrix product
    rng = np.random.default_rng(17)
    n = 500
    perms = [tuple(rng.permutation(3)) for _ in range(n)]
    x = np.zeros((n, 9), np.uint32)
    for i, p in enumerate(perms):
        for j in range(3):
            x[i, 3 * p[j] + j] = 1
    for exclusive in (False, True):
        y = oracle.scan_mat3(x, exclusive=exclusive)
        comp = (0, 1, 2)
        for i, p in enumerate(perms):
            if not exclusive:
                comp = tuple(p[comp[j]] for j in range(3))
            want = np.zeros(9, np.uint32)
            for j in range(3):
                want[3 * comp[j] + j] = 1
            assert np.array_equal(y[i], want), (exclusive, i)
            if exclusive:
                comp = tuple(p[comp[j]] for j in range(3))


def test_mat3_determinant_is_multiplicative():
    n = 1000
    x = si.uint32_full(18, 9 * n).reshape(n, 9)
    y = oracle.scan_mat3(x)
    M = 2**32

    def det(t):  # cofactor expansion along the first row
        a, b, c, d, e, f, g, h, k = (int(v) for v in t)
        return (a * (e * k - f * h) - b * (d * k - f * g) + c * (d * h - e * g)) % M
    acc = 1
    for i in range(n):
        acc = acc * det(x[i]) % M
        assert det(y[i]) == acc, i


# ---------------------------------------------------------------- CSR row offsets
# Building the CSR format is among the uses of a prefix sum listed in the
# introduction of "CUDA编程并行前缀和扫描详解"; its row pointer array has
# N + 1 entries ("UIUC ECE 408 应用并行编程", L09).

def test_csr_offsets_bruteforce():
    rng = np.random.default_rng(13)
    for n_rows, nnz in ((1, 0), (1, 5), (7, 30), (50, 200), (300, 40)):
        rows = rng.integers(0, n_rows + 3, nnz).astype(np.uint32)  # some out of range
        rp = oracle.csr_offsets(rows, n_rows)
        assert rp.shape == (n_rows + 1,)
        for r in range(n_rows + 1):
            assert int(rp[r]) == sum(1 for v in rows if int(v) < r), (n_rows, r)


def test_csr_offsets_closed_forms():
    # k entries in every row: row_ptr[r] = k * r
    n_rows, k = 1000, 7
    rows = np.repeat(np.arange(n_rows, dtype=np.uint32), k)
    np.testing.assert_array_equal(oracle.csr_offsets(rows, n_rows), k * np.arange(n_rows + 1))
    # sorted rows (with empty rows): row_ptr[r] is the first index whose row is >= r
    rows = np.sort(si.uint32_full(15, 20000) % 3000).astype(np.uint32)
    rp = oracle.csr_offsets(rows, 3000)
    np.testing.assert_array_equal(rp, np.searchsorted(rows, np.arange(3001), side="left"))
    # unsorted: the same offsets as the sorted indices
    perm = si.uint32_full(16, rows.size) .argsort(kind="stable")
    np.testing.assert_array_equal(oracle.csr_offsets(rows[perm], 3000), rp)
    # indices past the last row are not counted
    assert int(oracle.csr_offsets(np.array([0, 5, 9, 2], np.uint32), 5)[-1]) == 2
    np.testing.assert_array_equal(oracle.csr_offsets(np.zeros(0, np.uint32), 4), np.zeros(5, np.uint32))


# ---------------------------------------------------------------- radix-sort split pass
# "Lecture 7: 并行模式五 —— 前缀和 / 扫描", concept 2: radix sort splits by digit
# and places every element with a scan; a 32-bit key takes four 8-bit passes.

def test_radix_split_bruteforce():
    rng = np.random.default_rng(17)
    for n in (0, 1, 2, 9, 300):
        keys = rng.integers(0, 2**32, n, dtype=np.uint64).astype(np.uint32)
        vals = np.arange(n, dtype=np.uint32)
        for shift in (0, 8, 20, 24):
            ko, vo = oracle.radix_split(keys, shift, vals)
            digit = lambda k: (int(k) >> shift) & 255
            want = sorted(range(n), key=lambda i: (digit(keys[i]), i))  # stable by construction
            assert [int(v) for v in vo] == want
            assert [int(k) for k in ko] == [int(keys[i]) for i in want]


def test_radix_split_matches_stable_argsort():
    n = 100000
    keys = si.uint32_full(18, n) % np.uint32(5000)  # many equal keys and digits
    vals = si.uint32_full(19, n)
    for shift in (0, 4, 8):
        d = (keys >> np.uint32(shift)) & np.uint32(255)
        perm = np.argsort(d, kind="stable")
        ko, vo = oracle.radix_split(keys, shift, vals)
        np.testing.assert_array_equal(ko, keys[perm])
        np.testing.assert_array_equal(vo, vals[perm])
        ko2, none = oracle.radix_split(keys, shift)
        assert none is None
        np.testing.assert_array_equal(ko2, ko)


def test_radix_four_passes_sort():
    n = 50000
    keys = si.uint32_full(20, n)
    keys[::7] = keys[3]  # duplicates
    vals = np.arange(n, dtype=np.uint32)
    k, v = keys, vals
    for shift in (0, 8, 16, 24):
        k, v = oracle.radix_split(k, shift, v)
    np.testing.assert_array_equal(k, np.sort(keys))
    np.testing.assert_array_equal(v, np.argsort(keys, kind="stable"))
