"""Sequential CPU oracle for the device-wide prefix scan.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package.  The GPU library never calls it, and
the two share no code: the arithmetic lives in ``scan_oracle.c`` (plain C, one
left-to-right loop per definition, float sums in double), loaded here through
ctypes and wrapped for numpy arrays.

Pages cited:
  [L7]    "Lecture 7: 并行模式五 —— 前缀和 / 扫描：双缓冲与层次化算法"
          (UIUC ECE408 course notes, runguoli.com)
  [PMPP9] "第9章并行模式：前缀和 - Scan算法" (PMPP chapter 9 notes, bittern.cn)
  [YLY]   "CUDA编程并行前缀和扫描详解" (tutorial, m.youleyou.com)

Definitions: inclusive and exclusive scan [L7 concept 1; PMPP9 §9.1; YLY §2.1,
§2.2]; identities [PMPP9 §9.1 identity table]; compaction by an exclusive scan
of predicate flags [L7 concept 2; PMPP9 §9.6]; segmented scan [L7 concept 2,
radix-sort remark].  Every function here has a pin in tests/test_oracle.py
(worked examples printed on the pages, closed forms, invariants, brute force
on tiny inputs and special cases that reduce to numpy routines).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "scan_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

OPS = {"add": 0, "max": 1, "min": 2, "and": 3, "or": 4}

_lib = None


def build() -> str:
    """Compile scan_oracle.c with gcc into oracle/liboracle.so (always rebuilds)."""
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fPIC", "-shared",
           "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I = ctypes.c_int
    L = ctypes.c_int64
    sigs = {
        "oracle_scan_i32": [I, I, P, P, L],
        "oracle_scan_u32": [I, I, P, P, L],
        "oracle_scan_f32_add": [I, P, P, P, L],
        "oracle_scan_f32_minmax": [I, I, P, P, L],
        "oracle_scan_affine": [I, P, P, L],
        "oracle_scan_maxcount": [I, P, P, L],
        "oracle_scan_mat2": [I, P, P, L],
        "oracle_scan_mat3": [I, P, P, L],
        "oracle_csr_offsets": [P, L, ctypes.c_uint32, P],
        "oracle_radix_split": [P, P, L, ctypes.c_uint32, P, P],
        "oracle_segscan_i32": [I, I, P, P, P, L],
        "oracle_segscan_u32": [I, I, P, P, P, L],
        "oracle_segscan_f32_add": [I, P, P, P, P, L],
        "oracle_segscan_f32_minmax": [I, I, P, P, P, L],
        "oracle_compact_i32": [P, P, P, L],
        "oracle_compact_u32": [P, P, P, L],
        "oracle_compact_f32": [P, P, P, L],
    }
    for name, argtypes in sigs.items():
        fn = getattr(lib, name)
        fn.argtypes = argtypes
        fn.restype = L if name.startswith("oracle_compact") else None
    _lib = lib
    return lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _contig(x: np.ndarray, dtype) -> np.ndarray:
    x = np.asarray(x)
    if x.dtype != dtype:
        raise TypeError("expected %s, got %s" % (np.dtype(dtype), x.dtype))
    return np.ascontiguousarray(x)


def scan(op: str, x: np.ndarray, exclusive: bool = False):
    """Inclusive (default) or exclusive scan of a 1-D int32/uint32/float32 array;
    op in add, max, min, and (bitwise) or "and", "or" (bitwise, integers only).

    Returns y in the input dtype, except for float32 add, which returns the
    pair (y, s) of float64 arrays: y is the prefix sum accumulated in double
    and s the prefix sum of |x| over the same range (the tolerance scale).
    """
    lib = _load()
    x = np.asarray(x)
    n = x.shape[0]
    ex = 1 if exclusive else 0
    if x.dtype == np.int32:
        y = np.empty(n, np.int32)
        lib.oracle_scan_i32(OPS[op], ex, _ptr(_contig(x, np.int32)), _ptr(y), n)
        return y
    if x.dtype == np.uint32:
        y = np.empty(n, np.uint32)
        lib.oracle_scan_u32(OPS[op], ex, _ptr(_contig(x, np.uint32)), _ptr(y), n)
        return y
    if x.dtype == np.float32:
        if op in ("and", "or"):
            raise TypeError("bitwise scans take int32 or uint32")
        xc = _contig(x, np.float32)
        if op == "add":
            y = np.empty(n, np.float64)
            s = np.empty(n, np.float64)
            lib.oracle_scan_f32_add(ex, _ptr(xc), _ptr(y), _ptr(s), n)
            return y, s
        y = np.empty(n, np.float32)
        lib.oracle_scan_f32_minmax(OPS[op], ex, _ptr(xc), _ptr(y), n)
        return y
    raise TypeError("unsupported dtype %s" % x.dtype)


def scan_affine(ab: np.ndarray, exclusive: bool = False) -> np.ndarray:
    """Scan of affine maps; ab is an (n, 2) uint32 array of (a, b) pairs.

    Element i of an inclusive result is the composition of maps 0..i, the
    later map applied after the earlier: (a2,b2) o (a1,b1) = (a2*a1, a2*b1+b2)
    mod 2^32.  Its b component is the recurrence y_i = a_i*y_{i-1} + b_i.
    """
    lib = _load()
    ab = _contig(ab, np.uint32)
    if ab.ndim != 2 or ab.shape[1] != 2:
        raise ValueError("ab must have shape (n, 2)")
    n = ab.shape[0]
    y = np.empty((n, 2), np.uint32)
    lib.oracle_scan_affine(1 if exclusive else 0, _ptr(ab), _ptr(y), n)
    return y


def scan_maxcount(vc: np.ndarray, exclusive: bool = False) -> np.ndarray:
    """Scan of (value, count) pairs under the (maximum, occurrences) operator.

    vc is an (n, 2) int32 array: int32 values and counts (read as uint32).
    Element i of an inclusive result is (m, c) with m the largest value among
    elements 0..i and c the sum, mod 2^32, of the counts of the elements
    whose value is m.  The empty fold is (INT32_MIN, 0).
    """
    lib = _load()
    vc = _contig(vc.view(np.int32) if vc.dtype == np.uint32 else vc, np.int32)
    if vc.ndim != 2 or vc.shape[1] != 2:
        raise ValueError("vc must have shape (n, 2)")
    n = vc.shape[0]
    y = np.empty((n, 2), np.int32)
    lib.oracle_scan_maxcount(1 if exclusive else 0, _ptr(vc), _ptr(y), n)
    return y


def scan_mat2(x: np.ndarray, exclusive: bool = False) -> np.ndarray:
    """Scan of 2x2 uint32 matrices (rows of 4: a, b, c, d for [[a, b], [c, d]]).

    Element i of an inclusive result is X_i X_{i-1} ... X_0 mod 2^32, the
    later factor on the left; the empty product is the identity.
    """
    lib = _load()
    x = _contig(x, np.uint32)
    if x.ndim != 2 or x.shape[1] != 4:
        raise ValueError("x must have shape (n, 4)")
    n = x.shape[0]
    y = np.empty((n, 4), np.uint32)
    lib.oracle_scan_mat2(1 if exclusive else 0, _ptr(x), _ptr(y), n)
    return y


def scan_mat3(x: np.ndarray, exclusive: bool = False) -> np.ndarray:
    """Scan of 3x3 uint32 matrices, shape (n, 9) (row-major) or (n, 3, 3).

    Element i of an inclusive result is X_i X_{i-1} ... X_0 mod 2^32, the
    later factor on the left; the empty product is the identity.  Returns
    the shape it was given.
    """
    lib = _load()
    x = _contig(x, np.uint32)
    shape = x.shape
    if not ((x.ndim == 2 and x.shape[1] == 9) or (x.ndim == 3 and x.shape[1:] == (3, 3))):
        raise ValueError("x must have shape (n, 9) or (n, 3, 3)")
    n = x.shape[0]
    y = np.empty((n, 9), np.uint32)
    lib.oracle_scan_mat3(1 if exclusive else 0, _ptr(x), _ptr(y), n)
    return y.reshape(shape)


def csr_offsets(rows: np.ndarray, n_rows: int) -> np.ndarray:
    """CSR row pointers (n_rows + 1 uint32) of COO row indices: row_ptr[r] is
    the number of entries with row index < r; indices >= n_rows are ignored."""
    lib = _load()
    rows = _contig(rows, np.uint32)
    row_ptr = np.empty(n_rows + 1, np.uint32)
    lib.oracle_csr_offsets(_ptr(rows), rows.shape[0], n_rows, _ptr(row_ptr))
    return row_ptr


def radix_split(keys: np.ndarray, shift: int, vals: np.ndarray | None = None):
    """One stable radix-sort pass by the digit (key >> shift) & 255: returns
    (keys_out, vals_out or None)."""
    lib = _load()
    keys = _contig(keys, np.uint32)
    n = keys.shape[0]
    ko = np.empty(n, np.uint32)
    if vals is None:
        lib.oracle_radix_split(_ptr(keys), None, n, shift, _ptr(ko), None)
        return ko, None
    vals = _contig(vals, np.uint32)
    vo = np.empty(n, np.uint32)
    lib.oracle_radix_split(_ptr(keys), _ptr(vals), n, shift, _ptr(ko), _ptr(vo))
    return ko, vo


def segmented_scan(op: str, x: np.ndarray, heads: np.ndarray, exclusive: bool = False):
    """Segmented scan; heads is a uint8 array, nonzero starts a segment.

    Index 0 always starts a segment.  float32 add returns (y, s) in float64
    as scan() does, with s restarted at every head.
    """
    lib = _load()
    x = np.asarray(x)
    n = x.shape[0]
    h = _contig(heads, np.uint8)
    if h.shape[0] != n:
        raise ValueError("heads must have the length of x")
    ex = 1 if exclusive else 0
    if x.dtype == np.int32:
        y = np.empty(n, np.int32)
        lib.oracle_segscan_i32(OPS[op], ex, _ptr(_contig(x, np.int32)), _ptr(h), _ptr(y), n)
        return y
    if x.dtype == np.uint32:
        y = np.empty(n, np.uint32)
        lib.oracle_segscan_u32(OPS[op], ex, _ptr(_contig(x, np.uint32)), _ptr(h), _ptr(y), n)
        return y
    if x.dtype == np.float32:
        if op in ("and", "or"):
            raise TypeError("bitwise scans take int32 or uint32")
        xc = _contig(x, np.float32)
        if op == "add":
            y = np.empty(n, np.float64)
            s = np.empty(n, np.float64)
            lib.oracle_segscan_f32_add(ex, _ptr(xc), _ptr(h), _ptr(y), _ptr(s), n)
            return y, s
        y = np.empty(n, np.float32)
        lib.oracle_segscan_f32_minmax(OPS[op], ex, _ptr(xc), _ptr(h), _ptr(y), n)
        return y
    raise TypeError("unsupported dtype %s" % x.dtype)


def compact(x: np.ndarray):
    """Order-preserving compaction of the elements x > 0.

    Returns (out, count, pos): out holds the kept elements in input order,
    count their number, pos the exclusive scan of the 0/1 predicate flags.
    """
    lib = _load()
    x = np.asarray(x)
    n = x.shape[0]
    out = np.empty(n, x.dtype)
    pos = np.empty(n, np.uint32)
    fn = {np.dtype(np.int32): lib.oracle_compact_i32,
          np.dtype(np.uint32): lib.oracle_compact_u32,
          np.dtype(np.float32): lib.oracle_compact_f32}.get(x.dtype)
    if fn is None:
        raise TypeError("unsupported dtype %s" % x.dtype)
    xc = np.ascontiguousarray(x)
    count = int(fn(_ptr(xc), _ptr(out), _ptr(pos), n))
    return out[:count].copy(), count, pos
