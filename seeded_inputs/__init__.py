"""Seeded synthetic inputs shared by the oracle checks, the GPU tests and the bench.

This module only draws random numbers; it holds none of the scan's arithmetic.
Every array comes from SplitMix64 (Steele, Lea and Flood, "Fast splittable
pseudorandom number generators", OOPSLA 2014), written here from its published
definition: the i-th draw of a generator seeded with ``s`` is
``mix(s + (i + 1) * 0x9E3779B97F4A7C15)`` with the 64-bit finaliser

    z ^= z >> 30; z *= 0xBF58476D1CE4E5B9
    z ^= z >> 27; z *= 0x94D049BB133111EB
    z ^= z >> 31

Independent streams of one seed use ``s`` mixed with a stream number.

Workload recipes (the shapes and value distributions of the scan workloads):
  * int32 uniform in [0, 15]           -> top 4 bits of the draw
  * float32 uniform in [0, 1)          -> top 24 bits times 2^-24 (exact)
  * float32 ~ N(0, 1)                  -> Box-Muller in double, rounded to float
  * uint32 affine pairs (a, b)         -> low / high halves of one draw
  * int32 uniform in [-100, 100]       -> draw mod 201 - 100
  * segment heads, mean length L       -> head[i] = draw < 2^64 / L, head[0] = 1;
    i.i.d. Bernoulli(1/L) heads give Geometric(1/L) segment lengths (mean L)
  * int32 uniform over the full range  -> low 32 bits of the draw
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_CHUNK = 1 << 22
_THREADS = max(1, min(16, os.cpu_count() or 1))


def _parallel(n: int, work) -> None:
    """Run work(c0, c1) over [0, n) in chunks on a thread pool (numpy releases the GIL)."""
    spans = [(c0, min(n, c0 + _CHUNK)) for c0 in range(0, n, _CHUNK)]
    if len(spans) <= 1:
        for c0, c1 in spans:
            work(c0, c1)
        return
    with ThreadPoolExecutor(_THREADS) as ex:
        for f in [ex.submit(work, c0, c1) for c0, c1 in spans]:
            f.result()


def _mix(z: np.ndarray) -> np.ndarray:
    z ^= z >> np.uint64(30)
    z *= _M1
    z ^= z >> np.uint64(27)
    z *= _M2
    z ^= z >> np.uint64(31)
    return z


def _stream_seed(seed: int, stream: int) -> np.uint64:
    s = np.array([(seed * 0x9E3779B97F4A7C15 + stream * 0xD1B54A32D192ED03) & (2**64 - 1)],
                 dtype=np.uint64)
    return _mix(s)[0]


def _draws_span(s: np.uint64, start: int, count: int) -> np.ndarray:
    ctr = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    ctr *= GAMMA
    ctr += s
    return _mix(ctr)


def draws(seed: int, n: int, stream: int = 0, start: int = 0) -> np.ndarray:
    """n consecutive 64-bit SplitMix64 draws (counter start..start+n-1)."""
    s = _stream_seed(seed, stream)
    out = np.empty(n, np.uint64)

    def work(c0, c1):
        out[c0:c1] = _draws_span(s, start + c0, c1 - c0)
    _parallel(n, work)
    return out


def _map_chunks(seed: int, n: int, stream: int, dtype, fn) -> np.ndarray:
    s = _stream_seed(seed, stream)
    out = np.empty(n, dtype)

    def work(c0, c1):
        out[c0:c1] = fn(_draws_span(s, c0, c1 - c0))
    _parallel(n, work)
    return out


def int32_0_15(seed: int, n: int) -> np.ndarray:
    """int32 uniform in [0, 15]."""
    return _map_chunks(seed, n, 0, np.int32, lambda u: (u >> np.uint64(60)).astype(np.int32))


def float32_01(seed: int, n: int) -> np.ndarray:
    """float32 uniform in [0, 1) on the 2^-24 grid."""
    return _map_chunks(seed, n, 0, np.float32,
                       lambda u: ((u >> np.uint64(40)).astype(np.float64) * 2.0**-24).astype(np.float32))


def float32_normal(seed: int, n: int) -> np.ndarray:
    """float32 ~ N(0,1), Box-Muller on two independent uniform streams."""
    s1, s2 = _stream_seed(seed, 1), _stream_seed(seed, 2)
    out = np.empty(n, np.float32)

    def work(c0, c1):
        u1 = ((_draws_span(s1, c0, c1 - c0) >> np.uint64(11)).astype(np.float64) + 0.5) * 2.0**-53
        u2 = (_draws_span(s2, c0, c1 - c0) >> np.uint64(11)).astype(np.float64) * 2.0**-53
        out[c0:c1] = (np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * np.pi * u2)).astype(np.float32)
    _parallel(n, work)
    return out


def affine_pairs(seed: int, n: int, odd_a: bool = False) -> np.ndarray:
    """(n, 2) uint32 pairs (a, b); with odd_a the multipliers are forced odd."""
    s = _stream_seed(seed, 0)
    out = np.empty((n, 2), np.uint32)

    def work(c0, c1):
        u = _draws_span(s, c0, c1 - c0)
        a = (u & np.uint64(0xFFFFFFFF)).astype(np.uint32)
        if odd_a:
            a |= np.uint32(1)
        out[c0:c1, 0] = a
        out[c0:c1, 1] = (u >> np.uint64(32)).astype(np.uint32)
    _parallel(n, work)
    return out


def int32_pm100(seed: int, n: int) -> np.ndarray:
    """int32 uniform in [-100, 100]."""
    return _map_chunks(seed, n, 0, np.int32,
                       lambda u: ((u % np.uint64(201)).astype(np.int64) - 100).astype(np.int32))


def segment_heads(seed: int, n: int, mean_len: float = 1000.0) -> np.ndarray:
    """uint8 head flags with i.i.d. Bernoulli(1/mean_len) heads and head[0] = 1."""
    thr = np.uint64(int(2.0**64 / mean_len))
    h = _map_chunks(seed, n, 3, np.uint8, lambda u: (u < thr).astype(np.uint8))
    if n:
        h[0] = 1
    return h


def int32_full(seed: int, n: int) -> np.ndarray:
    """int32 uniform over the whole 32-bit range."""
    return _map_chunks(seed, n, 0, np.int32,
                       lambda u: (u & np.uint64(0xFFFFFFFF)).astype(np.uint32).view(np.int32))


def uint32_full(seed: int, n: int) -> np.ndarray:
    """uint32 uniform over the whole 32-bit range."""
    return _map_chunks(seed, n, 0, np.uint32,
                       lambda u: (u & np.uint64(0xFFFFFFFF)).astype(np.uint32))


def float32_sym(seed: int, n: int) -> np.ndarray:
    """float32 uniform in [-1, 1) on the 2^-23 grid."""
    return _map_chunks(seed, n, 0, np.float32,
                       lambda u: ((u >> np.uint64(40)).astype(np.float64) * 2.0**-23 - 1.0).astype(np.float32))


def maxcount_pairs(seed: int, n: int, span: int = 1000, unit_counts: bool = True) -> np.ndarray:
    """(n, 2) int32 pairs (value, count): values uniform in [-span, span] (so
    that the running maximum ties often), counts 1, or with unit_counts False
    uniform uint32 (stored as int32 bits)."""
    s = _stream_seed(seed, 0)
    out = np.empty((n, 2), np.int32)

    def work(c0, c1):
        u = _draws_span(s, c0, c1 - c0)
        out[c0:c1, 0] = ((u >> np.uint64(32)) % np.uint64(2 * span + 1)).astype(np.int64) - span
        if unit_counts:
            out[c0:c1, 1] = 1
        else:
            out[c0:c1, 1] = (u & np.uint64(0xFFFFFFFF)).astype(np.uint32).view(np.int32)
    _parallel(n, work)
    return out


def mat2_elems(seed: int, n: int) -> np.ndarray:
    """(n, 4) uint32: 2x2 matrices [[a, b], [c, d]] stored (a, b, c, d), entries uniform."""
    return uint32_full(seed, 4 * n).reshape(n, 4)


def mat3_elems(seed: int, n: int) -> np.ndarray:
    """(n, 9) uint32: 3x3 matrices stored row-major, entries uniform."""
    return uint32_full(seed, 9 * n).reshape(n, 9)
