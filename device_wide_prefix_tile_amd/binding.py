"""Thin ctypes binding of libdwpt_scan.so for torch tensors.

Argument marshalling only: every step of the scan runs in the HIP kernels of
the library.  The functions carry the C ABI's names (dwpt_scan.h); they take
torch tensors on the current CUDA (HIP) device, enqueue on the current torch
stream and return without synchronising.  There is no CPU fallback: if the
library cannot be loaded, every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

from . import build as _build

SCAN_OK, SCAN_ERR_INVALID, SCAN_ERR_UNSUPPORTED, SCAN_ERR_NOMEM, SCAN_ERR_HIP, SCAN_ERR_TIMEOUT = range(6)
SCAN_SMALL_N_AUTO = (1 << 64) - 1  # scan_set_small_n_max: one tile of the operation's shape
OPS = {"add": 0, "max": 1, "min": 2, "affine": 3, "maxcount": 4, "mat2": 5, "mat3": 6, "and": 7, "or": 8}
SCAN_I32, SCAN_U32, SCAN_F32, SCAN_U32X2, SCAN_I32_U32, SCAN_U32X4, SCAN_U32X9 = range(7)
_DTYPES = {torch.int32: SCAN_I32, torch.uint32: SCAN_U32, torch.float32: SCAN_F32}

EXPORTS = ("scan_inclusive", "scan_exclusive", "segmented_scan", "compact", "scan_status_string",
           "scan_get_device_error", "scan_release_workspace", "scan_set_small_n_max",
           "scan_set_spin_limit", "scan_set_multi_tile_mode", "scan_copy_probe", "csr_row_offsets",
           "radix_split", "scan_noalloc")

_lib = None


class ScanError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__("%s failed: %s (status %d)" % (what, status_string(status), status))


def lib() -> ctypes.CDLL:
    """The loaded library (built in-tree first if it is not there yet)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_build.LIB_PATH):
        _build.build()
    L = ctypes.CDLL(_build.LIB_PATH)
    P, S, I, U = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_uint32
    sig = {
        "scan_inclusive": ([I, I, P, P, S, P], I),
        "scan_exclusive": ([I, I, P, P, S, P], I),
        "segmented_scan": ([I, I, P, P, P, S, I, P], I),
        "compact": ([I, P, P, P, S, P], I),
        "scan_status_string": ([I], ctypes.c_char_p),
        "scan_get_device_error": ([P], I),
        "scan_release_workspace": ([], I),
        "scan_set_small_n_max": ([S], S),
        "scan_set_spin_limit": ([U], U),
        "scan_set_multi_tile_mode": ([I], I),
        "scan_copy_probe": ([P, P, S, P], I),
        "csr_row_offsets": ([P, S, U, P, P], I),
        "radix_split": ([P, P, S, U, P, P, P], I),
        "scan_noalloc": ([I, I, P, P, S, I, P], I),
    }
    for name, (argtypes, restype) in sig.items():
        fn = getattr(L, name)
        fn.argtypes = argtypes
        fn.restype = restype
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().scan_status_string(int(status)).decode()


scan_status_string = status_string


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream) -> int:
    """Handle of `stream` (a torch stream or a raw handle); None: the current device's current
    stream, read without building a torch Stream object (which costs more than a launch)."""
    if stream is None:
        if _raw_stream is not None:
            return _raw_stream(torch.cuda.current_device())
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check(status: int, what: str):
    if status != SCAN_OK:
        raise ScanError(status, what)


def _dtype_code(x: torch.Tensor, op: str) -> int:
    if op == "affine":
        if x.dtype not in (torch.int32, torch.uint32) or x.dim() != 2 or x.shape[1] != 2:
            raise TypeError("affine scans take an (n, 2) int32/uint32 tensor of (a, b) pairs")
        return SCAN_U32X2
    if op == "maxcount":
        if x.dtype not in (torch.int32, torch.uint32) or x.dim() != 2 or x.shape[1] != 2:
            raise TypeError("maxcount scans take an (n, 2) int32 tensor of (value, count) pairs")
        return SCAN_I32_U32
    if op == "mat2":
        if x.dtype not in (torch.int32, torch.uint32) or x.dim() != 2 or x.shape[1] != 4:
            raise TypeError("mat2 scans take an (n, 4) uint32 tensor of [[a, b], [c, d]] as (a, b, c, d)")
        return SCAN_U32X4
    if op == "mat3":
        if x.dtype not in (torch.int32, torch.uint32) or not (
                (x.dim() == 2 and x.shape[1] == 9) or (x.dim() == 3 and tuple(x.shape[1:]) == (3, 3))):
            raise TypeError("mat3 scans take an (n, 9) or (n, 3, 3) uint32 tensor of row-major 3x3 matrices")
        return SCAN_U32X9
    if x.dtype not in _DTYPES:
        raise TypeError("unsupported dtype %s" % x.dtype)
    if op in ("and", "or") and x.dtype == torch.float32:
        raise TypeError("bitwise scans take int32 or uint32")
    return _DTYPES[x.dtype]


def _prep(x: torch.Tensor, out):
    if not x.is_cuda:
        raise ValueError("input must be a device tensor")
    if not x.is_contiguous():
        raise ValueError("input must be contiguous")
    if out is None:
        out = torch.empty_like(x)
    elif out.shape != x.shape or out.dtype != x.dtype or not out.is_contiguous() or not out.is_cuda:
        raise ValueError("out must be a contiguous device tensor shaped like the input")
    return out


def scan_inclusive(x: torch.Tensor, op: str = "add", out: torch.Tensor | None = None, stream=None):
    """out[i] = x[0] (+) ... (+) x[i]; op in add/max/min/and/or (1-D), affine or maxcount ((n, 2)
    pairs), mat2 ((n, 4) matrices), mat3 ((n, 9) or (n, 3, 3) matrices)."""
    dt = _dtype_code(x, op)
    out = _prep(x, out)
    _check(lib().scan_inclusive(OPS[op], dt, x.data_ptr(), out.data_ptr(), x.shape[0], _stream(stream)),
           "scan_inclusive")
    return out


def scan_exclusive(x: torch.Tensor, op: str = "add", out: torch.Tensor | None = None, stream=None):
    """out[0] = identity, out[i] = x[0] (+) ... (+) x[i-1]."""
    dt = _dtype_code(x, op)
    out = _prep(x, out)
    _check(lib().scan_exclusive(OPS[op], dt, x.data_ptr(), out.data_ptr(), x.shape[0], _stream(stream)),
           "scan_exclusive")
    return out


def scan_noalloc(x: torch.Tensor, op: str = "add", exclusive: bool = False, out: torch.Tensor | None = None,
                 stream=None):
    """scan_inclusive / scan_exclusive without any device allocation by the library (its status
    words live in a static per-GPU array; calls overlapping on one GPU race).  `out` must be
    given by callers that cannot allocate."""
    dt = _dtype_code(x, op)
    out = _prep(x, out)
    _check(lib().scan_noalloc(OPS[op], dt, x.data_ptr(), out.data_ptr(), x.shape[0], 1 if exclusive else 0,
                              _stream(stream)), "scan_noalloc")
    return out


def segmented_scan(x: torch.Tensor, heads: torch.Tensor, op: str = "add", exclusive: bool = False,
                   out: torch.Tensor | None = None, stream=None):
    """Scan restarted at every nonzero head flag (uint8 tensor); x[0] always starts a segment."""
    if op not in ("add", "max", "min"):
        raise ValueError("segmented scans take add, max or min")
    dt = _dtype_code(x, op)
    if heads.dtype != torch.uint8 or heads.shape != x.shape or not heads.is_contiguous() or not heads.is_cuda:
        raise ValueError("heads must be a contiguous uint8 device tensor shaped like x")
    out = _prep(x, out)
    _check(lib().segmented_scan(OPS[op], dt, x.data_ptr(), heads.data_ptr(), out.data_ptr(), x.shape[0],
                                1 if exclusive else 0, _stream(stream)), "segmented_scan")
    return out


def csr_row_offsets(rows: torch.Tensor, n_rows: int, out: torch.Tensor | None = None, stream=None):
    """CSR row pointers of COO row indices: out[r] = #entries with row < r, r = 0 .. n_rows
    (n_rows + 1 values; indices >= n_rows are not counted).  rows: 1-D int32/uint32 device tensor."""
    if rows.dtype not in (torch.int32, torch.uint32) or rows.dim() != 1:
        raise TypeError("rows must be a 1-D int32/uint32 tensor")
    if not rows.is_cuda or not rows.is_contiguous():
        raise ValueError("rows must be a contiguous device tensor")
    if not 0 <= n_rows < 2**32 - 1:
        raise ValueError("n_rows out of range")
    if out is None:
        out = torch.empty(n_rows + 1, dtype=torch.uint32, device=rows.device)
    elif out.shape != (n_rows + 1,) or out.dtype not in (torch.int32, torch.uint32) or not out.is_contiguous():
        raise ValueError("out must be a contiguous (n_rows + 1,) int32/uint32 tensor")
    _check(lib().csr_row_offsets(rows.data_ptr(), rows.shape[0], n_rows, out.data_ptr(), _stream(stream)),
           "csr_row_offsets")
    return out


def _u32_vector(x: torch.Tensor, name: str):
    if x.dtype not in (torch.int32, torch.uint32) or x.dim() != 1:
        raise TypeError("%s must be a 1-D int32/uint32 tensor" % name)
    if not x.is_cuda or not x.is_contiguous():
        raise ValueError("%s must be a contiguous device tensor" % name)


def radix_split(keys: torch.Tensor, shift: int, vals: torch.Tensor | None = None,
                keys_out: torch.Tensor | None = None, vals_out: torch.Tensor | None = None, stream=None):
    """One stable radix-sort pass by the digit (key >> shift) & 255 of uint32 keys.

    Returns (keys_out, vals_out); vals_out is None when vals is None.  Outputs are
    allocated when not given and must not overlap the inputs."""
    _u32_vector(keys, "keys")
    n = keys.shape[0]
    if not 0 <= shift <= 31:
        raise ValueError("shift must be in 0 .. 31")
    if keys_out is None:
        keys_out = torch.empty_like(keys)
    _u32_vector(keys_out, "keys_out")
    if keys_out.shape[0] != n:
        raise ValueError("keys_out must hold n keys")
    vp = vop = None
    if vals is not None:
        _u32_vector(vals, "vals")
        if vals.shape[0] != n:
            raise ValueError("vals must hold n values")
        if vals_out is None:
            vals_out = torch.empty_like(vals)
        _u32_vector(vals_out, "vals_out")
        if vals_out.shape[0] != n:
            raise ValueError("vals_out must hold n values")
        vp, vop = vals.data_ptr(), vals_out.data_ptr()
    elif vals_out is not None:
        raise ValueError("vals_out given without vals")
    _check(lib().radix_split(keys.data_ptr(), vp, n, shift, keys_out.data_ptr(), vop, _stream(stream)),
           "radix_split")
    return keys_out, vals_out


def compact(x: torch.Tensor, out: torch.Tensor | None = None, count: torch.Tensor | None = None,
            stream=None):
    """Keeps x > 0 in order: returns (out, count) with out[:count] the kept elements.

    count is a 1-element uint32 device tensor; read it after synchronising.
    """
    dt = _dtype_code(x, "add")
    out = _prep(x, out)
    if count is None:
        count = torch.zeros(1, dtype=torch.uint32, device=x.device)
    _check(lib().compact(dt, x.data_ptr(), out.data_ptr(), count.data_ptr(), x.shape[0], _stream(stream)),
           "compact")
    return out, count


def scan_get_device_error(stream=None) -> int:
    return int(lib().scan_get_device_error(_stream(stream)))


def scan_release_workspace():
    _check(lib().scan_release_workspace(), "scan_release_workspace")


def scan_set_small_n_max(n_max: int) -> int:
    return int(lib().scan_set_small_n_max(int(n_max)))


def scan_set_multi_tile_mode(mode: int) -> int:
    """0: by size (default); 1: one workgroup per tile; 2: persistent pipelined kernel;
    3: reduce-then-scan (three launches)."""
    return int(lib().scan_set_multi_tile_mode(int(mode)))


def scan_set_spin_limit(polls: int) -> int:
    return int(lib().scan_set_spin_limit(int(polls)))


def scan_copy_probe(src: torch.Tensor, dst: torch.Tensor, stream=None):
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < nbytes:
        raise ValueError("dst too small")
    _check(lib().scan_copy_probe(src.data_ptr(), dst.data_ptr(), nbytes, _stream(stream)), "scan_copy_probe")
    return dst
