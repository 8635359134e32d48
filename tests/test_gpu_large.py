"""Inputs past 2^32 elements (and compaction/radix at their 2^32 - 1 limits).

Element indices, tile numbers times tile sizes, output positions and the
look-back carries must not wrap at 32 bits.  The oracle would need minutes
and tens of GB of host memory at these sizes, so the inputs are chosen so
that every output element has a closed form, from the definitions of the
pages: the inclusive scan of ones is y[i] = i + 1 and the exclusive one y[i] = i
("Lecture 7: 并行模式五 —— 前缀和 / 扫描", concept 1), here wrapped modulo 2^32 for
int32; compaction keeps the positive elements in order at the positions the
exclusive scan of the flags gives (concept 2); a stable split of the keys
0, 1, 2, ... by their low byte lists, for each digit in turn, the keys with
that low byte in increasing order.  Every output element is checked, on the
GPU, chunk by chunk.
"""
import pytest
import torch

import device_wide_prefix_tile_amd as dw

pytestmark = pytest.mark.gpu

CHUNK = 1 << 27


@pytest.fixture(autouse=True)
def fresh():
    yield
    torch.cuda.empty_cache()


class Mode:
    def __init__(self, mode):
        self.mode = mode

    def __enter__(self):
        self.old = dw.scan_set_multi_tile_mode(self.mode)

    def __exit__(self, *a):
        dw.scan_set_multi_tile_mode(self.old)


def wrap_i32(v: torch.Tensor) -> torch.Tensor:
    """int64 -> int32 modulo 2^32 (two's complement)."""
    return (((v + (1 << 31)) % (1 << 32)) - (1 << 31)).to(torch.int32)


def check_chunks(y: torch.Tensor, expected, what: str):
    n = y.shape[0]
    for s in range(0, n, CHUNK):
        e = min(n, s + CHUNK)
        want = expected(torch.arange(s, e, dtype=torch.int64, device=y.device))
        got = y[s:e]
        if not torch.equal(got, want):
            bad = torch.nonzero(got != want)[0].item()
            raise AssertionError("%s: first mismatch at %d: got %r, want %r" % (
                what, s + bad, got[bad].item(), want[bad].item()))


@pytest.mark.parametrize("mode", [0, 1, 3])
def test_int32_add_past_2p32(mode):
    n = (1 << 32) + 12347  # 279,622 tiles of 15,360; last one ragged
    print("int32 add of ones, n=%d, mode %d" % (n, mode), flush=True)
    x = torch.ones(n, dtype=torch.int32, device="cuda")
    with Mode(mode):
        y = dw.scan_inclusive(x, "add")
        check_chunks(y, lambda i: wrap_i32(i + 1), "inclusive mode %d" % mode)
        dw.scan_exclusive(x, "add", out=y)
        check_chunks(y, wrap_i32, "exclusive mode %d" % mode)
    assert dw.scan_get_device_error() == 0


def test_float32_add_past_2p32():
    """The inter-tile carry is kept in double: y[i] must be i + 1 rounded to float32 once
    (within the pages' float tolerance 1e-5 * prefix|x| + 1e-6)."""
    n = (1 << 32) + 12347
    print("float32 add of ones, n=%d" % n, flush=True)
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = dw.scan_inclusive(x, "add")
    for s in range(0, n, CHUNK):
        e = min(n, s + CHUNK)
        want = torch.arange(s + 1, e + 1, dtype=torch.float64, device="cuda")
        err = (y[s:e].to(torch.float64) - want).abs()
        assert bool((err <= 1e-5 * want + 1e-6).all()), "float32 add chunk at %d" % s
    assert dw.scan_get_device_error() == 0


def test_compaction_at_limit():
    """n = 2^32 - 1, the largest compaction: keep every third element."""
    n = (1 << 32) - 1
    print("int32 compaction, n=%d" % n, flush=True)
    x = torch.empty(n, dtype=torch.int32, device="cuda")
    for s in range(0, n, CHUNK):
        e = min(n, s + CHUNK)
        i = torch.arange(s, e, dtype=torch.int64, device="cuda")
        # positive (and distinct modulo 2^31) on multiples of 3, else 0: not kept
        x[s:e] = torch.where(i % 3 == 0, (i & 0x7FFFFFFF) | 1, torch.zeros_like(i)).to(torch.int32)
    out = torch.empty_like(x)
    out, cnt = dw.compact(x, out=out)
    torch.cuda.synchronize()
    kept = (n + 2) // 3
    assert int(cnt.cpu().numpy()[0]) == kept
    check_chunks(out[:kept], lambda j: (((3 * j) & 0x7FFFFFFF) | 1).to(torch.int32), "compaction")
    assert dw.scan_get_device_error() == 0


def test_radix_split_at_limit():
    """n = 2^32 - 256 keys 0, 1, 2, ...: the split by the low byte puts, for digit d, the
    2^24 - 1 keys j * 256 + d (j ascending) at positions d * (2^24 - 1) + j."""
    n = (1 << 32) - 256
    m = n // 256
    print("radix split of ascending keys, n=%d" % n, flush=True)
    keys = torch.empty(n, dtype=torch.int32, device="cuda")
    for s in range(0, n, CHUNK):
        e = min(n, s + CHUNK)
        keys[s:e] = wrap_i32(torch.arange(s, e, dtype=torch.int64, device="cuda"))
    keys = keys.view(torch.uint32)
    ko, _ = dw.radix_split(keys, 0)
    check_chunks(ko.view(torch.int32), lambda k: wrap_i32((k % m) * 256 + k // m), "low byte")
    # the top byte of ascending keys is already in order: the split leaves them in place
    dw.radix_split(keys, 24, keys_out=ko)
    check_chunks(ko.view(torch.int32), wrap_i32, "top byte")
