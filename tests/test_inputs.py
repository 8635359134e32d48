"""Checks of the seeded input generators (no GPU)."""
import numpy as np

import seeded_inputs as si


def test_splitmix64_published_vector():
    # first three outputs of SplitMix64 seeded with 0
    z = np.array([1, 2, 3], np.uint64) * si.GAMMA
    out = si._mix(z)
    assert [hex(int(v)) for v in out] == ["0xe220a8397b1dcdaf", "0x6e789e6aa1b965f4", "0x6c45d188009454f"]


def test_deterministic_and_chunk_independent():
    a = si.draws(7, 5000000)
    b = np.concatenate([si.draws(7, 3000000), si.draws(7, 2000000, start=3000000)])
    np.testing.assert_array_equal(a, b)
    assert not np.array_equal(si.draws(7, 100), si.draws(8, 100))
    assert not np.array_equal(si.draws(7, 100, stream=1), si.draws(7, 100))


def test_distributions():
    n = 1 << 20
    x = si.int32_0_15(1, n)
    assert x.min() == 0 and x.max() == 15 and abs(x.mean() - 7.5) < 0.05
    f = si.float32_01(2, n)
    assert f.min() >= 0.0 and f.max() < 1.0 and abs(f.mean() - 0.5) < 0.01
    g = si.float32_normal(3, n)
    assert abs(g.mean()) < 0.01 and abs(g.std() - 1.0) < 0.01
    assert abs((g > 0).mean() - 0.5) < 0.01
    v = si.int32_pm100(5, n)
    assert v.min() == -100 and v.max() == 100
    h = si.segment_heads(5, n, 1000.0)
    assert h[0] == 1
    mean_len = n / h.sum()
    assert 900 < mean_len < 1100
    ab = si.affine_pairs(4, 1000, odd_a=True)
    assert np.all(ab[:, 0] & 1)
