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


def test_full_range_generators():
    n = 1 << 20
    u = si.uint32_full(9, n)
    assert u.dtype == np.uint32
    assert u.min() < (1 << 20) and u.max() > 0xFFFFFFFF - (1 << 20)
    assert abs(u.astype(np.float64).mean() / 2.0**32 - 0.5) < 0.01
    # each of the four bytes is uniform over 0..255 (radix digits)
    for shift in (0, 8, 16, 24):
        counts = np.bincount((u >> np.uint32(shift)) & np.uint32(255), minlength=256)
        assert counts.min() > 0.9 * n / 256 and counts.max() < 1.1 * n / 256
    i = si.int32_full(9, n)
    assert np.array_equal(i.view(np.uint32), u)  # same draws, reinterpreted
    s = si.float32_sym(10, n)
    assert s.min() >= -1.0 and s.max() < 1.0 and abs(s.mean()) < 0.01
    assert np.all(s * np.float32(2.0**23) == np.round(s * np.float32(2.0**23)))  # on the 2^-23 grid


def test_pair_and_matrix_generators():
    n = 1 << 18
    mc = si.maxcount_pairs(11, n, span=50)
    assert mc.shape == (n, 2) and mc.dtype == np.int32
    assert mc[:, 0].min() == -50 and mc[:, 0].max() == 50 and np.all(mc[:, 1] == 1)
    mw = si.maxcount_pairs(11, n, span=50, unit_counts=False)
    assert np.array_equal(mw[:, 0], mc[:, 0])  # the values do not depend on the count mode
    assert len(np.unique(mw[:, 1])) > n // 2
    m = si.mat2_elems(12, n)
    assert m.shape == (n, 4) and m.dtype == np.uint32
    assert np.array_equal(m.reshape(-1), si.uint32_full(12, 4 * n))
    for seed in (11, 12):  # reproducible call to call
        assert np.array_equal(si.maxcount_pairs(seed, 1000), si.maxcount_pairs(seed, 1000))
    assert np.array_equal(si.mat2_elems(12, 1000), si.mat2_elems(12, 1000))
    m3 = si.mat3_elems(19, 1000)
    assert m3.shape == (1000, 9) and m3.dtype == np.uint32
    assert np.array_equal(m3.reshape(-1), si.uint32_full(19, 9000))
