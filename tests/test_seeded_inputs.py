"""Host-side checks of the seeded input generator (no GPU).

The generator is shared input plumbing, not part of what is checked; these
tests make sure its draws have the stated shape (moments, support, outlier
rate) and that any window of a tensor can be regenerated on its own.
"""

import numpy as np

import seeded_inputs as S


def test_window_regeneration_and_threads():
    a = S.host_f32(300_000, 17, S.GRAD, 3, 5, 0, 1e-3)
    b = S.host_f32(1000, 17, S.GRAD, 3, 5, 123_456, 1e-3)
    assert np.array_equal(a[123_456:124_456], b)
    c = S.host_bf16(300_000, 17, S.GRAD, 3, 5, 0, 1e-3)
    assert np.array_equal(c, (a.view(np.uint32) + 0x7FFF + ((a.view(np.uint32) >> 16) & 1)) >> 16)


def test_keys_are_distinct():
    base = S.host_f32(4096, 1, S.GRAD, 1, 0, 0, 1.0)
    for args in [(2, S.GRAD, 1, 0), (1, S.MASTER, 1, 0), (1, S.GRAD, 2, 0), (1, S.GRAD, 1, 1)]:
        other = S.host_f32(4096, args[0], args[1], args[2], args[3], 0, 1.0)
        assert abs(np.corrcoef(base, other)[0, 1]) < 0.05


def test_moments_support_and_outliers():
    z = S.host_f32(1 << 22, 3, S.GRAD, 1, 0, 0, 1.0).astype(np.float64)
    assert abs(z.mean()) < 3e-3 and abs(z.std() - 1) < 3e-3
    # Irwin-Hall(12): excess kurtosis -0.1, support [-6, 6]
    k = ((z - z.mean()) ** 4).mean() / z.var() ** 2
    assert abs(k - 2.9) < 0.02 and np.abs(z).max() <= 6
    w = S.by_name("gpt2-small-flat")
    g = S.host_f32(1 << 20, w.seed, S.GRAD, 1, 0, 0, w.grad_sigma, outliers=True)
    frac = np.mean(np.abs(g) > 8 * w.grad_sigma)
    assert 0.006 < frac < 0.011
    v = S.host_f32(1 << 16, 9, S.VAR, 0, 0, 0, 1e-6, kind=S.KIND_ABS)
    assert v.min() >= 0


def test_workload_geometry():
    sizes = {w.name: (w.shard_len, w.n_d) for w in S.WORKLOADS}
    assert sizes["tiny-zero1"] == (262_144, 4)
    assert sizes["gpt2-small-flat"] == (15_554_976, 8)
    assert sizes["7.5B-nd64"] == (117_187_500, 64)
    assert sizes["13B-nd16-clip-int8"] == (812_500_000, 16)
    w4 = S.by_name(4)
    assert w4.phi == 40 * (4 * 5120 * 5120 + 3 * 5120 * 13824) + 32000 * 5120
    assert w4.phi == 12_851_609_600 and all(s % 128 == 0 for _, s in w4.segments)
    assert [w.bytes_per_param() for w in S.WORKLOADS[:3]] == [34, 42, 154]


def test_int8_contributions_shape_and_windows():
    w = S.by_name("7.5B-nd64-zeropp")
    c, s = S.host_contrib_q8(w, 2, 0, 256 * 40)
    assert c.dtype == np.int8 and c.shape == (64, 256 * 40) and s.shape == (64, 40)
    assert abs(c.astype(np.float64).std() - 32) < 0.5 and np.abs(c).max() <= 127
    assert (s >= 0).all() and abs(s.mean() / (w.scale_sigma * 0.7979) - 1) < 0.05
    c2, s2 = S.host_contrib_q8(w, 2, 256 * 7, 256 * 3 + 5)
    assert np.array_equal(c2, c[:, 256 * 7: 256 * 10 + 5])
    assert np.array_equal(s2, s[:, 7:11])
