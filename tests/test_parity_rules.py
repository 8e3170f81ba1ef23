"""The comparison rules the GPU parity tests apply, checked on the CPU with
hand-made arrays: what passes, what must fail, and the diagnostics."""

import numpy as np
import pytest

from tests import _parity as P


def _f32(*xs):
    return np.array(xs, dtype=np.float32)


def test_f32_equal_bits_pass_with_full_diagnostics():
    a = np.random.default_rng(0).standard_normal(1000).astype(np.float32)
    r = P.f32_close("a", a, a.copy())
    assert r == {"bitwise": 1.0, "max_rel": 0.0, "ulp_hist": {"0": 1000, "1": 0, "2+": 0},
                 "rtol_only_out": 0}


def test_f32_one_ulp_and_signed_zero_and_nan():
    o = _f32(1.0, 0.0, np.nan, 3.0)
    g = o.copy()
    g[0] = np.nextafter(np.float32(1.0), np.float32(2.0))  # 1 ulp
    g[1] = np.float32(-0.0)                                 # other bits, same value
    g[2] = np.frombuffer(np.uint32(0x7FC00001).tobytes(), np.float32)[0]  # other NaN
    r = P.f32_close("x", g, o)
    assert r["ulp_hist"] == {"0": 3, "1": 1, "2+": 0}
    assert r["bitwise"] == pytest.approx(0.25)
    assert r["max_rel"] == pytest.approx(2.0 ** -23)


def test_f32_tolerance_is_abs_floor_plus_relative():
    o = _f32(1e-12, 1.0)
    g = _f32(1e-12 + 9e-10, 1.0 + 1.9e-6)  # within 1e-9 + 2e-6 |o|
    r = P.f32_close("x", g, o)
    assert r["rtol_only_out"] == 1  # the tiny value fails the relative bound alone
    with pytest.raises(AssertionError, match="out of tolerance"):
        P.f32_close("x", _f32(1e-12 + 2e-9, 1.0), o)
    with pytest.raises(AssertionError, match="first at 1"):
        P.f32_close("x", _f32(1e-12, 1.0 + 3e-6), o)
    with pytest.raises(AssertionError):
        P.f32_close("x", _f32(np.nan, 1.0), o)  # NaN only on one side


def test_bf16_one_apart_in_order_across_zero():
    o = np.array([0x3F80, 0x0000, 0x8001, 0x7FC0], dtype=np.uint16)
    g = np.array([0x3F81, 0x8000, 0x0000, 0x7FC1], dtype=np.uint16)
    r = P.bf16_close("p", g, o)       # +1 pattern; -0 == +0; -tiny vs +0 is 1 apart; NaNs
    assert r["bitwise"] == 0.0
    with pytest.raises(AssertionError, match="more than 1 ulp"):
        P.bf16_close("p", np.array([0x3F82], np.uint16), np.array([0x3F80], np.uint16))
    with pytest.raises(AssertionError):  # NaN against a number
        P.bf16_close("p", np.array([0x7FC0], np.uint16), np.array([0x3F80], np.uint16))


def test_int8_exact_on_identical_blocks_and_flags_the_rest():
    block, n = 4, 10  # 3 blocks, the last partial
    p = np.arange(n, dtype=np.uint16)
    codes = np.arange(n, dtype=np.int8)
    scales = _f32(1.0, 2.0, 3.0)
    diff = P.int8_exact("q", codes, scales, codes.copy(), scales.copy(), p, p.copy(), block)
    assert not diff.any()
    p2 = p.copy()
    p2[5] += 1  # block 1's input differs: its codes may differ too
    c2 = codes.copy()
    c2[5] = 99
    diff = P.int8_exact("q", c2, scales, codes, scales, p2, p, block)
    assert diff.tolist() == [False, True, False]
    c3 = codes.copy()
    c3[9] = 99  # tail block, identical input: must fail
    with pytest.raises(AssertionError, match="block 2"):
        P.int8_exact("q", c3, scales, codes, scales, p, p, block)
    s3 = scales.copy()
    s3[0] = np.float32(1.5)
    with pytest.raises(AssertionError, match="block 0"):
        P.int8_exact("q", codes, s3, codes, scales, p, p, block)


def test_sumsq_tolerance_grows_with_n_and_buckets():
    t1 = P.sumsq_tolerance(1 << 20, 1.0)
    assert 0 < t1 < 1e-9
    assert P.sumsq_tolerance(1 << 30, 1.0) > t1
    assert P.sumsq_tolerance(1 << 20, 1.0, buckets=26) > t1
    assert P.sumsq_tolerance(1 << 20, 4.0) == pytest.approx(4 * t1)
