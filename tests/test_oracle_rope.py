"""Pins of the oracle's RoPE: closed forms, invariants, exact arithmetic.  CPU only."""
import math

import mpmath
import numpy as np
import pytest

import oracle
from oracle.variants import brute_force_rotate_key


def test_inv_freq_endpoints():
    f = oracle.inv_freq(1.0e4, 128)
    assert f[0] == 1.0
    assert len(f) == 64
    assert math.isclose(f[-1], 1.0e4 ** (-126 / 128), rel_tol=1e-15)
    assert all(a > b for a, b in zip(f, f[1:]))


def test_position_zero_is_identity():
    c, s = oracle.rope_rows_f32(5.0e5, 128, [0])
    assert np.all(c == 1.0) and np.all(s == 0.0)
    rng = np.random.default_rng(0)
    x = rng.standard_normal((8, 128)).astype(np.float32)
    assert np.array_equal(oracle.rope_k_f32(x, c[0], s[0]), x)
    assert np.array_equal(oracle.rope_f64(x.astype(np.float64), 0, 5.0e5), x.astype(np.float64))


def test_d2_is_rotation_by_position_radians():
    # With D = 2 the only frequency is theta**0 = 1: a rotation by p radians.
    for p in (1, 2, 7, 1000):
        x = np.array([0.3, -1.7])
        y = oracle.rope_f64(x, p, 1.0e4)
        want = [0.3 * math.cos(p) + 1.7 * math.sin(p),
                -1.7 * math.cos(p) + 0.3 * math.sin(p)]
        assert np.allclose(y, want, rtol=0, atol=1e-15)


def test_pair_norms_preserved():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((4, 128))
    y = oracle.rope_f64(x, 12345, 5.0e5)
    n0 = x[:, :64] ** 2 + x[:, 64:] ** 2
    n1 = y[:, :64] ** 2 + y[:, 64:] ** 2
    assert np.max(np.abs(n1 - n0) / n0) < 1e-14
    # the float32 path keeps pair norms within a few float32 ulps
    c, s = oracle.rope_rows_f32(5.0e5, 128, [12345])
    y32 = oracle.rope_k_f32(x.astype(np.float32), c[0], s[0]).astype(np.float64)
    x32 = x.astype(np.float32).astype(np.float64)
    m0 = x32[:, :64] ** 2 + x32[:, 64:] ** 2
    m1 = y32[:, :64] ** 2 + y32[:, 64:] ** 2
    assert np.max(np.abs(m1 - m0) / m0) < 8 * 2.0 ** -23


def test_relative_position_property():
    # (R_m q) . (R_n k) == q . (R_{n-m} k)
    rng = np.random.default_rng(2)
    q = rng.standard_normal(64)
    k = rng.standard_normal(64)
    for m, n in [(3, 10), (100, 4000), (77, 77), (5000, 12)]:
        lhs = oracle.rope_f64(q, m, 1.0e4) @ oracle.rope_f64(k, n, 1.0e4)
        rhs = q @ oracle.rope_f64(k, n - m, 1.0e4)
        assert abs(lhs - rhs) < 1e-11 * (1 + abs(lhs))


def test_pairing_is_rotate_half():
    # dimension i pairs with i + D/2: a vector living only on dims (0, D/2)
    # stays on those dims.
    x = np.zeros(16)
    x[0] = 1.0
    y = oracle.rope_f64(x, 3, 100.0)
    assert np.count_nonzero(y) == 2 and y[0] != 0 and y[8] != 0
    assert math.isclose(y[0], math.cos(3.0), abs_tol=1e-15)
    assert math.isclose(y[8], math.sin(3.0), abs_tol=1e-15)


def test_table_within_one_f32_ulp_of_exact():
    mpmath.mp.dps = 40
    theta, d = 5.0e5, 128
    positions = [0, 1, 17, 1023, 8191, 131071]
    c, s = oracle.rope_rows_f32(theta, d, positions)
    for r, p in enumerate(positions):
        for i in range(0, d // 2, 5):
            ang = mpmath.mpf(p) * mpmath.power(mpmath.mpf(theta), mpmath.mpf(-2 * i) / d)
            for got, ex in ((c[r, i], mpmath.cos(ang)), (s[r, i], mpmath.sin(ang))):
                ulp = np.spacing(np.float32(abs(float(ex)))) if float(ex) != 0 else 2.0 ** -149
                assert abs(float(got) - float(ex)) <= float(ulp)


def test_f32_key_rotation_matches_exact_rationals():
    rng = np.random.default_rng(3)
    for pos, d in [(5, 16), (1000, 64), (130000, 128)]:
        k = rng.standard_normal((2, d)).astype(np.float32) * np.float32(3)
        c, s = oracle.rope_rows_f32(5.0e5, d, [pos])
        ours = oracle.rope_k_f32(k, c[0], s[0]).astype(np.float64)
        exact = brute_force_rotate_key(k, c[0], s[0])
        assert np.array_equal(ours, exact)


def test_f32_key_rotation_differs_from_fused_arithmetic_somewhere():
    # A fused multiply-add would change some results: the pinned arithmetic
    # is a real constraint, not a tautology.
    rng = np.random.default_rng(4)
    k = rng.standard_normal((64, 128)).astype(np.float32)
    c, s = oracle.rope_rows_f32(5.0e5, 128, [777])
    ours = oracle.rope_k_f32(k, c[0], s[0])
    x0, x1 = k[:, :64].astype(np.float64), k[:, 64:].astype(np.float64)
    fused = (x0 * c[0] - np.float32(x1 * s[0]).astype(np.float64)).astype(np.float32)
    assert not np.array_equal(ours[:, :64], fused)
