"""Pins of the oracle's rounding and smallest-exponent search.

rne is checked against Python's round() on exact Fractions (round half to
even) and against numpy's rint on exactly representable float64 values; the
smallest exponent ``need`` is checked against a brute-force scan over every
candidate exponent that uses np.rint, not the oracle's rounding.
"""

from fractions import Fraction

import numpy as np
import pytest

import oracle as o


def _round_frac(a, s):
    return round(Fraction(a) / Fraction(2) ** s)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_rne_int_matches_fraction_round(seed):
    rng = np.random.default_rng(seed)
    for _ in range(4000):
        a = int(rng.integers(-(1 << 40), 1 << 40))
        s = int(rng.integers(-8, 45))
        assert o.rne_int(a, s) == _round_frac(a, s)


def test_rne_ties_round_to_even():
    # exact halves: a = (2q+1) * 2**(s-1)
    for s in range(1, 20):
        for q in range(-40, 40):
            a = (2 * q + 1) << (s - 1)
            r = o.rne_int(a, s)
            assert r in (q, q + 1) and r % 2 == 0
    assert o.rne_int(127, 1) == 64
    assert o.rne_int(-3, 1) == -2
    assert o.rne_int(3, 1) == 2
    assert o.rne_int(1, 1) == 0
    assert o.rne_int(-1, 1) == 0
    assert o.rne_int(5, 1) == 2
    assert o.rne_int(-5, 1) == -2
    assert o.rne_int(7, -3) == 56


def test_rne_np_matches_rint():
    rng = np.random.default_rng(3)
    a = rng.integers(-(1 << 30), 1 << 30, size=200000)
    s = rng.integers(-4, 40, size=a.size)
    ref = np.rint(a.astype(np.float64) / np.exp2(s.astype(np.float64))).astype(np.int64)
    assert np.array_equal(o.rne_np(a, s), ref)
    # ties
    q = rng.integers(-1000, 1000, size=5000)
    s2 = rng.integers(1, 20, size=q.size)
    ties = (2 * q + 1) << (s2 - 1)
    ref2 = np.rint(ties.astype(np.float64) / np.exp2(s2.astype(np.float64))).astype(np.int64)
    assert np.array_equal(o.rne_np(ties, s2), ref2)


def test_rne_np_large_shifts_and_zero():
    a = np.array([0, 5, -5, 1 << 40, -(1 << 40), 0])
    s = np.array([300, 300, 300, 300, 300, -300])
    assert np.array_equal(o.rne_np(a, s), np.zeros(6, dtype=np.int64))


def _need_bruteforce(m):
    """Smallest s in [-10, 30] with |rint(m / 2**s)| <= 127 (float64 exact)."""
    s = np.arange(-10, 31, dtype=np.float64)
    v = np.abs(np.rint(m[:, None].astype(np.float64) / np.exp2(s[None, :])))
    ok = v <= 127
    return (np.argmax(ok, axis=1) - 10).astype(np.int64)


def test_need_exhaustive_16bit():
    m = np.arange(1, 1 << 16, dtype=np.int64)
    bf = _need_bruteforce(m)
    assert np.array_equal(o.need_np(m, 0), bf)
    assert np.array_equal(o.need_np(-m, 5), bf + 5)


def test_need_random_40bit():
    rng = np.random.default_rng(4)
    m = rng.integers(1, 1 << 40, size=20000)
    for a in m[:2000]:
        a = int(a)
        e = o.need_int(a, 0)
        assert abs(_round_frac(a, e)) <= 127 and abs(_round_frac(a, e - 1)) > 127
    bf = np.array([next(s for s in range(-10, 40) if abs(_round_frac(int(x), s)) <= 127) for x in m[:3000]])
    assert np.array_equal(o.need_np(m[:3000], 0), bf)


def test_need_closed_form_values():
    # 127 fits; 128 needs one halving; 255/2 = 127.5 ties to 128, so 255
    # needs two; 509/4 = 127.25 fits, 510/4 = 127.5 does not.
    for m, s in [(1, -6), (64, 0), (127, 0), (128, 1), (254, 1), (255, 2), (509, 2), (510, 3)]:
        assert o.need_int(m, 0) == s
        assert o.need_int(-m, 0) == s
    assert o.need_int(0, 3) is None
