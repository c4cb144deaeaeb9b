"""Pins of the oracle's group requantisation.

The oracle (per-element smallest exponent, then the group maximum) is checked
against requant_frac, which searches the group exponent directly on exact
Fractions, and against the invariants the definition implies: |C| <= 127, a
nonzero unclamped group has max|C| >= 64, idempotence, power-of-two
equivariance, odd symmetry and a half-ulp error bound.
"""

from fractions import Fraction

import numpy as np
import pytest

import oracle as o


def _rand_case(rng, rows, cols, mag_bits, eps_lo, eps_hi):
    acc = rng.integers(-(1 << mag_bits), 1 << mag_bits, size=(rows, cols))
    acc[rng.random(acc.shape) < 0.2] = 0
    eps = rng.integers(eps_lo, eps_hi + 1, size=(rows, cols))
    return acc, eps


@pytest.mark.parametrize("group", [o.TENSOR, o.ROW])
@pytest.mark.parametrize("seed", range(6))
def test_requant_matches_fraction_search(group, seed):
    rng = np.random.default_rng(seed)
    acc, eps = _rand_case(rng, 4, 7, [3, 9, 17, 27, 30, 12][seed], -30, 10)
    if seed == 5:
        eps[:] = eps[0, 0]                         # uniform exponent
    out = o.requant_np(acc, eps, group)
    vals = [[Fraction(int(acc[i, j])) * Fraction(2) ** int(eps[i, j]) for j in range(acc.shape[1])]
            for i in range(acc.shape[0])]
    rows, exps = o.requant_frac(vals, group)
    assert np.array_equal(out.mant.astype(np.int64), np.array(rows))
    assert list(out.exp.astype(int)) == exps


def test_requant_ties_and_neg128():
    acc = np.array([[255, -255, 510, 3, -128, 127]])
    eps = np.zeros_like(acc)
    out = o.requant_np(acc, eps, o.TENSOR)
    # max need is 510 -> s = 3: 510/8 = 63.75 -> 64, 255/8 = 31.875 -> 32, 3/8 -> 0
    assert out.exp[0] == 3
    assert out.mant[0].tolist() == [32, -32, 64, 0, -16, 16]


def test_requant_zero_group_and_clamp():
    acc = np.zeros((2, 3), dtype=np.int64)
    out = o.requant_np(acc, np.zeros_like(acc), o.ROW)
    assert list(out.exp) == [o.E_MIN, o.E_MIN] and not out.mant.any()
    # tiny values below E_MIN: exponent clamps, mantissas round
    acc = np.array([[3, 1, -2]])
    out = o.requant_np(acc, np.full_like(acc, -130), o.TENSOR)
    assert out.exp[0] == o.E_MIN
    assert out.mant[0].tolist() == [1, 0, 0]        # 0.75 -> 1, 0.25 -> 0, -0.5 -> 0 (even)


def test_requant_exp_range_error():
    acc = np.array([[1 << 20]])
    with pytest.raises(o.ExpRangeError):
        o.requant_np(acc, np.array([[120]]), o.TENSOR)


@pytest.mark.parametrize("seed", range(4))
def test_requant_invariants(seed):
    rng = np.random.default_rng(100 + seed)
    acc, eps = _rand_case(rng, 16, 33, 26, -60, 20)
    for group in (o.TENSOR, o.ROW):
        out = o.requant_np(acc, eps, group)
        c = out.mant.astype(np.int64)
        e = out.row_exp()
        assert np.all(np.abs(c) <= 127)
        # nonzero, unclamped groups are normalised
        if group == o.ROW:
            for i in range(acc.shape[0]):
                if acc[i].any() and e[i] > o.E_MIN:
                    assert np.abs(c[i]).max() >= 64
        elif acc.any():
            assert np.abs(c).max() >= 64
        # half-ulp error bound against the exact value
        for i in range(acc.shape[0]):
            for j in range(acc.shape[1]):
                exact = Fraction(int(acc[i, j])) * Fraction(2) ** int(eps[i, j])
                got = Fraction(int(c[i, j])) * Fraction(2) ** int(e[i])
                assert abs(got - exact) <= Fraction(2) ** int(e[i]) / 2
        # idempotence
        again = o.requant_np(c, np.broadcast_to(e[:, None], c.shape), group)
        assert np.array_equal(again.mant, out.mant) and np.array_equal(again.exp, out.exp)
        # odd symmetry
        neg = o.requant_np(-acc, eps, group)
        assert np.array_equal(neg.mant, -out.mant) and np.array_equal(neg.exp, out.exp)
        # power-of-two equivariance (no clamp in play: shift by +7)
        sh = o.requant_np(acc, eps + 7, group)
        assert np.array_equal(sh.mant, out.mant)
        nonzero = acc.reshape(acc.shape[0], -1).any(axis=1) if group == o.ROW else np.array([acc.any()])
        want = np.where(nonzero, out.exp.astype(int) + 7, o.E_MIN)
        assert np.array_equal(sh.exp.astype(int), want)


def test_align_rows_identity_and_rounding():
    t = o.qt([[127, -3, 3, 1], [10, 20, 30, 40]], [-5, -6], o.ROW)
    m, e = o.align_rows(t)
    assert e == -5
    assert m[0].tolist() == [127, -3, 3, 1]
    assert m[1].tolist() == [5, 10, 15, 20]
    t2 = o.qt([[127, -3, 3, 1]], [-4], o.ROW)
    m2, e2 = o.align_rows(o.QT(np.vstack([t2.mant, t2.mant]), np.array([-4, -3], dtype=np.int8), o.ROW))
    assert e2 == -3 and m2[0].tolist() == [64, -2, 2, 0]
    u = o.qt([[1, 2], [3, 4]], [-7], o.TENSOR)
    mu, eu = o.align_rows(u)
    assert eu == -7 and mu.tolist() == [[1, 2], [3, 4]]
