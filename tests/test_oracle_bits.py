"""Pins of the oracle's B-bit mantissa variant (Table 4, B in 8..4; reading:
a B-bit result has |C| <= 2**(B-1) - 1, the velocity stays INT8).

The smallest exponent is checked against a brute-force scan with np.rint,
group requantisation and Sum against the direct Fraction search, the update
against a Fraction re-derivation, and the ReLU6 cap against its closed form.
The memory column of Table 4 is pinned in test_oracle_pages.
"""

from fractions import Fraction

import numpy as np
import pytest

import oracle as o

BITS = [2, 3, 4, 5, 6, 7, 8]


def _need_bruteforce(m, qm):
    s = np.arange(-12, 31, dtype=np.float64)
    v = np.abs(np.rint(m[:, None].astype(np.float64) / np.exp2(s[None, :])))
    return (np.argmax(v <= qm, axis=1) - 12).astype(np.int64)


@pytest.mark.parametrize("bits", BITS)
def test_need_exhaustive_14bit(bits):
    qm = (1 << (bits - 1)) - 1
    assert o.q_max(bits) == qm
    m = np.arange(1, 1 << 14, dtype=np.int64)
    bf = _need_bruteforce(m, qm)
    assert np.array_equal(o.need_np(m, 0, bits), bf)
    assert np.array_equal(o.need_np(-m, -7, bits), bf - 7)
    for a in (1, 2, 3, qm, qm + 1, 2 * qm + 1, 2 * qm + 2, 1000, 16383):
        assert o.need_int(a, 0, bits) == bf[a - 1]


@pytest.mark.parametrize("bits", BITS)
def test_need_closed_forms(bits):
    # q_max fits as is; q_max + 1 needs one halving; 2 q_max + 1 halves to
    # q_max + 1/2, a tie that rounds to the even q_max + 1, so it needs two
    qm = o.q_max(bits)
    assert o.need_int(qm, 0, bits) == 0
    assert o.need_int(qm + 1, 0, bits) == 1
    assert o.need_int(2 * qm, 0, bits) == 1
    assert o.need_int(2 * qm + 1, 0, bits) == 2
    assert o.need_int(-(2 * qm + 1), 3, bits) == 5


@pytest.mark.parametrize("bits", [4, 5, 6, 7])
@pytest.mark.parametrize("group", [o.TENSOR, o.ROW])
def test_requant_bits_matches_fraction_search(bits, group):
    rng = np.random.default_rng(bits * 10 + group)
    for mag in (3, 9, 20, 30):
        acc = rng.integers(-(1 << mag), 1 << mag, size=(4, 7))
        acc[rng.random(acc.shape) < 0.2] = 0
        eps = rng.integers(-30, 10, size=acc.shape)
        out = o.requant_np(acc, eps, group, bits)
        vals = [[Fraction(int(acc[i, j])) * Fraction(2) ** int(eps[i, j]) for j in range(7)] for i in range(4)]
        rows, exps = o.requant_frac(vals, group, bits)
        assert np.array_equal(out.mant.astype(np.int64), np.array(rows))
        assert list(out.exp.astype(int)) == exps
        qm = o.q_max(bits)
        assert np.abs(out.mant.astype(int)).max() <= qm
        # canonical: a nonzero group whose exponent is above E_MIN has a
        # member of at least half the range
        re = out.row_exp()
        m = out.mant.astype(int).reshape(4, -1)
        groups = [m[i] for i in range(4)] if group == o.ROW else [m.reshape(-1)]
        for g, e in zip(groups, re if group == o.ROW else re[:1]):
            if np.any(g) and e > o.E_MIN:
                assert np.abs(g).max() >= (qm + 1) // 2


def test_requant_bits_idempotent_across_widths():
    """Narrowing a value that already fits B bits changes nothing: a tensor
    requantised at B bits, requantised again at B bits or wider, is unchanged
    (idempotence across widths)."""
    rng = np.random.default_rng(11)
    acc = rng.integers(-(1 << 20), 1 << 20, size=(5, 9))
    eps = rng.integers(-10, 10, size=acc.shape)
    for bits in (4, 5, 6, 7):
        q = o.requant_np(acc, eps, o.ROW, bits)
        for wider in range(bits, 9):
            again = o.requant_np(q.mant.astype(np.int64), np.broadcast_to(q.row_exp()[:, None], acc.shape),
                                 o.ROW, wider)
            # the wider form may lower the exponent (left shifts are exact),
            # but the value is the same
            assert all(a == b for ra, rb in zip(again.values(), q.values()) for a, b in zip(ra, rb))


@pytest.mark.parametrize("bits", [4, 5, 6, 7])
def test_sum_bits_matches_fraction(bits):
    rng = np.random.default_rng(300 + bits)
    for _ in range(12):
        ga, gb, go = (int(x) for x in rng.integers(0, 2, size=3))
        qa = (1 << (bits - 1)) - 1
        A = o.QT(rng.integers(-qa, qa + 1, size=(3, 5)).astype(np.int8),
                 rng.integers(-60, 60, size=1 if ga == o.TENSOR else 3).astype(np.int8), ga)
        B = o.QT(rng.integers(-qa, qa + 1, size=(3, 5)).astype(np.int8),
                 rng.integers(-60, 60, size=1 if gb == o.TENSOR else 3).astype(np.int8), gb)
        S = o.sum_op(A, B, go, bits)
        vals = [[a + b for a, b in zip(ra, rb)] for ra, rb in zip(A.values(), B.values())]
        rows, exps = o.requant_frac(vals, go, bits)
        assert S.mant.astype(int).tolist() == rows and S.exp.astype(int).tolist() == exps


@pytest.mark.parametrize("bits", [4, 5, 6, 7])
def test_update_bits_matches_fraction(bits):
    """The weight takes B bits, the velocity INT8 (Table 4)."""
    rng = np.random.default_rng(400 + bits)
    qa = (1 << (bits - 1)) - 1
    for trial in range(6):
        gw, gv = [(o.ROW, o.ROW), (o.TENSOR, o.ROW), (o.ROW, o.TENSOR)][trial % 3]

        def mk(group, lim, lo, hi):
            m = rng.integers(-lim, lim + 1, size=(3, 6)).astype(np.int8)
            n = 1 if group == o.TENSOR else 3
            return o.QT(m, rng.integers(lo, hi, size=n).astype(np.int8), group)

        W = mk(gw, qa, -20, -10)
        V = mk(gv, 127, -30, -20)
        G = mk(gv, qa, -30, -20)
        lr = o.Scalar(int(rng.integers(1, 128)), int(rng.integers(-8, 0)))
        beta = o.Scalar(115, -7)
        wd = o.Scalar(1, -13) if trial >= 3 else o.Scalar(0, 0)
        W2, V2 = o.sgd_update(W, V, G, lr, beta, wd, w_bits=bits)
        wv, vv, gvv = W.values(), V.values(), G.values()
        v_exact = [[beta.value() * v + g + wd.value() * w for v, g, w in zip(a, b, c)]
                   for a, b, c in zip(vv, gvv, wv)]
        vr, ve = o.requant_frac(v_exact, V.group, 8)
        vnew = [[Fraction(c) * Fraction(2) ** (ve[i] if V.group == o.ROW else ve[0]) for c in row]
                for i, row in enumerate(vr)]
        w_exact = [[w - lr.value() * v for w, v in zip(a, b)] for a, b in zip(wv, vnew)]
        wr, we = o.requant_frac(w_exact, W.group, bits)
        assert V2.mant.astype(int).tolist() == vr and V2.exp.astype(int).tolist() == ve
        assert W2.mant.astype(int).tolist() == wr and W2.exp.astype(int).tolist() == we
        assert np.abs(W2.mant.astype(int)).max() <= qa


@pytest.mark.parametrize("bits", [4, 5, 6, 7, 8])
def test_relu6_cap_bits(bits):
    qm = o.q_max(bits)
    for e in range(-12, 6):
        six = Fraction(6) / Fraction(2) ** e
        assert o.relu6_cap(e, bits) == min(int(six), qm)   # floor of 6 * 2^-e
    C = np.arange(-qm, qm + 1)
    dY = np.full(C.shape, 5)
    for e in (-5, -3, -1, 0, 1):
        c = o.relu6_cap(e, bits)
        assert o.relu6_fwd(C, e, bits).tolist() == [min(max(x, 0), c) for x in C]
        assert o.relu6_bwd(dY, C, e, bits).tolist() == [5 if 0 < x < c else 0 for x in C]
