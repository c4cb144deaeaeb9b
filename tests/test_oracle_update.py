"""Pins of the oracle's integer SGD-with-momentum update (Figure 1b, Table 5).

Hand-worked cases, the closed-form velocity sequence under a constant
gradient, the beta = 0 and lr = 0 special cases, and a Fraction brute force
over random cases that spans exponent gaps from 0 to 255.
"""

from fractions import Fraction

import numpy as np
import pytest

import oracle as o

LR = o.Scalar(1, -7)
BETA = o.Scalar(7, -3)


def test_hand_worked_update():
    # beta*V = 7*[64,-127,5,16,0] * 2**-15 = [448,-889,35,112,0] * 2**-15
    # G = [16,17,-127,2,1] * 2**-10 = [512,544,-4064,64,32] * 2**-15
    # v = [960,-345,-4029,176,32] * 2**-15; 4029/2**5 = 125.9 fits, /2**4 does
    # not -> e = -10; 960/32 = 30, -345/32 = -10.8 -> -11, -4029/32 -> -126,
    # 176/32 = 5.5 -> 6 (tie to even), 32/32 = 1.
    # w = [100,-64,3,0,-127]*2**-14 - [30,-11,-126,6,1]*2**-17
    #   = [770,-501,150,-6,-1017] * 2**-17; 1017/8 = 127.1 -> e = -14;
    # 770/8 = 96.25 -> 96, -501/8 -> -63, 150/8 = 18.75 -> 19, -6/8 -> -1,
    # -1017/8 = -127.1 -> -127.
    W = o.qt([[100, -64, 3, 0, -127]], [-14], o.ROW)
    V = o.qt([[64, -127, 5, 16, 0]], [-12], o.ROW)
    G = o.qt([[16, 17, -127, 2, 1]], [-10], o.ROW)
    W2, V2 = o.sgd_update(W, V, G, LR, BETA)
    assert V2.mant.tolist() == [[30, -11, -126, 6, 1]] and V2.exp.tolist() == [-10]
    assert W2.mant.tolist() == [[96, -63, 19, -1, -127]] and W2.exp.tolist() == [-14]


def test_constant_gradient_velocity_sequence():
    # g = 64 @ -10, V0 = 0:  64@-10, 120@-10 (= 64 + 56), then
    # 7/8*120 + 64 = 169 -> 84.5 -> 84 @ -9; 7/8*84*2 + 64 = 211 -> 105.5 -> 106 @ -9;
    # 7/8*106*2 + 64 = 249.5 -> 124.75 -> 125 @ -9.
    W = o.qt([[0]], [o.E_MIN], o.ROW)
    V = o.qt([[0]], [o.E_MIN], o.ROW)
    G = o.qt([[64]], [-10], o.ROW)
    seq = []
    for _ in range(5):
        W, V = o.sgd_update(W, V, G, o.Scalar(0, 0), BETA)
        seq.append((int(V.mant[0, 0]), int(V.exp[0])))
    assert seq == [(64, -10), (120, -10), (84, -9), (106, -9), (125, -9)]


def test_beta_zero_is_plain_sgd_and_lr_zero_canonicalises():
    rng = np.random.default_rng(1)
    W = o.QT(rng.integers(-40, 40, size=(3, 8)).astype(np.int8), np.array([-9, -7, -8], dtype=np.int8), o.ROW)
    V = o.QT(rng.integers(-127, 128, size=(3, 8)).astype(np.int8), np.array([-12, -11, -13], dtype=np.int8), o.ROW)
    G = o.QT(rng.integers(-127, 128, size=(3, 8)).astype(np.int8), np.array([-10, -14, -9], dtype=np.int8), o.ROW)
    W2, V2 = o.sgd_update(W, V, G, LR, o.Scalar(0, 0))
    g_req = o.requant_np(G.mant.astype(np.int64), np.broadcast_to(G.row_exp()[:, None], (3, 8)), o.ROW)
    assert np.array_equal(V2.mant, g_req.mant) and np.array_equal(V2.exp, g_req.exp)
    W3, _ = o.sgd_update(W, V, G, o.Scalar(0, 0), BETA)
    w_req = o.requant_np(W.mant.astype(np.int64), np.broadcast_to(W.row_exp()[:, None], (3, 8)), o.ROW)
    assert np.array_equal(W3.mant, w_req.mant) and np.array_equal(W3.exp, w_req.exp)


def _frac_update(W, V, G, lr, beta, wd):
    wv, vv, gv = W.values(), V.values(), G.values()
    v_exact = [[beta.value() * v + g + wd.value() * w for v, g, w in zip(vr, gr, wr)]
               for vr, gr, wr in zip(vv, gv, wv)]
    vr, ve = o.requant_frac(v_exact, V.group)
    vnew = [[Fraction(c) * Fraction(2) ** (ve[i] if V.group == o.ROW else ve[0]) for c in row]
            for i, row in enumerate(vr)]
    w_exact = [[w - lr.value() * v for w, v in zip(wr, nr)] for wr, nr in zip(wv, vnew)]
    wr_, we = o.requant_frac(w_exact, W.group)
    return wr_, we, vr, ve


@pytest.mark.parametrize("seed", range(12))
def test_update_matches_fraction_bruteforce(seed):
    rng = np.random.default_rng(50 + seed)
    rows, cols = 3, 6
    gw, gv, gg = [(o.ROW, o.ROW, o.ROW), (o.TENSOR, o.ROW, o.ROW), (o.ROW, o.TENSOR, o.TENSOR)][seed % 3]
    span = [4, 30, 120, 255][seed % 4]

    def mk(group, lo, hi):
        m = rng.integers(-128, 128, size=(rows, cols)).astype(np.int8)
        m[rng.random(m.shape) < 0.15] = 0
        n = 1 if group == o.TENSOR else rows
        e = np.clip(rng.integers(lo, hi + 1, size=n), o.E_MIN, o.E_MAX)
        return o.QT(m, e.astype(np.int8), group)

    lo = -110
    W = mk(gw, lo, lo + span)
    V = mk(gv, lo, lo + span)
    G = mk(gg, lo, lo + span)
    lr = o.Scalar(int(rng.integers(1, 128)), int(rng.integers(-12, 0)))
    beta = o.Scalar(int(rng.integers(0, 128)), int(rng.integers(-8, 0)))
    wd = o.Scalar(int(rng.integers(0, 3)), -13) if seed >= 6 else o.Scalar(0, 0)
    try:
        want = _frac_update(W, V, G, lr, beta, wd)
    except o.ExpRangeError:
        with pytest.raises(o.ExpRangeError):
            o.sgd_update(W, V, G, lr, beta, wd)
        return
    W2, V2 = o.sgd_update(W, V, G, lr, beta, wd)
    assert W2.mant.astype(int).tolist() == want[0] and W2.exp.astype(int).tolist() == want[1]
    assert V2.mant.astype(int).tolist() == want[2] and V2.exp.astype(int).tolist() == want[3]


def test_update_large_gap_breaks_ties_exactly():
    # beta*V = 7*23 * 2**(3-3) = 161: 161/2 = 80.5 is a tie.  A gradient 2**100
    # times smaller decides it: +tiny -> 81, -tiny -> 80; without it -> 80 (even).
    W = o.qt([[0, 0, 0]], [0], o.ROW)
    V = o.qt([[23, 23, 23]], [3], o.ROW)
    G = o.QT(np.array([[1, -1, 0]], dtype=np.int8), np.array([-100], dtype=np.int8), o.ROW)
    _, V2 = o.sgd_update(W, V, G, o.Scalar(0, 0), BETA)
    assert V2.mant.tolist() == [[81, 80, 80]] and V2.exp.tolist() == [1]
    # negative side: -80.5 - tiny -> -81
    V = o.qt([[-23, -23]], [3], o.ROW)
    G = o.qt([[-1, 1]], [-100], o.ROW)
    _, V3 = o.sgd_update(o.qt([[0, 0]], [0], o.ROW), V, G, o.Scalar(0, 0), BETA)
    assert V3.mant.tolist() == [[-81, -80]] and V3.exp.tolist() == [1]
