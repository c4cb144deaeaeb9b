"""GPU parity: every entry point of libie.so, called through the C ABI, is
bit-exact (mantissas and exponents) against the oracle on seeded inputs that
span several tiles and a ragged tail, and on the degenerate cases."""

import itertools

import numpy as np
import pytest
import torch

import oracle as o
from integer_only_dnn_amd import ie
from tests.gpu_util import announce, assert_same, qt_to_dev, rand_qt

pytestmark = pytest.mark.gpu

T, R = o.TENSOR, o.ROW
GROUPS = list(itertools.product([T, R], repeat=3))

LIN_SHAPES = [(64, 128, 256), (1, 1, 1), (3, 5, 7), (130, 200, 96), (257, 129, 300), (300, 256, 64), (129, 64, 1000)]


@pytest.fixture(scope="module")
def ws():
    return ie.Workspace("cuda")


@pytest.mark.parametrize("shape", LIN_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("groups", GROUPS, ids=lambda g: "".join("TR"[x] for x in g))
def test_linear_fwd(shape, groups, ws):
    M, N, K = shape
    gx, gw, gy = groups
    announce(f"linear_fwd M={M} N={N} K={K} groups={groups}")
    rng = np.random.default_rng(M * 7 + N * 3 + K + 100 * gx + 10 * gw + gy)
    X = rand_qt(rng, (M, K), gx)
    W = rand_qt(rng, (N, K), gw)
    want = o.linear_fwd(X, W, gy)
    Y = ie.Mat.empty(M, N, gy)
    ie.ie_linear_fwd(qt_to_dev(X), qt_to_dev(W), Y, ws)
    assert_same(Y, want, "linear_fwd")
    assert ws.status() == 0


@pytest.mark.parametrize("shape", LIN_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("groups", GROUPS, ids=lambda g: "".join("TR"[x] for x in g))
def test_linear_bwd_dx(shape, groups, ws):
    M, N, K = shape
    gdy, gw, gdx = groups
    announce(f"linear_bwd_dx M={M} N={N} K={K} groups={groups}")
    rng = np.random.default_rng(M * 5 + N * 11 + K + 100 * gdy + 10 * gw + gdx)
    dY = rand_qt(rng, (M, N), gdy)
    W = rand_qt(rng, (N, K), gw)
    want = o.linear_bwd_dx(dY, W, gdx)
    dX = ie.Mat.empty(M, K, gdx)
    ie.ie_linear_bwd_dx(qt_to_dev(dY), qt_to_dev(W), dX, ws)
    assert_same(dX, want, "linear_bwd_dx")


@pytest.mark.parametrize("shape", LIN_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("groups", GROUPS, ids=lambda g: "".join("TR"[x] for x in g))
def test_linear_bwd_dw(shape, groups, ws):
    M, N, K = shape
    gdy, gx, gdw = groups
    announce(f"linear_bwd_dw M={M} N={N} K={K} groups={groups}")
    rng = np.random.default_rng(M * 13 + N * 3 + K * 7 + 100 * gdy + 10 * gx + gdw)
    dY = rand_qt(rng, (M, N), gdy)
    X = rand_qt(rng, (M, K), gx)
    want = o.linear_bwd_dw(dY, X, gdw)
    dW = ie.Mat.empty(N, K, gdw)
    ie.ie_linear_bwd_dw(qt_to_dev(dY), qt_to_dev(X), dW, ws)
    assert_same(dW, want, "linear_bwd_dw")


def test_linear_degenerate(ws):
    rng = np.random.default_rng(9)
    announce("linear degenerate: K=0, M=0, N=0, all-zero operands")
    # empty contraction: all outputs zero with exponent E_MIN
    X = o.QT(np.zeros((5, 0), np.int8), np.array([3], np.int8), T)
    W = o.QT(np.zeros((4, 0), np.int8), np.array([1, 2, 3, 4], np.int8), R)
    for gy in (T, R):
        Y = ie.Mat.empty(5, 4, gy)
        ie.ie_linear_fwd(qt_to_dev(X, rows=5), qt_to_dev(W, rows=4), Y, ws)
        assert_same(Y, o.linear_fwd(X, W, gy), "K=0")
    # empty batch
    X = rand_qt(rng, (0, 16), T)
    W = rand_qt(rng, (8, 16), R)
    Y = ie.Mat.empty(0, 8, T)
    ie.ie_linear_fwd(qt_to_dev(X, rows=0), qt_to_dev(W), Y, ws)
    assert int(Y.exp.cpu()[0]) == o.E_MIN
    # all-zero operand -> zeros at E_MIN
    X = o.QT(np.zeros((70, 33), np.int8), np.array([-3], np.int8), T)
    W = rand_qt(rng, (140, 33), R)
    for gy in (T, R):
        Y = ie.Mat.empty(70, 140, gy)
        ie.ie_linear_fwd(qt_to_dev(X), qt_to_dev(W), Y, ws)
        assert_same(Y, o.linear_fwd(X, W, gy), "zero X")
    dY = o.QT(np.zeros((70, 140), np.int8), np.array([-3], np.int8), T)
    dW = ie.Mat.empty(140, 33, R)
    ie.ie_linear_bwd_dw(qt_to_dev(dY), qt_to_dev(X), dW, ws)
    assert_same(dW, o.linear_bwd_dw(dY, X, R), "zero dW")


def test_linear_extreme_exponents(ws):
    announce("linear extreme exponents: E_MIN clamp and overflow flag")
    rng = np.random.default_rng(10)
    # tiny values clamp at E_MIN and round
    X = rand_qt(rng, (40, 50), R, elo=-128, ehi=-120)
    W = rand_qt(rng, (60, 50), R, elo=-128, ehi=-120)
    for gy in (T, R):
        Y = ie.Mat.empty(40, 60, gy)
        ie.ie_linear_fwd(qt_to_dev(X), qt_to_dev(W), Y, ws)
        assert_same(Y, o.linear_fwd(X, W, gy), "E_MIN clamp")
    assert ws.status() == 0
    # exponents near the top overflow: the sticky flag is raised
    X = rand_qt(rng, (8, 64), T, elo=120, ehi=120)
    W = rand_qt(rng, (8, 64), T, elo=120, ehi=120)
    with pytest.raises(o.ExpRangeError):
        o.linear_fwd(X, W, T)
    Y = ie.Mat.empty(8, 8, T)
    ie.ie_linear_fwd(qt_to_dev(X), qt_to_dev(W), Y, ws)
    assert ws.status() & ie.FLAG_EXP_RANGE
    assert ws.status() == 0


def test_linear_wide_exponent_spread(ws):
    """Row exponents spread over 200: alignment shifts past the mantissa width."""
    announce("linear wide exponent spread")
    rng = np.random.default_rng(11)
    X = rand_qt(rng, (150, 70), R, elo=-110, ehi=60)
    W = rand_qt(rng, (90, 70), R, elo=-110, ehi=20)
    dY = rand_qt(rng, (150, 90), R, elo=-110, ehi=20)
    for g in (T, R):
        Y = ie.Mat.empty(150, 90, g)
        ie.ie_linear_fwd(qt_to_dev(X), qt_to_dev(W), Y, ws)
        assert_same(Y, o.linear_fwd(X, W, g), "fwd spread")
        dX = ie.Mat.empty(150, 70, g)
        ie.ie_linear_bwd_dx(qt_to_dev(dY), qt_to_dev(W), dX, ws)
        assert_same(dX, o.linear_bwd_dx(dY, W, g), "dx spread")
        dW = ie.Mat.empty(90, 70, g)
        ie.ie_linear_bwd_dw(qt_to_dev(dY), qt_to_dev(X), dW, ws)
        assert_same(dW, o.linear_bwd_dw(dY, X, g), "dw spread")


CONV_SHAPES = [
    (2, 7, 6, 3, 64, 3, 3, 1, 1),      # stem-like, C = 3
    (2, 8, 8, 16, 32, 3, 3, 2, 1),
    (1, 9, 7, 32, 48, 3, 3, 1, 1),
    (3, 5, 5, 16, 16, 1, 1, 1, 0),
    (2, 6, 6, 64, 128, 1, 1, 2, 0),
    (2, 10, 10, 8, 24, 3, 3, 2, 1),
    (4, 12, 12, 64, 64, 3, 3, 1, 1),
    (2, 9, 9, 24, 40, 3, 3, 2, 0),
]


@pytest.mark.parametrize("shape", CONV_SHAPES, ids=lambda s: "n{}h{}w{}c{}k{}r{}s{}st{}p{}".format(*s))
@pytest.mark.parametrize("wg", [T, R], ids=["WT", "WR"])
def test_conv(shape, wg, ws):
    n, h, w, c, k, r, s, st, pad = shape
    announce(f"conv shape={shape} w_group={wg}")
    d = o.ConvShape(n, h, w, c, k, r, s, st, pad)
    dd = ie.conv_desc(n, h, w, c, k, r, s, st, pad)
    rng = np.random.default_rng(sum(shape) * 31 + wg)
    X = rand_qt(rng, (n, h, w, c), T, zero_frac=0.3)
    W = rand_qt(rng, (k, r * s * c), wg)
    dY = rand_qt(rng, (n, d.p, d.q, k), T)
    Xd = qt_to_dev(X, rows=n * h * w)
    Wd = qt_to_dev(W)
    Y = ie.Mat.empty(n * d.p * d.q, k, T)
    ie.ie_conv_fwd(dd, Xd, Wd, Y, ws)
    assert_same(Y, o.conv_fwd(d, X, W, T), "conv_fwd")
    dX = ie.Mat.empty(n * h * w, c, T)
    dW = ie.Mat.empty(k, r * s * c, R)
    ie.ie_conv_bwd(dd, Xd, Wd, qt_to_dev(dY, rows=n * d.p * d.q), dX, dW, ws)
    assert_same(dX, o.conv_dgrad(d, dY, W, T), "conv dgrad")
    assert_same(dW, o.conv_wgrad(d, dY, X, R), "conv wgrad")
    dWt = ie.Mat.empty(k, r * s * c, T)
    ie.ie_conv_bwd(dd, Xd, Wd, qt_to_dev(dY, rows=n * d.p * d.q), None, dWt, ws)
    assert_same(dWt, o.conv_wgrad(d, dY, X, T), "conv wgrad tensor")
    assert ws.status() == 0


UPD_SHAPES = [(1, 5), (3, 7), (17, 64), (40, 256), (33, 768), (9, 1000), (12, 3072), (5, 4608)]


def _upd_case(rng, rows, cols, groups, span):
    gw, gv, gg = groups

    def mk(group, lo):
        m = rng.integers(-128, 128, size=(rows, cols)).astype(np.int8)
        m[rng.random(m.shape) < 0.1] = 0
        nn = 1 if group == T else rows
        e = np.clip(rng.integers(lo, lo + span + 1, size=nn), o.E_MIN, o.E_MAX)
        return o.QT(m, e.astype(np.int8), group)

    return mk(gw, -40), mk(gv, -40 - span // 2), mk(gg, -40 - span // 3)


@pytest.mark.parametrize("shape", UPD_SHAPES, ids=lambda s: f"{s[0]}x{s[1]}")
@pytest.mark.parametrize("groups", GROUPS, ids=lambda g: "".join("TR"[x] for x in g))
def test_sgd_update(shape, groups, ws):
    rows, cols = shape
    announce(f"sgd_update {rows}x{cols} groups(W,V,G)={groups}")
    rng = np.random.default_rng(rows * 101 + cols + 1000 * groups[0] + 100 * groups[1] + 10 * groups[2])
    for span in (6, 40, 200):
        W, V, G = _upd_case(rng, rows, cols, groups, span)
        lr = (int(rng.integers(1, 128)), int(rng.integers(-12, -1)))
        mom = (int(rng.integers(-128, 128)), int(rng.integers(-8, 0)))
        try:
            W2, V2 = o.sgd_update(W, V, G, o.Scalar(*lr), o.Scalar(*mom))
        except o.ExpRangeError:
            continue
        Wd, Vd, Gd = qt_to_dev(W), qt_to_dev(V), qt_to_dev(G)
        ie.ie_sgd_update(Wd, Vd, Gd, lr, mom, ws=ws)
        assert_same(Vd, V2, f"velocity span={span}")
        assert_same(Wd, W2, f"weight span={span}")
        assert ws.status() == 0


def test_sgd_update_multi(ws):
    """One call over a mixed batch equals the oracle tensor by tensor: several
    launch classes, more small tensors than one launch holds, a large tensor
    of a narrow class, every group combination, an empty tensor."""
    announce("sgd_update_multi mixed batch")
    rng = np.random.default_rng(4242)
    shapes = [(17, 64)] * 26 + [(40, 256), (9, 1000), (12, 3072), (5, 4608), (3, 7), (0, 64), (33, 768), (1025, 2048)]
    cases, devs = [], []
    for i, (rows, cols) in enumerate(shapes):
        groups = GROUPS[i % len(GROUPS)]
        W, V, G = _upd_case(rng, rows, cols, groups, 40)
        cases.append((W, V, G))
        devs.append((qt_to_dev(W, rows=rows), qt_to_dev(V, rows=rows), qt_to_dev(G, rows=rows)))
    lr, mom = (5, -9), (7, -3)
    ie.ie_sgd_update_multi([d[0] for d in devs], [d[1] for d in devs], [d[2] for d in devs], lr, mom, ws=ws)
    for i, ((W, V, G), (Wd, Vd, Gd)) in enumerate(zip(cases, devs)):
        W2, V2 = o.sgd_update(W, V, G, o.Scalar(*lr), o.Scalar(*mom))
        assert_same(Vd, V2, f"velocity of tensor {i} {shapes[i]}")
        assert_same(Wd, W2, f"weight of tensor {i} {shapes[i]}")
    assert ws.status() == 0


def test_sgd_update_gap_sweep(ws):
    """Every exponent gap from -255 to 255 between the two terms of a sum."""
    announce("sgd_update gap sweep")
    rng = np.random.default_rng(77)
    rows, cols = 511, 64
    ev = np.arange(rows) % 200 - 128
    eg = (np.arange(rows) * 7 + 3) % 200 - 128
    W = o.QT(rng.integers(-128, 128, (rows, cols)).astype(np.int8), rng.integers(-60, 61, rows).astype(np.int8), R)
    V = o.QT(rng.integers(-128, 128, (rows, cols)).astype(np.int8), ev.astype(np.int8), R)
    G = o.QT(rng.integers(-128, 128, (rows, cols)).astype(np.int8), eg.astype(np.int8), R)
    lr, mom = (3, -2), (7, -3)
    # keep results in range: the oracle raises on overflow
    W2, V2 = o.sgd_update(W, V, G, o.Scalar(*lr), o.Scalar(*mom))
    Wd, Vd, Gd = qt_to_dev(W), qt_to_dev(V), qt_to_dev(G)
    ie.ie_sgd_update(Wd, Vd, Gd, lr, mom, ws=ws)
    assert_same(Vd, V2, "velocity gap sweep")
    assert_same(Wd, W2, "weight gap sweep")


def test_sgd_update_ties_decided_by_tiny_term(ws):
    announce("sgd_update ties decided by a far smaller term")
    W = o.qt([[0, 0, 0, 0]], [0], R)
    V = o.qt([[23, 23, -23, -23]], [3], R)
    G = o.QT(np.array([[1, -1, -1, 1]], dtype=np.int8), np.array([-100], dtype=np.int8), R)
    W2, V2 = o.sgd_update(W, V, G, o.Scalar(0, 0), o.Scalar(7, -3))
    assert V2.mant.tolist() == [[81, 80, -81, -80]]
    Wd, Vd, Gd = qt_to_dev(W), qt_to_dev(V), qt_to_dev(G)
    ie.ie_sgd_update(Wd, Vd, Gd, (0, 0), (7, -3), ws=ws)
    assert_same(Vd, V2, "tie velocity")
    assert_same(Wd, W2, "tie weight")
