"""GPU parity of every execution plan: each instantiated workgroup tile, with
each epilogue (groups inside one tile, two-pass round-to-odd, split
contraction with the fused row finalize or the two-pass whole-tensor
finalize), forced through the planner's tuning overrides on ragged shapes,
bit-exact against the oracle."""

import numpy as np
import pytest

import oracle as o
from integer_only_dnn_amd import ie
from tests.gpu_util import announce, assert_same, qt_to_dev, rand_qt

pytestmark = pytest.mark.gpu

T, R = o.TENSOR, o.ROW
DENSE_TILES = [(2, 2), (4, 1), (1, 4), (2, 1), (1, 2), (1, 1)]
CONV_TILES = [(2, 2), (4, 1), (2, 1), (1, 1)]
WGRAD_TILES = [(2, 2), (1, 4), (4, 1), (1, 1)]
# (mode, splits): 1 = round-to-odd two-pass, 2 = split contraction,
# 3 = recomputed (group maxima first, then the product rounded directly)
MODES = [(1, 1), (2, 2), (2, 3), (3, 1)]


@pytest.fixture(scope="module")
def ws():
    return ie.Workspace("cuda")


@pytest.fixture
def plan(monkeypatch):
    def force(tile=None, mode=None, splits=1, wtile=None, wsplits=1):
        if tile is None:
            monkeypatch.delenv("IE_TILE", raising=False)
        else:
            monkeypatch.setenv("IE_TILE", f"{tile[0]},{tile[1]},{mode},{splits}")
        if wtile is None:
            monkeypatch.delenv("IE_WTILE", raising=False)
        else:
            monkeypatch.setenv("IE_WTILE", f"{wtile[0]},{wtile[1]},{wsplits}")
    yield force
    monkeypatch.delenv("IE_TILE", raising=False)
    monkeypatch.delenv("IE_WTILE", raising=False)


DENSE_CASES = [(t, m) for t in DENSE_TILES for m in MODES]


@pytest.mark.parametrize("tile,mode", DENSE_CASES,
                         ids=[f"{64 * t[0]}x{64 * t[1]}-m{m[0]}s{m[1]}" for t, m in DENSE_CASES])
def test_dense_plans(tile, mode, ws, plan):
    M, N, K = 200, 150, 392
    announce(f"dense plans tile={tile} mode={mode} M={M} N={N} K={K}")
    rng = np.random.default_rng(11 * tile[0] + 7 * tile[1] + 3 * mode[0] + mode[1])
    X = rand_qt(rng, (M, K), R)
    W = rand_qt(rng, (N, K), R)
    dY = rand_qt(rng, (M, N), R)
    Xd, Wd, dYd = qt_to_dev(X), qt_to_dev(W), qt_to_dev(dY)
    plan(tile, *mode)
    for gy in (T, R):
        Y = ie.Mat.empty(M, N, gy)
        ie.ie_linear_fwd(Xd, Wd, Y, ws)
        assert_same(Y, o.linear_fwd(X, W, gy), f"fwd group {gy}")
        dX = ie.Mat.empty(M, K, gy)
        ie.ie_linear_bwd_dx(dYd, Wd, dX, ws)
        assert_same(dX, o.linear_bwd_dx(dY, W, gy), f"dX group {gy}")
    assert ws.status() == 0


@pytest.mark.parametrize("tile", DENSE_TILES, ids=lambda t: f"{64 * t[0]}x{64 * t[1]}")
def test_dense_direct(tile, ws, plan):
    # one tile holds every group: the epilogue rounds in place
    M, N, K = 64 * tile[0] - 3, 64 * tile[1] - 5, 200
    announce(f"dense direct tile={tile} M={M} N={N} K={K}")
    rng = np.random.default_rng(5 + tile[0] * 3 + tile[1])
    X = rand_qt(rng, (M, K), R)
    W = rand_qt(rng, (N, K), T)
    plan(tile, 0, 1)
    for gy in (T, R):
        Y = ie.Mat.empty(M, N, gy)
        ie.ie_linear_fwd(qt_to_dev(X), qt_to_dev(W), Y, ws)
        assert_same(Y, o.linear_fwd(X, W, gy), f"direct group {gy}")


@pytest.mark.parametrize("M,N,K", [(200, 129, 392), (3000, 197, 64), (3000, 256, 392), (1000, 197, 300),
                                   (64, 197, 1100)])
def test_dense_planner_wide_rows(M, N, K, ws, plan):
    # the planner's own choice for row groups of 129..256 results (a 64 x 256
    # tile holding whole rows, one pass; the split plan for few long rows)
    announce(f"dense planner wide rows M={M} N={N} K={K}")
    rng = np.random.default_rng(M + N + K)
    X = rand_qt(rng, (M, K), R)
    W = rand_qt(rng, (N, K), R)
    plan()
    for gy in (R, T):
        Y = ie.Mat.empty(M, N, gy)
        ie.ie_linear_fwd(qt_to_dev(X), qt_to_dev(W), Y, ws)
        assert_same(Y, o.linear_fwd(X, W, gy), f"fwd group {gy}")
    # an input gradient with rows of N results: dY2 [M x K] . W2 [K x N]
    dY2 = rand_qt(rng, (M, K), R)
    W2 = rand_qt(rng, (K, N), R)
    dX = ie.Mat.empty(M, N, R)
    ie.ie_linear_bwd_dx(qt_to_dev(dY2), qt_to_dev(W2), dX, ws)
    assert_same(dX, o.linear_bwd_dx(dY2, W2, R), "dX group R")
    assert ws.status() == 0


def _relu(t: o.QT) -> o.QT:
    return o.QT(o.relu_fwd(t.mant).astype(np.int8), t.exp, t.group)


@pytest.mark.parametrize("tile", [(2, 2), (1, 1), (2, 1)], ids=lambda t: f"{64 * t[0]}x{64 * t[1]}")
@pytest.mark.parametrize("mode", [(0, 1)] + MODES, ids=lambda m: f"m{m[0]}s{m[1]}")
def test_fused_relu_plans(tile, mode, ws, plan):
    """The forward products with ReLU fused into their output equal the
    oracle's ReLU of the plain product, through every epilogue (direct,
    round-to-odd, split with the row finalize or the whole-tensor one)."""
    direct = mode[0] == 0
    M, N, K = (64 * tile[0] - 3, 64 * tile[1] - 5, 200) if direct else (200, 150, 392)
    announce(f"fused relu tile={tile} mode={mode} M={M} N={N} K={K}")
    rng = np.random.default_rng(3 * tile[0] + tile[1] + 17 * mode[0] + mode[1])
    X = rand_qt(rng, (M, K), R)
    W = rand_qt(rng, (N, K), R)
    Xd, Wd = qt_to_dev(X), qt_to_dev(W)
    plan(tile, *mode)
    for gy in (T, R):
        Y = ie.Mat.empty(M, N, gy)
        ie.ie_linear_fwd_act(Xd, Wd, Y, ie.ACT_RELU, ws)
        assert_same(Y, _relu(o.linear_fwd(X, W, gy)), f"linear relu group {gy}")
    if not direct:
        shape = (2, 10, 10, 32, 40, 3, 3, 1, 1)
        d, dd = o.ConvShape(*shape), ie.conv_desc(*shape)
        Xc = rand_qt(rng, (2, 10, 10, 32), T, zero_frac=0.2)
        Wc = rand_qt(rng, (40, 288), T)
        Y = ie.Mat.empty(2 * d.p * d.q, 40, T)
        ie.ie_conv_fwd_act(dd, qt_to_dev(Xc, rows=200), qt_to_dev(Wc), Y, ie.ACT_RELU, ws)
        assert_same(Y, _relu(o.conv_fwd(d, Xc, Wc, T)), "conv relu")
        Y0 = ie.Mat.empty(2 * d.p * d.q, 40, T)
        ie.ie_conv_fwd_act(dd, qt_to_dev(Xc, rows=200), qt_to_dev(Wc), Y0, ie.ACT_NONE, ws)
        assert_same(Y0, o.conv_fwd(d, Xc, Wc, T), "conv act none")
    assert ws.status() == 0


# 24 channels: the input gradient reads a transposed, aligned copy of W;
# 32 / 48 channels with a whole-tensor W: it reads W in place
CONV_CASES = [(2, 10, 10, 24, 40, 3, 3, 1, 1), (2, 9, 9, 24, 40, 3, 3, 2, 1),
              (2, 10, 10, 32, 40, 3, 3, 1, 1), (2, 9, 9, 48, 24, 3, 3, 2, 1),
              # 1x1, stride 1, no padding: the dense product kernels
              (2, 10, 10, 24, 40, 1, 1, 1, 0), (3, 9, 9, 32, 48, 1, 1, 1, 0)]


@pytest.mark.parametrize("shape", CONV_CASES, ids=lambda s: f"c{s[3]}r{s[5]}st{s[7]}")
@pytest.mark.parametrize("tile", CONV_TILES, ids=lambda t: f"{64 * t[0]}x{64 * t[1]}")
@pytest.mark.parametrize("mode", [(1, 1), (2, 2), (3, 1)], ids=lambda m: f"m{m[0]}s{m[1]}")
@pytest.mark.parametrize("wg", [T, R], ids=["WT", "WR"])
def test_conv_plans(shape, tile, mode, wg, ws, plan):
    n, h, w, c, k, r, s, st, pad = shape
    announce(f"conv plans shape={shape} tile={tile} mode={mode} w_group={wg}")
    d = o.ConvShape(*shape)
    dd = ie.conv_desc(*shape)
    rng = np.random.default_rng(sum(shape) + 13 * tile[0] + tile[1] + mode[1] + 7 * wg)
    X = rand_qt(rng, (n, h, w, c), T, zero_frac=0.2)
    W = rand_qt(rng, (k, r * s * c), wg)
    dY = rand_qt(rng, (n, d.p, d.q, k), T)
    Xd, Wd, dYd = qt_to_dev(X, rows=n * h * w), qt_to_dev(W), qt_to_dev(dY, rows=n * d.p * d.q)
    plan(tile, *mode)
    Y = ie.Mat.empty(n * d.p * d.q, k, T)
    ie.ie_conv_fwd(dd, Xd, Wd, Y, ws)
    assert_same(Y, o.conv_fwd(d, X, W, T), "conv fwd")
    dX = ie.Mat.empty(n * h * w, c, T)
    ie.ie_conv_bwd(dd, Xd, Wd, dYd, dX, None, ws)
    want_dx = o.conv_dgrad(d, dY, W, T)
    assert_same(dX, want_dx, "conv dgrad")
    # both gradients in one call: the paired grid where its kernels cover
    # the plans (round-to-odd or recomputed input gradient)
    dX2 = ie.Mat.empty(n * h * w, c, T)
    dW = ie.Mat.empty(k, r * s * c, R)
    ie.ie_conv_bwd(dd, Xd, Wd, dYd, dX2, dW, ws)
    assert_same(dX2, want_dx, "conv dgrad (paired)")
    assert_same(dW, o.conv_wgrad(d, dY, X, R), "conv wgrad (paired)")
    assert ws.status() == 0


# Stride-2 input gradients, decomposed into stride phases: kernels 1x1 (three
# phases without taps), 2x2, 3x3, 4x4 and 5x5, odd, unequal and one-pixel
# images, more output channels than one contraction step; with the
# planner's tile and every tile forced with the recomputed epilogue, alone
# and paired with the weight gradient.
PHASE_CASES = [(2, 9, 9, 16, 24, 1, 1, 2, 0), (3, 7, 5, 32, 40, 1, 1, 2, 0), (2, 8, 8, 16, 16, 1, 1, 2, 1),
               (1, 1, 1, 16, 16, 1, 1, 2, 0), (2, 2, 3, 16, 16, 3, 3, 2, 1), (2, 11, 6, 20, 30, 5, 5, 2, 2),
               (2, 6, 11, 16, 16, 2, 2, 2, 0), (2, 12, 12, 16, 48, 4, 4, 2, 1), (4, 5, 5, 16, 300, 3, 3, 2, 1),
               (2, 20, 20, 64, 64, 3, 3, 2, 1)]


@pytest.mark.parametrize("shape", PHASE_CASES, ids=lambda s: "n{}h{}w{}c{}k{}r{}s{}p{}".format(*s[:7], s[8]))
@pytest.mark.parametrize("tile", [None] + CONV_TILES, ids=lambda t: "planner" if t is None else f"{64 * t[0]}x{64 * t[1]}")
def test_conv_phases(shape, tile, ws, plan):
    n, h, w, c, k, r, s, st, pad = shape
    announce(f"conv phases shape={shape} tile={tile}")
    d, dd = o.ConvShape(*shape), ie.conv_desc(*shape)
    rng = np.random.default_rng(sum(shape) * 7 + (tile or (0, 0))[0])
    X = rand_qt(rng, (n, h, w, c), T, zero_frac=0.2)
    W = rand_qt(rng, (k, r * s * c), R if k % 2 == 0 else T)
    dY = rand_qt(rng, (n, d.p, d.q, k), T)
    Xd, Wd, dYd = qt_to_dev(X, rows=n * h * w), qt_to_dev(W), qt_to_dev(dY, rows=n * d.p * d.q)
    if tile is not None:
        plan(tile, 3, 1)
    want_dx = o.conv_dgrad(d, dY, W, T)
    dX = ie.Mat.empty(n * h * w, c, T)
    ie.ie_conv_bwd(dd, Xd, Wd, dYd, dX, None, ws)
    assert_same(dX, want_dx, "conv dgrad")
    dX2 = ie.Mat.empty(n * h * w, c, T)
    dW = ie.Mat.empty(k, r * s * c, R)
    ie.ie_conv_bwd(dd, Xd, Wd, dYd, dX2, dW, ws)
    assert_same(dX2, want_dx, "conv dgrad (paired)")
    assert_same(dW, o.conv_wgrad(d, dY, X, R), "conv wgrad (paired)")
    assert ws.status() == 0


@pytest.mark.parametrize("shape", [(2, 9, 9, 24, 40, 3, 3, 2, 1), (2, 10, 10, 32, 40, 3, 3, 1, 1)],
                         ids=["st2", "st1"])
def test_conv_dgrad_row_groups(shape, ws):
    # one exponent per input pixel: never decomposed, never paired (its
    # epilogue keeps a row per pixel); alone and with the weight gradient
    n, h, w, c, k, r, s, st, pad = shape
    announce(f"conv dgrad row groups shape={shape}")
    d, dd = o.ConvShape(*shape), ie.conv_desc(*shape)
    rng = np.random.default_rng(sum(shape) + 99)
    X = rand_qt(rng, (n, h, w, c), T)
    W = rand_qt(rng, (k, r * s * c), R)
    dY = rand_qt(rng, (n, d.p, d.q, k), T)
    Xd, Wd, dYd = qt_to_dev(X, rows=n * h * w), qt_to_dev(W), qt_to_dev(dY, rows=n * d.p * d.q)
    want = o.conv_dgrad(d, dY, W, R)
    dX = ie.Mat.empty(n * h * w, c, R)
    ie.ie_conv_bwd(dd, Xd, Wd, dYd, dX, None, ws)
    assert_same(dX, want, "row-grouped dgrad")
    dX2 = ie.Mat.empty(n * h * w, c, R)
    dW = ie.Mat.empty(k, r * s * c, R)
    ie.ie_conv_bwd(dd, Xd, Wd, dYd, dX2, dW, ws)
    assert_same(dX2, want, "row-grouped dgrad with dW")
    assert_same(dW, o.conv_wgrad(d, dY, X, R), "wgrad with row-grouped dgrad")
    assert ws.status() == 0


@pytest.mark.parametrize("tile", WGRAD_TILES, ids=lambda t: f"{64 * t[0]}x{64 * t[1]}")
@pytest.mark.parametrize("splits", [1, 3, 7])
def test_wgrad_plans(tile, splits, ws, plan):
    announce(f"wgrad plans tile={tile} splits={splits}")
    rng = np.random.default_rng(17 * tile[0] + 5 * tile[1] + splits)
    M, N, K = 700, 150, 100
    dY = rand_qt(rng, (M, N), R)
    X = rand_qt(rng, (M, K), T)
    plan(wtile=tile, wsplits=splits)
    for g in (T, R):
        dW = ie.Mat.empty(N, K, g)
        ie.ie_linear_bwd_dw(qt_to_dev(dY), qt_to_dev(X), dW, ws)
        assert_same(dW, o.linear_bwd_dw(dY, X, g), f"linear dW group {g}")
    shape = (2, 9, 9, 3, 40, 3, 3, 2, 1)   # 3 channels: padded source columns
    d = o.ConvShape(*shape)
    dd = ie.conv_desc(*shape)
    Xc = rand_qt(rng, (2, 9, 9, 3), T)
    Wc = rand_qt(rng, (40, 27), T)
    dYc = rand_qt(rng, (2, d.p, d.q, 40), T)
    for g in (T, R):
        dW = ie.Mat.empty(40, 27, g)
        ie.ie_conv_bwd(dd, qt_to_dev(Xc, rows=2 * 81), qt_to_dev(Wc), qt_to_dev(dYc, rows=2 * d.p * d.q), None, dW,
                       ws)
        assert_same(dW, o.conv_wgrad(d, dYc, Xc, g), f"conv dW group {g}")
    assert ws.status() == 0


# Input and weight gradient together: the paired kernel (both products in one
# grid) for every instantiated tile pair, forced through the overrides.
PAIR_D = [(2, 1), (1, 1), (2, 2)]
PAIR_W = [(1, 1), (2, 2)]


@pytest.mark.parametrize("dtile", PAIR_D, ids=lambda t: f"d{64 * t[0]}x{64 * t[1]}")
@pytest.mark.parametrize("wtile", PAIR_W, ids=lambda t: f"w{64 * t[0]}x{64 * t[1]}")
@pytest.mark.parametrize("wsplits", [1, 3])
def test_conv_bwd_pair(dtile, wtile, wsplits, ws, plan):
    shape = (2, 9, 9, 32, 40, 3, 3, 2, 1)
    n, h, w, c, k, r, s, st, pad = shape
    announce(f"conv bwd pair dtile={dtile} wtile={wtile} wsplits={wsplits} shape={shape}")
    d = o.ConvShape(*shape)
    dd = ie.conv_desc(*shape)
    rng = np.random.default_rng(31 * dtile[0] + 7 * dtile[1] + 5 * wtile[0] + wsplits)
    X = rand_qt(rng, (n, h, w, c), T, zero_frac=0.3)
    W = rand_qt(rng, (k, r * s * c), T)
    dY = rand_qt(rng, (n, d.p, d.q, k), T)
    plan(dtile, 1, 1, wtile, wsplits)
    dX = ie.Mat.empty(n * h * w, c, T)
    dW = ie.Mat.empty(k, r * s * c, R)
    ie.ie_conv_bwd(dd, qt_to_dev(X, rows=n * h * w), qt_to_dev(W), qt_to_dev(dY, rows=n * d.p * d.q), dX, dW, ws)
    assert_same(dX, o.conv_dgrad(d, dY, W, T), "conv dgrad")
    assert_same(dW, o.conv_wgrad(d, dY, X, R), "conv wgrad")
    assert ws.status() == 0
