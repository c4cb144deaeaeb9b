"""GPU parity of input gradients passed back through a ReLU in the same call
(ie_conv_bwd_act, ie_linear_bwd_dx_act): every way an input gradient is
stored (the direct epilogue, the round-to-odd finalize, the paired
finalize, the split finalizes, the recomputed and the stride-phased second
passes; 16-byte, 4-byte and byte-wise stores), bit-exact against the
oracle's input gradient followed by its ReLU backward (Table 7), and the
weight gradient unchanged."""

import numpy as np
import pytest
import torch

import oracle as o
from integer_only_dnn_amd import ie
from tests.gpu_util import announce, assert_same, qt_to_dev, rand_qt

pytestmark = pytest.mark.gpu

T, R = o.TENSOR, o.ROW


@pytest.fixture(scope="module")
def ws():
    return ie.Workspace("cuda")


@pytest.fixture
def plan(monkeypatch):
    def force(tile=None, mode=None, splits=1):
        if tile is None:
            monkeypatch.delenv("IE_TILE", raising=False)
        else:
            monkeypatch.setenv("IE_TILE", f"{tile[0]},{tile[1]},{mode},{splits}")
    yield force
    monkeypatch.delenv("IE_TILE", raising=False)


def _through_relu(dx: o.QT, X: o.QT) -> o.QT:
    """The oracle's input gradient passed through the ReLU whose output is X."""
    mask = np.asarray(X.mant).reshape(np.asarray(dx.mant).shape)
    return o.QT(o.relu_bwd(dx.mant, mask).astype(np.int8), dx.exp, dx.group)


# (mode, splits): None = the planner's plan; 0 direct, 1 round-to-odd,
# 2 split, 3 recomputed
CONV_MODES = [None, ((2, 2), 1, 1), ((1, 1), 1, 1), ((2, 2), 2, 3), ((1, 1), 3, 1), ((2, 1), 3, 1)]
# 24 channels: a transposed copy of W; 32 with a whole-tensor W: W in place;
# stride 2 with a whole-tensor dX: stride phases; 1x1 stride 1: the dense
# product kernels
CONV_SHAPES = [(2, 10, 10, 24, 40, 3, 3, 1, 1), (2, 10, 10, 32, 40, 3, 3, 1, 1), (2, 9, 9, 48, 24, 3, 3, 2, 1),
               (2, 10, 10, 24, 40, 1, 1, 1, 0), (4, 5, 5, 16, 300, 3, 3, 2, 1)]


@pytest.mark.parametrize("shape", CONV_SHAPES, ids=lambda s: f"c{s[3]}k{s[4]}r{s[5]}st{s[7]}")
@pytest.mark.parametrize("mode", CONV_MODES,
                         ids=lambda m: "planner" if m is None else f"{64 * m[0][0]}x{64 * m[0][1]}-m{m[1]}s{m[2]}")
@pytest.mark.parametrize("wg", [T, R], ids=["WT", "WR"])
def test_conv_bwd_relu(shape, mode, wg, ws, plan):
    n, h, w, c, k, r, s, st, pad = shape
    announce(f"conv bwd relu shape={shape} mode={mode} w_group={wg}")
    d, dd = o.ConvShape(*shape), ie.conv_desc(*shape)
    rng = np.random.default_rng(sum(shape) + 5 * wg + (0 if mode is None else 17 * mode[1] + mode[2]))
    # the mask's three cases: positive, zero and negative bytes
    X = rand_qt(rng, (n, h, w, c), T, zero_frac=0.4)
    W = rand_qt(rng, (k, r * s * c), wg)
    dY = rand_qt(rng, (n, d.p, d.q, k), T)
    Xd, Wd, dYd = qt_to_dev(X, rows=n * h * w), qt_to_dev(W), qt_to_dev(dY, rows=n * d.p * d.q)
    if mode is None:
        plan()
    else:
        plan(*mode)
    want_dx = _through_relu(o.conv_dgrad(d, dY, W, T), X)
    dX = ie.Mat.empty(n * h * w, c, T)
    ie.ie_conv_bwd_act(dd, Xd, Wd, dYd, dX, None, ie.ACT_RELU, ws)
    assert_same(dX, want_dx, "dX alone")
    dX2 = ie.Mat.empty(n * h * w, c, T)
    dW = ie.Mat.empty(k, r * s * c, R)
    ie.ie_conv_bwd_act(dd, Xd, Wd, dYd, dX2, dW, ie.ACT_RELU, ws)
    assert_same(dX2, want_dx, "dX with dW")
    assert_same(dW, o.conv_wgrad(d, dY, X, R), "dW")
    dX3 = ie.Mat.empty(n * h * w, c, T)
    ie.ie_conv_bwd_act(dd, Xd, Wd, dYd, dX3, None, ie.ACT_NONE, ws)
    assert_same(dX3, o.conv_dgrad(d, dY, W, T), "act none")
    assert ws.status() == 0


LINEAR_MODES = [None, ((2, 2), 0, 1), ((2, 2), 1, 1), ((1, 4), 1, 1), ((2, 2), 2, 2), ((1, 1), 2, 3),
                ((2, 1), 3, 1)]


def _unaligned(m: np.ndarray) -> torch.Tensor:
    """A device copy of m whose data starts one byte past a 16-byte boundary."""
    flat = torch.zeros(m.size + 16, dtype=torch.int8, device="cuda")
    v = flat[1:1 + m.size].view(m.shape)
    v.copy_(torch.from_numpy(np.ascontiguousarray(m)))
    return v


@pytest.mark.parametrize("mode", LINEAR_MODES,
                         ids=lambda m: "planner" if m is None else f"{64 * m[0][0]}x{64 * m[0][1]}-m{m[1]}s{m[2]}")
@pytest.mark.parametrize("M,N,K", [(200, 150, 392), (130, 96, 150), (64, 300, 128)])
def test_linear_bwd_dx_relu(mode, M, N, K, ws, plan):
    announce(f"linear bwd dx relu M={M} N={N} K={K} mode={mode}")
    rng = np.random.default_rng(M + 3 * N + 7 * K + (0 if mode is None else 11 * mode[1] + mode[2]))
    dY = rand_qt(rng, (M, N), R)
    W = rand_qt(rng, (N, K), R)
    X = rand_qt(rng, (M, K), R, zero_frac=0.3)
    dYd, Wd = qt_to_dev(dY), qt_to_dev(W)
    if mode is None:
        plan()
    else:
        if mode[1] == 0 and (M > 64 * mode[0][0] or K > 64 * mode[0][1]):
            pytest.skip("the direct epilogue needs every group inside one tile")
        plan(*mode)
    for gx in (R, T):
        want = _through_relu(o.linear_bwd_dx(dY, W, gx), X)
        # the mask aligned, and one byte off a 16-byte boundary (byte-wise forms)
        for Xmant in (torch.from_numpy(X.mant.copy()).cuda(), _unaligned(X.mant)):
            Xd = ie.Mat(Xmant, torch.from_numpy(X.exp.copy()).cuda(), X.group)
            dX = ie.Mat.empty(M, K, gx)
            ie.ie_linear_bwd_dx_act(dYd, Wd, Xd, dX, ie.ACT_RELU, ws)
            assert_same(dX, want, f"dX group {gx} mask at +{Xmant.data_ptr() % 16}")
    assert ws.status() == 0


def test_act_bwd_refusals(ws):
    announce("act bwd refusals")
    rng = np.random.default_rng(3)
    dY, W, X = rand_qt(rng, (64, 32), T), rand_qt(rng, (32, 48), T), rand_qt(rng, (64, 48), T)
    dYd, Wd, Xd = qt_to_dev(dY), qt_to_dev(W), qt_to_dev(X)
    with pytest.raises(ie.IeError):
        ie.ie_linear_bwd_dx_act(dYd, Wd, Xd, ie.Mat.empty(64, 48, T), 2, ws)  # no such activation
    with pytest.raises(ie.IeError):
        ie.ie_linear_bwd_dx_act(dYd, Wd, qt_to_dev(rand_qt(rng, (64, 40), T)), ie.Mat.empty(64, 48, T),
                                ie.ACT_RELU, ws)  # mask of another shape
    with pytest.raises(ie.IeError):
        ie.ie_linear_bwd_dx_act(dYd, Wd, Xd, Xd, ie.ACT_RELU, ws)  # dX is the mask
    shape = (2, 6, 6, 16, 16, 3, 3, 1, 1)
    d, dd = o.ConvShape(*shape), ie.conv_desc(*shape)
    Xc = qt_to_dev(rand_qt(rng, (2, 6, 6, 16), T), rows=72)
    Wc = qt_to_dev(rand_qt(rng, (16, 144), T))
    dYc = qt_to_dev(rand_qt(rng, (2, d.p, d.q, 16), T), rows=2 * d.p * d.q)
    with pytest.raises(ie.IeError):
        ie.ie_conv_bwd_act(dd, Xc, Wc, dYc, ie.Mat.empty(72, 16, T), None, 3, ws)
    with pytest.raises(ie.IeError):
        ie.ie_conv_bwd_act(dd, Xc, Wc, dYc, Xc, None, ie.ACT_RELU, ws)
