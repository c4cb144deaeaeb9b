"""GPU parity of the pointwise steps: ReLU / ReLU6 forward and backward masks
(Table 7) and the exact Sum (Table 6), called through the C ABI and compared
with the oracle bit for bit, over ragged shapes, both group kinds, in-place
calls and the degenerate cases."""

import numpy as np
import pytest
import torch

import oracle as o
from integer_only_dnn_amd import ie
from tests.gpu_util import announce, assert_same, qt_to_dev, rand_qt

pytestmark = pytest.mark.gpu

T, R = o.TENSOR, o.ROW
SHAPES = [(1, 1), (3, 5), (7, 16), (33, 17), (64, 256), (129, 1000), (1000, 3), (0, 8), (4, 0)]


@pytest.fixture(scope="module")
def ws():
    return ie.Workspace("cuda")


def _relu_want(X: o.QT, relu6: bool) -> o.QT:
    if not relu6:
        return o.QT(o.relu_fwd(X.mant).astype(np.int8), X.exp, X.group)
    re = X.row_exp() if X.mant.shape[0] else np.zeros(0, dtype=np.int64)
    m = np.stack([o.relu6_fwd(X.mant[i], int(re[i])) for i in range(X.mant.shape[0])]) \
        if X.mant.shape[0] else X.mant.astype(np.int64)
    return o.QT(m.reshape(X.mant.shape).astype(np.int8), X.exp, X.group)


def _relu_bwd_want(dY: o.QT, Y: o.QT, relu6: bool) -> o.QT:
    if not relu6:
        return o.QT(o.relu_bwd(dY.mant, Y.mant).astype(np.int8), dY.exp, dY.group)
    re = Y.row_exp() if Y.mant.shape[0] else np.zeros(0, dtype=np.int64)
    m = np.stack([o.relu6_bwd(dY.mant[i], Y.mant[i], int(re[i])) for i in range(Y.mant.shape[0])]) \
        if Y.mant.shape[0] else dY.mant.astype(np.int64)
    return o.QT(m.reshape(dY.mant.shape).astype(np.int8), dY.exp, dY.group)


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("group", [T, R], ids=["T", "R"])
@pytest.mark.parametrize("relu6", [False, True], ids=["relu", "relu6"])
def test_relu_fwd_bwd(shape, group, relu6):
    rows, cols = shape
    announce(f"relu{'6' if relu6 else ''} {rows}x{cols} group={group}")
    rng = np.random.default_rng(rows * 31 + cols + 7 * group + relu6)
    # exponents around the ReLU6 cap's regimes: 6 >> e (e >= 0), 6 << -e, capped at 127
    X = rand_qt(rng, (rows, cols), group, elo=-7, ehi=3, zero_frac=0.1)
    want = _relu_want(X, relu6)
    Xd = qt_to_dev(X)
    Y = ie.Mat.empty(rows, cols, group)
    ie.ie_relu_fwd(Xd, Y, relu6)
    assert_same(Y, want, "relu_fwd")
    # in place
    ie.ie_relu_fwd(Xd, Xd, relu6)
    assert_same(Xd, want, "relu_fwd in place")

    dY = rand_qt(rng, (rows, cols), group)
    want_b = _relu_bwd_want(dY, want, relu6)
    dYd = qt_to_dev(dY)
    dX = ie.Mat.empty(rows, cols, group)
    ie.ie_relu_bwd(dYd, Y, dX, relu6)
    assert_same(dX, want_b, "relu_bwd")
    ie.ie_relu_bwd(dYd, Y, dYd, relu6)
    assert_same(dYd, want_b, "relu_bwd in place")


def test_relu_bwd_mask_edges():
    """Mask at 0 and at the ReLU6 cap exactly, and -128 gradients kept."""
    announce("relu masks at 0 and at the cap")
    C = np.array([[-128, -1, 0, 1, 95, 96, 97, 127]], dtype=np.int8)
    e = np.array([-4], dtype=np.int8)  # cap 96
    dy = np.full((1, 8), -128, dtype=np.int8)
    Y = o.QT(C, e, R)
    dY = o.QT(dy, np.array([-3], dtype=np.int8), R)
    for relu6 in (False, True):
        dX = ie.Mat.empty(1, 8, R)
        ie.ie_relu_bwd(qt_to_dev(dY), qt_to_dev(Y), dX, relu6)
        assert_same(dX, _relu_bwd_want(dY, Y, relu6), f"edges relu6={relu6}")


ADD_SHAPES = [(1, 1), (5, 7), (64, 256), (129, 1000), (1500, 40), (0, 5), (3, 0)]


@pytest.mark.parametrize("shape", ADD_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("groups", [(T, T, T), (R, T, T), (T, R, R), (R, R, R), (R, R, T), (T, T, R)],
                         ids=lambda g: "".join("TR"[x] for x in g))
def test_add(shape, groups, ws):
    rows, cols = shape
    ga, gb, gz = groups
    announce(f"add {rows}x{cols} groups={groups}")
    rng = np.random.default_rng(rows * 13 + cols + 100 * ga + 10 * gb + gz)
    for span in (3, 20, 60):
        A = rand_qt(rng, (rows, cols), ga, elo=-20, ehi=-20 + span, zero_frac=0.05)
        B = rand_qt(rng, (rows, cols), gb, elo=-20, ehi=-20 + span, zero_frac=0.05)
        want = o.sum_op(A, B, gz)
        Z = ie.Mat.empty(rows, cols, gz)
        ie.ie_add(qt_to_dev(A), qt_to_dev(B), Z, ws)
        assert_same(Z, want, f"add span={span}")
    assert ws.status() == 0


def test_add_gap_sweep(ws):
    """Every exponent gap from -80 to 80 between the two terms (row-grouped
    operands, one gap per row), including the exact cancellations and the
    ties that the far smaller term decides."""
    announce("add gap sweep")
    rng = np.random.default_rng(99)
    gaps = np.arange(-80, 81)
    rows, cols = len(gaps), 64
    ea = np.full(rows, -40, dtype=np.int64)
    eb = ea - gaps
    ma = rng.integers(-128, 128, size=(rows, cols)).astype(np.int8)
    mb = rng.integers(-128, 128, size=(rows, cols)).astype(np.int8)
    # exact cancellation at gap 0, odd mantissas (ties after one shift) elsewhere
    mb[gaps == 0, :8] = -ma[gaps == 0, :8].clip(-127, 127)
    ma[:, 8:16] |= 1
    A = o.QT(ma, np.clip(ea, -128, 127).astype(np.int8), R)
    B = o.QT(mb, np.clip(eb, -128, 127).astype(np.int8), R)
    for gz in (R, T):
        want = o.sum_op(A, B, gz)
        Z = ie.Mat.empty(rows, cols, gz)
        ie.ie_add(qt_to_dev(A), qt_to_dev(B), Z, ws)
        assert_same(Z, want, f"gap sweep out group={gz}")
    assert ws.status() == 0


def test_add_tensor_gaps(ws):
    """Whole-tensor operands at every exponent gap from -30 to 30 (the int32
    form covers gaps up to 22), into both output group kinds."""
    announce("add whole-tensor gaps")
    rng = np.random.default_rng(5)
    for gap in range(-30, 31):
        A = o.QT(rng.integers(-128, 128, size=(37, 45)).astype(np.int8), np.array([-40], np.int8), T)
        B = o.QT(rng.integers(-128, 128, size=(37, 45)).astype(np.int8), np.array([-40 - gap], np.int8), T)
        for gz in (T, R):
            Z = ie.Mat.empty(37, 45, gz)
            ie.ie_add(qt_to_dev(A), qt_to_dev(B), Z, ws)
            assert_same(Z, o.sum_op(A, B, gz), f"gap {gap} out group={gz}")
    assert ws.status() == 0


def test_add_zero_and_overflow(ws):
    """All-zero sums give E_MIN; a sum whose exponent would pass 127 raises
    the sticky range flag."""
    announce("add zeros and exponent overflow")
    z = o.QT(np.zeros((4, 9), dtype=np.int8), np.array([5], dtype=np.int8), T)
    Z = ie.Mat.empty(4, 9, R)
    ie.ie_add(qt_to_dev(z), qt_to_dev(z), Z, ws)
    assert_same(Z, o.sum_op(z, z, R), "zeros")
    big = o.QT(np.full((2, 3), 127, dtype=np.int8), np.array([127], dtype=np.int8), T)
    Z = ie.Mat.empty(2, 3, T)
    ie.ie_add(qt_to_dev(big), qt_to_dev(big), Z, ws)
    assert ws.status() == ie.FLAG_EXP_RANGE
