"""GPU parity at mantissa widths below INT8 ("Memory-Efficient Integer-Only
Training of Deep Neural Networks", Table 4: B = 7, 6, 5, 4, the velocity kept
INT8): every product epilogue (direct with one shift or per-element shifts,
the fp32 and integer row paths, round-to-odd, split with either finalize, the
paired convolution backward), the fused ReLU, ReLU6's cap, Sum and the SGD
update, called through the C ABI with the output's width in ie_mat.bits and
compared with the oracle bit for bit."""

import numpy as np
import pytest

import oracle as o
from integer_only_dnn_amd import ie
from tests.gpu_util import announce, assert_same, qt_to_dev

pytestmark = pytest.mark.gpu

T, R = o.TENSOR, o.ROW
BITS = [4, 5, 6, 7]


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


def rand_b(rng, shape, group, bits, elo=-14, ehi=-2, zero_frac=0.0):
    """A (C, e) tensor whose mantissas fit B bits."""
    qm = o.q_max(bits)
    m = rng.integers(-qm, qm + 1, size=shape).astype(np.int8)
    if zero_frac:
        m[rng.random(shape) < zero_frac] = 0
    n = shape[0] if group == R else 1
    return o.QT(m, rng.integers(elo, ehi + 1, size=n).astype(np.int8), group)


def empty(rows, cols, group, bits):
    return ie.Mat.empty(rows, cols, group, bits=bits)


def _relu(t: o.QT) -> o.QT:
    return o.QT(o.relu_fwd(t.mant).astype(np.int8), t.exp, t.group)


# (mode, splits): 0 = direct (one tile holds every group), 1 = round-to-odd
# two-pass, 2 = split contraction, 3 = recomputed
MODES = [(0, 1), (1, 1), (2, 2), (2, 3), (3, 1)]


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("mode", MODES, ids=lambda m: f"m{m[0]}s{m[1]}")
@pytest.mark.parametrize("k", [200, 1100], ids=["k200", "k1100"])
def test_dense_bits(bits, mode, k, ws, plan):
    """Linear forward (plain and with ReLU) and input gradient; K = 1100
    takes the integer row path, K = 200 the fp32 one; whole-tensor operands
    take the one-shift forms."""
    direct = mode[0] == 0
    M, N = (125, 123) if direct else (200, 150)
    announce(f"dense bits={bits} mode={mode} M={M} N={N} K={k}")
    rng = np.random.default_rng(1000 * bits + 10 * mode[0] + mode[1] + k)
    plan((2, 2), *mode)
    for gx, gw in ((T, T), (R, R), (T, R)):
        X = rand_b(rng, (M, k), gx, bits)
        W = rand_b(rng, (N, k), gw, bits)
        dY = rand_b(rng, (M, N), gx, bits)
        Xd, Wd, dYd = qt_to_dev(X), qt_to_dev(W), qt_to_dev(dY)
        for gy in (T, R):
            Y = empty(M, N, gy, bits)
            ie.ie_linear_fwd(Xd, Wd, Y, ws)
            assert_same(Y, o.linear_fwd(X, W, gy, bits), f"fwd X{gx} W{gw} Y{gy}")
            ie.ie_linear_fwd_act(Xd, Wd, Y, ie.ACT_RELU, ws)
            assert_same(Y, _relu(o.linear_fwd(X, W, gy, bits)), f"fwd relu X{gx} W{gw} Y{gy}")
            if direct:
                continue  # dX [M x K] spans several tiles: no direct plan for it
            dX = empty(M, k, gy, bits)
            ie.ie_linear_bwd_dx(dYd, Wd, dX, ws)
            assert_same(dX, o.linear_bwd_dx(dY, W, gy, bits), f"dX dY{gx} W{gw} dX{gy}")
    assert ws.status() == 0


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("splits", [1, 3])
def test_wgrad_bits(bits, splits, ws, plan):
    """Weight gradients through the fused row finalize (ROW) and the
    two-pass finalize (TENSOR)."""
    announce(f"wgrad bits={bits} splits={splits}")
    rng = np.random.default_rng(77 * bits + splits)
    M, N, K = 700, 150, 100
    dY = rand_b(rng, (M, N), R, bits)
    X = rand_b(rng, (M, K), T, bits)
    plan(wtile=(2, 2), wsplits=splits)
    for g in (T, R):
        dW = empty(N, K, g, bits)
        ie.ie_linear_bwd_dw(qt_to_dev(dY), qt_to_dev(X), dW, ws)
        assert_same(dW, o.linear_bwd_dw(dY, X, g, bits), f"dW group {g}")
    assert ws.status() == 0


@pytest.mark.parametrize("bits", BITS)
def test_conv_bits(bits, ws, plan):
    """Convolution forward (plain and with ReLU), and the backward pass both
    as the paired launch (dX round-to-odd, dW split by rows) and as separate
    products (dW whole-tensor)."""
    shape = (2, 9, 9, 32, 40, 3, 3, 2, 1)
    n, h, w, c, k, r, s, st, pad = shape
    announce(f"conv bits={bits} shape={shape}")
    d, dd = o.ConvShape(*shape), ie.conv_desc(*shape)
    rng = np.random.default_rng(500 + bits)
    X = rand_b(rng, (n, h, w, c), T, bits, zero_frac=0.3)
    W = rand_b(rng, (k, r * s * c), T, bits)
    dY = rand_b(rng, (n, d.p, d.q, k), T, bits)
    Xd, Wd, dYd = qt_to_dev(X, rows=n * h * w), qt_to_dev(W), qt_to_dev(dY, rows=n * d.p * d.q)
    Y = empty(n * d.p * d.q, k, T, bits)
    ie.ie_conv_fwd(dd, Xd, Wd, Y, ws)
    assert_same(Y, o.conv_fwd(d, X, W, T, bits), "conv fwd")
    ie.ie_conv_fwd_act(dd, Xd, Wd, Y, ie.ACT_RELU, ws)
    assert_same(Y, _relu(o.conv_fwd(d, X, W, T, bits)), "conv fwd relu")
    dX = empty(n * h * w, c, T, bits)
    dW = empty(k, r * s * c, R, bits)
    plan((2, 1), 1, 1, (1, 1), 3)   # the paired launch's plans
    ie.ie_conv_bwd(dd, Xd, Wd, dYd, dX, dW, ws)
    assert_same(dX, o.conv_dgrad(d, dY, W, T, bits), "conv dgrad (pair)")
    assert_same(dW, o.conv_wgrad(d, dY, X, R, bits), "conv wgrad (pair)")
    plan()
    dWt = empty(k, r * s * c, T, bits)
    ie.ie_conv_bwd(dd, Xd, Wd, dYd, None, dWt, ws)
    assert_same(dWt, o.conv_wgrad(d, dY, X, T, bits), "conv wgrad tensor")
    assert ws.status() == 0


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("group", [T, R], ids=["T", "R"])
def test_relu6_bits(bits, group):
    """ReLU6's cap min(6 * 2^-e, 2^(B-1) - 1) in the forward clip and the
    backward mask, with exponents on both sides of where the width decides."""
    rows, cols = 37, 45
    announce(f"relu6 bits={bits} group={group}")
    rng = np.random.default_rng(900 + 2 * bits + group)
    X = rand_b(rng, (rows, cols), group, bits, elo=-6, ehi=2, zero_frac=0.1)
    re = X.row_exp()
    want = o.QT(np.stack([o.relu6_fwd(X.mant[i], int(re[i]), bits) for i in range(rows)]).astype(np.int8),
                X.exp, group)
    Y = empty(rows, cols, group, bits)
    ie.ie_relu_fwd(qt_to_dev(X), Y, True)
    assert_same(Y, want, "relu6 fwd")
    # a forward output with values at the width's cap, to hit the mask edge
    Yc = rand_b(rng, (rows, cols), group, bits, elo=-6, ehi=2)
    Yc.mant[:, :5] = o.q_max(bits)
    dY = rand_b(rng, (rows, cols), group, 8)
    rc = Yc.row_exp()
    want_b = o.QT(np.stack([o.relu6_bwd(dY.mant[i], Yc.mant[i], int(rc[i]), bits) for i in range(rows)])
                  .astype(np.int8), dY.exp, group)
    Ycd = qt_to_dev(Yc)
    Ycd.bits = bits
    dX = empty(rows, cols, group, 8)
    ie.ie_relu_bwd(qt_to_dev(dY), Ycd, dX, True)
    assert_same(dX, want_b, "relu6 bwd")


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("groups", [(T, T, T), (R, T, R), (T, R, T), (R, R, R)],
                         ids=lambda g: "".join("TR"[x] for x in g))
def test_add_bits(bits, groups, ws):
    """Sum rounded to B bits, over exponent spans that take the int32 form,
    the int64 form and the far-term stand-in."""
    ga, gb, gz = groups
    rows, cols = 129, 200
    announce(f"add bits={bits} groups={groups}")
    rng = np.random.default_rng(40 * bits + 4 * ga + 2 * gb + gz)
    for span in (3, 20, 60):
        A = rand_b(rng, (rows, cols), ga, bits, elo=-20, ehi=-20 + span, zero_frac=0.05)
        B = rand_b(rng, (rows, cols), gb, bits, elo=-20, ehi=-20 + span, zero_frac=0.05)
        Z = empty(rows, cols, gz, bits)
        ie.ie_add(qt_to_dev(A), qt_to_dev(B), Z, ws)
        assert_same(Z, o.sum_op(A, B, gz, bits), f"add span={span}")
    assert ws.status() == 0


def _upd_case(rng, rows, cols, groups, bits, span=20):
    gw, gv, gg = groups
    W = rand_b(rng, (rows, cols), gw, bits, elo=-20, ehi=-20 + span)
    V = rand_b(rng, (rows, cols), gv, 8, elo=-30, ehi=-30 + span)
    G = rand_b(rng, (rows, cols), gg, bits, elo=-30, ehi=-30 + span)
    return W, V, G


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("shape", [(7, 33), (64, 256), (33, 1030)], ids=lambda s: f"{s[0]}x{s[1]}")
def test_update_bits(bits, shape, ws):
    """W' rounded to B bits, V' to INT8, with and without weight decay, over
    narrow and wide exponent gaps."""
    rows, cols = shape
    announce(f"sgd_update bits={bits} {rows}x{cols}")
    rng = np.random.default_rng(60 * bits + rows + cols)
    for groups in ((R, R, R), (T, R, R), (T, T, T), (R, T, T)):
        for span in (4, 60):
            for wd in ((0, 0), (1, -13)):
                W, V, G = _upd_case(rng, rows, cols, groups, bits, span)
                lr = (int(rng.integers(1, 128)), int(rng.integers(-9, -1)))
                mom = (115, -7)
                W2, V2 = o.sgd_update(W, V, G, o.Scalar(*lr), o.Scalar(*mom), o.Scalar(*wd), w_bits=bits)
                Wd, Vd, Gd = qt_to_dev(W), qt_to_dev(V), qt_to_dev(G)
                Wd.bits = bits
                ie.ie_sgd_update(Wd, Vd, Gd, lr, mom, wd, ws=ws)
                what = f"groups={groups} span={span} wd={wd}"
                assert_same(Vd, V2, f"velocity {what}")
                assert_same(Wd, W2, f"weight {what}")
    assert ws.status() == 0


@pytest.mark.parametrize("wd", [(0, 0), (1, -13)], ids=["nowd", "wd"])
def test_update_multi_mixed_widths(wd, ws):
    """One multi-tensor call over tensors of different widths (8 down to 4,
    small ones in the shared launch and a large one on its own), with and
    without weight decay: each weight takes its own width."""
    announce(f"sgd_update_multi mixed widths wd={wd}")
    rng = np.random.default_rng(4242 + wd[0])
    shapes = [(3, 17), (64, 64), (10, 300), (5, 1000), (128, 96), (1025, 2048)]
    widths = [8, 7, 6, 5, 4, 6]
    lr, mom = (3, -5), (115, -7)
    cases, devs = [], []
    for (rows, cols), b in zip(shapes, widths):
        W, V, G = _upd_case(rng, rows, cols, (R, R, R), b)
        cases.append((W, V, G, b))
        Wd, Vd, Gd = qt_to_dev(W), qt_to_dev(V), qt_to_dev(G)
        Wd.bits = b
        devs.append((Wd, Vd, Gd))
    ie.ie_sgd_update_multi([d[0] for d in devs], [d[1] for d in devs], [d[2] for d in devs], lr, mom, wd, ws=ws)
    for (W, V, G, b), (Wd, Vd, Gd) in zip(cases, devs):
        W2, V2 = o.sgd_update(W, V, G, o.Scalar(*lr), o.Scalar(*mom), o.Scalar(*wd), w_bits=b)
        assert_same(Vd, V2, f"velocity {W.mant.shape} bits={b}")
        assert_same(Wd, W2, f"weight {W.mant.shape} bits={b}")
    assert ws.status() == 0
