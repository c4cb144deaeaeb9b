"""Guard regions around every buffer the library is given, for every plan
the planner can take: each output's mantissas and exponents, each input, and
a workspace of exactly the size its query returns sit between 4 KiB guards
filled with a known byte.  After each call the guards must be untouched,
the inputs unchanged and the results equal to the oracle's.  The plans are
forced through the planner's tuning overrides (every instantiated tile with
every epilogue, split contractions, the paired convolution backward) or left
to the planner, on ragged shapes; batched products, the SGD update and the
pointwise steps run their default plans."""

import numpy as np
import pytest
import torch

import oracle as o
from integer_only_dnn_amd import ie
from tests.gpu_util import announce, assert_same, rand_qt

pytestmark = pytest.mark.gpu

T, R = o.TENSOR, o.ROW
G = 4096          # guard bytes on each side (keeps every buffer 256-byte aligned)
CANARY = 0x5A


class Guarded:
    """Device buffers with guards; remembers inputs to check they are not written."""

    def __init__(self):
        self.bufs = []      # (guarded tensor, interior bytes, label)
        self.inputs = []    # (interior view, host copy, label)

    def alloc(self, n: int, label: str) -> torch.Tensor:
        buf = torch.full((G + n + G,), CANARY, dtype=torch.uint8, device="cuda")
        self.bufs.append((buf, n, label))
        return buf[G:G + n]

    def out(self, rows: int, cols: int, group: int, label: str, bits: int = 8) -> ie.Mat:
        m = self.alloc(rows * cols, label + ".mant").view(torch.int8).view(rows, cols)
        e = self.alloc(rows if group == R else 1, label + ".exp").view(torch.int8)
        return ie.Mat(m, e, group, bits)

    def inp(self, t: o.QT, label: str, rows: int = None) -> ie.Mat:
        mant = np.ascontiguousarray(t.mant, dtype=np.int8)
        mant = mant.reshape(rows if rows is not None else mant.shape[0], -1)
        exp = np.ascontiguousarray(t.exp, dtype=np.int8)
        m = self.alloc(mant.size, label + ".mant").view(torch.int8).view(mant.shape)
        e = self.alloc(exp.size, label + ".exp").view(torch.int8)
        m.copy_(torch.from_numpy(mant.copy()))
        e.copy_(torch.from_numpy(exp.copy()))
        self.inputs += [(m, mant.copy(), label + ".mant"), (e, exp.copy(), label + ".exp")]
        return ie.Mat(m, e, t.group)

    def check(self, what: str) -> None:
        torch.cuda.synchronize()
        for buf, n, label in self.bufs:
            h = buf.cpu().numpy()
            for part, name in ((h[:G], "before"), (h[G + n:], "after")):
                bad = np.nonzero(part != CANARY)[0]
                assert bad.size == 0, f"{what}: guard {name} {label} written at {bad[:8]}"
        for view, want, label in self.inputs:
            got = view.cpu().numpy().reshape(want.shape)
            assert np.array_equal(got, want), f"{what}: input {label} was modified"


class GuardedWorkspace(ie.Workspace):
    """A fresh workspace of exactly the queried size for every call, guarded."""

    def __init__(self, guards: Guarded):
        super().__init__("cuda")
        self.guards = guards

    def get(self, nbytes: int):
        if self.buf is not None:
            assert self.status() == 0
        n = max(int(nbytes), 256)
        self.buf = self.guards.alloc(n, f"workspace[{n}]")
        ie._check(ie.lib().ie_workspace_init(self.buf.data_ptr(), n, ie._stream(self.device)), "ie_workspace_init")
        return self.buf.data_ptr(), n


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


DENSE_TILES = [(2, 2), (4, 1), (1, 4), (2, 1), (1, 2), (1, 1)]
MODES = [(1, 1), (2, 2), (2, 3), (3, 1)]


@pytest.mark.parametrize("tile", DENSE_TILES + [None], ids=lambda t: "planner" if t is None else f"{64 * t[0]}x{64 * t[1]}")
@pytest.mark.parametrize("mode", [(0, 1)] + MODES, ids=lambda m: f"m{m[0]}s{m[1]}")
def test_guards_linear(tile, mode, plan):
    if tile is None and mode != (1, 1):
        pytest.skip("the planner's own choice is one case")
    direct = mode[0] == 0
    if direct:
        M, N, K = 64 * tile[0] - 3, 64 * tile[1] - 5, 200
    else:
        M, N, K = 200, 150, 392
    announce(f"guards linear tile={tile} mode={mode} M={M} N={N} K={K}")
    rng = np.random.default_rng(101 + 11 * (tile or (0, 0))[0] + (tile or (0, 0))[1] + 5 * mode[0] + mode[1])
    g = Guarded()
    ws = GuardedWorkspace(g)
    X, W, dY = rand_qt(rng, (M, K), R), rand_qt(rng, (N, K), R if not direct else T), rand_qt(rng, (M, N), R)
    Xd, Wd, dYd = g.inp(X, "X"), g.inp(W, "W"), g.inp(dY, "dY")
    plan(tile, *mode)
    for gy in (T, R):
        Y = g.out(M, N, gy, f"Y{gy}")
        ie.ie_linear_fwd(Xd, Wd, Y, ws)
        g.check(f"fwd group {gy}")
        assert_same(Y, o.linear_fwd(X, W, gy), f"fwd group {gy}")
        if direct:
            continue
        dX = g.out(M, K, gy, f"dX{gy}")
        ie.ie_linear_bwd_dx(dYd, Wd, dX, ws)
        g.check(f"dX group {gy}")
        assert_same(dX, o.linear_bwd_dx(dY, W, gy), f"dX group {gy}")
        Yr = g.out(M, N, gy, f"Yrelu{gy}")
        ie.ie_linear_fwd_act(Xd, Wd, Yr, ie.ACT_RELU, ws)
        g.check(f"fwd relu group {gy}")
    assert ws.status() == 0


@pytest.mark.parametrize("wtile", [(2, 2), (1, 4), (4, 1), (1, 1), None],
                         ids=lambda t: "planner" if t is None else f"{64 * t[0]}x{64 * t[1]}")
@pytest.mark.parametrize("splits", [1, 3])
def test_guards_weight_gradient(wtile, splits, plan):
    if wtile is None and splits != 1:
        pytest.skip("the planner's own choice is one case")
    M, N, K = 700, 150, 100
    announce(f"guards linear dW wtile={wtile} splits={splits} M={M} N={N} K={K}")
    rng = np.random.default_rng(7 + splits + 3 * (wtile or (0, 0))[0])
    g = Guarded()
    ws = GuardedWorkspace(g)
    dY, X = rand_qt(rng, (M, N), R), rand_qt(rng, (M, K), R)
    dYd, Xd = g.inp(dY, "dY"), g.inp(X, "X")
    if wtile is not None:
        plan(wtile=wtile, wsplits=splits)
    for gw in (T, R):
        dW = g.out(N, K, gw, f"dW{gw}")
        ie.ie_linear_bwd_dw(dYd, Xd, dW, ws)
        g.check(f"dW group {gw}")
        assert_same(dW, o.linear_bwd_dw(dY, X, gw), f"dW group {gw}")


CONV_CASES = [(2, 10, 10, 24, 40, 3, 3, 1, 1), (2, 9, 9, 48, 24, 3, 3, 2, 1)]
CONV_TILES = [(2, 2), (4, 1), (2, 1), (1, 1)]


@pytest.mark.parametrize("shape", CONV_CASES, ids=lambda s: f"c{s[3]}st{s[7]}")
@pytest.mark.parametrize("tile", CONV_TILES + [None], ids=lambda t: "planner" if t is None else f"{64 * t[0]}x{64 * t[1]}")
@pytest.mark.parametrize("mode", [(1, 1), (2, 2), (3, 1)], ids=lambda m: f"m{m[0]}s{m[1]}")
def test_guards_conv(shape, tile, mode, plan):
    if tile is None and mode != (1, 1):
        pytest.skip("the planner's own choice is one case")
    n, h, w, c, k, r, s, st, pad = shape
    announce(f"guards conv shape={shape} tile={tile} mode={mode}")
    d, dd = o.ConvShape(*shape), ie.conv_desc(*shape)
    rng = np.random.default_rng(sum(shape) + 13 * (tile or (0, 0))[0] + mode[0])
    g = Guarded()
    ws = GuardedWorkspace(g)
    X = rand_qt(rng, (n, h, w, c), T, zero_frac=0.2)
    W = rand_qt(rng, (k, r * s * c), R)
    dY = rand_qt(rng, (n, d.p, d.q, k), T)
    Xd, Wd, dYd = g.inp(X, "X", rows=n * h * w), g.inp(W, "W"), g.inp(dY, "dY", rows=n * d.p * d.q)
    plan(tile, *mode)
    Y = g.out(n * d.p * d.q, k, T, "Y")
    ie.ie_conv_fwd(dd, Xd, Wd, Y, ws)
    g.check("conv fwd")
    assert_same(Y, o.conv_fwd(d, X, W, T), "conv fwd")
    dX = g.out(n * h * w, c, T, "dX")
    dW = g.out(k, r * s * c, R, "dW")
    ie.ie_conv_bwd(dd, Xd, Wd, dYd, dX, dW, ws)
    g.check("conv bwd (both)")
    assert_same(dX, o.conv_dgrad(d, dY, W, T), "conv dgrad")
    assert_same(dW, o.conv_wgrad(d, dY, X, R), "conv wgrad")
    dX1 = g.out(n * h * w, c, T, "dX alone")
    ie.ie_conv_bwd(dd, Xd, Wd, dYd, dX1, None, ws)
    dW1 = g.out(k, r * s * c, T, "dW alone")
    ie.ie_conv_bwd(dd, Xd, Wd, dYd, None, dW1, ws)
    g.check("conv bwd (one output)")
    assert_same(dW1, o.conv_wgrad(d, dY, X, T), "conv wgrad alone")
    assert ws.status() == 0


@pytest.mark.parametrize("form", ["nt", "nn", "tn"])
@pytest.mark.parametrize("shape", [(3, 5, 7, 16), (2, 70, 130, 40), (2, 197, 197, 64), (3, 197, 64, 197)],
                         ids=lambda s: "b{}m{}n{}k{}".format(*s))
def test_guards_bmm(form, shape):
    batch, M, N, K = shape
    announce(f"guards bmm {form} batch={batch} M={M} N={N} K={K}")
    rng = np.random.default_rng(sum(shape) + ord(form[0]) + ord(form[1]))
    g = Guarded()
    ws = GuardedWorkspace(g)
    if form == "nt":
        A, B = rand_qt(rng, (batch * M, K), R), rand_qt(rng, (batch * N, K), R)
        fn, ref = ie.ie_bmm_nt, o.bmm_nt
    elif form == "nn":
        A, B = rand_qt(rng, (batch * M, K), R), rand_qt(rng, (batch * K, N), R, -24, 0)
        fn, ref = ie.ie_bmm_nn, o.bmm_nn
    else:
        A, B = rand_qt(rng, (batch * K, M), R, -24, 0), rand_qt(rng, (batch * K, N), R, -24, 0)
        fn, ref = ie.ie_bmm_tn, o.bmm_tn
    C = g.out(batch * M, N, R, "C")
    fn(batch, g.inp(A, "A"), g.inp(B, "B"), C, ws)
    g.check(f"bmm {form}")
    assert_same(C, ref(A, B, batch), f"bmm {form}")


@pytest.mark.parametrize("shape", [(1, 1), (7, 33), (64, 576), (130, 1000), (3, 5000)], ids=lambda s: f"{s[0]}x{s[1]}")
@pytest.mark.parametrize("groups", [(R, R, R), (T, R, T), (T, T, R)], ids=lambda g: "".join("TR"[x] for x in g))
def test_guards_update_and_pointwise(shape, groups):
    rows, cols = shape
    gw, gv, gg = groups
    announce(f"guards update/pointwise {rows}x{cols} groups={groups}")
    rng = np.random.default_rng(rows * 7 + cols + 3 * gw + gv)
    g = Guarded()
    ws = GuardedWorkspace(g)
    W, V, Gr = rand_qt(rng, shape, gw), rand_qt(rng, shape, gv, -20, -8), rand_qt(rng, shape, gg, -20, -6)
    # W and V are updated in place: guard them as outputs holding the inputs
    Wd, Vd = g.out(rows, cols, gw, "W"), g.out(rows, cols, gv, "V")
    for dst, src in ((Wd, W), (Vd, V)):
        dst.mant.copy_(torch.from_numpy(np.ascontiguousarray(src.mant)))
        dst.exp.copy_(torch.from_numpy(np.ascontiguousarray(src.exp)))
    lr, beta, wd = (1, -7), (7, -3), (1, -13)
    ie.ie_sgd_update(Wd, Vd, g.inp(Gr, "G"), lr, beta, wd, ws=ws)
    g.check("sgd update")
    W2, V2 = o.sgd_update(W, V, Gr, o.Scalar(*lr), o.Scalar(*beta), wd=o.Scalar(*wd))
    assert_same(Vd, V2, "velocity")
    assert_same(Wd, W2, "weight")
    A, B = rand_qt(rng, shape, gw), rand_qt(rng, shape, gg)
    Ad, Bd = g.inp(A, "A"), g.inp(B, "B")
    for gz in (T, R):
        Z = g.out(rows, cols, gz, f"Z{gz}")
        ie.ie_add(Ad, Bd, Z, ws)
        g.check(f"add group {gz}")
        assert_same(Z, o.sum_op(A, B, gz), f"add group {gz}")
    Y = g.out(rows, cols, gw, "relu")
    ie.ie_relu_fwd(Ad, Y)
    dX = g.out(rows, cols, gg, "relu bwd")
    ie.ie_relu_bwd(Bd, Y, dX)
    g.check("relu")
    assert_same(Y, o.QT(o.relu_fwd(A.mant).astype(np.int8), A.exp, A.group), "relu fwd")
    assert ws.status() == 0
