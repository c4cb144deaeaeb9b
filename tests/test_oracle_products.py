"""Pins of the oracle's products (linear and convolution, Table 6 "Product").

Accumulators are compared with numpy's int64 matmul, with brute-force Python
loops and with torch's float64 conv2d and its autograd (exact: every partial
sum is an integer below 2**53).  The requantised results are checked against
a Fraction brute force (align by exact rounding, sum exactly, search the group
exponent), and against a worked example done by hand.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as o


def _rand_qt(rng, shape, group, elo=-12, ehi=-2, allow_m128=True):
    lo = -128 if allow_m128 else -127
    m = rng.integers(lo, 128, size=shape).astype(np.int8)
    rows = shape[0]
    e = rng.integers(elo, ehi + 1, size=(1 if group == o.TENSOR else rows))
    return o.QT(m, e.astype(np.int8), group)


def test_worked_example_linear_forward():
    # X = [[100,-50,25],[-127,64,3]] @ -6, W = [[90,60,-30],[-127,127,1]] @ -8.
    # acc = X W^T: 100*90-50*60-25*30 = 5250; 100*-127-50*127+25 = -19025;
    # -127*90+64*60-3*30 = -7680; 127*127+64*127+3 = 24260; exponent -14.
    # 24260 has 15 bits, 24260/2**8 = 94.77 fits and /2**7 = 189.5 does not,
    # so e = -14 + 8 = -6: 5250/256 = 20.51 -> 21, -19025/256 = -74.32 -> -74,
    # -7680/256 = -30 exactly, 24260/256 = 94.77 -> 95.
    X = o.qt([[100, -50, 25], [-127, 64, 3]], -6, o.TENSOR)
    W = o.qt([[90, 60, -30], [-127, 127, 1]], -8, o.TENSOR)
    acc, eps = o.linear_fwd_acc(X, W)
    assert acc.tolist() == [[5250, -19025], [-7680, 24260]]
    assert np.all(eps == -14)
    Y = o.linear_fwd(X, W, o.TENSOR)
    assert Y.mant.tolist() == [[21, -74], [-30, 95]] and Y.exp.tolist() == [-6]
    Yr = o.linear_fwd(X, W, o.ROW)
    # row 0: max 19025 -> 19025/2**8 = 74.3 fits, /2**7 = 148.6 does not -> -6;
    # row 1: 24260 -> -6 as well.
    assert Yr.mant.tolist() == [[21, -74], [-30, 95]] and Yr.exp.tolist() == [-6, -6]


@pytest.mark.parametrize("seed", range(3))
def test_linear_accumulators_match_int64_matmul(seed):
    rng = np.random.default_rng(seed)
    M, N, K = 37, 29, 301
    X = _rand_qt(rng, (M, K), o.ROW)
    W = _rand_qt(rng, (N, K), o.TENSOR)
    dY = _rand_qt(rng, (M, N), o.ROW)
    acc, _ = o.linear_fwd_acc(X, W)
    assert np.array_equal(acc, np.matmul(X.mant.astype(np.int64), W.mant.astype(np.int64).T))
    acc_dx, _ = o.linear_bwd_dx_acc(dY, W)
    assert np.array_equal(acc_dx, np.matmul(dY.mant.astype(np.int64), W.mant.astype(np.int64)))


def _brute_align(t: o.QT):
    re = t.row_exp()
    es = int(re.max())
    out = []
    for i in range(t.mant.shape[0]):
        out.append([round(Fraction(int(c)) / Fraction(2) ** (es - int(re[i]))) for c in t.mant[i]])
    return out, es


def _brute_product(a_rows, a_exps, b_rows, b_exps, out_group):
    """C[i][j] = sum_k a[i][k] * b[j][k], exact, then group search."""
    vals = []
    for i, ar in enumerate(a_rows):
        row = []
        for j, br in enumerate(b_rows):
            s = sum(x * y for x, y in zip(ar, br))
            row.append(Fraction(s) * Fraction(2) ** (a_exps[i] + b_exps[j]))
        vals.append(row)
    return o.requant_frac(vals, out_group)


@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("out_group", [o.TENSOR, o.ROW])
def test_linear_ops_match_fraction_bruteforce(seed, out_group):
    rng = np.random.default_rng(10 + seed)
    M, N, K = 5, 4, 9
    gx, gw, gdy = [(o.TENSOR, o.TENSOR, o.TENSOR), (o.ROW, o.ROW, o.ROW),
                   (o.ROW, o.TENSOR, o.ROW), (o.TENSOR, o.ROW, o.TENSOR)][seed]
    X = _rand_qt(rng, (M, K), gx)
    W = _rand_qt(rng, (N, K), gw)
    dY = _rand_qt(rng, (M, N), gdy)
    xr, wr, dyr = X.row_exp().tolist(), W.row_exp().tolist(), dY.row_exp().tolist()
    # forward: no alignment (no exponent varies along K)
    Y = o.linear_fwd(X, W, out_group)
    rows, exps = _brute_product(X.mant.astype(int).tolist(), xr, W.mant.astype(int).tolist(), wr, out_group)
    assert Y.mant.astype(int).tolist() == rows and Y.exp.astype(int).tolist() == exps
    # dX = dY W: W's rows lie along the contraction -> align W
    w_al, ew = _brute_align(W)
    w_t = [list(col) for col in zip(*w_al)]              # [K][N]
    dX = o.linear_bwd_dx(dY, W, out_group)
    rows, exps = _brute_product(dY.mant.astype(int).tolist(), dyr, w_t, [ew] * K, out_group)
    assert dX.mant.astype(int).tolist() == rows and dX.exp.astype(int).tolist() == exps
    # dW = dY^T X: both aligned over rows
    dy_al, edy = _brute_align(dY)
    x_al, ex = _brute_align(X)
    dW = o.linear_bwd_dw(dY, X, out_group)
    rows, exps = _brute_product([list(c) for c in zip(*dy_al)], [edy] * N,
                                [list(c) for c in zip(*x_al)], [ex] * K, out_group)
    assert dW.mant.astype(int).tolist() == rows and dW.exp.astype(int).tolist() == exps


def test_forward_within_half_ulp_of_float64():
    rng = np.random.default_rng(7)
    X = _rand_qt(rng, (16, 48), o.ROW)
    W = _rand_qt(rng, (24, 48), o.ROW)
    Y = o.linear_fwd(X, W, o.ROW)
    xf = X.mant.astype(np.float64) * np.exp2(X.row_exp())[:, None]
    wf = W.mant.astype(np.float64) * np.exp2(W.row_exp())[:, None]
    ref = xf @ wf.T
    got = Y.mant.astype(np.float64) * np.exp2(Y.row_exp())[:, None]
    ulp = np.exp2(Y.row_exp().astype(np.float64))[:, None]
    assert np.all(np.abs(got - ref) <= ulp / 2)


# ---------------------------------------------------------------------------
# Convolution
# ---------------------------------------------------------------------------

CONV_CASES = [
    o.ConvShape(2, 7, 6, 3, 5, 3, 3, 1, 1),
    o.ConvShape(2, 8, 8, 4, 6, 3, 3, 2, 1),
    o.ConvShape(1, 9, 7, 5, 3, 3, 3, 2, 1),
    o.ConvShape(3, 5, 5, 6, 4, 1, 1, 1, 0),
    o.ConvShape(2, 6, 6, 4, 8, 1, 1, 2, 0),
    o.ConvShape(1, 6, 5, 2, 3, 3, 3, 1, 0),
]


def _torch_conv(d, x, w):
    xt = torch.from_numpy(x.astype(np.float64)).permute(0, 3, 1, 2)
    wt = torch.from_numpy(w.astype(np.float64)).permute(0, 3, 1, 2)
    return xt, wt


@pytest.mark.parametrize("d", CONV_CASES, ids=lambda d: f"{d.h}x{d.w}c{d.c}k{d.k}r{d.r}s{d.stride}p{d.pad}")
def test_conv_accumulators_match_torch_float64(d):
    rng = np.random.default_rng(d.h * 100 + d.c)
    x = rng.integers(-128, 128, size=(d.n, d.h, d.w, d.c))
    w = rng.integers(-128, 128, size=(d.k, d.r, d.s, d.c))
    dy = rng.integers(-128, 128, size=(d.n, d.p, d.q, d.k))
    xt, wt = _torch_conv(d, x, w)
    xt.requires_grad_(True)
    wt.requires_grad_(True)
    yt = torch.nn.functional.conv2d(xt, wt, stride=d.stride, padding=d.pad)
    acc = o.conv_fwd_acc(d, x, w)
    assert np.array_equal(acc, yt.detach().permute(0, 2, 3, 1).numpy().astype(np.int64))
    dyt = torch.from_numpy(dy.astype(np.float64)).permute(0, 3, 1, 2)
    gx, gw = torch.autograd.grad(yt, (xt, wt), dyt)
    assert np.array_equal(o.conv_dgrad_acc(d, dy, w), gx.permute(0, 2, 3, 1).numpy().astype(np.int64))
    assert np.array_equal(o.conv_wgrad_acc(d, dy, x), gw.permute(0, 2, 3, 1).numpy().astype(np.int64))


def test_conv_bruteforce_loops_and_adjoint():
    d = o.ConvShape(1, 5, 4, 2, 3, 3, 3, 2, 1)
    rng = np.random.default_rng(5)
    x = rng.integers(-128, 128, size=(d.n, d.h, d.w, d.c))
    w = rng.integers(-128, 128, size=(d.k, d.r, d.s, d.c))
    dy = rng.integers(-128, 128, size=(d.n, d.p, d.q, d.k))
    y = np.zeros((d.n, d.p, d.q, d.k), dtype=np.int64)
    for n in range(d.n):
        for p in range(d.p):
            for q in range(d.q):
                for k in range(d.k):
                    s = 0
                    for r in range(d.r):
                        for t in range(d.s):
                            h, ww = p * d.stride + r - d.pad, q * d.stride + t - d.pad
                            if 0 <= h < d.h and 0 <= ww < d.w:
                                s += int(np.dot(x[n, h, ww], w[k, r, t]))
                    y[n, p, q, k] = s
    assert np.array_equal(o.conv_fwd_acc(d, x, w), y)
    lhs = int((y * dy).sum())
    assert lhs == int((x * o.conv_dgrad_acc(d, dy, w)).sum())
    assert lhs == int((w * o.conv_wgrad_acc(d, dy, x)).sum())


def test_conv_1x1_equals_linear():
    d = o.ConvShape(2, 3, 4, 16, 8, 1, 1, 1, 0)
    rng = np.random.default_rng(6)
    X = _rand_qt(rng, (d.n * d.h * d.w, d.c), o.TENSOR)
    W = _rand_qt(rng, (d.k, d.c), o.ROW)
    dY = _rand_qt(rng, (d.n * d.h * d.w, d.k), o.TENSOR)
    Xc = o.QT(X.mant.reshape(d.n, d.h, d.w, d.c), X.exp, o.TENSOR)
    dYc = o.QT(dY.mant.reshape(d.n, d.h, d.w, d.k), dY.exp, o.TENSOR)
    y1 = o.conv_fwd(d, Xc, W, o.TENSOR)
    y2 = o.linear_fwd(X, W, o.TENSOR)
    assert np.array_equal(y1.mant.reshape(-1, d.k), y2.mant) and np.array_equal(y1.exp, y2.exp)
    dx1 = o.conv_dgrad(d, dYc, W, o.TENSOR)
    dx2 = o.linear_bwd_dx(dY, W, o.TENSOR)
    assert np.array_equal(dx1.mant.reshape(-1, d.c), dx2.mant) and np.array_equal(dx1.exp, dx2.exp)
    dw1 = o.conv_wgrad(d, dYc, Xc, o.ROW)
    dw2 = o.linear_bwd_dw(dY, X, o.ROW)
    assert np.array_equal(dw1.mant, dw2.mant) and np.array_equal(dw1.exp, dw2.exp)


def test_conv_requant_matches_fraction_bruteforce():
    d = o.ConvShape(1, 4, 4, 2, 3, 3, 3, 1, 1)
    rng = np.random.default_rng(8)
    X = _rand_qt(rng, (d.n, d.h, d.w, d.c), o.TENSOR)
    W = _rand_qt(rng, (d.k, d.r * d.s * d.c), o.ROW)
    Y = o.conv_fwd(d, X, W, o.TENSOR)
    acc = o.conv_fwd_acc(d, X.mant.astype(np.int64), W.mant.reshape(d.k, d.r, d.s, d.c))
    ex, ew = int(X.exp[0]), W.row_exp()
    vals = [[Fraction(int(acc.reshape(-1, d.k)[i, k])) * Fraction(2) ** (ex + int(ew[k]))
             for k in range(d.k)] for i in range(acc.size // d.k)]
    rows, exps = o.requant_frac(vals, o.TENSOR)
    assert Y.mant.reshape(-1, d.k).astype(int).tolist() == rows and Y.exp.tolist() == exps
