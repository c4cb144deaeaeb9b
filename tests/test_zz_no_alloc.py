"""ie_linear_fwd_noalloc, the forward product that allocates nothing (its
scratch is a fixed device array of the library), against ie_linear_fwd on
the same inputs, bit for bit: several calls in a row on one GPU, each
smaller than the one before, covering the plans that use scratch (padded
operands, the two-pass round-to-odd epilogue, split contractions with both
finalizes) and the direct one; then a shape beyond the scratch, refused
before anything is enqueued, and the exponent-range flag landing in the
caller's word."""

import ctypes
from ctypes import byref

import numpy as np
import pytest
import torch

import oracle as o
from integer_only_dnn_amd import ie
from tests.gpu_util import announce, from_dev, qt_to_dev, rand_qt

pytestmark = pytest.mark.gpu

T, R = o.TENSOR, o.ROW


def _noalloc(X: ie.Mat, W: ie.Mat, Y: ie.Mat, flags) -> int:
    x, w, y = X.c(), W.c(), Y.c()
    fp = ctypes.c_void_p(flags.data_ptr()) if flags is not None else None
    return ie.lib().ie_linear_fwd_noalloc(byref(x), byref(w), byref(y), fp, ie._stream(torch.device("cuda")))


# (M, N, K, X group, W group, Y group): decreasing sizes; the plans they take
# in this order: round-to-odd whole-tensor, padded K with row groups,
# split contraction (two-pass finalize), split with the row finalize, direct
CASES = [
    (1000, 300, 200, R, R, T),
    (700, 257, 100, T, R, R),
    (90, 80, 4096, R, T, T),
    (64, 70, 2048, T, T, R),
    (60, 50, 48, T, R, T),
]


def test_noalloc_matches_linear_fwd():
    ws = ie.Workspace("cuda")
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    rng = np.random.default_rng(77)
    for M, N, K, gx, gw, gy in CASES:
        announce(f"noalloc M={M} N={N} K={K} groups x{gx} w{gw} y{gy}")
        X, W = rand_qt(rng, (M, K), gx), rand_qt(rng, (N, K), gw)
        Xd, Wd = qt_to_dev(X), qt_to_dev(W)
        Y1 = ie.Mat.empty(M, N, gy)
        ie.ie_linear_fwd(Xd, Wd, Y1, ws)
        Y2 = ie.Mat.empty(M, N, gy)
        Y2.mant.fill_(55)
        Y2.exp.fill_(55)
        assert _noalloc(Xd, Wd, Y2, flags) == 0
        m1, e1 = from_dev(Y1)
        m2, e2 = from_dev(Y2)
        assert np.array_equal(e1, e2), f"exponents differ for {M}x{N}x{K}"
        assert np.array_equal(m1, m2), f"{int((m1 != m2).sum())} mantissas differ for {M}x{N}x{K}"
    torch.cuda.synchronize()
    assert int(flags.item()) == 0
    assert ws.status() == 0


def test_noalloc_refuses_beyond_scratch_and_reports_range():
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    # a whole-tensor result of 50432 x 3072 needs ~310 MB of int16 values
    X = ie.Mat.empty(50432, 768, T)
    W = ie.Mat.empty(3072, 768, T)
    Y = ie.Mat.empty(50432, 3072, T)
    assert _noalloc(X, W, Y, flags) == 9  # IE_ERR_SCRATCH, nothing enqueued
    # exponents 120 + 120 overflow the int8 exponent: the flag goes to the
    # caller's word
    rng = np.random.default_rng(5)
    Xq, Wq = rand_qt(rng, (64, 64), T, 120, 120), rand_qt(rng, (32, 64), T, 120, 120)
    Y = ie.Mat.empty(64, 32, T)
    assert _noalloc(qt_to_dev(Xq), qt_to_dev(Wq), Y, flags) == 0
    torch.cuda.synchronize()
    assert int(flags.item()) & ie.FLAG_EXP_RANGE
