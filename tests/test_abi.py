"""The C ABI library loads, exports every entry point include/ie.h declares,
and rejects bad arguments on the host before touching the GPU."""

import ctypes
import os
import re

import pytest

from integer_only_dnn_amd import ie

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "ie.h")).read()
    return sorted(set(re.findall(r"\b(ie_[a-z0-9_]+)\s*\(", src)))


def test_header_symbols_are_exported():
    L = ie.lib()
    names = _declared()
    assert "ie_linear_fwd" in names and "ie_sgd_update" in names and "ie_conv_bwd" in names
    for n in names:
        assert hasattr(L, n), n
    assert sorted(n for n, _, _ in ie.EXPORTS) == names


def test_status_strings():
    L = ie.lib()
    for code, name in ie.STATUS.items():
        assert L.ie_status_str(code).decode() == name


def _mat(rows, cols, group=0, mant=256, exp=256, bits=0):
    return ie.ie_mat(mant, exp, rows, cols, group, bits)


def test_mat_layout():
    # 40 bytes: two pointers, two int64 sizes, group and mantissa width
    assert ctypes.sizeof(ie.ie_mat) == 40 and ie.ie_mat.bits.offset == 36


def test_bits_argument_errors():
    """Mantissa widths outside 2..8 (0 reads as 8), and a velocity that is
    not INT8, are refused before anything is enqueued."""
    L = ie.lib()
    by = ctypes.byref
    X, W = _mat(4, 8), _mat(3, 8)
    for bad in (1, 9, -1, 16):
        assert L.ie_linear_fwd(by(X), by(W), by(_mat(4, 3, bits=bad)), 1, 1 << 20, None) == 8
        assert L.ie_relu_fwd(by(_mat(4, 3, bits=bad)), by(_mat(4, 3)), 0, None) == 8
    S = ie.ie_scalar
    for vb in (2, 4, 7):
        assert L.ie_sgd_update(by(W), by(_mat(3, 8, bits=vb)), by(W), S(1, -7), S(7, -3), S(0, 0),
                               1, 4096, None) == 8


def test_linear_argument_errors():
    L = ie.lib()
    by = ctypes.byref
    X, W, Y = _mat(4, 8), _mat(3, 8), _mat(4, 3)
    assert L.ie_linear_fwd(None, by(W), by(Y), 1, 1 << 20, None) == 1
    assert L.ie_linear_fwd(by(X), by(_mat(3, 9)), by(Y), 1, 1 << 20, None) == 2
    assert L.ie_linear_fwd(by(X), by(W), by(_mat(4, 3, group=7)), 1, 1 << 20, None) == 3
    assert L.ie_linear_fwd(by(X), by(W), by(Y), None, 1 << 20, None) == 4
    assert L.ie_linear_fwd(by(X), by(W), by(Y), 1, 16, None) == 4
    assert L.ie_linear_fwd(by(_mat(4, 8, mant=1)), by(W), by(Y), 1, 1 << 20, None) == 6
    assert L.ie_linear_fwd(by(_mat(4, 8, mant=0)), by(W), by(Y), 1, 1 << 20, None) == 1
    assert L.ie_linear_fwd(by(_mat(4, 70000)), by(_mat(3, 70000)), by(Y), 1, 1 << 30, None) == 6
    assert L.ie_linear_bwd_dx(by(Y), by(W), by(_mat(4, 9)), 1, 1 << 20, None) == 2
    assert L.ie_linear_bwd_dw(by(Y), by(X), by(_mat(3, 9)), 1, 1 << 20, None) == 2


def test_bmm_argument_errors():
    """Batched products: stacks not divisible by the batch, mismatched
    slices, a whole-tensor result, and a short workspace are refused before
    anything is enqueued."""
    L = ie.lib()
    by = ctypes.byref
    nt, nn, tn = L.ie_bmm_nt, L.ie_bmm_nn, L.ie_bmm_tn
    A, B, C = _mat(3 * 5, 16), _mat(3 * 7, 16), _mat(3 * 5, 7, group=1)
    big = 1 << 30
    assert nt(3, by(A), by(_mat(20, 16)), by(C), 1, big, None) == 2      # 20 rows, batch 3
    assert nt(3, by(A), by(_mat(21, 17)), by(C), 1, big, None) == 2      # K differs
    assert nt(3, by(A), by(B), by(_mat(15, 8, group=1)), 1, big, None) == 2
    assert nt(-1, by(A), by(B), by(C), 1, big, None) == 2
    assert nt(3, by(A), by(B), by(_mat(15, 7, group=0)), 1, big, None) == 6
    assert nt(3, by(A), by(B), by(C), None, big, None) == 4
    assert nt(3, by(A), by(B), by(C), 1, 64, None) == 4
    assert nn(3, by(A), by(_mat(3 * 15, 7)), by(C), 1, big, None) == 2   # B slices of 15 rows, K = 16
    assert tn(3, by(_mat(3 * 16, 5)), by(_mat(3 * 15, 7)), by(C), 1, big, None) == 2
    assert tn(3, by(_mat(3 * 16, 5)), by(_mat(3 * 16, 7)), by(_mat(15, 7, group=0)), 1, big, None) == 6
    assert L.ie_bmm_workspace(3, 5, 7, 16) >= 256 and L.ie_bmm_workspace(-1, 5, 7, 16) == 0


def test_conv_and_update_argument_errors():
    L = ie.lib()
    by = ctypes.byref
    d = ie.conv_desc(2, 8, 8, 16, 32, 3, 3, 1, 1)
    X, W, Y = _mat(2 * 64, 16), _mat(32, 144), _mat(2 * 64, 32)
    assert L.ie_conv_fwd(by(d), by(X), by(_mat(32, 145)), by(Y), 1, 1 << 30, None) == 2
    assert L.ie_conv_fwd(by(ie.conv_desc(2, 8, 8, 16, 32, 3, 3, 0, 1)), by(X), by(W), by(Y), 1, 1 << 30, None) == 2
    assert L.ie_conv_fwd(by(d), by(_mat(2 * 64, 16, group=1)), by(W), by(Y), 1, 1 << 30, None) == 6
    assert L.ie_conv_bwd(by(d), by(X), by(W), by(Y), by(_mat(5, 16)), None, 1, 1 << 30, None) == 2
    # filters of more than 15 taps per axis are out of the loaders' tap masks
    d16 = ie.conv_desc(1, 16, 16, 16, 16, 16, 1, 1, 0)
    X16, W16, Y16 = _mat(256, 16), _mat(16, 256), _mat(16, 16)
    assert L.ie_conv_fwd(by(d16), by(X16), by(W16), by(Y16), 1, 1 << 30, None) == 6
    assert L.ie_conv_bwd(by(d16), by(X16), by(W16), by(Y16), by(X16), None, 1, 1 << 30, None) == 6
    # weight-gradient rows wider than a 2^30-byte window of 128 contraction rows
    wide = (1 << 23) + 16
    assert L.ie_linear_bwd_dw(by(_mat(4, wide)), by(_mat(4, 8)), by(_mat(wide, 8)), 1, 1 << 30, None) == 6
    S = ie.ie_scalar
    assert L.ie_sgd_update(by(W), by(_mat(32, 144)), by(_mat(31, 144)), S(1, -7), S(7, -3), S(0, 0),
                           1, 4096, None) == 2
    assert L.ie_sgd_update(by(W), by(W), by(_mat(31, 144)), S(1, -7), S(7, -3), S(1, -13), 1, 4096, None) == 2
    arr = ie.ie_mat * 2
    Ws, Vs, Gs = arr(W, W), arr(W, W), arr(W, _mat(31, 144))
    big = 1 << 20
    assert L.ie_sgd_update_multi(-1, Ws, Ws, Ws, S(1, -7), S(7, -3), S(0, 0), 1, big, None) == 2
    assert L.ie_sgd_update_multi(0, None, None, None, S(1, -7), S(7, -3), S(0, 0), None, 0, None) == 0
    assert L.ie_sgd_update_multi(2, None, Vs, Gs, S(1, -7), S(7, -3), S(0, 0), 1, big, None) == 1
    assert L.ie_sgd_update_multi(2, Ws, Vs, Gs, S(1, -7), S(7, -3), S(0, 0), 1, big, None) == 2
    assert L.ie_sgd_update_multi(2, Ws, Vs, Vs, S(1, -7), S(7, -3), S(0, 0), 1, 16, None) == 4
    assert L.ie_sgd_update_multi_workspace(3) > L.ie_sgd_update_multi_workspace(1)


def test_workspace_sizes_grow_with_shape():
    L = ie.lib()
    a = L.ie_linear_fwd_workspace(64, 128, 256)
    b = L.ie_linear_fwd_workspace(6400, 1280, 256)
    assert 256 <= a < b
    assert L.ie_linear_fwd_workspace(-1, 1, 1) == 0
    d = ie.conv_desc(128, 32, 32, 64, 64, 3, 3, 1, 1)
    assert L.ie_conv_bwd_workspace(ctypes.byref(d)) > L.ie_conv_fwd_workspace(ctypes.byref(d)) > 0


def test_pointwise_argument_errors():
    L = ie.lib()
    by = ctypes.byref
    A, B = _mat(4, 8), _mat(4, 8)
    assert L.ie_relu_fwd(by(A), by(_mat(4, 9)), 0, None) == 2
    assert L.ie_relu_fwd(by(A), by(_mat(4, 8, group=1)), 0, None) == 3
    assert L.ie_relu_fwd(by(A), by(B), 2, None) == 2
    assert L.ie_relu_fwd(None, by(B), 0, None) == 1
    assert L.ie_relu_bwd(by(A), by(_mat(5, 8)), by(B), 0, None) == 2
    assert L.ie_relu_bwd(by(A), by(B), by(_mat(4, 8, group=1)), 1, None) == 3
    assert L.ie_add(by(A), by(B), by(_mat(4, 8)), None, 0, None) == 4
    assert L.ie_add(by(A), by(B), by(_mat(4, 8)), 1, 16, None) == 4
    assert L.ie_add(by(A), by(_mat(4, 7)), by(_mat(4, 8)), 1, 1 << 20, None) == 2
    assert L.ie_add_workspace(4, 8) >= 256
    # fused activations: only none and ReLU
    X, W, Y = _mat(4, 8), _mat(3, 8), _mat(4, 3)
    assert L.ie_linear_fwd_act(by(X), by(W), by(Y), 2, 1, 1 << 20, None) == 6
    d = ie.conv_desc(2, 8, 8, 16, 32, 3, 3, 1, 1)
    assert L.ie_conv_fwd_act(by(d), by(_mat(128, 16)), by(_mat(32, 144)), by(_mat(128, 32)), 5, 1, 1 << 30,
                             None) == 6


@pytest.mark.parametrize("force", ["1,1,0,1", "2,2,0", "0,1", "1,0,1", "3,1,1", "4,4,1", "8,8,1", "1,1,7"])
def test_forced_plans_without_kernel_are_refused(force, monkeypatch):
    """A forced plan (tests and tuning only) is validated like any other: a
    direct epilogue on groups spanning several tiles, a zero or unbuilt tile
    or an unknown mode returns IE_ERR_UNSUPPORTED before anything is
    enqueued (the pointers here are never dereferenced)."""
    L = ie.lib()
    by = ctypes.byref
    monkeypatch.setenv("IE_TILE", force)
    M, N, K = 200, 150, 64
    X, W = _mat(M, K), _mat(N, K)
    ws_bytes = L.ie_linear_fwd_workspace(M, N, K)
    assert ws_bytes >= 256
    for group in (0, 1):
        st = L.ie_linear_fwd(by(X), by(W), by(_mat(M, N, group)), 256, ws_bytes, None)
        assert st == 6, (force, group, st)
