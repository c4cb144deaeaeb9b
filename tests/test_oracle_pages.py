"""Pins against numbers the page prints, and the remaining building blocks.

* Table 5's exponent memory equals one byte per output channel of every
  weight tensor (per-group) or one per tensor (per-tensor), with KB = 1024 B:
  this fixes the velocity/gradient group as the output channel.
* Tables 3, 4 and 9: (b_W + b_G + b_V) P + b_A N A bytes in GiB reproduces the
  printed training memory, with the velocity kept at INT8 for INT7..INT4.
* Sum (Table 6) and divide-by-constant (Table 6) against exact Fractions;
  ReLU / ReLU6 forward and backward (Table 7) closed forms.
"""

import os
from fractions import Fraction

import numpy as np
import pytest

import oracle as o

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def resnet18_cifar_out_channels():
    # stem, 4 convs at 64, 4 convs + 1 projection at 128/256/512, fc 10
    return [64] + [64] * 4 + [128] * 5 + [256] * 5 + [512] * 5 + [10]


def vit_ti_out_channels():
    # patch embedding, 12 x (qkv, proj, fc1, fc2), head
    return [192] + [576, 192, 768, 192] * 12 + [10]


def mobilenetv2_out_channels():
    # stem 32; inverted residual blocks (expansion t, out c, repeats n);
    # each block: expand 1x1 (if t > 1), depthwise 3x3, project 1x1; then
    # 1x1 to 1280 and the classifier.
    chans = [32]
    cin = 32
    for t, c, n in [(1, 16, 1), (6, 24, 2), (6, 32, 3), (6, 64, 4), (6, 96, 3), (6, 160, 3), (6, 320, 1)]:
        for _ in range(n):
            hid = cin * t
            if t != 1:
                chans.append(hid)
            chans.append(hid)
            chans.append(c)
            cin = c
    return chans + [1280, 10]


def test_table5_exponent_memory():
    printed = {r[0]: (float(r[1]), float(r[2])) for r in _read("table5_exponent_memory.txt")}
    models = {"resnet18_cifar": resnet18_cifar_out_channels(),
              "mobilenetv2_cifar": mobilenetv2_out_channels(),
              "vit_ti_cifar": vit_ti_out_channels()}
    for name, chans in models.items():
        without_kb, with_kb = printed[name]
        got = o.exponent_bytes(chans, per_group=True) / 1024
        if name == "vit_ti_cifar":
            # 20938 B = 20.447 KB against a printed 20.5: within rounding of a
            # two-step round (20.447 -> 20.45 -> 20.5); the exact figures of
            # the two CNNs fix the one-byte-per-output-channel reading.
            assert abs(got - with_kb) < 0.06
        else:
            assert round(got, 1) == with_kb
        assert round(o.exponent_bytes(chans, per_group=False) / 1024, 2) == without_kb
    assert o.exponent_bytes(models["resnet18_cifar"], True) == 4810
    assert o.exponent_bytes(models["vit_ti_cifar"], True) == 20938


def test_training_memory_equation():
    rows = _read("training_memory.txt")
    inputs = {r[1]: (float(r[2]) * 1e6, float(r[3]) * 1e6, int(r[4])) for r in rows if r[0] == "input"}
    mismatches = []
    for r in rows:
        if r[0] != "memory":
            continue
        P, A, N = inputs[r[1]]
        bw, bg, bv, ba = map(float, r[3:7])
        got = o.training_memory_gib(P, A, N, bw, bg, bv, ba)
        # printed to two decimals; 2.1549 printed as 2.16 suggests a two-step
        # round, so allow just over half a printed digit
        if abs(got - float(r[7])) > 0.0055:
            mismatches.append((r[1], r[2], round(got, 3), float(r[7])))
    # The one printed figure the equation does not reproduce: ResNet-34 INT8
    # computes to 0.539 GiB against a printed 0.55.
    assert mismatches == [("resnet34_cifar100", "int8", 0.539, 0.55)]


def test_sum_matches_fraction():
    rng = np.random.default_rng(3)
    for trial in range(20):
        ga, gb, go = rng.integers(0, 2, size=3)
        A = o.QT(rng.integers(-128, 128, size=(3, 5)).astype(np.int8),
                 rng.integers(-60, 60, size=1 if ga == o.TENSOR else 3).astype(np.int8), int(ga))
        B = o.QT(rng.integers(-128, 128, size=(3, 5)).astype(np.int8),
                 rng.integers(-60, 60, size=1 if gb == o.TENSOR else 3).astype(np.int8), int(gb))
        S = o.sum_op(A, B, int(go))
        vals = [[a + b for a, b in zip(ra, rb)] for ra, rb in zip(A.values(), B.values())]
        rows, exps = o.requant_frac(vals, int(go))
        assert S.mant.astype(int).tolist() == rows and S.exp.astype(int).tolist() == exps
    # x + 0 = R(x)
    A = o.qt([[3, -5, 100]], [-4], o.ROW)
    Z = o.qt([[0, 0, 0]], [o.E_MIN], o.ROW)
    S = o.sum_op(A, Z, o.ROW)
    R = o.requant_np(A.mant.astype(np.int64), np.full((1, 3), -4), o.ROW)
    assert np.array_equal(S.mant, R.mant) and np.array_equal(S.exp, R.exp)


def test_divide_by_constant():
    A = o.qt([[100, -7, 3, 64]], [-3], o.TENSOR)
    rows, exps = o.divide_const(A, 3, o.TENSOR)
    vals = [Fraction(c, 3) * Fraction(2) ** -3 for c in [100, -7, 3, 64]]
    e = exps[0]
    assert all(abs(Fraction(c) * Fraction(2) ** e - v) <= Fraction(2) ** e / 2 for c, v in zip(rows[0], vals))
    assert max(abs(c) for c in rows[0]) >= 64
    # divide by 2**k is an exponent shift
    rows4, exps4 = o.divide_const(A, 4, o.TENSOR)
    base = o.requant_np(A.mant.astype(np.int64), np.full((1, 4), -3), o.TENSOR)
    assert rows4[0] == base.mant[0].astype(int).tolist() and exps4[0] == int(base.exp[0]) - 2


def test_avg_pool_2x2():
    d = o.ConvShape(1, 2, 2, 1, 1, 2, 2, 2, 0)
    X = o.QT(np.array([[[[1], [2]], [[3], [5]]]], dtype=np.int8), np.array([0], dtype=np.int8), o.TENSOR)
    m, e = o.avg_pool(d, X)
    # (1+2+3+5)/4 = 2.75 -> canonical: 2.75 = 88 * 2**-5
    assert m.reshape(-1).tolist() == [88] and e == -5


def test_relu_family_closed_forms():
    C = np.array([-5, 0, 3, 100, 127])
    dY = np.array([7, 7, 7, 7, 7])
    assert o.relu_fwd(C).tolist() == [0, 0, 3, 100, 127]
    assert o.relu_bwd(dY, C).tolist() == [0, 0, 7, 7, 7]
    # e = -4: cap = 6 * 16 = 96
    assert o.relu6_cap(-4) == 96
    assert o.relu6_fwd(C, -4).tolist() == [0, 0, 3, 96, 96]
    assert o.relu6_bwd(dY, C, -4).tolist() == [0, 0, 7, 0, 0]
    # e = -5: 6 * 32 = 192 > q_max -> cap 127
    assert o.relu6_cap(-5) == 127
    assert o.relu6_cap(1) == 3
