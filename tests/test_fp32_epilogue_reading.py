"""The row-group epilogue's fp32 path, emulated in numpy float32 and held
against the oracle's integer requantisation (CPU only).

Products whose output has one exponent per row and whose right operand has
one exponent per column may round in the fp32 unit.  There fp32 carries no
stored value and no approximation: each exact integer accumulator is
converted to fp32 (exact while |acc| <= 2^24, i.e. a contraction of at most
1024 int8 products), multiplied by powers of two (exact while nothing
overflows or, for the direct rounding, while a result that underflows would
round to 0 anyway), and the only roundings are the final round-half-even or
floor-with-sticky, which then act on the exact value.  The need of a row is
read from the fp32 bit pattern of its largest scaled magnitude.  The kernel
takes this path when the contraction is at most 1024 long and the tile's
column exponents span at most 96; otherwise it computes in integers.

This module restates that path step by step with numpy float32 (IEEE
round-to-nearest products, subnormals kept, or flushed to zero as an
option) and checks it bit for bit against oracle.requant_np at the edges
that decide its exactness: contractions of 1024 (and, to show the limit is
needed, the first length where it would fail), column-exponent spreads of 96
and 97 (and the overflow that caps the spread), exact ties, and rows whose
scale falls below the fp32 normal range.  Reading of the paper page
("Memory-Efficient Integer-Only Training of Deep Neural Networks", Figure 1
caption: no floating-point storage or arithmetic): the fp32 unit is used
here as an exact shifter of integers.
"""

import numpy as np
import pytest

import oracle as o

E_MIN, E_MAX = o.E_MIN, o.E_MAX
NONE = -(1 << 40)


def fpath_taken(k: int, eb: np.ndarray) -> bool:
    """The kernel's choice of the fp32 path for one tile."""
    return k <= 1024 and int(eb.max() - eb.min()) <= 96


def _f32_pow2(n):
    """2^n as float32 (subnormal or 0 below the normal range)."""
    n = np.asarray(n, dtype=np.int64)
    with np.errstate(over="ignore"):
        return np.ldexp(np.ones(n.shape, np.float32), np.clip(n, -200, 200).astype(np.int32)).astype(np.float32)


def _flush(x: np.ndarray, flush: bool) -> np.ndarray:
    if not flush:
        return x
    return np.where(np.abs(x) < np.float32(2.0 ** -126), np.float32(0), x).astype(np.float32)


def emulate(acc, ea, eb, bits: int, direct: bool, flush: bool = False):
    """The fp32 path for one tile spanning whole rows.

    acc: exact int64 accumulators [rows x cols]; ea: row exponents of the
    left operand; eb: column exponents of the right one.  Returns
    (values, exponent): for the direct rounding the int8 mantissas and the
    row exponent; for the round-to-odd form the int16 values at exponent
    need - 2 and that need (NONE for an all-zero row).
    """
    acc = np.asarray(acc, dtype=np.int64)
    ea = np.asarray(ea, dtype=np.int64)
    eb = np.asarray(eb, dtype=np.int64)
    wq = bits - 1
    ebmin = int(eb.min())
    cs = _f32_pow2(eb - ebmin)
    with np.errstate(over="ignore", invalid="ignore"):
        prod = (acc.astype(np.float32) * cs[None, :]).astype(np.float32)
        m = np.abs(prod).max(axis=1).astype(np.float32)
    key = m.view(np.int32).astype(np.int64)
    ones = (1 << wq) - 1
    s = ((key >> 23) - 127) - (wq - 1) + (((key >> (23 - wq)) & ones) == ones)
    zero = key == 0
    rm = np.where(zero, NONE, ea + ebmin + s)
    if direct:
        tgt = np.maximum(E_MIN, rm)
        rs = np.where(zero, np.float32(0), _flush(_f32_pow2(ea + ebmin - tgt), flush)).astype(np.float32)
        with np.errstate(over="ignore", invalid="ignore"):
            y = _flush((prod * rs[:, None]).astype(np.float32), flush)
        with np.errstate(invalid="ignore"):
            return np.rint(y).astype(np.int64), tgt
    rs = np.where(zero, np.float32(1), _f32_pow2(2 - s)).astype(np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        y = (prod * rs[:, None]).astype(np.float32)
    q = np.floor(y)
    return q.astype(np.int64) | (y != q).astype(np.int64), rm


def finish_rto(v, rm):
    """The finalize's integer rounding of round-to-odd values (one tile)."""
    e = np.maximum(E_MIN, rm)
    return o.rne_np(v, (e - (rm - 2))[:, None]), e


def check_against_oracle(acc, ea, eb, bits, flush=False, exact_rto=True):
    want = o.requant_np(acc, ea[:, None] + eb[None, :], o.ROW, bits)
    wm, we = want.mant.astype(np.int64), want.exp.astype(np.int64)
    c, e = emulate(acc, ea, eb, bits, direct=True, flush=flush)
    assert np.array_equal(e, we), "direct: row exponents differ"
    assert np.array_equal(c, wm), f"direct: {int((c != wm).sum())} mantissas differ"
    v, rm = emulate(acc, ea, eb, bits, direct=False, flush=flush)
    # the int16 values are the exact floor-with-sticky of acc 2^(eps - (need - 2))
    for i in range(acc.shape[0] if exact_rto else 0):
        if rm[i] == NONE:
            assert not v[i].any()
            continue
        for j in range(acc.shape[1]):
            sh = int(rm[i] - 2 - ea[i] - eb[j])
            a = int(acc[i, j])
            ex = (a << -sh) if sh <= 0 else (a >> sh) | int((a & ((1 << sh) - 1)) != 0)
            assert int(v[i, j]) == ex, f"round-to-odd value ({i},{j})"
    assert np.all(np.abs(v) < (1 << 15))
    c2, e2 = finish_rto(v, rm)
    assert np.array_equal(e2, we), "round-to-odd: row exponents differ"
    assert np.array_equal(c2, wm), "round-to-odd: mantissas differ"


def _products(rng, rows, k, lo=-128, hi=127):
    a = rng.integers(lo, hi + 1, (rows, k), dtype=np.int64)
    b = rng.integers(lo, hi + 1, (k, 8), dtype=np.int64)
    return a @ b


@pytest.mark.parametrize("bits", [8, 6, 4])
def test_contraction_of_1024_extremes(bits):
    """K = 1024: the largest |acc| (all products of -128 by -128 give exactly
    2^24) and random full-range accumulators round as the oracle does."""
    rng = np.random.default_rng(bits)
    k = 1024
    acc = _products(rng, 6, k)
    acc[0, :] = k * 128 * 128                       # 2^24
    acc[1, :] = -(k * 128 * 128)
    acc[2, 0] = k * 128 * 128 - 1                   # just below, all bits set
    acc[3, :] = 0                                   # all-zero row
    eb = rng.integers(-20, 20, 8)
    assert fpath_taken(k, eb)
    assert np.abs(acc).max() <= 1 << 24
    for ea0 in (-60, 0, 40):
        check_against_oracle(acc, np.full(6, ea0, np.int64) + np.arange(6), eb, bits)


def test_contraction_limit_is_needed():
    """Past 2^24 the int -> fp32 conversion rounds.  At K = 1025 the largest
    |acc| is 2^24 + 2^14 and no rounding decision changes yet, but at
    K = 1033 acc = 2^24 + 2^17 + 1 (1032 products of 128 x 128 and one of 1)
    becomes the tie 2^24 + 2^17 in fp32 and both roundings go wrong, so the
    kernel's K <= 1024 is within a few products of the real limit."""
    assert not fpath_taken(1025, np.zeros(1))
    acc = np.array([[1032 * 128 * 128 + 1, 5]], dtype=np.int64)
    ea, eb = np.array([0]), np.array([0, 0])
    want = o.requant_np(acc, ea[:, None] + eb[None, :], o.ROW, 8)
    c, e = emulate(acc, ea, eb, 8, direct=True)
    assert int(e[0]) == int(want.exp[0]) == 18
    assert int(want.mant[0, 0]) == 65 and int(c[0, 0]) == 64
    v, rm = emulate(acc, ea, eb, 8, direct=False)
    c2, _ = finish_rto(v, rm)
    assert int(c2[0, 0]) == 64
    # K = 1025's largest accumulators still round to the oracle's results,
    # though 2^24 + 1 loses its sticky bit in the round-to-odd values
    acc = np.array([[1025 * 128 * 128, 1024 * 128 * 128 + 1, -3]], dtype=np.int64)
    v, _ = emulate(acc, np.array([0]), np.array([0, 0, 0]), 8, direct=False)
    assert int(v[0, 1]) == 256  # exact: 256 + sticky = 257
    check_against_oracle(acc, np.array([0]), np.array([0, 0, 0]), 8, exact_rto=False)


@pytest.mark.parametrize("spread", [96, 97, 103])
def test_column_exponent_spread(spread):
    """Spreads of 96 (taken) and 97 (not taken, integer path) round exactly
    in fp32 all the same: the products stay below 2^(24 + 103) < 2^128, so
    the kernel's bound keeps a margin of 7 binades.  Each row holds the
    largest |acc| at the top column exponent and 1 at the bottom one."""
    rng = np.random.default_rng(spread)
    k = 1024
    acc = _products(rng, 5, k)
    acc[0, 0], acc[0, 7] = 1 << 24, 1
    acc[1, 0], acc[1, 7] = -(1 << 24), -1
    acc[2, 0], acc[2, 7] = (1 << 24) - 1, 3
    eb = np.array([spread, 50, 40, 30, 20, 10, 5, 0], dtype=np.int64) - 60
    assert fpath_taken(k, eb) == (spread <= 96)
    check_against_oracle(acc, np.array([-40, -10, 0, 5, 20]), eb, 8)


def test_spread_overflow_bounds_the_path():
    """At a spread of 104 the scaled 2^24 reaches 2^128 and overflows fp32:
    the emulated path would fail there, which is what the spread bound
    guards against."""
    acc = np.array([[1 << 24, 1]], dtype=np.int64)
    eb = np.array([104, 0], dtype=np.int64) - 100
    with pytest.raises(AssertionError):
        check_against_oracle(acc, np.array([0]), eb, 8)


@pytest.mark.parametrize("bits", [8, 5])
def test_ties_round_half_even(bits):
    """Accumulators that land exactly half-way after the row's shift, in
    columns with different exponents, round to even on both paths."""
    rng = np.random.default_rng(100 + bits)
    rows, cols = 64, 8
    eb = rng.integers(-6, 7, cols)
    qm = o.q_max(bits)
    acc = np.zeros((rows, cols), dtype=np.int64)
    for i in range(rows):
        s = int(rng.integers(1, 14))
        for j in range(cols):
            # odd multiples of 2^(s - 1) relative to the row's grid: a tie at
            # the shift s once the column exponent is folded in
            t = s - int(eb[j] - eb.min())
            t = max(t, 1)
            m = int(rng.integers(0, qm))
            acc[i, j] = ((2 * m + 1) << (t - 1)) * (1 if rng.random() < 0.5 else -1)
    ties = 0
    want = o.requant_np(acc, eb[None, :], o.ROW, bits)
    for i in range(rows):
        for j in range(cols):
            sh = int(want.exp[i]) - int(eb[j])
            if sh > 0 and (abs(int(acc[i, j])) & ((1 << sh) - 1)) == 1 << (sh - 1):
                ties += 1
    assert ties > rows  # the construction really produces ties
    check_against_oracle(acc, np.zeros(rows, np.int64), eb, bits)


@pytest.mark.parametrize("flush", [False, True])
def test_tiny_scales_below_normal_range(flush):
    """Rows whose exponent is clamped at -128 far above their need: the
    scale 2^(ea + ebmin - e) is subnormal or zero in fp32, every result is
    below 1/2 and rounds to 0 (direct) whether the hardware keeps or
    flushes subnormals.  The round-to-odd scale 2^(2 - s) stays normal
    (s <= 24 + 96 - 6), so its sticky bits are exact."""
    rng = np.random.default_rng(7)
    acc = _products(rng, 8, 512)
    acc[0, :] = 1
    acc[1, 0] = 1 << 24
    eb = np.array([-128, -128, -100, -64, -40, -33, -32, -128], dtype=np.int64)
    ea = np.array([-128, -128, -127, -120, -100, -90, -60, -128], dtype=np.int64)
    assert fpath_taken(512, eb)
    check_against_oracle(acc, ea, eb, 8, flush=flush)
    check_against_oracle(acc, ea, eb, 4, flush=flush)


def test_random_sweep_matches_oracle():
    """Random row and column exponents (spread up to 96), random widths and
    contraction lengths up to 1024, including the exponent clamp at -128."""
    rng = np.random.default_rng(2024)
    done = 0
    for trial in range(40):
        k = int(rng.integers(1, 1025))
        rows = int(rng.integers(1, 9))
        acc = _products(rng, rows, k)
        if trial % 5 == 0:
            acc[rng.integers(0, rows)] = 0
        spread = int(rng.integers(0, 97))
        eb = rng.integers(0, spread + 1, 8) - int(rng.integers(0, 140))
        eb[0] = eb.min() + spread if rng.random() < 0.5 else eb[0]
        if not fpath_taken(k, eb):
            continue
        ea = rng.integers(-128, 40, rows)
        bits = int(rng.choice([8, 7, 6, 4]))
        nd = o.need_np(acc, ea[:, None] + eb[None, :], bits)
        if nd.max() > E_MAX:
            continue
        check_against_oracle(acc, ea, eb, bits, flush=bool(trial & 1))
        done += 1
    assert done >= 25
