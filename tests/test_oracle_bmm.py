"""Pins of the oracle's batched products (attention's Q . K^T, P . V and their
gradients as the Product primitive per slice).

Checked against a Fraction brute force that re-derives every element from
the definition (alignment of a row-grouped contraction axis at its largest
exponent, round half to even via Python's round on exact Fractions, the
smallest row exponent by direct search), against the transpose identities
between the three forms, and against slice independence.
"""

from fractions import Fraction

import numpy as np
import pytest

import oracle as o

T, R = o.TENSOR, o.ROW


def _qt(rng, rows, cols, group, elo=-12, ehi=-2):
    m = rng.integers(-128, 128, size=(rows, cols)).astype(np.int8)
    m[rng.random(m.shape) < 0.15] = 0
    n = rows if group == R else 1
    return o.QT(m, rng.integers(elo, ehi + 1, size=n).astype(np.int8), group)


def _vals(t: o.QT):
    """Exact values as a list of rows of Fractions."""
    return t.values()


def _align(rows_vals, mants, exps):
    """Re-express every row at the largest row exponent (round half to even)."""
    es = max(exps)
    return [[Fraction(round(Fraction(int(c)) / Fraction(2) ** (es - e))) * Fraction(2) ** es for c in row]
            for row, e in zip(mants, exps)]


def _slice_rows(t: o.QT, batch, z):
    rows = t.mant.shape[0] // batch
    m = t.mant[z * rows:(z + 1) * rows].astype(int).tolist()
    re = t.row_exp()[z * rows:(z + 1) * rows].tolist()
    return m, re


def _brute(kind, A, B, batch, bits):
    out_rows, out_exps = [], []
    for z in range(batch):
        am, ae = _slice_rows(A, batch, z)
        bm, be = _slice_rows(B, batch, z)
        av = [[Fraction(c) * Fraction(2) ** e for c in row] for row, e in zip(am, ae)]
        bv = [[Fraction(c) * Fraction(2) ** e for c in row] for row, e in zip(bm, be)]
        if kind == "nt":      # C[i][j] = sum_k A[i][k] B[j][k]
            c = [[sum(a * b for a, b in zip(ar, br)) for br in bv] for ar in av]
        elif kind == "nn":    # C[i][n] = sum_k A[i][k] B[k][n], B aligned over its rows
            bal = _align(bv, bm, be)
            c = [[sum(ar[k] * bal[k][n] for k in range(len(bal))) for n in range(len(bal[0]))] for ar in av]
        else:                 # C[m][n] = sum_k A[k][m] B[k][n], both aligned over rows
            aal = _align(av, am, ae)
            bal = _align(bv, bm, be)
            c = [[sum(aal[k][m] * bal[k][n] for k in range(len(aal))) for n in range(len(bal[0]))]
                 for m in range(len(aal[0]))]
        rows, exps = o.requant_frac(c, R, bits)
        out_rows += rows
        out_exps += exps
    return out_rows, out_exps


@pytest.mark.parametrize("kind", ["nt", "nn", "tn"])
@pytest.mark.parametrize("seed", range(4))
def test_bmm_matches_fraction_bruteforce(kind, seed):
    rng = np.random.default_rng(70 + seed + 10 * ["nt", "nn", "tn"].index(kind))
    batch, M, N, K = 3, 4, 5, 6
    ga, gb = [(R, R), (T, R), (R, T), (T, T)][seed]
    bits = [8, 8, 6, 4][seed]
    if kind == "nt":
        A, B = _qt(rng, batch * M, K, ga), _qt(rng, batch * N, K, gb)
        got = o.bmm_nt(A, B, batch, bits)
    elif kind == "nn":
        A, B = _qt(rng, batch * M, K, ga), _qt(rng, batch * K, N, gb, elo=-20, ehi=0)
        got = o.bmm_nn(A, B, batch, bits)
    else:
        A, B = _qt(rng, batch * K, M, ga, elo=-20, ehi=0), _qt(rng, batch * K, N, gb, elo=-20, ehi=0)
        got = o.bmm_tn(A, B, batch, bits)
    rows, exps = _brute(kind, A, B, batch, bits)
    assert got.group == R
    assert got.mant.astype(int).tolist() == rows
    assert got.exp.astype(int).tolist() == exps


def _transpose_slices(t: o.QT, batch):
    """Slice-wise transpose of a whole-tensor-grouped stack."""
    assert t.group == T
    rows = t.mant.shape[0] // batch
    m = np.concatenate([t.mant[z * rows:(z + 1) * rows].T for z in range(batch)])
    return o.QT(np.ascontiguousarray(m), t.exp, T)


def test_bmm_transpose_identities():
    """With whole-tensor operands (no alignment): A.B = A.(B^T)^T and
    A^T.B = (A^T).(B^T)^T, so the three forms agree with one another."""
    rng = np.random.default_rng(5)
    batch, M, N, K = 4, 9, 7, 33
    A = _qt(rng, batch * M, K, T)
    Bn = _qt(rng, batch * K, N, T)
    assert np.array_equal(o.bmm_nn(A, Bn, batch).mant, o.bmm_nt(A, _transpose_slices(Bn, batch), batch).mant)
    At = _qt(rng, batch * K, M, T)
    got = o.bmm_tn(At, Bn, batch)
    want = o.bmm_nt(_transpose_slices(At, batch), _transpose_slices(Bn, batch), batch)
    assert np.array_equal(got.mant, want.mant) and np.array_equal(got.exp, want.exp)


def test_bmm_slices_independent():
    """Reordering the slices reorders the results and nothing else; a slice
    of zeros gives zeros at the smallest exponent."""
    rng = np.random.default_rng(6)
    batch, M, N, K = 5, 6, 8, 40
    A, B = _qt(rng, batch * M, K, R), _qt(rng, batch * N, K, R)
    A.mant[2 * M:3 * M] = 0
    C = o.bmm_nt(A, B, batch)
    perm = [3, 0, 4, 2, 1]
    Ap = o.QT(np.concatenate([A.mant[z * M:(z + 1) * M] for z in perm]),
              np.concatenate([A.exp[z * M:(z + 1) * M] for z in perm]), R)
    Bp = o.QT(np.concatenate([B.mant[z * N:(z + 1) * N] for z in perm]),
              np.concatenate([B.exp[z * N:(z + 1) * N] for z in perm]), R)
    Cp = o.bmm_nt(Ap, Bp, batch)
    for i, z in enumerate(perm):
        assert np.array_equal(Cp.mant[i * M:(i + 1) * M], C.mant[z * M:(z + 1) * M])
        assert np.array_equal(Cp.exp[i * M:(i + 1) * M], C.exp[z * M:(z + 1) * M])
    assert not C.mant[2 * M:3 * M].any() and (C.exp[2 * M:3 * M] == o.E_MIN).all()
