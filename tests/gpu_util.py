"""Helpers shared by the GPU parity tests: move (C, e) data between numpy and
the device, and compare device results with the oracle bit for bit."""

import sys

import numpy as np
import torch

import oracle as o
from integer_only_dnn_amd import ie


def announce(msg: str) -> None:
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(mant: np.ndarray, exp: np.ndarray, group: int, rows: int = None) -> ie.Mat:
    m = np.ascontiguousarray(mant, dtype=np.int8)
    if m.ndim != 2:
        m = m.reshape(rows if rows is not None else m.shape[0], -1)
    return ie.Mat(torch.from_numpy(m.copy()).cuda(), torch.from_numpy(np.asarray(exp, dtype=np.int8).copy()).cuda(),
                  group)


def qt_to_dev(t: o.QT, rows: int = None) -> ie.Mat:
    return to_dev(t.mant, t.exp, t.group, rows)


def from_dev(M: ie.Mat):
    torch.cuda.synchronize()
    return M.mant.cpu().numpy(), M.exp.cpu().numpy()


def assert_same(M: ie.Mat, want: o.QT, what: str = "") -> None:
    got_m, got_e = from_dev(M)
    wm = np.asarray(want.mant, dtype=np.int8).reshape(got_m.shape)
    we = np.asarray(want.exp, dtype=np.int8).reshape(got_e.shape)
    if not np.array_equal(got_e, we):
        bad = np.nonzero(got_e != we)[0]
        raise AssertionError(f"{what}: exponents differ at {bad[:8]}: got {got_e[bad[:8]]} want {we[bad[:8]]}")
    if not np.array_equal(got_m, wm):
        bad = np.argwhere(got_m != wm)
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} mantissas differ, first at {i}: got {got_m[i]} want {wm[i]}")


def rand_qt(rng, shape, group, elo=-14, ehi=-2, zero_frac=0.0):
    m = rng.integers(-128, 128, size=shape).astype(np.int8)
    if zero_frac:
        m[rng.random(shape) < zero_frac] = 0
    n = shape[0] if group == o.ROW else 1
    e = rng.integers(elo, ehi + 1, size=n).astype(np.int8)
    return o.QT(m, e, group)
