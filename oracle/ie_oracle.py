"""Plain, slow CPU oracle of the (C, e) building blocks — test infrastructure.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg use
this module; the HIP product path never imports it and it imports nothing of
the product path.

Source: "Memory-Efficient Integer-Only Training of Deep Neural Networks",
Abstract, Figure 1, Tables 5-7.  The page says that every tensor is a signed
integer mantissa C paired with an explicit power-of-two exponent e (the value
is C * 2**e, Figure 1's Eq. 1), that all storage is INT8, and that training is
built from five integer blocks: products, sums, divide-by-constant, nonlinear
functions and weight updates.  It does not print the bodies of the equations
it cites (Eqs. 1, 3, 5, 6, 7, 8), so the following readings are taken and used
identically everywhere:

R1  value(C, e) = C * 2**e, C in [-127, 127] on output (-128 accepted on
    input), e a signed byte in [E_MIN, E_MAX] = [-128, 127].
R2  every right shift rounds half to even; a result is rounded exactly once,
    from the exact value, when it is stored.
R3  a group's exponent is the smallest e with every |C| <= Q_MAX (canonical
    form; left shifts are allowed and exact); an all-zero group, or one whose
    smallest exponent lies below E_MIN, gets E_MIN; above E_MAX is an error.
R4  groups: TENSOR = one exponent for the whole tensor, ROW = one exponent
    per leading index (per output channel for weights [N x K], per row /
    token / pixel for activations).  Table 5's exponent memory equals one
    byte per output channel, which fixes the velocity and gradient groups.
R5  an operand whose exponent varies along a contraction axis is first
    re-expressed at the largest exponent on that axis (align, rounding as R2).
R6  products are exact integer sums of int8 x int8 terms, exponent e_a + e_b.
R7  the optimizer is SGD with momentum in the PyTorch form
    v <- beta*v + g,  w <- w - lr*v  (no dampening), the velocity rounded
    first and the weight update using the stored, rounded velocity.
R8  mantissa width B (Table 4, B in 8..4): a B-bit result has
    |C| <= 2**(B-1) - 1 in R1 and R3, stored in the same int8 container;
    the velocity stays INT8 whatever B the weights use.  Every requantising
    function takes ``bits`` (default 8).

Integer contractions use float64 matrix products: every partial sum is an
integer of magnitude < 2**53 (asserted), where float64 addition is exact in
any order, so the float64 result is the exact integer sum.
"""

from __future__ import annotations

from dataclasses import dataclass
from fractions import Fraction

import numpy as np

Q_BITS = 8                       # mantissa width B (INT8)
Q_MAX = (1 << (Q_BITS - 1)) - 1  # 127
E_MIN = -128
E_MAX = 127

TENSOR = 0
ROW = 1

_F64_EXACT = 1 << 53


class ExpRangeError(ArithmeticError):
    """A group's smallest valid exponent exceeds E_MAX (reading R3)."""


# ---------------------------------------------------------------------------
# (C, e) tensors
# ---------------------------------------------------------------------------

@dataclass
class QT:
    """A (C, e) tensor: int8 mantissas and int8 exponents (reading R1, R4).

    ``mant`` has any shape whose leading axis is the row axis; ``exp`` has one
    entry (TENSOR) or ``mant.shape[0]`` entries (ROW).
    """

    mant: np.ndarray
    exp: np.ndarray
    group: int

    def row_exp(self) -> np.ndarray:
        """Exponent of each leading-index row, as int64."""
        rows = self.mant.shape[0]
        e = np.asarray(self.exp, dtype=np.int64).reshape(-1)
        if self.group == TENSOR:
            assert e.size == 1
            return np.full(rows, e[0], dtype=np.int64)
        assert e.size == rows
        return e

    def values(self) -> list:
        """Exact values as Fractions (small tensors only)."""
        re = self.row_exp()
        out = []
        flat = self.mant.reshape(self.mant.shape[0], -1)
        for i in range(flat.shape[0]):
            out.append([Fraction(int(c)) * Fraction(2) ** int(re[i]) for c in flat[i]])
        return out


def qt(mant, exp, group) -> QT:
    mant = np.asarray(mant, dtype=np.int8)
    exp = np.atleast_1d(np.asarray(exp, dtype=np.int64))
    assert np.all((exp >= E_MIN) & (exp <= E_MAX))
    return QT(mant, exp.astype(np.int8), group)


# ---------------------------------------------------------------------------
# Rounding (reading R2)
# ---------------------------------------------------------------------------

def rne_int(a: int, s: int) -> int:
    """a / 2**s rounded half to even, for Python ints; exact a * 2**-s if s <= 0."""
    a, s = int(a), int(s)
    if s <= 0:
        return a << (-s)
    q = a >> s                      # floor
    r = a - (q << s)                # 0 <= r < 2**s
    half = 1 << (s - 1)
    if r > half or (r == half and (q & 1)):
        q += 1
    return q


def rne_frac(v: Fraction) -> int:
    """Nearest integer to a rational, ties to even."""
    fl = v.numerator // v.denominator
    r = v - fl
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and (fl & 1)):
        fl += 1
    return fl


def rne_np(a: np.ndarray, s) -> np.ndarray:
    """Vectorised rne_int on int64 arrays (|a| < 2**53, results fit int64)."""
    a = np.asarray(a, dtype=np.int64)
    s = np.broadcast_to(np.asarray(s, dtype=np.int64), a.shape)
    out = np.empty_like(a)
    left = s <= 0
    if np.any(left):
        al = a[left]
        sl = -s[left]
        assert np.all((al == 0) | (sl < 62))
        out[left] = np.where(al == 0, 0, al << np.minimum(sl, 62))
    right = ~left
    if np.any(right):
        ar = a[right]
        # |a| < 2**53 <= 2**(s-1) for s >= 54: the result is 0 (a tie is
        # impossible), so clamping s at 60 keeps the shifts defined.
        sr = np.minimum(s[right], 60)
        q = ar >> sr
        r = ar - (q << sr)
        half = np.int64(1) << (sr - 1)
        up = (r > half) | ((r == half) & ((q & 1) == 1))
        out[right] = q + up.astype(np.int64)
    return out


# ---------------------------------------------------------------------------
# Smallest exponent for one exact value (reading R3)
# ---------------------------------------------------------------------------

def q_max(bits: int = Q_BITS) -> int:
    """Largest output mantissa magnitude of a B-bit tensor (reading R8)."""
    assert 2 <= bits <= 8
    return (1 << (bits - 1)) - 1


def need_int(a: int, eps: int, bits: int = Q_BITS):
    """Smallest e with |rne(a * 2**eps, at exponent e)| <= q_max(bits); None if a == 0.

    Walks e upward from a point where the bound certainly fails; |rne| is
    non-increasing in the shift, so the first e that satisfies it is the
    smallest one.
    """
    a, eps = int(a), int(eps)
    if a == 0:
        return None
    qm = q_max(bits)
    s = abs(a).bit_length() - bits - 1   # |a| / 2**s >= 2**bits > qm
    assert abs(rne_int(a, s)) > qm
    while abs(rne_int(a, s)) > qm:
        s += 1
    return eps + s


def _bitlen_np(m: np.ndarray) -> np.ndarray:
    """Bit length of non-negative int64 values below 2**53 (0 -> 0)."""
    m = np.asarray(m, dtype=np.int64)
    assert np.all(m < _F64_EXACT)
    _, ex = np.frexp(m.astype(np.float64))
    return np.where(m == 0, 0, ex).astype(np.int64)


def need_np(a: np.ndarray, eps, bits: int = Q_BITS) -> np.ndarray:
    """Vectorised need_int; entries with a == 0 get a very small sentinel."""
    a = np.asarray(a, dtype=np.int64)
    eps = np.broadcast_to(np.asarray(eps, dtype=np.int64), a.shape)
    qm = q_max(bits)
    s = _bitlen_np(np.abs(a)) - bits - 1
    nz = a != 0
    assert np.all(np.abs(rne_np(a[nz], s[nz])) > qm)
    bad = nz.copy()
    while np.any(bad):
        s = np.where(bad, s + 1, s)
        bad = nz & (np.abs(rne_np(a, s)) > qm)
    return np.where(nz, eps + s, np.int64(-(1 << 40)))


# ---------------------------------------------------------------------------
# Requantisation of a group of exact values (reading R3)
# ---------------------------------------------------------------------------

def group_exponent(needs) -> int:
    """Exponent of a group given the needs of its nonzero members."""
    needs = [n for n in needs if n is not None]
    e = max([E_MIN] + needs)
    if e > E_MAX:
        raise ExpRangeError(f"group exponent {e} > {E_MAX}")
    return e


def requant_np(acc: np.ndarray, eps: np.ndarray, group: int, bits: int = Q_BITS) -> QT:
    """Requantise exact values acc * 2**eps (int64, 2-D [rows x cols]).

    ROW: one exponent per row; TENSOR: one for the whole array.
    """
    acc = np.asarray(acc, dtype=np.int64)
    eps = np.broadcast_to(np.asarray(eps, dtype=np.int64), acc.shape)
    assert acc.ndim == 2
    nd = need_np(acc, eps, bits)
    if group == ROW:
        gmax = nd.max(axis=1) if acc.shape[1] else np.full(acc.shape[0], -(1 << 40))
        e = np.maximum(gmax, E_MIN)
        if np.any(e > E_MAX):
            raise ExpRangeError(f"row exponent {int(e.max())} > {E_MAX}")
        c = rne_np(acc, e[:, None] - eps)
        eo = e
    else:
        gmax = int(nd.max()) if acc.size else -(1 << 40)
        e = max(gmax, E_MIN)
        if e > E_MAX:
            raise ExpRangeError(f"tensor exponent {e} > {E_MAX}")
        c = rne_np(acc, e - eps)
        eo = np.array([e])
    assert np.all(np.abs(c) <= q_max(bits))
    return QT(c.astype(np.int8), eo.astype(np.int8), group)


def requant_frac(vals: list, group: int, bits: int = Q_BITS) -> tuple:
    """Requantise nested lists of exact Fractions (small inputs, reading R3).

    Returns (mantissa rows as lists of int, exponent list).  The group
    exponent is found by direct search over e, independent of need_int.
    """
    groups = vals if group == ROW else [[v for row in vals for v in row]]

    def fits(g, e):
        return all(abs(rne_frac(v / Fraction(2) ** e)) <= q_max(bits) for v in g)

    exps = []
    for g in groups:
        if all(v == 0 for v in g):
            exps.append(E_MIN)
            continue
        e = E_MIN
        while not fits(g, e):
            e += 1
            if e > E_MAX:
                raise ExpRangeError("group exponent above E_MAX")
        exps.append(e)
    rows = []
    for i, row in enumerate(vals):
        e = exps[i] if group == ROW else exps[0]
        rows.append([rne_frac(v / Fraction(2) ** e) for v in row])
    return rows, exps


# ---------------------------------------------------------------------------
# Alignment along a contraction axis (reading R5)
# ---------------------------------------------------------------------------

def align_rows(t: QT) -> tuple:
    """Re-express every row of t at the largest row exponent.

    Returns (int64 mantissas, common exponent).  For TENSOR groups, or ROW
    groups whose exponents are all equal, this is the identity.
    """
    re = t.row_exp()
    m = t.mant.astype(np.int64).reshape(t.mant.shape[0], int(np.prod(t.mant.shape[1:], dtype=np.int64)))
    if re.size == 0:
        return m.reshape(t.mant.shape), E_MIN
    e_star = int(re.max())
    shift = (e_star - re)[:, None]
    out = rne_np(m, np.broadcast_to(shift, m.shape))
    return out.reshape(t.mant.shape), e_star


# ---------------------------------------------------------------------------
# Exact integer contraction (reading R6)
# ---------------------------------------------------------------------------

def _exact_matmul(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Exact a @ b for small-integer int64 matrices, via float64."""
    k = a.shape[1]
    ma = int(np.abs(a).max()) if a.size else 0
    mb = int(np.abs(b).max()) if b.size else 0
    assert k * ma * mb < _F64_EXACT, "partial sums could exceed 2**53"
    return (a.astype(np.float64) @ b.astype(np.float64)).astype(np.int64)


# ---------------------------------------------------------------------------
# Linear layer: Table 6 "Linear / fully-connected -> Product"
# ---------------------------------------------------------------------------

def linear_fwd_acc(X: QT, W: QT):
    """Exact Y accumulators and per-element exponents: Y = X . W^T."""
    acc = _exact_matmul(X.mant.astype(np.int64), W.mant.astype(np.int64).T)
    eps = X.row_exp()[:, None] + W.row_exp()[None, :]
    return acc, eps


def linear_fwd(X: QT, W: QT, y_group: int, bits: int = Q_BITS) -> QT:
    """Forward product Y = X . W^T requantised into y_group (Figure 1a)."""
    acc, eps = linear_fwd_acc(X, W)
    return requant_np(acc, eps, y_group, bits)


def linear_bwd_dx_acc(dY: QT, W: QT):
    """Exact dX = dY . W accumulators; W aligned along its rows first (R5)."""
    w_al, e_w = align_rows(W)
    acc = _exact_matmul(dY.mant.astype(np.int64), w_al)
    eps = np.broadcast_to(dY.row_exp()[:, None] + e_w, acc.shape)
    return acc, eps


def linear_bwd_dx(dY: QT, W: QT, dx_group: int, bits: int = Q_BITS) -> QT:
    """Backward input gradient dX = dY . W (Figure 1a)."""
    acc, eps = linear_bwd_dx_acc(dY, W)
    return requant_np(acc, eps, dx_group, bits)


def linear_bwd_dw_acc(dY: QT, X: QT):
    """Exact dW = dY^T . X accumulators; dY and X aligned over rows (R5)."""
    dy_al, e_dy = align_rows(dY)
    x_al, e_x = align_rows(X)
    acc = _exact_matmul(dy_al.T, x_al)
    return acc, np.full(acc.shape, e_dy + e_x, dtype=np.int64)


def linear_bwd_dw(dY: QT, X: QT, dw_group: int, bits: int = Q_BITS) -> QT:
    """Backward weight gradient dW = dY^T . X (Figure 1a); per output channel
    groups for ROW (Table 5)."""
    acc, eps = linear_bwd_dw_acc(dY, X)
    return requant_np(acc, eps, dw_group, bits)


# ---------------------------------------------------------------------------
# Batched products: the Product primitive applied independently to a stack of
# matrices, e.g. a ViT's attention per (image, head): scores Q . K^T, context
# P . V and their gradients (ViT-Ti / ViT-B in the Abstract and Table 11 use
# them; the page names no other primitive for them).  Every operand is a
# stack [batch * rows x cols]; slice z is rows z*rows .. (z+1)*rows - 1.  The
# result's groups are ROW (one exponent per row of every slice).
# ---------------------------------------------------------------------------

def _slice(t: QT, batch: int, z: int) -> QT:
    rows = t.mant.shape[0] // batch
    m = t.mant[z * rows:(z + 1) * rows]
    e = t.exp if t.group == TENSOR else t.exp[z * rows:(z + 1) * rows]
    return QT(m, e, t.group)


def _stack(parts: list, cols: int) -> QT:
    mant = np.concatenate([p.mant for p in parts]) if parts else np.zeros((0, cols), np.int8)
    exp = np.concatenate([p.exp for p in parts]) if parts else np.zeros(0, np.int8)
    return QT(mant.astype(np.int8), exp.astype(np.int8), ROW)


def bmm_nt(A: QT, B: QT, batch: int, bits: int = Q_BITS) -> QT:
    """C_z = A_z . B_z^T for every slice (A_z [M x K], B_z [N x K]): the
    linear forward product per slice; ROW groups."""
    n = B.mant.shape[0] // batch if batch else 0
    return _stack([linear_fwd(_slice(A, batch, z), _slice(B, batch, z), ROW, bits) for z in range(batch)], n)


def bmm_nn(A: QT, B: QT, batch: int, bits: int = Q_BITS) -> QT:
    """C_z = A_z . B_z (A_z [M x K], B_z [K x N]): the contraction runs over
    B_z's rows, so a row-grouped B_z is first re-expressed at the largest of
    its own row exponents (reading R5), as in the linear input gradient."""
    n = B.mant.shape[1]
    return _stack([linear_bwd_dx(_slice(A, batch, z), _slice(B, batch, z), ROW, bits) for z in range(batch)], n)


def bmm_tn(A: QT, B: QT, batch: int, bits: int = Q_BITS) -> QT:
    """C_z = A_z^T . B_z (A_z [K x M], B_z [K x N]): both contracted over
    their rows, each slice aligned at its own largest row exponent (R5), as
    in the linear weight gradient."""
    n = B.mant.shape[1]
    return _stack([linear_bwd_dw(_slice(A, batch, z), _slice(B, batch, z), ROW, bits) for z in range(batch)], n)


# ---------------------------------------------------------------------------
# Convolution: Table 6 "Convolution (incl. 1x1, depthwise) -> Product"
# Activations NHWC, weights [K, R, S, C]; zero padding; cross-correlation.
# ---------------------------------------------------------------------------

@dataclass
class ConvShape:
    n: int
    h: int
    w: int
    c: int
    k: int
    r: int
    s: int
    stride: int
    pad: int

    @property
    def p(self) -> int:
        return (self.h + 2 * self.pad - self.r) // self.stride + 1

    @property
    def q(self) -> int:
        return (self.w + 2 * self.pad - self.s) // self.stride + 1


def conv_fwd_acc(d: ConvShape, x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """Exact Y[n,p,q,k] = sum_{r,s,c} X[n, p*st+r-pad, q*st+s-pad, c] W[k,r,s,c]."""
    st, P, Q = d.stride, d.p, d.q
    xp = np.zeros((d.n, d.h + 2 * d.pad, d.w + 2 * d.pad, d.c), dtype=np.int64)
    xp[:, d.pad:d.pad + d.h, d.pad:d.pad + d.w, :] = x
    acc = np.zeros((d.n * P * Q, d.k), dtype=np.int64)
    for r in range(d.r):
        for s in range(d.s):
            xs = xp[:, r:r + st * (P - 1) + 1:st, s:s + st * (Q - 1) + 1:st, :]
            acc += _exact_matmul(xs.reshape(-1, d.c), w[:, r, s, :].astype(np.int64).T)
    return acc.reshape(d.n, P, Q, d.k)


def conv_dgrad_acc(d: ConvShape, dy: np.ndarray, w: np.ndarray) -> np.ndarray:
    """Exact adjoint of conv_fwd_acc in X: scatter every tap back."""
    st, P, Q = d.stride, d.p, d.q
    dxp = np.zeros((d.n, d.h + 2 * d.pad + st, d.w + 2 * d.pad + st, d.c), dtype=np.int64)
    dy2 = dy.reshape(-1, d.k).astype(np.int64)
    for r in range(d.r):
        for s in range(d.s):
            contrib = _exact_matmul(dy2, w[:, r, s, :].astype(np.int64))
            dxp[:, r:r + st * (P - 1) + 1:st, s:s + st * (Q - 1) + 1:st, :] += \
                contrib.reshape(d.n, P, Q, d.c)
    return dxp[:, d.pad:d.pad + d.h, d.pad:d.pad + d.w, :]


def conv_wgrad_acc(d: ConvShape, dy: np.ndarray, x: np.ndarray) -> np.ndarray:
    """Exact adjoint of conv_fwd_acc in W: dW[k,r,s,c]."""
    st, P, Q = d.stride, d.p, d.q
    xp = np.zeros((d.n, d.h + 2 * d.pad, d.w + 2 * d.pad, d.c), dtype=np.int64)
    xp[:, d.pad:d.pad + d.h, d.pad:d.pad + d.w, :] = x
    dy2 = dy.reshape(-1, d.k).astype(np.int64)
    acc = np.zeros((d.k, d.r, d.s, d.c), dtype=np.int64)
    for r in range(d.r):
        for s in range(d.s):
            xs = xp[:, r:r + st * (P - 1) + 1:st, s:s + st * (Q - 1) + 1:st, :]
            acc[:, r, s, :] = _exact_matmul(dy2.T, xs.reshape(-1, d.c))
    return acc


def conv_fwd(d: ConvShape, X: QT, W: QT, y_group: int = TENSOR, bits: int = Q_BITS) -> QT:
    """Y = conv(X, W): X NHWC TENSOR-grouped, W [K x RSC] TENSOR or ROW."""
    assert X.group == TENSOR
    acc = conv_fwd_acc(d, X.mant.reshape(d.n, d.h, d.w, d.c).astype(np.int64),
                       W.mant.reshape(d.k, d.r, d.s, d.c))
    eps = int(X.row_exp()[0]) + W.row_exp()[None, :]
    out = requant_np(acc.reshape(-1, d.k), np.broadcast_to(eps, (acc.size // d.k, d.k)), y_group, bits)
    return QT(out.mant.reshape(d.n, d.p, d.q, d.k), out.exp, y_group)


def conv_dgrad(d: ConvShape, dY: QT, W: QT, dx_group: int = TENSOR, bits: int = Q_BITS) -> QT:
    """dX: W aligned over output channels (R5), then the exact adjoint."""
    assert dY.group == TENSOR
    w_al, e_w = align_rows(QT(W.mant.reshape(d.k, -1), W.exp, W.group))
    acc = conv_dgrad_acc(d, dY.mant.reshape(d.n, d.p, d.q, d.k), w_al.reshape(d.k, d.r, d.s, d.c))
    eps = int(dY.row_exp()[0]) + e_w
    out = requant_np(acc.reshape(-1, d.c), np.full((acc.size // d.c, d.c), eps), dx_group, bits)
    return QT(out.mant.reshape(d.n, d.h, d.w, d.c), out.exp, dx_group)


def conv_wgrad(d: ConvShape, dY: QT, X: QT, dw_group: int = ROW, bits: int = Q_BITS) -> QT:
    """dW [K x RSC]: exact adjoint, per output channel groups (Table 5)."""
    assert dY.group == TENSOR and X.group == TENSOR
    acc = conv_wgrad_acc(d, dY.mant.reshape(d.n, d.p, d.q, d.k),
                         X.mant.reshape(d.n, d.h, d.w, d.c).astype(np.int64))
    eps = int(dY.row_exp()[0]) + int(X.row_exp()[0])
    return requant_np(acc.reshape(d.k, -1), np.full((d.k, d.r * d.s * d.c), eps), dw_group, bits)


# ---------------------------------------------------------------------------
# Exact sums of (C, e) terms with different exponents
# ---------------------------------------------------------------------------

def exact_sum(terms):
    """Exact elementwise sum of terms (mant int array, exp int array).

    Returns (numerator, exponent): value = numerator * 2**exponent, with the
    exponent the smallest of the terms' exponents.  Numerators are int64 where
    they provably fit, Python ints (object arrays) elsewhere.
    """
    mants = [np.asarray(m, dtype=np.int64) for m, _ in terms]
    exps = [np.broadcast_to(np.asarray(e, dtype=np.int64), mants[0].shape) for _, e in terms]
    base = np.minimum.reduce(exps)
    gaps = [e - base for e in exps]
    mag = sum(np.abs(m) for m in mants)
    small = np.ones(base.shape, dtype=bool)
    for g in gaps:
        small &= g <= 30
    assert np.all(mag < (1 << 21))
    num64 = np.zeros(base.shape, dtype=np.int64)
    for m, g in zip(mants, gaps):
        num64 += np.where(small, m << np.where(small, g, 0), 0)
    if np.all(small):
        return num64, base
    num = num64.astype(object)
    idx = np.nonzero(~small)
    for pos in zip(*idx):
        v = 0
        for m, g in zip(mants, gaps):
            v += int(m[pos]) << int(g[pos])
        num[pos] = v
    return num, base


def requant_exact(num, base, group_of: np.ndarray, n_groups: int, bits: int = Q_BITS):
    """Requantise exact values num * 2**base into groups (reading R3).

    group_of gives each element's group index.  Returns (int8 mantissas,
    int8 exponents per group).
    """
    if num.dtype != object:
        nd = need_np(num, base, bits)
        gmax = np.full(n_groups, -(1 << 40), dtype=np.int64)
        np.maximum.at(gmax, group_of.reshape(-1), nd.reshape(-1))
        e = np.maximum(gmax, E_MIN)
        if np.any(e > E_MAX):
            raise ExpRangeError(f"group exponent {int(e.max())} > {E_MAX}")
        c = rne_np(num, e[group_of] - base)
    else:
        flat_n = num.reshape(-1)
        flat_b = base.reshape(-1)
        flat_g = group_of.reshape(-1)
        gmax = [E_MIN] * n_groups
        for i in range(flat_n.size):
            nd = need_int(flat_n[i], flat_b[i], bits)
            if nd is not None and nd > gmax[flat_g[i]]:
                gmax[flat_g[i]] = nd
        if max(gmax) > E_MAX:
            raise ExpRangeError(f"group exponent {max(gmax)} > {E_MAX}")
        e = np.array(gmax, dtype=np.int64)
        c = np.array([rne_int(flat_n[i], int(e[flat_g[i]]) - int(flat_b[i]))
                      for i in range(flat_n.size)], dtype=np.int64).reshape(num.shape)
    assert np.all(np.abs(c) <= q_max(bits))
    return c.astype(np.int8), e.astype(np.int8)


def _group_index(t: QT) -> tuple:
    rows = t.mant.shape[0]
    per_row = int(np.prod(t.mant.shape[1:], dtype=np.int64))
    if t.group == ROW:
        g = np.repeat(np.arange(rows), per_row).reshape(rows, per_row)
        return g, rows
    return np.zeros((rows, per_row), dtype=np.int64), 1


# ---------------------------------------------------------------------------
# Sum (Table 6 "Residual add, gradient merge -> Sum")
# ---------------------------------------------------------------------------

def sum_op(A: QT, B: QT, out_group: int, bits: int = Q_BITS) -> QT:
    """Exact elementwise A + B, requantised once into out_group."""
    rows = A.mant.shape[0]
    per_row = int(np.prod(A.mant.shape[1:], dtype=np.int64))
    ma = A.mant.reshape(rows, per_row)
    mb = B.mant.reshape(rows, per_row)
    ea = np.broadcast_to(A.row_exp()[:, None], ma.shape)
    eb = np.broadcast_to(B.row_exp()[:, None], mb.shape)
    num, base = exact_sum([(ma, ea), (mb, eb)])
    if out_group == ROW:
        g, ng = np.repeat(np.arange(rows), ma.shape[1]).reshape(ma.shape), rows
    else:
        g, ng = np.zeros(ma.shape, dtype=np.int64), 1
    c, e = requant_exact(num, base, g, ng, bits)
    return QT(c.reshape(A.mant.shape), e, out_group)


# ---------------------------------------------------------------------------
# Divide by a constant (Table 6 "Average pool -> Divide-by-constant")
# ---------------------------------------------------------------------------

def divide_const(A: QT, d: int, out_group: int) -> tuple:
    """Exact rational A / d (d a positive integer), requantised once.

    Rounding is half-to-even on the exact rational (the page's Eqs. 7-8 are
    not printed; a fixed-point reciprocal there would differ).  Small inputs
    only; returns (mantissa rows, exponent list) like requant_frac.
    """
    assert d >= 1
    vals = [[v / d for v in row] for row in A.values()]
    return requant_frac(vals, out_group)


def avg_pool(d: ConvShape, X: QT) -> tuple:
    """K x K average pool (stride K, no padding) of an NHWC TENSOR-grouped
    activation: exact window sum, then divide-by-constant K*K."""
    k = d.r
    x = X.mant.reshape(d.n, d.h, d.w, d.c).astype(np.int64)
    ho, wo = d.h // k, d.w // k
    s = x[:, :ho * k, :wo * k, :].reshape(d.n, ho, k, wo, k, d.c).sum(axis=(2, 4))
    e = int(X.row_exp()[0])
    vals = [[Fraction(int(v)) * Fraction(2) ** e / (k * k) for v in s.reshape(-1)]]
    rows, exps = requant_frac(vals, TENSOR)
    return np.array(rows[0], dtype=np.int64).reshape(d.n, ho, wo, d.c), exps[0]


# ---------------------------------------------------------------------------
# Integer SGD with momentum and per-group velocity (Figure 1b, Table 5)
# ---------------------------------------------------------------------------

@dataclass
class Scalar:
    """A (C, e) scalar such as the learning rate or the momentum."""
    mant: int
    exp: int

    def value(self) -> Fraction:
        return Fraction(self.mant) * Fraction(2) ** self.exp


def sgd_update(W: QT, V: QT, G: QT, lr: Scalar, beta: Scalar,
               wd: Scalar = Scalar(0, 0), w_bits: int = Q_BITS) -> tuple:
    """One integer SGD-with-momentum step on a [N x K] weight (reading R7).

    v_exact = beta*V + G (+ wd*W)        -> V' = requant over V's groups
    w_exact = W - lr*V'                  -> W' = requant over W's groups
    W' takes w_bits of mantissa; V' is always INT8 (reading R8).
    Returns (W', V') as QT.
    """
    rows = W.mant.shape[0]
    shp = (rows, int(np.prod(W.mant.shape[1:], dtype=np.int64)))
    mw = W.mant.reshape(shp).astype(np.int64)
    mv = V.mant.reshape(shp).astype(np.int64)
    mg = G.mant.reshape(shp).astype(np.int64)
    ew = np.broadcast_to(W.row_exp()[:, None], shp)
    ev = np.broadcast_to(V.row_exp()[:, None], shp)
    eg = np.broadcast_to(G.row_exp()[:, None], shp)

    terms = [(beta.mant * mv, ev + beta.exp), (mg, eg)]
    if wd.mant != 0:
        terms.append((wd.mant * mw, ew + wd.exp))
    num_v, base_v = exact_sum(terms)
    gv, ngv = _group_index(QT(mv, V.exp, V.group))
    cv, e_v = requant_exact(num_v, base_v, gv, ngv)
    V_new = QT(cv.reshape(V.mant.shape), e_v, V.group)

    ev_new = np.broadcast_to(V_new.row_exp()[:, None], shp)
    num_w, base_w = exact_sum([(mw, ew), (-lr.mant * cv.astype(np.int64), ev_new + lr.exp)])
    gw, ngw = _group_index(QT(mw, W.exp, W.group))
    cw, e_w = requant_exact(num_w, base_w, gw, ngw, w_bits)
    W_new = QT(cw.reshape(W.mant.shape), e_w, W.group)
    return W_new, V_new


# ---------------------------------------------------------------------------
# Clip activations (Table 7) — forward and backward masks on the mantissa
# ---------------------------------------------------------------------------

def relu_fwd(C: np.ndarray) -> np.ndarray:
    """max(C, 0); the exponent is carried through unchanged (Table 7)."""
    return np.maximum(np.asarray(C, dtype=np.int64), 0)


def relu_bwd(dY: np.ndarray, C: np.ndarray) -> np.ndarray:
    """dY * 1[C > 0] (Table 7)."""
    return np.where(np.asarray(C) > 0, np.asarray(dY, dtype=np.int64), 0)


def relu6_cap(e: int, bits: int = Q_BITS) -> int:
    """c = min(6 >> e, q_max), reading 6 >> e as 6 * 2**-e rounded down
    (a right shift for e > 0, a left shift for e < 0); q_max is that of the
    activation's mantissa width (reading R8)."""
    v = 6 >> e if e >= 0 else 6 << min(-e, 8)
    return min(v, q_max(bits))


def relu6_fwd(C: np.ndarray, e: int, bits: int = Q_BITS) -> np.ndarray:
    """clip(C, 0, c) with c = relu6_cap(e, bits) (Table 7)."""
    return np.clip(np.asarray(C, dtype=np.int64), 0, relu6_cap(e, bits))


def relu6_bwd(dY: np.ndarray, C: np.ndarray, e: int, bits: int = Q_BITS) -> np.ndarray:
    """dY * 1[0 < C < c] (Table 7)."""
    C = np.asarray(C)
    c = relu6_cap(e, bits)
    return np.where((C > 0) & (C < c), np.asarray(dY, dtype=np.int64), 0)


# ---------------------------------------------------------------------------
# Exponent memory (Table 5) and training memory (Table 9's Eq. 28 inputs)
# ---------------------------------------------------------------------------

def exponent_bytes(out_channels_per_layer, per_group: bool) -> int:
    """Exponent storage: one byte per output channel of every weight tensor
    (per-group) or one byte per weight tensor (per-tensor)."""
    if per_group:
        return int(sum(out_channels_per_layer))
    return len(out_channels_per_layer)


def training_memory_gib(params: float, acts_per_sample: float, batch: int,
                        b_w: float, b_g: float, b_v: float, b_a: float) -> float:
    """(b_W + b_G + b_V) * P + b_A * N * A bytes, in GiB."""
    return ((b_w + b_g + b_v) * params + b_a * batch * acts_per_sample) / 2 ** 30
