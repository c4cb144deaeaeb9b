"""GPU parity of the batched products (attention's Q.K^T, P.V and their
gradients as one Product per slice), through the C ABI, bit for bit against
the oracle: the three forms over ragged shapes, both input group kinds, both
epilogues and every tile the planner picks, narrower result widths, empty and
degenerate stacks, and ViT-B's attention at batch 64 with sampled slices."""

import numpy as np
import pytest

import oracle as o
from integer_only_dnn_amd import ie
from tests.gpu_util import announce, assert_same, qt_to_dev

pytestmark = pytest.mark.gpu

T, R = o.TENSOR, o.ROW
FORMS = {"nt": (o.bmm_nt, ie.ie_bmm_nt), "nn": (o.bmm_nn, ie.ie_bmm_nn), "tn": (o.bmm_tn, ie.ie_bmm_tn)}


@pytest.fixture(scope="module")
def ws():
    return ie.Workspace("cuda")


def _qt(rng, rows, cols, group, elo=-14, ehi=-2, zero_frac=0.05, bits=8):
    qm = o.q_max(bits) if bits < 8 else 127
    lo = -qm - 1 if bits == 8 else -qm
    m = rng.integers(lo, qm + 1, size=(rows, cols)).astype(np.int8)
    if zero_frac:
        m[rng.random(m.shape) < zero_frac] = 0
    n = rows if group == R else 1
    return o.QT(m, rng.integers(elo, ehi + 1, size=n).astype(np.int8), group)


def _operands(rng, form, batch, M, N, K, ga, gb, bits=8):
    if form == "nt":
        return _qt(rng, batch * M, K, ga, bits=bits), _qt(rng, batch * N, K, gb, bits=bits)
    if form == "nn":
        return _qt(rng, batch * M, K, ga, bits=bits), _qt(rng, batch * K, N, gb, elo=-24, ehi=0, bits=bits)
    return (_qt(rng, batch * K, M, ga, elo=-24, ehi=0, bits=bits),
            _qt(rng, batch * K, N, gb, elo=-24, ehi=0, bits=bits))


def _run(form, batch, A, B, M, N, ws, bits=8):
    C = ie.Mat.empty(batch * M, N, R, bits=bits)
    FORMS[form][1](batch, qt_to_dev(A), qt_to_dev(B), C, ws)
    return C


SHAPES = [(1, 1, 1, 1), (3, 5, 7, 16), (2, 70, 130, 40), (5, 33, 64, 100), (2, 197, 197, 64), (3, 197, 64, 197),
          (2, 130, 200, 300)]


@pytest.mark.parametrize("form", list(FORMS))
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "b{}m{}n{}k{}".format(*s))
@pytest.mark.parametrize("groups", [(T, T), (R, R), (R, T), (T, R)], ids=lambda g: "".join("TR"[x] for x in g))
def test_bmm(form, shape, groups, ws):
    batch, M, N, K = shape
    announce(f"bmm {form} batch={batch} M={M} N={N} K={K} groups={groups}")
    rng = np.random.default_rng(sum(shape) + 7 * groups[0] + 3 * groups[1] + len(form) * 100 + ord(form[0]))
    A, B = _operands(rng, form, batch, M, N, K, *groups)
    C = _run(form, batch, A, B, M, N, ws)
    assert_same(C, FORMS[form][0](A, B, batch), f"bmm {form}")
    assert ws.status() == 0


# Shapes that lead the planner to each tile and epilogue of the batched
# kernel (512 work items fill the chip): 64x256 direct for A . B^T (rows of
# 129..256; its one-step form when K <= 128), 128x128 direct (rows of
# 65..128) and round-to-odd (rows past 256), 128x64 direct (rows up to 64),
# 64x64 direct and round-to-odd (few slices).
PLAN_SHAPES = [(128, 260, 200, 40), (128, 260, 200, 200), (256, 200, 100, 40), (100, 200, 300, 24),
               (256, 200, 50, 40), (3, 150, 60, 90), (3, 150, 150, 90)]


@pytest.mark.parametrize("form", list(FORMS))
@pytest.mark.parametrize("shape", PLAN_SHAPES, ids=lambda s: "b{}m{}n{}k{}".format(*s))
def test_bmm_plans(form, shape, ws):
    """Every tile and epilogue the planner picks, reached through the shape."""
    batch, M, N, K = shape
    announce(f"bmm plans {form} batch={batch} M={M} N={N} K={K}")
    rng = np.random.default_rng(sum(shape) + ord(form[1]))
    A, B = _operands(rng, form, batch, M, N, K, R, R)
    C = _run(form, batch, A, B, M, N, ws)
    assert_same(C, FORMS[form][0](A, B, batch), f"bmm {form} plan")
    assert ws.status() == 0


@pytest.mark.parametrize("form", list(FORMS))
@pytest.mark.parametrize("bits", [4, 6])
def test_bmm_bits(form, bits, ws):
    batch, M, N, K = 4, 97, 150, 72
    announce(f"bmm {form} bits={bits}")
    rng = np.random.default_rng(300 + bits + ord(form[0]))
    A, B = _operands(rng, form, batch, M, N, K, R, T, bits=bits)
    C = _run(form, batch, A, B, M, N, ws, bits=bits)
    assert_same(C, FORMS[form][0](A, B, batch, bits), f"bmm {form} bits={bits}")


@pytest.mark.parametrize("form", list(FORMS))
def test_bmm_degenerate(form, ws):
    """Empty contraction (zeros at the smallest exponent), empty rows, one
    all-zero slice, and exponents apart by more than 60 between slices."""
    announce(f"bmm {form} degenerate")
    rng = np.random.default_rng(17)
    for batch, M, N, K in ((3, 4, 5, 0), (2, 0, 5, 7), (4, 6, 0, 9)):
        A, B = _operands(rng, form, batch, M, N, K, R, R)
        C = _run(form, batch, A, B, M, N, ws)
        assert_same(C, FORMS[form][0](A, B, batch), f"bmm {form} {batch}x{M}x{N}x{K}")
    batch, M, N, K = 4, 20, 70, 33
    A, B = _operands(rng, form, batch, M, N, K, R, R)
    ra = A.mant.shape[0] // batch
    A.mant[ra:2 * ra] = 0
    A.exp[2 * ra:3 * ra] = np.int8(-100)
    B.exp[:B.mant.shape[0] // batch] = np.int8(40)
    C = _run(form, batch, A, B, M, N, ws)
    assert_same(C, FORMS[form][0](A, B, batch), f"bmm {form} zero slice and far exponents")
    assert ws.status() == 0


def test_bmm_vitb_attention_sampled(ws):
    """ViT-B attention at batch 64 (12 heads, 197 tokens, head size 64: 768
    slices), all six products; slices are independent, so a sample of
    slices is checked against the oracle exactly."""
    batch, heads, S, D = 64, 12, 197, 64
    Z = batch * heads
    announce(f"bmm vitb attention Z={Z} S={S} D={D}")
    rng = np.random.default_rng(2024)
    Q, K, V, dO = (_qt(rng, Z * S, D, R) for _ in range(4))
    P = _qt(rng, Z * S, S, R, elo=-9, ehi=-7)
    dS = _qt(rng, Z * S, S, R)
    Qd, Kd, Vd, dOd, Pd, dSd = (qt_to_dev(t) for t in (Q, K, V, dO, P, dS))
    out = {}
    for name, fn, a, b, n in (("scores", ie.ie_bmm_nt, Qd, Kd, S), ("context", ie.ie_bmm_nn, Pd, Vd, D),
                              ("dP", ie.ie_bmm_nt, dOd, Vd, S), ("dV", ie.ie_bmm_tn, Pd, dOd, D),
                              ("dQ", ie.ie_bmm_nn, dSd, Kd, D), ("dK", ie.ie_bmm_tn, dSd, Qd, D)):
        C = ie.Mat.empty(Z * S, n, R)
        fn(Z, a, b, C, ws)
        out[name] = C
    assert ws.status() == 0

    def sl(t, z):
        rows = t.mant.shape[0] // Z
        return o.QT(t.mant[z * rows:(z + 1) * rows], t.exp[z * rows:(z + 1) * rows], t.group)

    for z in (0, 1, 385, Z - 1):
        want = {"scores": o.bmm_nt(sl(Q, z), sl(K, z), 1), "context": o.bmm_nn(sl(P, z), sl(V, z), 1),
                "dP": o.bmm_nt(sl(dO, z), sl(V, z), 1), "dV": o.bmm_tn(sl(P, z), sl(dO, z), 1),
                "dQ": o.bmm_nn(sl(dS, z), sl(K, z), 1), "dK": o.bmm_tn(sl(dS, z), sl(Q, z), 1)}
        for name, w in want.items():
            C = out[name]
            got = ie.Mat(C.mant[z * S:(z + 1) * S].contiguous(), C.exp[z * S:(z + 1) * S].contiguous(), R)
            assert_same(got, w, f"{name} slice {z}")
