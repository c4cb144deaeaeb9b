"""ctypes binding of libie.so: argument marshalling only.

Every function here forwards to the C entry point of the same name declared
in include/ie.h; all arithmetic runs in the library's HIP kernels.  PyTorch
supplies device memory (int8 CUDA tensors) and the current stream.  The
library must be built (integer_only_dnn_amd/build.py); nothing here falls
back to another implementation.
"""

from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, byref, c_char_p, c_int, c_int8, c_int32, c_int64, c_size_t, c_uint32, c_void_p

import torch

TENSOR = 0
ROW = 1
FLAG_EXP_RANGE = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libie.so")

STATUS = {0: "IE_OK", 1: "IE_ERR_NULL", 2: "IE_ERR_SHAPE", 3: "IE_ERR_GROUP", 4: "IE_ERR_WORKSPACE",
          5: "IE_ERR_EXP_RANGE", 6: "IE_ERR_UNSUPPORTED", 7: "IE_ERR_HIP", 8: "IE_ERR_BITS", 9: "IE_ERR_SCRATCH"}


class IeError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__(f"{where}: {STATUS.get(code, code)}")
        self.code = code


class ie_mat(ctypes.Structure):
    _fields_ = [("mant", c_void_p), ("exp", c_void_p), ("rows", c_int64), ("cols", c_int64),
                ("group", c_int32), ("bits", c_int32)]


class ie_conv_desc(ctypes.Structure):
    _fields_ = [(n, c_int32) for n in ("n", "h", "w", "c", "k", "r", "s", "stride", "pad")]


class ie_scalar(ctypes.Structure):
    _fields_ = [("mant", c_int8), ("exp", c_int8)]


EXPORTS = [
    ("ie_linear_fwd_workspace", c_size_t, [c_int64, c_int64, c_int64]),
    ("ie_linear_bwd_dx_workspace", c_size_t, [c_int64, c_int64, c_int64]),
    ("ie_linear_bwd_dw_workspace", c_size_t, [c_int64, c_int64, c_int64]),
    ("ie_conv_fwd_workspace", c_size_t, [POINTER(ie_conv_desc)]),
    ("ie_conv_bwd_workspace", c_size_t, [POINTER(ie_conv_desc)]),
    ("ie_sgd_update_workspace", c_size_t, [c_int64, c_int64]),
    ("ie_sgd_update_multi_workspace", c_size_t, [c_int32]),
    ("ie_workspace_init", c_int, [c_void_p, c_size_t, c_void_p]),
    ("ie_linear_fwd", c_int, [POINTER(ie_mat)] * 3 + [c_void_p, c_size_t, c_void_p]),
    ("ie_linear_fwd_noalloc", c_int, [POINTER(ie_mat)] * 3 + [c_void_p, c_void_p]),
    ("ie_linear_bwd_dx", c_int, [POINTER(ie_mat)] * 3 + [c_void_p, c_size_t, c_void_p]),
    ("ie_linear_bwd_dw", c_int, [POINTER(ie_mat)] * 3 + [c_void_p, c_size_t, c_void_p]),
    ("ie_conv_fwd", c_int, [POINTER(ie_conv_desc)] + [POINTER(ie_mat)] * 3 + [c_void_p, c_size_t, c_void_p]),
    ("ie_conv_bwd", c_int, [POINTER(ie_conv_desc)] + [POINTER(ie_mat)] * 5 + [c_void_p, c_size_t, c_void_p]),
    ("ie_sgd_update", c_int, [POINTER(ie_mat)] * 3 + [ie_scalar] * 3 + [c_void_p, c_size_t, c_void_p]),
    ("ie_bmm_workspace", c_size_t, [c_int32, c_int64, c_int64, c_int64]),
    ("ie_bmm_nt", c_int, [c_int32] + [POINTER(ie_mat)] * 3 + [c_void_p, c_size_t, c_void_p]),
    ("ie_bmm_nn", c_int, [c_int32] + [POINTER(ie_mat)] * 3 + [c_void_p, c_size_t, c_void_p]),
    ("ie_bmm_tn", c_int, [c_int32] + [POINTER(ie_mat)] * 3 + [c_void_p, c_size_t, c_void_p]),
    ("ie_sgd_update_multi", c_int, [c_int32] + [POINTER(ie_mat)] * 3 + [ie_scalar] * 3 + [c_void_p, c_size_t, c_void_p]),
    ("ie_linear_fwd_act", c_int, [POINTER(ie_mat)] * 3 + [c_int, c_void_p, c_size_t, c_void_p]),
    ("ie_conv_fwd_act", c_int, [POINTER(ie_conv_desc)] + [POINTER(ie_mat)] * 3 + [c_int, c_void_p, c_size_t, c_void_p]),
    ("ie_linear_bwd_dx_act", c_int, [POINTER(ie_mat)] * 4 + [c_int, c_void_p, c_size_t, c_void_p]),
    ("ie_conv_bwd_act", c_int, [POINTER(ie_conv_desc)] + [POINTER(ie_mat)] * 5 + [c_int, c_void_p, c_size_t, c_void_p]),
    ("ie_relu_fwd", c_int, [POINTER(ie_mat)] * 2 + [c_int, c_void_p]),
    ("ie_relu_bwd", c_int, [POINTER(ie_mat)] * 3 + [c_int, c_void_p]),
    ("ie_add_workspace", c_size_t, [c_int64, c_int64]),
    ("ie_add", c_int, [POINTER(ie_mat)] * 3 + [c_void_p, c_size_t, c_void_p]),
    ("ie_device_status", c_int, [c_void_p, c_void_p, POINTER(c_uint32), c_int]),
    ("ie_profile_enable", c_int, [c_int]),
    ("ie_profile_select", c_int, [c_int]),
    ("ie_profile_read", c_int, [POINTER(ctypes.c_float), POINTER(c_int), c_int]),
    ("ie_status_str", c_char_p, [c_int]),
]

_lib = None


def lib() -> ctypes.CDLL:
    """Load libie.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with integer_only_dnn_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        for name, res, args in EXPORTS:
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(code: int, where: str) -> None:
    if code != 0:
        raise IeError(code, where)


def _stream(dev: torch.device) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


class Mat:
    """A (C, e) matrix in device memory: int8 mantissas [rows, cols],
    int8 exponents (1 entry for TENSOR, `rows` for ROW), and the mantissa
    width `bits` (2..8) that results rounded into it take."""

    def __init__(self, mant: torch.Tensor, exp: torch.Tensor, group: int, bits: int = 8):
        assert mant.dtype == torch.int8 and exp.dtype == torch.int8
        assert mant.is_contiguous() and exp.is_contiguous()
        self.mant = mant
        self.exp = exp
        self.group = int(group)
        self.bits = int(bits)
        self._desc = {}  # (rows, cols, bits) -> (mant, exp, ie_mat): descriptors built once per view

    @staticmethod
    def empty(rows: int, cols: int, group: int, device="cuda", bits: int = 8) -> "Mat":
        m = torch.empty((rows, cols), dtype=torch.int8, device=device)
        e = torch.empty((rows if group == ROW else 1,), dtype=torch.int8, device=device)
        return Mat(m, e, group, bits)

    def c(self, rows=None, cols=None) -> ie_mat:
        """The C descriptor; `rows`/`cols` view an NHWC tensor as [N*H*W x C].
        Built once per view and reused while `mant` and `exp` are the same
        tensors."""
        key = (rows, cols, self.bits)
        hit = self._desc.get(key)
        if hit is not None and hit[0] is self.mant and hit[1] is self.exp:
            return hit[2]
        r, c = rows, cols
        if r is None:
            assert self.mant.dim() == 2
            r, c = self.mant.shape
        d = ie_mat(self.mant.data_ptr(), self.exp.data_ptr(), r, c, self.group, self.bits)
        self._desc[key] = (self.mant, self.exp, d)
        return d


class Workspace:
    """Device scratch for the library, grown on demand; its first 256 bytes
    hold the sticky status flags (zeroed when the buffer is created)."""

    def __init__(self, device="cuda"):
        self.device = torch.device(device)
        self.buf = None

    def get(self, nbytes: int):
        if self.buf is None or self.buf.numel() < nbytes:
            flags = self.status(clear=False) if self.buf is not None else 0
            self.buf = torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=self.device)
            _check(lib().ie_workspace_init(self.buf.data_ptr(), self.buf.numel(), _stream(self.device)),
                   "ie_workspace_init")
            if flags:
                raise IeError(5, "workspace flags were set before it grew")
        return self.buf.data_ptr(), self.buf.numel()

    def status(self, clear: bool = True) -> int:
        if self.buf is None:
            return 0
        f = c_uint32(0)
        _check(lib().ie_device_status(self.buf.data_ptr(), _stream(self.device), byref(f), int(clear)),
               "ie_device_status")
        return f.value


def conv_desc(n, h, w, c, k, r, s, stride, pad) -> ie_conv_desc:
    return ie_conv_desc(n, h, w, c, k, r, s, stride, pad)


_ws_sizes = {}


def _ws_size(name: str, *args) -> int:
    """The library's workspace size for a call shape (memoised: the library
    plans the call to answer; the planner's tuning overrides are part of the
    key)."""
    key = (name, os.environ.get("IE_TILE"), os.environ.get("IE_WTILE")) + tuple((a.n, a.h, a.w, a.c, a.k, a.r, a.s, a.stride, a.pad) if isinstance(a, ie_conv_desc) else a
                          for a in args)
    n = _ws_sizes.get(key)
    if n is None:
        fn = getattr(lib(), name)
        n = fn(*[byref(a) if isinstance(a, ie_conv_desc) else a for a in args])
        _ws_sizes[key] = n
    return n


def ie_linear_fwd(X: Mat, W: Mat, Y: Mat, ws: Workspace) -> None:
    x, w, y = X.c(), W.c(), Y.c()
    p, b = ws.get(_ws_size("ie_linear_fwd_workspace", x.rows, w.rows, x.cols))
    _check(lib().ie_linear_fwd(byref(x), byref(w), byref(y), p, b, _stream(ws.device)), "ie_linear_fwd")


def ie_linear_fwd_noalloc(X: Mat, W: Mat, Y: Mat, flags: torch.Tensor | None = None) -> None:
    """ie_linear_fwd on the library's fixed device scratch (no workspace);
    flags: an int32 device tensor receiving the exponent-range flag, or None."""
    x, w, y = X.c(), W.c(), Y.c()
    fp = c_void_p(flags.data_ptr()) if flags is not None else None
    _check(lib().ie_linear_fwd_noalloc(byref(x), byref(w), byref(y), fp, _stream(X.mant.device)),
           "ie_linear_fwd_noalloc")


def ie_linear_bwd_dx(dY: Mat, W: Mat, dX: Mat, ws: Workspace) -> None:
    dy, w, dx = dY.c(), W.c(), dX.c()
    p, b = ws.get(_ws_size("ie_linear_bwd_dx_workspace", dy.rows, dy.cols, w.cols))
    _check(lib().ie_linear_bwd_dx(byref(dy), byref(w), byref(dx), p, b, _stream(ws.device)), "ie_linear_bwd_dx")


def ie_linear_bwd_dw(dY: Mat, X: Mat, dW: Mat, ws: Workspace) -> None:
    dy, x, dw = dY.c(), X.c(), dW.c()
    p, b = ws.get(_ws_size("ie_linear_bwd_dw_workspace", dy.rows, dy.cols, x.cols))
    _check(lib().ie_linear_bwd_dw(byref(dy), byref(x), byref(dw), p, b, _stream(ws.device)), "ie_linear_bwd_dw")


def ie_conv_fwd(d: ie_conv_desc, X: Mat, W: Mat, Y: Mat, ws: Workspace) -> None:
    x = X.c(d.n * d.h * d.w, d.c)
    w = W.c(d.k, d.r * d.s * d.c)
    P = (d.h + 2 * d.pad - d.r) // d.stride + 1
    Q = (d.w + 2 * d.pad - d.s) // d.stride + 1
    y = Y.c(d.n * P * Q, d.k)
    p, b = ws.get(_ws_size("ie_conv_fwd_workspace", d))
    _check(lib().ie_conv_fwd(byref(d), byref(x), byref(w), byref(y), p, b, _stream(ws.device)), "ie_conv_fwd")


def ie_conv_bwd(d: ie_conv_desc, X: Mat, W: Mat, dY: Mat, dX: Mat | None, dW: Mat | None,
                ws: Workspace) -> None:
    P = (d.h + 2 * d.pad - d.r) // d.stride + 1
    Q = (d.w + 2 * d.pad - d.s) // d.stride + 1
    x = X.c(d.n * d.h * d.w, d.c)
    w = W.c(d.k, d.r * d.s * d.c)
    dy = dY.c(d.n * P * Q, d.k)
    dx = dX.c(d.n * d.h * d.w, d.c) if dX is not None else None
    dw = dW.c(d.k, d.r * d.s * d.c) if dW is not None else None
    p, b = ws.get(_ws_size("ie_conv_bwd_workspace", d))
    _check(lib().ie_conv_bwd(byref(d), byref(x), byref(w), byref(dy),
                             byref(dx) if dx is not None else None,
                             byref(dw) if dw is not None else None, p, b, _stream(ws.device)), "ie_conv_bwd")


def ie_conv_bwd_act(d: ie_conv_desc, X: Mat, W: Mat, dY: Mat, dX: Mat | None, dW: Mat | None, act: int,
                    ws: Workspace) -> None:
    """ie_conv_bwd with dX passed back through the activation whose output is X."""
    P = (d.h + 2 * d.pad - d.r) // d.stride + 1
    Q = (d.w + 2 * d.pad - d.s) // d.stride + 1
    x = X.c(d.n * d.h * d.w, d.c)
    w = W.c(d.k, d.r * d.s * d.c)
    dy = dY.c(d.n * P * Q, d.k)
    dx = dX.c(d.n * d.h * d.w, d.c) if dX is not None else None
    dw = dW.c(d.k, d.r * d.s * d.c) if dW is not None else None
    p, b = ws.get(_ws_size("ie_conv_bwd_workspace", d))
    _check(lib().ie_conv_bwd_act(byref(d), byref(x), byref(w), byref(dy),
                                 byref(dx) if dx is not None else None,
                                 byref(dw) if dw is not None else None, int(act), p, b, _stream(ws.device)),
           "ie_conv_bwd_act")


def ie_linear_bwd_dx_act(dY: Mat, W: Mat, X: Mat, dX: Mat, act: int, ws: Workspace) -> None:
    """ie_linear_bwd_dx with dX passed back through the activation whose output is X."""
    dy, w, x, dx = dY.c(), W.c(), X.c(), dX.c()
    p, b = ws.get(_ws_size("ie_linear_bwd_dx_workspace", dy.rows, dy.cols, w.cols))
    _check(lib().ie_linear_bwd_dx_act(byref(dy), byref(w), byref(x), byref(dx), int(act), p, b, _stream(ws.device)),
           "ie_linear_bwd_dx_act")


def ie_sgd_update(W: Mat, V: Mat, G: Mat, lr, momentum, weight_decay=(0, 0), ws: Workspace = None) -> None:
    w, v, g = W.c(), V.c(), G.c()
    p, b = ws.get(_ws_size("ie_sgd_update_workspace", w.rows, w.cols))
    _check(lib().ie_sgd_update(byref(w), byref(v), byref(g), ie_scalar(*lr), ie_scalar(*momentum),
                               ie_scalar(*weight_decay), p, b, _stream(ws.device)), "ie_sgd_update")


def ie_sgd_update_multi(Ws, Vs, Gs, lr, momentum, weight_decay=(0, 0), ws: Workspace = None) -> None:
    """ie_sgd_update over lists of tensors (one optimiser step for many layers)."""
    n = len(Ws)
    if len(Vs) != n or len(Gs) != n:
        raise ValueError("W, V and G lists differ in length")
    arr = ie_mat * max(n, 1)
    w = arr(*[m.c() for m in Ws])
    v = arr(*[m.c() for m in Vs])
    g = arr(*[m.c() for m in Gs])
    p, b = ws.get(_ws_size("ie_sgd_update_multi_workspace", n))
    _check(lib().ie_sgd_update_multi(n, w, v, g, ie_scalar(*lr), ie_scalar(*momentum), ie_scalar(*weight_decay),
                                     p, b, _stream(ws.device)), "ie_sgd_update_multi")


def _bmm(name: str, batch: int, A: Mat, B: Mat, C: Mat, ws: Workspace) -> None:
    a, b, c = A.c(), B.c(), C.c()
    if name == "ie_bmm_nt":
        m, n, k = a.rows // max(batch, 1), b.rows // max(batch, 1), a.cols
    elif name == "ie_bmm_nn":
        m, n, k = a.rows // max(batch, 1), b.cols, a.cols
    else:
        m, n, k = a.cols, b.cols, a.rows // max(batch, 1)
    p, nb = ws.get(lib().ie_bmm_workspace(batch, m, n, k))
    _check(getattr(lib(), name)(batch, byref(a), byref(b), byref(c), p, nb, _stream(ws.device)), name)


def ie_bmm_nt(batch: int, A: Mat, B: Mat, C: Mat, ws: Workspace) -> None:
    """C_z = A_z . B_z^T for every slice z of the stacks (attention scores)."""
    _bmm("ie_bmm_nt", batch, A, B, C, ws)


def ie_bmm_nn(batch: int, A: Mat, B: Mat, C: Mat, ws: Workspace) -> None:
    """C_z = A_z . B_z (attention context P . V)."""
    _bmm("ie_bmm_nn", batch, A, B, C, ws)


def ie_bmm_tn(batch: int, A: Mat, B: Mat, C: Mat, ws: Workspace) -> None:
    """C_z = A_z^T . B_z (attention's key and value gradients)."""
    _bmm("ie_bmm_tn", batch, A, B, C, ws)


ACT_NONE, ACT_RELU = 0, 1


def ie_linear_fwd_act(X: Mat, W: Mat, Y: Mat, act: int, ws: Workspace) -> None:
    """ie_linear_fwd with the activation fused into the output."""
    x, w, y = X.c(), W.c(), Y.c()
    p, b = ws.get(_ws_size("ie_linear_fwd_workspace", x.rows, w.rows, x.cols))
    _check(lib().ie_linear_fwd_act(byref(x), byref(w), byref(y), int(act), p, b, _stream(ws.device)),
           "ie_linear_fwd_act")


def ie_conv_fwd_act(d: ie_conv_desc, X: Mat, W: Mat, Y: Mat, act: int, ws: Workspace) -> None:
    """ie_conv_fwd with the activation fused into the output."""
    x = X.c(d.n * d.h * d.w, d.c)
    w = W.c(d.k, d.r * d.s * d.c)
    P = (d.h + 2 * d.pad - d.r) // d.stride + 1
    Q = (d.w + 2 * d.pad - d.s) // d.stride + 1
    y = Y.c(d.n * P * Q, d.k)
    p, b = ws.get(_ws_size("ie_conv_fwd_workspace", d))
    _check(lib().ie_conv_fwd_act(byref(d), byref(x), byref(w), byref(y), int(act), p, b, _stream(ws.device)),
           "ie_conv_fwd_act")


def ie_relu_fwd(X: Mat, Y: Mat, relu6: bool = False) -> None:
    """ReLU (or ReLU6) of X's mantissas into Y; Y may be X."""
    x, y = X.c(), Y.c()
    _check(lib().ie_relu_fwd(byref(x), byref(y), int(relu6), _stream(X.mant.device)), "ie_relu_fwd")


def ie_relu_bwd(dY: Mat, Y: Mat, dX: Mat, relu6: bool = False) -> None:
    """dY masked where the forward output Y was clipped, into dX; dX may be dY."""
    dy, y, dx = dY.c(), Y.c(), dX.c()
    _check(lib().ie_relu_bwd(byref(dy), byref(y), byref(dx), int(relu6), _stream(dY.mant.device)), "ie_relu_bwd")


def ie_add(A: Mat, B: Mat, Z: Mat, ws: Workspace) -> None:
    """Z = A + B, exact, rounded once into Z's groups."""
    a, b, z = A.c(), B.c(), Z.c()
    p, nb = ws.get(_ws_size("ie_add_workspace", a.rows, a.cols))
    _check(lib().ie_add(byref(a), byref(b), byref(z), p, nb, _stream(ws.device)), "ie_add")


def ie_profile_enable(on: bool = True) -> None:
    _check(lib().ie_profile_enable(int(on)), "ie_profile_enable")


def ie_profile_select(kind: int = 0) -> None:
    """Time only kernels of this kind (0: all)."""
    _check(lib().ie_profile_select(int(kind)), "ie_profile_select")


def ie_profile_read(max_records: int = 1 << 16):
    """[(milliseconds, kind)] of the kernels launched since the last read."""
    ms = (ctypes.c_float * max_records)()
    kind = (c_int * max_records)()
    n = lib().ie_profile_read(ms, kind, max_records)
    return [(ms[i], kind[i]) for i in range(min(n, max_records))]
