"""Benchmark of the integer-only (C, e) layer step on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input:
for every layer, the forward product, the input gradient and the weight
gradient, then one integer SGD-momentum update of every layer's weights (a
single multi-tensor call, as an optimiser step runs after the backward pass).

Default workload: the bottleneck convolutions of a ResNet-50 on 224x224x3
inputs at batch 128 (23 layer shapes, 52 instances, each with its own
tensors; NHWC, per-tensor activation exponents, per-output-channel weight,
weight-gradient and velocity exponents), the largest of the workloads.
Other workloads (--workload) are the ResNet-18 3x3 convolutions on 32x32x3
inputs, the ViT-B and ViT-Ti block linears, the single small linear layer,
the pointwise steps and the ViT-B attention products.

Output: one JSON line (rank 0).  `value` is the step's algorithmic int8 ops
(2*M*N*K per product; the input gradient counted at the forward MAC count)
divided by the measured step time (K steps with no instrumentation).
`roofline` describes the kernel that takes the most time: an untimed
breakdown pass, with HIP events around every kernel launch, picks it; the
same K steps then run again with HIP events (on the launch stream) around
that kernel's launches only, the other launches unbracketed, which gives its
average launch time (`ms_per_step_with_kernel_events` is that pass's step
time).  `kernels` (--kernels) is the breakdown pass.  `cpu_baseline` times the oracle on a bounded sample of the same
workload on the host cores.
"""

from __future__ import annotations

import argparse
import gc
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads as wl  # noqa: E402

PEAK_INT8_TOPS = 5000.0      # MI355X dense INT8 MFMA, 5.0 POP/s
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, 8 TB/s
# ops per algorithmic byte at which the two roofs meet (625)
RIDGE_OPS_PER_BYTE = PEAK_INT8_TOPS * 1e12 / (PEAK_HBM_GBS * 1e9)


def roofline(ops, nbytes, ms):
    """Roofline entry of a kernel that did `ops` int8 operations and moved
    `nbytes` algorithmic bytes in `ms` milliseconds: a contraction whose ops
    per byte reach the ridge point is priced against the MFMA peak, anything
    below it (or with no ops) against HBM bandwidth."""
    if ops > 0 and nbytes > 0 and ops / nbytes >= RIDGE_OPS_PER_BYTE:
        achieved = ops / (ms * 1e-3) / 1e12
        return {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_INT8_TOPS, "unit": "TOPS",
                "frac": round(achieved / PEAK_INT8_TOPS, 4), "traffic": None}
    achieved = nbytes / (ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None}
METRIC = "int8 layer fwd+bwd TOPS & % INT8 MFMA peak; SGD-update GB/s & % HBM"

LOADER = {0: "K", 1: "T", 2: "im2col", 3: "dgrad", 4: "im2colT", 5: "WT"}
EPI = {0: "direct", 1: "rto", 2: "partial", 4: "bmm_direct", 5: "bmm_rto", 6: "bmm1_direct", 7: "bmm1_rto",
       8: "max", 9: "given"}
OTHER = {2000: ("sgd_pass0", "sgd_rows_kernel"), 2001: ("sgd_pass1", "sgd_rows_kernel"),
         2002: ("sgd_pass2", "sgd_rows_kernel"), 3000: ("rto_finalize", "rto_finalize_kernel"),
         3100: ("partial_reduce", "partial_reduce_kernel"), 3150: ("round_sums", "round_sums_kernel"),
         3200: ("pad_align", "pad_rows_kernel / align_transpose_kernel"),
         3210: ("pad_align_z", "pad_rows_z_kernel"),
         3300: ("split_round", "split_round_rows_kernel"),
         3400: ("finalize_pair", "finalize_pair_kernel"),
         3500: ("relu_fwd", "relu_fwd_kernel"), 3510: ("relu_bwd", "relu_bwd_kernel"),
         3520: ("add_need", "add_need_kernel"), 3521: ("add_round", "add_round_kernel"),
         3530: ("add_rows", "add_rows_kernel")}


ONE_KIND = 99000000  # added to the code of a one-step (K <= 128) contraction kernel
ROW_KIND = 200000000  # added to the code of a kernel built for row-grouped results


def is_gemm(kind: int) -> bool:
    return kind >= 10000 and 1000 <= kind % 10000 < 2000


def is_row(kind: int) -> bool:
    return is_gemm(kind) and kind >= ROW_KIND


def _base(kind: int) -> int:
    return kind - ROW_KIND if is_row(kind) else kind


def is_one(kind: int) -> bool:
    return _base(kind) >= ONE_KIND


def is_pair(kind: int) -> bool:
    """Input and weight gradient of a convolution in one grid (two products)."""
    return is_gemm(kind) and (kind % 10000 - 1000) // 100 == 3


def _decode(kind: int):
    t1, t2 = (kind // 10000) % 100, kind // 1000000
    k = kind % 10000 - 1000
    return t1 // 10, t1 % 10, t2 // 10, t2 % 10, (k % 100) // 10, k % 10, k // 100


def kind_name(kind: int) -> str:
    if not is_gemm(kind):
        return OTHER.get(kind, (str(kind), ""))[0]
    if is_row(kind):
        return kind_name(_base(kind)) + "_rows"
    if is_one(kind):
        return kind_name(kind - ONE_KIND) + "_1step"
    mi, ni, mi2, ni2, ka, kb, epi = _decode(kind)
    if is_pair(kind):
        return f"gemm_pair_{LOADER[ka]}_{LOADER[kb]}_rto_{64 * mi}x{64 * ni}+T_im2colT_partial_{64 * mi2}x{64 * ni2}"
    return f"gemm_{LOADER[ka]}_{LOADER[kb]}_{EPI[epi]}_{64 * mi}x{64 * ni}"


def kind_symbol(kind: int) -> str:
    """The kernel's name as rocprofv3 reports it."""
    if not is_gemm(kind):
        return OTHER.get(kind, ("", str(kind)))[1]
    rg = 1 if is_row(kind) else 0
    kind = _base(kind)
    if is_one(kind):
        mi, ni, _, _, ka, kb, epi = _decode(kind - ONE_KIND)
        if epi == 8:
            return f"gemm_max_kernel<{ka}, {kb}, {mi}, {ni}, true, {rg}>"
        return f"gemm_i8_kernel<{ka}, {kb}, {mi}, {ni}, false, true, {rg}, {0 if epi == 1 else 1}>"
    mi, ni, mi2, ni2, ka, kb, epi = _decode(kind)
    if is_pair(kind):
        return f"gemm_pair_kernel<{ka}, {kb}, {mi}, {ni}, 1, 4, {mi2}, {ni2}>"
    if epi in (4, 5, 6, 7):
        return f"gemm_batched_kernel<{ka}, {kb}, {mi}, {ni}, {'true' if epi >= 6 else 'false'}>"
    if epi == 8:
        return f"gemm_max_kernel<{ka}, {kb}, {mi}, {ni}, false, {rg}>"
    if epi == 2:
        return f"gemm_i8_kernel<{ka}, {kb}, {mi}, {ni}, true, false, 0, 0>"
    return f"gemm_i8_kernel<{ka}, {kb}, {mi}, {ni}, false, false, {rg}, {0 if epi == 1 else 1}>"


# ---------------------------------------------------------------------------
# Workload construction (device side)
# ---------------------------------------------------------------------------

class Call:
    """One library call of the step: a closure plus what it computes."""

    def __init__(self, label, fn, ops=0.0, bytes_=0.0, io=0.0, outs=(), prep=()):
        self.label = label
        self.fn = fn
        self.ops = ops          # algorithmic int8 ops of its contraction(s)
        self.bytes = bytes_     # algorithmic HBM bytes (update)
        self.io = io            # algorithmic bytes of each contraction: operands read once, result written once
        self.outs = list(outs)  # int8 result bytes of each contraction, in launch order
        self.prep = list(prep)  # algorithmic bytes of each padding / alignment copy, in launch order
        self.ios = None         # per-contraction algorithmic bytes, in launch order (default: io each)
        self.pair_io = io       # a paired launch of two products: operands read once, both results written
        self.kinds = None


def _dev(torch, ie, code, rows=None):
    m = np.ascontiguousarray(code.mant)
    if m.ndim != 2:
        m = m.reshape(rows if rows is not None else m.shape[0], -1)
    return ie.Mat(torch.from_numpy(m).cuda(), torch.from_numpy(np.ascontiguousarray(code.exp)).cuda(), code.group)


def build_resnet18(torch, ie, ws, batch):
    calls, meta = [], {"layers": [], "params": 0}
    upd_w, upd_v, upd_g, upd_bytes = [], [], [], 0.0
    layers = wl.resnet18_cifar_layers(batch)
    seed = 2000
    for L in layers:
        for inst in range(L.count):
            seed += 1
            inp = wl.resnet18_conv_inputs(L, seed)
            d = ie.conv_desc(L.n, L.h, L.w, L.c, L.k, L.r, L.s, L.stride, L.pad)
            M, N, K = L.gemm_mnk()
            X = _dev(torch, ie, inp.X, rows=L.n * L.h * L.w)
            W = _dev(torch, ie, inp.W)
            dY = _dev(torch, ie, inp.dY, rows=M)
            Y = ie.Mat.empty(M, N, wl.TENSOR)
            dX = None if L.first else ie.Mat.empty(L.n * L.h * L.w, L.c, wl.TENSOR)
            dW = ie.Mat.empty(N, K, wl.ROW)
            upd = wl.update_inputs(N, K, seed + 50000, w_group=wl.TENSOR)
            V = _dev(torch, ie, upd.V)
            ops = 2.0 * M * N * K
            io = _conv_ios(L, M, N, K)
            name = f"{L.name}#{inst}"
            calls.append(Call(f"{name}:fwd", lambda d=d, X=X, W=W, Y=Y: ie.ie_conv_fwd(d, X, W, Y, ws), ops,
                              io=io["fwd"], outs=[M * N]))
            bwd_ops = ops * (1 if L.first else 2)
            c = Call(f"{name}:bwd", lambda d=d, X=X, W=W, dY=dY, dX=dX, dW=dW:
                     ie.ie_conv_bwd(d, X, W, dY, dX, dW, ws), bwd_ops, io=io["wgrad"] if L.first else io["dgrad"],
                     outs=([] if L.first else [L.n * L.h * L.w * L.c]) + [N * K])
            c.ios = [io["wgrad"]] if L.first else [io["dgrad"], io["wgrad"]]
            c.pair_io = io["pair"]
            calls.append(c)
            params = N * K
            # read W, V, G and write W, V (1 byte each) + group exponents
            upd_bytes += 5.0 * params + 3.0 * N + 2.0
            upd_w.append(W)
            upd_v.append(V)
            upd_g.append(dW)
            meta["params"] += params
        meta["layers"].append({"name": L.name, "count": L.count, "gemm_mnk": list(L.gemm_mnk())})
    # one optimiser step over every layer, after the products
    calls.append(Call("update_all", lambda: ie.ie_sgd_update_multi(upd_w, upd_v, upd_g, wl.LR, wl.MOMENTUM, ws=ws),
                      0.0, upd_bytes))
    return calls, meta


def _conv_ios(L, M, N, K):
    """Algorithmic bytes of a convolution's products: forward (X, W read, Y
    written), input gradient (dY, W read, dX written), weight gradient (dY, X
    read, dW written), and the paired backward launch (dY, W, X read once, dX
    and dW written)."""
    x, w, y = float(L.n * L.h * L.w * L.c), float(N * K), float(M * N)
    return {"fwd": x + w + y, "dgrad": y + w + x, "wgrad": y + x + w, "pair": y + w + x + x + w}


def build_resnet50(torch, ie, ws, batch):
    """Every bottleneck convolution instance of a ResNet-50 at batch 128 with
    its own device tensors (the step's working set is several GB, far beyond
    the 256 MB last-level cache), then one SGD-momentum update of every conv
    weight (per-output-channel weight, velocity and gradient exponents)."""
    calls, meta = [], {"layers": [], "params": 0}
    upd_w, upd_v, upd_g, upd_bytes = [], [], [], 0.0
    seed = 4000
    for L in wl.resnet50_layers(batch):
        seed += 1
        inp = wl.resnet50_conv_inputs(L, seed)
        upd = wl.update_inputs(L.k, L.r * L.s * L.c, seed + 50000)
        d = ie.conv_desc(L.n, L.h, L.w, L.c, L.k, L.r, L.s, L.stride, L.pad)
        M, N, K = L.gemm_mnk()
        ops = 2.0 * M * N * K
        io = _conv_ios(L, M, N, K)
        for inst in range(L.count):
            # distinct device copies per instance: no instance reads another's
            # data from cache
            X = _dev(torch, ie, inp.X, rows=L.n * L.h * L.w)
            W = _dev(torch, ie, inp.W)
            dY = _dev(torch, ie, inp.dY, rows=M)
            V = _dev(torch, ie, upd.V)
            Y = ie.Mat.empty(M, N, wl.TENSOR)
            dX = ie.Mat.empty(L.n * L.h * L.w, L.c, wl.TENSOR)
            dW = ie.Mat.empty(N, K, wl.ROW)
            calls.append(Call(f"{L.name}#{inst}:fwd", lambda d=d, X=X, W=W, Y=Y: ie.ie_conv_fwd(d, X, W, Y, ws), ops,
                              io=io["fwd"], outs=[M * N]))
            c = Call(f"{L.name}#{inst}:bwd", lambda d=d, X=X, W=W, dY=dY, dX=dX, dW=dW:
                     ie.ie_conv_bwd(d, X, W, dY, dX, dW, ws), 2 * ops, io=io["dgrad"],
                     outs=[L.n * L.h * L.w * L.c, N * K])
            c.ios = [io["dgrad"], io["wgrad"]]
            c.pair_io = io["pair"]
            calls.append(c)
            upd_bytes += 5.0 * N * K + 5.0 * N
            upd_w.append(W)
            upd_v.append(V)
            upd_g.append(dW)
            meta["params"] += N * K
        meta["layers"].append({"name": L.name, "count": L.count, "gemm_mnk": [M, N, K]})
    calls.append(Call("update_all", lambda: ie.ie_sgd_update_multi(upd_w, upd_v, upd_g, wl.LR, wl.MOMENTUM, ws=ws),
                      0.0, upd_bytes))
    return calls, meta


def build_vit(torch, ie, ws, layers, with_update):
    calls, meta = [], {"layers": [], "params": 0}
    seed = 5000
    for L in layers:
        seed += 1
        inp = wl.vit_linear_inputs(L, seed)
        X, W, dY = _dev(torch, ie, inp.X), _dev(torch, ie, inp.W), _dev(torch, ie, inp.dY)
        Y = ie.Mat.empty(L.m, L.n, inp.y_group)
        dX = ie.Mat.empty(L.m, L.k, inp.dx_group)
        dW = ie.Mat.empty(L.n, L.k, inp.dw_group)
        ops = 2.0 * L.m * L.n * L.k
        io = float(L.m * L.k + L.n * L.k + L.m * L.n)
        calls.append(Call(f"{L.name}:fwd", lambda X=X, W=W, Y=Y: ie.ie_linear_fwd(X, W, Y, ws), ops, io=io,
                          outs=[L.m * L.n]))
        calls.append(Call(f"{L.name}:dx", lambda dY=dY, W=W, dX=dX: ie.ie_linear_bwd_dx(dY, W, dX, ws), ops, io=io,
                          outs=[L.m * L.k]))
        calls.append(Call(f"{L.name}:dw", lambda dY=dY, X=X, dW=dW: ie.ie_linear_bwd_dw(dY, X, dW, ws), ops, io=io,
                          outs=[L.n * L.k]))
        meta["layers"].append({"name": L.name, "gemm_mnk": [L.m, L.n, L.k]})
    if with_update:
        ws_, vs_, gs_, ubytes = [], [], [], 0.0
        for i, (rows, cols) in enumerate(wl.vit_b_param_arenas()):
            upd = wl.update_inputs(rows, cols, 6000 + i)
            ws_.append(_dev(torch, ie, upd.W))
            vs_.append(_dev(torch, ie, upd.V))
            gs_.append(_dev(torch, ie, upd.G))
            ubytes += 5.0 * rows * cols + 5.0 * rows
            meta["params"] += rows * cols
        calls.append(Call("update_all", lambda: ie.ie_sgd_update_multi(ws_, vs_, gs_, wl.LR, wl.MOMENTUM, ws=ws),
                          0.0, ubytes))
    return calls, meta


def build_linear_small(torch, ie, ws):
    inp = wl.linear_small_inputs(seed=1)
    X, W, dY = _dev(torch, ie, inp.X), _dev(torch, ie, inp.W), _dev(torch, ie, inp.dY)
    Y, dX, dW = ie.Mat.empty(64, 128, 0), ie.Mat.empty(64, 256, 0), ie.Mat.empty(128, 256, 1)
    import torch as t
    V = ie.Mat(t.zeros((128, 256), dtype=t.int8, device="cuda"), t.full((128,), -128, dtype=t.int8, device="cuda"), 1)
    ops = 2.0 * 64 * 128 * 256
    io = float(64 * 256 + 128 * 256 + 64 * 128)
    calls = [Call("fwd", lambda: ie.ie_linear_fwd(X, W, Y, ws), ops, io=io, outs=[64 * 128]),
             Call("dx", lambda: ie.ie_linear_bwd_dx(dY, W, dX, ws), ops, io=io, outs=[64 * 256]),
             Call("dw", lambda: ie.ie_linear_bwd_dw(dY, X, dW, ws), ops, io=io, outs=[128 * 256]),
             Call("update", lambda: ie.ie_sgd_update(W, V, dW, wl.LR, wl.MOMENTUM, ws=ws), 0.0,
                  5.0 * 128 * 256 + 3 * 128 + 2)]
    return calls, {"layers": [{"name": "linear", "gemm_mnk": [64, 128, 256]}], "params": 128 * 256}


def build_pointwise(torch, ie, ws, batch):
    """For every ResNet-18 conv output [N*P*Q x K] (per instance): ReLU in
    place, the ReLU mask of an incoming gradient (in place) and the residual
    Sum into a third tensor; whole-tensor groups as in the step.  Algorithmic
    bytes: 2, 3 and 3 per element."""
    calls, meta = [], {"layers": [], "params": 0}
    for i, L in enumerate(wl.resnet18_cifar_layers(batch)):
        M, N, _ = L.gemm_mnk()
        g = torch.Generator(device="cuda").manual_seed(7000 + i)
        def rnd(lo=-127, hi=128):
            return torch.randint(lo, hi, (M, N), dtype=torch.int8, device="cuda", generator=g)
        e = lambda v: torch.tensor([v], dtype=torch.int8, device="cuda")
        Y = ie.Mat(rnd(), e(-6), wl.TENSOR)
        dY = ie.Mat(rnd(), e(-10), wl.TENSOR)
        Rz = ie.Mat(rnd(0, 128), e(-5), wl.TENSOR)
        Z = ie.Mat.empty(M, N, wl.TENSOR)
        n = float(M * N)
        for inst in range(L.count):
            calls.append(Call(f"{L.name}#{inst}:relu", lambda Y=Y: ie.ie_relu_fwd(Y, Y), 0.0, 2 * n))
            calls.append(Call(f"{L.name}#{inst}:relu_bwd", lambda dY=dY, Y=Y: ie.ie_relu_bwd(dY, Y, dY), 0.0, 3 * n))
            calls.append(Call(f"{L.name}#{inst}:add", lambda Y=Y, Rz=Rz, Z=Z: ie.ie_add(Y, Rz, Z, ws), 0.0, 3 * n))
        meta["layers"].append({"name": L.name, "count": L.count, "elements": M * N})
    return calls, meta


def build_vit_attention(torch, ie, ws, batch, heads=12, seq=197, dim=64):
    """ViT-B attention products per (image, head), forward and backward:
    scores Q.K^T, context P.V, dP = dO.V^T, dV = P^T.dO, dQ = dS.K and
    dK = dS^T.Q (softmax and its backward are not products: P and dS are
    synthetic inputs), every result one exponent per row."""
    inp = wl.vit_attention_inputs(batch, heads, seq, dim, 8000)
    Z, S, D = inp.z, seq, dim
    Q, K, V, dO, P, dS = (_dev(torch, ie, c) for c in (inp.Q, inp.K, inp.V, inp.dO, inp.P, inp.dS))
    outs = {n: ie.Mat.empty(Z * S, c, wl.ROW) for n, c in
            (("scores", S), ("context", D), ("dP", S), ("dV", D), ("dQ", D), ("dK", D))}
    ops = 2.0 * Z * S * S * D
    sd, ss = float(Z * S * D), float(Z * S * S)
    # copies: an S x S stack padded to rows of 16 (read S, write S rounded up)
    # and a D-wide stack aligned (read and write D)
    sp = 16 * ((S + 15) // 16)
    pad_ss, pad_sd = ss + float(Z * S * sp), 2 * sd
    calls = [
        Call("scores", lambda: ie.ie_bmm_nt(Z, Q, K, outs["scores"], ws), ops, io=2 * sd + ss, outs=[ss]),
        Call("context", lambda: ie.ie_bmm_nn(Z, P, V, outs["context"], ws), ops, io=ss + 2 * sd, outs=[sd],
             prep=[pad_ss, pad_sd]),
        Call("dP", lambda: ie.ie_bmm_nt(Z, dO, V, outs["dP"], ws), ops, io=2 * sd + ss, outs=[ss]),
        Call("dV", lambda: ie.ie_bmm_tn(Z, P, dO, outs["dV"], ws), ops, io=ss + 2 * sd, outs=[sd],
             prep=[pad_ss, pad_sd]),
        Call("dQ", lambda: ie.ie_bmm_nn(Z, dS, K, outs["dQ"], ws), ops, io=ss + 2 * sd, outs=[sd],
             prep=[pad_ss, pad_sd]),
        Call("dK", lambda: ie.ie_bmm_tn(Z, dS, Q, outs["dK"], ws), ops, io=ss + 2 * sd, outs=[sd],
             prep=[pad_ss, pad_sd]),
    ]
    meta = {"layers": [{"name": "attention", "slices": Z, "seq": S, "head_dim": D}], "params": 0}
    return calls, meta


WORKLOADS = {
    "resnet18": ("resnet18_cifar_conv3x3_batch128", "ResNet-18 3x3 convolutions on 32x32x3 inputs, batch 128"),
    "vitb": ("vit_b_block_linears_128x197_plus_update_85M", "ViT-B block linears (128 x 197 tokens) + update of 84.9M params"),
    "vitti": ("vit_ti_block_linears_256x197", "ViT-Ti block linears (256 x 197 tokens)"),
    "resnet50": ("resnet50_bottleneck_convs_batch128",
                 "ResNet-50 bottleneck convolutions on 224x224x3 inputs, batch 128, + update of their 23.4M weights"),
    "linear_small": ("linear_64x256x128", "single linear layer 64x256 -> 128"),
    "vitb_attn": ("vit_b_attention_products_128x12_heads",
                  "ViT-B attention products per (image, head), forward and backward, batch 128, 12 heads, "
                  "197 tokens, head size 64"),
    "pointwise": ("resnet18_pointwise_batch128",
                  "ReLU forward and backward masks and the residual Sum on the ResNet-18 conv outputs, batch 128"),
}


def build_workload(name, torch, ie, ws):
    if name == "resnet18":
        return build_resnet18(torch, ie, ws, 128)
    if name == "resnet50":
        return build_resnet50(torch, ie, ws, 128)
    if name == "vitb":
        return build_vit(torch, ie, ws, wl.vit_b_linears(128), True)
    if name == "vitti":
        return build_vit(torch, ie, ws, wl.vit_ti_linears(256), False)
    if name == "linear_small":
        return build_linear_small(torch, ie, ws)
    if name == "pointwise":
        return build_pointwise(torch, ie, ws, 128)
    if name == "vitb_attn":
        return build_vit_attention(torch, ie, ws, 128)
    raise SystemExit(f"unknown workload {name}")


# ---------------------------------------------------------------------------
# CPU baseline: the oracle on a bounded sample of the workload
# ---------------------------------------------------------------------------

def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(name: str):
    out = _cpu_baseline(name)
    out["cpu_model"] = cpu_model()
    out["host_cpus"] = len(os.sched_getaffinity(0))
    return out


def _cpu_baseline(name: str):
    import oracle as o
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = 1
    t0 = time.perf_counter()
    ops = 0.0
    if name == "pointwise":
        # the three steps on every layer's output once, at batch 16
        rng = np.random.default_rng(7)
        nbytes = 0.0
        for L in wl.resnet18_cifar_layers(16):
            M, N, _ = L.gemm_mnk()
            Y = o.QT(rng.integers(-127, 128, (M, N)).astype(np.int8), np.array([-6], np.int8), o.TENSOR)
            dY = o.QT(rng.integers(-127, 128, (M, N)).astype(np.int8), np.array([-10], np.int8), o.TENSOR)
            Rz = o.QT(rng.integers(0, 128, (M, N)).astype(np.int8), np.array([-5], np.int8), o.TENSOR)
            Y = o.QT(o.relu_fwd(Y.mant).astype(np.int8), Y.exp, Y.group)
            o.relu_bwd(dY.mant, Y.mant)
            o.sum_op(Y, Rz, o.TENSOR)
            nbytes += 8.0 * M * N
        dt = time.perf_counter() - t0
        return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
                "sample": "ReLU, ReLU mask and Sum on every ResNet-18 conv output once at batch 16",
                "seconds": round(dt, 3)}
    if name == "vitb_attn":
        # the six products on 576 (image, head) slices (48 images)
        inp = wl.vit_attention_inputs(128, 12, 197, 64, 9100, slices=576)
        q = {n: o.QT(c.mant, c.exp, c.group) for n, c in
             (("Q", inp.Q), ("K", inp.K), ("V", inp.V), ("dO", inp.dO), ("P", inp.P), ("dS", inp.dS))}
        t0 = time.perf_counter()
        o.bmm_nt(q["Q"], q["K"], inp.z)
        o.bmm_nn(q["P"], q["V"], inp.z)
        o.bmm_nt(q["dO"], q["V"], inp.z)
        o.bmm_tn(q["P"], q["dO"], inp.z)
        o.bmm_nn(q["dS"], q["K"], inp.z)
        o.bmm_tn(q["dS"], q["Q"], inp.z)
        ops = 6 * 2.0 * inp.z * inp.s * inp.s * inp.d
        sample = "the six attention products on 576 of the 1536 (image, head) slices"
    elif name in ("resnet18", "resnet50"):
        batch = 128
        layers = wl.resnet18_cifar_layers(batch) if name == "resnet18" else wl.resnet50_layers(2)
        sample = (f"every layer once at batch {batch if name == 'resnet18' else 2} "
                  f"(fwd, input and weight gradients, update)")
        for i, L in enumerate(layers):
            inp = (wl.resnet18_conv_inputs if name == "resnet18" else wl.resnet50_conv_inputs)(L, 9000 + i)
            d = o.ConvShape(L.n, L.h, L.w, L.c, L.k, L.r, L.s, L.stride, L.pad)
            X = o.QT(inp.X.mant, inp.X.exp, inp.X.group)
            W = o.QT(inp.W.mant, inp.W.exp, inp.W.group)
            dY = o.QT(inp.dY.mant, inp.dY.exp, inp.dY.group)
            M, N, K = L.gemm_mnk()
            o.conv_fwd(d, X, W, o.TENSOR)
            if not L.first:
                o.conv_dgrad(d, dY, W, o.TENSOR)
            dW = o.conv_wgrad(d, dY, X, o.ROW)
            upd = wl.update_inputs(N, K, 9500 + i, w_group=W.group)
            o.sgd_update(W, o.QT(upd.V.mant, upd.V.exp, upd.V.group), dW, o.Scalar(*wl.LR), o.Scalar(*wl.MOMENTUM))
            ops += 2.0 * M * N * K * (2 if L.first else 3)
    else:
        layers = (wl.vit_b_linears(128) if name == "vitb" else wl.vit_ti_linears(256)) \
            if name in ("vitb", "vitti") else [wl.LinearLayer("linear", 64, 128, 256)]
        rows = 1024 if name in ("vitb", "vitti") else 64
        sample = f"every linear at {rows} tokens (fwd, dX, dW)"
        for i, L in enumerate(layers):
            inp = wl.vit_linear_inputs(L, 9000 + i, m_rows=rows)
            X = o.QT(inp.X.mant, inp.X.exp, inp.X.group)
            W = o.QT(inp.W.mant, inp.W.exp, inp.W.group)
            dY = o.QT(inp.dY.mant, inp.dY.exp, inp.dY.group)
            o.linear_fwd(X, W, o.ROW)
            o.linear_bwd_dx(dY, W, o.ROW)
            o.linear_bwd_dw(dY, X, o.ROW)
            ops += 3 * 2.0 * rows * L.n * L.k
    dt = time.perf_counter() - t0
    return {"value": ops / dt / 1e12, "unit": "TOPS", "cores": threads, "kind": "oracle",
            "sample": sample, "seconds": round(dt, 3), "sample_gop": round(ops / 1e9, 3)}


# ---------------------------------------------------------------------------
# HBM traffic of the dominant kernel from the committed counter table
# ---------------------------------------------------------------------------

def measured_traffic(workload: str, kernel: str) -> dict:
    """HBM bytes per launch of `kernel` from profiles/hbm_traffic_<workload>.txt
    (two rocprofv3 --pmc runs, copy-calibrated); null when there is no table,
    the kernel is missing from it or the library sources changed since."""
    from integer_only_dnn_amd import prof_summary
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.txt")
    out = {"traffic": None}
    if not os.path.exists(path):
        out["traffic_note"] = "no counter table"
        return out
    digest, table = prof_summary.read_traffic(path)
    if digest != prof_summary.source_digest():
        out["traffic_note"] = "kernels changed since the counters were taken"
        return out
    if kernel not in table:
        out["traffic_note"] = "kernel not in the counter table"
        return out
    fetch, write = table[kernel]
    out["traffic"] = round(fetch + write)
    out["traffic_fetch"] = round(fetch)
    out["traffic_write"] = round(write)
    return out


# ---------------------------------------------------------------------------
# Main
# ---------------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="resnet50", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kernels", action="store_true", help="also print the per-kernel breakdown")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="first run one plain device copy of MIB MiB (scale for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    from integer_only_dnn_amd import ie
    ie.lib()
    torch.cuda.set_device(0)
    ws = ie.Workspace("cuda")
    if args.copy_calibration:
        src = torch.ones(args.copy_calibration << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    wl_id, wl_desc = WORKLOADS[args.workload]
    calls, meta = build_workload(args.workload, torch, ie, ws)
    torch.cuda.synchronize()

    # Calibration step (untimed): learn each call's kernel sequence.
    ie.ie_profile_select(0)
    ie.ie_profile_enable(True)
    for c in calls:
        c.fn()
        torch.cuda.synchronize()
        c.kinds = [k for _, k in ie.ie_profile_read()]
    ie.ie_profile_enable(False)
    for _ in range(args.warmup):
        for c in calls:
            c.fn()
    torch.cuda.synchronize()
    if ws.status() != 0:
        raise SystemExit("exponent range flag raised during warmup")

    def attribute(recs, n_steps, only=None):
        """Per-kind totals of event records taken over n_steps steps (all
        kernels, or only kernels of kind `only`), in launch order."""
        agg, pos = {}, 0
        for _ in range(n_steps):
            for c in calls:
                n_gemm = sum(1 for k in c.kinds if is_gemm(k))
                n_upd = sum(1 for k in c.kinds if 2000 <= k < 3000)
                n_pw = sum(1 for k in c.kinds if 3500 <= k < 3600)
                prod = -1  # index of the last contraction launched
                fin = 0    # index of the contraction the next finalize belongs to
                npre = 0   # padding / alignment copies of this call so far
                for k in c.kinds:
                    if is_gemm(k):
                        prod += 2 if is_pair(k) else 1
                        fin = prod - 1 if is_pair(k) else prod
                    pre = -1
                    if k in (3200, 3210):
                        pre, npre = npre, npre + 1
                    if only is not None and k != only:
                        continue
                    ms, kind = recs[pos]
                    assert kind == k, (kind, k)
                    pos += 1
                    a = agg.setdefault(kind, {"ms": 0.0, "launches": 0, "ops": 0.0, "bytes": 0.0})
                    a["ms"] += ms
                    a["launches"] += 1
                    if is_gemm(kind):
                        a["ops"] += c.ops / n_gemm
                        if is_pair(kind):
                            a["bytes"] += c.pair_io
                        elif c.ios:
                            a["bytes"] += c.ios[min(max(prod, 0), len(c.ios) - 1)]
                        else:
                            a["bytes"] += c.io
                    elif 2000 <= kind < 3000 and c.bytes:
                        a["bytes"] += c.bytes / n_upd
                    elif 3500 <= kind < 3600:
                        # pointwise step: the call's algorithmic bytes over its launches
                        a["bytes"] += c.bytes / n_pw
                    elif pre >= 0 and c.prep:
                        # a padding / alignment copy with its own byte count
                        a["bytes"] += c.prep[min(pre, len(c.prep) - 1)]
                    elif kind == 3400:
                        # both finalizes of a convolution's backward pass
                        a["bytes"] += sum(c.outs)
                    elif c.outs:
                        # finalize or pre-pass of a contraction: its int8 result
                        a["bytes"] += c.outs[min(max(fin, 0), len(c.outs) - 1)]
                        if prod >= 0:
                            fin = min(fin + 1, prod)
        assert pos == len(recs), (pos, len(recs))
        return agg

    # Breakdown pass (untimed): every kernel bracketed by events; picks the
    # kernel with the largest share of the step.
    n_bd = max(2, min(args.steps, 5))
    ie.ie_profile_enable(True)
    for _ in range(n_bd):
        for c in calls:
            c.fn()
    torch.cuda.synchronize()
    breakdown = attribute(ie.ie_profile_read(), n_bd)
    ie.ie_profile_enable(False)
    dom = max(breakdown, key=lambda k: breakdown[k]["ms"])

    # Timed region: K steps with no instrumentation (the step time); then the
    # same K steps again with HIP events bracketing the launches of the
    # dominant kernel only, on the stream they are launched on (its average
    # launch time; recording the events costs host time between launches,
    # so that pass is not the step time).  The collector stays off while
    # steps are issued: a full collection between two launches would leave
    # the GPU idle.
    def timed(instrumented):
        if instrumented:
            ie.ie_profile_select(dom)
            ie.ie_profile_enable(True)
        gc.collect()
        gc.disable()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            for c in calls:
                c.fn()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        gc.enable()
        return (t1 - t0) * 1e3 / args.steps

    ms_per_step = timed(False)
    ms_instrumented = timed(True)
    A = attribute(ie.ie_profile_read(), args.steps, only=dom)[dom]
    ie.ie_profile_enable(False)
    ie.ie_profile_select(0)
    if ws.status() != 0:
        raise SystemExit("exponent range flag raised in the timed region")

    step_ops = sum(c.ops for c in calls)
    value = step_ops / (ms_per_step * 1e-3) / 1e12
    unit = "TOPS"
    if step_ops == 0:
        # a pointwise workload: algorithmic bytes per second
        value = sum(c.bytes for c in calls) / (ms_per_step * 1e-3) / 1e9
        unit = "GB/s"
    roof = roofline(A["ops"] if is_gemm(dom) else 0.0, A["bytes"], A["ms"])
    roof["kernel"] = kind_symbol(dom)
    roof["avg_launch_us"] = round(A["ms"] * 1e3 / A["launches"], 2)
    roof["launches_per_step"] = A["launches"] // args.steps
    roof["algorithmic_bytes_per_launch"] = round(A["bytes"] / A["launches"])
    roof.update(measured_traffic(args.workload, roof["kernel"]))
    agg = breakdown
    upd_ms = sum(v["ms"] for k, v in agg.items() if 2000 <= k < 3000) / n_bd
    upd_bytes = sum(c.bytes for c in calls if any(2000 <= k < 3000 for k in c.kinds))
    gemm_ms = sum(v["ms"] for k, v in agg.items() if is_gemm(k)) / n_bd
    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "ms_per_step_with_kernel_events": round(ms_instrumented, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": wl_id, "description": wl_desc, "step_gop": round(step_ops / 1e9, 3),
                   "params_updated": meta["params"]},
        "frac_int8_peak": round(value / PEAK_INT8_TOPS, 4) if step_ops else None,
        "frac_hbm": round(value / PEAK_HBM_GBS, 4) if not step_ops else None,
        "contraction_tops": round(step_ops / (gemm_ms * 1e-3) / 1e12, 2) if gemm_ms else None,
        "update": ({"gbps": round(upd_bytes / (upd_ms * 1e-3) / 1e9, 1),
                    "frac_hbm": round(upd_bytes / (upd_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                    "ms_per_step": round(upd_ms, 4), "algorithmic_bytes": upd_bytes} if upd_ms else None),
        "roofline": roof,
    }
    if args.kernels:
        out["kernels"] = {kind_name(k): {"ms_per_step": round(v["ms"] / n_bd, 4),
                                         "launches_per_step": v["launches"] // n_bd,
                                         "avg_us": round(v["ms"] * 1e3 / v["launches"], 2)}
                          for k, v in sorted(agg.items())}
    out["cpu_baseline"] = None if args.no_cpu_baseline else cpu_baseline(args.workload)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
