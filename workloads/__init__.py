"""Seeded synthetic (C, e) inputs for the integer layer step.

This module only draws numbers and shapes; it holds none of the method's
arithmetic (no products, no requantisation, no update).  Both the oracle-side
tests and the GPU-side tests and benchmark take their inputs from here.

The page trains on CIFAR-10/100 and ImageNet ("Memory-Efficient Integer-Only
Training of Deep Neural Networks", Abstract, Tables 3-5, 9-10); none of those
datasets is used.  Instead every tensor is drawn from a seeded normal
distribution with the shapes of the page's models (ResNet-18 on 32x32 inputs,
ResNet-50 on 224x224 inputs, ViT-Ti and ViT-B with 197 tokens):

* ``clip_code(z, a)``: mantissa = clip(rint(a * z), -127, 127) with a fixed
  exponent.
* ``max127_code(z)``: per group, mantissa = rint(127 * z / max|z|) (so the
  largest |C| is 127) and exponent = ceil(log2(max|z|)) - 7.

``rint`` is numpy's round-half-to-even on float64; these floats exist only to
make synthetic integer data.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

TENSOR = 0
ROW = 1


@dataclass
class Code:
    """Synthetic (C, e) data: int8 mantissas, int8 exponents and group kind."""
    mant: np.ndarray
    exp: np.ndarray
    group: int


def clip_code(z: np.ndarray, scale: float, exp: int) -> Code:
    c = np.clip(np.rint(scale * z), -127, 127).astype(np.int8)
    return Code(c, np.array([exp], dtype=np.int8), TENSOR)


def max127_code(z: np.ndarray, group: int) -> Code:
    """Max-127 rule per row (ROW) or over the whole array (TENSOR)."""
    rows = z.shape[0]
    flat = z.reshape(rows, -1)
    if group == ROW:
        mx = np.abs(flat).max(axis=1)
        mx = np.where(mx == 0, 1.0, mx)
        c = np.rint(127.0 * flat / mx[:, None])
        e = np.ceil(np.log2(mx)) - 7
    else:
        mx = float(np.abs(flat).max()) or 1.0
        c = np.rint(127.0 * flat / mx)
        e = np.array([np.ceil(np.log2(mx)) - 7])
    return Code(c.astype(np.int8).reshape(z.shape), e.astype(np.int8), group)


def uniform_exps(rng: np.random.Generator, n: int, lo: int, hi: int) -> np.ndarray:
    """n exponents drawn uniformly from the integers lo..hi inclusive."""
    return rng.integers(lo, hi + 1, size=n).astype(np.int8)


# ---------------------------------------------------------------------------
# Layer shapes
# ---------------------------------------------------------------------------

@dataclass
class ConvLayer:
    name: str
    n: int
    h: int
    w: int
    c: int
    k: int
    r: int
    s: int
    stride: int
    pad: int
    count: int = 1
    first: bool = False          # the network's first layer has no input gradient

    @property
    def p(self) -> int:
        return (self.h + 2 * self.pad - self.r) // self.stride + 1

    @property
    def q(self) -> int:
        return (self.w + 2 * self.pad - self.s) // self.stride + 1

    def gemm_mnk(self):
        """(M, N, K) of the forward implicit GEMM."""
        return self.n * self.p * self.q, self.k, self.r * self.s * self.c


@dataclass
class LinearLayer:
    name: str
    m: int
    n: int
    k: int
    count: int = 1


def resnet18_cifar_layers(batch: int = 128):
    """3x3 pad-1 convolutions of a ResNet-18 on 32x32x3 inputs (NHWC)."""
    L = []
    L.append(ConvLayer("stem_3_64@32", batch, 32, 32, 3, 64, 3, 3, 1, 1, 1, first=True))
    L.append(ConvLayer("conv_64_64@32", batch, 32, 32, 64, 64, 3, 3, 1, 1, 4))
    L.append(ConvLayer("conv_64_128_s2@32", batch, 32, 32, 64, 128, 3, 3, 2, 1, 1))
    L.append(ConvLayer("conv_128_128@16", batch, 16, 16, 128, 128, 3, 3, 1, 1, 3))
    L.append(ConvLayer("conv_128_256_s2@16", batch, 16, 16, 128, 256, 3, 3, 2, 1, 1))
    L.append(ConvLayer("conv_256_256@8", batch, 8, 8, 256, 256, 3, 3, 1, 1, 3))
    L.append(ConvLayer("conv_256_512_s2@8", batch, 8, 8, 256, 512, 3, 3, 2, 1, 1))
    L.append(ConvLayer("conv_512_512@4", batch, 4, 4, 512, 512, 3, 3, 1, 1, 3))
    return L


def resnet50_layers(batch: int = 128):
    """ResNet-50 (v1.5) bottleneck convolutions on 224x224x3 inputs: 1x1/3x3/1x1
    with projection shortcuts, stride on the 3x3, NHWC."""
    def c1(name, hw, cin, cout, count, stride=1):
        return ConvLayer(name, batch, hw, hw, cin, cout, 1, 1, stride, 0, count)

    def c3(name, hw, ch, count, stride=1):
        return ConvLayer(name, batch, hw, hw, ch, ch, 3, 3, stride, 1, count)

    return [
        c1("s1_1x1_64_64@56", 56, 64, 64, 1),
        c1("s1_1x1_256_64@56", 56, 256, 64, 2),
        c3("s1_3x3_64@56", 56, 64, 3),
        c1("s1_1x1_64_256@56", 56, 64, 256, 3),
        c1("s1_sc_64_256@56", 56, 64, 256, 1),
        c1("s2_1x1_256_128@56", 56, 256, 128, 1),
        c3("s2_3x3_128_s2@56", 56, 128, 1, 2),
        c1("s2_1x1_512_128@28", 28, 512, 128, 3),
        c3("s2_3x3_128@28", 28, 128, 3),
        c1("s2_1x1_128_512@28", 28, 128, 512, 4),
        c1("s2_sc_256_512_s2@56", 56, 256, 512, 1, 2),
        c1("s3_1x1_512_256@28", 28, 512, 256, 1),
        c3("s3_3x3_256_s2@28", 28, 256, 1, 2),
        c1("s3_1x1_1024_256@14", 14, 1024, 256, 5),
        c3("s3_3x3_256@14", 14, 256, 5),
        c1("s3_1x1_256_1024@14", 14, 256, 1024, 6),
        c1("s3_sc_512_1024_s2@28", 28, 512, 1024, 1, 2),
        c1("s4_1x1_1024_512@14", 14, 1024, 512, 1),
        c3("s4_3x3_512_s2@14", 14, 512, 1, 2),
        c1("s4_1x1_2048_512@7", 7, 2048, 512, 2),
        c3("s4_3x3_512@7", 7, 512, 2),
        c1("s4_1x1_512_2048@7", 7, 512, 2048, 3),
        c1("s4_sc_1024_2048_s2@14", 14, 1024, 2048, 1, 2),
    ]


def vit_block_linears(batch: int, tokens: int, hidden: int, mlp: int):
    m = batch * tokens
    return [
        LinearLayer("qkv", m, 3 * hidden, hidden),
        LinearLayer("proj", m, hidden, hidden),
        LinearLayer("fc1", m, mlp, hidden),
        LinearLayer("fc2", m, hidden, mlp),
    ]


def vit_ti_linears(batch: int = 256):
    return vit_block_linears(batch, 197, 192, 768)


def vit_b_linears(batch: int = 128):
    return vit_block_linears(batch, 197, 768, 3072)


VIT_B_BLOCKS = 12


def vit_b_param_arenas():
    """ViT-B's 48 block weight matrices stacked by row width: [(rows, cols)].

    Per block qkv [2304 x 768], proj [768 x 768], fc1 [3072 x 768] share width
    768; fc2 [768 x 3072] has width 3072.  12 blocks: 84 934 656 parameters in
    82 944 output-channel groups.
    """
    return [((2304 + 768 + 3072) * VIT_B_BLOCKS, 768), (768 * VIT_B_BLOCKS, 3072)]


# ---------------------------------------------------------------------------
# Input recipes per workload (draw order is part of the recipe)
# ---------------------------------------------------------------------------

@dataclass
class LinearInputs:
    X: Code
    W: Code
    dY: Code
    y_group: int
    dx_group: int
    dw_group: int


def linear_small_inputs(seed: int = 1) -> LinearInputs:
    """Single linear layer X [64x256], W [128x256], dY [64x128]; mantissas
    clip(rint(40 z)), per-tensor exponents X -6, W -8, dY -10."""
    rng = np.random.default_rng(seed)
    X = clip_code(rng.standard_normal((64, 256)), 40.0, -6)
    W = clip_code(rng.standard_normal((128, 256)), 40.0, -8)
    dY = clip_code(rng.standard_normal((64, 128)), 40.0, -10)
    return LinearInputs(X, W, dY, TENSOR, TENSOR, ROW)


def vit_linear_inputs(layer: LinearLayer, seed: int, m_rows: int = None) -> LinearInputs:
    """Per-row (token) activation groups and per-output-channel weight groups,
    mantissas by the max-127 rule on N(0,1) (weights scaled by K**-0.5)."""
    rng = np.random.default_rng(seed)
    m = layer.m if m_rows is None else m_rows
    X = max127_code(rng.standard_normal((m, layer.k)), ROW)
    W = max127_code(rng.standard_normal((layer.n, layer.k)) * layer.k ** -0.5, ROW)
    dY = max127_code(rng.standard_normal((m, layer.n)), ROW)
    return LinearInputs(X, W, dY, ROW, ROW, ROW)


@dataclass
class ConvInputs:
    X: Code
    W: Code
    dY: Code


def resnet18_conv_inputs(layer: ConvLayer, seed: int) -> ConvInputs:
    """X: max-127 rule on relu(z) (about half zeros); W: max-127 rule on
    z * sqrt(2 / (R*S*C)) (He scale); dY: clip(rint(40 z)) at exponent -10.
    All per-tensor; W is [K x R*S*C]."""
    rng = np.random.default_rng(seed)
    x = np.maximum(rng.standard_normal((layer.n, layer.h, layer.w, layer.c)), 0.0)
    X = max127_code(x.reshape(1, -1), TENSOR)
    X = Code(X.mant.reshape(x.shape), X.exp, TENSOR)
    fan_in = layer.r * layer.s * layer.c
    W = max127_code((rng.standard_normal((layer.k, fan_in)) * np.sqrt(2.0 / fan_in)).reshape(1, -1), TENSOR)
    W = Code(W.mant.reshape(layer.k, fan_in), W.exp, TENSOR)
    dY = clip_code(rng.standard_normal((layer.n, layer.p, layer.q, layer.k)), 40.0, -10)
    return ConvInputs(X, W, dY)


def resnet50_conv_inputs(layer: ConvLayer, seed: int) -> ConvInputs:
    """clip(rint(30 z)) mantissas; X and dY per-tensor exponents and W
    per-output-channel exponents drawn uniformly from -12..-4."""
    rng = np.random.default_rng(seed)
    fan_in = layer.r * layer.s * layer.c
    X = clip_code(rng.standard_normal((layer.n, layer.h, layer.w, layer.c)), 30.0, 0)
    X.exp = uniform_exps(rng, 1, -12, -4)
    W = clip_code(rng.standard_normal((layer.k, fan_in)), 30.0, 0)
    W = Code(W.mant, uniform_exps(rng, layer.k, -12, -4), ROW)
    dY = clip_code(rng.standard_normal((layer.n, layer.p, layer.q, layer.k)), 30.0, 0)
    dY.exp = uniform_exps(rng, 1, -12, -4)
    return ConvInputs(X, W, dY)


@dataclass
class UpdateInputs:
    W: Code
    V: Code
    G: Code


def update_inputs(rows: int, cols: int, seed: int, w_group: int = ROW,
                  fan_in: int = None) -> UpdateInputs:
    """Weights by the max-127 rule on z * fan_in**-0.5 (per output channel or
    per tensor); velocity and gradient mantissas by the max-127 rule per
    output channel with exponents drawn uniformly from -16..-6."""
    rng = np.random.default_rng(seed)
    fan_in = cols if fan_in is None else fan_in
    W = max127_code(rng.standard_normal((rows, cols)) * fan_in ** -0.5, w_group)
    V = max127_code(rng.standard_normal((rows, cols)), ROW)
    V.exp = uniform_exps(rng, rows, -16, -6)
    G = max127_code(rng.standard_normal((rows, cols)), ROW)
    G.exp = uniform_exps(rng, rows, -16, -6)
    return UpdateInputs(W, V, G)


# Learning rate 2**-7 and momentum 7/8 as (C, e) scalars.
LR = (1, -7)
MOMENTUM = (7, -3)


# ---------------------------------------------------------------------------
# ViT attention products per (image, head): stacks of slices
# ---------------------------------------------------------------------------

@dataclass
class AttentionInputs:
    """Stacked per-(image, head) operands: Q, K, V, dO [Z*S x D] and P, dS
    [Z*S x S], every row its own group (one exponent per token and head)."""
    z: int
    s: int
    d: int
    Q: Code
    K: Code
    V: Code
    dO: Code
    P: Code
    dS: Code


def vit_attention_inputs(batch: int, heads: int, seq: int, dim: int, seed: int,
                         slices: int = None) -> AttentionInputs:
    """Q, K, V, dO and dS from normal draws; P as attention probabilities
    (every row the softmax of normal logits: non-negative, summing to one).
    `slices` draws only the first that many (image, head) slices."""
    rng = np.random.default_rng(seed)
    z = batch * heads if slices is None else slices
    f = np.float32

    def normal(rows, cols):
        return rng.standard_normal((rows, cols), dtype=f)

    q, k, v, do = (max127_code(normal(z * seq, dim), ROW) for _ in range(4))
    logits = normal(z * seq, seq)
    p = np.exp(logits - logits.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    P = max127_code(p, ROW)
    dS = max127_code(normal(z * seq, seq), ROW)
    return AttentionInputs(z, seq, dim, q, k, v, do, P, dS)
