"""Seeded synthetic inputs for the binary linear / conv2d forward workloads.

This module only draws numbers: it holds none of the method's arithmetic (no
sign, no packing, no dot products). Both the CPU oracle and the GPU path take
their inputs from here, so the two sides always see identical bits.

Recipe, per workload: a CPU ``torch.Generator`` seeded with the workload's seed
draws, in this order and in float32, the activation ``x = mu + randn(shape)``,
the weight ``W = randn(shape)``, then ``scale_a`` and ``scale_w``; afterwards
``x`` and ``W`` are cast to their stated dtypes (the casts are exact for the
representable values and round-to-nearest-even otherwise). Scales drawn from
U(0.01, 1) are ``0.01 + 0.99 * rand()`` in float32, widened to a Python float.

Workload shapes are those of the binarized layers the pages describe
(bitorch-engine's BinaryLinearCuda / BinaryConv2dCutlass forward), sized as
an LLM-shaped linear layer, a ResNet-18 stage-3 3x3 conv, a strided and a
dilated 3x3 conv, and a large linear layer with on-the-fly activation packing.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional, Tuple

import torch

__all__ = ["Workload", "WORKLOADS", "make_inputs", "make_grad", "conv_out_size", "edge_values",
           "random_linear_case", "random_conv_case", "make_shift"]

_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str                      # "linear" | "conv"
    x_dtype: str
    w_dtype: str
    out_dtype: str
    seed: int
    # linear: x [m, k], W [n, k]
    m: int = 0
    n: int = 0
    k: int = 0
    # conv: x [batch, c, h, w] NCHW, W [o, c, ks, ks] OIHW
    batch: int = 0
    c: int = 0
    h: int = 0
    w: int = 0
    o: int = 0
    ks: int = 0
    stride: int = 1
    padding: int = 0
    dilation: int = 1
    mu: float = 0.0
    fixed_scales: Optional[Tuple[float, float]] = None
    note: str = field(default="", compare=False)

    def x_shape(self):
        return (self.m, self.k) if self.kind == "linear" else (self.batch, self.c, self.h, self.w)

    def w_shape(self):
        return (self.n, self.k) if self.kind == "linear" else (self.o, self.c, self.ks, self.ks)

    def out_shape(self):
        if self.kind == "linear":
            return (self.m, self.n)
        ho = conv_out_size(self.h, self.ks, self.stride, self.padding, self.dilation)
        wo = conv_out_size(self.w, self.ks, self.stride, self.padding, self.dilation)
        return (self.batch, self.o, ho, wo)

    def gemm_mnk(self):
        """(M, N, K) of the contraction: for conv M = batch*Ho*Wo, N = o, K = c*ks*ks."""
        if self.kind == "linear":
            return self.m, self.n, self.k
        b, o, ho, wo = self.out_shape()
        return b * ho * wo, o, self.c * self.ks * self.ks

    def binary_ops(self):
        m, n, k = self.gemm_mnk()
        return 2 * m * n * k


def conv_out_size(size: int, ks: int, stride: int, padding: int, dilation: int) -> int:
    """Output extent of a conv along one axis, floor((size + 2p - d(ks-1) - 1)/s + 1)."""
    return math.floor((size + 2 * padding - dilation * (ks - 1) - 1) / stride + 1)


WORKLOADS = {
    "linear_64x256x512_f32": Workload(
        "linear_64x256x512_f32", "linear", "f32", "f32", "f32", seed=1001,
        m=64, n=256, k=512, fixed_scales=(0.5, 0.25),
        note="small binary linear forward"),
    "linear_2048x4096x4096_f16": Workload(
        "linear_2048x4096x4096_f16", "linear", "f16", "f16", "f16", seed=1002,
        m=2048, n=4096, k=4096, note="LLM-shaped binary linear forward, W pre-packed"),
    "conv_resnet18_s3_f32": Workload(
        "conv_resnet18_s3_f32", "conv", "f32", "f32", "f32", seed=1003,
        batch=32, c=256, h=14, w=14, o=256, ks=3, stride=1, padding=1, dilation=1,
        note="ResNet-18 stage-3 3x3 conv shape"),
    "conv_down_s2_f16": Workload(
        "conv_down_s2_f16", "conv", "f16", "f16", "f16", seed=1004,
        batch=128, c=128, h=28, w=28, o=256, ks=3, stride=2, padding=1, dilation=1, mu=0.1,
        note="downsampling 3x3 conv, stride 2"),
    "conv_dil2_f16": Workload(
        "conv_dil2_f16", "conv", "f16", "f16", "f16", seed=1004,
        batch=128, c=128, h=28, w=28, o=256, ks=3, stride=1, padding=2, dilation=2, mu=0.1,
        note="dilated 3x3 conv, dilation 2"),
    "linear_16384x8192x8192_bf16": Workload(
        "linear_16384x8192x8192_bf16", "linear", "bf16", "f32", "f32", seed=1005,
        m=16384, n=8192, k=8192, note="large binary linear, activations packed on the fly"),
}


def _draw_scale(g: torch.Generator) -> float:
    return float(0.01 + 0.99 * torch.rand((), generator=g, dtype=torch.float32))


def make_inputs(wl: Workload, draw_weight: bool = True):
    """Draw (x, W, scale_a, scale_w) for a workload on the CPU.

    ``x`` and ``W`` are contiguous CPU tensors in the workload's dtypes; the
    scales are Python floats. ``draw_weight=False`` still consumes the same
    random stream for W (so scales are unchanged) but returns ``None`` for it.
    """
    g = torch.Generator("cpu").manual_seed(wl.seed)
    x = torch.randn(wl.x_shape(), generator=g, dtype=torch.float32)
    if wl.mu:
        x += wl.mu
    w = torch.randn(wl.w_shape(), generator=g, dtype=torch.float32)
    sa = _draw_scale(g)
    sw = _draw_scale(g)
    if wl.fixed_scales is not None:
        sa, sw = wl.fixed_scales
    x = x.to(_DT[wl.x_dtype]).contiguous()
    w = w.to(_DT[wl.w_dtype]).contiguous() if draw_weight else None
    return x, w, sa, sw


def edge_values(dtype: str):
    """IEEE special values for the dtype, as a tensor: +0, -0, NaN, +inf, -inf,
    +smallest subnormal, -smallest subnormal, +largest finite, -largest finite."""
    dt = _DT[dtype]
    bits = {
        "f32": [0x00000000, 0x80000000, 0x7FC00000, 0x7F800000, 0xFF800000,
                0x00000001, 0x80000001, 0x7F7FFFFF, 0xFF7FFFFF, 0xFFC00000, 0x7F800001],
        "f16": [0x0000, 0x8000, 0x7E00, 0x7C00, 0xFC00, 0x0001, 0x8001, 0x7BFF, 0xFBFF,
                0xFE00, 0x7C01],
        "bf16": [0x0000, 0x8000, 0x7FC0, 0x7F80, 0xFF80, 0x0001, 0x8001, 0x7F7F, 0xFF7F,
                 0xFFC0, 0x7F81],
    }[dtype]
    if dtype == "f32":
        t = torch.tensor([b - (1 << 32) if b >= (1 << 31) else b for b in bits], dtype=torch.int32)
        return t.view(torch.float32)
    t = torch.tensor([b - (1 << 16) if b >= (1 << 15) else b for b in bits], dtype=torch.int16)
    return t.view(dt)


def inject_edges(x: torch.Tensor, seed: int, count: int) -> torch.Tensor:
    """Overwrite ``count`` seeded positions of a copy of ``x`` with the dtype's special values."""
    name = {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16"}[x.dtype]
    ev = edge_values(name)
    g = torch.Generator("cpu").manual_seed(seed)
    flat = x.clone().reshape(-1)
    pos = torch.randint(0, flat.numel(), (count,), generator=g)
    pick = torch.randint(0, ev.numel(), (count,), generator=g)
    flat[pos] = ev[pick]
    return flat.reshape(x.shape)


def random_linear_case(seed: int, max_m=97, max_n=97, max_kw=24, dtype=None):
    """A small random linear case with ragged M, N and K a multiple of 32."""
    g = torch.Generator("cpu").manual_seed(seed)
    m = int(torch.randint(1, max_m + 1, (), generator=g))
    n = int(torch.randint(1, max_n + 1, (), generator=g))
    k = 32 * int(torch.randint(1, max_kw + 1, (), generator=g))
    dts = ["f32", "f16", "bf16"]
    xd = dtype or dts[int(torch.randint(0, 3, (), generator=g))]
    wd = dts[int(torch.randint(0, 3, (), generator=g))]
    od = dts[int(torch.randint(0, 3, (), generator=g))]
    x = torch.randn((m, k), generator=g).to(_DT[xd])
    w = torch.randn((n, k), generator=g).to(_DT[wd])
    sa, sw = _draw_scale(g), _draw_scale(g)
    return dict(m=m, n=n, k=k, x=x, w=w, scale_a=sa, scale_w=sw, out_dtype=od)


def random_conv_case(seed: int):
    """A small random conv case: ragged spatial sizes, k in {1,2,3,5}, s in {1,2,3},
    p in {0..3}, d in {1,2,3}, C a multiple of 32. Re-draws until the output is non-empty."""
    g = torch.Generator("cpu").manual_seed(seed)

    def ri(lo, hi):
        return int(torch.randint(lo, hi + 1, (), generator=g))

    while True:
        b, c, h, w, o = ri(1, 3), 32 * ri(1, 4), ri(1, 17), ri(1, 17), ri(1, 70)
        ks, s, p, d = [1, 2, 3, 5][ri(0, 3)], ri(1, 3), ri(0, 3), ri(1, 3)
        ho = conv_out_size(h, ks, s, p, d)
        wo = conv_out_size(w, ks, s, p, d)
        if ho > 0 and wo > 0:
            break
    dts = ["f32", "f16", "bf16"]
    xd = dts[ri(0, 2)]
    wd = dts[ri(0, 2)]
    od = dts[ri(0, 2)]
    x = torch.randn((b, c, h, w), generator=g).to(_DT[xd])
    wt = torch.randn((o, c, ks, ks), generator=g).to(_DT[wd])
    sa, sw = _draw_scale(g), _draw_scale(g)
    return dict(batch=b, c=c, h=h, w=w, o=o, ks=ks, stride=s, padding=p, dilation=d,
                x=x, w_=wt, scale_a=sa, scale_w=sw, out_dtype=od)


def make_shift(n: int, dtype: str, seed: int, axis_values=None) -> torch.Tensor:
    """A learnable-shift vector of ``n`` values for the activation prologue, in ``dtype``.

    Recipe: a CPU generator seeded with ``seed`` draws ``0.5 * randn(n)`` in float32. Then every
    seventh entry is set to the negation of an input value of its own column or channel
    (``axis_values(i)`` returns one such input as a float, or None to skip), so that the sum
    x + bias is exactly zero there for some element; every eleventh entry takes one of the dtype's
    special values (signed zeros, NaN, infinities, subnormals, extremes). The result is cast to
    ``dtype`` (a cancellation survives the cast only when the input value is representable in it).
    """
    g = torch.Generator("cpu").manual_seed(seed)
    b = 0.5 * torch.randn(n, generator=g, dtype=torch.float32)
    if axis_values is not None:
        for i in range(0, n, 7):
            v = axis_values(i)
            if v is not None:
                b[i] = -v
    b = b.to(_DT[dtype])
    ev = edge_values(dtype)
    for j, i in enumerate(range(3, n, 11)):
        b[i] = ev[j % ev.numel()]
    return b.contiguous()


def make_grad(m: int, n: int, dtype: str, seed: int) -> torch.Tensor:
    """An output gradient [m, n] for the straight-through backward: ``randn`` in float32 from a
    CPU generator seeded with ``seed``, cast to ``dtype``."""
    g = torch.Generator("cpu").manual_seed(seed)
    return torch.randn((m, n), generator=g, dtype=torch.float32).to(_DT[dtype]).contiguous()
