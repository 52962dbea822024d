"""Seeded synthetic inputs for the forward-convolution workloads.

This module holds shapes, dtypes, seeds and value distributions only. It
contains no convolution arithmetic: the CPU oracle (``oracle/``) and the HIP
library (``convolution_forward_amd``) each compute outputs their own way. Both
sides draw their inputs here, so they see identical bits.

Values are drawn on the CPU with ``torch.Generator().manual_seed(seed)``, the
input tensor first and the filter second. ``uniform`` is ``rand * 2 - 1``
(values in [-1, 1)); ``normal`` is ``randn * std`` with ``std`` the standard
deviation. bf16 tensors are the fp32 draws rounded to nearest-even; the fp32
run of a bf16 workload uses the same draws without rounding.

The depthwise sweep takes only its layer shapes from the MobileNetV3-large
depthwise table of the "Depthwise convolution" page (section "Measured"); the
values are synthetic, not activations or trained weights.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch


@dataclass(frozen=True)
class DenseWorkload:
    """NHWC input [N,H,W,Cin], KKIO filter [KH,KW,Cin,Cout], stride 1, no padding."""
    name: str
    N: int
    H: int
    W: int
    Cin: int
    KH: int
    KW: int
    Cout: int
    dtype: str              # "f32" or "bf16": the dtype of X and F
    x_dist: str             # "uniform" or "normal"
    f_std: float | None     # std of F for "normal"; None means F is uniform too
    seed: int

    @property
    def x_shape(self):
        return (self.N, self.H, self.W, self.Cin)

    @property
    def f_shape(self):
        return (self.KH, self.KW, self.Cin, self.Cout)


@dataclass(frozen=True)
class DepthwiseWorkload:
    """NCHW input [N,C,H,W], weights [C*mult,KH,KW], symmetric zero padding."""
    name: str
    N: int
    C: int
    H: int
    W: int
    mult: int
    KH: int
    KW: int
    stride: int
    pad: int
    dil: int
    mode: str               # "exact" or "fast"
    seed: int

    @property
    def x_shape(self):
        return (self.N, self.C, self.H, self.W)

    @property
    def w_shape(self):
        return (self.C * self.mult, self.KH, self.KW)


def _draw(gen: torch.Generator, shape, dist: str, std: float | None = None) -> torch.Tensor:
    if dist == "uniform":
        return torch.rand(shape, generator=gen, dtype=torch.float32) * 2 - 1
    if dist == "normal":
        return torch.randn(shape, generator=gen, dtype=torch.float32) * float(std)
    raise ValueError(f"unknown distribution {dist!r}")


def dense_inputs(wl: DenseWorkload, dtype: str | None = None):
    """Return (X, F) as CPU tensors. ``dtype`` overrides ``wl.dtype`` for the
    fp32 run of a bf16 workload (same draws, no rounding)."""
    gen = torch.Generator().manual_seed(wl.seed)
    x = _draw(gen, wl.x_shape, wl.x_dist, 1.0)
    if wl.f_std is None:
        f = _draw(gen, wl.f_shape, "uniform")
    else:
        f = _draw(gen, wl.f_shape, "normal", wl.f_std)
    dt = dtype or wl.dtype
    if dt == "bf16":
        return x.to(torch.bfloat16), f.to(torch.bfloat16)
    if dt == "f32":
        return x, f
    raise ValueError(f"unknown dtype {dt!r}")


def depthwise_inputs(wl: DepthwiseWorkload):
    """Return (X, w) as fp32 CPU tensors, uniform in [-1, 1)."""
    gen = torch.Generator().manual_seed(wl.seed)
    x = _draw(gen, wl.x_shape, "uniform")
    w = _draw(gen, wl.w_shape, "uniform")
    return x, w


def random_tensor(shape, seed: int, dist: str = "uniform", dtype=torch.float32,
                  integer_range: int | None = None) -> torch.Tensor:
    """Generic seeded tensor for property and edge-case tests.

    With ``integer_range=r`` the values are integers in [-r, r]: sums of their
    products are exact in fp32 as long as they stay below 2**24, so every
    accumulation order gives the same bits.
    """
    gen = torch.Generator().manual_seed(seed)
    if integer_range is not None:
        t = torch.randint(-integer_range, integer_range + 1, tuple(shape), generator=gen)
        return t.to(dtype)
    return _draw(gen, tuple(shape), dist, 1.0).to(dtype)


# --- the workloads -----------------------------------------------------------
# Seeds follow 100 * workload_index + layer_index.

DENSE_TINY_F32 = DenseWorkload("dense_tiny_f32", 2, 8, 8, 3, 3, 3, 4, "f32", "uniform", None, 0)
DENSE_3X3_BF16 = DenseWorkload("dense3x3_bf16", 32, 58, 58, 64, 3, 3, 64, "bf16", "normal",
                               math.sqrt(2.0 / 576.0), 100)
DENSE_1X1_BF16 = DenseWorkload("dense1x1_bf16", 32, 28, 28, 256, 1, 1, 512, "bf16", "normal",
                               math.sqrt(2.0 / 256.0), 200)

DW_5X5S2_EXACT = DepthwiseWorkload("dw_c72_5x5s2_56_exact", 8, 72, 56, 56, 1, 5, 5, 2, 2, 1, "exact", 300)

# MobileNetV3-large-shaped sweep, batch 32, pad = K // 2, multiplier 1.
DW_SWEEP = [
    DepthwiseWorkload("dw_c16_3x3s1_112", 32, 16, 112, 112, 1, 3, 3, 1, 1, 1, "fast", 400),
    DepthwiseWorkload("dw_c64_3x3s2_112", 32, 64, 112, 112, 1, 3, 3, 2, 1, 1, "fast", 401),
    DepthwiseWorkload("dw_c120_5x5s1_28", 32, 120, 28, 28, 1, 5, 5, 1, 2, 1, "fast", 402),
    DepthwiseWorkload("dw_c672_5x5s2_14", 32, 672, 14, 14, 1, 5, 5, 2, 2, 1, "fast", 403),
    DepthwiseWorkload("dw_c960_5x5s1_7", 32, 960, 7, 7, 1, 5, 5, 1, 2, 1, "fast", 404),
]

DENSE_WORKLOADS = [DENSE_TINY_F32, DENSE_3X3_BF16, DENSE_1X1_BF16]
DEPTHWISE_WORKLOADS = [DW_5X5S2_EXACT] + DW_SWEEP
