"""Parity of the fp32 1x1 kernel that runs on the bf16 matrix cores (each fp32
value split exactly into three bf16 parts, six of the nine part products
summed in fp32) against the fp64 CPU oracle.

The bar is the fp32 one: max |g - r| / max |r| <= 1e-5. Integer-valued
inputs up to 2^8 have no middle or low parts, so their sums are exact and
must match bit for bit. Infinities and NaNs keep their class. The cases hit
the tile edges: pixels that do not fill a 208-pixel tile, output channels
that do not fill a 128-channel tile, input channels that do not fill a
32-channel chunk, pixel strides of a channel slice, bias; and grids of more
than one round of workgroups (an odd number of chunks, ragged pixel and
channel tiles).
"""
import numpy as np
import pytest
import torch

import convolution_forward_amd as cf
import oracle
import workloads as wl
from parity import F32_MAX_REL, max_rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

CASES = [  # N, H, W, Cin, Cout, bias
    (2, 7, 11, 256, 136, False),     # 154 pixels: a ragged pixel tile, a ragged channel tile
    (4, 10, 13, 256, 512, True),     # four channel tiles, bias
    (1, 5, 9, 36, 64, False),        # 36 input channels: a partial second chunk
    (3, 8, 8, 4, 4, True),           # the smallest channel counts the kernel takes
    (8, 28, 28, 64, 128, False),     # 6272 pixels, 31 tiles
    (3, 37, 37, 36, 3600, True),     # 20 x 29 = 580 tiles (past one round), ragged pixel and channel tiles, bias
    (4, 44, 44, 68, 2048, False),    # 38 x 16 = 608 tiles, three chunks (the last of 4 channels)
]


def _run(X, F, bias=None, out=None):
    Y = cf.conv2d_nhwc(X.to(DEV), F.to(DEV), bias=None if bias is None else bias.to(DEV), out=out)
    torch.cuda.synchronize()
    return Y


@pytest.mark.parametrize("case", CASES)
def test_gpu_f32x6_shapes(case):
    N, H, W, C, O, has_bias = case
    seed = 9100 + CASES.index(case)
    X = wl.random_tensor((N, H, W, C), seed, dist="normal")
    F = wl.random_tensor((1, 1, C, O), seed + 1, dist="normal") * (2.0 / C) ** 0.5
    b = wl.random_tensor((O,), seed + 2) if has_bias else None
    assert cf.dense_variant_for(X.to(DEV), F.to(DEV)) == cf.VARIANT_TILED
    ref = oracle.conv2d_nhwc(X, F, bias=b)
    assert max_rel_err(_run(X, F, b), ref) <= F32_MAX_REL


def test_gpu_f32x6_integer_bitwise():
    """Integers in [-16, 16]: no middle or low parts, every sum exact."""
    X = wl.random_tensor((2, 9, 14, 96), 9200, integer_range=16)
    F = wl.random_tensor((1, 1, 96, 72), 9201, integer_range=16)
    Y = _run(X, F).cpu().numpy()
    np.testing.assert_array_equal(Y, oracle.conv2d_nhwc(X, F).astype(np.float32))


def test_gpu_f32x6_channel_slice_views():
    """X and Y as channel slices of wider tensors (pixel strides 160 and 96)."""
    Xw = wl.random_tensor((2, 6, 10, 160), 9300, dist="normal")
    F = wl.random_tensor((1, 1, 64, 48), 9301, dist="normal") * 0.125
    X = Xw[..., 32:96]
    Yw = torch.full((2, 6, 10, 96), float("nan"), device=DEV)
    Y = Yw[..., 16:64]
    _run(X, F, out=Y)
    ref = oracle.conv2d_nhwc(X.contiguous(), F)
    assert max_rel_err(Y, ref) <= F32_MAX_REL
    rest = torch.cat([Yw[..., :16], Yw[..., 64:]], dim=-1)
    assert torch.isnan(rest).all(), "wrote outside the output slice"


def test_gpu_f32x6_wide_range_and_specials():
    """Values across the exponent range (the split is exact by truncation, so
    large values cannot round up to infinity), then infinities and NaNs. A
    non-finite input gives a non-finite output wherever the fp64 sum is
    non-finite (an infinity can come out as NaN: it also meets the zero
    middle or low part of a weight), NaN wherever the sum is NaN, and the
    finite outputs stay within the fp32 bound."""
    rng = np.random.default_rng(9400)
    X = (rng.standard_normal((1, 4, 8, 64)) * np.exp2(rng.integers(-60, 60, (1, 4, 8, 64)))).astype(np.float32)
    F = (rng.standard_normal((1, 1, 64, 32)) * 0.1).astype(np.float32)
    X = torch.from_numpy(X)
    F = torch.from_numpy(F)
    Y = _run(X, F)
    ref = oracle.conv2d_nhwc(X, F)
    # Relative to each output's own scale of |x * w| sums (outputs differ by
    # up to 2^120 in size here).
    absref = oracle.conv2d_nhwc(X.abs(), F.abs())
    err = np.abs(Y.cpu().numpy().astype(np.float64) - ref) / np.maximum(absref, 1e-300)
    assert err.max() <= 1e-5
    X2 = X.clone()
    X2[0, 0, 0, 3] = float("inf")
    X2[0, 1, 2, 5] = float("nan")
    X2[0, 2, 3, 7] = float("-inf")
    Y2 = _run(X2, F).cpu().numpy()
    ref2 = oracle.conv2d_nhwc(X2, F)
    np.testing.assert_array_equal(np.isfinite(Y2), np.isfinite(ref2))
    assert np.isnan(Y2[np.isnan(ref2)]).all()
    fin = np.isfinite(ref2)
    assert np.max(np.abs(Y2[fin] - ref2[fin]) / np.maximum(absref[fin], 1e-300)) <= 1e-5
