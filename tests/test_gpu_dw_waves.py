"""Parity of the one-task-per-wave depthwise kernel (stride 2, 3x3 and 5x5
windows, output rows of at most 64 columns) at the edges of its tiling,
against the CPU oracle: bitwise in exact mode, bitwise except NaN payloads in
fast mode.

Each wave loads the padded input rows of its own band of output rows into
its own LDS region, so the cases cover: bands that run past the last output
row, several row groups per wave with idle lanes (64 / Wo not whole), one row
group of exactly 64 columns, no padding, the widest left padding the region
keeps (4), unequal padding before and after each axis (the window entry
point), inputs shorter than a band's rows, bias, and many planes.
"""
import numpy as np
import pytest
import torch

import convolution_forward_amd as cf
import oracle
import workloads as wl
from parity import bits

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

WAVES = [  # N, C, H, W, K, pad, bias
    (2, 8, 56, 56, 5, 2, False),      # the exact-mode workload's plane: 2 row groups of 28, 2 rows per lane
    (3, 5, 61, 44, 5, 2, True),       # Wo 22: 2 groups (20 idle lanes), last band 3 of 4 rows, bias
    (1, 4, 33, 32, 3, 0, False),      # no padding, Wo 15: 4 groups; the last input row is never read
    (2, 3, 112, 112, 3, 1, True),     # the 112-wide 3x3 layer's plane: one group of 56, 4 rows per lane
    (1, 2, 20, 128, 3, 1, False),     # Wo 64: one full group, every lane active
    (2, 6, 9, 64, 3, 1, False),       # Wo 32: exactly 2 groups; 5 output rows in one band of 8
    (1, 3, 4, 8, 5, 4, True),         # input shorter than a band, padding 4 on every side
    (1, 1, 10, 4, 5, 2, False),       # a 4-wide input (one 16-byte unit per row)
    (4, 40, 26, 36, 5, 1, False),     # 160 planes, odd output size (12 x 17)
]


def _assert_bits(y, ref, mode):
    g, r = bits(y), bits(ref)
    if mode == "exact":
        np.testing.assert_array_equal(g, r)
    else:
        gn, rn = np.isnan(y.cpu().numpy()), np.isnan(ref)
        np.testing.assert_array_equal(gn, rn)
        np.testing.assert_array_equal(g[~gn], r[~rn])


@pytest.mark.parametrize("case", WAVES)
@pytest.mark.parametrize("mode", ["exact", "fast"])
def test_gpu_dw_waves_kernel_bitwise(case, mode):
    N, C, H, W, K, p, has_bias = case
    seed = 8100 + WAVES.index(case)
    X = wl.random_tensor((N, C, H, W), seed)
    w = wl.random_tensor((C, K, K), seed + 1)
    b = wl.random_tensor((C,), seed + 2) if has_bias else None
    assert cf.depthwise_variant_for(X.to(DEV), w.to(DEV), 2, p) == cf.VARIANT_TILED
    y = cf.conv_depthwise(X.to(DEV), w.to(DEV), bias=None if b is None else b.to(DEV), stride=2, padding=p,
                          exact=(mode == "exact"))
    torch.cuda.synchronize()
    ref = oracle.depthwise_nchw(X, w, bias=b, stride=2, padding=p, mode=mode)
    _assert_bits(y, ref, mode)


@pytest.mark.parametrize("mode", ["exact", "fast"])
@pytest.mark.parametrize("pads", [(0, 2, 1, 3), (3, 0, 4, 0), (1, 1, 0, 2)])
def test_gpu_dw_waves_kernel_unequal_padding(mode, pads):
    """The window entry point with unequal padding: the oracle runs on the
    input with those zero rows and columns written out (a padding tap is a
    multiplication by +0, so both give the same bits)."""
    top, bottom, left, right = pads
    X = wl.random_tensor((2, 6, 30, 40), 8200 + sum(pads))
    w = wl.random_tensor((6, 5, 5), 8201)
    b = wl.random_tensor((6,), 8202)
    y = cf.conv_depthwise(X.to(DEV), w.to(DEV), bias=b.to(DEV), stride=2, padding=pads, exact=(mode == "exact"))
    torch.cuda.synchronize()
    Xp = np.zeros((2, 6, 30 + top + bottom, 40 + left + right), dtype=np.float32)
    Xp[:, :, top:top + 30, left:left + 40] = X.numpy()
    ref = oracle.depthwise_nchw(Xp, w, bias=b, stride=2, padding=0, mode=mode)
    assert y.shape == ref.shape
    _assert_bits(y, ref, mode)


def test_gpu_dw_waves_kernel_coverage_and_repeat():
    """Every output written (NaN sentinel), identical bits on a second call."""
    X = wl.random_tensor((3, 7, 61, 44), 8300)
    w = wl.random_tensor((7, 5, 5), 8301)
    out = torch.full((3, 7, 31, 22), float("nan"), device=DEV)
    y1 = cf.conv_depthwise(X.to(DEV), w.to(DEV), stride=2, padding=2, exact=True, out=out).clone()
    torch.cuda.synchronize()
    assert not torch.isnan(y1).any()
    y2 = cf.conv_depthwise(X.to(DEV), w.to(DEV), stride=2, padding=2, exact=True)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int32), y2.view(torch.int32))
