"""Depthwise conv parity on the GPU: the HIP path (through the C ABI) against
the CPU oracle on identical seeded inputs, bit for bit.

Exact mode must match the oracle's bits everywhere (canonical NaN included).
Fast mode must match too: both sides use one correctly rounded fused
multiply-add per tap in the same order; only NaN payloads may differ.
"""
import numpy as np
import pytest
import torch

import convolution_forward_amd as cf
import oracle
import workloads as wl
from conftest import golden
from parity import bits

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
VARIANTS = [cf.VARIANT_DIRECT, cf.VARIANT_TILED]


def gpu_dw(x, w, bias=None, stride=1, padding=0, dilation=1, mode="exact", variant=cf.VARIANT_AUTO, out=None):
    y = cf.conv_depthwise(x.to(DEV), w.to(DEV), bias=None if bias is None else bias.to(DEV), stride=stride,
                          padding=padding, dilation=dilation, exact=(mode == "exact"), variant=variant, out=out)
    torch.cuda.synchronize()
    return y


def assert_same_bits(got, ref, mode):
    g, r = bits(got), bits(ref)
    if mode == "exact":
        np.testing.assert_array_equal(g, r)
    else:
        gn = np.isnan(got.cpu().numpy() if isinstance(got, torch.Tensor) else got)
        rn = np.isnan(ref)
        np.testing.assert_array_equal(gn, rn)
        np.testing.assert_array_equal(g[~gn], r[~rn])


def check(x, w, bias=None, stride=1, padding=0, dilation=1, mode="exact", variants=(cf.VARIANT_AUTO, *VARIANTS)):
    ref = oracle.depthwise_nchw(x, w, bias=bias, stride=stride, padding=padding, dilation=dilation, mode=mode)
    outs = []
    for v in variants:
        try:
            y = gpu_dw(x, w, bias, stride, padding, dilation, mode, variant=v)
        except cf.ConvArgumentError as e:
            if v == cf.VARIANT_TILED and e.status == cf.CONV_ERR_UNSUPPORTED:
                continue
            raise
        assert_same_bits(y, ref, mode)
        outs.append(y)
    return ref, outs


# --- the exact-mode workload and the MobileNetV3-shaped sweep, full tensors ---

def test_gpu_dw_exact_workload_bitwise():
    w_ = wl.DW_5X5S2_EXACT
    X, w = wl.depthwise_inputs(w_)
    ref, outs = check(X, w, stride=w_.stride, padding=w_.pad, dilation=w_.dil, mode="exact")
    assert tuple(outs[0].shape) == (8, 72, 28, 28)
    for y in outs[1:]:
        assert torch.equal(y.view(torch.int32), outs[0].view(torch.int32))


@pytest.mark.parametrize("layer", wl.DW_SWEEP, ids=lambda l: l.name)
@pytest.mark.parametrize("mode", ["fast", "exact"])
def test_gpu_dw_sweep_bitwise(layer, mode):
    X, w = wl.depthwise_inputs(layer)
    check(X, w, stride=layer.stride, padding=layer.pad, dilation=layer.dil, mode=mode)


# --- odd shapes: multiplier, dilation, large strides, ragged widths -----------

ODD = [  # N, C, H, W, mult, KH, KW, stride, pad, dil, bias
    (2, 3, 9, 13, 2, 3, 3, 1, 1, 1, True),
    (1, 5, 17, 10, 1, 3, 5, (2, 1), (1, 2), 1, False),
    (2, 4, 11, 11, 3, 3, 3, 3, 0, 1, True),            # stride 3 (generic path)
    (1, 2, 19, 23, 1, 3, 3, 1, 2, 2, False),           # dilation 2
    (1, 3, 1, 37, 1, 1, 5, 1, (0, 2), 1, False),       # 1D (H = 1)
    (3, 2, 6, 1, 1, 3, 1, 1, 1, 1, True),              # width 1
    (1, 1, 4, 4, 1, 3, 3, 1, 4, 1, False),             # padding wider than the kernel
    (2, 7, 33, 65, 1, 5, 5, 2, 2, 1, False),           # ragged rows, stride 2
    (1, 2, 15, 15, 1, 7, 7, 1, 3, 1, True),
    (1, 4, 40, 40, 2, 3, 3, 2, 1, 3, False),           # stride 2, dilation 3
    (1, 16, 3, 3, 1, 3, 3, 1, 1, 1, False),
    (1, 1, 70, 300, 1, 3, 3, 1, 1, 1, False),          # wide rows
]


@pytest.mark.parametrize("case", ODD)
@pytest.mark.parametrize("mode", ["exact", "fast"])
def test_gpu_dw_odd_shapes_bitwise(case, mode):
    N, C, H, W, m, KH, KW, s, p, d, has_bias = case
    seed = 5000 + ODD.index(case)
    X = wl.random_tensor((N, C, H, W), seed)
    w = wl.random_tensor((C * m, KH, KW), seed + 1)
    b = wl.random_tensor((C * m,), seed + 2) if has_bias else None
    check(X, w, bias=b, stride=s, padding=p, dilation=d, mode=mode)


# Shapes the LDS-tiled kernel takes, chosen to hit its tile boundaries:
# planes that do not divide into whole tiles, ragged row bands, multipliers
# whose output planes straddle tiles, both strides, both kernel sizes, odd
# padding, bias. Each runs on every variant (auto, direct, tiled) and must
# give the oracle's bits.
TILED = [  # N, C, H, W, mult, K, stride, pad, bias
    (2, 4, 12, 12, 3, 3, 1, 1, True),
    (3, 5, 14, 14, 2, 5, 2, 2, False),
    (1, 3, 8, 8, 1, 5, 1, 0, True),
    (1, 2, 100, 60, 1, 3, 1, 1, False),       # 4 bands, last one ragged
    (1, 3, 58, 46, 1, 5, 2, 2, True),         # stride 2, ragged band
    (2, 3, 30, 30, 1, 5, 1, 1, False),        # pad 1 with a 5x5 window
    (1, 6, 9, 12, 4, 3, 2, 0, True),          # multiplier 4, stride 2, no pad
    (4, 37, 7, 8, 1, 5, 1, 2, False),         # tiles of 36 planes, 148 planes
    (1, 1, 250, 250, 1, 3, 1, 1, False),      # widest rows the kernel takes
    (1, 2, 226, 226, 1, 3, 2, 1, True),       # stride 2 onto 113 columns
    (2, 20, 14, 14, 1, 5, 2, 2, True),        # 14-wide rows, 128 threads: 18 planes a tile, 40 planes
    (1, 11, 14, 14, 1, 3, 1, 1, False),       # 14 output rows: 9 planes a tile, a partial second tile
    (3, 7, 14, 14, 2, 3, 2, 1, False),        # 14-wide rows with multiplier 2
]


@pytest.mark.parametrize("case", TILED)
@pytest.mark.parametrize("mode", ["exact", "fast"])
def test_gpu_dw_tiled_shapes_bitwise(case, mode):
    N, C, H, W, m, K, s, p, has_bias = case
    seed = 6000 + TILED.index(case)
    X = wl.random_tensor((N, C, H, W), seed)
    w = wl.random_tensor((C * m, K, K), seed + 1)
    b = wl.random_tensor((C * m,), seed + 2) if has_bias else None
    assert cf.depthwise_variant_for(X.to(DEV), w.to(DEV), s, p) == cf.VARIANT_TILED
    check(X, w, bias=b, stride=s, padding=p, mode=mode)


# --- the pages' examples and special values ------------------------------------

def test_gpu_dw_worked_examples():
    g = golden("wxb_1d_examples.json")["window"]
    for mode in ("exact", "fast"):
        y = gpu_dw(torch.tensor(g["x"], dtype=torch.float32).reshape(1, 1, 1, -1),
                   torch.tensor(g["k"], dtype=torch.float32).reshape(1, 1, -1),
                   bias=torch.tensor([float(g["bias"])]), mode=mode)
        assert y.cpu().ravel().tolist() == g["y"]
    sb = golden("wxb_2d_examples.json")["sobel"]
    img = torch.zeros(1, 1, 6, 6)
    img[..., 3:] = 1
    w = torch.stack([torch.tensor(sb["gx"], dtype=torch.float32), torch.tensor(sb["gy"], dtype=torch.float32)])
    y = gpu_dw(img, w)
    assert y.cpu()[0, 0].tolist() == sb["gx_output"] and y.cpu()[0, 1].tolist() == sb["gy_output"]


def special_input(seed, shape):
    """Random values with NaNs (with payloads and signs), infinities, signed
    zeros and subnormals sprinkled in."""
    x = wl.random_tensor(shape, seed).numpy()
    u = x.view(np.uint32).copy()
    rng = np.random.default_rng(seed)
    flat = u.reshape(-1)
    picks = rng.choice(flat.size, size=max(8, flat.size // 40), replace=False)
    specials = np.array([0x7FC00000, 0xFFC12345, 0x7F800001, 0x7F800000, 0xFF800000, 0x00000000, 0x80000000,
                         0x00000001, 0x807FFFFF, 0x00400000], dtype=np.uint32)
    flat[picks] = specials[rng.integers(0, specials.size, size=picks.size)]
    return torch.from_numpy(u.view(np.float32).copy())


@pytest.mark.parametrize("mode", ["exact", "fast"])
def test_gpu_dw_special_values(mode):
    X = special_input(11, (2, 3, 14, 15))
    w = special_input(12, (6, 3, 3))
    w[0] = torch.tensor([[float("inf"), 0, 0], [0, 1, 0], [0, 0, 0]])       # inf meets padding in the corner
    b = wl.random_tensor((6,), 13)
    check(X, w, bias=b, stride=1, padding=1, mode=mode)
    check(X, w, stride=2, padding=2, mode=mode)


@pytest.mark.parametrize("mode", ["exact", "fast"])
def test_gpu_dw_subnormals(mode):
    X = wl.random_tensor((1, 4, 20, 20), 21) * 2.0 ** -70
    w = wl.random_tensor((4, 5, 5), 22) * 2.0 ** -70
    ref, outs = check(X, w, padding=2, mode=mode)
    assert np.any((ref != 0) & (np.abs(ref) < np.finfo(np.float32).tiny))


def test_gpu_dw_exact_vs_fast_rounding():
    a = 1 + 2.0 ** -12
    X = torch.tensor([1.0, a], dtype=torch.float32).reshape(1, 1, 1, 2)
    w = torch.tensor([-1.0, a], dtype=torch.float32).reshape(1, 1, 2)
    for v in VARIANTS:
        try:
            assert gpu_dw(X, w, mode="exact", variant=v).item() == 2.0 ** -11
            assert gpu_dw(X, w, mode="fast", variant=v).item() == 2.0 ** -11 + 2.0 ** -24
        except cf.ConvArgumentError as e:
            assert v == cf.VARIANT_TILED and e.status == cf.CONV_ERR_UNSUPPORTED


def test_gpu_dw_write_coverage_and_determinism():
    layer = wl.DW_SWEEP[3]
    X, w = wl.depthwise_inputs(layer)
    out = torch.full((32, 672, 7, 7), float("nan"), device=DEV)
    y1 = gpu_dw(X, w, stride=2, padding=2, mode="fast", out=out).clone()
    assert not torch.isnan(y1).any()
    y2 = gpu_dw(X, w, stride=2, padding=2, mode="fast")
    assert torch.equal(y1.view(torch.int32), y2.view(torch.int32))


# Small planes (whole planes per workgroup) from and into buffers that start
# 4 bytes past a 16-byte boundary: the kernel reads X four bytes at a time
# and falls back to 4-byte stores for a Y it cannot write in 16-byte pieces.
UNALIGNED = [  # N, C, H, W, mult, K, stride, pad, bias
    (2, 37, 7, 7, 1, 5, 1, 2, True),
    (3, 5, 14, 14, 2, 5, 2, 2, False),
    (2, 9, 9, 13, 1, 3, 1, 1, True),
]


@pytest.mark.parametrize("case", UNALIGNED)
@pytest.mark.parametrize("mode", ["exact", "fast"])
def test_gpu_dw_unaligned_buffers(case, mode):
    N, C, H, W, m, K, s, p, has_bias = case
    seed = 7000 + UNALIGNED.index(case)
    X = wl.random_tensor((N, C, H, W), seed)
    w = wl.random_tensor((C * m, K, K), seed + 1)
    b = wl.random_tensor((C * m,), seed + 2) if has_bias else None
    ref = oracle.depthwise_nchw(X, w, bias=b, stride=s, padding=p, mode=mode)
    xbuf = torch.zeros(X.numel() + 1, device=DEV)
    xv = xbuf[1:].view(X.shape)
    xv.copy_(X.to(DEV))
    ybuf = torch.full((ref.size + 1,), float("nan"), device=DEV)
    yv = ybuf[1:].view(ref.shape)
    wd = w.to(DEV)
    bd = None if b is None else b.to(DEV)
    assert xv.data_ptr() % 16 == 4 and yv.data_ptr() % 16 == 4
    assert cf.depthwise_variant_for(xv, wd, s, p, exact=(mode == "exact"), bias=bd, out=yv) == cf.VARIANT_TILED
    cf.conv_depthwise(xv, wd, bias=bd, stride=s, padding=p, exact=(mode == "exact"), out=yv)
    torch.cuda.synchronize()
    assert_same_bits(yv, ref, mode)
    assert torch.isnan(ybuf[0]).item()          # nothing written before Y
