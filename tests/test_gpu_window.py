"""The convolution window on the GPU (stride, padding before/after each axis,
dilation, groups) against the CPU oracle, through the window entry points.

"Convolution Is Wx+b Moving Across a Signal" defines stride, padding and
dilation per axis (section "Why 1D? Why 2D?"), grouped channel sums (section
"Find the same sum in CKE's C kernels"), causal and strided Conv1D (section
"Where this shows up in models I work with") and the patch stem (section
"Images going in: two ways to make patches"). Padding that differs before
and after an axis is checked against the oracle run on the input with the
zero rows and columns written out, which the oracle pins show is the same
thing (tests/test_oracle_pins.py).
"""
import numpy as np
import pytest
import torch

import bench
import convolution_forward_amd as cf
import oracle
import workloads as wl
from parity import BF16_RMS_REL, F32_MAX_REL, bf16_rounding_ok, bits, max_rel_err, rms_rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def pads4(padding):
    if isinstance(padding, int):
        return padding, padding, padding, padding
    if len(padding) == 2:
        return padding[0], padding[0], padding[1], padding[1]
    return tuple(padding)


def dense_ref(X, F, bias, stride, padding, dilation, groups):
    pt, pb, pl, pr = pads4(padding)
    Xp = np.pad(X.float().numpy(), ((0, 0), (pt, pb), (pl, pr), (0, 0)))
    return oracle.conv2d_nhwc(Xp, F.float().numpy(), bias=None if bias is None else bias.numpy(), stride=stride,
                              dilation=dilation, groups=groups)


DENSE = [  # name, (N,H,W,Cin), (KH,KW,Cout), stride, padding, dilation, groups
    ("same_3x3", (2, 13, 17, 16), (3, 3, 24), 1, 1, 1, 1),
    ("stride2_pad1", (2, 15, 14, 32), (3, 3, 40), 2, 1, 1, 1),
    ("asym_pad", (1, 10, 9, 8), (3, 3, 8), (2, 1), (1, 0, 2, 1), 1, 1),
    ("dilated", (1, 16, 15, 12), (3, 3, 10), 1, 2, (2, 3), 1),
    ("grouped", (2, 9, 9, 32), (3, 3, 48), 2, 1, 1, 4),
    ("grouped_1x1", (2, 6, 7, 24), (1, 1, 36), 1, 0, 1, 3),
    ("patch_stem", (2, 64, 48, 3), (16, 16, 32), 16, 0, 1, 1),
    ("conv1d_stride2", (1, 1, 300, 80), (1, 3, 64), (1, 2), (0, 1), 1, 1),
    ("causal_conv1d", (2, 1, 129, 16), (1, 4, 8), 1, (0, 0, 3, 0), 1, 1),
    ("causal_dilated", (1, 1, 77, 8), (1, 3, 8), 1, (0, 0, 4, 0), (1, 2), 1),
    # windows the bf16 matrix-core kernel takes (padding, stride 2, groups)
    ("mfma_same_3x3", (2, 20, 30, 64), (3, 3, 64), 1, 1, 1, 1),
    ("mfma_stride2_3x3", (2, 33, 40, 32), (3, 3, 48), 2, 1, 1, 1),
    ("mfma_stride2_asym", (1, 28, 28, 16), (3, 3, 16), 2, (0, 1, 0, 1), 1, 1),
    ("mfma_grouped_3x3", (2, 12, 14, 64), (3, 3, 64), 1, 1, 1, 4),
    ("mfma_grouped_1x1_s2", (2, 14, 14, 64), (1, 1, 128), 2, 0, 1, 2),
    ("mfma_1x1_padded", (1, 9, 10, 32), (1, 1, 40), 1, 1, 1, 1),
    ("mfma_wide_same", (1, 6, 120, 16), (3, 3, 16), 1, 1, 1, 1),
    ("mfma_pad_2_stride2", (1, 17, 9, 24), (3, 3, 8), 2, 2, 1, 1),
    # small groups packed block-diagonally into 64-channel tiles
    ("mfma_pack_g8_stride2", (2, 15, 18, 128), (3, 3, 128), 2, 1, 1, 16),
    ("mfma_pack_g32_1x1", (2, 9, 10, 128), (1, 1, 128), 1, 0, 1, 4),
    ("mfma_pack_g16_wide", (1, 7, 100, 128), (3, 3, 128), 1, 1, 1, 8),
    ("mfma_pack_g16_ragged", (3, 5, 21, 64), (3, 3, 64), 1, (1, 0, 2, 1), 1, 4),
    # windows only the streamed-filter GEMM kernel takes
    ("gemm_3x3_cin128", (2, 14, 15, 128), (3, 3, 72), 1, 1, 1, 1),
    ("gemm_dilated", (1, 20, 18, 32), (3, 3, 40), 1, 2, 2, 1),
    ("gemm_5x5_s2", (2, 23, 19, 24), (5, 5, 32), 2, 2, 1, 1),
    ("gemm_conv1d_s2", (2, 1, 700, 96), (1, 3, 128), (1, 2), (0, 1), 1, 1),
    ("gemm_grouped_cin128", (1, 9, 11, 256), (3, 3, 128), 1, 1, 1, 2),
    ("gemm_unequal_stride", (1, 16, 30, 16), (3, 3, 16), (2, 3), (1, 0, 1, 1), 1, 1),
]


@pytest.mark.parametrize("case", DENSE, ids=lambda c: c[0])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gpu_dense_window(case, dtype):
    name, (N, H, W, C), (KH, KW, O), stride, padding, dilation, groups = case
    seed = 9000 + DENSE.index(case)
    X = wl.random_tensor((N, H, W, C), seed)
    F = wl.random_tensor((KH, KW, C // groups, O), seed + 1) * (1.0 / (KH * KW * C / groups) ** 0.5)
    b = wl.random_tensor((O,), seed + 2)
    if dtype == "bf16":
        X, F = X.to(torch.bfloat16), F.to(torch.bfloat16)
    ref = dense_ref(X, F, b, stride, padding, dilation, groups)
    kw = dict(stride=stride, padding=padding, dilation=dilation, groups=groups)
    Y = cf.conv2d_nhwc(X.to(DEV), F.to(DEV), bias=b.to(DEV), out_dtype=torch.float32, **kw)
    torch.cuda.synchronize()
    assert tuple(Y.shape) == ref.shape
    if dtype == "f32":
        assert max_rel_err(Y, ref) <= F32_MAX_REL
    else:
        assert rms_rel_err(Y, ref) <= 1e-3
        Yb = cf.conv2d_nhwc(X.to(DEV), F.to(DEV), bias=b.to(DEV), **kw)
        torch.cuda.synchronize()
        assert rms_rel_err(Yb, ref) <= BF16_RMS_REL
        absref = dense_ref(X.float().abs(), F.float().abs(), b.abs(), stride, padding, dilation, groups)
        assert bf16_rounding_ok(Yb, ref, absref, KH * KW * C // groups)
        # the bf16 epilogue rounds the same fp32 accumulator to nearest-even
        assert torch.equal(Yb.cpu().view(torch.int16), Y.cpu().to(torch.bfloat16).view(torch.int16))
    # fp32 operands take the matrix cores in every window; bf16 in those named for them
    meant_tiled = dtype == "f32" or name.startswith("mfma") or name.startswith("gemm")
    if meant_tiled:
        assert cf.dense_variant_for(X.to(DEV), F.to(DEV), bias=b.to(DEV), **kw) == cf.VARIANT_TILED
    # every variant that accepts the window gives the same contract; the
    # windows meant for the matrix-core kernels must not be declined by them
    for v in (cf.VARIANT_DIRECT, cf.VARIANT_TILED):
        try:
            Yv = cf.conv2d_nhwc(X.to(DEV), F.to(DEV), bias=b.to(DEV), out_dtype=torch.float32, variant=v, **kw)
        except cf.ConvArgumentError as e:
            assert v == cf.VARIANT_TILED and e.status == cf.CONV_ERR_UNSUPPORTED and not meant_tiled
            continue
        torch.cuda.synchronize()
        assert (max_rel_err(Yv, ref) <= F32_MAX_REL) if dtype == "f32" else (rms_rel_err(Yv, ref) <= 1e-3)


F32_GEMM = [  # name, (N,H,W,Cin), (KH,KW,Cout), stride, padding, dilation, groups, (out channels, offset)
    # groups of 48 output channels straddle the 64-channel tiles
    ("groups_across_tiles", (2, 9, 11, 96), (3, 3, 144), 1, 1, 1, 3, None),
    # three input channels (the small first layer), stride 2, Cout not a multiple of 4
    ("cin3_stride2", (2, 33, 31, 3), (3, 3, 5), 2, 1, 1, 1, None),
    ("cin3_7x7_s2_pad3", (1, 40, 36, 3), (7, 7, 64), 2, 3, 1, 1, None),
    # one group per channel, through the dense entry point
    ("channel_groups", (1, 10, 12, 16), (3, 3, 16), 1, 1, 1, 16, None),
    # 2700 k values: many chunks and a ragged last one; pixel count ragged too
    ("long_k", (1, 6, 7, 300), (3, 3, 70), 1, 1, 1, 1, None),
    ("dilated_unequal", (2, 19, 23, 12), (3, 2, 20), (2, 1), (2, 0, 1, 1), (2, 3), 2, None),
    # output into a channel slice: 16-byte aligned (vector stores) or not (scalar)
    ("slice_aligned", (2, 9, 10, 20), (3, 3, 24), 1, 1, 1, 1, (40, 8)),
    ("slice_unaligned", (2, 9, 10, 20), (3, 3, 24), 1, 1, 1, 1, (29, 3)),
]


@pytest.mark.parametrize("case", F32_GEMM, ids=lambda c: c[0])
def test_gpu_dense_f32_gemm_kernel(case):
    """fp32 windows the row kernel declines run on the fp32 matrix-core GEMM
    kernel (AUTO picks it): every output against the oracle within the fp32
    bar, nothing outside an output slice written."""
    name, (N, H, W, C), (KH, KW, O), stride, padding, dilation, groups, slice_ = case
    seed = 9700 + F32_GEMM.index(case)
    X = wl.random_tensor((N, H, W, C), seed)
    F = wl.random_tensor((KH, KW, C // groups, O), seed + 1) * (1.0 / (KH * KW * C / groups) ** 0.5)
    b = wl.random_tensor((O,), seed + 2)
    ref = dense_ref(X, F, b, stride, padding, dilation, groups)
    kw = dict(stride=stride, padding=padding, dilation=dilation, groups=groups)
    Xd, Fd, bd = X.to(DEV), F.to(DEV), b.to(DEV)
    assert cf.dense_variant_for(Xd, Fd, bias=bd, **kw) == cf.VARIANT_TILED
    if slice_ is None:
        Y = cf.conv2d_nhwc(Xd, Fd, bias=bd, **kw)
        torch.cuda.synchronize()
    else:
        total, off = slice_
        buf = torch.full(ref.shape[:3] + (total,), float("nan"), device=DEV)
        Y = buf[..., off:off + O]
        cf.conv2d_nhwc(Xd, Fd, bias=bd, out=Y, **kw)
        torch.cuda.synchronize()
        outside = torch.cat([buf[..., :off], buf[..., off + O:]], dim=-1)
        assert torch.isnan(outside).all()
    assert tuple(Y.shape) == ref.shape
    assert max_rel_err(Y, ref) <= F32_MAX_REL


DW = [  # name, (N,C,H,W), mult, (KH,KW), stride, padding (t,b,l,r), dilation
    ("causal_dw_conv1d", (2, 16, 1, 200), 1, (1, 4), 1, (0, 0, 3, 0), 1),
    ("causal_dw_dilated", (1, 8, 1, 97), 2, (1, 3), 1, (0, 0, 4, 0), (1, 2)),
    ("same_even_stride2", (2, 12, 28, 28), 1, (3, 3), 2, (0, 1, 0, 1), 1),
    ("asym_5x5", (1, 6, 19, 22), 1, (5, 5), 1, (2, 1, 0, 3), 1),
    ("asym_tiled_3x3", (2, 8, 30, 32), 1, (3, 3), 2, (1, 0, 1, 0), 1),
    # one-row filters on the row kernel: several segments, ragged tails,
    # stride 2, multiplier 2, rows of pure padding above the input
    ("row_causal_long", (1, 3, 1, 5000), 1, (1, 4), 1, (0, 0, 3, 0), 1),
    ("row_stride2_k5", (2, 6, 1, 333), 2, (1, 5), (1, 2), (0, 0, 2, 2), 1),
    ("row_rows_k3", (1, 4, 5, 2100), 1, (1, 3), (2, 1), (1, 0, 1, 1), 1),
]


@pytest.mark.parametrize("case", DW, ids=lambda c: c[0])
@pytest.mark.parametrize("mode", ["exact", "fast"])
def test_gpu_depthwise_window_bitwise(case, mode):
    name, (N, C, H, W), m, (KH, KW), stride, padding, dilation = case
    seed = 9500 + DW.index(case)
    X = wl.random_tensor((N, C, H, W), seed)
    w = wl.random_tensor((C * m, KH, KW), seed + 1)
    b = wl.random_tensor((C * m,), seed + 2)
    pt, pb, pl, pr = padding
    Xp = np.pad(X.numpy(), ((0, 0), (0, 0), (pt, pb), (pl, pr)))
    ref = oracle.depthwise_nchw(Xp, w.numpy(), bias=b.numpy(), stride=stride, padding=0, dilation=dilation,
                                mode=mode)
    outs = []
    for v in (cf.VARIANT_AUTO, cf.VARIANT_DIRECT, cf.VARIANT_TILED):
        try:
            Y = cf.conv_depthwise(X.to(DEV), w.to(DEV), bias=b.to(DEV), stride=stride, padding=padding,
                                  dilation=dilation, exact=(mode == "exact"), variant=v)
        except cf.ConvArgumentError as e:
            assert v == cf.VARIANT_TILED and e.status == cf.CONV_ERR_UNSUPPORTED
            continue
        torch.cuda.synchronize()
        assert tuple(Y.shape) == ref.shape
        g, r = bits(Y), bits(ref)
        if mode == "exact":
            np.testing.assert_array_equal(g, r)
        else:
            gn, rn = np.isnan(Y.cpu().numpy()), np.isnan(ref)
            np.testing.assert_array_equal(gn, rn)
            np.testing.assert_array_equal(g[~gn], r[~rn])
        outs.append(Y)
    if name == "asym_tiled_3x3" or name.startswith("row_") or name == "causal_dw_conv1d":
        assert cf.depthwise_variant_for(X.to(DEV), w.to(DEV), stride, padding, dilation) == cf.VARIANT_TILED


@pytest.mark.parametrize("total,offset", [(136, 64), (76, 2)], ids=["aligned_slice", "unaligned_slice"])
def test_gpu_gemm_bf16_into_channel_slice(total, offset):
    """A window only the streamed GEMM kernel takes, written as bf16 into a
    channel slice of a wider buffer. With a 16-byte aligned slice and pixel
    stride the kernel's whole-row stores run; otherwise another variant takes
    the call. Either way the slice gets the contract's values and nothing
    outside it is written."""
    X = wl.random_tensor((2, 14, 15, 128), 9300).to(torch.bfloat16)
    F = (wl.random_tensor((3, 3, 128, 72), 9301) * (1.0 / (9 * 128) ** 0.5)).to(torch.bfloat16)
    b = wl.random_tensor((72,), 9302)
    ref = dense_ref(X, F, b, 1, 1, 1, 1)
    buf = torch.full((2, 14, 15, total), float("nan"), dtype=torch.bfloat16, device=DEV)
    out = buf[..., offset:offset + 72]
    y = cf.conv2d_nhwc(X.to(DEV), F.to(DEV), bias=b.to(DEV), padding=1, out=out)
    y32 = cf.conv2d_nhwc(X.to(DEV), F.to(DEV), bias=b.to(DEV), padding=1, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert y.data_ptr() == out.data_ptr()
    assert rms_rel_err(out, ref) <= BF16_RMS_REL
    absref = dense_ref(X.float().abs(), F.float().abs(), b.abs(), 1, 1, 1, 1)
    assert bf16_rounding_ok(out, ref, absref, 9 * 128)
    if offset % 8 == 0:
        # same kernel and accumulation as the fp32 call: its rounding, bit for bit
        assert torch.equal(out.cpu().view(torch.int16), y32.cpu().to(torch.bfloat16).view(torch.int16))
    outside = torch.cat([buf[..., :offset], buf[..., offset + 72:]], dim=-1)
    assert torch.isnan(outside.float()).all()


@pytest.mark.parametrize("layer", bench.WINDOW_LAYERS, ids=lambda l: l[0].split(" (")[0].replace(" ", "_"))
def test_gpu_window_layer_full_size(layer):
    """The window layers the benchmark times, at their full sizes, on the
    tiled MFMA path: every output against the oracle, bias included."""
    name, (N, H, W, C), (KH, KW, O), stride, padding, groups, _ = layer
    seed = 9400 + bench.WINDOW_LAYERS.index(layer)
    X = wl.random_tensor((N, H, W, C), seed).to(torch.bfloat16)
    F = (wl.random_tensor((KH, KW, C // groups, O), seed + 1) * (1.0 / (KH * KW * C / groups) ** 0.5)).to(torch.bfloat16)
    b = wl.random_tensor((O,), seed + 2)
    kw = dict(stride=stride, padding=padding, groups=groups)
    Xd, Fd = X.to(DEV), F.to(DEV)
    bd = b.to(DEV)
    assert cf.dense_variant_for(Xd, Fd, bias=bd, **kw) == cf.VARIANT_TILED
    Y = cf.conv2d_nhwc(Xd, Fd, bias=bd, **kw)
    torch.cuda.synchronize()
    ref = oracle.conv2d_nhwc(X, F, bias=b, **kw)
    assert tuple(Y.shape) == ref.shape
    assert rms_rel_err(Y, ref) <= BF16_RMS_REL
    absref = oracle.conv2d_nhwc(X.float().abs(), F.float().abs(), bias=b.abs(), **kw)
    assert bf16_rounding_ok(Y, ref, absref, KH * KW * C // groups)
    assert torch.isfinite(Y.float()).all()
