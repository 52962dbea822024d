"""Dense conv2d parity on the GPU: the HIP path (through the C ABI) against
the fp64 CPU oracle on identical seeded inputs.

Tolerances: fp32 max relative error 1e-5 (relative to the largest output);
bf16 inputs with fp32 accumulation 2e-2 relative to the output RMS; integer-
valued inputs bitwise (every partial sum is an exact integer in fp32).
"""
import numpy as np
import pytest
import torch

import convolution_forward_amd as cf
import oracle
import workloads as wl
from conftest import golden
from parity import (BF16_RMS_REL, F32_MAX_REL, abs_sum_dense, bf16_rounding_ok, bits, max_rel_err, rms_rel_err,
                    to_f64)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
VARIANTS = [cf.VARIANT_DIRECT, cf.VARIANT_TILED]


def run(x, f, bias=None, out_dtype=None, variant=cf.VARIANT_AUTO, out=None):
    y = cf.conv2d_nhwc(x.to(DEV) if not x.is_cuda else x, f.to(DEV), bias=None if bias is None else bias.to(DEV),
                       out_dtype=out_dtype, variant=variant, out=out)
    torch.cuda.synchronize()
    return y


def supported(x, f, variant, out_dtype=None):
    """Whether a forced variant accepts the shape (UNSUPPORTED otherwise)."""
    if variant != cf.VARIANT_TILED:
        return True
    xd = x.to(DEV)
    return cf.dense_variant_for(xd, f, out_dtype) == cf.VARIANT_TILED


# --- the pages' worked examples on the GPU -------------------------------------

def test_gpu_lecture_arange_example():
    g = golden("lecture14_arange_patches.json")
    X = torch.arange(36, dtype=torch.float32).reshape(1, 6, 6, 1)
    F = torch.arange(9, dtype=torch.float32).reshape(3, 3, 1, 1)
    Y = run(X, F)
    assert Y.cpu()[0, :, :, 0].tolist() == g["output"]


def test_gpu_wxb_examples():
    g1 = golden("wxb_1d_examples.json")
    w = g1["window"]
    Y = run(torch.tensor(w["x"], dtype=torch.float32).reshape(1, 1, -1, 1),
            torch.tensor(w["k"], dtype=torch.float32).reshape(1, -1, 1, 1),
            bias=torch.tensor([float(w["bias"])]))
    assert Y.cpu().ravel().tolist() == w["y"]
    t = g1["two_filters"]
    Y = run(torch.tensor(t["x"], dtype=torch.float32).reshape(1, 1, -1, 1),
            torch.tensor(t["K_taps_by_filters"], dtype=torch.float32).reshape(1, 3, 1, 2),
            bias=torch.tensor(t["bias"], dtype=torch.float32))
    assert Y.cpu()[0, 0].tolist() == t["y_positions_by_filters"]
    g2 = golden("wxb_2d_examples.json")
    s = g2["small"]
    Y = run(torch.tensor(s["image"], dtype=torch.float32).reshape(1, 3, 3, 1),
            torch.tensor(s["filter"], dtype=torch.float32).reshape(2, 2, 1, 1))
    assert Y.cpu()[0, :, :, 0].tolist() == s["output"]
    sb = g2["sobel"]
    img = torch.zeros(6, 6)
    img[:, 3:] = 1
    F = torch.stack([torch.tensor(sb["gx"], dtype=torch.float32), torch.tensor(sb["gy"], dtype=torch.float32)], -1)
    for dt in (torch.float32, torch.bfloat16):
        Y = run(img.reshape(1, 6, 6, 1).to(dt), F.reshape(3, 3, 1, 2).to(dt), out_dtype=torch.float32)
        assert Y.cpu()[0, :, :, 0].tolist() == sb["gx_output"]
        assert Y.cpu()[0, :, :, 1].tolist() == sb["gy_output"]


# --- the tiny fp32 workload, full tensor ---------------------------------------

@pytest.mark.parametrize("variant", [cf.VARIANT_AUTO] + VARIANTS)
def test_gpu_dense_tiny_f32(variant):
    w = wl.DENSE_TINY_F32
    X, F = wl.dense_inputs(w)
    # three input channels are zero-filled to the fp32 matrix cores' k granularity
    assert cf.dense_variant_for(X.to(DEV), F.to(DEV)) == cf.VARIANT_TILED
    ref = oracle.conv2d_nhwc(X, F)
    Y = run(X, F, variant=variant)
    assert tuple(Y.shape) == (2, 6, 6, 4)
    assert max_rel_err(Y, ref) <= F32_MAX_REL


# --- shapes spanning several tiles with ragged tails ---------------------------

SHAPES = [  # N, H, W, Cin, K, Cout
    (2, 17, 23, 64, 3, 64),
    (1, 30, 9, 32, 3, 48),
    (3, 12, 40, 16, 5, 24),
    (2, 20, 19, 128, 1, 96),
    (1, 8, 70, 8, 2, 8),
    (2, 11, 13, 3, 3, 5),
    (1, 7, 7, 40, 7, 16),          # filter spans the whole image
]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("variant", VARIANTS)
def test_gpu_dense_shapes(shape, dtype, variant):
    N, H, W, C, K, O = shape
    seed = 1000 + SHAPES.index(shape)
    X = wl.random_tensor((N, H, W, C), seed)
    F = wl.random_tensor((K, K, C, O), seed + 1) * (1.0 / (K * K * C) ** 0.5)
    if dtype == "bf16":
        X, F = X.to(torch.bfloat16), F.to(torch.bfloat16)
    if not supported(X, F.to(DEV), variant):
        pytest.skip("shape outside the tiled variant")
    ref = oracle.conv2d_nhwc(X, F)
    Y = run(X, F, variant=variant, out_dtype=torch.float32)
    if dtype == "f32":
        assert max_rel_err(Y, ref) <= F32_MAX_REL
    else:
        assert rms_rel_err(Y, ref) <= 1e-3          # fp32 output: only accumulation order differs
        Yb = run(X, F, variant=variant)
        assert Yb.dtype == torch.bfloat16
        assert rms_rel_err(Yb, ref) <= BF16_RMS_REL
        assert bf16_rounding_ok(Yb, ref, abs_sum_dense(oracle, X, F), K * K * C)
        # the bf16 epilogue rounds the same fp32 accumulator to nearest-even
        assert torch.equal(Yb.cpu().view(torch.int16), Y.cpu().to(torch.bfloat16).view(torch.int16))


@pytest.mark.parametrize("variant", VARIANTS)
def test_gpu_dense_integer_bitwise(variant):
    """Integer-valued inputs keep every partial sum exact, so any accumulation
    order must reproduce the oracle bit for bit."""
    X = wl.random_tensor((2, 13, 21, 64), 77, integer_range=4)
    F = wl.random_tensor((3, 3, 64, 32), 78, integer_range=4)
    ref = oracle.conv2d_nhwc(X, F)
    assert np.max(np.abs(ref)) < 2 ** 24
    for dt in (torch.float32, torch.bfloat16):
        if not supported(X.to(dt), F.to(dt).to(DEV), variant):
            continue
        Y = run(X.to(dt), F.to(dt), variant=variant, out_dtype=torch.float32)
        np.testing.assert_array_equal(to_f64(Y), ref)


@pytest.mark.parametrize("variant", VARIANTS)
def test_gpu_dense_bf16_output_rounds_to_nearest_even(variant):
    """Integer sums are exact in fp32, so the bf16 output must be exactly the
    exact sum rounded to nearest-even (torch's CPU fp32->bf16 conversion).
    Values above 256 need rounding; truncation or ties-away would differ."""
    X = wl.random_tensor((2, 9, 30, 64), 81, integer_range=6).to(torch.bfloat16)
    F = wl.random_tensor((3, 3, 64, 32), 82, integer_range=6).to(torch.bfloat16)
    if not supported(X, F.to(DEV), variant):
        pytest.skip("outside the tiled variant")
    ref = oracle.conv2d_nhwc(X, F)
    assert np.max(np.abs(ref)) < 2 ** 24 and np.mean(np.abs(ref) > 256) > 0.3
    expect = torch.from_numpy(ref.astype(np.float32)).to(torch.bfloat16)
    Y = run(X, F, variant=variant)
    assert torch.equal(Y.cpu().view(torch.int16), expect.view(torch.int16))


@pytest.mark.parametrize("variant", VARIANTS)
def test_gpu_dense_bias_and_views(variant):
    """Bias in the epilogue; X as a non-contiguous view (channel stride 1) and
    Y written through strides into a larger buffer, untouched elsewhere."""
    base = wl.random_tensor((2, 14, 20, 80), 91).to(torch.bfloat16).to(DEV)
    X = base[:, 1:13, 2:18, 8:72]                    # [2,12,16,64], strided
    F = (wl.random_tensor((3, 3, 64, 32), 92) * 0.05).to(torch.bfloat16)
    b = wl.random_tensor((32,), 93)
    if not supported(X, F.to(DEV), variant):
        pytest.skip("view outside the tiled variant")
    ref = oracle.conv2d_nhwc(X.cpu(), F, bias=b)
    big = torch.full((2, 12, 16, 48), float("nan"), dtype=torch.float32, device=DEV)
    Yv = big[:, 1:11, 1:15, 8:40]
    run(X, F, bias=b, variant=variant, out=Yv)
    assert rms_rel_err(Yv, ref) <= 1e-3
    mask = torch.ones_like(big, dtype=torch.bool)
    mask[:, 1:11, 1:15, 8:40] = False
    assert torch.isnan(big[mask]).all()


@pytest.mark.parametrize("variant", VARIANTS)
def test_gpu_dense_write_coverage_and_determinism(variant):
    X = wl.random_tensor((3, 19, 27, 32), 55).to(torch.bfloat16)
    F = (wl.random_tensor((3, 3, 32, 40), 56) * 0.1).to(torch.bfloat16)
    if not supported(X, F.to(DEV), variant):
        pytest.skip("outside the tiled variant")
    out = torch.full((3, 17, 25, 40), float("nan"), dtype=torch.bfloat16, device=DEV)
    Y1 = run(X, F, variant=variant, out=out).clone()
    assert not torch.isnan(Y1).any()
    Y2 = run(X, F, variant=variant)
    assert torch.equal(Y1.view(torch.int16), Y2.view(torch.int16))


# --- fp32 operands on the matrix-core kernel ------------------------------------

F32_MFMA = [  # N, H, W, Cin, K, Cout
    (2, 9, 66, 16, 3, 20),        # 64-pixel rows (two blocks per wave), partial channel tile
    (1, 5, 34, 64, 3, 64),
    (3, 6, 50, 32, 3, 72),        # two channel tiles, the second nearly empty
    (2, 7, 11, 256, 1, 136),      # 1x1 regrouped, three channel tiles
    (1, 3, 64, 48, 1, 8),
]


@pytest.mark.parametrize("shape", F32_MFMA)
def test_gpu_dense_f32_matrix_cores(shape):
    N, H, W, C, K, O = shape
    seed = 8000 + F32_MFMA.index(shape)
    X = wl.random_tensor((N, H, W, C), seed)
    F = wl.random_tensor((K, K, C, O), seed + 1) * (1.0 / (K * K * C) ** 0.5)
    b = wl.random_tensor((O,), seed + 2)
    assert cf.dense_variant_for(X.to(DEV), F.to(DEV)) == cf.VARIANT_TILED
    ref = oracle.conv2d_nhwc(X, F, bias=b)
    Ho, Wo = H - K + 1, W - K + 1
    big = torch.full((N, Ho, Wo, O + 8), float("nan"), dtype=torch.float32, device=DEV)
    Y = run(X, F, bias=b, out=big[..., 4:O + 4], variant=cf.VARIANT_TILED)
    assert max_rel_err(Y, ref) <= F32_MAX_REL
    assert torch.isnan(big[..., :4]).all() and torch.isnan(big[..., O + 4:]).all()
    Yd = run(X, F, bias=b, variant=cf.VARIANT_DIRECT)
    assert max_rel_err(Yd, ref) <= F32_MAX_REL


# --- 1x1 filters: the pixel regrouping and the layouts that prevent it --------

POINTWISE = [  # name, X base shape, X view slices, Cout
    ("batch_contiguous", (4, 10, 13, 64), None, 80),          # 520 pixels, regrouped into rows of 104
    ("prime_pixels", (1, 1, 127, 32), None, 24),               # 127 pixels: no regrouping
    ("image_contiguous", (3, 9, 16, 48), "batch", 40),         # batch stride padded
    ("cropped", (2, 12, 20, 32), "crop", 64),                  # rows not at one pixel stride
    ("channel_slice", (2, 7, 9, 96), "chan", 72),              # pixel stride 96, 64 channels used
]


@pytest.mark.parametrize("case", POINTWISE, ids=lambda c: c[0])
def test_gpu_dense_pointwise_layouts(case):
    name, shape, view, O = case
    seed = 7000 + POINTWISE.index(case)
    base = wl.random_tensor(shape, seed).to(torch.bfloat16).to(DEV)
    if view == "batch":
        big = torch.zeros((shape[0], shape[1] + 1, shape[2], shape[3]), dtype=torch.bfloat16, device=DEV)
        big[:, :shape[1]] = base
        X = big[:, :shape[1]]
    elif view == "crop":
        X = base[:, 1:-1, 2:-1]
    elif view == "chan":
        X = base[..., 16:80]
    else:
        X = base
    C = X.shape[-1]
    F = (wl.random_tensor((1, 1, C, O), seed + 1) * (1.0 / C ** 0.5)).to(torch.bfloat16)
    b = wl.random_tensor((O,), seed + 2)
    ref = oracle.conv2d_nhwc(X.cpu(), F, bias=b)
    for variant in [cf.VARIANT_AUTO] + VARIANTS:
        if not supported(X, F.to(DEV), variant, torch.float32):
            continue
        out = torch.full(tuple(X.shape[:3]) + (O + 8,), float("nan"), dtype=torch.float32, device=DEV)
        Y = run(X, F, bias=b, variant=variant, out=out[..., :O], out_dtype=torch.float32)
        assert rms_rel_err(Y, ref) <= 1e-3, variant
        assert torch.isnan(out[..., O:]).all()
        Yb = run(X, F, bias=b, variant=variant)
        assert rms_rel_err(Yb, ref) <= BF16_RMS_REL
        assert bf16_rounding_ok(Yb, ref, abs_sum_dense(oracle, X.cpu(), F, bias=b), C)


# --- the full-size workloads, in the launch configuration the benchmark uses ---

@pytest.mark.parametrize("work", [wl.DENSE_3X3_BF16, wl.DENSE_1X1_BF16], ids=lambda w: w.name)
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32], ids=["ybf16", "yf32"])
@pytest.mark.parametrize("with_bias", [False, True], ids=["nobias", "bias"])
def test_gpu_dense_full_size(work, out_dtype, with_bias):
    """Every output of the full-size layer against the fp64 oracle (the
    benchmark's launch, without bias; and the same launch with a bias)."""
    X, F = wl.dense_inputs(work)
    b = wl.random_tensor((work.Cout,), work.seed + 7) if with_bias else None
    Y = run(X, F, bias=b, out_dtype=out_dtype)
    shape = (work.N, work.H - work.KH + 1, work.W - work.KW + 1, work.Cout)
    assert tuple(Y.shape) == shape
    ref = oracle.conv2d_nhwc(X, F, bias=b)
    if out_dtype == torch.bfloat16:
        assert rms_rel_err(Y, ref) <= BF16_RMS_REL
        assert bf16_rounding_ok(Y, ref, abs_sum_dense(oracle, X, F, bias=b), work.KH * work.KW * work.Cin)
    else:
        assert rms_rel_err(Y, ref) <= 1e-4
    assert torch.isfinite(Y).all()


def test_gpu_dense_1x1_f32_full_size():
    work = wl.DENSE_1X1_BF16
    X, F = wl.dense_inputs(work, dtype="f32")
    Y = run(X, F)
    assert tuple(Y.shape) == (work.N, work.H, work.W, work.Cout)
    assert max_rel_err(Y, oracle.conv2d_nhwc(X, F)) <= F32_MAX_REL


def test_gpu_calls_allocate_no_device_memory():
    """No hidden copy: with every buffer allocated by the caller, the
    convolution calls leave the device's free memory unchanged (after one
    warm-up call per kernel, which lets the runtime load its code)."""
    X, F = wl.dense_inputs(wl.DENSE_3X3_BF16)
    X, F = X.to(DEV), F.to(DEV)
    Y = torch.empty((32, 56, 56, 64), dtype=torch.bfloat16, device=DEV)
    Xp, Fp = wl.dense_inputs(wl.DENSE_1X1_BF16)
    Xp, Fp = Xp.to(DEV), Fp.to(DEV)
    Yp = torch.empty((32, 28, 28, 512), dtype=torch.bfloat16, device=DEV)
    Xd, wd = wl.depthwise_inputs(wl.DW_5X5S2_EXACT)
    Xd, wd = Xd.to(DEV), wd.to(DEV)
    Yd = torch.empty((8, 72, 28, 28), dtype=torch.float32, device=DEV)
    Xf, Ff = wl.dense_inputs(wl.DENSE_1X1_BF16, dtype="f32")
    Xf, Ff = Xf.to(DEV), Ff.to(DEV)
    Yf = torch.empty((32, 28, 28, 512), dtype=torch.float32, device=DEV)
    Xg = torch.zeros((4, 12, 14, 128), dtype=torch.bfloat16, device=DEV)
    Fg = torch.zeros((3, 3, 16, 128), dtype=torch.bfloat16, device=DEV)
    Yg = torch.empty((4, 12, 14, 128), dtype=torch.bfloat16, device=DEV)
    calls = [lambda: cf.conv2d_nhwc(X, F, out=Y),
             lambda: cf.conv2d_nhwc(Xp, Fp, out=Yp),
             lambda: cf.conv2d_nhwc(Xf, Ff, out=Yf),
             lambda: cf.conv2d_nhwc(Xg, Fg, out=Yg, padding=1, groups=8),
             lambda: cf.conv2d_nhwc(X[:, 1:, 1:], F, out=Y[:, :55, :55], variant=cf.VARIANT_DIRECT),
             lambda: cf.conv_depthwise(Xd, wd, stride=2, padding=2, exact=True, out=Yd)]
    for c in calls:
        c()
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    for _ in range(5):
        for c in calls:
            c()
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert free1 == free0
