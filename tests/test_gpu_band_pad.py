"""Parity of the band kernel (dense 3x3, unit stride, bf16 in and out) and of
the padded depthwise kernel (zero border staged in LDS) at the edges of
their tilings, against the CPU oracle.

Dense bf16: 2e-2 relative to the output RMS, plus the per-element bound on
round-to-nearest of an fp32 accumulation (``parity.bf16_rounding_ok``);
integer-valued inputs bitwise. Depthwise: bitwise (exact mode everywhere,
fast mode except NaN payloads).
"""
import numpy as np
import pytest
import torch

import convolution_forward_amd as cf
import oracle
import workloads as wl
from parity import BF16_RMS_REL, abs_sum_dense, bf16_rounding_ok, bits, rms_rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

# --- band kernel ----------------------------------------------------------------

# N, H, W, Cin, Cout, pad, groups, bias. The band height follows from
# N * channel tiles: 16 images x 2 tiles give 3-row bands (the last one of 2
# rows), 32 x 1 give 7-row bands (the last one of 6).
BAND = [
    (16, 25, 25, 64, 128, 0, 1, False),    # bands of 3 rows, ragged last band, two channel tiles
    (32, 16, 12, 64, 64, 1, 1, True),      # bands of 7 rows over 16 (7, 7, 2), same padding, bias
    (2, 9, 64, 64, 64, 0, 1, False),       # 62 output columns: 64 staged pixel slots, the most one row holds
    (2, 9, 62, 64, 64, 1, 1, False),       # the same width reached through the padding
    (3, 10, 30, 32, 40, 1, 1, True),       # one 32-channel step, partial channel tile
    (2, 8, 20, 24, 16, 0, 1, False),       # channels padded up to the step (24 of 32)
    (2, 11, 19, 48, 72, 1, 1, False),      # 48 of 64 channels, a second tile of 8
    (4, 12, 14, 128, 128, 1, 8, True),     # 8 groups of 16 packed block-diagonally
    (2, 10, 10, 64, 64, 1, 2, False),      # 2 groups of 32 packed
    (4, 12, 14, 128, 128, 1, 16, False),   # 16 groups of 8 packed: each wave runs one channel step per tap
    (3, 9, 20, 128, 128, 0, 4, True),      # 4 groups of 32 over two packed tiles
    (1, 3, 5, 64, 64, 0, 1, False),        # one output row, three pixels
]


@pytest.mark.parametrize("case", BAND)
def test_gpu_band_kernel_shapes(case):
    N, H, W, C, O, pad, groups, has_bias = case
    seed = 7000 + BAND.index(case)
    X = wl.random_tensor((N, H, W, C), seed).to(torch.bfloat16)
    F = (wl.random_tensor((3, 3, C // groups, O), seed + 1) * (1.0 / (9 * C / groups) ** 0.5)).to(torch.bfloat16)
    b = wl.random_tensor((O,), seed + 2) if has_bias else None
    assert cf.dense_variant_for(X.to(DEV), F.to(DEV), padding=pad, groups=groups,
                                bias=None if b is None else b.to(DEV)) == cf.VARIANT_TILED
    ref = oracle.conv2d_nhwc(X, F, bias=b, padding=pad, groups=groups)
    y = cf.conv2d_nhwc(X.to(DEV), F.to(DEV), bias=None if b is None else b.to(DEV), padding=pad, groups=groups)
    torch.cuda.synchronize()
    assert y.dtype == torch.bfloat16
    assert rms_rel_err(y, ref) <= BF16_RMS_REL
    absref = abs_sum_dense(oracle, X, F, bias=b, padding=pad, groups=groups)
    assert bf16_rounding_ok(y, ref, absref, 9 * C // groups)


def test_gpu_band_kernel_integer_bitwise():
    """Small integers: every partial sum is exact in fp32 and every output
    fits bf16's 8 significant bits, so any summation order gives the oracle's
    bits."""
    g = torch.Generator().manual_seed(7100)
    X = torch.randint(-1, 2, (32, 16, 12, 64), generator=g).to(torch.bfloat16)
    F = torch.randint(-1, 2, (3, 3, 64, 64), generator=g).to(torch.bfloat16)
    ref = oracle.conv2d_nhwc(X, F, padding=1)
    assert np.max(np.abs(ref)) <= 256
    y = cf.conv2d_nhwc(X.to(DEV), F.to(DEV), padding=1)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(y.float().cpu().numpy(), ref.astype(np.float32))


@pytest.mark.parametrize("groups", [4, 8, 16])
def test_gpu_band_kernel_grouped_integer_bitwise(groups):
    """Packed small groups (32, 16 and 8 channels), bf16 and fp32 outputs:
    integer-valued sums are exact whatever the order, so every output must
    equal the oracle's per-group sum, and no group may see another's input
    channels or weights."""
    g = torch.Generator().manual_seed(7150 + groups)
    X = torch.randint(-2, 3, (4, 11, 13, 128), generator=g).to(torch.bfloat16)
    F = torch.randint(-1, 2, (3, 3, 128 // groups, 128), generator=g).to(torch.bfloat16)
    ref = oracle.conv2d_nhwc(X, F, padding=1, groups=groups)
    assert np.max(np.abs(ref)) <= 256
    for odt in (torch.bfloat16, torch.float32):
        out = torch.full((4, 11, 13, 128), float("nan"), dtype=odt, device=DEV)
        assert cf.dense_variant_for(X.to(DEV), F.to(DEV), padding=1, groups=groups, out=out) == cf.VARIANT_TILED
        y = cf.conv2d_nhwc(X.to(DEV), F.to(DEV), padding=1, groups=groups, out=out)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(y.float().cpu().numpy(), ref.astype(np.float32))


def test_gpu_band_kernel_packed_groups_nonfinite_input():
    """An infinite input value in group 0. With 32-channel groups each wave's
    channel step holds one group only, so every output of groups 1-3 equals
    the oracle's (finite) value. With 16-channel groups, group 1 shares
    group 0's 32-channel step (its filter zeros meet the infinity: NaN near
    that pixel, the documented deviation from the per-group sum); groups 2-7
    are unaffected."""
    for groups in (4, 8):
        G = 128 // groups
        g = torch.Generator().manual_seed(7180 + groups)
        X = torch.randint(-2, 3, (2, 9, 11, 128), generator=g).to(torch.bfloat16)
        F = torch.randint(-1, 2, (3, 3, G, 128), generator=g).to(torch.bfloat16)
        X[1, 4, 5, 3] = float("inf")                     # channel 3: group 0
        ref = oracle.conv2d_nhwc(X, F, padding=1, groups=groups)
        out = torch.empty((2, 9, 11, 128), dtype=torch.float32, device=DEV)   # integer sums: exact in fp32
        y = cf.conv2d_nhwc(X.to(DEV), F.to(DEV), padding=1, groups=groups, out=out).cpu().numpy()
        torch.cuda.synchronize()
        clean = slice(G, 128) if groups == 4 else slice(2 * G, 128)
        np.testing.assert_array_equal(y[..., clean], ref[..., clean].astype(np.float32))
        assert np.isfinite(ref[..., G:]).all()
        # group 0: non-finite exactly where the oracle is non-finite, equal elsewhere
        r0, y0 = ref[..., :G], y[..., :G]
        np.testing.assert_array_equal(np.isfinite(y0), np.isfinite(r0))
        np.testing.assert_array_equal(y0[np.isfinite(r0)], r0[np.isfinite(r0)].astype(np.float32))
        if groups == 8:
            # the partner group: finite and exact away from the infinite input's window
            y1 = y[..., G:2 * G]
            near = np.zeros(y1.shape[:3], dtype=bool)
            near[1, 3:6, 4:7] = True
            assert np.isfinite(y1[~near]).all()
            np.testing.assert_array_equal(y1[~near], ref[..., G:2 * G][~near].astype(np.float32))


def test_gpu_band_kernel_repeat_and_coverage():
    """Every output written (Y starts as NaN) and identical bits on a rerun."""
    X = wl.random_tensor((16, 25, 25, 64), 7200).to(torch.bfloat16).to(DEV)
    F = (wl.random_tensor((3, 3, 64, 128), 7201) * 0.04).to(torch.bfloat16).to(DEV)
    out = torch.full((16, 23, 23, 128), float("nan"), dtype=torch.bfloat16, device=DEV)
    y1 = cf.conv2d_nhwc(X, F, out=out).clone()
    assert not torch.isnan(y1.float()).any()
    y2 = cf.conv2d_nhwc(X, F)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


# --- padded depthwise kernel -----------------------------------------------------

PADDED = [  # N, C, H, W, K, stride, pad, bias
    (3, 37, 7, 8, 5, 1, 2, False),         # whole planes, last tile partly empty
    (2, 3, 61, 44, 5, 2, 2, True),         # stride 2, odd height, ragged row bands
    (1, 4, 33, 32, 3, 2, 0, False),        # stride 2, no padding: the last input row is never read
    (2, 5, 12, 12, 5, 1, 4, False),        # padding 4 (the widest border kept in LDS)
    (1, 3, 9, 16, 3, 1, 2, True),          # padding 2 on a 3x3 window
    (1, 2, 120, 64, 3, 1, 1, False),       # bands of rows, last one ragged
    (4, 6, 28, 28, 5, 1, 2, True),         # the 28x28 layer shape, bias
    (2, 8, 56, 56, 5, 2, 2, False),        # the exact-mode workload's plane shape
    (1, 3, 40, 136, 5, 2, 2, True),        # stride 2 with 68 output columns (rows past 64 stay on this kernel)
]


def _dw(x, w, bias, stride, padding, mode, out=None):
    y = cf.conv_depthwise(x.to(DEV), w.to(DEV), bias=None if bias is None else bias.to(DEV), stride=stride,
                          padding=padding, exact=(mode == "exact"), out=out)
    torch.cuda.synchronize()
    return y


def _assert_bits(y, ref, mode):
    g, r = bits(y), bits(ref)
    if mode == "exact":
        np.testing.assert_array_equal(g, r)
    else:
        gn, rn = np.isnan(y.cpu().numpy()), np.isnan(ref)
        np.testing.assert_array_equal(gn, rn)
        np.testing.assert_array_equal(g[~gn], r[~rn])


@pytest.mark.parametrize("case", PADDED)
@pytest.mark.parametrize("mode", ["exact", "fast"])
def test_gpu_dw_padded_kernel_bitwise(case, mode):
    N, C, H, W, K, s, p, has_bias = case
    seed = 7300 + PADDED.index(case)
    X = wl.random_tensor((N, C, H, W), seed)
    w = wl.random_tensor((C, K, K), seed + 1)
    b = wl.random_tensor((C,), seed + 2) if has_bias else None
    assert cf.depthwise_variant_for(X.to(DEV), w.to(DEV), s, p) == cf.VARIANT_TILED
    ref = oracle.depthwise_nchw(X, w, bias=b, stride=s, padding=p, mode=mode)
    _assert_bits(_dw(X, w, b, s, p, mode), ref, mode)


@pytest.mark.parametrize("mode", ["exact", "fast"])
def test_gpu_dw_padded_kernel_special_values(mode):
    """NaNs with payloads, infinities, signed zeros and subnormals in X and w,
    an infinite weight whose taps reach the zero border (inf * +0 = NaN, which
    exact mode canonicalises)."""
    rng = np.random.default_rng(7400)
    specials = np.array([0x7FC00000, 0xFFC12345, 0x7F800000, 0xFF800000, 0x00000000, 0x80000000, 0x00000001,
                         0x807FFFFF], dtype=np.uint32)
    X = wl.random_tensor((2, 4, 16, 16), 7401).numpy().view(np.uint32).copy()
    picks = rng.choice(X.size, size=X.size // 30, replace=False)
    X.reshape(-1)[picks] = specials[rng.integers(0, specials.size, size=picks.size)]
    X = torch.from_numpy(X.view(np.float32))
    w = wl.random_tensor((4, 5, 5), 7402)
    w[1, 0, 0] = float("inf")
    w[2, 4, 4] = float("-inf")
    b = wl.random_tensor((4,), 7403)
    for s, p in [(1, 2), (2, 2), (1, 1)]:
        ref = oracle.depthwise_nchw(X, w, bias=b, stride=s, padding=p, mode=mode)
        _assert_bits(_dw(X, w, b, s, p, mode), ref, mode)


def test_gpu_dw_padded_kernel_coverage_and_repeat():
    X = wl.random_tensor((3, 37, 7, 8), 7500)
    w = wl.random_tensor((37, 5, 5), 7501)
    out = torch.full((3, 37, 7, 8), float("nan"), device=DEV)
    y1 = _dw(X, w, None, 1, 2, "fast", out=out).clone()
    assert not torch.isnan(y1).any()
    y2 = _dw(X, w, None, 1, 2, "fast")
    assert torch.equal(y1.view(torch.int32), y2.view(torch.int32))


# --- pointwise (1x1) GEMM kernel ------------------------------------------------

POINTWISE = [  # N, H, W, Cin, Cout, out dtype, bias, pixel stride of X (None: contiguous)
    (2, 7, 11, 256, 136, torch.bfloat16, False, None),   # 154 pixels: a ragged last block, a partial channel tile
    (4, 10, 13, 256, 512, torch.bfloat16, True, None),   # four channel tiles, bias
    (1, 5, 9, 128, 64, torch.bfloat16, False, None),     # two 32-channel steps per filter half
    (2, 7, 11, 256, 136, torch.float32, True, None),     # fp32 output straight from the accumulators
    (8, 28, 28, 256, 128, torch.bfloat16, False, None),  # 6272 pixels: many tiles of up to 28 blocks
    (2, 6, 10, 128, 72, torch.bfloat16, False, 200),     # X pixels 200 channels apart (a channel slice)
]


@pytest.mark.parametrize("case", POINTWISE)
def test_gpu_pointwise_kernel(case):
    N, H, W, C, O, odt, has_bias, xstride = case
    seed = 7600 + POINTWISE.index(case)
    base = wl.random_tensor((N, H, W, xstride or C), seed).to(torch.bfloat16)
    X = base[..., :C]
    F = (wl.random_tensor((1, 1, C, O), seed + 1) * (1.0 / C ** 0.5)).to(torch.bfloat16)
    b = wl.random_tensor((O,), seed + 2) if has_bias else None
    ref = oracle.conv2d_nhwc(X, F, bias=b)
    y = cf.conv2d_nhwc(base.to(DEV)[..., :C], F.to(DEV), bias=None if b is None else b.to(DEV), out_dtype=odt)
    torch.cuda.synchronize()
    assert y.dtype == odt
    if odt == torch.float32:
        from parity import max_rel_err
        assert max_rel_err(y, ref) <= 1e-5
    else:
        assert rms_rel_err(y, ref) <= BF16_RMS_REL
        assert bf16_rounding_ok(y, ref, abs_sum_dense(oracle, X, F, bias=b), C)


def test_gpu_pointwise_kernel_integer_bitwise():
    g = torch.Generator().manual_seed(7700)
    X = torch.randint(-1, 2, (4, 12, 13, 256), generator=g).to(torch.bfloat16)
    F = torch.randint(-1, 2, (1, 1, 256, 256), generator=g).to(torch.bfloat16)
    ref = oracle.conv2d_nhwc(X, F)
    assert np.max(np.abs(ref)) <= 256
    y = cf.conv2d_nhwc(X.to(DEV), F.to(DEV))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(y.float().cpu().numpy(), ref.astype(np.float32))
