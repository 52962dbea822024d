"""Pins for the CPU oracle: the pages' worked examples, closed forms,
invariants, library cross-checks and exact brute force on tiny inputs.

Nothing here needs a GPU. Each test names the passage it follows.
"""
import math

import numpy as np
import pytest
import torch

from conftest import golden
import fp32_exact as fx
from workloads import random_tensor


def nhwc(a2d):
    """A 2D single-channel image as an NHWC array [1,H,W,1]."""
    a = np.asarray(a2d, dtype=np.float32)
    return a.reshape(1, a.shape[0], a.shape[1], 1)


def kkio(k2d):
    k = np.asarray(k2d, dtype=np.float32)
    return k.reshape(k.shape[0], k.shape[1], 1, 1)


# --- worked examples -----------------------------------------------------------

def test_lecture_arange_example(oracle_mod):
    """CMU DLSys Lecture 14, section 4: arange(36) image, arange(9) filter."""
    g = golden("lecture14_arange_patches.json")
    A = np.arange(36, dtype=np.float32).reshape(6, 6)
    Fk = np.arange(9, dtype=np.float32).reshape(3, 3)
    Y = oracle_mod.conv2d_nhwc(nhwc(A), kkio(Fk))
    assert Y.shape == (1, 4, 4, 1)
    np.testing.assert_array_equal(Y[0, :, :, 0], np.array(g["output"], dtype=np.float64))
    # Closed form derived from the index contract: Y[y,x] = Y[0,0] + 36x + 216y,
    # since sum_{i,j}(3i+j) = 36 and the row stride of A is 6.
    yy, xx = np.meshgrid(np.arange(4), np.arange(4), indexing="ij")
    np.testing.assert_array_equal(Y[0, :, :, 0], 366 + 36 * xx + 216 * yy)
    # The im2col route gives the same values.
    np.testing.assert_array_equal(oracle_mod.conv2d_nhwc_im2col(nhwc(A), kkio(Fk)), Y)


def test_lecture_patch_rows(oracle_mod):
    """Lecture 14, sections 4-5: each patch is one row in (i,j,c) order."""
    g = golden("lecture14_arange_patches.json")
    A = np.arange(36, dtype=np.float32).reshape(6, 6)
    cols = oracle_mod.im2col_nhwc(nhwc(A), 3, 3)
    assert list(cols.shape) == g["patch_matrix_shape"]
    np.testing.assert_array_equal(cols[0], g["patch_row_0"])
    np.testing.assert_array_equal(cols[1], g["patch_row_1"])
    assert cols.size == g["patch_values"] and A.size == g["input_values"]
    # Section 4's patch tensor from its index equation P[y, x, i, j] = A[y + i, x + j],
    # built by gathering (a copy), must equal the patch rows.
    yy, xx, ii, jj = np.meshgrid(np.arange(4), np.arange(4), np.arange(3), np.arange(3), indexing="ij")
    P = A[yy + ii, xx + jj]
    np.testing.assert_array_equal(P.reshape(16, 9), cols)
    # The same tensor as a view: the address of P[y,x,i,j] is (y+i)*row + (x+j)*col
    # bytes, so its byte strides are (row, col, row, col) and neighbouring patches
    # alias. numpy's sliding-window view is such a view; reshaping it to the
    # patch matrix has to copy.
    row, col = A.strides
    assert [row, col, row, col] == g["patch_view_byte_strides"]
    V = np.lib.stride_tricks.sliding_window_view(A, (3, 3))
    assert list(V.strides) == g["patch_view_byte_strides"]
    np.testing.assert_array_equal(V, P)
    assert V[0, 0, 0, 1] == V[0, 1, 0, 0] == A[0, 1]
    assert np.shares_memory(V, A) and not np.shares_memory(V.reshape(16, 9), A)


def test_lecture_tile_view():
    """Lecture 14, section 3: a view re-addresses, packing re-orders (the test
    harness relies on numpy strides this way for non-contiguous inputs)."""
    g = golden("lecture14_tile_view.json")
    A = np.arange(36, dtype=np.float32).reshape(6, 6)
    assert list(A.strides) == g["array"]["byte_strides"]
    T = np.lib.stride_tricks.as_strided(A, shape=(3, 3, 2, 2), strides=(48, 8, 24, 4))
    assert list(T.strides) == g["tile_view_byte_strides"]
    np.testing.assert_array_equal(T[0, 0].ravel(), g["first_tile"])
    np.testing.assert_array_equal(A.reshape(3, 3, 2, 2)[0, 0].ravel(), g["plain_reshape_first_tile"])
    Tc = np.ascontiguousarray(T)
    assert list(Tc.strides) == g["packed_byte_strides"]
    np.testing.assert_array_equal(Tc.ravel()[:8], g["packed_sequence_start"])


def test_lecture_storage_bill(oracle_mod):
    """Lecture 14, section 6: patch matrix size and expansion ratio."""
    g = golden("lecture14_storage_bill.json")
    s = g["shape"]
    X = np.zeros((s["N"], s["H"], s["W"], s["Cin"]), dtype=np.float32)
    cols = oracle_mod.im2col_nhwc(X, s["K"], s["K"])
    assert list(cols.shape) == g["patch_matrix_shape"]
    v = g["values"]
    assert X.size == v["input"] and cols.size == v["patch_matrix"]
    assert s["K"] * s["K"] * s["Cin"] * s["Cout"] == v["filter"]
    Ho = oracle_mod.out_size(s["H"], s["K"])
    assert s["N"] * Ho * Ho * s["Cout"] == v["output"]
    assert cols.size / X.size == g["rho"] == Ho * Ho * s["K"] ** 2 / (s["H"] * s["W"])
    mb = g["megabytes_f32"]
    assert X.nbytes / 1e6 == pytest.approx(mb["input"]) and cols.nbytes / 1e6 == pytest.approx(mb["patch_matrix"])
    sm = g["small_example"]
    assert sm["patch_values"] / sm["input_values"] == sm["ratio"]


def test_wxb_window_with_bias(oracle_mod):
    """'Convolution Is Wx+b', sections 'One window...' / 'The matrix connection'."""
    g = golden("wxb_1d_examples.json")["window"]
    x = np.asarray(g["x"], np.float32).reshape(1, 1, -1, 1)
    k = np.asarray(g["k"], np.float32).reshape(1, -1, 1, 1)
    b = np.asarray([g["bias"]], np.float32)
    Y = oracle_mod.conv2d_nhwc(x, k, bias=b)
    np.testing.assert_array_equal(Y.ravel(), g["y"])
    # The same window sum through the depthwise loop (one channel), both modes.
    for mode in ("exact", "fast"):
        Yd = oracle_mod.depthwise_nchw(np.asarray(g["x"], np.float32).reshape(1, 1, 1, -1),
                                       np.asarray(g["k"], np.float32).reshape(1, 1, -1), bias=b, mode=mode)
        np.testing.assert_array_equal(Yd.ravel(), g["y"])


@pytest.mark.parametrize("case", ["average", "difference", "motif"])
def test_wxb_three_1d_uses(oracle_mod, case):
    """'Convolution Is Wx+b', section 'Three ways to use the same 1D operation'."""
    g = golden("wxb_1d_examples.json")[case]
    k = [1 / 3] * 3 if case == "average" else g["k"]
    x = np.asarray(g["x"], np.float32).reshape(1, 1, -1, 1)
    Y = oracle_mod.conv2d_nhwc(x, np.asarray(k, np.float32).reshape(1, -1, 1, 1))
    tol = 1e-6 if case == "average" else 0
    np.testing.assert_allclose(Y.ravel(), g["y"], rtol=0, atol=tol)


def test_wxb_two_filter_gemm(oracle_mod):
    """'Convolution Is Wx+b', section 'The matrix connection': two filters."""
    g = golden("wxb_1d_examples.json")["two_filters"]
    x = np.asarray(g["x"], np.float32).reshape(1, 1, -1, 1)
    K = np.asarray(g["K_taps_by_filters"], np.float32).reshape(1, 3, 1, 2)
    Y = oracle_mod.conv2d_nhwc(x, K, bias=np.asarray(g["bias"], np.float32))
    np.testing.assert_array_equal(Y[0, 0], g["y_positions_by_filters"])


def test_wxb_small_2d(oracle_mod):
    """'Convolution Is Wx+b', section 'Why 1D? Why 2D?': 3x3 image, 2x2 filter."""
    g = golden("wxb_2d_examples.json")["small"]
    Y = oracle_mod.conv2d_nhwc(nhwc(g["image"]), kkio(g["filter"]))
    np.testing.assert_array_equal(Y[0, :, :, 0], g["output"])
    Yd = oracle_mod.depthwise_nchw(np.asarray(g["image"], np.float32)[None, None],
                                   np.asarray(g["filter"], np.float32)[None])
    np.testing.assert_array_equal(Yd[0, 0], g["output"])


def sobel_image():
    img = np.zeros((6, 6), np.float32)
    img[:, 3:] = 1
    return img


def test_wxb_sobel(oracle_mod):
    """'Convolution Is Wx+b', section 'Build an image-gradient map': Gx and Gy as
    two output channels of one dense conv (the [16,9] @ [9,2] view), and as a
    depthwise conv with multiplier 2."""
    g = golden("wxb_2d_examples.json")["sobel"]
    img = sobel_image()
    F = np.stack([np.asarray(g["gx"], np.float32), np.asarray(g["gy"], np.float32)], axis=-1)
    Y = oracle_mod.conv2d_nhwc(nhwc(img), F.reshape(3, 3, 1, 2))
    np.testing.assert_array_equal(Y[0, :, :, 0], g["gx_output"])
    np.testing.assert_array_equal(Y[0, :, :, 1], g["gy_output"])
    cols = oracle_mod.im2col_nhwc(nhwc(img), 3, 3)
    np.testing.assert_array_equal(cols[1], g["patch_row_at_0_1"])     # output (row 0, col 1)
    w = np.stack([np.asarray(g["gx"], np.float32), np.asarray(g["gy"], np.float32)])
    for mode in ("exact", "fast"):
        Yd = oracle_mod.depthwise_nchw(img[None, None], w, mode=mode)
        np.testing.assert_array_equal(Yd[0, 0], g["gx_output"])
        np.testing.assert_array_equal(Yd[0, 1], g["gy_output"])


def test_out_size_rule(oracle_mod):
    """'Convolution Is Wx+b', section 'Why 1D? Why 2D?': output-size rule."""
    g = golden("wxb_1d_examples.json")["out_size"]
    assert oracle_mod.out_size(g["in"], g["k"]) == g["out"]
    # The depthwise workload shapes (stride s, pad K//2).
    assert oracle_mod.out_size(56, 5, 2, 2, 1) == 28
    assert oracle_mod.out_size(112, 3, 1, 1, 1) == 112
    assert oracle_mod.out_size(112, 3, 2, 1, 1) == 56
    assert oracle_mod.out_size(14, 5, 2, 2, 1) == 7
    assert oracle_mod.out_size(7, 5, 1, 2, 1) == 7
    assert oracle_mod.out_size(7, 3, 1, 0, 3) == 1      # effective kernel 7
    assert oracle_mod.out_size(7, 3, 1, 0, 4) <= 0      # effective kernel 9 > 7


# --- invariants ----------------------------------------------------------------

SHAPES = [  # (N, H, W, Cin, K, Cout): small, non-square, distinct channels
    (1, 5, 7, 3, 3, 2), (2, 6, 4, 5, 2, 3), (2, 4, 9, 1, 1, 4), (1, 3, 3, 2, 3, 3),
    (3, 7, 5, 4, 4, 1), (1, 8, 6, 6, 1, 5),
]


@pytest.mark.parametrize("shape", SHAPES)
def test_k1_is_matmul_and_shifted_matmuls(oracle_mod, shape):
    """Lecture 14, section 2: K=1 is X @ F[0,0]; for larger K the output is the
    sum of K^2 shifted channel matmuls. Integer-valued inputs keep every sum
    exact, so any accumulation order must give identical values."""
    N, H, W, C, K, O = shape
    seed = hash(shape) & 0xFFFF
    X = random_tensor((N, H, W, C), seed, integer_range=4).numpy()
    F = random_tensor((K, K, C, O), seed + 1, integer_range=4).numpy()
    Y = oracle_mod.conv2d_nhwc(X, F)
    Ho, Wo = H - K + 1, W - K + 1
    # The K^2 shifted copies of X stacked on a tap axis (shift (i, j) holds
    # X[n, y+i, x+j, :]), each contracted over channels with F[i, j] and summed
    # over the taps in one tensordot.
    shifted = np.stack([np.roll(X, (-i, -j), axis=(1, 2))[:, :Ho, :Wo, :]
                        for i in range(K) for j in range(K)], axis=3).astype(np.float64)
    ref = np.tensordot(shifted, F.reshape(K * K, C, O).astype(np.float64), axes=([3, 4], [0, 1]))
    np.testing.assert_array_equal(Y, ref)
    np.testing.assert_array_equal(oracle_mod.conv2d_nhwc_im2col(X, F), Y)
    X1 = X.astype(np.float64).reshape(-1, C) @ F[0, 0].astype(np.float64)
    np.testing.assert_array_equal(oracle_mod.conv2d_nhwc(X, F[:1, :1]).reshape(-1, O), X1)


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_full_image_filter(oracle_mod, seed):
    """Lecture 14, section 5 test advice: a square input whose filter spans the
    whole image gives one output per image, X[n].ravel() @ F.reshape(-1, O)."""
    N, S, C, O = 2, 5, 3, 4
    X = random_tensor((N, S, S, C), seed).numpy()
    F = random_tensor((S, S, C, O), seed + 10).numpy()
    Y = oracle_mod.conv2d_nhwc(X, F)
    assert Y.shape == (N, 1, 1, O)
    ref = X.reshape(N, -1).astype(np.float64) @ F.reshape(-1, O).astype(np.float64)
    np.testing.assert_allclose(Y[:, 0, 0, :], ref, rtol=1e-13, atol=1e-13)


GENERAL = [  # (N,H,W,Cin,KH,KW,Cout, stride, pad, dil, groups)
    (2, 7, 9, 3, 3, 3, 4, 1, 0, 1, 1),
    (1, 8, 6, 4, 3, 2, 6, 2, 1, 1, 2),
    (2, 9, 9, 6, 3, 3, 6, 1, 2, 2, 3),
    (1, 10, 7, 4, 5, 5, 4, (2, 1), (2, 1), 1, 4),
    (1, 6, 5, 2, 1, 3, 3, 1, (0, 1), (1, 2), 1),
]


@pytest.mark.parametrize("case", GENERAL)
def test_dense_matches_torch_conv2d(oracle_mod, case):
    """Lecture 14, section 1: a library comparison converts NHWC inputs with
    transpose(0,3,1,2) and KKIO filters with transpose(3,2,0,1). torch's CPU
    conv2d in fp64 must agree with the loops, including the stride / padding /
    dilation / groups superset."""
    N, H, W, C, KH, KW, O, s, p, d, g = case
    X = random_tensor((N, H, W, C), 7).numpy()
    F = random_tensor((KH, KW, C // g, O), 8).numpy()
    b = random_tensor((O,), 9).numpy()
    Y = oracle_mod.conv2d_nhwc(X, F, bias=b, stride=s, padding=p, dilation=d, groups=g)
    xt = torch.from_numpy(X).double().permute(0, 3, 1, 2)
    ft = torch.from_numpy(F).double().permute(3, 2, 0, 1)
    ref = torch.nn.functional.conv2d(xt, ft, torch.from_numpy(b).double(), stride=s, padding=p,
                                     dilation=d, groups=g).permute(0, 2, 3, 1).numpy()
    np.testing.assert_allclose(Y, ref, rtol=1e-12, atol=1e-12)


def test_dense_noncontiguous_input(oracle_mod):
    """Lecture 14, section 5: the patch view uses the actual input strides, so
    sliced or transposed inputs keep their logical meaning."""
    base = random_tensor((2, 9, 11, 8), 21).numpy()
    F = random_tensor((3, 3, 3, 5), 22).numpy()
    views = [base[:, 1:8, 2:10, 1:4],                          # sliced, channel stride 1
             base[:, ::2, ::2, ::2][..., :3],                  # stepped, channel stride 2
             np.ascontiguousarray(base[..., :3].transpose(0, 2, 1, 3)).transpose(0, 2, 1, 3)]
    for v in views:
        assert not v.flags["C_CONTIGUOUS"]
        np.testing.assert_array_equal(oracle_mod.conv2d_nhwc(v, F), oracle_mod.conv2d_nhwc(np.ascontiguousarray(v), F))


def test_dense_translation_equivariance(oracle_mod):
    """'Convolution Is Wx+b', section 'Why convolution is still important':
    at stride 1, shifting the input by one pixel shifts the response by one,
    away from the borders."""
    X = random_tensor((1, 9, 10, 3), 31).numpy()
    F = random_tensor((3, 3, 3, 2), 32).numpy()
    Xs = np.zeros_like(X)
    Xs[:, 1:, 1:, :] = X[:, :-1, :-1, :]
    Y, Ys = oracle_mod.conv2d_nhwc(X, F), oracle_mod.conv2d_nhwc(Xs, F)
    np.testing.assert_array_equal(Ys[:, 1:, 1:, :], Y[:, :-1, :-1, :])


AT_CASES = [  # (N,H,W,Cin,KH,KW,Cout, stride, pad, dil, groups, bias)
    (2, 7, 6, 5, 2, 3, 3, 1, 0, 1, 1, False),
    (2, 9, 8, 4, 3, 3, 6, 1, 1, 1, 1, True),             # same padding
    (1, 11, 10, 6, 3, 3, 4, 2, 1, 1, 2, True),           # stride 2, groups
    (2, 10, 9, 4, 3, 2, 4, (2, 1), (2, 0), (2, 1), 4, False),  # unequal stride / pad, dilation, depthwise-like groups
    (1, 1, 23, 6, 1, 3, 5, (1, 2), (0, 1), 1, 1, True),  # strided Conv1D stem shape
    (3, 8, 8, 8, 5, 5, 8, 1, 2, 2, 8, False),            # 5x5 dilated depthwise as groups
]


@pytest.mark.parametrize("case", AT_CASES)
def test_dense_sampled_equals_full(oracle_mod, case):
    """The sampled form is the same sum at chosen indices: equal to the full
    loops on every output index, over the stride / padding / dilation / groups
    / bias superset, for indices given in any order and with repeats, and on
    a strided (non-contiguous) input view."""
    N, H, W, C, KH, KW, O, s, p, d, g, has_bias = case
    seed = hash(case) & 0xFFFF
    base = random_tensor((N, H, W, C + 3), seed).numpy()
    X = base[..., 1:C + 1]
    F = random_tensor((KH, KW, C // g, O), seed + 1).numpy()
    b = random_tensor((O,), seed + 2).numpy() if has_bias else None
    Y = oracle_mod.conv2d_nhwc(X, F, bias=b, stride=s, padding=p, dilation=d, groups=g)
    idx = np.arange(Y.size, dtype=np.int64)
    got = oracle_mod.conv2d_nhwc_at(X, F, idx, bias=b, stride=s, padding=p, dilation=d, groups=g)
    np.testing.assert_array_equal(got, Y.ravel())
    perm = np.random.default_rng(seed).permutation(Y.size)
    perm = np.concatenate([perm, perm[:7]])
    got = oracle_mod.conv2d_nhwc_at(X, F, perm, bias=b, stride=s, padding=p, dilation=d, groups=g)
    np.testing.assert_array_equal(got, Y.ravel()[perm])


# --- depthwise -----------------------------------------------------------------

def brute_depthwise(X, w, bias, stride, pad, dil, mode):
    """Exact-rational brute force of the depthwise output definition
    ("Depthwise convolution", section 'What each output is')."""
    N, C, H, W = X.shape
    Cout, KH, KW = w.shape
    mult = Cout // C
    sh, sw = stride
    ph, pw = pad
    dh, dw = dil
    Ho = (H + 2 * ph - (dh * (KH - 1) + 1)) // sh + 1
    Wo = (W + 2 * pw - (dw * (KW - 1) + 1)) // sw + 1
    out = np.empty((N, Cout, Ho, Wo), np.float32)
    for n in range(N):
        for oc in range(Cout):
            ic = oc // mult
            for oy in range(Ho):
                for ox in range(Wo):
                    acc = 0.0
                    for ky in range(KH):
                        for kx in range(KW):
                            r, c = oy * sh + ky * dh - ph, ox * sw + kx * dw - pw
                            xv = float(X[n, ic, r, c]) if (0 <= r < H and 0 <= c < W) else 0.0
                            wv = float(w[oc, ky, kx])
                            if mode == "exact":
                                acc = fx.add(acc, fx.mul(wv, xv))
                            else:
                                acc = fx.fma(wv, xv, acc)
                    if bias is not None:
                        acc = fx.add(acc, float(bias[oc]))
                    if mode == "exact" and math.isnan(acc):
                        acc = fx.from_bits(0x7FC00000)
                    out[n, oc, oy, ox] = acc
    return out


DW_CASES = [  # (N,C,H,W, mult, KH,KW, stride, pad, dil, bias)
    (1, 2, 5, 6, 1, 3, 3, (1, 1), (1, 1), (1, 1), False),
    (2, 1, 7, 5, 2, 3, 2, (2, 1), (1, 0), (1, 1), True),
    (1, 3, 6, 7, 1, 5, 5, (2, 2), (2, 2), (1, 1), False),
    (1, 2, 8, 8, 3, 3, 3, (1, 2), (2, 2), (2, 2), True),
    (1, 1, 9, 4, 1, 2, 3, (3, 3), (0, 1), (1, 1), False),
]


@pytest.mark.parametrize("case", DW_CASES)
@pytest.mark.parametrize("mode", ["exact", "fast"])
def test_depthwise_bitwise_brute_force(oracle_mod, case, mode):
    """Depthwise oracle vs an exact-rational model of each fp32 step; bits must match."""
    N, C, H, W, m, KH, KW, s, p, d, has_bias = case
    seed = hash(case) & 0xFFFF
    X = random_tensor((N, C, H, W), seed).numpy()
    w = random_tensor((C * m, KH, KW), seed + 1).numpy()
    b = random_tensor((C * m,), seed + 2).numpy() if has_bias else None
    got = oracle_mod.depthwise_nchw(X, w, bias=b, stride=s, padding=p, dilation=d, mode=mode)
    ref = brute_depthwise(X, w, b, s, p, d, mode)
    np.testing.assert_array_equal(got.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("mode", ["exact", "fast"])
def test_depthwise_subnormal_bitwise(oracle_mod, mode):
    """Products and sums in the subnormal range keep IEEE gradual underflow."""
    X = (random_tensor((1, 2, 6, 6), 51).numpy() * np.float32(2.0 ** -70)).astype(np.float32)
    w = (random_tensor((2, 3, 3), 52).numpy() * np.float32(2.0 ** -70)).astype(np.float32)
    got = oracle_mod.depthwise_nchw(X, w, padding=1, mode=mode)
    ref = brute_depthwise(X, w, None, (1, 1), (1, 1), (1, 1), mode)
    assert np.any((got != 0) & (np.abs(got) < np.finfo(np.float32).tiny))    # subnormals occur
    np.testing.assert_array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_depthwise_exact_vs_fast_rounding(oracle_mod):
    """Exact mode rounds the product before the sum; fast mode fuses them.
    Taps (w, x): (-1, 1) then (1+2^-12, 1+2^-12). The second product is
    1 + 2^-11 + 2^-24, a tie that rounds to 1 + 2^-11, so exact mode gives
    2^-11 while the fused form keeps 2^-11 + 2^-24."""
    a = np.float32(1 + 2.0 ** -12)
    X = np.array([1, a], np.float32).reshape(1, 1, 1, 2)
    w = np.array([-1, a], np.float32).reshape(1, 1, 2)
    assert oracle_mod.depthwise_nchw(X, w, mode="exact").item() == 2.0 ** -11
    assert oracle_mod.depthwise_nchw(X, w, mode="fast").item() == 2.0 ** -11 + 2.0 ** -24


def bits(a):
    return np.asarray(a, np.float32).view(np.uint32)


def test_depthwise_special_values_exact(oracle_mod):
    """'Depthwise convolution', section 'What each output is': padding is a real
    zero (an infinite weight meeting it gives NaN), NaN results are rewritten to
    0x7FC00000, and an accumulator that starts at +0 never ends at -0."""
    nan_payload = fx.from_bits(0xFFC12345)           # negative NaN with a payload
    X = np.array([[1.0, 2.0, 3.0], [4.0, nan_payload, 6.0], [7.0, 8.0, 9.0]], np.float32)[None, None]
    w = np.ones((1, 3, 3), np.float32)
    Y = oracle_mod.depthwise_nchw(X, w, padding=1, mode="exact")
    assert np.all(bits(Y) == 0x7FC00000)                 # every window sees the centre NaN
    # An infinite weight in a corner tap: only windows whose corner is padding get NaN.
    X = np.ones((1, 1, 3, 3), np.float32)
    w = np.zeros((1, 3, 3), np.float32)
    w[0, 0, 0] = np.inf
    Y = oracle_mod.depthwise_nchw(X, w, padding=1, mode="exact")
    assert bits(Y)[0, 0, 0, 0] == 0x7FC00000                  # corner tap is padding: inf * 0
    assert Y[0, 0, 1, 1] == np.inf                            # corner tap reads X = 1
    # +inf + -inf cancels to NaN.
    X = np.array([[1.0, 1.0]], np.float32)[None, None]
    w = np.array([[[np.inf, -np.inf]]], np.float32)
    assert bits(oracle_mod.depthwise_nchw(X, w, mode="exact")).item() == 0x7FC00000
    # Negative weights times +0 inputs give -0 products; +0 + -0 = +0.
    X = np.zeros((1, 1, 3, 3), np.float32)
    w = -np.ones((1, 2, 2), np.float32)
    Y = oracle_mod.depthwise_nchw(X, w, mode="exact")
    assert np.all(bits(Y) == 0)
    # Fast mode: NaN stays NaN (payload unspecified) and padding still multiplies.
    Yf = oracle_mod.depthwise_nchw(np.ones((1, 1, 3, 3), np.float32),
                                   np.where(np.arange(9).reshape(1, 3, 3) == 0, np.inf, 0).astype(np.float32),
                                   padding=1, mode="fast")
    assert np.isnan(Yf[0, 0, 0, 0]) and Yf[0, 0, 1, 1] == np.inf


@pytest.mark.parametrize("case", DW_CASES)
def test_depthwise_equals_block_diagonal_dense(oracle_mod, case):
    """'Depthwise convolution': groups == C, output channel oc reads input
    channel oc / mult. So depthwise equals the dense conv with the
    block-diagonal filter F[i,j,c,o] = w[o,i,j] * [c == o // mult], and the
    grouped dense conv with groups = C. Integer inputs keep every sum exact."""
    N, C, H, W, m, KH, KW, s, p, d, has_bias = case
    seed = (hash(case) & 0xFFFF) + 5
    X = random_tensor((N, C, H, W), seed, integer_range=3).numpy()
    w = random_tensor((C * m, KH, KW), seed + 1, integer_range=3).numpy()
    b = random_tensor((C * m,), seed + 2, integer_range=3).numpy() if has_bias else None
    Xn = np.ascontiguousarray(X.transpose(0, 2, 3, 1))
    Fblock = np.zeros((KH, KW, C, C * m), np.float32)
    for o in range(C * m):
        Fblock[:, :, o // m, o] = w[o]
    Fgroup = np.ascontiguousarray(w.transpose(1, 2, 0)[:, :, None, :])
    for mode in ("exact", "fast"):
        Yd = oracle_mod.depthwise_nchw(X, w, bias=b, stride=s, padding=p, dilation=d, mode=mode)
        for F, g in ((Fblock, 1), (Fgroup, C)):
            Yn = oracle_mod.conv2d_nhwc(Xn, F, bias=b, stride=s, padding=p, dilation=d, groups=g)
            np.testing.assert_array_equal(Yd, Yn.transpose(0, 3, 1, 2).astype(np.float32))


@pytest.mark.parametrize("case", DW_CASES)
def test_depthwise_matches_torch(oracle_mod, case):
    """torch's CPU conv2d with groups = C and weights viewed as [Cout,1,KH,KW]."""
    N, C, H, W, m, KH, KW, s, p, d, has_bias = case
    X = random_tensor((N, C, H, W), 61).numpy()
    w = random_tensor((C * m, KH, KW), 62).numpy()
    b = random_tensor((C * m,), 63).numpy() if has_bias else None
    ref = torch.nn.functional.conv2d(torch.from_numpy(X).double(),
                                     torch.from_numpy(w).double().view(C * m, 1, KH, KW),
                                     None if b is None else torch.from_numpy(b).double(),
                                     stride=s, padding=p, dilation=d, groups=C).numpy()
    for mode in ("exact", "fast"):
        got = oracle_mod.depthwise_nchw(X, w, bias=b, stride=s, padding=p, dilation=d, mode=mode)
        np.testing.assert_allclose(got, ref, rtol=1e-5, atol=1e-5)


# --- the window superset: each property reduces it to the lecture's operator ----

WINDOW_SHAPES = [  # (N, H, W, Cin, KH, KW, Cout)
    (1, 9, 7, 3, 3, 3, 2), (2, 6, 11, 2, 2, 3, 3), (1, 12, 12, 4, 5, 5, 1),
]


def _int_inputs(shape, seed):
    N, H, W, C, KH, KW, O = shape
    X = random_tensor((N, H, W, C), seed, integer_range=4).numpy()
    F = random_tensor((KH, KW, C, O), seed + 1, integer_range=4).numpy()
    return X, F


@pytest.mark.parametrize("shape", WINDOW_SHAPES)
def test_padding_is_explicit_zero_rows_and_columns(oracle_mod, shape):
    """'Convolution Is Wx+b', section 'Why 1D? Why 2D?': padding inserts zeros
    at the edges. The padded conv equals the unpadded conv of the input with
    the zero rows and columns written out (numpy's pad), for each of the four
    sides separately and together. Integer inputs keep the sums exact."""
    X, F = _int_inputs(shape, 31)
    for ph, pw in [(1, 0), (0, 2), (2, 1), (3, 3)]:
        Xp = np.pad(X, ((0, 0), (ph, ph), (pw, pw), (0, 0)))
        np.testing.assert_array_equal(oracle_mod.conv2d_nhwc(X, F, padding=(ph, pw)),
                                      oracle_mod.conv2d_nhwc(Xp, F))


@pytest.mark.parametrize("shape", WINDOW_SHAPES)
def test_stride_subsamples_the_unit_stride_output(oracle_mod, shape):
    """Same section: stride chooses how far the window moves, so the strided
    output is every s-th row / column of the unit-stride output."""
    X, F = _int_inputs(shape, 32)
    full = oracle_mod.conv2d_nhwc(X, F, padding=1)
    for sh, sw in [(2, 1), (1, 3), (2, 2), (3, 2)]:
        got = oracle_mod.conv2d_nhwc(X, F, stride=(sh, sw), padding=1)
        np.testing.assert_array_equal(got, full[:, ::sh, ::sw, :])


@pytest.mark.parametrize("shape", WINDOW_SHAPES)
def test_dilation_spaces_the_taps(oracle_mod, shape):
    """Same section: dilation spaces the filter's taps apart, the same as a
    filter of d*(k-1)+1 taps with zeros between the original ones."""
    X, F = _int_inputs(shape, 33)
    KH, KW = F.shape[:2]
    for dh, dw in [(2, 1), (1, 2), (2, 2)]:
        Fd = np.zeros((dh * (KH - 1) + 1, dw * (KW - 1) + 1) + F.shape[2:], dtype=np.float32)
        Fd[::dh, ::dw] = F
        if Fd.shape[0] > X.shape[1] + 2 or Fd.shape[1] > X.shape[2] + 2:
            continue
        np.testing.assert_array_equal(oracle_mod.conv2d_nhwc(X, F, padding=1, dilation=(dh, dw)),
                                      oracle_mod.conv2d_nhwc(X, Fd, padding=1))


@pytest.mark.parametrize("groups", [2, 3, 6])
def test_groups_are_independent_dense_convs(oracle_mod, groups):
    """'Convolution Is Wx+b', section 'Find the same sum in CKE's C kernels':
    an output channel sums over its own group of input channels only. So the
    grouped conv is the concatenation of one dense conv per group, each on its
    slice of input channels and output channels."""
    N, H, W, C, K, O = 2, 7, 8, 6, 3, 12
    X = random_tensor((N, H, W, C), 34, integer_range=4).numpy()
    F = random_tensor((K, K, C // groups, O), 35, integer_range=4).numpy()
    got = oracle_mod.conv2d_nhwc(X, F, stride=2, padding=1, groups=groups)
    cg, og = C // groups, O // groups
    parts = [oracle_mod.conv2d_nhwc(np.ascontiguousarray(X[..., g * cg:(g + 1) * cg]),
                                    np.ascontiguousarray(F[..., g * og:(g + 1) * og]), stride=2, padding=1)
             for g in range(groups)]
    np.testing.assert_array_equal(got, np.concatenate(parts, axis=-1))


@pytest.mark.parametrize("P", [2, 4, 7])
def test_patch_stem_is_a_linear_map_of_flattened_patches(oracle_mod, P):
    """'Convolution Is Wx+b', section 'Images going in: two ways to make
    patches': a conv with a P x P kernel and stride P over non-overlapping
    patches equals flattening each patch (row, column, channel) and applying
    the [P*P*Cin, D] weight matrix."""
    N, Hp, Wp, C, D = 2, 3, 4, 3, 5
    X = random_tensor((N, Hp * P, Wp * P, C), 36).numpy()
    F = random_tensor((P, P, C, D), 37).numpy()
    got = oracle_mod.conv2d_nhwc(X, F, stride=P)
    patches = X.reshape(N, Hp, P, Wp, P, C).transpose(0, 1, 3, 2, 4, 5).reshape(N, Hp, Wp, P * P * C)
    ref = patches.astype(np.float64) @ F.reshape(P * P * C, D).astype(np.float64)
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-13)


def test_causal_conv1d_is_left_padding(oracle_mod):
    """'Convolution Is Wx+b', section 'Where this shows up in models I work
    with' (causal Conv1D): output t sees inputs t-(K-1)*d .. t only. With the
    signal on the width axis that is K-1 (times dilation) zero columns before
    it and none after, and the first L outputs of the symmetric padding."""
    L, C, K, O, d = 11, 3, 4, 2, 2
    X = random_tensor((1, 1, L, C), 38, integer_range=4).numpy()
    F = random_tensor((1, K, C, O), 39, integer_range=4).numpy()
    pad = d * (K - 1)
    left = oracle_mod.conv2d_nhwc(np.pad(X, ((0, 0), (0, 0), (pad, 0), (0, 0))), F, dilation=(1, d))
    assert left.shape == (1, 1, L, O)
    sym = oracle_mod.conv2d_nhwc(X, F, padding=(0, pad), dilation=(1, d))
    np.testing.assert_array_equal(left, sym[:, :, :L, :])
    # brute force of the causal definition
    ref = np.zeros((L, O))
    for t in range(L):
        for k in range(K):
            src = t - (K - 1 - k) * d
            if src >= 0:
                ref[t] += X[0, 0, src].astype(np.float64) @ F[0, k].astype(np.float64)
    np.testing.assert_array_equal(left[0, 0], ref)
