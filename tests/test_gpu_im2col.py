"""The explicit patch matrix (the im2col route's packing step) on the GPU.

"CMU DLSys Lecture 14", sections 4-7: the matrix holds, for every output
position, the K*K*Cin input values it reads in (i, j, c) order; section 6
gives its size. The GPU matrix is a copy, so it must equal the oracle's bit
for bit; with a window it must reproduce the convolution when multiplied by
the reshaped filter.
"""
import numpy as np
import pytest
import torch

import convolution_forward_amd as cf
import oracle
import workloads as wl
from conftest import golden
from parity import BF16_RMS_REL, rms_rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def test_gpu_im2col_lecture_patches():
    g = golden("lecture14_arange_patches.json")
    X = torch.arange(36, dtype=torch.float32).reshape(1, 6, 6, 1).to(DEV)
    cols = cf.im2col_nhwc(X, 3, 3).cpu()
    assert list(cols.shape) == g["patch_matrix_shape"]
    assert cols[0].tolist() == g["patch_row_0"] and cols[1].tolist() == g["patch_row_1"]
    assert cols.numel() == g["patch_values"]
    F = torch.arange(9, dtype=torch.float32).reshape(9, 1)
    assert (cols @ F).reshape(4, 4).tolist() == g["output"]


def test_gpu_im2col_storage_bill():
    g = golden("lecture14_storage_bill.json")
    sh = g["shape"]
    X = wl.random_tensor((sh["N"], sh["H"], sh["W"], sh["Cin"]), 71).to(DEV)
    cols = cf.im2col_nhwc(X, sh["K"], sh["K"])
    assert list(cols.shape) == g["patch_matrix_shape"]
    assert cols.numel() == g["values"]["patch_matrix"]
    assert cols.numel() / X.numel() == g["rho"]
    np.testing.assert_array_equal(cols.cpu().numpy(), oracle.im2col_nhwc(X.cpu(), sh["K"], sh["K"]))


PLAIN = [  # (N, H, W, Cin, KH, KW), dtype
    ((2, 7, 9, 16, 3, 3), "f32"), ((2, 7, 9, 16, 3, 3), "bf16"), ((1, 5, 6, 3, 2, 3), "f32"),
    ((3, 4, 4, 8, 1, 1), "bf16"), ((1, 8, 5, 5, 3, 2), "bf16"),
]


@pytest.mark.parametrize("case", PLAIN)
def test_gpu_im2col_bitwise(case):
    (N, H, W, C, KH, KW), dt = case
    X = wl.random_tensor((N, H, W, C), 72 + PLAIN.index(case))
    if dt == "bf16":
        X = X.to(torch.bfloat16)
    cols = cf.im2col_nhwc(X.to(DEV), KH, KW)
    ref = oracle.im2col_nhwc(X.float(), KH, KW)
    np.testing.assert_array_equal(cols.float().cpu().numpy(), ref)


def test_gpu_im2col_strided_view():
    base = wl.random_tensor((2, 9, 12, 24), 80).to(DEV)
    X = base[:, 1:8, ::2, 4:20]          # pixel stride 48, channel stride 1
    cols = cf.im2col_nhwc(X, 3, 3)
    np.testing.assert_array_equal(cols.cpu().numpy(), oracle.im2col_nhwc(X.cpu(), 3, 3))


WINDOWS = [  # (N,H,W,Cin,KH,KW,Cout), stride, padding, dilation
    ((2, 11, 10, 8, 3, 3, 5), 2, 1, 1),
    ((1, 12, 9, 4, 3, 2, 3), (1, 2), (1, 0, 2, 1), 1),
    ((1, 13, 13, 6, 3, 3, 4), 1, 2, 2),
    ((2, 32, 32, 3, 8, 8, 6), 8, 0, 1),
]


@pytest.mark.parametrize("case", WINDOWS)
def test_gpu_im2col_window(case):
    (N, H, W, C, KH, KW, O), s, p, d = case
    X = wl.random_tensor((N, H, W, C), 90 + WINDOWS.index(case))
    F = wl.random_tensor((KH, KW, C, O), 95)
    cols = cf.im2col_nhwc(X.to(DEV), KH, KW, stride=s, padding=p, dilation=d).cpu().numpy()
    pads = cf._pads(p)
    Xp = np.pad(X.numpy(), ((0, 0), (pads[0], pads[1]), (pads[2], pads[3]), (0, 0)))
    ref = oracle.conv2d_nhwc(Xp, F.numpy(), stride=s, dilation=d)
    got = (cols.astype(np.float64) @ F.numpy().reshape(-1, O).astype(np.float64)).reshape(ref.shape)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)
    if d == 1:
        # rows of the stride-1 matrix of the padded input, subsampled
        sh, sw = cf._pair(s)
        full = oracle.im2col_nhwc(Xp, KH, KW).reshape(N, Xp.shape[1] - KH + 1, Xp.shape[2] - KW + 1, -1)
        np.testing.assert_array_equal(cols.reshape(ref.shape[:3] + (-1,)), full[:, ::sh, ::sw][:, :ref.shape[1], :ref.shape[2]])


def test_gpu_im2col_route_matches_implicit_gemm():
    """The comparison route (patch matrix, then a library matmul) and the
    implicit GEMM compute the same convolution within bf16 tolerance."""
    work = wl.DENSE_3X3_BF16
    X, F = wl.dense_inputs(work)
    X, F = X[:4].contiguous(), F
    cols = cf.im2col_nhwc(X.to(DEV), work.KH, work.KW)
    Yr = (cols @ F.to(DEV).reshape(-1, work.Cout)).reshape(4, work.H - 2, work.W - 2, work.Cout)
    Yi = cf.conv2d_nhwc(X.to(DEV), F.to(DEV))
    torch.cuda.synchronize()
    ref = oracle.conv2d_nhwc(X, F)
    assert rms_rel_err(Yi, ref) <= BF16_RMS_REL
    assert rms_rel_err(Yr, ref) <= BF16_RMS_REL
