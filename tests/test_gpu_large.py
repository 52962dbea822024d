"""Maximum sizes on the GPU: inputs past 4 GiB (dense) and past 2**31
elements (depthwise), through the tiled kernels the benchmark times.

Each large input repeats a seeded base batch of 8 images along N (built on the
GPU, so no host copy of the large tensor exists). The base images are checked
against the oracle; every repeat must then equal its base image bit for bit,
which checks every output of the large launch, including the images whose
byte offsets cross 2**31 and 2**32.
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


def test_gpu_dense_bf16_input_past_4gib():
    base = 8
    Xb = wl.random_tensor((base, 58, 58, 64), 12001).to(torch.bfloat16)
    F = (wl.random_tensor((3, 3, 64, 64), 12002) * (1.0 / 576 ** 0.5)).to(torch.bfloat16)
    reps = 1250                                   # N = 10000: X is 4.31 GB, Y 4.01 GB
    X = Xb.to(DEV).repeat(reps, 1, 1, 1)
    assert X.numel() * 2 > 2 ** 32
    Fd = F.to(DEV)
    assert cf.dense_variant_for(X, Fd) == cf.VARIANT_TILED
    Y = cf.conv2d_nhwc(X, Fd)
    torch.cuda.synchronize()
    del X
    ref = oracle.conv2d_nhwc(Xb, F)
    Y0 = Y[:base].cpu()
    assert rms_rel_err(Y0, ref) <= BF16_RMS_REL
    assert bf16_rounding_ok(Y0, ref, abs_sum_dense(oracle, Xb, F), 576)
    same = torch.equal(Y.view(reps, base, 56, 56, 64).view(torch.int16),
                       Y[:base].unsqueeze(0).expand(reps, -1, -1, -1, -1).view(torch.int16))
    del Y
    torch.cuda.empty_cache()
    assert same


def test_gpu_depthwise_exact_input_past_2_31_elements():
    base = 8
    Xb = wl.random_tensor((base, 72, 56, 56), 12011)
    w = wl.random_tensor((72, 5, 5), 12012)
    reps = 1190                                   # N = 9520: 2.149e9 elements (8.6 GB)
    X = Xb.to(DEV).repeat(reps, 1, 1, 1)
    assert X.numel() > 2 ** 31
    assert cf.depthwise_variant_for(X, w.to(DEV), stride=2, padding=2) == cf.VARIANT_TILED
    Y = cf.conv_depthwise(X, w.to(DEV), stride=2, padding=2, exact=True)
    torch.cuda.synchronize()
    del X
    ref = oracle.depthwise_nchw(Xb, w, stride=2, padding=2, mode="exact")
    np.testing.assert_array_equal(bits(Y[:base]), bits(ref))
    same = torch.equal(Y.view(reps, base, 72, 28, 28).view(torch.int32),
                       Y[:base].unsqueeze(0).expand(reps, -1, -1, -1, -1).view(torch.int32))
    del Y
    torch.cuda.empty_cache()
    assert same
