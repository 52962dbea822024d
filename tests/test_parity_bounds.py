"""CPU checks of the tolerance helpers the GPU parity tests rely on: the bf16
spacing function and the rounding bound accept a correct fp32-accumulated,
round-to-nearest result (even where it sits two bf16 ulps from the rounded
oracle) and reject a result off by two ulps."""
import numpy as np
import torch

import oracle
import workloads as wl
from parity import abs_sum_dense, bf16_rounding_ok, bf16_spacing


def test_bf16_spacing():
    v = np.array([1.0, 1.5, 1.9921875, 2.0, 3.0, 0.25, -0.75, 0.0, 2.0 ** -130])
    expect = np.array([2.0 ** -7, 2.0 ** -7, 2.0 ** -7, 2.0 ** -6, 2.0 ** -6, 2.0 ** -9, 2.0 ** -8,
                       2.0 ** -133, 2.0 ** -133])
    np.testing.assert_array_equal(bf16_spacing(v), expect)


def _case():
    N, H, W, C, K, O = 2, 8, 9, 128, 3, 24
    X = wl.random_tensor((N, H, W, C), 4242).to(torch.bfloat16)
    F = (wl.random_tensor((K, K, C, O), 4243) * (1.0 / (K * K * C) ** 0.5)).to(torch.bfloat16)
    b = wl.random_tensor((O,), 4244)
    ref = oracle.conv2d_nhwc(X, F, bias=b)
    absref = abs_sum_dense(oracle, X, F, bias=b)
    # an fp32 accumulation in another order (torch's CPU conv), rounded RNE
    y = torch.nn.functional.conv2d(X.float().permute(0, 3, 1, 2), F.float().permute(3, 2, 0, 1).contiguous(), b)
    yb = y.permute(0, 2, 3, 1).contiguous().to(torch.bfloat16)
    return ref, absref, yb, K * K * C


def test_bound_accepts_correct_rounding():
    ref, absref, yb, n = _case()
    assert bf16_rounding_ok(yb, ref, absref, n)


def test_bound_rejects_two_ulp_error():
    ref, absref, yb, n = _case()
    bad = yb.clone().view(torch.int16)
    i = int(torch.from_numpy(np.abs(ref)).reshape(-1).argmax())
    flat = bad.reshape(-1)
    flat[i] = flat[i] + 2                     # two bf16 ulps away from the magnitude
    assert not bf16_rounding_ok(bad.view(torch.bfloat16), ref, absref, n)


def test_bound_rejects_dropped_bias():
    ref, absref, yb, n = _case()
    assert not bf16_rounding_ok(yb - 0.05, ref, absref, n)
