"""Tolerance metrics for comparing the HIP path with the fp64 oracle.

Dense fp32: max_i |g_i - r_i| / max_i |r_i| <= 1e-5 (elementwise relative
error is undefined where outputs cancel to near zero, so the scale is the
largest output).
Dense bf16 inputs, fp32 accumulate: max_i |g_i - r_i| / rms(r) <= 2e-2.
Depthwise: bitwise.
"""
import numpy as np
import torch

F32_MAX_REL = 1e-5
BF16_RMS_REL = 2e-2


def to_f64(t) -> np.ndarray:
    if isinstance(t, np.ndarray):
        return t.astype(np.float64)
    return t.detach().float().cpu().numpy().astype(np.float64)


def max_rel_err(got, ref) -> float:
    g, r = to_f64(got), to_f64(ref)
    scale = np.max(np.abs(r))
    return float(np.max(np.abs(g - r)) / scale) if scale > 0 else float(np.max(np.abs(g - r)))


def rms_rel_err(got, ref) -> float:
    g, r = to_f64(got), to_f64(ref)
    rms = np.sqrt(np.mean(r * r))
    return float(np.max(np.abs(g - r)) / rms) if rms > 0 else float(np.max(np.abs(g - r)))


def bf16_ulp_distance(got_bf16: torch.Tensor, ref_f64: np.ndarray) -> int:
    """Largest distance, in bf16 units in the last place, between the GPU's
    bf16 output and the fp64 oracle rounded to bf16 (nearest-even)."""
    ref_b = torch.from_numpy(np.asarray(ref_f64, np.float64)).to(torch.float32).to(torch.bfloat16)
    a = got_bf16.detach().cpu().view(torch.int16).to(torch.int32)
    b = ref_b.view(torch.int16).to(torch.int32)
    # map sign-magnitude to a monotone integer line
    a = torch.where(a < 0, -(a & 0x7FFF), a)
    b = torch.where(b < 0, -(b & 0x7FFF), b)
    return int((a - b).abs().max().item()) if a.numel() else 0


def bits(t) -> np.ndarray:
    a = t.detach().cpu().numpy() if isinstance(t, torch.Tensor) else np.asarray(t)
    return np.ascontiguousarray(a.astype(np.float32)).view(np.uint32)
