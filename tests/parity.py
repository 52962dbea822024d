"""Tolerance metrics for comparing the HIP path with the fp64 oracle.

Dense fp32: max_i |g_i - r_i| / max_i |r_i| <= 1e-5 (elementwise relative
error is undefined where outputs cancel to near zero, so the scale is the
largest output).
Dense bf16 inputs, fp32 accumulate: max_i |g_i - r_i| / rms(r) <= 2e-2, and
for bf16 outputs a per-element bound on round-to-nearest plus fp32
accumulation error (``bf16_rounding_ok``).
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


def bf16_spacing(v: np.ndarray) -> np.ndarray:
    """Distance between neighbouring bf16 values in the binade of each v (8
    significant bits, fp32's exponent range; subnormal spacing 2^-133)."""
    v = np.abs(np.asarray(v, np.float64))
    _, e = np.frexp(v)                     # v = m * 2^e, m in [0.5, 1)
    e = np.where(v == 0, -125, e)          # zero sits in the subnormal range
    return np.ldexp(1.0, np.maximum(e - 8, -133))


def bf16_rounding_ok(got_bf16, ref, absref, n_terms: int) -> bool:
    """Rigorous per-element bound for a bf16 output g = RNE(s) where s is an
    fp32 accumulation of n_terms products in any order, plus one bias add.

    |g - s| <= spacing(g)/2 (round to nearest; rounding is monotone, so g's
    binade is at least s's). |s - r| <= gamma * sum|x_k w_k| with
    gamma = k u / (1 - k u), u = 2^-24, the classical bound for floating-point
    summation in any order (Higham, "Accuracy and Stability of Numerical
    Algorithms", section 3.1); k = 2 n + 2 leaves room for the matrix cores'
    internal accumulation and the bias add. ``absref`` is the oracle's sum of
    |x_k w_k| (+ |bias|) per output.

    A fixed "at most 1 ulp from the rounded oracle" rule is not a valid test:
    where an output nearly cancels, fp32 accumulation error alone spans
    several bf16 ulps (torch's own fp32 CPU conv, rounded, shows 2 on a
    3x3x128 window)."""
    g, r, a = to_f64(got_bf16), to_f64(ref), to_f64(absref)
    u = 2.0 ** -24
    k = 2 * n_terms + 2
    gamma = k * u / (1 - k * u)
    bound = 0.5 * bf16_spacing(g) + gamma * a
    return bool(np.all(np.abs(g - r) <= bound))


def abs_sum_dense(oracle_mod, X, F, bias=None, **window):
    """The oracle's sum of |x_k w_k| (+ |bias|) per output: the scale of the
    accumulation error bound in ``bf16_rounding_ok``."""
    # |v| of an fp32 or bf16 value is exact in fp32
    Xa, Fa = np.abs(to_f64(X)).astype(np.float32), np.abs(to_f64(F)).astype(np.float32)
    ba = None if bias is None else np.abs(to_f64(bias)).astype(np.float32)
    return oracle_mod.conv2d_nhwc(Xa, Fa, bias=ba, **window)


def bits(t) -> np.ndarray:
    a = t.detach().cpu().numpy() if isinstance(t, torch.Tensor) else np.asarray(t)
    return np.ascontiguousarray(a.astype(np.float32)).view(np.uint32)
