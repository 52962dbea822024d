"""CPU oracle for the forward 2D convolution operator (ctypes wrapper).

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The product
path (``convolution_forward_amd``) never imports, links or calls it, and the
two share no code: only the seeded input generators in ``workloads.py`` serve
both.

The arithmetic lives in ``convfwd_oracle.c`` (plain C, gcc -O2
-ffp-contract=off). This wrapper only marshals numpy arrays, plus one fp64
matmul (numpy) that turns the explicit patch matrix into an output.

Entry points and how each is pinned (``tests/test_oracle_pins.py``):

* ``conv2d_nhwc`` -- dense cross-correlation, fp64 accumulate ("CMU DLSys
  Lecture 14", section 1). Pinned by the pages' worked examples (the 6x6
  arange patch example of section 4, the 1D window / average / difference /
  motif filters, the 3x3 * 2x2 image, the Sobel maps and the two-filter GEMM
  of "Convolution Is Wx+b Moving Across a Signal"), by the K=1 matmul and the
  sum of shifted channel matmuls (lecture section 2), by the full-image filter,
  by torch's CPU conv2d through the axis conversions of section 1, by brute
  force with Python integers, and by translation equivariance.
* ``conv2d_nhwc_at`` -- the same sum at sampled output indices; pinned by
  agreement with ``conv2d_nhwc``.
* ``im2col_nhwc`` / ``conv2d_nhwc_im2col`` -- the explicit patch matrix of
  lecture section 5; pinned by the patch rows the lecture prints, the matrix
  sizes of section 6, and agreement with the loop form.
* ``depthwise_nchw`` -- per-output depthwise loop, exact and fast modes
  ("Depthwise convolution", section "What each output is"). Pinned by an
  exact-rational brute force that rounds each step to fp32 independently of
  numpy and of C, by hand-derived special values (canonical NaN, an infinite
  weight meeting padding, +0 results, a case where fused and unfused rounding
  differ), by the block-diagonal dense equivalence, and by torch's CPU
  grouped conv2d.
* ``out_size`` -- the per-axis output-size rule ("Convolution Is Wx+b",
  section "Why 1D? Why 2D?"); pinned by the pages' 5-3+1=3 example and the
  workload shapes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "convfwd_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_CFLAGS = ["-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-Wno-unused-parameter"]

_lib = None


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc. Returns the library path."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", *_CFLAGS, _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build(force=True)
    lib = ctypes.CDLL(_LIB)
    i, ll, p = ctypes.c_int, ctypes.c_longlong, ctypes.c_void_p
    lib.oracle_out_size.restype = ll
    lib.oracle_out_size.argtypes = [ll, ll, ll, ll, ll]
    lib.oracle_conv2d_nhwc_f64.restype = i
    lib.oracle_conv2d_nhwc_f64.argtypes = [p, p, p, p, p] + [i] * 7 + [i] * 7 + [i]
    lib.oracle_conv2d_nhwc_f64_at.restype = i
    lib.oracle_conv2d_nhwc_f64_at.argtypes = [p, p, p, p, p, ll, p] + [i] * 7 + [i] * 7 + [i]
    lib.oracle_im2col_nhwc.restype = i
    lib.oracle_im2col_nhwc.argtypes = [p, p, p] + [i] * 6
    lib.oracle_depthwise_nchw_f32.restype = i
    lib.oracle_depthwise_nchw_f32.argtypes = [p, p, p, p] + [i] * 15
    _lib = lib
    return lib


def default_threads() -> int:
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        return int(env)
    return os.cpu_count() or 1


def _pair(v):
    if isinstance(v, (tuple, list)):
        a, b = v
        return int(a), int(b)
    return int(v), int(v)


def _as_f32(a) -> np.ndarray:
    """Accept numpy arrays or CPU torch tensors (fp32 or bf16). bf16 values are
    widened to fp32, which is exact. Strides are kept."""
    if not isinstance(a, np.ndarray):
        import torch
        t = a.detach().cpu()
        if t.dtype != torch.float32:
            t = t.to(torch.float32)
        a = t.numpy()
    if a.dtype != np.float32:
        raise ValueError("oracle inputs must be float32 (or bf16 torch tensors)")
    return a


def _elem_strides(a: np.ndarray) -> np.ndarray:
    return np.asarray([s // a.itemsize for s in a.strides], dtype=np.int64)


def _ptr(a) -> int | None:
    return None if a is None else a.ctypes.data


def out_size(n: int, k: int, stride: int = 1, pad: int = 0, dil: int = 1) -> int:
    """Per-axis output size; <= 0 means no window fits."""
    return int(_load().oracle_out_size(n, k, stride, pad, dil))


def conv2d_nhwc(X, F, bias=None, stride=1, padding=0, dilation=1, groups=1, threads=None) -> np.ndarray:
    """Dense NHWC cross-correlation. X [N,H,W,Cin] (any strides), F
    [KH,KW,Cin/groups,Cout]. Returns fp64 [N,Ho,Wo,Cout]."""
    X = _as_f32(X)
    F = np.ascontiguousarray(_as_f32(F))
    b = None if bias is None else np.ascontiguousarray(_as_f32(bias))
    N, H, W, Cin = X.shape
    KH, KW, _, Cout = F.shape
    sh, sw = _pair(stride)
    ph, pw = _pair(padding)
    dh, dw = _pair(dilation)
    Ho, Wo = out_size(H, KH, sh, ph, dh), out_size(W, KW, sw, pw, dw)
    if Ho <= 0 or Wo <= 0:
        raise ValueError("Incompatible input and filter")
    if F.shape[2] * groups != Cin:
        raise ValueError("filter channels do not match Cin / groups")
    Y = np.empty((N, Ho, Wo, Cout), dtype=np.float64)
    xs = _elem_strides(X)
    rc = _load().oracle_conv2d_nhwc_f64(X.ctypes.data, xs.ctypes.data, F.ctypes.data, _ptr(b),
                                        Y.ctypes.data, N, H, W, Cin, KH, KW, Cout, sh, sw, ph, pw,
                                        dh, dw, groups, threads or default_threads())
    if rc != 0:
        raise ValueError("oracle_conv2d_nhwc_f64 rejected its arguments")
    return Y


def conv2d_nhwc_at(X, F, flat_idx, bias=None, stride=1, padding=0, dilation=1, groups=1,
                   threads=None) -> np.ndarray:
    """conv2d_nhwc evaluated only at flat indices of the contiguous output."""
    X = _as_f32(X)
    F = np.ascontiguousarray(_as_f32(F))
    b = None if bias is None else np.ascontiguousarray(_as_f32(bias))
    idx = np.ascontiguousarray(np.asarray(flat_idx, dtype=np.int64))
    N, H, W, Cin = X.shape
    KH, KW, _, Cout = F.shape
    sh, sw = _pair(stride)
    ph, pw = _pair(padding)
    dh, dw = _pair(dilation)
    out = np.empty(idx.shape[0], dtype=np.float64)
    xs = _elem_strides(X)
    rc = _load().oracle_conv2d_nhwc_f64_at(X.ctypes.data, xs.ctypes.data, F.ctypes.data, _ptr(b),
                                           idx.ctypes.data, idx.shape[0], out.ctypes.data, N, H, W,
                                           Cin, KH, KW, Cout, sh, sw, ph, pw, dh, dw, groups,
                                           threads or default_threads())
    if rc != 0:
        raise ValueError("oracle_conv2d_nhwc_f64_at rejected its arguments")
    return out


def im2col_nhwc(X, KH: int, KW: int) -> np.ndarray:
    """Explicit patch matrix [(N*Ho*Wo), KH*KW*C] in (i,j,c) column order."""
    X = _as_f32(X)
    N, H, W, C = X.shape
    if KH > H or KW > W:
        raise ValueError("Incompatible input and filter")
    Ho, Wo = H - KH + 1, W - KW + 1
    cols = np.empty((N * Ho * Wo, KH * KW * C), dtype=np.float32)
    xs = _elem_strides(X)
    rc = _load().oracle_im2col_nhwc(X.ctypes.data, xs.ctypes.data, cols.ctypes.data, N, H, W, C, KH, KW)
    if rc != 0:
        raise ValueError("oracle_im2col_nhwc rejected its arguments")
    return cols


def conv2d_nhwc_im2col(X, F) -> np.ndarray:
    """Second route: explicit patch matrix times the reshaped filter, in fp64."""
    X = _as_f32(X)
    F = np.ascontiguousarray(_as_f32(F))
    N, H, W, C = X.shape
    KH, KW, _, Cout = F.shape
    cols = im2col_nhwc(X, KH, KW).astype(np.float64)
    Y = cols @ F.reshape(KH * KW * C, Cout).astype(np.float64)
    return Y.reshape(N, H - KH + 1, W - KW + 1, Cout)


def depthwise_nchw(X, w, bias=None, stride=1, padding=0, dilation=1, mode="exact",
                   threads=None) -> np.ndarray:
    """Depthwise conv, NCHW fp32. w [C*mult,KH,KW]. mode "exact" or "fast"."""
    X = np.ascontiguousarray(_as_f32(X))
    w = np.ascontiguousarray(_as_f32(w))
    b = None if bias is None else np.ascontiguousarray(_as_f32(bias))
    N, C, H, W = X.shape
    Cout, KH, KW = w.shape
    if Cout % C != 0:
        raise ValueError("weight channels must be a multiple of input channels")
    mult = Cout // C
    sh, sw = _pair(stride)
    ph, pw = _pair(padding)
    dh, dw = _pair(dilation)
    Ho, Wo = out_size(H, KH, sh, ph, dh), out_size(W, KW, sw, pw, dw)
    if Ho <= 0 or Wo <= 0:
        raise ValueError("Incompatible input and filter")
    m = {"exact": 0, "fast": 1}[mode]
    Y = np.empty((N, Cout, Ho, Wo), dtype=np.float32)
    rc = _load().oracle_depthwise_nchw_f32(X.ctypes.data, w.ctypes.data, _ptr(b), Y.ctypes.data, N, C,
                                           H, W, mult, KH, KW, sh, sw, ph, pw, dh, dw, m,
                                           threads or default_threads())
    if rc != 0:
        raise ValueError("oracle_depthwise_nchw_f32 rejected its arguments")
    return Y
