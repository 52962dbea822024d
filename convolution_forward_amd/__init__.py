"""convolution_forward_amd -- Python binding of libconvfwd (MI355X / gfx950).

Argument marshalling only: every step of the convolution runs in the HIP
kernels behind the C ABI declared in include/convfwd.h. PyTorch supplies
device memory and the current stream; nothing here computes on the CPU, and
there is no fallback: if the library is not built, or a tensor is not on a
GPU, the call raises.

    conv2d_nhwc(x, f, bias=None, out=None, out_dtype=None, stride=1, padding=0, dilation=1, groups=1)
        Dense cross-correlation, X [N,H,W,Cin] (channel stride 1, other
        strides free), F [KH,KW,Cin/groups,Cout] contiguous -> Y [N,Ho,Wo,Cout].
    conv_depthwise(x, w, bias=None, stride=1, padding=0, dilation=1, exact=True)
        Depthwise, X [N,C,H,W], w [C*mult,KH,KW] -> Y [N,C*mult,Ho,Wo].

padding is an int (all sides), a pair (rows, columns; the same before and
after), or four values (top, bottom, left, right).
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "_lib", "libconvfwd.so")

# conv_status values (include/convfwd.h)
CONV_OK = 0
CONV_ERR_NULL = 1
CONV_ERR_NONPOSITIVE = 2
CONV_ERR_SHAPE = 3
CONV_ERR_DTYPE = 4
CONV_ERR_LAYOUT = 5
CONV_ERR_ALIAS = 6
CONV_ERR_UNSUPPORTED = 7
CONV_ERR_HIP = 8

CONV_F32 = 0
CONV_BF16 = 1
CONV_DW_EXACT = 0
CONV_DW_FAST = 1
VARIANT_AUTO = 0
VARIANT_DIRECT = 1
VARIANT_TILED = 2

EXPORTED = ("conv2d_nhwc_fwd", "conv2d_nhwc_fwd_variant", "conv2d_nhwc_fwd_window", "conv_depthwise_fwd",
            "conv_depthwise_fwd_variant", "conv_depthwise_fwd_window", "conv2d_nhwc_auto_variant",
            "conv2d_nhwc_window_auto_variant", "conv_depthwise_auto_variant", "conv_depthwise_window_auto_variant",
            "conv_out_size", "conv_out_size_window", "conv_status_str", "conv_copy_bytes", "conv_copy_bytes_wide",
            "conv_im2col_nhwc")


class ConvWindow(ctypes.Structure):
    """struct conv_window (include/convfwd.h)."""
    _fields_ = [(name, ctypes.c_int) for name in
                ("stride_h", "stride_w", "pad_top", "pad_bottom", "pad_left", "pad_right", "dil_h", "dil_w",
                 "groups")]


class ConvError(RuntimeError):
    """A non-OK conv_status; ``status`` holds the code."""

    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


class ConvArgumentError(ConvError, ValueError):
    """An argument error reported by the library (nothing was launched)."""


_lib = None


def load_library():
    """Load libconvfwd.so (built in-tree by convolution_forward_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m convolution_forward_amd.build` "
                           "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(LIB_PATH)
    p, i, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    lib.conv2d_nhwc_fwd.restype = i
    lib.conv2d_nhwc_fwd.argtypes = [p, p, p, p, p, p] + [i] * 7 + [i, i, p]
    lib.conv2d_nhwc_fwd_variant.restype = i
    lib.conv2d_nhwc_fwd_variant.argtypes = [p, p, p, p, p, p] + [i] * 7 + [i, i, i, p]
    lib.conv_depthwise_fwd.restype = i
    lib.conv_depthwise_fwd.argtypes = [p, p, p, p] + [i] * 13 + [i, p]
    lib.conv_depthwise_fwd_variant.restype = i
    lib.conv_depthwise_fwd_variant.argtypes = [p, p, p, p] + [i] * 13 + [i, i, p]
    lib.conv2d_nhwc_auto_variant.restype = i
    lib.conv2d_nhwc_auto_variant.argtypes = [p, p, p, p, p, p] + [i] * 7 + [i, i]
    lib.conv_depthwise_auto_variant.restype = i
    lib.conv_depthwise_auto_variant.argtypes = [p, p, p, p] + [i] * 13 + [i]
    lib.conv_out_size.restype = i64
    lib.conv_out_size.argtypes = [i64, i, i, i, i]
    wp = ctypes.POINTER(ConvWindow)
    lib.conv2d_nhwc_fwd_window.restype = i
    lib.conv2d_nhwc_fwd_window.argtypes = [p, p, p, p, p, p] + [i] * 7 + [wp, i, i, i, p]
    lib.conv_depthwise_fwd_window.restype = i
    lib.conv_depthwise_fwd_window.argtypes = [p, p, p, p] + [i] * 7 + [wp, i, i, p]
    lib.conv2d_nhwc_window_auto_variant.restype = i
    lib.conv2d_nhwc_window_auto_variant.argtypes = [p, p, p, p, p, p] + [i] * 7 + [wp, i, i]
    lib.conv_depthwise_window_auto_variant.restype = i
    lib.conv_depthwise_window_auto_variant.argtypes = [p, p, p, p] + [i] * 7 + [wp, i]
    lib.conv_im2col_nhwc.restype = i
    lib.conv_im2col_nhwc.argtypes = [p, p, p] + [i] * 6 + [wp, i, p]
    lib.conv_out_size_window.restype = i64
    lib.conv_out_size_window.argtypes = [i64, i, i, i, i, i]
    lib.conv_status_str.restype = ctypes.c_char_p
    lib.conv_status_str.argtypes = [i]
    lib.conv_copy_bytes.restype = i
    lib.conv_copy_bytes.argtypes = [p, p, i64, p]
    lib.conv_copy_bytes_wide.restype = i
    lib.conv_copy_bytes_wide.argtypes = [p, p, i64, p]
    _lib = lib
    return lib


def status_str(status: int) -> str:
    return load_library().conv_status_str(status).decode()


def _check(status: int, what: str):
    if status == CONV_OK:
        return
    msg = f"{what}: {status_str(status)} (status {status})"
    if status == CONV_ERR_HIP:
        raise ConvError(status, msg)
    raise ConvArgumentError(status, msg)


def out_size(n: int, k: int, stride: int = 1, pad: int = 0, dil: int = 1) -> int:
    return int(load_library().conv_out_size(n, k, stride, pad, dil))


def out_size_window(n: int, k: int, stride: int = 1, pad_before: int = 0, pad_after: int = 0, dil: int = 1) -> int:
    return int(load_library().conv_out_size_window(n, k, stride, pad_before, pad_after, dil))


def _pair(v):
    if isinstance(v, (tuple, list)):
        a, b = v
        return int(a), int(b)
    return int(v), int(v)


def _pads(padding):
    """(top, bottom, left, right) from an int, a (rows, columns) pair or four values."""
    if isinstance(padding, (tuple, list)) and len(padding) == 4:
        return tuple(int(v) for v in padding)
    ph, pw = _pair(padding)
    return ph, ph, pw, pw


def window(stride=1, padding=0, dilation=1, groups: int = 1) -> ConvWindow:
    sh, sw = _pair(stride)
    pt, pb, pl, pr = _pads(padding)
    dh, dw = _pair(dilation)
    return ConvWindow(sh, sw, pt, pb, pl, pr, dh, dw, int(groups))


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t == torch.float32:
        return CONV_F32
    if t == torch.bfloat16:
        return CONV_BF16
    raise ValueError(f"unsupported dtype {t}; use float32 or bfloat16")


def _stream_ptr(device) -> int:
    return _torch().cuda.current_stream(device).cuda_stream


def _require_gpu(*tensors):
    for t in tensors:
        if t is not None and not t.is_cuda:
            raise ValueError("tensors must live on the GPU (no CPU path exists)")


def _strides_arr(t):
    return (ctypes.c_int64 * 4)(*t.stride())


def conv2d_nhwc(x, f, bias=None, out=None, out_dtype=None, variant: int = VARIANT_AUTO, stride=1, padding=0,
                dilation=1, groups: int = 1):
    """Dense NHWC cross-correlation on the GPU (see include/convfwd.h)."""
    torch = _torch()
    lib = load_library()
    _require_gpu(x, f, bias, out)
    if x.dim() != 4 or f.dim() != 4:
        raise ValueError("expected X as [N,H,W,Cin] and F as [KH,KW,Cin/groups,Cout]")
    N, H, W, Cin = x.shape
    KH, KW, Cf, Cout = f.shape
    if groups < 1 or Cf * groups != Cin:
        raise ValueError(f"filter input channels {Cf} x groups {groups} != input channels {Cin}")
    if f.dtype != x.dtype:
        raise ValueError("X and F must share a dtype")
    if not f.is_contiguous():
        raise ValueError("F must be contiguous [KH,KW,Cin,Cout]")
    if bias is not None and (bias.dtype != torch.float32 or not bias.is_contiguous() or bias.numel() != Cout):
        raise ValueError("bias must be a contiguous float32 tensor of Cout values")
    win = window(stride, padding, dilation, groups)
    Ho = out_size_window(H, KH, win.stride_h, win.pad_top, win.pad_bottom, win.dil_h)
    Wo = out_size_window(W, KW, win.stride_w, win.pad_left, win.pad_right, win.dil_w)
    ydt = out.dtype if out is not None else (out_dtype or x.dtype)
    if out is None:
        if Ho <= 0 or Wo <= 0 or min(N, H, W, Cin, KH, KW, Cout) <= 0:
            # Let the library classify the error; no output buffer is needed.
            st = lib.conv2d_nhwc_fwd_window(x.data_ptr() or 1, _strides_arr(x), f.data_ptr() or 1, None, 1,
                                            None, N, H, W, Cin, KH, KW, Cout, ctypes.byref(win),
                                            _dtype_code(x.dtype), _dtype_code(ydt), variant, None)
            _check(st if st != CONV_OK else CONV_ERR_SHAPE, "conv2d_nhwc_fwd_window")
        out = torch.empty((N, Ho, Wo, Cout), dtype=ydt, device=x.device)
    elif tuple(out.shape) != (N, Ho, Wo, Cout):
        raise ValueError(f"out has shape {tuple(out.shape)}, expected {(N, Ho, Wo, Cout)}")
    st = lib.conv2d_nhwc_fwd_window(x.data_ptr(), _strides_arr(x), f.data_ptr(),
                                    None if bias is None else bias.data_ptr(), out.data_ptr(), _strides_arr(out),
                                    N, H, W, Cin, KH, KW, Cout, ctypes.byref(win), _dtype_code(x.dtype),
                                    _dtype_code(out.dtype), variant, _stream_ptr(x.device))
    _check(st, "conv2d_nhwc_fwd_window")
    return out


def conv_depthwise(x, w, bias=None, stride=1, padding=0, dilation=1, exact: bool = True, out=None,
                   variant: int = VARIANT_AUTO):
    """Depthwise convolution on the GPU, NCHW fp32 (see include/convfwd.h)."""
    torch = _torch()
    lib = load_library()
    _require_gpu(x, w, bias, out)
    if x.dim() != 4 or w.dim() != 3:
        raise ValueError("expected X as [N,C,H,W] and w as [C*multiplier,KH,KW]")
    if x.dtype != torch.float32 or w.dtype != torch.float32:
        raise ValueError("depthwise runs in float32")
    if not x.is_contiguous() or not w.is_contiguous():
        raise ValueError("X and w must be contiguous")
    N, C, H, W = x.shape
    Cout, KH, KW = w.shape
    if C <= 0 or Cout % C != 0:
        raise ValueError("weight channels must be a positive multiple of input channels")
    mult = Cout // C
    if bias is not None and (bias.dtype != torch.float32 or not bias.is_contiguous() or bias.numel() != Cout):
        raise ValueError("bias must be a contiguous float32 tensor of C*multiplier values")
    win = window(stride, padding, dilation)
    Ho = out_size_window(H, KH, win.stride_h, win.pad_top, win.pad_bottom, win.dil_h)
    Wo = out_size_window(W, KW, win.stride_w, win.pad_left, win.pad_right, win.dil_w)
    mode = CONV_DW_EXACT if exact else CONV_DW_FAST
    if out is None:
        if Ho <= 0 or Wo <= 0:
            # Let the library classify the error (it returns before touching
            # any pointer); no output buffer is needed.
            st = lib.conv_depthwise_fwd_window(x.data_ptr() or 1, w.data_ptr() or 1, None, 1, N, C, H, W, mult,
                                               KH, KW, ctypes.byref(win), mode, variant, None)
            _check(st if st != CONV_OK else CONV_ERR_SHAPE, "conv_depthwise_fwd_window")
        out = torch.empty((N, Cout, Ho, Wo), dtype=torch.float32, device=x.device)
    elif tuple(out.shape) != (N, Cout, Ho, Wo) or not out.is_contiguous() or out.dtype != torch.float32:
        raise ValueError(f"out must be a contiguous float32 tensor of shape {(N, Cout, Ho, Wo)}")
    st = lib.conv_depthwise_fwd_window(x.data_ptr(), w.data_ptr(), None if bias is None else bias.data_ptr(),
                                       out.data_ptr(), N, C, H, W, mult, KH, KW, ctypes.byref(win), mode, variant,
                                       _stream_ptr(x.device))
    _check(st, "conv_depthwise_fwd_window")
    return out


def im2col_nhwc(x, KH: int, KW: int, stride=1, padding=0, dilation=1, out=None):
    """Explicit patch matrix [N*Ho*Wo, KH*KW*Cin] of X on the GPU (see
    include/convfwd.h): the packing step of the im2col route, for comparison
    with the implicit-GEMM kernels, which never build it."""
    torch = _torch()
    lib = load_library()
    _require_gpu(x, out)
    if x.dim() != 4:
        raise ValueError("expected X as [N,H,W,Cin]")
    N, H, W, Cin = x.shape
    win = window(stride, padding, dilation)
    Ho = out_size_window(H, KH, win.stride_h, win.pad_top, win.pad_bottom, win.dil_h)
    Wo = out_size_window(W, KW, win.stride_w, win.pad_left, win.pad_right, win.dil_w)
    shape = (N * max(Ho, 0) * max(Wo, 0), KH * KW * Cin)
    if out is None:
        if Ho <= 0 or Wo <= 0:
            _check(CONV_ERR_SHAPE, "conv_im2col_nhwc")
        out = torch.empty(shape, dtype=x.dtype, device=x.device)
    elif tuple(out.shape) != shape or not out.is_contiguous() or out.dtype != x.dtype:
        raise ValueError(f"out must be a contiguous {x.dtype} tensor of shape {shape}")
    st = lib.conv_im2col_nhwc(x.data_ptr(), _strides_arr(x), out.data_ptr(), N, H, W, Cin, KH, KW,
                              ctypes.byref(win), _dtype_code(x.dtype), _stream_ptr(x.device))
    _check(st, "conv_im2col_nhwc")
    return out


def dense_variant_for(x, f, out_dtype=None, stride=1, padding=0, dilation=1, groups: int = 1, bias=None,
                      out=None) -> int:
    """The variant CONV_VARIANT_AUTO launches for conv2d_nhwc with these
    arguments (host query; -1 where the call would fail). Without `out` the
    query describes the fresh output conv2d_nhwc allocates."""
    N, H, W, Cin = x.shape
    KH, KW, _, Cout = f.shape
    win = window(stride, padding, dilation, groups)
    ydt = out.dtype if out is not None else (out_dtype or x.dtype)
    return int(load_library().conv2d_nhwc_window_auto_variant(
        x.data_ptr(), _strides_arr(x), f.data_ptr(), None if bias is None else bias.data_ptr(),
        None if out is None else out.data_ptr(), None if out is None else _strides_arr(out),
        N, H, W, Cin, KH, KW, Cout, ctypes.byref(win), _dtype_code(x.dtype), _dtype_code(ydt)))


def depthwise_variant_for(x, w, stride=1, padding=0, dilation=1, exact: bool = True, bias=None, out=None) -> int:
    """The variant CONV_VARIANT_AUTO launches for conv_depthwise with these
    tensors (host query; -1 where the call would fail). Without `out` the
    query uses a stand-in output address past X (fresh allocations are
    256-byte aligned; no alignment of Y is looked at)."""
    N, C, H, W = x.shape
    Cout, KH, KW = w.shape
    win = window(stride, padding, dilation)
    if out is not None:
        y = out.data_ptr()
    else:
        # one past X, rounded up to 256 bytes: never overlapping X, w or bias
        # as long as those were not allocated right behind X
        y = (x.data_ptr() + x.numel() * 4 + 255) // 256 * 256
        y = max(y, (w.data_ptr() + w.numel() * 4 + 255) // 256 * 256)
        if bias is not None:
            y = max(y, (bias.data_ptr() + bias.numel() * 4 + 255) // 256 * 256)
    return int(load_library().conv_depthwise_window_auto_variant(
        x.data_ptr(), w.data_ptr(), None if bias is None else bias.data_ptr(), y, N, C, H, W, Cout // C, KH, KW,
        ctypes.byref(win), CONV_DW_EXACT if exact else CONV_DW_FAST))


def copy_bytes(src, dst, nbytes: int | None = None, wide: bool = False):
    """Streaming copy kernel (bandwidth / counter calibration): the plain
    grid-stride copy, or with wide=True the one with eight loads in flight
    per thread."""
    _require_gpu(src, dst)
    n = src.numel() * src.element_size() if nbytes is None else int(nbytes)
    if n > dst.numel() * dst.element_size() or n > src.numel() * src.element_size():
        raise ValueError("copy larger than a buffer")
    fn = load_library().conv_copy_bytes_wide if wide else load_library().conv_copy_bytes
    _check(fn(src.data_ptr(), dst.data_ptr(), n, _stream_ptr(src.device)),
           "conv_copy_bytes_wide" if wide else "conv_copy_bytes")
    return dst
