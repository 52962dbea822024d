"""The C ABI, checked without a GPU: the library loads, exports exactly what
include/convfwd.h declares, and rejects every invalid argument before any HIP
call (so these calls are safe on a machine with no GPU: fake, distinct device
addresses are passed and never dereferenced)."""
import ctypes
import os
import re
import subprocess

import pytest

import convolution_forward_amd as cf
from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "convfwd.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(cf.LIB_PATH):
        from convolution_forward_amd import build
        build.build()
    return cf.load_library()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"CONVFWD_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)))


def test_exports_match_header(lib):
    names = declared_functions()
    assert set(names) == set(cf.EXPORTED)
    out = subprocess.run(["nm", "-D", "--defined-only", cf.LIB_PATH], capture_output=True, text=True, check=True)
    exported = {line.split()[-1] for line in out.stdout.splitlines() if " T " in line}
    assert exported == set(names), f"exported {sorted(exported)} vs declared {names}"
    for n in names:
        getattr(lib, n)


def test_library_never_allocates_device_memory(lib):
    """No hidden copy: the library imports no allocation or synchronisation API."""
    out = subprocess.run(["nm", "-D", "--undefined-only", cf.LIB_PATH], capture_output=True, text=True, check=True)
    undefined = {line.split()[-1] for line in out.stdout.splitlines()}
    bad = [s for s in undefined if re.match(r"hip(Ext)?(Malloc|Free|MallocAsync|HostMalloc|MallocManaged|"
                                              r"DeviceSynchronize|StreamSynchronize|Memcpy)", s)]
    assert not bad, bad


def test_status_strings(lib):
    for s in range(9):
        assert len(cf.status_str(s)) >= 2
    assert cf.status_str(99) == "unknown status"


def test_out_size(lib):
    assert cf.out_size(5, 3) == 3                       # the pages' 1D example
    assert cf.out_size(56, 5, 2, 2, 1) == 28
    assert cf.out_size(112, 3, 2, 1, 1) == 56
    assert cf.out_size(7, 5, 1, 2, 1) == 7
    assert cf.out_size(3, 5) <= 0
    assert cf.out_size(0, 1) <= 0 and cf.out_size(4, 1, 0) <= 0 and cf.out_size(4, 1, 1, -1) <= 0


# Fake, widely separated device addresses: validation only compares them.
XA, FA, BA, YA = 0x10000000, 0x20000000, 0x30000000, 0x40000000


def dense(lib, X=XA, xs=None, F=FA, bias=None, Y=YA, ys=None, shape=(2, 8, 8, 3, 3, 3, 4), xdt=0, ydt=0,
          variant=0):
    N, H, W, Cin, KH, KW, Cout = shape
    xs_arr = None if xs is None else (ctypes.c_int64 * 4)(*xs)
    ys_arr = None if ys is None else (ctypes.c_int64 * 4)(*ys)
    return lib.conv2d_nhwc_fwd_variant(X, xs_arr, F, bias, Y, ys_arr, N, H, W, Cin, KH, KW, Cout, xdt, ydt,
                                       variant, None)


def test_dense_errors(lib):
    assert dense(lib, X=None) == cf.CONV_ERR_NULL
    assert dense(lib, F=None) == cf.CONV_ERR_NULL
    assert dense(lib, Y=None) == cf.CONV_ERR_NULL
    for i in range(7):
        shape = [2, 8, 8, 3, 3, 3, 4]
        shape[i] = 0
        assert dense(lib, shape=tuple(shape)) == cf.CONV_ERR_NONPOSITIVE
        shape[i] = -1
        assert dense(lib, shape=tuple(shape)) == cf.CONV_ERR_NONPOSITIVE
    assert dense(lib, shape=(1, 2, 8, 3, 3, 3, 4)) == cf.CONV_ERR_SHAPE       # KH > H
    assert dense(lib, shape=(1, 8, 2, 3, 3, 3, 4)) == cf.CONV_ERR_SHAPE       # KW > W
    assert dense(lib, xdt=2) == cf.CONV_ERR_DTYPE
    assert dense(lib, ydt=7) == cf.CONV_ERR_DTYPE
    assert dense(lib, xdt=cf.CONV_F32, ydt=cf.CONV_BF16) == cf.CONV_ERR_DTYPE
    assert dense(lib, xs=(192, 24, 3, 2)) == cf.CONV_ERR_LAYOUT               # channel stride != 1
    assert dense(lib, xs=(192, -24, 3, 1)) == cf.CONV_ERR_LAYOUT              # negative stride
    assert dense(lib, ys=(144, 24, 4, 2)) == cf.CONV_ERR_LAYOUT
    assert dense(lib, ys=(144, 24, 3, 1)) == cf.CONV_ERR_LAYOUT               # pixels overlap (sW < Cout)
    assert dense(lib, ys=(144, 20, 4, 1)) == cf.CONV_ERR_LAYOUT               # rows overlap
    assert dense(lib, ys=(100, 24, 4, 1)) == cf.CONV_ERR_LAYOUT               # images overlap
    # Y overlapping X (element 5 of X), F or bias.
    assert dense(lib, Y=XA + 20) == cf.CONV_ERR_ALIAS
    assert dense(lib, Y=FA - 8) == cf.CONV_ERR_ALIAS
    assert dense(lib, bias=YA + 4) == cf.CONV_ERR_ALIAS
    # X is read-only: overlapping X and F, or a zero stride in X, is legal.
    assert dense(lib, F=XA + 4, variant=99) == cf.CONV_ERR_UNSUPPORTED
    assert dense(lib, xs=(0, 24, 3, 1), variant=99) == cf.CONV_ERR_UNSUPPORTED
    assert dense(lib, variant=99) == cf.CONV_ERR_UNSUPPORTED


def dw(lib, X=XA, w=FA, bias=None, Y=YA, shape=(8, 72, 56, 56, 1, 5, 5, 2, 2, 2, 2, 1, 1), mode=0, variant=0):
    return lib.conv_depthwise_fwd_variant(X, w, bias, Y, *shape, mode, variant, None)


def test_depthwise_errors(lib):
    assert dw(lib, X=None) == cf.CONV_ERR_NULL
    assert dw(lib, w=None) == cf.CONV_ERR_NULL
    assert dw(lib, Y=None) == cf.CONV_ERR_NULL
    base = [8, 72, 56, 56, 1, 5, 5, 2, 2, 2, 2, 1, 1]
    for i in range(7):                        # sizes, multiplier, KH, KW
        s = list(base)
        s[i] = 0
        assert dw(lib, shape=tuple(s)) == cf.CONV_ERR_NONPOSITIVE
    for i in (7, 8, 11, 12):                  # stride, dilation < 1
        s = list(base)
        s[i] = 0
        assert dw(lib, shape=tuple(s)) == cf.CONV_ERR_NONPOSITIVE
    for i in (9, 10):                         # padding < 0
        s = list(base)
        s[i] = -1
        assert dw(lib, shape=tuple(s)) == cf.CONV_ERR_NONPOSITIVE
    assert dw(lib, shape=(1, 1, 3, 3, 1, 5, 5, 1, 1, 0, 0, 1, 1)) == cf.CONV_ERR_SHAPE
    assert dw(lib, shape=(1, 1, 7, 7, 1, 3, 3, 1, 1, 0, 0, 4, 1)) == cf.CONV_ERR_SHAPE   # dilated span 9 > 7
    assert dw(lib, mode=2) == cf.CONV_ERR_UNSUPPORTED
    assert dw(lib, Y=XA + 4096) == cf.CONV_ERR_ALIAS
    assert dw(lib, bias=YA) == cf.CONV_ERR_ALIAS
    assert dw(lib, w=YA + 8) == cf.CONV_ERR_ALIAS
    assert dw(lib, variant=99) == cf.CONV_ERR_UNSUPPORTED


def test_copy_errors(lib):
    assert lib.conv_copy_bytes(None, YA, 16, None) == cf.CONV_ERR_NULL
    assert lib.conv_copy_bytes(XA, YA, -1, None) == cf.CONV_ERR_NONPOSITIVE
    assert lib.conv_copy_bytes(XA, XA + 8, 16, None) == cf.CONV_ERR_ALIAS
    assert lib.conv_copy_bytes(XA, YA, 0, None) == cf.CONV_OK        # nothing enqueued
    assert lib.conv_copy_bytes_wide(None, YA, 16, None) == cf.CONV_ERR_NULL
    assert lib.conv_copy_bytes_wide(XA, YA, -16, None) == cf.CONV_ERR_NONPOSITIVE
    assert lib.conv_copy_bytes_wide(XA, YA, 24, None) == cf.CONV_ERR_LAYOUT
    assert lib.conv_copy_bytes_wide(XA + 8, YA, 16, None) == cf.CONV_ERR_LAYOUT
    assert lib.conv_copy_bytes_wide(XA, XA + 16, 32, None) == cf.CONV_ERR_ALIAS
    assert lib.conv_copy_bytes_wide(XA, YA, 0, None) == cf.CONV_OK


def dq_shape(lib, N, C, H, W, m, KH, KW, sh, sw, ph, pw, dh, dw, X=XA):
    return lib.conv_depthwise_auto_variant(X, FA, None, YA, N, C, H, W, m, KH, KW, sh, sw, ph, pw, dh, dw,
                                           cf.CONV_DW_EXACT)


def test_auto_variant_queries(lib):
    q = lambda N=2, X=XA, F=FA, Y=YA, ys=None, xdt=0, ydt=0, C=3, O=4: lib.conv2d_nhwc_auto_variant(
        X, None, F, None, Y, ys, N, 8, 8, C, 3, 3, O, xdt, ydt)
    assert q(N=0) == -1
    assert q(X=None) == -1 and q(F=None) == -1
    assert q() in (cf.VARIANT_DIRECT, cf.VARIANT_TILED)
    assert q(Y=XA + 8) == -1                               # the call would fail with CONV_ERR_ALIAS
    assert dq_shape(lib, 1, 1, 3, 3, 1, 5, 5, 1, 1, 0, 0, 1, 1) == -1
    # Every measured depthwise workload runs on the LDS-tiled kernel.
    import workloads as wl
    for l in (wl.DW_5X5S2_EXACT, *wl.DW_SWEEP):
        v = dq_shape(lib, l.N, l.C, l.H, l.W, l.mult, l.KH, l.KW, l.stride, l.stride, l.pad, l.pad, l.dil, l.dil)
        assert v == cf.VARIANT_TILED, l.name
    # An input that is not 16-byte aligned: planes small enough for whole
    # planes per workgroup still run tiled (that kernel reads X four bytes at
    # a time); the large-plane kernels need 16-byte rows and fall back.
    l = wl.DW_5X5S2_EXACT
    assert dq_shape(lib, l.N, l.C, l.H, l.W, 1, 5, 5, 2, 2, 2, 2, 1, 1, X=XA + 4) == cf.VARIANT_TILED
    l = wl.DW_SWEEP[0]
    assert dq_shape(lib, l.N, l.C, l.H, l.W, 1, 3, 3, 1, 1, 1, 1, 1, 1, X=XA + 4) == cf.VARIANT_DIRECT
    # Shapes the tiled kernel does not take fall back to the direct kernel.
    assert dq_shape(lib, 2, 4, 11, 11, 3, 3, 3, 3, 3, 0, 0, 1, 1) == cf.VARIANT_DIRECT
    assert dq_shape(lib, 1, 2, 19, 23, 1, 3, 3, 1, 1, 2, 2, 2, 2) == cf.VARIANT_DIRECT


def test_dense_query_sees_output_layout(lib):
    """The dense query takes the call's own F, Y and Y strides: a bf16 3x3
    layer runs tiled into an aligned, contiguous output and on the direct
    kernel when Y (or F for fp32) is misaligned or Y's pixel stride breaks the
    kernels' 16-byte pieces."""
    BF = cf.CONV_BF16
    ys = lambda *v: (ctypes.c_int64 * 4)(*v)
    q = lambda Y=YA, y_strides=None, F=FA, dt=BF: lib.conv2d_nhwc_auto_variant(
        XA, None, F, None, Y, y_strides, 2, 12, 12, 64, 3, 3, 64, dt, dt)
    assert q() == cf.VARIANT_TILED
    assert q(Y=None) == cf.VARIANT_TILED                      # a fresh output
    assert q(Y=YA + 2) == cf.VARIANT_DIRECT                   # 2-byte aligned Y
    assert q(y_strides=ys(10 * 10 * 68, 10 * 68, 68, 1)) == cf.VARIANT_DIRECT   # pixel stride 68 bf16
    assert q(y_strides=ys(10 * 10 * 72, 10 * 72, 72, 1)) == cf.VARIANT_TILED    # pixel stride 72 bf16


def test_extents_past_the_addressable_range(lib):
    """Strided extents whose byte size overflows (or passes 2^60) are layout
    errors, checked with overflow-safe arithmetic before anything else."""
    big = (ctypes.c_int64 * 4)(1 << 40, 1 << 40, 1 << 40, 1)
    n = 2 ** 31 - 1                                  # (n - 1) * 2^40 overflows int64
    st = lib.conv2d_nhwc_fwd(XA, big, FA, None, YA, None, n, n, n, 8, 1, 1, 8, cf.CONV_BF16, cf.CONV_BF16, None)
    assert st == cf.CONV_ERR_LAYOUT
    # 2^20 * 2^40 * 2 bytes = 2^61 > 2^60 without overflowing int64
    mid = (ctypes.c_int64 * 4)(1 << 40, 1 << 30, 8, 1)
    st = lib.conv2d_nhwc_fwd(XA, mid, FA, None, YA, None, 2 ** 20 + 1, 4, 4, 8, 1, 1, 8, cf.CONV_BF16, cf.CONV_BF16,
                             None)
    assert st == cf.CONV_ERR_LAYOUT
    ybig = (ctypes.c_int64 * 4)(1 << 40, 1 << 30, 8, 1)
    st = lib.conv2d_nhwc_fwd(XA, None, FA, None, YA, ybig, 2 ** 20 + 1, 4, 4, 8, 1, 1, 8, cf.CONV_BF16,
                             cf.CONV_BF16, None)
    assert st == cf.CONV_ERR_LAYOUT
    # contiguous, but N*H*W*Cin*2 bytes is far past 2^60
    st = lib.conv2d_nhwc_fwd(XA, None, FA, None, YA, None, 2 ** 31 - 1, 2 ** 31 - 1, 2 ** 31 - 1, 8, 1, 1, 8,
                             cf.CONV_BF16, cf.CONV_BF16, None)
    assert st == cf.CONV_ERR_LAYOUT
    st = lib.conv_depthwise_fwd(XA, FA, None, YA, 2 ** 31 - 1, 2 ** 31 - 1, 2 ** 20, 2 ** 20, 1, 3, 3, 1, 1, 1, 1,
                                1, 1, cf.CONV_DW_EXACT, None)
    assert st == cf.CONV_ERR_UNSUPPORTED


def test_binding_rejects_cpu_tensors(lib):
    import torch
    x = torch.zeros(1, 4, 4, 8)
    f = torch.zeros(3, 3, 8, 8)
    with pytest.raises(ValueError):
        cf.conv2d_nhwc(x, f)
    with pytest.raises(ValueError):
        cf.conv_depthwise(torch.zeros(1, 2, 4, 4), torch.zeros(2, 3, 3))


def test_window_entry_points(lib):
    """The window entry points: the same argument classes, checked before any
    HIP call (fake device addresses are never dereferenced)."""
    XA, FA, YA = 0x10000000, 0x20000000, 0x30000000
    W = cf.window
    call = lambda win, **k: lib.conv2d_nhwc_fwd_window(
        XA, None, FA, None, YA, None, k.get("N", 1), k.get("H", 8), k.get("Wd", 8), k.get("Cin", 6),
        k.get("KH", 3), k.get("KW", 3), k.get("Cout", 6), ctypes.byref(win) if win is not None else None,
        cf.CONV_F32, cf.CONV_F32, cf.VARIANT_AUTO, None)
    assert call(None) == cf.CONV_ERR_NULL
    assert call(W(stride=0)) == cf.CONV_ERR_NONPOSITIVE
    assert call(W(dilation=(1, 0))) == cf.CONV_ERR_NONPOSITIVE
    assert call(W(padding=(0, 0, -1, 0))) == cf.CONV_ERR_NONPOSITIVE
    assert call(W(groups=0)) == cf.CONV_ERR_NONPOSITIVE
    assert call(W(groups=4)) == cf.CONV_ERR_SHAPE                  # 4 does not divide 6
    assert call(W(dilation=5)) == cf.CONV_ERR_SHAPE                # window spans 11 > 8
    assert call(W(dilation=5, padding=2)) != cf.CONV_ERR_SHAPE     # 8 + 4 >= 11: one output
    # Y overlapping F: F holds KH*KW*(Cin/groups)*Cout floats.
    F_end = FA + 3 * 3 * 2 * 6 * 4
    st = lib.conv2d_nhwc_fwd_window(XA, None, FA, None, F_end - 4, None, 1, 8, 8, 6, 3, 3, 6,
                                    ctypes.byref(W(groups=3)), cf.CONV_F32, cf.CONV_F32, cf.VARIANT_AUTO, None)
    assert st == cf.CONV_ERR_ALIAS
    # depthwise: groups must be 1, asymmetric pads accepted
    dw = lambda win: lib.conv_depthwise_fwd_window(XA, FA, None, YA, 1, 2, 1, 9, 1, 1, 4,
                                                   ctypes.byref(win) if win is not None else None,
                                                   cf.CONV_DW_EXACT, cf.VARIANT_AUTO, None)
    assert dw(None) == cf.CONV_ERR_NULL
    assert dw(W(groups=2)) == cf.CONV_ERR_UNSUPPORTED
    assert dw(W(padding=(0, 0, -1, 0))) == cf.CONV_ERR_NONPOSITIVE
    assert dw(W(padding=(0, 0, 0, 0), dilation=(1, 3))) == cf.CONV_ERR_SHAPE


def test_out_size_window(lib):
    assert cf.out_size_window(5, 3) == 3
    assert cf.out_size_window(11, 4, 1, 3, 0, 1) == 11           # causal: K-1 before, none after
    assert cf.out_size_window(11, 4, 1, 6, 0, 2) == 11           # dilated causal
    assert cf.out_size_window(224, 16, 16, 0, 0, 1) == 14        # patch stem
    assert cf.out_size_window(7, 3, 2, 1, 0, 1) == 3
    assert cf.out_size_window(7, 3, 2, 1, 1, 1) == 4
    assert cf.out_size_window(2, 5, 1, 0, 0, 1) == 0
    assert cf.out_size_window(5, 3, 1, -1, 0, 1) == 0
    for n, k, s, p, d in [(56, 5, 2, 2, 1), (112, 3, 2, 1, 1), (7, 5, 1, 2, 1), (9, 3, 2, 4, 3)]:
        assert cf.out_size_window(n, k, s, p, p, d) == cf.out_size(n, k, s, p, d)


def test_window_auto_variants(lib):
    """Windows of any shape go to a matrix-core kernel (a dilated bf16 window
    to the streamed-filter GEMM, an fp32 one to the fp32 GEMM kernel). The
    plain window through the window entry point is routed like
    conv2d_nhwc_fwd."""
    W = cf.window
    q = lambda win, dt=cf.CONV_BF16, **k: lib.conv2d_nhwc_window_auto_variant(
        XA, None, FA, None, YA, None, k.get("N", 2), k.get("H", 12), k.get("Wd", 12), 64, 3, 3, 64, ctypes.byref(win),
        dt, dt)
    assert q(W()) == lib.conv2d_nhwc_auto_variant(XA, None, FA, None, YA, None, 2, 12, 12, 64, 3, 3, 64, cf.CONV_BF16,
                                                  cf.CONV_BF16)
    assert q(W(groups=0)) == -1
    assert q(W(padding=1, dilation=2)) == cf.VARIANT_TILED
    assert q(W(padding=1, dilation=2), cf.CONV_F32) == cf.VARIANT_TILED
    assert q(W(stride=2, padding=3, groups=4), cf.CONV_F32) == cf.VARIANT_TILED
    dq = lambda win: lib.conv_depthwise_window_auto_variant(XA, FA, None, YA, 8, 72, 56, 56, 1, 5, 5,
                                                            ctypes.byref(win), cf.CONV_DW_EXACT)
    assert dq(W(stride=2, padding=2)) == dq_shape(lib, 8, 72, 56, 56, 1, 5, 5, 2, 2, 2, 2, 1, 1)
    assert dq(W(groups=2)) == -1


def test_im2col_errors(lib):
    XA, CA = 0x10000000, 0x50000000
    W = cf.window
    call = lambda X, cols, win, **k: lib.conv_im2col_nhwc(
        X, None, cols, k.get("N", 1), k.get("H", 6), k.get("Wd", 6), k.get("Cin", 4), k.get("KH", 3), k.get("KW", 3),
        ctypes.byref(win) if win is not None else None, k.get("dt", cf.CONV_F32), None)
    assert call(0, CA, W()) == cf.CONV_ERR_NULL
    assert call(XA, 0, W()) == cf.CONV_ERR_NULL
    assert call(XA, CA, None) == cf.CONV_ERR_NULL
    assert call(XA, CA, W(groups=2)) == cf.CONV_ERR_UNSUPPORTED
    assert call(XA, CA, W(), H=2) == cf.CONV_ERR_SHAPE
    assert call(XA, CA, W(), Cin=0) == cf.CONV_ERR_NONPOSITIVE
    assert call(XA, CA, W(), dt=7) == cf.CONV_ERR_DTYPE
    assert call(XA, XA + 64, W()) == cf.CONV_ERR_ALIAS
