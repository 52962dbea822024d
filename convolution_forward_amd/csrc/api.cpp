// C ABI of the convolution library: argument validation, output shapes,
// variant choice and launch. Every argument error is returned before the
// first HIP call; kernels are enqueued on the caller's stream and nothing is
// allocated or synchronised here.
#include <limits.h>
#include <stdint.h>

#include "internal.h"

using namespace convfwd;

namespace {

bool dtype_known(conv_dtype d) { return d == CONV_F32 || d == CONV_BF16; }

int64_t dtype_size(conv_dtype d) { return d == CONV_BF16 ? 2 : 4; }

// Half-open byte range [lo, hi) touched by a strided 4-D tensor with
// non-negative strides.
struct Range {
    uintptr_t lo, hi;
};

// Largest byte extent of a tensor the library addresses. Kernels form
// element and byte offsets as int64 sums of index * stride terms, each no
// larger than the extent, so every such sum stays far from overflow.
constexpr int64_t MAX_EXTENT_BYTES = int64_t(1) << 60;

// Bytes from the first to one past the last element of a strided 4-D
// tensor (sizes >= 1, strides >= 0), or -1 when that exceeds
// MAX_EXTENT_BYTES (or int64 arithmetic would overflow on the way).
int64_t strided_extent(const int64_t *dims, const int64_t *strides, int64_t esize)
{
    int64_t last = 0;
    for (int d = 0; d < 4; ++d) {
        int64_t term;
        if (__builtin_mul_overflow(dims[d] - 1, strides[d], &term) || __builtin_add_overflow(last, term, &last))
            return -1;
    }
    int64_t bytes;
    if (__builtin_add_overflow(last, (int64_t)1, &last) || __builtin_mul_overflow(last, esize, &bytes) ||
        bytes > MAX_EXTENT_BYTES)
        return -1;
    return bytes;
}

Range strided_range(const void *base, int64_t extent_bytes)
{
    uintptr_t lo = (uintptr_t)base;
    return Range{lo, lo + (uintptr_t)extent_bytes};
}

// Bytes of a contiguous fp32 tensor of a*b*c*d elements (sizes >= 1), or -1
// past MAX_EXTENT_BYTES.
int64_t flat_bytes4(int64_t a, int64_t b, int64_t c, int64_t d)
{
    int64_t n;
    if (__builtin_mul_overflow(a, b, &n) || __builtin_mul_overflow(n, c, &n) || __builtin_mul_overflow(n, d, &n) ||
        __builtin_mul_overflow(n, (int64_t)4, &n) || n > MAX_EXTENT_BYTES)
        return -1;
    return n;
}

Range flat_range(const void *base, int64_t bytes)
{
    uintptr_t lo = (uintptr_t)base;
    return Range{lo, lo + (uintptr_t)bytes};
}

bool overlaps(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

// Products of sizes must stay far from int64 overflow; every size here is an
// int, so four of them fit, but stride arithmetic is checked separately.
bool stride_ok(int64_t s) { return s >= 0 && s <= (int64_t(1) << 40); }

// The lecture's restricted window: unit stride, no padding, one group.
constexpr conv_window PLAIN_WINDOW = {1, 1, 0, 0, 0, 0, 1, 1, 1};

// Shape, window, dtype and layout checks (no pointer checks); fills p
// except pointers.
conv_status check_dense_shape(const int64_t *x_strides, const int64_t *y_strides, int N, int H, int W,
                              int Cin, int KH, int KW, int Cout, const conv_window &win, conv_dtype x_dtype,
                              conv_dtype y_dtype, DenseProblem *p)
{
    if (N <= 0 || H <= 0 || W <= 0 || Cin <= 0 || KH <= 0 || KW <= 0 || Cout <= 0)
        return CONV_ERR_NONPOSITIVE;
    if (win.stride_h < 1 || win.stride_w < 1 || win.dil_h < 1 || win.dil_w < 1 || win.groups < 1 ||
        win.pad_top < 0 || win.pad_bottom < 0 || win.pad_left < 0 || win.pad_right < 0)
        return CONV_ERR_NONPOSITIVE;
    const int64_t Ho64 = conv_out_size_window(H, KH, win.stride_h, win.pad_top, win.pad_bottom, win.dil_h);
    const int64_t Wo64 = conv_out_size_window(W, KW, win.stride_w, win.pad_left, win.pad_right, win.dil_w);
    if (Ho64 <= 0 || Wo64 <= 0 || Cin % win.groups != 0 || Cout % win.groups != 0)
        return CONV_ERR_SHAPE;
    if (Ho64 > INT_MAX || Wo64 > INT_MAX)
        return CONV_ERR_UNSUPPORTED;
    if (!dtype_known(x_dtype) || !dtype_known(y_dtype))
        return CONV_ERR_DTYPE;
    if (x_dtype == CONV_F32 && y_dtype == CONV_BF16)
        return CONV_ERR_DTYPE;
    const int Ho = (int)Ho64, Wo = (int)Wo64;

    int64_t xs[4], ys[4];
    if (x_strides) {
        for (int d = 0; d < 4; ++d) {
            if (!stride_ok(x_strides[d]))
                return CONV_ERR_LAYOUT;
            xs[d] = x_strides[d];
        }
        if (xs[3] != 1)
            return CONV_ERR_LAYOUT;
    } else {
        xs[3] = 1;
        xs[2] = Cin;
        xs[1] = (int64_t)W * Cin;
        xs[0] = (int64_t)H * W * Cin;
    }
    const int64_t xdims[4] = {N, H, W, Cin};
    if (strided_extent(xdims, xs, dtype_size(x_dtype)) < 0)
        return CONV_ERR_LAYOUT;
    if (y_strides) {
        for (int d = 0; d < 4; ++d) {
            if (!stride_ok(y_strides[d]))
                return CONV_ERR_LAYOUT;
            ys[d] = y_strides[d];
        }
        // No self-overlap: each coarser axis steps past the whole extent of the finer ones.
        const int64_t pix = Cout;
        const int64_t row = (int64_t)(Wo - 1) * ys[2] + pix;
        const int64_t img = (int64_t)(Ho - 1) * ys[1] + row;
        if (ys[3] != 1 || ys[2] < pix || ys[1] < row || (N > 1 && ys[0] < img))
            return CONV_ERR_LAYOUT;
    } else {
        ys[3] = 1;
        ys[2] = Cout;
        ys[1] = (int64_t)Wo * Cout;
        ys[0] = (int64_t)Ho * Wo * Cout;
    }
    const int64_t ydims[4] = {N, Ho, Wo, Cout};
    if (strided_extent(ydims, ys, dtype_size(y_dtype)) < 0)
        return CONV_ERR_LAYOUT;

    p->X = nullptr;
    p->F = nullptr;
    p->bias = nullptr;
    p->Y = nullptr;
    for (int d = 0; d < 4; ++d) {
        p->xs[d] = xs[d];
        p->ys[d] = ys[d];
    }
    p->N = N;
    p->H = H;
    p->W = W;
    p->Cin = Cin;
    p->KH = KH;
    p->KW = KW;
    p->Cout = Cout;
    p->Ho = Ho;
    p->Wo = Wo;
    p->xdt = x_dtype;
    p->ydt = y_dtype;
    p->sh = win.stride_h;
    p->sw = win.stride_w;
    p->pt = win.pad_top;
    p->pl = win.pad_left;
    p->dh = win.dil_h;
    p->dw = win.dil_w;
    p->groups = win.groups;
    return CONV_OK;
}

conv_status validate_dense(const void *X, const int64_t *x_strides, const void *F, const float *bias,
                           void *Y, const int64_t *y_strides, int N, int H, int W, int Cin, int KH,
                           int KW, int Cout, const conv_window &win, conv_dtype x_dtype, conv_dtype y_dtype,
                           DenseProblem *p)
{
    if (!X || !F || !Y)
        return CONV_ERR_NULL;
    conv_status st =
        check_dense_shape(x_strides, y_strides, N, H, W, Cin, KH, KW, Cout, win, x_dtype, y_dtype, p);
    if (st != CONV_OK)
        return st;
    const int64_t xdims[4] = {N, H, W, Cin};
    const int64_t ydims[4] = {N, p->Ho, p->Wo, Cout};
    // Both extents were checked by check_dense_shape.
    const Range ry = strided_range(Y, strided_extent(ydims, p->ys, dtype_size(y_dtype)));
    if (overlaps(ry, strided_range(X, strided_extent(xdims, p->xs, dtype_size(x_dtype)))) ||
        overlaps(ry, flat_range(F, (int64_t)KH * KW * (Cin / win.groups) * Cout * dtype_size(x_dtype))) ||
        (bias && overlaps(ry, flat_range(bias, (int64_t)Cout * 4))))
        return CONV_ERR_ALIAS;
    p->X = X;
    p->F = F;
    p->bias = bias;
    p->Y = Y;
    return CONV_OK;
}

// The tiled (matrix-core) variant: one kernel family per operand type.
bool dense_tiled_supports(const DenseProblem &p)
{
    if (p.xdt == CONV_BF16)
        return dense_mfma_bf16_supports(p) || dense_gemm_bf16_supports(p);
    return (plain_window(p) && dense_mfma_f32_supports(p)) || dense_gemm_f32_supports(p);
}

// The row kernel where its plan fits (band rows in LDS, filter in
// registers; fp32 only for the lecture's plain window), else the GEMM
// kernel of the operand type.
hipError_t launch_dense_tiled(const DenseProblem &p, hipStream_t s)
{
    if (p.xdt != CONV_BF16) {
        // fp32 1x1 layers: three bf16 parts per value on the bf16 matrix
        // cores (dense_pw_f32x6.hip).
        if (dense_f32x6_supports(p))
            return launch_dense_f32x6(p, s);
        return plain_window(p) && dense_mfma_f32_supports(p) ? launch_dense_mfma_f32(p, s)
                                                              : launch_dense_gemm_f32(p, s);
    }
    // Strided windows whose groups fill 64-channel tiles: the GEMM kernel
    // (3x3 stride 2 -> 128 channels: 10.9 us against 16.9 on the row
    // kernel). Narrower groups stay with the row kernel's block-diagonal
    // packing.
    const bool strided = p.sh > 1 || p.sw > 1;
    const bool wide_groups = p.groups == 1 || (p.Cout / p.groups) % 64 == 0;
    if (strided && wide_groups && dense_gemm_bf16_supports(p))
        return launch_dense_gemm_bf16(p, s);
    if (dense_mfma_bf16_supports(p))
        return launch_dense_mfma_bf16(p, s);
    return launch_dense_gemm_bf16(p, s);
}

int dense_auto(const DenseProblem &p) { return dense_tiled_supports(p) ? CONV_VARIANT_TILED : CONV_VARIANT_DIRECT; }

// Shape and mode checks (no pointer checks); fills p except pointers.
conv_status check_dw_shape(int N, int C, int H, int W, int mult, int KH, int KW, int sh, int sw, int ph, int pb,
                           int pw, int pr, int dh, int dw, conv_dw_mode mode, DwProblem *p)
{
    if (N <= 0 || C <= 0 || H <= 0 || W <= 0 || mult <= 0 || KH <= 0 || KW <= 0 || sh < 1 || sw < 1 ||
        dh < 1 || dw < 1 || ph < 0 || pw < 0 || pb < 0 || pr < 0)
        return CONV_ERR_NONPOSITIVE;
    if (mode != CONV_DW_EXACT && mode != CONV_DW_FAST)
        return CONV_ERR_UNSUPPORTED;
    const int64_t Ho = conv_out_size_window(H, KH, sh, ph, pb, dh);
    const int64_t Wo = conv_out_size_window(W, KW, sw, pw, pr, dw);
    if (Ho <= 0 || Wo <= 0)
        return CONV_ERR_SHAPE;
    if (Ho > INT_MAX || Wo > INT_MAX)
        return CONV_ERR_UNSUPPORTED;
    if ((int64_t)C * mult > INT_MAX)
        return CONV_ERR_UNSUPPORTED;
    // Byte sizes of X, w and Y must be addressable (see MAX_EXTENT_BYTES).
    if (flat_bytes4(N, C, H, W) < 0 || flat_bytes4(1, (int64_t)C * mult, KH, KW) < 0 ||
        flat_bytes4(N, (int64_t)C * mult, Ho, Wo) < 0)
        return CONV_ERR_UNSUPPORTED;
    p->X = nullptr;
    p->w = nullptr;
    p->bias = nullptr;
    p->Y = nullptr;
    p->N = N;
    p->C = C;
    p->H = H;
    p->W = W;
    p->mult = mult;
    p->KH = KH;
    p->KW = KW;
    p->sh = sh;
    p->sw = sw;
    p->ph = ph;
    p->pw = pw;
    p->pb = pb;
    p->pr = pr;
    p->dh = dh;
    p->dw = dw;
    p->Ho = (int)Ho;
    p->Wo = (int)Wo;
    p->mode = mode;
    return CONV_OK;
}

conv_status validate_dw(const float *X, const float *w, const float *bias, float *Y, int N, int C, int H,
                        int W, int mult, int KH, int KW, int sh, int sw, int ph, int pb, int pw, int pr, int dh,
                        int dw, conv_dw_mode mode, DwProblem *p)
{
    if (!X || !w || !Y)
        return CONV_ERR_NULL;
    conv_status st = check_dw_shape(N, C, H, W, mult, KH, KW, sh, sw, ph, pb, pw, pr, dh, dw, mode, p);
    if (st != CONV_OK)
        return st;
    const int64_t Cout = (int64_t)C * mult;
    // Every size was checked by check_dw_shape.
    const Range ry = flat_range(Y, flat_bytes4(N, Cout, p->Ho, p->Wo));
    if (overlaps(ry, flat_range(X, flat_bytes4(N, C, H, W))) || overlaps(ry, flat_range(w, flat_bytes4(1, Cout, KH, KW))) ||
        (bias && overlaps(ry, flat_range(bias, Cout * 4))))
        return CONV_ERR_ALIAS;
    p->X = X;
    p->w = w;
    p->bias = bias;
    p->Y = Y;
    return CONV_OK;
}

int dw_auto(const DwProblem &p) { return dw_tiled_supports(p) ? CONV_VARIANT_TILED : CONV_VARIANT_DIRECT; }

conv_status launched(hipError_t e)
{
    if (e != hipSuccess)
        return CONV_ERR_HIP;
    return hipGetLastError() == hipSuccess ? CONV_OK : CONV_ERR_HIP;
}

}  // namespace

extern "C" {

int64_t conv_out_size(int64_t in, int k, int stride, int pad, int dil)
{
    if (in <= 0 || k <= 0 || stride <= 0 || pad < 0 || dil <= 0)
        return 0;
    const int64_t eff = (int64_t)dil * (k - 1) + 1;
    const int64_t span = in + 2 * (int64_t)pad - eff;
    if (span < 0)
        return 0;
    return span / stride + 1;
}

int64_t conv_out_size_window(int64_t in, int k, int stride, int pad_before, int pad_after, int dil)
{
    if (in <= 0 || k <= 0 || stride <= 0 || pad_before < 0 || pad_after < 0 || dil <= 0)
        return 0;
    const int64_t eff = (int64_t)dil * (k - 1) + 1;
    const int64_t span = in + (int64_t)pad_before + pad_after - eff;
    if (span < 0)
        return 0;
    return span / stride + 1;
}

const char *conv_status_str(conv_status s)
{
    switch (s) {
    case CONV_OK: return "ok";
    case CONV_ERR_NULL: return "a required pointer is NULL";
    case CONV_ERR_NONPOSITIVE: return "sizes must be positive, strides and dilations >= 1, padding >= 0";
    case CONV_ERR_SHAPE: return "the filter does not fit the input: no output position";
    case CONV_ERR_DTYPE: return "unsupported dtype combination";
    case CONV_ERR_LAYOUT: return "unsupported memory layout (channel stride must be 1, output must not overlap itself)";
    case CONV_ERR_ALIAS: return "the output overlaps an input";
    case CONV_ERR_UNSUPPORTED: return "arguments outside what this kernel handles";
    case CONV_ERR_HIP: return "HIP runtime error at launch";
    }
    return "unknown status";
}

conv_status conv2d_nhwc_fwd_window(const void *X, const int64_t *x_strides, const void *F, const float *bias,
                                   void *Y, const int64_t *y_strides, int N, int H, int W, int Cin, int KH, int KW,
                                   int Cout, const conv_window *win, conv_dtype x_dtype, conv_dtype y_dtype,
                                   int variant, void *stream)
{
    if (!win)
        return CONV_ERR_NULL;
    DenseProblem p;
    conv_status st = validate_dense(X, x_strides, F, bias, Y, y_strides, N, H, W, Cin, KH, KW, Cout, *win,
                                    x_dtype, y_dtype, &p);
    if (st != CONV_OK)
        return st;
    if (variant == CONV_VARIANT_AUTO)
        variant = dense_auto(p);
    hipStream_t s = (hipStream_t)stream;
    switch (variant) {
    case CONV_VARIANT_DIRECT:
        return launched(launch_dense_direct(p, s));
    case CONV_VARIANT_TILED:
        if (!dense_tiled_supports(p))
            return CONV_ERR_UNSUPPORTED;
        return launched(launch_dense_tiled(p, s));
    default:
        return CONV_ERR_UNSUPPORTED;
    }
}

conv_status conv2d_nhwc_fwd_variant(const void *X, const int64_t *x_strides, const void *F,
                                    const float *bias, void *Y, const int64_t *y_strides, int N, int H,
                                    int W, int Cin, int KH, int KW, int Cout, conv_dtype x_dtype,
                                    conv_dtype y_dtype, int variant, void *stream)
{
    // The lecture's precondition K <= min(H, W) is the window's Ho, Wo >= 1.
    return conv2d_nhwc_fwd_window(X, x_strides, F, bias, Y, y_strides, N, H, W, Cin, KH, KW, Cout, &PLAIN_WINDOW,
                                  x_dtype, y_dtype, variant, stream);
}

conv_status conv2d_nhwc_fwd(const void *X, const int64_t *x_strides, const void *F, const float *bias,
                            void *Y, const int64_t *y_strides, int N, int H, int W, int Cin, int KH,
                            int KW, int Cout, conv_dtype x_dtype, conv_dtype y_dtype, void *stream)
{
    return conv2d_nhwc_fwd_variant(X, x_strides, F, bias, Y, y_strides, N, H, W, Cin, KH, KW, Cout, x_dtype,
                                   y_dtype, CONV_VARIANT_AUTO, stream);
}

int conv2d_nhwc_window_auto_variant(const void *X, const int64_t *x_strides, const void *F, const float *bias,
                                    const void *Y, const int64_t *y_strides, int N, int H, int W, int Cin, int KH,
                                    int KW, int Cout, const conv_window *win, conv_dtype x_dtype, conv_dtype y_dtype)
{
    if (!win || !X || !F)
        return -1;
    DenseProblem p;
    if (Y) {
        // Exactly the checks of the call itself, aliasing included.
        if (validate_dense(X, x_strides, F, bias, const_cast<void *>(Y), y_strides, N, H, W, Cin, KH, KW, Cout,
                           *win, x_dtype, y_dtype, &p) != CONV_OK)
            return -1;
    } else {
        // A fresh contiguous output, 256-byte aligned, that the caller has
        // yet to allocate.
        if (check_dense_shape(x_strides, nullptr, N, H, W, Cin, KH, KW, Cout, *win, x_dtype, y_dtype, &p) != CONV_OK)
            return -1;
        p.X = X;
        p.F = F;
        p.bias = bias;
        p.Y = reinterpret_cast<void *>(uintptr_t(256));
    }
    return dense_auto(p);
}

int conv2d_nhwc_auto_variant(const void *X, const int64_t *x_strides, const void *F, const float *bias, const void *Y,
                             const int64_t *y_strides, int N, int H, int W, int Cin, int KH, int KW, int Cout,
                             conv_dtype x_dtype, conv_dtype y_dtype)
{
    return conv2d_nhwc_window_auto_variant(X, x_strides, F, bias, Y, y_strides, N, H, W, Cin, KH, KW, Cout,
                                           &PLAIN_WINDOW, x_dtype, y_dtype);
}

conv_status conv_depthwise_fwd_window(const float *X, const float *w, const float *bias, float *Y, int N, int C,
                                      int H, int W, int multiplier, int KH, int KW, const conv_window *win,
                                      conv_dw_mode mode, int variant, void *stream)
{
    if (!win)
        return CONV_ERR_NULL;
    if (win->groups != 1)
        return CONV_ERR_UNSUPPORTED;
    DwProblem p;
    conv_status st = validate_dw(X, w, bias, Y, N, C, H, W, multiplier, KH, KW, win->stride_h, win->stride_w,
                                 win->pad_top, win->pad_bottom, win->pad_left, win->pad_right, win->dil_h,
                                 win->dil_w, mode, &p);
    if (st != CONV_OK)
        return st;
    if (variant == CONV_VARIANT_AUTO)
        variant = dw_auto(p);
    hipStream_t s = (hipStream_t)stream;
    switch (variant) {
    case CONV_VARIANT_DIRECT:
        return launched(launch_dw_direct(p, s));
    case CONV_VARIANT_TILED:
        if (!dw_tiled_supports(p))
            return CONV_ERR_UNSUPPORTED;
        return launched(launch_dw_tiled(p, s));
    default:
        return CONV_ERR_UNSUPPORTED;
    }
}

conv_status conv_depthwise_fwd_variant(const float *X, const float *w, const float *bias, float *Y, int N,
                                       int C, int H, int W, int multiplier, int KH, int KW, int stride_h,
                                       int stride_w, int pad_h, int pad_w, int dil_h, int dil_w,
                                       conv_dw_mode mode, int variant, void *stream)
{
    const conv_window win = {stride_h, stride_w, pad_h, pad_h, pad_w, pad_w, dil_h, dil_w, 1};
    return conv_depthwise_fwd_window(X, w, bias, Y, N, C, H, W, multiplier, KH, KW, &win, mode, variant, stream);
}

conv_status conv_depthwise_fwd(const float *X, const float *w, const float *bias, float *Y, int N, int C, int H,
                               int W, int multiplier, int KH, int KW, int stride_h, int stride_w, int pad_h,
                               int pad_w, int dil_h, int dil_w, conv_dw_mode mode, void *stream)
{
    return conv_depthwise_fwd_variant(X, w, bias, Y, N, C, H, W, multiplier, KH, KW, stride_h, stride_w, pad_h,
                                      pad_w, dil_h, dil_w, mode, CONV_VARIANT_AUTO, stream);
}

int conv_depthwise_window_auto_variant(const float *X, const float *w, const float *bias, const float *Y, int N,
                                       int C, int H, int W, int multiplier, int KH, int KW, const conv_window *win,
                                       conv_dw_mode mode)
{
    if (!win || win->groups != 1)
        return -1;
    DwProblem p;
    if (validate_dw(X, w, bias, const_cast<float *>(Y), N, C, H, W, multiplier, KH, KW, win->stride_h,
                    win->stride_w, win->pad_top, win->pad_bottom, win->pad_left, win->pad_right, win->dil_h,
                    win->dil_w, mode, &p) != CONV_OK)
        return -1;
    return dw_auto(p);
}

int conv_depthwise_auto_variant(const float *X, const float *w, const float *bias, const float *Y, int N, int C,
                                int H, int W, int multiplier, int KH, int KW, int stride_h, int stride_w, int pad_h,
                                int pad_w, int dil_h, int dil_w, conv_dw_mode mode)
{
    const conv_window win = {stride_h, stride_w, pad_h, pad_h, pad_w, pad_w, dil_h, dil_w, 1};
    return conv_depthwise_window_auto_variant(X, w, bias, Y, N, C, H, W, multiplier, KH, KW, &win, mode);
}

conv_status conv_im2col_nhwc(const void *X, const int64_t *x_strides, void *cols, int N, int H, int W, int Cin,
                             int KH, int KW, const conv_window *win, conv_dtype dtype, void *stream)
{
    if (!X || !cols || !win)
        return CONV_ERR_NULL;
    if (win->groups != 1)
        return CONV_ERR_UNSUPPORTED;
    // The dense checks with Cout = 1 give the output shape and X's layout.
    DenseProblem d;
    const conv_status st = check_dense_shape(x_strides, nullptr, N, H, W, Cin, KH, KW, 1, *win, dtype, dtype, &d);
    if (st != CONV_OK)
        return st;
    const int64_t xdims[4] = {N, H, W, Cin};
    int64_t cols_bytes = 0;
    if (__builtin_mul_overflow((int64_t)N * d.Ho, (int64_t)d.Wo * KH, &cols_bytes) ||
        __builtin_mul_overflow(cols_bytes, (int64_t)KW * Cin * dtype_size(dtype), &cols_bytes) ||
        cols_bytes > MAX_EXTENT_BYTES)
        return CONV_ERR_UNSUPPORTED;
    if (overlaps(flat_range(cols, cols_bytes), strided_range(X, strided_extent(xdims, d.xs, dtype_size(dtype)))))
        return CONV_ERR_ALIAS;
    Im2colProblem p;
    p.X = X;
    for (int k = 0; k < 4; ++k)
        p.xs[k] = d.xs[k];
    p.cols = cols;
    p.N = N;
    p.H = H;
    p.W = W;
    p.Cin = Cin;
    p.KH = KH;
    p.KW = KW;
    p.Ho = d.Ho;
    p.Wo = d.Wo;
    p.sh = d.sh;
    p.sw = d.sw;
    p.pt = d.pt;
    p.pl = d.pl;
    p.dh = d.dh;
    p.dw = d.dw;
    p.dtype = dtype;
    return launched(launch_im2col(p, (hipStream_t)stream));
}

conv_status conv_copy_bytes(const void *src, void *dst, int64_t bytes, void *stream)
{
    if (!src || !dst)
        return CONV_ERR_NULL;
    if (bytes < 0)
        return CONV_ERR_NONPOSITIVE;
    if (overlaps(flat_range(src, bytes), flat_range(dst, bytes)))
        return CONV_ERR_ALIAS;
    if (bytes == 0)
        return CONV_OK;
    return launched(launch_copy_bytes(src, dst, bytes, (hipStream_t)stream));
}

conv_status conv_copy_bytes_wide(const void *src, void *dst, int64_t bytes, void *stream)
{
    if (!src || !dst)
        return CONV_ERR_NULL;
    if (bytes < 0)
        return CONV_ERR_NONPOSITIVE;
    if ((uintptr_t)src % 16 != 0 || (uintptr_t)dst % 16 != 0 || bytes % 16 != 0)
        return CONV_ERR_LAYOUT;
    if (bytes > (int64_t(1) << 40))
        return CONV_ERR_UNSUPPORTED;
    if (overlaps(flat_range(src, bytes), flat_range(dst, bytes)))
        return CONV_ERR_ALIAS;
    if (bytes == 0)
        return CONV_OK;
    return launched(launch_copy_wide(src, dst, bytes, (hipStream_t)stream));
}

}  // extern "C"
