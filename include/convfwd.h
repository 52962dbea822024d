/*
 * convfwd -- forward 2D convolution on AMD Instinct MI355X (gfx950).
 *
 * A C ABI over hand-written HIP kernels. Every argument is a plain pointer or
 * integer; device buffers are owned by the caller. The library never
 * allocates device memory and never synchronises: each call validates its
 * arguments on the host, then enqueues kernels on the caller's stream and
 * returns. Its only state is, per kernel and device, whether that kernel's
 * dynamic LDS limit has been raised (hipFuncSetAttribute, done on the first
 * launch there and remembered only once it succeeds); calls are thread-safe.
 *
 * Two operators:
 *
 *  - Dense NHWC cross-correlation, as fixed by "CMU DLSys Lecture 14:
 *    Convolutional Network Implementation", section 1 (the index contract):
 *    Y[n,y,x,o] = sum over i<KH, j<KW, c<Cin of X[n,y+i,x+j,c] * F[i,j,c,o],
 *    no flip, unit stride, no padding, Ho = H-KH+1, Wo = W-KW+1. The lecture
 *    uses square filters; KH and KW are separate here so that 1D filters
 *    (KH = 1) from "Convolution Is Wx+b Moving Across a Signal" run too.
 *
 *  - Depthwise convolution, as fixed by "Depthwise convolution" (onemodel
 *    docs), section "What each output is": one input channel per group,
 *    Cout = C * multiplier, output channel oc reads input channel
 *    oc / multiplier; stride, symmetric zero padding and dilation per axis;
 *    taps summed row-major starting from +0; exact or fast rounding.
 *
 * Return values: every function that can fail returns a conv_status. All
 * argument errors are detected before any HIP call, and then nothing is
 * written and nothing is enqueued. CONV_ERR_HIP reports a failed launch.
 */
#ifndef CONVFWD_H
#define CONVFWD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Exported symbols; everything else in the library is hidden. */
#if defined(__GNUC__) || defined(__clang__)
#define CONVFWD_API __attribute__((visibility("default")))
#else
#define CONVFWD_API
#endif

typedef enum conv_status {
    CONV_OK = 0,
    CONV_ERR_NULL = 1,          /* a required pointer is NULL */
    CONV_ERR_NONPOSITIVE = 2,   /* a size <= 0, stride or dilation < 1, or padding < 0 */
    CONV_ERR_SHAPE = 3,         /* the filter does not fit (no output position) */
    CONV_ERR_DTYPE = 4,         /* unknown dtype, or bf16 output requested from fp32 input */
    CONV_ERR_LAYOUT = 5,        /* a stride the operator cannot address (see each call) */
    CONV_ERR_ALIAS = 6,         /* the output's address range overlaps an input's */
    CONV_ERR_UNSUPPORTED = 7,   /* valid arguments outside what the (forced) kernel handles */
    CONV_ERR_HIP = 8            /* the HIP runtime reported an error at launch */
} conv_status;

typedef enum conv_dtype {
    CONV_F32 = 0,   /* IEEE binary32 */
    CONV_BF16 = 1   /* bfloat16 (upper half of a binary32) */
} conv_dtype;

typedef enum conv_dw_mode {
    CONV_DW_EXACT = 0,  /* round the product, then round the sum; NaN -> 0x7FC00000 */
    CONV_DW_FAST = 1    /* one fused multiply-add per tap */
} conv_dw_mode;

/* Kernel variants. CONV_VARIANT_AUTO picks by shape; the others force one
 * kernel family and return CONV_ERR_UNSUPPORTED if it cannot take the shape.
 * Every variant computes the same contract; dense variants may differ in
 * fp32 accumulation order only, depthwise variants give identical bits. */
enum {
    CONV_VARIANT_AUTO = 0,
    CONV_VARIANT_DIRECT = 1,     /* one thread per output, any legal shape */
    CONV_VARIANT_TILED = 2       /* dense: MFMA implicit GEMM; depthwise: LDS-staged tiles */
};

/*
 * conv2d_nhwc_fwd -- dense forward cross-correlation.
 *
 * Contract: "CMU DLSys Lecture 14", section 1 (above); the filter is used as
 * the matrix F.reshape(KH*KW*Cin, Cout) with rows in (i,j,c) order (section 5),
 * but no patch matrix is ever built: patches are gathered on the fly.
 *
 *   X          device pointer, logical NHWC [N,H,W,Cin], dtype x_dtype.
 *   x_strides  host array of 4 element strides (n,h,w,c), or NULL for the
 *              contiguous layout. Like the lecture's strided patch view, any
 *              non-negative strides are accepted as long as the channel
 *              stride is 1 (CONV_ERR_LAYOUT otherwise); X may be a view.
 *   F          device pointer, contiguous [KH,KW,Cin,Cout] (KKIO), dtype x_dtype.
 *   bias       device pointer to Cout fp32 values added to every output, or NULL.
 *   Y          device pointer, logical NHWC [N,Ho,Wo,Cout], dtype y_dtype.
 *   y_strides  host array of 4 element strides, or NULL for contiguous. The
 *              channel stride must be 1 and the layout must not overlap
 *              itself (sW >= Cout, sH >= (Wo-1)*sW + Cout,
 *              sN >= (Ho-1)*sH + (Wo-1)*sW + Cout); CONV_ERR_LAYOUT otherwise.
 *   x_dtype    CONV_F32 or CONV_BF16 (X and F share it).
 *   y_dtype    CONV_F32, or CONV_BF16 when x_dtype is CONV_BF16. Accumulation
 *              is fp32; bf16 output is rounded to nearest-even once at the end.
 *   stream     a hipStream_t (NULL = the default stream).
 *
 * Errors: CONV_ERR_NULL (X, F or Y NULL), CONV_ERR_NONPOSITIVE (any size
 * <= 0), CONV_ERR_SHAPE (KH > H or KW > W), CONV_ERR_DTYPE, CONV_ERR_LAYOUT
 * (also when X's or Y's strided byte extent passes 2^60 bytes),
 * CONV_ERR_ALIAS (Y's byte range overlaps X, F or bias), CONV_ERR_HIP.
 * Y is fully overwritten on success; nothing accumulates into it.
 */
CONVFWD_API conv_status conv2d_nhwc_fwd(const void *X, const int64_t *x_strides, const void *F, const float *bias,
                            void *Y, const int64_t *y_strides, int N, int H, int W, int Cin, int KH,
                            int KW, int Cout, conv_dtype x_dtype, conv_dtype y_dtype, void *stream);

/* conv2d_nhwc_fwd with a forced kernel variant (CONV_VARIANT_*). With bf16
 * operands the MFMA variant needs X with a 16-byte-aligned base and 16-byte
 * aligned pixel strides (8 channels), and Cin and Cout that are multiples of
 * 8. With fp32 operands it takes any layout, window and channel count as
 * long as N*Ho*Wo, KH*KW*Cin and Cout stay below 2^31 - 64. Otherwise it returns
 * CONV_ERR_UNSUPPORTED. */
CONVFWD_API conv_status conv2d_nhwc_fwd_variant(const void *X, const int64_t *x_strides, const void *F,
                                    const float *bias, void *Y, const int64_t *y_strides, int N, int H,
                                    int W, int Cin, int KH, int KW, int Cout, conv_dtype x_dtype,
                                    conv_dtype y_dtype, int variant, void *stream);

/*
 * conv_depthwise_fwd -- depthwise forward convolution, fp32, NCHW planes.
 *
 * Contract: "Depthwise convolution" (onemodel docs), section "What each
 * output is". For output plane (n, oc), input plane (n, oc / multiplier):
 *   acc = +0; for ky < KH: for kx < KW:
 *     acc = acc + w[oc,ky,kx] * xpad[oy*stride_h + ky*dil_h, ox*stride_w + kx*dil_w]
 * where xpad is the input plane with pad_h / pad_w rows / columns of real
 * zeros on each side (a padding tap is a multiplication by +0, so an
 * infinite or NaN weight there yields NaN). Output size per axis follows
 * conv_out_size.
 *   mode CONV_DW_EXACT: each product and each sum rounded to fp32 separately,
 *        in the row-major order above; a NaN result becomes 0x7FC00000.
 *   mode CONV_DW_FAST: acc = fma(w, x, acc) per tap, same order.
 *   bias (nullable, Cout fp32): one rounded addition per output after the
 *        taps (and before the NaN rewrite of exact mode).
 * Results are bit-identical across kernel variants and launches.
 *
 *   X  device, contiguous [N,C,H,W] fp32.   w  device, contiguous [C*multiplier,KH,KW] fp32.
 *   Y  device, contiguous [N,C*multiplier,Ho,Wo] fp32, fully overwritten.
 *
 * Errors: CONV_ERR_NULL (X, w or Y NULL), CONV_ERR_NONPOSITIVE (a size or
 * multiplier <= 0, stride or dilation < 1, padding < 0), CONV_ERR_SHAPE (an
 * output size <= 0), CONV_ERR_UNSUPPORTED (unknown mode, a tensor past 2^60
 * bytes, or a forced variant that cannot take the shape), CONV_ERR_ALIAS (Y
 * overlaps X, w or bias),
 * CONV_ERR_HIP.
 */
CONVFWD_API conv_status conv_depthwise_fwd(const float *X, const float *w, const float *bias, float *Y, int N, int C,
                               int H, int W, int multiplier, int KH, int KW, int stride_h, int stride_w,
                               int pad_h, int pad_w, int dil_h, int dil_w, conv_dw_mode mode,
                               void *stream);

/* conv_depthwise_fwd with a forced kernel variant (CONV_VARIANT_*). */
CONVFWD_API conv_status conv_depthwise_fwd_variant(const float *X, const float *w, const float *bias, float *Y, int N,
                                       int C, int H, int W, int multiplier, int KH, int KW, int stride_h,
                                       int stride_w, int pad_h, int pad_w, int dil_h, int dil_w,
                                       conv_dw_mode mode, int variant, void *stream);

/*
 * conv_window -- the window of a convolution beyond the lecture's restricted
 * operator. "Convolution Is Wx+b Moving Across a Signal", section "Why 1D?
 * Why 2D?", defines stride, zero padding and dilation per axis (the output
 * size rule of conv_out_size_window); its section "Find the same sum in
 * CKE's C kernels" sums, for one output channel, over the taps of its group
 * of input channels only; its section "Where this shows up in models I work
 * with" names causal Conv1D, which is padding placed entirely before the
 * signal (pad_left = dil_w*(KW-1), pad_right = 0).
 *
 * Output row y reads input rows y*stride_h + i*dil_h - pad_top (i < KH) and
 * columns x*stride_w + j*dil_w - pad_left (j < KW); positions outside the
 * input read zero.
 */
typedef struct conv_window {
    int stride_h, stride_w;     /* >= 1 */
    int pad_top, pad_bottom;    /* zero rows before / after the input, >= 0 */
    int pad_left, pad_right;    /* zero columns before / after the input, >= 0 */
    int dil_h, dil_w;           /* >= 1 */
    int groups;                 /* dense: >= 1 and divides Cin and Cout; depthwise: must be 1 */
} conv_window;

/*
 * conv2d_nhwc_fwd_window -- dense forward cross-correlation with a window.
 *
 * Arguments as conv2d_nhwc_fwd, plus `win` (host pointer, not NULL). With
 * groups = g the filter is [KH,KW,Cin/g,Cout] (contiguous) and output
 * channel o belongs to group o / (Cout/g), reading input channels
 * [(o / (Cout/g)) * Cin/g, ... + Cin/g). Ho and Wo follow
 * conv_out_size_window. With stride 1, no padding, dilation 1 and one group
 * this is conv2d_nhwc_fwd.
 *
 * Errors: as conv2d_nhwc_fwd; CONV_ERR_NULL also for win NULL;
 * CONV_ERR_NONPOSITIVE for a stride, dilation or group count < 1 or a pad
 * < 0; CONV_ERR_SHAPE when Ho or Wo <= 0 or groups does not divide Cin and
 * Cout.
 */
CONVFWD_API conv_status conv2d_nhwc_fwd_window(const void *X, const int64_t *x_strides, const void *F,
                                   const float *bias, void *Y, const int64_t *y_strides, int N, int H, int W,
                                   int Cin, int KH, int KW, int Cout, const conv_window *win,
                                   conv_dtype x_dtype, conv_dtype y_dtype, int variant, void *stream);

/*
 * conv_depthwise_fwd_window -- depthwise forward convolution with a window
 * whose padding may differ before and after each axis (win->groups must be
 * 1: the depthwise grouping is implied). Same contract, modes, layouts and
 * errors as conv_depthwise_fwd, with xpad holding pad_top / pad_bottom rows
 * and pad_left / pad_right columns of zeros; Ho and Wo follow
 * conv_out_size_window. CONV_ERR_NULL also for win NULL; CONV_ERR_UNSUPPORTED
 * for groups != 1.
 */
CONVFWD_API conv_status conv_depthwise_fwd_window(const float *X, const float *w, const float *bias, float *Y, int N,
                                      int C, int H, int W, int multiplier, int KH, int KW,
                                      const conv_window *win, conv_dw_mode mode, int variant, void *stream);

/*
 * conv_im2col_nhwc -- the explicit patch matrix of the dense operator.
 *
 * "CMU DLSys Lecture 14", section 5: row m = (n*Ho + y)*Wo + x holds the
 * KH*KW*Cin input values output (n, y, x) reads, in (i, j, c) order, so that
 * cols @ F.reshape(KH*KW*Cin, Cout) is the convolution. Section 6 prices
 * this copy; section 7 asks that a timing of the matrix route include it.
 * The convolution entry points never build it; this call exists for that
 * comparison. With a window, tap (i, j) of output (y, x) reads input row
 * y*stride_h + i*dil_h - pad_top and column x*stride_w + j*dil_w - pad_left,
 * and taps in the padding are zeros.
 *
 *   X         device, logical NHWC [N,H,W,Cin], channel stride 1 (x_strides
 *             as for conv2d_nhwc_fwd, NULL = contiguous), dtype `dtype`.
 *   cols      device, contiguous [N*Ho*Wo, KH*KW*Cin], dtype `dtype`, caller
 *             owned (this is the storage the explicit route costs), fully
 *             overwritten.
 *   win       host pointer, not NULL; win->groups must be 1.
 *   dtype     CONV_F32 or CONV_BF16; values are copied bit for bit.
 *
 * Errors: CONV_ERR_NULL, CONV_ERR_NONPOSITIVE, CONV_ERR_SHAPE (Ho or Wo
 * <= 0), CONV_ERR_DTYPE, CONV_ERR_LAYOUT (channel stride != 1),
 * CONV_ERR_UNSUPPORTED (groups != 1), CONV_ERR_ALIAS (cols overlaps X),
 * CONV_ERR_HIP.
 */
CONVFWD_API conv_status conv_im2col_nhwc(const void *X, const int64_t *x_strides, void *cols, int N, int H, int W,
                             int Cin, int KH, int KW, const conv_window *win, conv_dtype dtype, void *stream);

/*
 * Which variant CONV_VARIANT_AUTO launches for exactly these arguments (a
 * CONV_VARIANT_* value), or -1 where the call itself would return an error.
 * Arguments are those of conv2d_nhwc_fwd_window / conv2d_nhwc_fwd and
 * conv_depthwise_fwd_window / conv_depthwise_fwd, without variant and
 * stream: the kernel choice looks at the pointers' alignment and the
 * strides, so these are the pointers and strides the call will pass. For
 * the dense queries Y may be NULL, meaning a fresh contiguous output on a
 * 256-byte boundary that the caller is about to allocate (y_strides is then
 * ignored). Host-only: no HIP call, nothing dereferenced.
 */
CONVFWD_API int conv2d_nhwc_window_auto_variant(const void *X, const int64_t *x_strides, const void *F,
                                                const float *bias, const void *Y, const int64_t *y_strides, int N,
                                                int H, int W, int Cin, int KH, int KW, int Cout,
                                                const conv_window *win, conv_dtype x_dtype, conv_dtype y_dtype);
CONVFWD_API int conv2d_nhwc_auto_variant(const void *X, const int64_t *x_strides, const void *F, const float *bias,
                                         const void *Y, const int64_t *y_strides, int N, int H, int W, int Cin,
                                         int KH, int KW, int Cout, conv_dtype x_dtype, conv_dtype y_dtype);
CONVFWD_API int conv_depthwise_window_auto_variant(const float *X, const float *w, const float *bias, const float *Y,
                                                   int N, int C, int H, int W, int multiplier, int KH, int KW,
                                                   const conv_window *win, conv_dw_mode mode);
CONVFWD_API int conv_depthwise_auto_variant(const float *X, const float *w, const float *bias, const float *Y, int N,
                                            int C, int H, int W, int multiplier, int KH, int KW, int stride_h,
                                            int stride_w, int pad_h, int pad_w, int dil_h, int dil_w,
                                            conv_dw_mode mode);

/* Output size along one axis: floor((in + 2*pad - (dil*(k-1)+1)) / stride) + 1
 * ("Convolution Is Wx+b Moving Across a Signal", section "Why 1D? Why 2D?").
 * Returns a value <= 0 when no window fits or an argument is out of range. */
CONVFWD_API int64_t conv_out_size(int64_t in, int k, int stride, int pad, int dil);

/* The same rule with padding that differs before and after the axis:
 * floor((in + pad_before + pad_after - (dil*(k-1)+1)) / stride) + 1. */
CONVFWD_API int64_t conv_out_size_window(int64_t in, int k, int stride, int pad_before, int pad_after, int dil);

/* Static, NUL-terminated description of a status code. */
CONVFWD_API const char *conv_status_str(conv_status s);

/* Copy `bytes` bytes from src to dst (device pointers, non-overlapping) with a
 * plain streaming kernel on `stream`. It is not part of the convolution; it
 * calibrates memory-traffic counters and the achievable HBM bandwidth.
 * Errors: CONV_ERR_NULL, CONV_ERR_NONPOSITIVE (bytes < 0), CONV_ERR_ALIAS,
 * CONV_ERR_HIP. bytes == 0 enqueues nothing. */
CONVFWD_API conv_status conv_copy_bytes(const void *src, void *dst, int64_t bytes, void *stream);

/* The same copy with as many bytes in flight as the chip takes: each thread
 * issues eight 16-byte loads before its first store, every workgroup is
 * resident at once, and stores write through (device scope, streaming hint).
 * It bounds from above what a kernel that must read and write these byte
 * counts once can reach. src, dst and bytes must be multiples of 16
 * (CONV_ERR_LAYOUT otherwise); bytes <= 2^40 (CONV_ERR_UNSUPPORTED);
 * CONV_ERR_NULL, CONV_ERR_NONPOSITIVE, CONV_ERR_ALIAS, CONV_ERR_HIP as
 * conv_copy_bytes. */
CONVFWD_API conv_status conv_copy_bytes_wide(const void *src, void *dst, int64_t bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* CONVFWD_H */
