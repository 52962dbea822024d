/*
 * CPU oracle for the forward 2D convolution operator.
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the CPU-baseline
 * leg of the benchmark may load this library. The HIP product library never
 * links, loads or calls it, and this file shares no code, header, table or
 * helper with it.
 *
 * Everything here is the plain definition written out as nested loops, in the
 * order the pages state it. No blocking, no fusion, no reordering.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -fopenmp -fPIC -shared.
 * -ffp-contract=off keeps every fp32 multiply and add separately rounded (on
 * x86-64 FLT_EVAL_METHOD is 0, so each float operation rounds to fp32), and
 * each parallel region clears the SSE flush-to-zero and denormals-are-zero
 * bits, so subnormal values behave as IEEE 754 says.
 *
 * Parity status of every entry point is given in the module docstring of
 * oracle/__init__.py (all are pinned there by tests/test_oracle_pins.py).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <xmmintrin.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_BAD_ARG 1

/* IEEE behaviour for subnormals in the calling thread: clear FTZ (bit 15) and
 * DAZ (bit 6) of MXCSR. Returns the previous value so it can be restored. */
static unsigned int oracle_ieee_mode(void)
{
    unsigned int old = _mm_getcsr();
    _mm_setcsr(old & ~((1u << 15) | (1u << 6)));
    return old;
}

/* One axis of the output-size rule from "Convolution Is Wx+b Moving Across a
 * Signal", section "Why 1D? Why 2D?": the effective kernel spans
 * dil*(k-1)+1 input positions, and the output holds
 * floor((in + 2*pad - effective) / stride) + 1 positions. Returns <= 0 when
 * no window fits. */
long long oracle_out_size(long long in, long long k, long long stride, long long pad, long long dil)
{
    long long eff, span;
    if (in <= 0 || k <= 0 || stride <= 0 || pad < 0 || dil <= 0)
        return 0;
    eff = dil * (k - 1) + 1;
    span = in + 2 * pad - eff;
    if (span < 0)
        return 0;
    return span / stride + 1;
}

/* ---------------------------------------------------------------------------
 * Dense NHWC cross-correlation, accumulated in fp64.
 *
 * "CMU DLSys Lecture 14: Convolutional Network Implementation", section 1
 * (the index contract): Y[n,y,x,o] = sum over i<K, j<K, c<Cin of
 * X[n,y+i,x+j,c] * F[i,j,c,o], with no flip of the filter, Ho = H-K+1 and
 * Wo = W-K+1. The seven loops below are that sum, in the (n,y,x,o,i,j,c)
 * order the lecture uses for its loop oracle.
 *
 * The same loops also take the general form used as a superset for cross
 * checks: stride (sh,sw), symmetric zero padding (ph,pw), dilation (dh,dw),
 * groups, and an optional bias. A tap whose input position falls in the
 * padding reads zero. With groups = g, output channel o belongs to group
 * o / (Cout/g) and reads input channels of that group only, and F has shape
 * [KH,KW,Cin/g,Cout]. With stride 1, no padding, dilation 1, one group and no
 * bias this is exactly the lecture's operator.
 *
 * X is addressed through element strides xs[4] (NHWC order), so any strided
 * view of a float32 array can be passed; F is contiguous KKIO; Y is a
 * contiguous [N,Ho,Wo,Cout] fp64 array. Input values are fp32 (bf16 values
 * are exact in fp32); every product and sum is done in fp64.
 * ------------------------------------------------------------------------- */
static double dense_one_output(const float *X, const int64_t *xs, const float *F, const float *bias,
                               int H, int W, int Cin, int KH, int KW, int Cout,
                               int sh, int sw, int ph, int pw, int dh, int dw, int groups,
                               long long n, long long y, long long x, int o)
{
    int cg = Cin / groups;
    int g = o / (Cout / groups);
    double acc = 0.0;
    int i, j, c;
    for (i = 0; i < KH; ++i) {
        long long r = y * sh + (long long)i * dh - ph;
        for (j = 0; j < KW; ++j) {
            long long col = x * sw + (long long)j * dw - pw;
            for (c = 0; c < cg; ++c) {
                double xv = 0.0;
                if (r >= 0 && r < H && col >= 0 && col < W)
                    xv = (double)X[n * xs[0] + r * xs[1] + col * xs[2] + (long long)(g * cg + c) * xs[3]];
                acc += xv * (double)F[(((long long)i * KW + j) * cg + c) * Cout + o];
            }
        }
    }
    if (bias)
        acc += (double)bias[o];
    return acc;
}

static int dense_args_ok(const float *X, const int64_t *xs, const float *F, int N, int H, int W, int Cin,
                         int KH, int KW, int Cout, int sh, int sw, int ph, int pw, int dh, int dw,
                         int groups)
{
    if (!X || !xs || !F)
        return 0;
    if (N <= 0 || H <= 0 || W <= 0 || Cin <= 0 || KH <= 0 || KW <= 0 || Cout <= 0)
        return 0;
    if (sh <= 0 || sw <= 0 || dh <= 0 || dw <= 0 || ph < 0 || pw < 0 || groups <= 0)
        return 0;
    if (Cin % groups != 0 || Cout % groups != 0)
        return 0;
    if (oracle_out_size(H, KH, sh, ph, dh) <= 0 || oracle_out_size(W, KW, sw, pw, dw) <= 0)
        return 0;
    return 1;
}

int oracle_conv2d_nhwc_f64(const float *X, const int64_t *xs, const float *F, const float *bias,
                           double *Y, int N, int H, int W, int Cin, int KH, int KW, int Cout,
                           int sh, int sw, int ph, int pw, int dh, int dw, int groups, int nthreads)
{
    long long Ho, Wo, n, y;
    if (!Y || !dense_args_ok(X, xs, F, N, H, W, Cin, KH, KW, Cout, sh, sw, ph, pw, dh, dw, groups))
        return ORACLE_BAD_ARG;
    Ho = oracle_out_size(H, KH, sh, ph, dh);
    Wo = oracle_out_size(W, KW, sw, pw, dw);
    if (nthreads <= 0)
        nthreads = 1;
#pragma omp parallel num_threads(nthreads)
    {
        unsigned int saved = oracle_ieee_mode();
#pragma omp for collapse(2) schedule(static)
        for (n = 0; n < N; ++n) {
            for (y = 0; y < Ho; ++y) {
                long long x;
                int o;
                for (x = 0; x < Wo; ++x) {
                    for (o = 0; o < Cout; ++o) {
                        Y[((n * Ho + y) * Wo + x) * Cout + o] =
                            dense_one_output(X, xs, F, bias, H, W, Cin, KH, KW, Cout, sh, sw, ph, pw,
                                             dh, dw, groups, n, y, x, o);
                    }
                }
            }
        }
        _mm_setcsr(saved);
    }
    return ORACLE_OK;
}

/* The same sum evaluated only at selected outputs: idx[k] is a flat index
 * into the contiguous [N,Ho,Wo,Cout] output, and out[k] receives Y at that
 * index. Used to check full-size launches on sampled outputs. */
int oracle_conv2d_nhwc_f64_at(const float *X, const int64_t *xs, const float *F, const float *bias,
                              const int64_t *idx, long long count, double *out,
                              int N, int H, int W, int Cin, int KH, int KW, int Cout,
                              int sh, int sw, int ph, int pw, int dh, int dw, int groups, int nthreads)
{
    long long Ho, Wo, total, k;
    int bad = 0;
    if (!idx || !out || count < 0 ||
        !dense_args_ok(X, xs, F, N, H, W, Cin, KH, KW, Cout, sh, sw, ph, pw, dh, dw, groups))
        return ORACLE_BAD_ARG;
    Ho = oracle_out_size(H, KH, sh, ph, dh);
    Wo = oracle_out_size(W, KW, sw, pw, dw);
    total = (long long)N * Ho * Wo * Cout;
    for (k = 0; k < count; ++k)
        if (idx[k] < 0 || idx[k] >= total)
            bad = 1;
    if (bad)
        return ORACLE_BAD_ARG;
    if (nthreads <= 0)
        nthreads = 1;
#pragma omp parallel num_threads(nthreads)
    {
        unsigned int saved = oracle_ieee_mode();
#pragma omp for schedule(static)
        for (k = 0; k < count; ++k) {
            long long f = idx[k];
            int o = (int)(f % Cout);
            long long x = (f / Cout) % Wo;
            long long y = (f / Cout / Wo) % Ho;
            long long n = f / Cout / Wo / Ho;
            out[k] = dense_one_output(X, xs, F, bias, H, W, Cin, KH, KW, Cout, sh, sw, ph, pw, dh, dw,
                                      groups, n, y, x, o);
        }
        _mm_setcsr(saved);
    }
    return ORACLE_OK;
}

/* ---------------------------------------------------------------------------
 * Explicit patch matrix (im2col), NHWC, stride 1, no padding.
 *
 * "CMU DLSys Lecture 14", section 5 (the patch matrix): the six-axis patch
 * view has shape (N,Ho,Wo,K,K,Cin); flattening its last three axes in (i,j,c)
 * order gives a (N*Ho*Wo) x (K*K*Cin) matrix whose product with the filter
 * reshaped to (K*K*Cin) x Cout is the output. Row m = (n*Ho + y)*Wo + x,
 * column (i*KW + j)*Cin + c holds X[n, y+i, x+j, c]. This is the packing
 * copy the lecture warns about; the oracle builds it only as a second route
 * to the same index map.
 * ------------------------------------------------------------------------- */
int oracle_im2col_nhwc(const float *X, const int64_t *xs, float *cols, int N, int H, int W, int C,
                       int KH, int KW)
{
    long long Ho, Wo, n, y, x;
    int i, j, c;
    if (!X || !xs || !cols || N <= 0 || H <= 0 || W <= 0 || C <= 0 || KH <= 0 || KW <= 0 ||
        KH > H || KW > W)
        return ORACLE_BAD_ARG;
    Ho = H - KH + 1;
    Wo = W - KW + 1;
    for (n = 0; n < N; ++n)
        for (y = 0; y < Ho; ++y)
            for (x = 0; x < Wo; ++x) {
                long long m = (n * Ho + y) * Wo + x;
                for (i = 0; i < KH; ++i)
                    for (j = 0; j < KW; ++j)
                        for (c = 0; c < C; ++c)
                            cols[m * ((long long)KH * KW * C) + ((long long)i * KW + j) * C + c] =
                                X[n * xs[0] + (y + i) * xs[1] + (x + j) * xs[2] + (long long)c * xs[3]];
            }
    return ORACLE_OK;
}

/* ---------------------------------------------------------------------------
 * Depthwise convolution, NCHW planes, fp32.
 *
 * "Depthwise convolution" (onemodel docs), section "What each output is":
 * groups == C, Cout = C * mult, output channel oc reads input channel
 * oc / mult. For each output (n, oc, oy, ox) the accumulator starts at +0 and
 * the taps are visited row-major (ky outer, kx inner); each tap multiplies
 * the weight w[oc,ky,kx] by the zero-padded input at row oy*sh + ky*dh and
 * column ox*sw + kx*dw of the padded plane. Padding is a real zero, so a
 * padding tap is an actual multiplication by +0 (an infinite or NaN weight
 * there gives NaN).
 *
 * mode 0 (exact): the product is rounded to fp32, then the sum is rounded to
 *   fp32 (no fused operation); a NaN final value becomes the canonical NaN
 *   0x7FC00000.
 * mode 1 (fast): one fused multiply-add per tap, acc = fma(w, x, acc), one
 *   rounding; NaN values are left as produced.
 * bias (optional): a separate pass, one rounded fp32 addition per output,
 *   before the NaN rewrite of exact mode.
 *
 * X is contiguous [N,C,H,W], w contiguous [C*mult,KH,KW], Y contiguous
 * [N,C*mult,Ho,Wo] with Ho, Wo from oracle_out_size.
 * ------------------------------------------------------------------------- */
static float dw_one_output(const float *X, const float *w, const float *bias, int C, int H, int W,
                           int mult, int KH, int KW, int sh, int sw, int ph, int pw, int dh, int dw,
                           int mode, long long n, int oc, long long oy, long long ox)
{
    int ic = oc / mult;
    const float *plane = X + (n * C + ic) * (long long)H * W;
    float acc = +0.0f;
    int ky, kx;
    for (ky = 0; ky < KH; ++ky) {
        for (kx = 0; kx < KW; ++kx) {
            long long r = oy * sh + (long long)ky * dh - ph;
            long long c = ox * sw + (long long)kx * dw - pw;
            float xv = +0.0f;
            float wv = w[((long long)oc * KH + ky) * KW + kx];
            if (r >= 0 && r < H && c >= 0 && c < W)
                xv = plane[r * W + c];
            if (mode == 0) {
                float p = wv * xv;
                acc = acc + p;
            } else {
                acc = fmaf(wv, xv, acc);
            }
        }
    }
    if (bias)
        acc = acc + bias[oc];
    if (mode == 0 && acc != acc) {
        uint32_t canon = 0x7FC00000u;
        memcpy(&acc, &canon, sizeof acc);
    }
    return acc;
}

int oracle_depthwise_nchw_f32(const float *X, const float *w, const float *bias, float *Y, int N, int C,
                              int H, int W, int mult, int KH, int KW, int sh, int sw, int ph, int pw,
                              int dh, int dw, int mode, int nthreads)
{
    long long Ho, Wo, q;
    int Cout;
    if (!X || !w || !Y || N <= 0 || C <= 0 || H <= 0 || W <= 0 || mult <= 0 || KH <= 0 || KW <= 0 ||
        sh <= 0 || sw <= 0 || dh <= 0 || dw <= 0 || ph < 0 || pw < 0 || (mode != 0 && mode != 1))
        return ORACLE_BAD_ARG;
    Ho = oracle_out_size(H, KH, sh, ph, dh);
    Wo = oracle_out_size(W, KW, sw, pw, dw);
    if (Ho <= 0 || Wo <= 0)
        return ORACLE_BAD_ARG;
    Cout = C * mult;
    if (nthreads <= 0)
        nthreads = 1;
#pragma omp parallel num_threads(nthreads)
    {
        unsigned int saved = oracle_ieee_mode();
#pragma omp for schedule(static)
        for (q = 0; q < (long long)N * Cout; ++q) {
            long long n = q / Cout;
            int oc = (int)(q % Cout);
            long long oy, ox;
            for (oy = 0; oy < Ho; ++oy)
                for (ox = 0; ox < Wo; ++ox)
                    Y[(q * Ho + oy) * Wo + ox] = dw_one_output(X, w, bias, C, H, W, mult, KH, KW, sh, sw,
                                                               ph, pw, dh, dw, mode, n, oc, oy, ox);
        }
        _mm_setcsr(saved);
    }
    return ORACLE_OK;
}
