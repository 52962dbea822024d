// Depthwise convolution, one thread per output, reading the input straight
// from global memory. It takes every legal shape and serves as the reference
// variant on the GPU: the tiled kernels must reproduce its bits exactly.
//
// "Depthwise convolution" (onemodel docs), section "What each output is":
// acc starts at +0; taps in row-major order; a tap outside the input reads a
// real +0 (so inf/NaN weights still meet it as NaN); exact mode rounds the
// product then the sum; fast mode fuses them; the bias is a separate rounded
// addition; exact mode rewrites a NaN result to 0x7FC00000.
//
// This file is compiled with -ffp-contract=off, and exact-mode arithmetic
// sits under "#pragma clang fp contract(off)" as well, so a product and the
// following sum are never fused; fast mode calls __builtin_fmaf explicitly.
#include "common.h"
#include "internal.h"

namespace convfwd {
namespace {

struct DwArgs {
    const float *X;
    const float *w;
    const float *bias;
    float *Y;
    int C, H, W, mult, KH, KW, sh, sw, ph, pw, dh, dw, Ho, Wo;
    int64_t total;
};

template <int EXACT>
__global__ __launch_bounds__(256) void dw_direct_kernel(DwArgs a)
{
#pragma clang fp contract(off)
    const int Cout = a.C * a.mult;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < a.total; t += stride) {
        const int ox = (int)(t % a.Wo);
        int64_t r = t / a.Wo;
        const int oy = (int)(r % a.Ho);
        const int64_t q = r / a.Ho;          // output plane (n, oc)
        const int oc = (int)(q % Cout);
        const int64_t n = q / Cout;
        const float *plane = a.X + (n * a.C + oc / a.mult) * (int64_t)a.H * a.W;
        const float *wk = a.w + (int64_t)oc * a.KH * a.KW;
        float acc = +0.0f;
        for (int ky = 0; ky < a.KH; ++ky) {
            const int row = oy * a.sh + ky * a.dh - a.ph;
            const bool row_in = row >= 0 && row < a.H;
            for (int kx = 0; kx < a.KW; ++kx) {
                const int col = ox * a.sw + kx * a.dw - a.pw;
                const float xv = (row_in && col >= 0 && col < a.W) ? plane[(int64_t)row * a.W + col] : +0.0f;
                const float wv = wk[ky * a.KW + kx];
                if (EXACT) {
                    const float prod = wv * xv;
                    acc = acc + prod;
                } else {
                    acc = __builtin_fmaf(wv, xv, acc);
                }
            }
        }
        if (a.bias)
            acc = acc + a.bias[oc];
        if (EXACT && __builtin_isnan(acc))
            acc = __uint_as_float(0x7FC00000u);
        a.Y[t] = acc;
    }
}

}  // namespace

hipError_t launch_dw_direct(const DwProblem &p, hipStream_t s)
{
    DwArgs a;
    a.X = p.X;
    a.w = p.w;
    a.bias = p.bias;
    a.Y = p.Y;
    a.C = p.C;
    a.H = p.H;
    a.W = p.W;
    a.mult = p.mult;
    a.KH = p.KH;
    a.KW = p.KW;
    a.sh = p.sh;
    a.sw = p.sw;
    a.ph = p.ph;
    a.pw = p.pw;
    a.dh = p.dh;
    a.dw = p.dw;
    a.Ho = p.Ho;
    a.Wo = p.Wo;
    a.total = (int64_t)p.N * p.C * p.mult * p.Ho * p.Wo;
    const int block = 256;
    const unsigned grid = grid_for(a.total, block);
    if (p.mode == CONV_DW_EXACT)
        hipLaunchKernelGGL(dw_direct_kernel<1>, dim3(grid), dim3(block), 0, s, a);
    else
        hipLaunchKernelGGL(dw_direct_kernel<0>, dim3(grid), dim3(block), 0, s, a);
    return hipGetLastError();
}

}  // namespace convfwd
