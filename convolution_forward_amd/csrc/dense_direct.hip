// Dense NHWC cross-correlation, one thread per output element.
//
// "CMU DLSys Lecture 14: Convolutional Network Implementation", section 1:
// Y[n,y,x,o] = sum over (i,j,c) of X[n,y+i,x+j,c] * F[i,j,c,o], no flip.
// The same loops take the window of "Convolution Is Wx+b Moving Across a
// Signal" (section "Why 1D? Why 2D?"): output (y, x) reads input row
// y*sh + i*dh - pt and column x*sw + j*dw - pl, zero outside the input; and
// groups (section "Find the same sum in CKE's C kernels"): output channel o
// sums over the Cin/groups input channels of its group only, with F of shape
// [KH,KW,Cin/groups,Cout].
// This is the variant that takes every legal shape and stride: threads are
// laid out with o fastest, so F and Y accesses are coalesced along Cout and X
// is read as a broadcast. fp32 accumulation in (i,j,c) order; a padding
// position contributes 0 * F like any other tap.
#include "common.h"
#include "internal.h"

namespace convfwd {
namespace {

struct DirectArgs {
    const void *X;
    const void *F;
    const float *bias;
    void *Y;
    int64_t xs0, xs1, xs2, ys0, ys1, ys2;
    int H, W, Cin, KH, KW, Cout, Ho, Wo;
    int sh, sw, pt, pl, dh, dw, groups;
    int64_t total;
};

template <typename TX, typename TY>
__global__ __launch_bounds__(256) void dense_direct_kernel(DirectArgs a)
{
    const TX *X = static_cast<const TX *>(a.X);
    const TX *F = static_cast<const TX *>(a.F);
    TY *Y = static_cast<TY *>(a.Y);
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < a.total; t += stride) {
        const int o = (int)(t % a.Cout);
        int64_t r = t / a.Cout;
        const int x = (int)(r % a.Wo);
        r /= a.Wo;
        const int y = (int)(r % a.Ho);
        const int64_t n = r / a.Ho;
        const int cg = a.Cin / a.groups;                 // input channels per group
        const int c0 = o / (a.Cout / a.groups) * cg;     // first input channel of o's group
        float acc = 0.0f;
        for (int i = 0; i < a.KH; ++i) {
            const int r = y * a.sh + i * a.dh - a.pt;
            for (int j = 0; j < a.KW; ++j) {
                const int col = x * a.sw + j * a.dw - a.pl;
                const bool in = r >= 0 && r < a.H && col >= 0 && col < a.W;
                const TX *xp = X + n * a.xs0 + (int64_t)(in ? r : 0) * a.xs1 + (int64_t)(in ? col : 0) * a.xs2 + c0;
                const TX *fp = F + ((int64_t)(i * a.KW + j) * cg) * a.Cout + o;
                for (int c = 0; c < cg; ++c) {
                    const float xv = in ? load_as_f32(xp + c) : 0.0f;
                    acc = __builtin_fmaf(xv, load_as_f32(fp + (int64_t)c * a.Cout), acc);
                }
            }
        }
        if (a.bias)
            acc += a.bias[o];
        store_from_f32(Y + n * a.ys0 + (int64_t)y * a.ys1 + (int64_t)x * a.ys2 + o, acc);
    }
}

}  // namespace

hipError_t launch_dense_direct(const DenseProblem &p, hipStream_t s)
{
    DirectArgs a;
    a.X = p.X;
    a.F = p.F;
    a.bias = p.bias;
    a.Y = p.Y;
    a.xs0 = p.xs[0];
    a.xs1 = p.xs[1];
    a.xs2 = p.xs[2];
    a.ys0 = p.ys[0];
    a.ys1 = p.ys[1];
    a.ys2 = p.ys[2];
    a.H = p.H;
    a.W = p.W;
    a.sh = p.sh;
    a.sw = p.sw;
    a.pt = p.pt;
    a.pl = p.pl;
    a.dh = p.dh;
    a.dw = p.dw;
    a.groups = p.groups;
    a.Cin = p.Cin;
    a.KH = p.KH;
    a.KW = p.KW;
    a.Cout = p.Cout;
    a.Ho = p.Ho;
    a.Wo = p.Wo;
    a.total = (int64_t)p.N * p.Ho * p.Wo * p.Cout;
    const int block = 256;
    const unsigned grid = grid_for(a.total, block);
    if (p.xdt == CONV_F32)
        hipLaunchKernelGGL((dense_direct_kernel<float, float>), dim3(grid), dim3(block), 0, s, a);
    else if (p.ydt == CONV_F32)
        hipLaunchKernelGGL((dense_direct_kernel<uint16_t, float>), dim3(grid), dim3(block), 0, s, a);
    else
        hipLaunchKernelGGL((dense_direct_kernel<uint16_t, uint16_t>), dim3(grid), dim3(block), 0, s, a);
    return hipGetLastError();
}

}  // namespace convfwd
