// Explicit patch matrix (im2col): the packing step of the comparison route.
//
// "CMU DLSys Lecture 14: Convolutional Network Implementation", section 5:
// row m = (n*Ho + y)*Wo + x of the patch matrix holds the K*K*Cin input
// values that output (n, y, x) reads, flattened in (i, j, c) order, so that
// the convolution is that matrix times F.reshape(K*K*Cin, Cout). Section 6
// prices the copy (rho times the input); section 7 asks that a timing of the
// matrix route include it. The implicit-GEMM kernels never build this
// matrix; this kernel exists so the two routes can be compared.
//
// With a window ("Convolution Is Wx+b Moving Across a Signal", section "Why
// 1D? Why 2D?"), tap (i, j) of output (y, x) reads input row
// y*sh + i*dh - pt and column x*sw + j*dw - pl; taps in the padding are
// zeros in the matrix.
//
// One thread writes one 16-byte chunk of the matrix (8 bf16 or 4 fp32
// channels of one tap) when Cin fills whole chunks, else one element:
// consecutive threads write consecutive bytes, and each chunk is read from
// one contiguous run of a pixel's channels.
#include "common.h"
#include "internal.h"

namespace convfwd {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

struct Im2colArgs {
    const char *X;
    char *cols;
    int64_t xs0, xs1, xs2;        // element strides of X
    int H, W, Cin, KW, Ho, Wo;
    int sh, sw, pt, pl, dh, dw;
    int vec;                      // elements per work item (16-byte chunk or 1)
    int esz;                      // bytes per element
    int64_t items;                // work items in the whole matrix
    int64_t row_items;            // work items per matrix row (K*K*Cin / vec)
    int tap_items;                // work items per tap (Cin / vec)
};

template <int VEC16>
__global__ __launch_bounds__(256) void im2col_kernel(Im2colArgs a)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < a.items; t += stride) {
        const int64_t m = t / a.row_items;                  // matrix row: output (n, y, x)
        const int64_t kq = t - m * a.row_items;             // item within the row
        const int tap = (int)(kq / a.tap_items);            // i * KW + j
        const int cq = (int)(kq - (int64_t)tap * a.tap_items);
        const int i = tap / a.KW, j = tap - (tap / a.KW) * a.KW;
        const int x = (int)(m % a.Wo);
        const int64_t ny = m / a.Wo;
        const int y = (int)(ny % a.Ho);
        const int64_t n = ny / a.Ho;
        const int r = y * a.sh + i * a.dh - a.pt;
        const int col = x * a.sw + j * a.dw - a.pl;
        const bool in = r >= 0 && r < a.H && col >= 0 && col < a.W;
        const int64_t src = (n * a.xs0 + (int64_t)r * a.xs1 + (int64_t)col * a.xs2 + (int64_t)cq * a.vec) * a.esz;
        char *dst = a.cols + t * a.vec * a.esz;
        if constexpr (VEC16) {
            u32x4 v = {0, 0, 0, 0};
            if (in)
                v = *reinterpret_cast<const u32x4 *>(a.X + src);
            *reinterpret_cast<u32x4 *>(dst) = v;
        } else {
            if (a.esz == 2) {
                const uint16_t v = in ? *reinterpret_cast<const uint16_t *>(a.X + src) : (uint16_t)0;
                *reinterpret_cast<uint16_t *>(dst) = v;
            } else {
                const uint32_t v = in ? *reinterpret_cast<const uint32_t *>(a.X + src) : 0u;
                *reinterpret_cast<uint32_t *>(dst) = v;
            }
        }
    }
}

}  // namespace

hipError_t launch_im2col(const Im2colProblem &p, hipStream_t s)
{
    Im2colArgs a;
    a.X = static_cast<const char *>(p.X);
    a.cols = static_cast<char *>(p.cols);
    a.xs0 = p.xs[0];
    a.xs1 = p.xs[1];
    a.xs2 = p.xs[2];
    a.H = p.H;
    a.W = p.W;
    a.Cin = p.Cin;
    a.KW = p.KW;
    a.Ho = p.Ho;
    a.Wo = p.Wo;
    a.sh = p.sh;
    a.sw = p.sw;
    a.pt = p.pt;
    a.pl = p.pl;
    a.dh = p.dh;
    a.dw = p.dw;
    a.esz = p.dtype == CONV_BF16 ? 2 : 4;
    const int per16 = 16 / a.esz;
    // 16-byte chunks need whole chunks per tap and 16-byte aligned pixels.
    const bool vec16 = p.Cin % per16 == 0 && (uintptr_t)p.X % 16 == 0 && (uintptr_t)p.cols % 16 == 0 &&
                       p.xs[0] % per16 == 0 && p.xs[1] % per16 == 0 && p.xs[2] % per16 == 0;
    a.vec = vec16 ? per16 : 1;
    a.tap_items = p.Cin / a.vec;
    a.row_items = (int64_t)p.KH * p.KW * a.tap_items;
    a.items = (int64_t)p.N * p.Ho * p.Wo * a.row_items;
    const int block = 256;
    const unsigned grid = grid_for(a.items, block, (int64_t)256 * 256);
    if (vec16)
        hipLaunchKernelGGL(im2col_kernel<1>, dim3(grid), dim3(block), 0, s, a);
    else
        hipLaunchKernelGGL(im2col_kernel<0>, dim3(grid), dim3(block), 0, s, a);
    return hipGetLastError();
}

}  // namespace convfwd
