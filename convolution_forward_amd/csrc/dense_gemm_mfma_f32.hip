// Dense NHWC cross-correlation with fp32 operands, any window, as an implicit
// GEMM on CDNA4 matrix cores (v_mfma_f32_16x16x4_f32).
//
// Contract: "CMU DLSys Lecture 14: Convolutional Network Implementation",
// sections 1 and 5 (Y = patch matrix times F.reshape(K*K*Cin, Cout), the
// patch matrix never built), with the window of "Convolution Is Wx+b Moving
// Across a Signal" (section "Why 1D? Why 2D?": output (y, x) reads input
// row y*sh + i*dh - pt and column x*sw + j*dw - pl, zero outside) and its
// groups (section "Find the same sum in CKE's C kernels").
//
// This kernel takes every fp32 problem the row kernel (dense_mfma_f32.hip)
// declines: padding, strides, dilation, groups, any filter size, and channel
// counts that are not a multiple of 4 (the small first layer with three
// input channels).
//
// Work decomposition (one workgroup = 4 waves = 256 threads):
//  * A tile is 64 output pixels (flat index m = (n*Ho + y)*Wo + x) by 64
//    output channels. Wave w owns the 16-channel column block w and all four
//    16-pixel blocks of the tile: four accumulators.
//  * The K axis is the lecture's (i, j, c) order, flattened:
//    k = (i*KW + j)*span + c', where the channel span covers the groups of
//    the tile's output channels (one group when that group's channels fill
//    the tile) and c = first channel of the span + c'. A filter value whose
//    input channel lies outside its output channel's group is a zero of the
//    tile (block-diagonal), so small groups share a tile.
//  * A chunk is 32 values of k. Its patch values (64 pixels) and filter
//    values (64 channels) are loaded into registers, zeros for padding taps,
//    k past the end and other groups, written to LDS (double buffered: the
//    next chunk's loads are in flight while the current chunk feeds the
//    MFMAs) and read back as fragments, one fp32 value per lane and operand.
//  * The filter fragment is the MFMA's A operand (rows are output channels)
//    and the patch fragment its B operand (columns are pixels): a lane's four
//    results are four consecutive channels of one pixel, one 16-byte store
//    when Y's layout allows it.
//
// LDS rows of a chunk hold 64 values at a pitch of 80 floats: the four
// 16-lane groups of a fragment read sit 16 banks apart.
#include "common.h"
#include "internal.h"

namespace convfwd {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int GT = 256;                 // threads per workgroup
constexpr int TM = 64;                  // output pixels per tile
constexpr int TN = 64;                  // output channels per tile
constexpr int KC = 32;                  // k values per chunk
constexpr int PITCH = 80;               // LDS row pitch (floats)
constexpr int BUF = KC * PITCH;         // floats per operand buffer

// Division by a runtime constant d < 2^31 for dividends n < 2^31
// (Granlund and Montgomery, "Division by invariant integers using
// multiplication", 1994): with l = ceil(log2 d) and
// m = floor(2^32 * (2^l - d) / d) + 1, n / d = (umulhi(n, m) + n) >> l.
struct Div {
    uint32_t m, l;
};

__host__ __device__ inline Div make_div(uint32_t d)
{
    uint32_t l = 0;
    while (l < 31 && (1u << l) < d)
        ++l;
    const uint64_t m = ((uint64_t(1) << 32) * ((uint64_t(1) << l) - d)) / d + 1;
    return Div{(uint32_t)m, l};
}

__device__ __forceinline__ uint32_t div_by(uint32_t n, Div d) { return (__umulhi(n, d.m) + n) >> d.l; }

struct GemmArgsF {
    const float *X;
    const float *F;
    const float *bias;
    float *Y;
    int64_t xs0, xs1, xs2, ys0, ys1, ys2;
    int H, W, Cin, Cout, Ho, Wo, KH, KW;
    int sh, sw, pt, pl, dh, dw;
    int cin_g, cout_g;      // channels per group
    int M;                  // N * Ho * Wo
    int ntiles;             // channel tiles
    int vec_store;          // Y takes 16-byte stores of 4 channels
    Div div_kw, div_wo, div_ho, div_coutg;
};

__global__ __launch_bounds__(GT) void dense_gemm_mfma_f32(GemmArgsF a)
{
    __shared__ __align__(16) float lds[4 * BUF];    // [buffer][A: filter | B: patches]
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int tile = with_args_loaded((int)blockIdx.x, a);
    const int mt = tile / a.ntiles;
    const int o0 = (tile - mt * a.ntiles) * TN;
    const int m0 = mt * TM;

    // The channel span of the tile's groups.
    const int glo = (int)div_by((uint32_t)o0, a.div_coutg);
    const int ghi = (int)div_by((uint32_t)min(o0 + TN - 1, a.Cout - 1), a.div_coutg);
    const int span = (ghi - glo + 1) * a.cin_g;
    const int c_lo = glo * a.cin_g;
    const int K = a.KH * a.KW * span;
    const Div div_span = make_div((uint32_t)span);
    const int nch = (K + KC - 1) / KC;

    // Patch loads: this thread's pixels p = lane/8 + 16*wave + 8*pq and k
    // values kl = lane%8 + 8*kq of each chunk.
    int64_t xbase[2];
    int iy0[2], ix0[2];
    bool pok[2];
#pragma unroll
    for (int pq = 0; pq < 2; ++pq) {
        const int m = m0 + (lane >> 3) + 16 * wave + 8 * pq;
        pok[pq] = m < a.M;
        const int mm = pok[pq] ? m : 0;
        const int row = (int)div_by((uint32_t)mm, a.div_wo);    // n*Ho + y
        const int x = mm - row * a.Wo;
        const int n = (int)div_by((uint32_t)row, a.div_ho);
        const int y = row - n * a.Ho;
        xbase[pq] = (int64_t)n * a.xs0;
        iy0[pq] = y * a.sh - a.pt;
        ix0[pq] = x * a.sw - a.pl;
    }
    // Filter loads: this thread's channel o = o0 + lane and k values
    // kl = wave + 4*e of each chunk.
    const int o = o0 + lane;
    const bool ook = o < a.Cout;
    const int cgo = ook ? (int)div_by((uint32_t)o, a.div_coutg) * a.cin_g - c_lo : 0;   // o's group start in the span

    float ra[8], rb[8];
    auto load_chunk = [&](int ch) __attribute__((always_inline)) {
#pragma unroll
        for (int kq = 0; kq < 4; ++kq) {
            const int k = ch * KC + (lane & 7) + 8 * kq;
            const int tap = (int)div_by((uint32_t)k, div_span);
            const int c = c_lo + (k - tap * span);
            const int i = (int)div_by((uint32_t)tap, a.div_kw);
            const int j = tap - i * a.KW;
#pragma unroll
            for (int pq = 0; pq < 2; ++pq) {
                const int iy = iy0[pq] + i * a.dh;
                const int ix = ix0[pq] + j * a.dw;
                const bool ok = pok[pq] && k < K && (unsigned)iy < (unsigned)a.H && (unsigned)ix < (unsigned)a.W;
                float v = 0.f;
                if (ok)
                    v = a.X[xbase[pq] + (int64_t)iy * a.xs1 + (int64_t)ix * a.xs2 + c];
                rb[kq * 2 + pq] = v;
            }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int k = ch * KC + wave + 4 * e;
            const int tap = (int)div_by((uint32_t)k, div_span);
            const int cl = k - tap * span - cgo;      // input channel within o's group
            const bool ok = ook && k < K && (unsigned)cl < (unsigned)a.cin_g;
            float v = 0.f;
            if (ok)
                v = a.F[((int64_t)tap * a.cin_g + cl) * a.Cout + o];
            ra[e] = v;
        }
    };
    auto put_chunk = [&](int buf) __attribute__((always_inline)) {
        float *fa = lds + buf * 2 * BUF;
        float *pb = fa + BUF;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            fa[(wave + 4 * e) * PITCH + lane] = ra[e];
#pragma unroll
        for (int kq = 0; kq < 4; ++kq)
#pragma unroll
            for (int pq = 0; pq < 2; ++pq)
                pb[((lane & 7) + 8 * kq) * PITCH + (lane >> 3) + 16 * wave + 8 * pq] = rb[kq * 2 + pq];
    };

    f32x4 acc[4];
#pragma unroll
    for (int b = 0; b < 4; ++b)
        acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int g = lane >> 4;
    const int r = lane & 15;

    load_chunk(0);
    put_chunk(0);
    if (nch > 1)
        load_chunk(1);
    __syncthreads();
    for (int ch = 0; ch < nch; ++ch) {
        const float *fa = lds + (ch & 1) * 2 * BUF;
        const float *pb = fa + BUF;
#pragma unroll
        for (int s = 0; s < KC / 4; ++s) {
            const int kk = 4 * s + g;
            const float av = fa[kk * PITCH + wave * 16 + r];
#pragma unroll
            for (int b = 0; b < 4; ++b)
                acc[b] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, pb[kk * PITCH + b * 16 + r], acc[b], 0, 0, 0);
        }
        if (ch + 1 < nch)
            put_chunk((ch + 1) & 1);
        __syncthreads();
        if (ch + 2 < nch)
            load_chunk(ch + 2);
    }

    // Lane (g, r) of block b holds channels oc..oc+3 of pixel m0 + 16b + r.
    const int oc = o0 + wave * 16 + 4 * g;
    float bq[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
        bq[q] = (a.bias && oc + q < a.Cout) ? a.bias[oc + q] : 0.f;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const int m = m0 + 16 * b + r;
        if (m >= a.M || oc >= a.Cout)
            continue;
        const int row = (int)div_by((uint32_t)m, a.div_wo);
        const int x = m - row * a.Wo;
        const int n = (int)div_by((uint32_t)row, a.div_ho);
        const int y = row - n * a.Ho;
        float *yp = a.Y + (int64_t)n * a.ys0 + (int64_t)y * a.ys1 + (int64_t)x * a.ys2 + oc;
        const f32x4 v = {acc[b][0] + bq[0], acc[b][1] + bq[1], acc[b][2] + bq[2], acc[b][3] + bq[3]};
        if (a.vec_store) {
            *reinterpret_cast<f32x4 *>(yp) = v;
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (oc + q < a.Cout)
                    yp[q] = v[q];
        }
    }
}

// Whether the 32-bit index arithmetic above holds for the problem.
bool fits(const DenseProblem &p)
{
    if (p.xdt != CONV_F32 || p.ydt != CONV_F32)
        return false;
    const int64_t M = (int64_t)p.N * p.Ho * p.Wo;
    const int64_t tiles = (M + TM - 1) / TM * ((p.Cout + TN - 1) / TN);
    const int64_t K = (int64_t)p.KH * p.KW * p.Cin + TM;
    return M + TM < (int64_t(1) << 31) && tiles < (int64_t(1) << 31) && K < (int64_t(1) << 31) &&
           (int64_t)p.Cout + TN < (int64_t(1) << 31);
}

}  // namespace

bool dense_gemm_f32_supports(const DenseProblem &p) { return fits(p); }

hipError_t launch_dense_gemm_f32(const DenseProblem &p, hipStream_t s)
{
    if (!fits(p))
        return hipErrorNotSupported;
    GemmArgsF a;
    a.X = static_cast<const float *>(p.X);
    a.F = static_cast<const float *>(p.F);
    a.bias = p.bias;
    a.Y = static_cast<float *>(p.Y);
    a.xs0 = p.xs[0];
    a.xs1 = p.xs[1];
    a.xs2 = p.xs[2];
    a.ys0 = p.ys[0];
    a.ys1 = p.ys[1];
    a.ys2 = p.ys[2];
    a.H = p.H;
    a.W = p.W;
    a.Cin = p.Cin;
    a.Cout = p.Cout;
    a.Ho = p.Ho;
    a.Wo = p.Wo;
    a.KH = p.KH;
    a.KW = p.KW;
    a.sh = p.sh;
    a.sw = p.sw;
    a.pt = p.pt;
    a.pl = p.pl;
    a.dh = p.dh;
    a.dw = p.dw;
    a.cin_g = p.Cin / p.groups;
    a.cout_g = p.Cout / p.groups;
    a.M = (int)((int64_t)p.N * p.Ho * p.Wo);
    a.ntiles = (p.Cout + TN - 1) / TN;
    a.vec_store = (uintptr_t)p.Y % 16 == 0 && p.ys[0] % 4 == 0 && p.ys[1] % 4 == 0 && p.ys[2] % 4 == 0 &&
                  p.Cout % 4 == 0;
    a.div_kw = make_div((uint32_t)p.KW);
    a.div_wo = make_div((uint32_t)p.Wo);
    a.div_ho = make_div((uint32_t)p.Ho);
    a.div_coutg = make_div((uint32_t)a.cout_g);
    const int64_t tiles = (int64_t)(a.M + TM - 1) / TM * a.ntiles;
    hipLaunchKernelGGL(dense_gemm_mfma_f32, dim3((unsigned)tiles), dim3(GT), 0, s, a);
    return hipGetLastError();
}

}  // namespace convfwd
