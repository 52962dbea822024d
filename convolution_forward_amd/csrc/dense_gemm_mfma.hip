// Dense NHWC cross-correlation, any window, as an implicit GEMM on matrix
// cores with the filter streamed through LDS.
//
// Contract: "CMU DLSys Lecture 14: Convolutional Network Implementation",
// sections 1 and 5 (Y = patch matrix times F.reshape(K*K*Cin, Cout), the
// patch matrix never built), with the window of "Convolution Is Wx+b Moving
// Across a Signal" (section "Why 1D? Why 2D?": output (y, x) reads input
// row y*sh + i*dh - pt and column x*sw + j*dw - pl, zero outside) and its
// groups (section "Find the same sum in CKE's C kernels").
//
// This kernel takes what the row kernel (dense_mfma.hip) declines: more
// than 64 input channels under a 3x3 window, 5x5 and larger windows,
// dilation, unequal strides, and 1D sequences longer than a row tile. It
// holds nothing per band: the GEMM's M axis is the flat output pixel index
// m = (n*Ho + y)*Wo + x, so any output shape tiles evenly.
//
// Work decomposition (one workgroup = 4 waves = 256 threads):
//  * A tile is 256 output pixels x 64 output channels of one group. Wave w
//    owns pixels 64w..64w+63 of the tile (four 16-pixel blocks) and all 64
//    channels (four 16-channel column blocks): 16 accumulators, each MFMA
//    reading 256 bytes of LDS for A and 256 bytes of memory for B.
//  * The K axis runs over (tap i, tap j, 32-channel step), the lecture's
//    (i, j, c) order. A chunk of KC steps of the filter slice
//    F[i, j, c, o0:o0+64] is loaded coalesced, written to LDS in its natural
//    layout (double buffered: the next chunk's loads are in flight while the
//    current chunk is used) and read as A fragments with the gfx950
//    transpose read ds_read_b64_tr_b16.
//  * B fragments (8 channels of one pixel, 16 bytes per lane) are gathered
//    straight from X for each step, one step ahead of use. Taps in the
//    padding and pixels past the end use out-of-range buffer offsets, which
//    load zeros without touching memory.
//  * bf16 results are regrouped through the (by then idle) filter buffer:
//    each wave parks its 64 pixels x 64 channels there, then eight lanes
//    store each pixel's 128-byte row whole (stores of 8 bytes in 32-byte
//    runs drain several times slower). fp32 results leave straight from the
//    accumulators, 16 bytes per lane in 64-byte runs.
#include <type_traits>

#include "common.h"
#include "internal.h"

namespace convfwd {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));

constexpr int GT = 256;                 // threads per workgroup
constexpr int GM = 256;                 // output pixels per tile
constexpr int GN = 64;                  // output channels per tile
constexpr int BLK = 4;                  // 16-pixel blocks per wave
constexpr int NB = 4;                   // 16-channel column blocks per wave
constexpr int KC = 4;                   // 32-channel steps per filter chunk
constexpr int FP = GN + 8;              // LDS row pitch of a filter chunk (elements)
constexpr int CHUNK_ELEMS = KC * 32 * FP;
constexpr int FITEMS = KC * 32 * (GN / 8) / GT;   // 16-byte filter loads per thread per chunk
constexpr int OPITCH = GN * 2 + 16;     // LDS pitch of one pixel of a wave's bf16 output patch (bytes)
static_assert(GT / 64 * 64 * OPITCH <= 2 * CHUNK_ELEMS * 2, "output patches fit in the filter buffer");
constexpr uint32_t OOB = 0x80000000u;
constexpr int BUF_WORD3 = 0x00020000;

struct FastDivG {
    uint32_t m, s;
};

FastDivG make_fastdiv_g(uint32_t d)
{
    uint32_t s = 0;
    while ((1ull << s) < d)
        ++s;
    return FastDivG{(uint32_t)(((1ull << 32) * ((1ull << s) - d)) / d + 1), s};
}

__device__ __forceinline__ uint32_t fdiv_g(uint32_t n, FastDivG f) { return (__umulhi(n, f.m) + n) >> f.s; }

struct GemmArgs {
    const uint16_t *X;
    const uint16_t *F;
    const float *bias;
    void *Y;
    int64_t xs0, xs1, xs2, ys0, ys1, ys2;
    int H, W, Ho, Wo, KW;
    int Cin, Cout;          // channels of one group
    int f_ld;               // F row length (output channels of all groups)
    int sh, sw, pt, pl, dh, dw;
    int cs_steps;           // 32-channel steps per tap
    int ksteps;             // KH * KW * cs_steps
    int m_total;            // N * Ho * Wo
    int n_tiles;            // 64-channel tiles per group
    int nt_all;             // n_tiles * groups: channel tiles per pixel tile
    int tiles;              // pixel tiles * nt_all
    uint32_t x_records, f_records, b_records;
    FastDivG div_wo, div_ho;
};

template <bool OUT_BF16>
__global__ __launch_bounds__(GT) void dense_gemm_mfma(GemmArgs a)
{
    constexpr int ESZ = OUT_BF16 ? 2 : 4;
    __shared__ __align__(16) uint16_t fbuf[2][CHUNK_ELEMS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int g = lane >> 4;                 // k-group of the lane
    const int r = lane & 15;
    // Slot s runs on XCD s % 8; consecutive tiles (the channel tiles of one
    // pixel tile first) go to one XCD so the X rows they share meet in its L2.
    const int tile = (int)(blockIdx.x & 7) * (int)(gridDim.x >> 3) + (int)(blockIdx.x >> 3);
    if (tile >= a.tiles)
        return;
    const int mt = tile / a.nt_all;
    const int nt = tile - mt * a.nt_all;
    const int grp = nt / a.n_tiles;
    const int o0 = (nt - grp * a.n_tiles) * GN;
    const int xc0 = grp * a.Cin, oc0 = grp * a.Cout;

    // This lane's pixel in each of the wave's four blocks.
    int iy0[BLK], ix0[BLK], yo[BLK], xo[BLK];
    uint32_t nb0[BLK];
    bool mok[BLK];
#pragma unroll
    for (int b = 0; b < BLK; ++b) {
        const int m = mt * GM + wave * 64 + b * 16 + r;
        mok[b] = m < a.m_total;
        const uint32_t mm = mok[b] ? (uint32_t)m : 0u;
        const uint32_t ny = fdiv_g(mm, a.div_wo);
        xo[b] = (int)(mm - ny * (uint32_t)a.Wo);
        const uint32_t n = fdiv_g(ny, a.div_ho);
        yo[b] = (int)(ny - n * (uint32_t)a.Ho);
        nb0[b] = n;
        iy0[b] = yo[b] * a.sh - a.pt;
        ix0[b] = xo[b] * a.sw - a.pl;
    }

    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(a.X), 0, (int)a.x_records, BUF_WORD3);
    const __amdgpu_buffer_rsrc_t fr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(a.F), 0, (int)a.f_records, BUF_WORD3);

    // Filter chunk q: items it -> (8-channel output group og fastest, then
    // row kk*32 + c of the chunk).
    auto chunk_load = [&](int q, u32x4 (&fv)[FITEMS]) __attribute__((always_inline)) {
#pragma unroll
        for (int t = 0; t < FITEMS; ++t) {
            const int it = tid + t * GT;
            const int og = it & 7;
            const int row = it >> 3;
            const int ks = q * KC + row / 32;
            const int c = row % 32;
            const int tap = ks / a.cs_steps;
            const int cc = (ks - tap * a.cs_steps) * 32 + c;
            const int o = o0 + og * 8;
            const bool ok = ks < a.ksteps && cc < a.Cin && o < a.Cout;
            fv[t] = __builtin_amdgcn_raw_buffer_load_b128(
                fr, ok ? (uint32_t)((((int64_t)tap * a.Cin + cc) * a.f_ld + oc0 + o) * 2) : OOB, 0, 0);
        }
    };
    auto chunk_store = [&](int buf, const u32x4 (&fv)[FITEMS]) __attribute__((always_inline)) {
#pragma unroll
        for (int t = 0; t < FITEMS; ++t) {
            const int it = tid + t * GT;
            *reinterpret_cast<u32x4 *>(&fbuf[buf][(it >> 3) * FP + (it & 7) * 8]) = fv[t];
        }
    };
    // B fragments of step ks for the four blocks.
    auto b_load = [&](int ks, bf16x8 (&xb)[BLK]) __attribute__((always_inline)) {
        const int tap = ks / a.cs_steps;
        const int cs = ks - tap * a.cs_steps;
        const int i = tap / a.KW;
        const int j = tap - i * a.KW;
        const int c = cs * 32 + g * 8;
#pragma unroll
        for (int b = 0; b < BLK; ++b) {
            const int iy = iy0[b] + i * a.dh;
            const int ix = ix0[b] + j * a.dw;
            const bool ok = mok[b] && ks < a.ksteps && iy >= 0 && iy < a.H && ix >= 0 && ix < a.W && c < a.Cin;
            const uint32_t off = ok ? (uint32_t)(((int64_t)nb0[b] * a.xs0 + (int64_t)iy * a.xs1 +
                                                  (int64_t)ix * a.xs2 + xc0 + c) * 2)
                                    : OOB;
            xb[b] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0));
        }
    };

    f32x4 acc[BLK][NB];
#pragma unroll
    for (int b = 0; b < BLK; ++b)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
            acc[b][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nchunks = (a.ksteps + KC - 1) / KC;
    u32x4 fv[FITEMS];
    chunk_load(0, fv);
    bf16x8 xb[BLK], xn[BLK];
    b_load(0, xn);
    chunk_store(0, fv);
    __syncthreads();

    for (int q = 0; q < nchunks; ++q) {
        if (q + 1 < nchunks)
            chunk_load(q + 1, fv);
        const uint16_t *ft = fbuf[q & 1];
#pragma unroll
        for (int kk = 0; kk < KC; ++kk) {
            const int ks = q * KC + kk;
            if (ks < a.ksteps) {
                // A fragments (see FilterSlice in dense_mfma.hip for the
                // transpose-read lane layout): lane r of a 16-lane group
                // addresses row kk*32 + 8g + 4h + r/4, columns 4*(r%4).
                bf16x8 wf[NB];
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    i16x4 part[2];
#pragma unroll
                    for (int h = 0; h < 2; ++h)
                        part[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (__attribute__((address_space(3))) i16x4 *)(ft + (kk * 32 + g * 8 + h * 4 + (r >> 2)) * FP +
                                                                         nb * 16 + 4 * (r & 3)));
                    const i16x8 both = {part[0][0], part[0][1], part[0][2], part[0][3],
                                        part[1][0], part[1][1], part[1][2], part[1][3]};
                    wf[nb] = __builtin_bit_cast(bf16x8, both);
                }
#pragma unroll
                for (int b = 0; b < BLK; ++b)
                    xb[b] = xn[b];
                b_load(ks + 1, xn);
#pragma unroll
                for (int b = 0; b < BLK; ++b)
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb)
                        acc[b][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[nb], xb[b], acc[b][nb], 0, 0, 0);
            }
        }
        if (q + 1 < nchunks) {
            // The other buffer was last read in chunk q - 1, before the
            // barrier that ended it.
            chunk_store((q + 1) & 1, fv);
            __syncthreads();
        }
    }

    // Epilogue: lane holds channels o0 + 16nb + 4g + {0..3} of its pixel in
    // each block.
    const __amdgpu_buffer_rsrc_t br = __builtin_amdgcn_make_buffer_rsrc(
        a.bias ? (void *)(a.bias + oc0) : (void *)a.F, 0, a.bias ? (int)a.b_records : 0, BUF_WORD3);
    u32x4 bq[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
        bq[nb] = __builtin_amdgcn_raw_buffer_load_b128(br, (uint32_t)((o0 + nb * 16 + g * 4) * 4), 0, 0);
    if constexpr (OUT_BF16) {
        // Every wave is done with the filter buffer before any overwrites it.
        __syncthreads();
        uint8_t *patch = reinterpret_cast<uint8_t *>(&fbuf[0][0]) + wave * 64 * OPITCH;
#pragma unroll
        for (int b = 0; b < BLK; ++b)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const f32x4 v = acc[b][nb];
                const uint32_t lo = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)(v[0] + __uint_as_float(bq[nb][0]))) |
                                    ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)(v[1] + __uint_as_float(bq[nb][1]))) << 16);
                const uint32_t hi = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)(v[2] + __uint_as_float(bq[nb][2]))) |
                                    ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)(v[3] + __uint_as_float(bq[nb][3]))) << 16);
                *reinterpret_cast<u32x2 *>(patch + (b * 16 + r) * OPITCH + (nb * 16 + g * 4) * 2) = u32x2{lo, hi};
            }
        // The patch is this wave's own: its LDS writes complete before its
        // reads (in order), no barrier. Store i: lane L takes pixel
        // 8i + L/8 of the wave's 64, channels 8*(L%8)..+7.
        const int ch = o0 + (lane & 7) * 8;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int pp = i * 8 + (lane >> 3);
            const u32x4 w = *reinterpret_cast<const u32x4 *>(patch + pp * OPITCH + (lane & 7) * 16);
            const int m = mt * GM + wave * 64 + pp;
            if (m < a.m_total && ch < a.Cout) {
                const uint32_t ny = fdiv_g((uint32_t)m, a.div_wo);
                const int x = (int)((uint32_t)m - ny * (uint32_t)a.Wo);
                const uint32_t n = fdiv_g(ny, a.div_ho);
                const int y = (int)(ny - n * (uint32_t)a.Ho);
                char *yp = static_cast<char *>(a.Y) +
                           ((int64_t)n * a.ys0 + (int64_t)y * a.ys1 + (int64_t)x * a.ys2 + oc0 + ch) * 2;
                __builtin_nontemporal_store(w, reinterpret_cast<u32x4 *>(yp));   // nt: Conv1D stem -2.5 %
            }
        }
    } else {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int ch = o0 + nb * 16 + g * 4;
#pragma unroll
            for (int b = 0; b < BLK; ++b) {
                if (!mok[b] || ch >= a.Cout)
                    continue;
                const f32x4 v = acc[b][nb];
                char *yp = static_cast<char *>(a.Y) +
                           ((int64_t)nb0[b] * a.ys0 + (int64_t)yo[b] * a.ys1 + (int64_t)xo[b] * a.ys2 + oc0 + ch) * ESZ;
                *reinterpret_cast<f32x4 *>(yp) = f32x4{v[0] + __uint_as_float(bq[nb][0]), v[1] + __uint_as_float(bq[nb][1]),
                                                       v[2] + __uint_as_float(bq[nb][2]), v[3] + __uint_as_float(bq[nb][3])};
            }
        }
    }
}

}  // namespace

bool dense_gemm_bf16_supports(const DenseProblem &p)
{
    if (p.xdt != CONV_BF16)
        return false;
    const int cin_g = p.Cin / p.groups, cout_g = p.Cout / p.groups;
    if (cin_g % 8 != 0 || cout_g % 8 != 0)
        return false;
    if ((uintptr_t)p.X % 16 != 0 || p.xs[0] % 8 != 0 || p.xs[1] % 8 != 0 || p.xs[2] % 8 != 0)
        return false;
    const int yesz = p.ydt == CONV_BF16 ? 2 : 4;
    if ((uintptr_t)p.Y % (4 * yesz) != 0 || p.ys[0] % 4 != 0 || p.ys[1] % 4 != 0 || p.ys[2] % 4 != 0)
        return false;
    // bf16 rows leave in 16-byte pieces of 8 channels.
    if (p.ydt == CONV_BF16 && ((uintptr_t)p.Y % 16 != 0 || p.ys[0] % 8 != 0 || p.ys[1] % 8 != 0 || p.ys[2] % 8 != 0))
        return false;
    if ((uintptr_t)p.F % 16 != 0)
        return false;
    // 32-bit buffer offsets over all of X and F.
    const int64_t x_extent = ((int64_t)(p.N - 1) * p.xs[0] + (int64_t)(p.H - 1) * p.xs[1] +
                              (int64_t)(p.W - 1) * p.xs[2] + p.Cin) * 2;
    if (x_extent >= (int64_t(1) << 31) || (int64_t)p.KH * p.KW * cin_g * p.Cout * 2 >= (int64_t(1) << 31))
        return false;
    const int64_t m_total = (int64_t)p.N * p.Ho * p.Wo;
    const int64_t tiles = (m_total + GM - 1) / GM * ((cout_g + GN - 1) / GN) * p.groups;
    return m_total < (int64_t(1) << 31) - GM && tiles * 8 < (int64_t(1) << 31);
}

hipError_t launch_dense_gemm_bf16(const DenseProblem &p, hipStream_t s)
{
    if (!dense_gemm_bf16_supports(p))
        return hipErrorNotSupported;
    GemmArgs a;
    a.X = static_cast<const uint16_t *>(p.X);
    a.F = static_cast<const uint16_t *>(p.F);
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
    a.Ho = p.Ho;
    a.Wo = p.Wo;
    a.KW = p.KW;
    a.Cin = p.Cin / p.groups;
    a.Cout = p.Cout / p.groups;
    a.f_ld = p.Cout;
    a.sh = p.sh;
    a.sw = p.sw;
    a.pt = p.pt;
    a.pl = p.pl;
    a.dh = p.dh;
    a.dw = p.dw;
    a.cs_steps = (a.Cin + 31) / 32;
    a.ksteps = p.KH * p.KW * a.cs_steps;
    a.m_total = p.N * p.Ho * p.Wo;
    a.n_tiles = (a.Cout + GN - 1) / GN;
    const int m_tiles = (a.m_total + GM - 1) / GM;
    a.nt_all = a.n_tiles * p.groups;
    a.tiles = m_tiles * a.nt_all;
    a.x_records = (uint32_t)(((int64_t)(p.N - 1) * p.xs[0] + (int64_t)(p.H - 1) * p.xs[1] +
                              (int64_t)(p.W - 1) * p.xs[2] + p.Cin) * 2);
    a.f_records = (uint32_t)((int64_t)p.KH * p.KW * a.Cin * p.Cout * 2);
    a.b_records = (uint32_t)(a.Cout * 4);
    a.div_wo = make_fastdiv_g((uint32_t)p.Wo);
    a.div_ho = make_fastdiv_g((uint32_t)p.Ho);
    const unsigned grid = (unsigned)((a.tiles + 7) / 8 * 8);
    if (p.ydt == CONV_BF16)
        hipLaunchKernelGGL(dense_gemm_mfma<true>, dim3(grid), dim3(GT), 0, s, a);
    else
        hipLaunchKernelGGL(dense_gemm_mfma<false>, dim3(grid), dim3(GT), 0, s, a);
    return hipGetLastError();
}

}  // namespace convfwd
