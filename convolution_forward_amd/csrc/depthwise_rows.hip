// Depthwise convolution of 7- and 14-wide planes, one output row per thread.
//
// "Depthwise convolution" (onemodel docs), sections "What each output is"
// and "Layout of the work": output plane q = (n, oc) reads input plane
// q / multiplier; the sum starts at +0 and takes the taps row by row; a tap
// outside the input multiplies a real +0; exact mode rounds each product and
// then each sum, fast mode fuses them; the bias is one more rounded addition
// and exact mode rewrites a NaN result to 0x7FC00000. The arithmetic and its
// order are those of the direct kernel, so the bits are the same.
//
// The last stages of the mobile networks the page measures run 3x3 and 5x5
// windows with "same" padding over 7x7 and 14x14 planes (stride 1, or stride
// 2 from 14 to 7). With the row width W, the window and the stride fixed at
// compile time, a thread that owns a whole output row knows which of its
// taps fall in the left and right border: those multiply a literal +0 and
// read nothing. The rows above and below the plane are zero rows in LDS.
// So the only per-element work besides the multiply-adds is one LDS read
// per input word of the window rows; the copy is one division per element
// (which plane), since each plane's rows sit in LDS as they sit in X, after
// ph zero rows.
//  * A workgroup of NT threads (256, or 128 for 14-wide planes) takes
//    PPW = NT / Ho whole output planes; thread tid owns
//    output row tid % Ho of tile plane tid / Ho.
//  * The planes' pitch in LDS is chosen on the host so that the row starts
//    of the 64 lanes of a wave fall on as few shared banks as possible.
//  * The tile's outputs are one contiguous range of Y, written from LDS in
//    16-byte streaming stores.
#include <algorithm>

#include "common.h"
#include "dw_range_store.h"
#include "fastdiv.h"
#include "internal.h"

namespace convfwd {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Threads per workgroup: 256 for the 7-wide planes, 128 for the 14-wide
// ones (half as many planes per workgroup, twice as many workgroups: the
// 672-channel 5x5/2 layer 7.55 -> 7.20 us; the 960-channel 7-wide layer is
// 1.5 % slower that way and 12 % slower with 512).
constexpr int threads_for(int W) { return W == 14 ? 128 : 256; }
constexpr int BATCH = 8;             // 4-byte loads in flight per thread per round
constexpr int BATCH4 = 4;            // 16-byte loads in flight per thread per round
constexpr uint32_t OOB = 0x80000000u;
constexpr int BUF_WORD3 = 0x00020000;
constexpr int LDS_LIMIT = 64 * 1024;
constexpr int BANKS = 64;

struct RowsArgs {
    const float *X;
    const float *w;
    const float *bias;
    float *Y;
    int HW, Cout, Ho, HoWo, ph;
    int planes;        // N * Cout output planes
    int PPW;           // output planes per workgroup
    int PP;            // LDS words per plane (zero rows, data rows, zero rows, bank padding)
    int zero_words;    // LDS words cleared before the copy (a multiple of 4)
    int y_aligned;     // Y starts on a 16-byte boundary
    int x_chunks;      // X is 16-byte aligned and a whole number of 16-byte pieces
    FastDiv div_ho, div_mult, div_cout, div_hw;
};

template <int W, int K, int S, int EXACT, int NT>
__global__ __launch_bounds__(NT) void dw_rows_kernel(RowsArgs a)
{
#pragma clang fp contract(off)
    extern __shared__ __align__(16) float lds[];
    constexpr int PAD = K / 2;                       // border columns on each side
    constexpr int WO = (W + 2 * PAD - K) / S + 1;    // outputs per row
    constexpr int XW = (WO - 1) * S + K;             // padded columns the row's outputs read
    constexpr int KK = K * K;
    const int tid = threadIdx.x;

    // Output planes [q0, qend) read input planes [ip0, ip0 + nip).
    const int q0 = with_args_loaded((int)blockIdx.x, a) * a.PPW;
    const int qend = min(q0 + a.PPW, a.planes);
    const int ip0 = (int)fdiv((uint32_t)q0, a.div_mult);
    const int nip = (int)fdiv((uint32_t)(qend - 1), a.div_mult) - ip0 + 1;

    // The thread's task: output row oy of tile plane p.
    const int p = (int)fdiv((uint32_t)tid, a.div_ho);
    const int oy = tid - p * a.Ho;
    const int q = q0 + p;
    const bool active = p < a.PPW && q < qend;
    const int qc = active ? q : q0;
    const int ip = (int)fdiv((uint32_t)qc, a.div_mult);
    const int occ = qc - (int)fdiv((uint32_t)qc, a.div_cout) * a.Cout;

    // Element j of the tile's input planes, X[ip0 * HW + j], goes to LDS word
    // j + pl * (PP - HW) + ph * W with pl = j / HW.
    const int nelem = nip * a.HW;
    const int gap = a.PP - a.HW;
    const int top = a.ph * W;
    float wv[KK];
    float bv = 0.0f;
    // Behind the first loads: the weights and bias of the thread's plane, and
    // the zero rows (the whole area is cleared).
    auto behind_first_loads = [&]() {
#pragma unroll
        for (int k = 0; k < KK; ++k)
            wv[k] = a.w[(int64_t)occ * KK + k];
        if (a.bias)
            bv = a.bias[occ];
        for (int e = tid * 4; e < a.zero_words; e += NT * 4)
            *reinterpret_cast<f32x4 *>(lds + e) = f32x4{0.f, 0.f, 0.f, 0.f};
        __syncthreads();
    };
    if (a.x_chunks) {
        // Piece k holds elements 4k - lead .. 4k - lead + 3 of the tile; it
        // is 16-byte aligned because X is and X's length is a multiple of 4.
        const int lead = (int)(((int64_t)ip0 * a.HW) & 3);
        const int nch = (lead + nelem + 3) >> 2;
        const __amdgpu_buffer_rsrc_t cr = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float *>(a.X + ((int64_t)ip0 * a.HW - lead)), 0, nch * 16, BUF_WORD3);
        auto issue = [&](int base, f32x4 *v) {
#pragma unroll
            for (int u = 0; u < BATCH4; ++u) {
                const int k = base + u * NT + tid;
                if (base + u * NT < nch)
                    v[u] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                         cr, k < nch ? (uint32_t)k * 16 : OOB, 0, 0));
            }
        };
        auto place = [&](int base, const f32x4 *v) {
#pragma unroll
            for (int u = 0; u < BATCH4; ++u) {
                const int k = base + u * NT + tid;
                if (base + u * NT < nch && k < nch) {
                    // One division per piece: the plane of its first element,
                    // and how many of its elements stay in that plane.
                    const int j0 = 4 * k - lead;
                    const int pl = (int)fdiv((uint32_t)max(j0, 0), a.div_hw);
                    const int in_plane = (pl + 1) * a.HW - j0;
                    float *d0 = lds + (j0 + pl * gap + top);
                    if (j0 >= 0 && j0 + 4 <= nelem) {
                        // Whole piece inside the tile. Planes of a multiple of
                        // 4 elements never split a piece; otherwise the
                        // elements past the plane's end move on by the gap.
                        if (a.HW % 4 == 0) {
#pragma unroll
                            for (int i = 0; i < 4; ++i)
                                d0[i] = v[u][i];
                        } else {
                            d0[0] = v[u][0];
#pragma unroll
                            for (int i = 1; i < 4; ++i)
                                d0[i + (i >= in_plane ? gap : 0)] = v[u][i];
                        }
                    } else {
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            if (j0 + i >= 0 && j0 + i < nelem)
                                d0[i + (i >= in_plane ? gap : 0)] = v[u][i];
                    }
                }
            }
        };
        f32x4 v[BATCH4];
        issue(0, v);
        behind_first_loads();
        place(0, v);
        for (int base = NT * BATCH4; base < nch; base += NT * BATCH4) {
            issue(base, v);
            place(base, v);
        }
    } else {
        const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float *>(a.X + (int64_t)ip0 * a.HW), 0, nelem * 4, BUF_WORD3);
        auto issue = [&](int base, float *v) {
#pragma unroll
            for (int u = 0; u < BATCH; ++u) {
                const int j = base + u * NT + tid;
                if (base + u * NT < nelem)
                    v[u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(xr, j < nelem ? (uint32_t)j * 4 : OOB, 0, 0));
            }
        };
        auto place = [&](int base, const float *v) {
#pragma unroll
            for (int u = 0; u < BATCH; ++u) {
                const int j = base + u * NT + tid;
                if (base + u * NT < nelem && j < nelem) {
                    const int pl = (int)fdiv((uint32_t)j, a.div_hw);
                    lds[j + pl * gap + top] = v[u];
                }
            }
        };
        float v[BATCH];
        issue(0, v);
        behind_first_loads();
        place(0, v);
        for (int base = NT * BATCH; base < nelem; base += NT * BATCH) {
            issue(base, v);
            place(base, v);
        }
    }
    __syncthreads();

    float acc[WO];
#pragma unroll
    for (int t = 0; t < WO; ++t)
        acc[t] = +0.0f;
    if (active) {
        // Filter row ky of output row oy reads LDS row oy * S + ky of the
        // plane (row 0 is the first of the ph zero rows).
        const float *pb = lds + (ip - ip0) * a.PP + oy * S * W;
#pragma unroll
        for (int ky = 0; ky < K; ++ky) {
            const float *rp = pb + ky * W;
            // Padded column c is input column c - PAD: a literal +0 outside.
            float xv[XW];
#pragma unroll
            for (int c = 0; c < XW; ++c)
                xv[c] = (c - PAD >= 0 && c - PAD < W) ? rp[c - PAD] : +0.0f;
#pragma unroll
            for (int ox = 0; ox < WO; ++ox) {
#pragma unroll
                for (int kx = 0; kx < K; ++kx) {
                    if constexpr (EXACT) {
                        const float prod = wv[ky * K + kx] * xv[ox * S + kx];
                        acc[ox] = acc[ox] + prod;
                    } else {
                        acc[ox] = __builtin_fmaf(wv[ky * K + kx], xv[ox * S + kx], acc[ox]);
                    }
                }
            }
        }
    }

    // Outputs: Y elements [ostart, ostart + olen) through LDS (lead as in
    // store_range_from_lds).
    const int64_t ostart = (int64_t)q0 * a.HoWo;
    const int olen = (qend - q0) * a.HoWo;
    const int lead = a.y_aligned ? (int)(ostart & 3) : 0;
    __syncthreads();                                   // every tap read is done
    if (active) {
        float *op = lds + lead + p * a.HoWo + oy * WO;
#pragma unroll
        for (int ox = 0; ox < WO; ++ox) {
            float r = acc[ox];
            if (a.bias)
                r = r + bv;
            if (EXACT && __builtin_isnan(r))
                r = __uint_as_float(0x7FC00000u);
            op[ox] = r;
        }
    }
    __syncthreads();
    store_range_from_lds<NT, NT * WO + 3>(lds, a.Y, ostart, olen, lead, a.y_aligned, tid);
}

// --- host side -------------------------------------------------------------

struct RowsPlan {
    int PPW, PP;
    int64_t lds_words;
};

// The most lanes of one wave whose row start falls on one bank, for plane
// pitch pp (thread tid reads from word (tid / Ho) * pp + (tid % Ho) * S * W).
int worst_bank_share(int pp, int Ho, int S, int W, int ppw, int nt)
{
    int worst = 0;
    for (int w0 = 0; w0 < nt; w0 += 64) {
        int count[BANKS] = {};
        for (int t = w0; t < w0 + 64; ++t) {
            const int p = t / Ho, oy = t % Ho;
            if (p >= ppw)
                continue;
            const int b = (int)(((int64_t)p * pp + (int64_t)oy * S * W) % BANKS);
            worst = std::max(worst, ++count[b]);
        }
    }
    return worst;
}

bool rows_plan(const DwProblem &p, RowsPlan &t)
{
    const int K = p.KH;
    if (p.KH != p.KW || (K != 3 && K != 5) || (p.W != 7 && p.W != 14))
        return false;
    if (p.sh != p.sw || (p.sh != 1 && p.sh != 2) || p.dh != 1 || p.dw != 1)
        return false;
    if (p.pw != K / 2 || p.pr != K / 2 || p.ph >= K || p.pb >= K)
        return false;       // "same" columns; every output window overlaps the input
    const int S = p.sh;
    const int WO = (p.W + 2 * (K / 2) - K) / S + 1;
    const int nt = threads_for(p.W);
    if (p.Wo != WO || p.Ho < 1 || p.Ho * 2 > nt)
        return false;
    const int64_t planes = (int64_t)p.N * p.C * p.mult;
    if (planes >= (1ll << 31) - nt || planes * p.Ho * p.Wo >= (1ll << 40) ||
        (int64_t)p.C * p.mult * K * K >= (1ll << 31) || (int64_t)p.H * p.W >= (1ll << 24) ||
        (int64_t)p.N * p.C * p.H * p.W >= (1ll << 40))
        return false;
    // LDS rows per plane: ph zero rows, H data rows, then zero rows down to
    // the last row an output reads.
    const int rows = std::max(p.H + p.ph, (p.Ho - 1) * S + K);
    const int pp0 = rows * p.W;
    t.PPW = nt / p.Ho;
    int best = 1 << 30;
    for (int pp = pp0; pp < pp0 + BANKS; ++pp) {
        const int share = worst_bank_share(pp, p.Ho, S, p.W, t.PPW, nt);
        if (share < best) {
            best = share;
            t.PP = pp;
        }
    }
    auto words_for = [&](int ppw) {
        const int64_t nip = (ppw - 1 + p.mult - 1) / p.mult + 1;
        const int64_t in = ((nip * t.PP + 3) / 4) * 4;
        return std::max<int64_t>(in, (int64_t)nt * WO + 4);
    };
    while (t.PPW > 2 && words_for(t.PPW) * 4 > LDS_LIMIT)
        --t.PPW;
    if (words_for(t.PPW) * 4 > LDS_LIMIT)
        return false;
    t.lds_words = words_for(t.PPW);
    return (planes + t.PPW - 1) / t.PPW < (1ll << 31);
}

template <int W, int K, int S>
hipError_t launch_wks(const RowsArgs &a, unsigned grid, size_t lds, bool exact, hipStream_t s)
{
    constexpr int NT = threads_for(W);
    if (exact)
        hipLaunchKernelGGL((dw_rows_kernel<W, K, S, 1, NT>), dim3(grid), dim3(NT), lds, s, a);
    else
        hipLaunchKernelGGL((dw_rows_kernel<W, K, S, 0, NT>), dim3(grid), dim3(NT), lds, s, a);
    return hipGetLastError();
}

template <int W>
hipError_t launch_w(const RowsArgs &a, int K, int S, unsigned grid, size_t lds, bool exact, hipStream_t s)
{
    if (K == 3)
        return S == 1 ? launch_wks<W, 3, 1>(a, grid, lds, exact, s) : launch_wks<W, 3, 2>(a, grid, lds, exact, s);
    return S == 1 ? launch_wks<W, 5, 1>(a, grid, lds, exact, s) : launch_wks<W, 5, 2>(a, grid, lds, exact, s);
}

}  // namespace

bool dw_rows_supports(const DwProblem &p)
{
    RowsPlan t;
    return rows_plan(p, t);
}

hipError_t launch_dw_rows(const DwProblem &p, hipStream_t s)
{
    RowsPlan t;
    if (!rows_plan(p, t))
        return hipErrorNotSupported;
    RowsArgs a;
    a.X = p.X;
    a.w = p.w;
    a.bias = p.bias;
    a.Y = p.Y;
    a.HW = p.H * p.W;
    a.Cout = p.C * p.mult;
    a.Ho = p.Ho;
    a.HoWo = p.Ho * p.Wo;
    a.ph = p.ph;
    a.planes = p.N * p.C * p.mult;
    a.PPW = t.PPW;
    a.PP = t.PP;
    const int nip_max = (t.PPW - 1 + p.mult - 1) / p.mult + 1;
    a.zero_words = ((nip_max * t.PP + 3) / 4) * 4;
    a.y_aligned = (reinterpret_cast<uintptr_t>(p.Y) & 15) == 0;
    a.x_chunks = (reinterpret_cast<uintptr_t>(p.X) & 15) == 0 && ((int64_t)p.N * p.C * p.H * p.W) % 4 == 0;
    a.div_ho = make_fastdiv((uint32_t)p.Ho);
    a.div_mult = make_fastdiv((uint32_t)p.mult);
    a.div_cout = make_fastdiv((uint32_t)a.Cout);
    a.div_hw = make_fastdiv((uint32_t)a.HW);
    const int64_t tiles = ((int64_t)a.planes + t.PPW - 1) / t.PPW;
    const size_t lds = (size_t)t.lds_words * 4;
    const bool exact = p.mode == CONV_DW_EXACT;
    return p.W == 7 ? launch_w<7>(a, p.KH, p.sh, (unsigned)tiles, lds, exact, s)
                    : launch_w<14>(a, p.KH, p.sh, (unsigned)tiles, lds, exact, s);
}

}  // namespace convfwd
