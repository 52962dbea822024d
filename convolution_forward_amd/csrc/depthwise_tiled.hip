// Depthwise convolution staged through LDS: the bandwidth-bound kernel.
//
// "Depthwise convolution" (onemodel docs), sections "What each output is"
// and "Layout of the work": output plane q = (n, oc) reads input
// plane q / multiplier; the sum starts at +0 and takes the taps row by row;
// a tap outside the input multiplies a real +0; exact mode rounds each
// product and then each sum, fast mode fuses them; the bias is one more
// rounded addition and exact mode rewrites a NaN result to 0x7FC00000. The
// same page asks for identical bits on every code path, so this kernel must
// reproduce the direct kernel (and the oracle) exactly: it differs only in
// how the input reaches the arithmetic, never in the arithmetic or its order.
//
// Organisation (one workgroup = 256 threads):
//  * A tile is PPW consecutive output planes (small planes) or a band of RB
//    output rows of one plane (large planes). Its input is one contiguous
//    range of X (NCHW planes are contiguous, and so are consecutive rows and
//    consecutive planes). The workgroup copies that range, widened to 16-byte
//    chunks plus a few elements of slack on each side, into LDS with 16-byte
//    buffer loads, all issued before the first wait so the whole tile is in
//    flight at once. Chunks outside X load as zeros.
//  * Stride 2: the copy splits elements by the parity of their index into
//    two phase planes (even half, odd half). Input columns 2*ox + kx of
//    neighbouring lanes then sit at neighbouring LDS words, as they do at
//    stride 1, so tap reads stay free of bank conflicts. (Row lengths are
//    even, so index parity is column parity.)
//  * A thread owns one output column of RT consecutive output rows (the
//    narrow-row idea: each input value read from LDS serves up to KH of the
//    thread's outputs). Neighbouring lanes own neighbouring columns.
//  * Taps that fall in the padding read whatever neighbour sits in LDS and
//    replace it with +0 before the multiply: the arithmetic sees exactly the
//    zero the definition puts there.
//  * The weights of the tile's planes follow the tile into LDS, one 4-byte
//    load straight into LDS per weight, issued behind the tile's first
//    loads; after the copy each thread takes its plane's weights into
//    registers.
//  * The thread stores its RT outputs directly, with streaming stores
//    (neighbouring lanes write neighbouring words of a row). Small planes
//    (whole planes per workgroup) normally go to the kernel in
//    depthwise_planes.hip; this one takes them only when that one declines.
#include <algorithm>

#include "common.h"
#include "fastdiv.h"
#include "internal.h"

namespace convfwd {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int THREADS = 256;
constexpr int BATCH = 8;             // 16-byte loads in flight per thread per round
constexpr int SLACK = 12;            // LDS elements before/after the tile range (>= max pad, multiple of 4)
constexpr int MAX_PAD = 8;
constexpr uint32_t OOB = 0x80000000u;
constexpr int BUF_WORD3 = 0x00020000;
constexpr int LDS_LIMIT = 64 * 1024;

struct TileArgs {
    const float *X;
    const float *w;
    const float *bias;
    float *Y;
    int64_t XE;        // elements of X
    int64_t HW;        // elements per input plane
    int H, W, Cout, Ho, Wo, ph, pw;
    int planes;        // N * Cout output planes
    int PPW;           // output planes per tile
    int bands;         // tiles per plane (1 when PPW > 1)
    int RB;            // output rows per band
    int TPP;           // threads per plane: (row groups) * Wo
    int half;          // LDS elements per phase plane (stride 2)
    int wofs;          // LDS element where the tile's weights start
    int HoWo;          // outputs per plane
    FastDiv div_bands, div_tpp, div_wo, div_mult, div_cout;
};

template <int KH, int KW, int S, int RT, int EXACT>
__global__ __launch_bounds__(THREADS) void dw_tiled_kernel(TileArgs a)
{
#pragma clang fp contract(off)
    extern __shared__ __align__(16) float lds[];
    const int tid = threadIdx.x;

    // Tile: output planes [q0, qend), output rows [oy_lo, oy_hi).
    const uint32_t bid = (uint32_t)with_args_loaded((int)blockIdx.x, a);
    const uint32_t tile = fdiv(bid, a.div_bands);
    const int band = (int)(bid - tile * (uint32_t)a.bands);
    const int q0 = (int)tile * a.PPW;
    const int qend = min(q0 + a.PPW, a.planes);
    const int oy_lo = band * a.RB;
    const int oy_hi = min(a.Ho, oy_lo + a.RB);
    // Input rows any output of the tile reads, clipped to the plane.
    const int iy_lo = max(0, oy_lo * S - a.ph);
    const int iy_hi = min(a.H, (oy_hi - 1) * S - a.ph + KH);
    const int ip0 = (int)fdiv((uint32_t)q0, a.div_mult);
    const int ip1 = (int)fdiv((uint32_t)(qend - 1), a.div_mult);
    const int64_t e0 = (int64_t)ip0 * a.HW + (int64_t)iy_lo * a.W;
    const int64_t e1 = (int64_t)ip1 * a.HW + (int64_t)iy_hi * a.W;
    const int64_t a0 = (e0 & ~(int64_t)3) - SLACK;                 // X index of LDS element 0
    const int nchunks = (int)((((e1 + 3) & ~(int64_t)3) + SLACK - a0) >> 2);

    // The thread's task (decided now so the weight loads overlap the copy).
    const int p = (int)fdiv((uint32_t)tid, a.div_tpp);
    const int rem = tid - p * a.TPP;
    const int g = (int)fdiv((uint32_t)rem, a.div_wo);
    const int ox = rem - g * a.Wo;
    const int q = q0 + p;
    const int oy0 = oy_lo + g * RT;
    const bool active = p < a.PPW && q < qend && oy0 < oy_hi;
    const int qc = active ? q : q0;
    const int ip = (int)fdiv((uint32_t)qc, a.div_mult);
    const int occ = qc - (int)fdiv((uint32_t)qc, a.div_cout) * a.Cout;
    constexpr int KK = KH * KW;
    float *wl = lds + a.wofs;
    float bv = 0.0f;

    // Copy the tile range into LDS, BATCH chunks per thread per round: all
    // loads of a round are issued before the first write waits for them.
    const int64_t abase = a0 > 0 ? a0 : 0;
    const int64_t avail = (a.XE - abase) * 4;
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float *>(a.X + abase), 0, (int)(avail < 0x7FFFFFF0 ? avail : 0x7FFFFFF0), BUF_WORD3);
    for (int base = 0; base < nchunks; base += THREADS * BATCH) {
        f32x4 v[BATCH];
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            // Slots past the range for the whole workgroup issue nothing.
            if (base + u * THREADS < nchunks) {
                const int k = base + tid + u * THREADS;
                const int64_t e = a0 + 4 * (int64_t)k;
                const bool ok = k < nchunks && e >= 0 && e < a.XE;
                v[u] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                     xr, ok ? (uint32_t)((e - abase) * 4) : OOB, 0, 0));
            }
        }
        if (base == 0) {
            // Weight e of the tile is tap e % KK of plane q0 + e / KK, whose
            // output channel is the plane's index modulo Cout.
            const __amdgpu_buffer_rsrc_t wr =
                __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(a.w), 0, a.Cout * KK * 4, BUF_WORD3);
            const int nw = (qend - q0) * KK;
            for (int w0 = 0; w0 < nw; w0 += THREADS) {
                const int e = w0 + tid;
                const int pe = e / KK;
                const int qe = q0 + (e < nw ? pe : 0);
                const int ce = qe - (int)fdiv((uint32_t)qe, a.div_cout) * a.Cout;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    wr, (__attribute__((address_space(3))) void *)(wl + w0 + (tid & ~63)), 4,
                    e < nw ? (uint32_t)((ce * KK + e - pe * KK) * 4) : OOB, 0, 0, 0);
            }
            if (a.bias)
                bv = a.bias[occ];
        }
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            const int k = base + tid + u * THREADS;
            if (k < nchunks) {
                if constexpr (S == 1) {
                    *reinterpret_cast<f32x4 *>(lds + 4 * k) = v[u];
                } else {
                    *reinterpret_cast<f32x2 *>(lds + 2 * k) = f32x2{v[u][0], v[u][2]};
                    *reinterpret_cast<f32x2 *>(lds + a.half + 2 * k) = f32x2{v[u][1], v[u][3]};
                }
            }
        }
    }
    __syncthreads();
    if (!active)
        return;

    float acc[RT];
#pragma unroll
    for (int t = 0; t < RT; ++t)
        acc[t] = +0.0f;
    float wv[KK];
#pragma unroll
    for (int k = 0; k < KK; ++k)
        wv[k] = wl[p * KK + k];

    // Column validity of each tap (the same for every row).
    const int ix0 = ox * S - a.pw;
    bool cok[KW];
#pragma unroll
    for (int kx = 0; kx < KW; ++kx)
        cok[kx] = (unsigned)(ix0 + kx) < (unsigned)a.W;

    // Input row iy of plane ip sits at LDS element (ip*HW + iy*W - a0) (stride
    // 1). Rows outside the plane are read from a clamped row and zeroed.
    const int plane_rel = (int)((int64_t)ip * a.HW - a0);

    constexpr int NIR = (RT - 1) * S + KH;     // input rows the thread's outputs read
#pragma unroll
    for (int ir = 0; ir < NIR; ++ir) {
        const int iy = oy0 * S - a.ph + ir;
        const bool rok = (unsigned)iy < (unsigned)a.H;
        const int iyc = min(max(iy, iy_lo), iy_hi - 1);
        const int rb = plane_rel + iyc * a.W + ix0;   // LDS element of tap kx = 0 (stride 1)
        float xv[KW];
        if constexpr (S == 1) {
#pragma unroll
            for (int kx = 0; kx < KW; ++kx)
                xv[kx] = lds[rb + kx];
        } else {
            // Element e lives at (e & 1) * half + (e >> 1); rb >= 0 here.
            const int b0 = (rb & 1) * a.half + (rb >> 1);
            const int b1 = ((rb + 1) & 1) * a.half + ((rb + 1) >> 1);
#pragma unroll
            for (int kx = 0; kx < KW; ++kx)
                xv[kx] = (kx & 1) ? lds[b1 + (kx >> 1)] : lds[b0 + (kx >> 1)];
        }
#pragma unroll
        for (int kx = 0; kx < KW; ++kx)
            xv[kx] = (rok && cok[kx]) ? xv[kx] : +0.0f;
        // This input row is filter row ky = ir - t*S of output row t.
#pragma unroll
        for (int t = 0; t < RT; ++t) {
            const int ky = ir - t * S;
            if (ky >= 0 && ky < KH) {
#pragma unroll
                for (int kx = 0; kx < KW; ++kx) {
                    if constexpr (EXACT) {
                        const float prod = wv[ky * KW + kx] * xv[kx];
                        acc[t] = acc[t] + prod;
                    } else {
                        acc[t] = __builtin_fmaf(wv[ky * KW + kx], xv[kx], acc[t]);
                    }
                }
            }
        }
        // One input row at a time (its sums pinned here), so the compiler
        // does not read every row ahead of the arithmetic.
#pragma unroll
        for (int t = 0; t < RT; ++t)
            asm volatile("" : "+v"(acc[t]));
    }

    // Direct streaming stores: neighbouring lanes write neighbouring words
    // of an output row.
    float *yp = a.Y + (int64_t)q * a.HoWo + ox;
#pragma unroll
    for (int t = 0; t < RT; ++t) {
        const int oy = oy0 + t;
        if (oy < oy_hi) {
            float r = acc[t];
            if (a.bias)
                r = r + bv;
            if (EXACT && __builtin_isnan(r))
                r = __uint_as_float(0x7FC00000u);
            __builtin_nontemporal_store(r, &yp[(int64_t)oy * a.Wo]);
        }
    }
}

// Filters one row tall (1D along the width: causal and strided Conv1D over
// a sequence, "Convolution Is Wx+b Moving Across a Signal", section "Where
// this shows up in models I work with"). Planes are single rows here, so a
// workgroup takes a segment of SEG outputs of one output row instead of
// whole planes: it copies the input span the segment reads (zeros outside
// the row) into LDS with one 4-byte load per element, then each thread
// computes V consecutive outputs with the same arithmetic, in the same
// order, as the kernels above.
constexpr int ROW_V = 4;                          // outputs per thread
constexpr int ROW_SEG = THREADS * ROW_V;          // outputs per workgroup

struct RowArgs1d {
    const float *X;
    const float *w;
    const float *bias;
    float *Y;
    int64_t XE;              // elements of X
    int C, H, W, mult, Cout, Ho, Wo, sh, pt, pl;
    int segs;                // segments per output row
    int span;                // input elements a full segment reads
    FastDiv div_segs, div_ho, div_cout, div_mult;
};

template <int KW, int S, int EXACT>
__global__ __launch_bounds__(THREADS) void dw_row1d_kernel(RowArgs1d a)
{
#pragma clang fp contract(off)
    extern __shared__ __align__(16) float lds[];
    const int tid = threadIdx.x;
    // Output row (n, oc, oy) and segment.
    const uint32_t bid = (uint32_t)with_args_loaded((int)blockIdx.x, a);
    const uint32_t row = fdiv(bid, a.div_segs);
    const int seg = (int)(bid - row * (uint32_t)a.segs);
    const uint32_t plane = fdiv(row, a.div_ho);            // n * Cout + oc
    const int oy = (int)(row - plane * (uint32_t)a.Ho);
    const uint32_t n = fdiv(plane, a.div_cout);
    const int oc = (int)(plane - n * (uint32_t)a.Cout);
    const int ic = (int)fdiv((uint32_t)oc, a.div_mult);
    const int iy = oy * a.sh - a.pt;                         // the input row (KH = 1)
    const bool row_in = iy >= 0 && iy < a.H;
    const int ox0 = seg * ROW_SEG;
    const int c0 = ox0 * S - a.pl;                           // input column of LDS element 0

    float wv[KW];
#pragma unroll
    for (int k = 0; k < KW; ++k)
        wv[k] = a.w[(int64_t)oc * KW + k];

    // Input span into LDS: element e is column c0 + e of input row iy, or
    // +0 outside the row (the padding the definition multiplies).
    const int64_t rbase = (((int64_t)n * a.C + ic) * a.H + (row_in ? iy : 0)) * a.W;
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float *>(a.X + rbase), 0, a.W * 4, BUF_WORD3);
    constexpr int LOADS = (ROW_SEG * S + KW + THREADS - 1) / THREADS;
    float v[LOADS];
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
        const int e = tid + u * THREADS;
        const int col = c0 + e;
        const bool ok = row_in && e < a.span && col >= 0 && col < a.W;
        v[u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(xr, ok ? (uint32_t)col * 4 : OOB, 0, 0));
    }
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
        const int e = tid + u * THREADS;
        if (e < a.span)
            lds[e] = v[u];
    }
    __syncthreads();

    const float bv = a.bias ? a.bias[oc] : 0.0f;
    float *yrow = a.Y + (int64_t)row * a.Wo;
#pragma unroll
    for (int q = 0; q < ROW_V; ++q) {
        const int j = tid * ROW_V + q;                       // output within the segment
        const int ox = ox0 + j;
        if (ox < a.Wo) {
            float acc = +0.0f;
#pragma unroll
            for (int kx = 0; kx < KW; ++kx) {
                const float xv = lds[j * S + kx];
                if constexpr (EXACT) {
                    const float prod = wv[kx] * xv;
                    acc = acc + prod;
                } else {
                    acc = __builtin_fmaf(wv[kx], xv, acc);
                }
            }
            if (a.bias)
                acc = acc + bv;
            if (EXACT && __builtin_isnan(acc))
                acc = __uint_as_float(0x7FC00000u);
            yrow[ox] = acc;
        }
    }
}

// --- host side -------------------------------------------------------------

struct TilePlan {
    int RT, PPW, bands, RB, TPP;
    int64_t tile_elems;  // the input range (with slack), a multiple of 4
    int64_t lds_elems;   // tile and weights
    double util;        // fraction of thread-row slots that hold an output
    double score;       // util, discounted when the grid is too small to hide latency
};

// Waves (three per SIMD of the 1024) below which a launch cannot keep enough
// loads in flight or overlap one wave's arithmetic with another's waiting.
constexpr double WAVES_WANTED = 3.0 * 1024;

// Tile shape for rows-per-thread RT: whole planes when a plane's outputs fit
// one workgroup, else bands of rows of one plane. A constant of the shape.
TilePlan plan_for(const DwProblem &p, int RT)
{
    TilePlan t{};
    t.RT = RT;
    const int S = p.sh;
    const int groups_full = (p.Ho + RT - 1) / RT;
    if ((int64_t)groups_full * p.Wo <= THREADS) {
        t.TPP = groups_full * p.Wo;
        t.PPW = THREADS / t.TPP;
        t.bands = 1;
        t.RB = groups_full * RT;
    } else {
        const int gr = THREADS / p.Wo;
        t.TPP = gr * p.Wo;
        t.PPW = 1;
        t.RB = gr * RT;
        t.bands = (p.Ho + t.RB - 1) / t.RB;
    }
    const int64_t HW = (int64_t)p.H * p.W;
    auto tile_for = [&](int ppw) {
        // q0/mult .. (q0+ppw-1)/mult: at most ceil((ppw-1)/mult) plane steps.
        const int64_t plane_steps = (ppw - 1 + p.mult - 1) / p.mult;
        const int64_t rows = std::min<int64_t>(p.H, (int64_t)(t.RB - 1) * S + p.KH);
        const int64_t elems = plane_steps * HW + rows * p.W + 8 + 2 * SLACK;
        return ((elems + 3) / 4) * 4;
    };
    auto lds_for = [&](int ppw) { return tile_for(ppw) + (((int64_t)ppw * p.KH * p.KW + 3) / 4) * 4; };
    while (t.PPW > 1 && lds_for(t.PPW) * 4 > LDS_LIMIT)
        --t.PPW;
    t.tile_elems = tile_for(t.PPW);
    t.lds_elems = lds_for(t.PPW);
    const int64_t planes = (int64_t)p.N * p.C * p.mult;
    const int64_t tiles = (planes + t.PPW - 1) / t.PPW * t.bands;
    const double slots = (double)tiles * THREADS * RT;
    t.util = (double)planes * p.Ho * p.Wo / slots;
    const double waves = (double)tiles * THREADS / 64;
    t.score = t.util * (waves < WAVES_WANTED ? waves / WAVES_WANTED : 1.0);
    return t;
}

// The row kernel takes filters one row tall with 3, 4 or 5 taps, unit
// dilation and a stride of 1 or 2 along the width.
bool row1d_takes(const DwProblem &p)
{
    if (p.KH != 1 || (p.KW != 3 && p.KW != 4 && p.KW != 5) || p.dw != 1 || (p.sw != 1 && p.sw != 2))
        return false;
    const int64_t rows = (int64_t)p.N * p.C * p.mult * p.Ho;
    const int64_t segs = (p.Wo + ROW_SEG - 1) / ROW_SEG;
    return rows * segs < (int64_t(1) << 31) && (int64_t)p.N * p.C * p.H * p.W < (int64_t(1) << 40) &&
           p.W < (1 << 29);
}

template <int KW, int S>
hipError_t launch_row1d_k(const RowArgs1d &a, unsigned grid, size_t lds, bool exact, hipStream_t s)
{
    if (exact)
        hipLaunchKernelGGL((dw_row1d_kernel<KW, S, 1>), dim3(grid), dim3(THREADS), lds, s, a);
    else
        hipLaunchKernelGGL((dw_row1d_kernel<KW, S, 0>), dim3(grid), dim3(THREADS), lds, s, a);
    return hipGetLastError();
}

hipError_t launch_row1d(const DwProblem &p, hipStream_t s)
{
    RowArgs1d a;
    a.X = p.X;
    a.w = p.w;
    a.bias = p.bias;
    a.Y = p.Y;
    a.XE = (int64_t)p.N * p.C * p.H * p.W;
    a.C = p.C;
    a.H = p.H;
    a.W = p.W;
    a.mult = p.mult;
    a.Cout = p.C * p.mult;
    a.Ho = p.Ho;
    a.Wo = p.Wo;
    a.sh = p.sh;
    a.pt = p.ph;
    a.pl = p.pw;
    a.segs = (p.Wo + ROW_SEG - 1) / ROW_SEG;
    a.span = (ROW_SEG - 1) * p.sw + p.KW;
    a.div_segs = make_fastdiv((uint32_t)a.segs);
    a.div_ho = make_fastdiv((uint32_t)p.Ho);
    a.div_cout = make_fastdiv((uint32_t)a.Cout);
    a.div_mult = make_fastdiv((uint32_t)p.mult);
    const int64_t grid = (int64_t)p.N * a.Cout * p.Ho * a.segs;
    const size_t lds = (size_t)a.span * 4;
    const bool exact = p.mode == CONV_DW_EXACT;
    const bool s2 = p.sw == 2;
    switch (p.KW) {
    case 3: return s2 ? launch_row1d_k<3, 2>(a, (unsigned)grid, lds, exact, s) : launch_row1d_k<3, 1>(a, (unsigned)grid, lds, exact, s);
    case 4: return s2 ? launch_row1d_k<4, 2>(a, (unsigned)grid, lds, exact, s) : launch_row1d_k<4, 1>(a, (unsigned)grid, lds, exact, s);
    default: return s2 ? launch_row1d_k<5, 2>(a, (unsigned)grid, lds, exact, s) : launch_row1d_k<5, 1>(a, (unsigned)grid, lds, exact, s);
    }
}

bool plan(const DwProblem &p, TilePlan &out)
{
    if (!((p.KH == 3 && p.KW == 3) || (p.KH == 5 && p.KW == 5)))
        return false;
    if (p.sh != p.sw || (p.sh != 1 && p.sh != 2) || p.dh != 1 || p.dw != 1)
        return false;
    if (p.ph > MAX_PAD || p.pw > MAX_PAD || p.ph >= p.KH || p.pw >= p.KW || p.pb >= p.KH || p.pr >= p.KW ||
        p.Wo > THREADS)
        return false;       // every output window must overlap the input
    if (p.sh == 2 && (p.W % 2) != 0)
        return false;       // phase planes need even rows
    const int64_t XE = (int64_t)p.N * p.C * p.H * p.W;
    const int64_t planes = (int64_t)p.N * p.C * p.mult;
    if (XE % 4 != 0 || (reinterpret_cast<uintptr_t>(p.X) & 15) != 0)
        return false;       // 16-byte chunks must tile X exactly
    if (planes >= (1ll << 31) - THREADS || planes * p.Ho * p.Wo >= (1ll << 40) ||
        (int64_t)p.Ho * p.Wo >= (1ll << 31) || (int64_t)p.C * p.mult * p.KH * p.KW * 4 >= (1ll << 31))
        return false;
    bool have = false;
    // Rows per thread: more rows reuse each LDS value for more outputs,
    // fewer rows give more waves. Take the best score; on a tie, more rows.
    for (int RT : {2, 4, 7}) {
        TilePlan t = plan_for(p, RT);
        if (t.lds_elems * 4 > LDS_LIMIT)
            continue;
        if (!have || t.score > out.score + 1e-9 || (t.score > out.score - 1e-9 && RT > out.RT)) {
            out = t;
            have = true;
        }
    }
    if (have) {
        const int64_t tiles = (planes + out.PPW - 1) / out.PPW * out.bands;
        if (tiles >= (1ll << 31))
            return false;
    }
    return have;
}

template <int KH, int KW, int S, int RT>
hipError_t launch_rt(const TileArgs &a, unsigned grid, size_t lds, bool exact, hipStream_t s)
{
    if (exact)
        hipLaunchKernelGGL((dw_tiled_kernel<KH, KW, S, RT, 1>), dim3(grid), dim3(THREADS), lds, s, a);
    else
        hipLaunchKernelGGL((dw_tiled_kernel<KH, KW, S, RT, 0>), dim3(grid), dim3(THREADS), lds, s, a);
    return hipGetLastError();
}

template <int KH, int KW, int S>
hipError_t launch_s(const TileArgs &a, int RT, unsigned grid, size_t lds, bool exact, hipStream_t s)
{
    switch (RT) {
    case 2: return launch_rt<KH, KW, S, 2>(a, grid, lds, exact, s);
    case 4: return launch_rt<KH, KW, S, 4>(a, grid, lds, exact, s);
    default: return launch_rt<KH, KW, S, 7>(a, grid, lds, exact, s);
    }
}

template <int KH, int KW>
hipError_t launch_k(const TileArgs &a, int S, int RT, unsigned grid, size_t lds, bool exact, hipStream_t s)
{
    return S == 1 ? launch_s<KH, KW, 1>(a, RT, grid, lds, exact, s) : launch_s<KH, KW, 2>(a, RT, grid, lds, exact, s);
}

}  // namespace

bool dw_tiled_supports(const DwProblem &p)
{
    TilePlan t;
    return row1d_takes(p) || dw_waves_supports(p) || dw_pad_supports(p) || dw_rows_supports(p) || dw_planes_supports(p) || plan(p, t);
}

hipError_t launch_dw_tiled(const DwProblem &p, hipStream_t s)
{
    if (row1d_takes(p))
        return launch_row1d(p, s);
    // Stride-2 windows on rows of at most 64 outputs: one task per wave, no
    // workgroup barrier (depthwise_waves.hip).
    if (dw_waves_supports(p))
        return launch_dw_waves(p, s);
    // Windows with the zero border in LDS (depthwise_pad.hip) when it fits.
    if (dw_pad_supports(p))
        return launch_dw_pad(p, s);
    // 7- and 14-wide planes with "same" padding, a row per thread
    // (depthwise_rows.hip).
    if (dw_rows_supports(p))
        return launch_dw_rows(p, s);
    // Other small planes with the zero border in LDS (depthwise_planes.hip).
    if (dw_planes_supports(p))
        return launch_dw_planes(p, s);
    TilePlan t;
    if (!plan(p, t))
        return hipErrorNotSupported;
    TileArgs a;
    a.X = p.X;
    a.w = p.w;
    a.bias = p.bias;
    a.Y = p.Y;
    a.XE = (int64_t)p.N * p.C * p.H * p.W;
    a.HW = (int64_t)p.H * p.W;
    a.H = p.H;
    a.W = p.W;
    a.Cout = p.C * p.mult;
    a.Ho = p.Ho;
    a.Wo = p.Wo;
    a.ph = p.ph;
    a.pw = p.pw;
    a.planes = p.N * p.C * p.mult;
    a.PPW = t.PPW;
    a.bands = t.bands;
    a.RB = t.RB;
    a.TPP = t.TPP;
    // Phase planes: half of the tile range each (the range is a multiple of 4).
    a.half = (int)(t.tile_elems / 2);
    a.wofs = (int)t.tile_elems;
    a.HoWo = p.Ho * p.Wo;
    a.div_cout = make_fastdiv((uint32_t)a.Cout);
    a.div_bands = make_fastdiv((uint32_t)t.bands);
    a.div_tpp = make_fastdiv((uint32_t)t.TPP);
    a.div_wo = make_fastdiv((uint32_t)p.Wo);
    a.div_mult = make_fastdiv((uint32_t)p.mult);
    const int64_t tiles = ((int64_t)a.planes + t.PPW - 1) / t.PPW * t.bands;
    const size_t lds = (size_t)t.lds_elems * 4;
    const bool exact = p.mode == CONV_DW_EXACT;
    if (p.KH == 3)
        return launch_k<3, 3>(a, p.sh, t.RT, (unsigned)tiles, lds, exact, s);
    return launch_k<5, 5>(a, p.sh, t.RT, (unsigned)tiles, lds, exact, s);
}

}  // namespace convfwd
