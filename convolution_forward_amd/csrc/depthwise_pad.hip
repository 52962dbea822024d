// Depthwise convolution with the padding written into LDS: the tap loop is
// nothing but LDS reads at fixed offsets and the multiply-adds.
//
// "Depthwise convolution" (onemodel docs), sections "What each output is"
// and "Layout of the work": output plane q = (n, oc) reads input plane
// q / multiplier (here multiplier 1: plane q); the sum starts at +0 and
// takes the taps row by row; a tap outside the input multiplies a real +0;
// exact mode rounds each product and then each sum, fast mode fuses them;
// the bias is one more rounded addition and exact mode rewrites a NaN result
// to 0x7FC00000. The arithmetic and its order are those of the direct
// kernel and of the oracle, bit for bit; only the way the input reaches the
// arithmetic differs.
//
// Why a second tiled kernel. Timestamps of the LDS-tiled kernel
// (depthwise_tiled.hip) show each workgroup spending as long on its
// arithmetic as on its copy, with more than half of that arithmetic spent
// on clamping row indices, 64-bit addresses and per-tap selects that
// replace out-of-image values by +0. Here the tile is staged in LDS with
// its zero border already in place:
//  * A tile is PPW consecutive planes (whole planes) or a band of RB output
//    rows of one plane, as in the other kernel. Each plane of the tile gets
//    an LDS block of RP padded rows x WP columns; padded row r holds input
//    row iy_top + r, padded column PL + ix holds input column ix (PL = 4),
//    and every cell outside the image is +0.
//  * The block is zeroed while the tile's loads are in flight, then the
//    loaded rows are written over it in 16-byte pieces (rows are a multiple
//    of 4 elements long; narrower rows, whose planes are small, stay with
//    the other kernel, which loads them as one contiguous range).
//  * A thread owns output column ox of RT consecutive output rows of one
//    plane (neighbouring lanes, neighbouring columns). Tap (ky, kx) of
//    output row t reads padded row (t*S + ky) relative to the thread's
//    first row and padded column PL - pw + ox*S + kx: one address per input
//    row, taps at immediate offsets, no selects, no bounds checks.
#include <algorithm>

#include "common.h"
#include "fastdiv.h"
#include "internal.h"

namespace convfwd {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int THREADS = 256;
constexpr int PL = 4;                 // padded columns before the image (>= pw)
constexpr uint32_t OOB = 0x80000000u;
constexpr int BUF_WORD3 = 0x00020000;
constexpr int LDS_LIMIT = 64 * 1024;

struct PadArgs {
    const float *X;
    const float *w;
    const float *bias;
    float *Y;
    int64_t HW;        // elements per input plane
    int C, H, W, Ho, Wo, ph, pw;
    int planes;        // N * C output planes
    int PPW;           // planes per tile
    int bands;         // tiles per plane (1 when PPW > 1)
    int RB;            // output rows per band
    int TPP;           // threads per plane: (row groups) * Wo
    int WP;            // LDS pitch of a padded row (elements, multiple of 4)
    int RP;            // padded rows per plane block
    int PS;            // LDS elements per plane block
    int tile_elems;    // LDS elements zeroed per tile (whole blocks plus slack)
    int cpr;           // 16-byte copy pieces per input row (W / 4)
    FastDiv div_bands, div_tpp, div_wo, div_cpr, div_rows;  // div_rows: rows copied per whole plane
    FastDiv div_c;
};

// BATCH: 16-byte loads in flight per thread per copy round. Four cover
// every tile of up to 1024 pieces in one round; larger tiles take eight
// (fewer rounds) at the price of registers, i.e. of resident workgroups.
template <int KH, int KW, int S, int RT, int BATCH, int EXACT>
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(8))) void dw_pad_kernel(PadArgs a)
{
#pragma clang fp contract(off)
    extern __shared__ __align__(16) float lds[];
    const int tid = threadIdx.x;

    // Tile: output planes [q0, qend), output rows [oy_lo, oy_hi). Padded
    // row 0 of every block is input row iy_top.
    const uint32_t bid = (uint32_t)with_args_loaded((int)blockIdx.x, a);
    const uint32_t tile = fdiv(bid, a.div_bands);
    const int band = (int)(bid - tile * (uint32_t)a.bands);
    const int q0 = (int)tile * a.PPW;
    const int np = min(a.PPW, a.planes - q0);
    const int oy_lo = band * a.RB;
    const int oy_hi = min(a.Ho, oy_lo + a.RB);
    const int iy_top = oy_lo * S - a.ph;
    const int iy_first = max(0, iy_top);
    const int iy_last = min(a.H, iy_top + a.RP);               // one past the last row copied
    const int nr = iy_last - iy_first;                          // input rows copied per plane

    // The thread's task.
    const int p = (int)fdiv((uint32_t)tid, a.div_tpp);
    const int rem = tid - p * a.TPP;
    const int g = (int)fdiv((uint32_t)rem, a.div_wo);
    const int ox = rem - g * a.Wo;
    const int oy0 = oy_lo + g * RT;
    const bool active = p < np && oy0 < oy_hi;
    const int q = q0 + (active ? p : 0);
    const int oc = (int)(q - fdiv((uint32_t)q, a.div_c) * (uint32_t)a.C);
    constexpr int KK = KH * KW;
    // The weights of the tile's planes sit in LDS behind the tile: one
    // 4-byte load per weight, straight into LDS, issued behind the tile's
    // first loads. Held in registers from the start they kept 25 registers
    // busy through the copy (the 5x5 variants then did not fit 8 waves per
    // SIMD).
    float *wl = lds + a.tile_elems;

    // Copy: piece k of the tile is row k / cpr (of the np*nr rows, plane
    // major) and columns 4*(k % cpr) .. +3.
    const int64_t xbase = (int64_t)q0 * a.HW + (int64_t)iy_first * a.W;
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float *>(a.X + xbase), 0, (int)(((int64_t)(np - 1) * a.HW + (int64_t)nr * a.W) * 4), BUF_WORD3);
    const int npieces = np * nr * a.cpr;
    for (int base = 0; base < npieces; base += THREADS * BATCH) {
        u32x4 v[BATCH];
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            // Slots past the tile for the whole workgroup issue nothing.
            if (base + u * THREADS < npieces) {
                const int k = base + tid + u * THREADS;
                const int row = (int)fdiv((uint32_t)k, a.div_cpr);
                const int cx = k - row * a.cpr;
                const int pp = a.PPW > 1 ? (int)fdiv((uint32_t)row, a.div_rows) : 0;  // whole planes: nr is fixed
                const int rr = row - pp * nr;
                const uint32_t off = (uint32_t)(((int64_t)pp * a.HW + (int64_t)rr * a.W + cx * 4) * 4);
                v[u] = __builtin_amdgcn_raw_buffer_load_b128(xr, k < npieces ? off : OOB, 0, 0);
            }
        }
        if (base == 0) {
            // Weight e of the tile is tap e % KK of plane q0 + e / KK, whose
            // channel is the plane's index modulo C.
            const __amdgpu_buffer_rsrc_t wr =
                __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(a.w), 0, a.C * KK * 4, BUF_WORD3);
            const int nw = np * KK;
            for (int w0 = 0; w0 < nw; w0 += THREADS) {
                const int e = w0 + tid;
                const int pe = e / KK;
                const int qe = q0 + (e < nw ? pe : 0);
                const int ce = qe - (int)fdiv((uint32_t)qe, a.div_c) * a.C;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    wr, (__attribute__((address_space(3))) void *)(wl + w0 + (tid & ~63)), 4,
                    e < nw ? (uint32_t)((ce * KK + e - pe * KK) * 4) : OOB, 0, 0, 0);
            }
            // Zero the tile's blocks while the first loads are in flight.
            for (int e = tid * 4; e < a.tile_elems; e += THREADS * 4)
                *reinterpret_cast<f32x4 *>(lds + e) = f32x4{0.f, 0.f, 0.f, 0.f};
            __syncthreads();
        }
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            const int k = base + tid + u * THREADS;
            if (k < npieces) {
                const int row = (int)fdiv((uint32_t)k, a.div_cpr);
                const int cx = k - row * a.cpr;
                const int pp = a.PPW > 1 ? (int)fdiv((uint32_t)row, a.div_rows) : 0;
                const int rr = row - pp * nr;
                float *dst = lds + pp * a.PS + (iy_first - iy_top + rr) * a.WP + PL + cx * 4;
                *reinterpret_cast<u32x4 *>(dst) = v[u];
            }
        }
    }
    __syncthreads();
    if (!active)
        return;
    float wv[KK];
#pragma unroll
    for (int k = 0; k < KK; ++k)
        wv[k] = wl[p * KK + k];

    // Tap (ky, kx) of output row t: padded row g*RT*S + t*S + ky of block
    // p, padded column PL - pw + ox*S + kx.
    const float *tb = lds + p * a.PS + g * RT * S * a.WP + PL - a.pw + ox * S;
    float acc[RT];
#pragma unroll
    for (int t = 0; t < RT; ++t)
        acc[t] = +0.0f;
    constexpr int NIR = (RT - 1) * S + KH;     // input rows the thread's outputs read
#pragma unroll
    for (int ir = 0; ir < NIR; ++ir) {
        const float *rp = tb + ir * a.WP;
        float xv[KW];
#pragma unroll
        for (int kx = 0; kx < KW; ++kx)
            xv[kx] = rp[kx];
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
        // One input row at a time: the row's sums are pinned here, so its
        // inputs die before the next row is read. Left alone, the compiler
        // reads every row ahead of the arithmetic (88 registers for the 5x5
        // seven-row variant) and fewer workgroups fit a CU.
#pragma unroll
        for (int t = 0; t < RT; ++t)
            asm volatile("" : "+v"(acc[t]));
    }

    const float bv = a.bias ? a.bias[oc] : 0.0f;
    float *yp = a.Y + (int64_t)q * a.Ho * a.Wo + ox;
#pragma unroll
    for (int t = 0; t < RT; ++t) {
        const int oy = oy0 + t;
        if (oy < oy_hi) {
            float r = acc[t];
            if (a.bias)
                r = r + bv;
            if (EXACT && __builtin_isnan(r))
                r = __uint_as_float(0x7FC00000u);
            // Streaming (nt) stores: the 112-wide planes 3-5% faster; the
            // contiguous-range kernel's short rows are slower with them.
            __builtin_nontemporal_store(r, &yp[(int64_t)oy * a.Wo]);
        }
    }
}

// --- host side -------------------------------------------------------------

struct PadPlan {
    int RT, PPW, bands, RB, TPP, WP, RP, PS, tile_elems, batch;
    int64_t lds_bytes;  // the tile's blocks and the weights of its planes
    double score;
};

constexpr double WAVES_WANTED = 3.0 * 1024;

PadPlan pad_plan_for(const DwProblem &p, int RT)
{
    PadPlan t{};
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
    // Padded columns read: PL - pw .. PL - pw + (Wo-1)*S + KW - 1; the image
    // sits at PL .. PL + W - 1.
    const int cols = std::max(PL + p.W, PL - p.pw + (p.Wo - 1) * S + p.KW);
    t.WP = (cols + 3) / 4 * 4;
    // Rows a thread reads: its RT outputs, rounded up to whole row groups
    // (the last group may run past the band; those outputs are not stored).
    t.RP = (t.RB - 1) * S + p.KH;
    t.PS = t.RP * t.WP;
    const int KK = p.KH * p.KW;
    auto tile_for = [&](int ppw) { return ((int64_t)ppw * t.PS + 4 + 3) / 4 * 4; };
    auto lds_for = [&](int ppw) { return (tile_for(ppw) + ((int64_t)ppw * KK + THREADS - 1) / THREADS * THREADS) * 4; };
    while (t.PPW > 1 && lds_for(t.PPW) > LDS_LIMIT)
        --t.PPW;
    t.tile_elems = (int)tile_for(t.PPW);
    t.lds_bytes = lds_for(t.PPW);
    // 16-byte pieces of the largest tile: its planes, or its band's rows.
    const int64_t rows = t.PPW > 1 ? std::min<int64_t>(p.H, t.RP - p.ph) : std::min<int64_t>(p.H, t.RP);
    t.batch = (int64_t)t.PPW * rows * (p.W / 4) <= 4 * THREADS ? 4 : 8;
    const int64_t planes = (int64_t)p.N * p.C;
    const int64_t tiles = (planes + t.PPW - 1) / t.PPW * t.bands;
    const double slots = (double)tiles * THREADS * RT;
    const double util = (double)planes * p.Ho * p.Wo / slots;
    const double waves = (double)tiles * THREADS / 64;
    t.score = util * (waves < WAVES_WANTED ? waves / WAVES_WANTED : 1.0);
    return t;
}

bool pad_plan(const DwProblem &p, PadPlan &out)
{
    if (!((p.KH == 3 && p.KW == 3) || (p.KH == 5 && p.KW == 5)))
        return false;
    if (p.mult != 1 || p.sh != p.sw || (p.sh != 1 && p.sh != 2) || p.dh != 1 || p.dw != 1)
        return false;
    if (p.pw > PL || p.ph >= p.KH || p.pw >= p.KW || p.pb >= p.KH || p.pr >= p.KW || p.Wo > THREADS)
        return false;
    if ((reinterpret_cast<uintptr_t>(p.X) & 15) != 0 || p.W % 4 != 0)
        return false;
    const int64_t planes = (int64_t)p.N * p.C;
    if (planes >= (1ll << 31) - THREADS || planes * p.Ho * p.Wo >= (1ll << 40) || (int64_t)p.H * p.W >= (1ll << 28))
        return false;
    if ((int64_t)p.C * p.KH * p.KW * 4 >= (1ll << 31))
        return false;       // weight offsets are 32-bit
    bool have = false;
    for (int RT : {2, 4, 7}) {
        PadPlan t = pad_plan_for(p, RT);
        if (t.lds_bytes > LDS_LIMIT)
            continue;
        if ((int64_t)t.PPW * p.H * p.W * 4 >= (1ll << 31))
            continue;
        if (!have || t.score > out.score + 1e-9 || (t.score > out.score - 1e-9 && RT > out.RT)) {
            out = t;
            have = true;
        }
    }
    if (have && (planes + out.PPW - 1) / out.PPW * out.bands >= (1ll << 31))
        return false;
    return have;
}

template <int KH, int KW, int S, int RT, int BATCH>
hipError_t launch_pad_b(const PadArgs &a, unsigned grid, size_t lds, bool exact, hipStream_t s)
{
    if (exact)
        hipLaunchKernelGGL((dw_pad_kernel<KH, KW, S, RT, BATCH, 1>), dim3(grid), dim3(THREADS), lds, s, a);
    else
        hipLaunchKernelGGL((dw_pad_kernel<KH, KW, S, RT, BATCH, 0>), dim3(grid), dim3(THREADS), lds, s, a);
    return hipGetLastError();
}

template <int KH, int KW, int S, int RT>
hipError_t launch_pad_rt(const PadArgs &a, int batch, unsigned grid, size_t lds, bool exact, hipStream_t s)
{
    return batch == 4 ? launch_pad_b<KH, KW, S, RT, 4>(a, grid, lds, exact, s)
                      : launch_pad_b<KH, KW, S, RT, 8>(a, grid, lds, exact, s);
}

template <int KH, int KW, int S>
hipError_t launch_pad_s(const PadArgs &a, const PadPlan &t, unsigned grid, size_t lds, bool exact, hipStream_t s)
{
    switch (t.RT) {
    case 2: return launch_pad_rt<KH, KW, S, 2>(a, t.batch, grid, lds, exact, s);
    case 4: return launch_pad_rt<KH, KW, S, 4>(a, t.batch, grid, lds, exact, s);
    default: return launch_pad_rt<KH, KW, S, 7>(a, t.batch, grid, lds, exact, s);
    }
}

}  // namespace

bool dw_pad_supports(const DwProblem &p)
{
    PadPlan t;
    return pad_plan(p, t);
}

hipError_t launch_dw_pad(const DwProblem &p, hipStream_t s)
{
    PadPlan t;
    if (!pad_plan(p, t))
        return hipErrorNotSupported;
    PadArgs a;
    a.X = p.X;
    a.w = p.w;
    a.bias = p.bias;
    a.Y = p.Y;
    a.HW = (int64_t)p.H * p.W;
    a.C = p.C;
    a.H = p.H;
    a.W = p.W;
    a.Ho = p.Ho;
    a.Wo = p.Wo;
    a.ph = p.ph;
    a.pw = p.pw;
    a.planes = p.N * p.C;
    a.PPW = t.PPW;
    a.bands = t.bands;
    a.RB = t.RB;
    a.TPP = t.TPP;
    a.WP = t.WP;
    a.RP = t.RP;
    a.PS = t.PS;
    a.tile_elems = t.tile_elems;
    a.cpr = p.W / 4;
    a.div_bands = make_fastdiv((uint32_t)t.bands);
    a.div_tpp = make_fastdiv((uint32_t)t.TPP);
    a.div_wo = make_fastdiv((uint32_t)p.Wo);
    a.div_cpr = make_fastdiv((uint32_t)a.cpr);
    a.div_c = make_fastdiv((uint32_t)p.C);
    // Whole-plane tiles start at input row -ph: every tile copies the same
    // rows, min(H, RP - ph) of them.
    a.div_rows = make_fastdiv((uint32_t)std::max(1, std::min(p.H, t.RP - p.ph)));
    const int64_t tiles = ((int64_t)a.planes + t.PPW - 1) / t.PPW * t.bands;
    const size_t lds = (size_t)t.lds_bytes;
    const bool exact = p.mode == CONV_DW_EXACT;
    if (p.KH == 3)
        return p.sh == 1 ? launch_pad_s<3, 3, 1>(a, t, (unsigned)tiles, lds, exact, s)
                         : launch_pad_s<3, 3, 2>(a, t, (unsigned)tiles, lds, exact, s);
    return p.sh == 1 ? launch_pad_s<5, 5, 1>(a, t, (unsigned)tiles, lds, exact, s)
                     : launch_pad_s<5, 5, 2>(a, t, (unsigned)tiles, lds, exact, s);
}

}  // namespace convfwd
