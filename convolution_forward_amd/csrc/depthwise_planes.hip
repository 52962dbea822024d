// Depthwise convolution of small planes (whole planes per workgroup) with the
// zero border held in LDS.
//
// "Depthwise convolution" (onemodel docs), sections "What each output is"
// and "Layout of the work": output plane q = (n, oc) reads input plane
// q / multiplier; the sum starts at +0 and takes the taps row by row; a tap
// outside the input multiplies a real +0; exact mode rounds each product and
// then each sum, fast mode fuses them; the bias is one more rounded addition
// and exact mode rewrites a NaN result to 0x7FC00000. The arithmetic and its
// order are those of the direct kernel, so the bits are the same.
//
// The late layers of the mobile networks the page measures have planes of
// 7x7 or 14x14: a workgroup takes PPW whole output planes. On such planes
// almost every thread's window touches the border, and a kernel that keeps
// the planes packed in LDS (the tiled kernel) spends more vector
// instructions on replacing border taps with +0 and clamping rows than on
// the multiply-adds. Here every input plane of the tile sits in LDS inside
// its zero border, one padded row of WP words per input row:
//  * The workgroup zeroes the padded planes, then writes each input element
//    to its place. The tile's input planes are one contiguous range of X,
//    read in aligned 16-byte pieces (one position computed per piece, the
//    next three stepped from it) or, from an X that is not 16-byte aligned,
//    4 bytes per element.
//  * Stride 2: a padded row holds its even columns in its first half and its
//    odd columns in its second half (the page's phase planes), so tap
//    (ky, kx) of neighbouring output columns still reads neighbouring words.
//  * A thread owns one output column of RT consecutive rows of one plane.
//    Its taps are plain LDS reads at offsets fixed by (ky, kx): no test, no
//    select, no clamp. The plane pitch in LDS is padded so that the planes a
//    wave touches start on different banks.
//  * The thread's weights are loaded into registers behind the tile's loads.
//  * The tile's outputs are one contiguous range of Y. The threads leave
//    their sums in LDS and the workgroup writes the range with 16-byte
//    streaming stores.
#include <algorithm>

#include "common.h"
#include "dw_range_store.h"
#include "fastdiv.h"
#include "internal.h"

namespace convfwd {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int THREADS = 256;
constexpr int BATCH = 8;             // 4-byte loads in flight per thread per round
constexpr int BATCH4 = 4;            // 16-byte loads in flight per thread per round
constexpr uint32_t OOB = 0x80000000u;
constexpr int BUF_WORD3 = 0x00020000;
constexpr int LDS_LIMIT = 64 * 1024;
constexpr int BANKS = 64;

struct PlaneArgs {
    const float *X;
    const float *w;
    const float *bias;
    float *Y;
    int HW, H, W, Cout, Ho, Wo, HoWo, ph, pw;
    int planes;        // N * Cout output planes
    int PPW;           // output planes per workgroup
    int TPP;           // threads per plane: (row groups) * Wo
    int WP;            // LDS words per padded row
    int half;          // WP / 2: the odd columns' offset in a padded row (stride 2)
    int PS;            // LDS words per padded plane
    int zero_words;    // LDS words cleared before the copy (a multiple of 4)
    int y_aligned;     // Y starts on a 16-byte boundary
    int x_chunks;      // X is 16-byte aligned and a whole number of 16-byte pieces
    FastDiv div_tpp, div_wo, div_mult, div_cout, div_hw, div_w;
};

template <int KH, int KW, int S, int RT, int EXACT>
__global__ __launch_bounds__(THREADS) void dw_planes_kernel(PlaneArgs a)
{
#pragma clang fp contract(off)
    extern __shared__ __align__(16) float lds[];
    const int tid = threadIdx.x;
    constexpr int KK = KH * KW;

    // Output planes [q0, qend) read input planes [ip0, ip0 + nip).
    const int q0 = with_args_loaded((int)blockIdx.x, a) * a.PPW;
    const int qend = min(q0 + a.PPW, a.planes);
    const int ip0 = (int)fdiv((uint32_t)q0, a.div_mult);
    const int nip = (int)fdiv((uint32_t)(qend - 1), a.div_mult) - ip0 + 1;

    // The thread's task: plane p of the tile, output column ox, rows
    // oy0 .. oy0 + RT - 1.
    const int p = (int)fdiv((uint32_t)tid, a.div_tpp);
    const int rem = tid - p * a.TPP;
    const int g = (int)fdiv((uint32_t)rem, a.div_wo);
    const int ox = rem - g * a.Wo;
    const int q = q0 + p;
    const int oy0 = g * RT;
    const bool active = p < a.PPW && q < qend;
    const int qc = active ? q : q0;
    const int ip = (int)fdiv((uint32_t)qc, a.div_mult);
    const int occ = qc - (int)fdiv((uint32_t)qc, a.div_cout) * a.Cout;

    // Copy: element j of the tile's input planes is X[ip0 * HW + j].
    const int nelem = nip * a.HW;
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float *>(a.X + (int64_t)ip0 * a.HW), 0, nelem * 4, BUF_WORD3);
    float wv[KK];
#pragma unroll
    for (int k = 0; k < KK; ++k)
        wv[k] = 0.0f;
    float bv = 0.0f;
    // Behind the first loads: the weights and bias of the thread's plane,
    // and the zero border (the whole padded area).
    auto behind_first_loads = [&]() {
#pragma unroll
        for (int k = 0; k < KK; ++k)
            wv[k] = a.w[(int64_t)occ * KK + k];
        if (a.bias)
            bv = a.bias[occ];
        for (int e = tid * 4; e < a.zero_words; e += THREADS * 4)
            *reinterpret_cast<f32x4 *>(lds + e) = f32x4{0.f, 0.f, 0.f, 0.f};
        __syncthreads();
    };
    // Word of padded column pc within a padded row (stride 2: the even
    // columns, then the odd ones).
    auto col_of = [&](int pc) { return S == 1 ? pc : (pc & 1) * a.half + (pc >> 1); };
    if (a.x_chunks) {
        // Piece k holds elements 4k - lead .. 4k - lead + 3 of the tile; it
        // is 16-byte aligned because X is and X's length is a multiple of 4.
        const int lead = (int)(((int64_t)ip0 * a.HW) & 3);
        const int nch = (lead + nelem + 3) >> 2;
        const __amdgpu_buffer_rsrc_t cr = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float *>(a.X + ((int64_t)ip0 * a.HW - lead)), 0, nch * 16, BUF_WORD3);
        for (int base = 0; base < nch; base += THREADS * BATCH4) {
            f32x4 v[BATCH4];
#pragma unroll
            for (int u = 0; u < BATCH4; ++u) {
                const int k = base + u * THREADS + tid;
                if (base + u * THREADS < nch)
                    v[u] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                         cr, k < nch ? (uint32_t)k * 16 : OOB, 0, 0));
            }
            if (base == 0)
                behind_first_loads();
#pragma unroll
            for (int u = 0; u < BATCH4; ++u) {
                const int k = base + u * THREADS + tid;
                if (base + u * THREADS < nch && k < nch) {
                    // Position of the piece's first element inside the tile
                    // (the first piece may start before the tile).
                    const int j0 = 4 * k - lead;
                    const int js = max(j0, 0);
                    int pl = (int)fdiv((uint32_t)js, a.div_hw);
                    const int r0 = js - pl * a.HW;
                    int r = (int)fdiv((uint32_t)r0, a.div_w);
                    int c = r0 - r * a.W;
                    int row = pl * a.PS + (r + a.ph) * a.WP;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int j = j0 + i;
                        if (j >= 0 && j < nelem) {
                            lds[row + col_of(c + a.pw)] = v[u][i];
                            // Step to element j + 1.
                            ++c;
                            if (c == a.W) {
                                c = 0;
                                ++r;
                                row += a.WP;
                                if (r == a.H) {
                                    r = 0;
                                    row += a.PS - a.H * a.WP;
                                }
                            }
                        }
                    }
                }
            }
        }
    } else {
        for (int base = 0; base < nelem; base += THREADS * BATCH) {
            float v[BATCH];
#pragma unroll
            for (int u = 0; u < BATCH; ++u) {
                const int j = base + u * THREADS + tid;
                if (base + u * THREADS < nelem)
                    v[u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(xr, j < nelem ? (uint32_t)j * 4 : OOB, 0, 0));
            }
            if (base == 0)
                behind_first_loads();
#pragma unroll
            for (int u = 0; u < BATCH; ++u) {
                const int j = base + u * THREADS + tid;
                if (base + u * THREADS < nelem && j < nelem) {
                    const int pl = (int)fdiv((uint32_t)j, a.div_hw);
                    const int r0 = j - pl * a.HW;
                    const int r = (int)fdiv((uint32_t)r0, a.div_w);
                    lds[pl * a.PS + (r + a.ph) * a.WP + col_of(r0 - r * a.W + a.pw)] = v[u];
                }
            }
        }
    }
    __syncthreads();

    float acc[RT];
#pragma unroll
    for (int t = 0; t < RT; ++t)
        acc[t] = +0.0f;
    if (active) {
        // Tap (ky, kx) of output row oy0 + t: padded row (oy0 + t) * S + ky,
        // padded column ox * S + kx.
        const float *tb = lds + (ip - ip0) * a.PS + oy0 * S * a.WP + ox;
        constexpr int NIR = (RT - 1) * S + KH;     // input rows the thread's outputs read
#pragma unroll
        for (int ir = 0; ir < NIR; ++ir) {
            const float *rp = tb + ir * a.WP;
            float xv[KW];
#pragma unroll
            for (int kx = 0; kx < KW; ++kx)
                xv[kx] = S == 1 ? rp[kx] : rp[(kx & 1) * a.half + (kx >> 1)];
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
        }
    }

    // Outputs: Y elements [ostart, ostart + olen) through LDS. Element
    // ostart + j sits at LDS word lead + j (lead = ostart mod 4 when Y is
    // 16-byte aligned), so LDS words 4c..4c+3 are one aligned piece of Y.
    const int64_t ostart = (int64_t)q0 * a.HoWo;
    const int olen = (qend - q0) * a.HoWo;
    const int lead = a.y_aligned ? (int)(ostart & 3) : 0;
    __syncthreads();                                   // every tap read is done
    if (active) {
        float *op = lds + lead + p * a.HoWo + oy0 * a.Wo + ox;
#pragma unroll
        for (int t = 0; t < RT; ++t) {
            if (oy0 + t < a.Ho) {
                float r = acc[t];
                if (a.bias)
                    r = r + bv;
                if (EXACT && __builtin_isnan(r))
                    r = __uint_as_float(0x7FC00000u);
                op[t * a.Wo] = r;
            }
        }
    }
    __syncthreads();
    store_range_from_lds<THREADS, THREADS * RT + 3>(lds, a.Y, ostart, olen, lead, a.y_aligned, tid);
}

// --- host side -------------------------------------------------------------

struct PlanePlan {
    int RT, PPW, TPP, WP, PS;
    int64_t lds_words;
    double score;
};

// Waves (three per SIMD) below which a launch cannot keep enough loads in
// flight or overlap one wave's arithmetic with another's waiting.
constexpr double WAVES_WANTED = 3.0 * 1024;

// Whole planes per workgroup for rows-per-thread RT, or PPW = 0 if a plane's
// outputs do not fit one workgroup twice over.
PlanePlan plane_plan_for(const DwProblem &p, int RT)
{
    PlanePlan t{};
    t.RT = RT;
    const int groups = (p.Ho + RT - 1) / RT;
    t.TPP = groups * p.Wo;
    if (t.TPP * 2 > THREADS)
        return t;
    const int S = p.sh;
    // Padded rows: every data row, and every row a thread of the last group
    // reads (its rows past Ho are computed, never stored).
    const int HP = std::max(p.H + p.ph, (groups * RT - 1) * S + p.KH);
    t.WP = (p.W + p.pw + p.pr + 1) & ~1;
    t.PS = HP * t.WP;
    // Plane pitch = TPP (mod BANKS): the planes one wave touches then start
    // on consecutive runs of banks.
    t.PS += ((t.TPP - t.PS) % BANKS + BANKS) % BANKS;
    t.PPW = THREADS / t.TPP;
    auto words_for = [&](int ppw) {
        const int64_t nip = (ppw - 1 + p.mult - 1) / p.mult + 1;
        const int64_t in = ((nip * t.PS + 3) / 4) * 4;
        return std::max<int64_t>(in, (int64_t)THREADS * RT + 4);
    };
    while (t.PPW > 1 && words_for(t.PPW) * 4 > LDS_LIMIT)
        --t.PPW;
    if (t.PPW < 2 || words_for(t.PPW) * 4 > LDS_LIMIT) {
        t.PPW = 0;
        return t;
    }
    t.lds_words = words_for(t.PPW);
    const int64_t planes = (int64_t)p.N * p.C * p.mult;
    const int64_t tiles = (planes + t.PPW - 1) / t.PPW;
    const double util = (double)planes * p.Ho * p.Wo / ((double)tiles * THREADS * RT);
    const double waves = (double)tiles * THREADS / 64;
    t.score = util * (waves < WAVES_WANTED ? waves / WAVES_WANTED : 1.0);
    return t;
}

bool planes_plan(const DwProblem &p, PlanePlan &out)
{
    if (!((p.KH == 3 && p.KW == 3) || (p.KH == 5 && p.KW == 5)))
        return false;
    if (p.sh != p.sw || (p.sh != 1 && p.sh != 2) || p.dh != 1 || p.dw != 1)
        return false;
    if (p.ph >= p.KH || p.pw >= p.KW || p.pb >= p.KH || p.pr >= p.KW)
        return false;       // every output window overlaps the input
    const int64_t planes = (int64_t)p.N * p.C * p.mult;
    if (planes >= (1ll << 31) - THREADS || planes * p.Ho * p.Wo >= (1ll << 40) ||
        (int64_t)p.C * p.mult * p.KH * p.KW >= (1ll << 31) || (int64_t)p.H * p.W >= (1ll << 24) ||
        (int64_t)p.N * p.C * p.H * p.W >= (1ll << 40))
        return false;
    bool have = false;
    for (int RT : {2, 4, 7}) {
        PlanePlan t = plane_plan_for(p, RT);
        if (t.PPW == 0)
            continue;
        if (!have || t.score > out.score + 1e-9 || (t.score > out.score - 1e-9 && RT > out.RT)) {
            out = t;
            have = true;
        }
    }
    return have;
}

template <int KH, int KW, int S, int RT>
hipError_t launch_rt(const PlaneArgs &a, unsigned grid, size_t lds, bool exact, hipStream_t s)
{
    if (exact)
        hipLaunchKernelGGL((dw_planes_kernel<KH, KW, S, RT, 1>), dim3(grid), dim3(THREADS), lds, s, a);
    else
        hipLaunchKernelGGL((dw_planes_kernel<KH, KW, S, RT, 0>), dim3(grid), dim3(THREADS), lds, s, a);
    return hipGetLastError();
}

template <int KH, int KW, int S>
hipError_t launch_s(const PlaneArgs &a, int RT, unsigned grid, size_t lds, bool exact, hipStream_t s)
{
    switch (RT) {
    case 2: return launch_rt<KH, KW, S, 2>(a, grid, lds, exact, s);
    case 4: return launch_rt<KH, KW, S, 4>(a, grid, lds, exact, s);
    default: return launch_rt<KH, KW, S, 7>(a, grid, lds, exact, s);
    }
}

template <int KH, int KW>
hipError_t launch_k(const PlaneArgs &a, int S, int RT, unsigned grid, size_t lds, bool exact, hipStream_t s)
{
    return S == 1 ? launch_s<KH, KW, 1>(a, RT, grid, lds, exact, s) : launch_s<KH, KW, 2>(a, RT, grid, lds, exact, s);
}

}  // namespace

bool dw_planes_supports(const DwProblem &p)
{
    PlanePlan t;
    return planes_plan(p, t);
}

hipError_t launch_dw_planes(const DwProblem &p, hipStream_t s)
{
    PlanePlan t;
    if (!planes_plan(p, t))
        return hipErrorNotSupported;
    PlaneArgs a;
    a.X = p.X;
    a.w = p.w;
    a.bias = p.bias;
    a.Y = p.Y;
    a.HW = p.H * p.W;
    a.H = p.H;
    a.W = p.W;
    a.Cout = p.C * p.mult;
    a.Ho = p.Ho;
    a.Wo = p.Wo;
    a.HoWo = p.Ho * p.Wo;
    a.ph = p.ph;
    a.pw = p.pw;
    a.planes = p.N * p.C * p.mult;
    a.PPW = t.PPW;
    a.TPP = t.TPP;
    a.WP = t.WP;
    a.half = t.WP / 2;
    a.PS = t.PS;
    const int nip_max = (t.PPW - 1 + p.mult - 1) / p.mult + 1;
    a.zero_words = ((nip_max * t.PS + 3) / 4) * 4;
    a.y_aligned = (reinterpret_cast<uintptr_t>(p.Y) & 15) == 0;
    a.x_chunks = (reinterpret_cast<uintptr_t>(p.X) & 15) == 0 && ((int64_t)p.N * p.C * p.H * p.W) % 4 == 0;
    a.div_tpp = make_fastdiv((uint32_t)t.TPP);
    a.div_wo = make_fastdiv((uint32_t)p.Wo);
    a.div_mult = make_fastdiv((uint32_t)p.mult);
    a.div_cout = make_fastdiv((uint32_t)a.Cout);
    a.div_hw = make_fastdiv((uint32_t)a.HW);
    a.div_w = make_fastdiv((uint32_t)p.W);
    const int64_t tiles = ((int64_t)a.planes + t.PPW - 1) / t.PPW;
    const size_t lds = (size_t)t.lds_words * 4;
    const bool exact = p.mode == CONV_DW_EXACT;
    if (p.KH == 3)
        return launch_k<3, 3>(a, p.sh, t.RT, (unsigned)tiles, lds, exact, s);
    return launch_k<5, 5>(a, p.sh, t.RT, (unsigned)tiles, lds, exact, s);
}

}  // namespace convfwd
