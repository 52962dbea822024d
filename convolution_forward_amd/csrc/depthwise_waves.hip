// Depthwise convolution, stride 2, with one independent task per wave: each wave
// loads the padded input rows of its own band of output rows straight into
// its own LDS region (buffer loads that write LDS, zero border included),
// waits for its own loads only, and computes. No workgroup barrier: a wave
// starts its arithmetic as soon as its rows have landed, while other waves
// of the compute unit are still waiting for theirs, so the arithmetic of a
// layer overlaps its memory traffic instead of following it.
//
// "Depthwise convolution" (onemodel docs), sections "What each output is"
// and "Layout of the work": output plane q = (n, oc) reads input plane q
// (multiplier 1); the sum starts at +0 and takes the taps row by row; a tap
// outside the input multiplies a real +0; exact mode rounds each product and
// then each sum, fast mode fuses them; the bias is one more rounded addition
// and exact mode rewrites a NaN result to 0x7FC00000. The arithmetic and its
// order are those of the other depthwise kernels and of the oracle, bit for
// bit.
//
//  * Region layout: padded row r of a wave's region holds input row
//    r0*S - ph + r (r0: the wave's first output row); padded column PL + ix
//    holds input column ix (PL = 4), everything else is +0. A padded row is
//    WP = 4*UPR words; 16-byte unit u of the region is word 4u, so lane L of
//    load instruction i fills unit 64 i + L: the region is filled in whole
//    1 KB instructions, and units outside the image load zeros.
//  * Lanes: lane = g * Wo + ox owns output column ox of RT consecutive
//    output rows r0 + g*RT .. (G = 64 / Wo row groups per wave; lanes past
//    G * Wo compute row group 0 again and store nothing).
//  * Why. Per-workgroup timestamps of the padded-row kernel on the
//    72-channel 5x5 stride-2 exact layer showed every workgroup of a compute
//    unit waiting for its tile (1.1-3.1 us after it started), then all of
//    them computing at once (about 1 us each: exact mode's separate multiply
//    and add keep the vector units busy), then storing. Here each wave's
//    arithmetic starts when its own rows land: 5.92 -> 4.89 us on that layer,
//    bitwise equal.
#include <algorithm>

#include "common.h"
#include "fastdiv.h"
#include "internal.h"

namespace convfwd {
namespace {

constexpr int THREADS = 256;
constexpr int WAVES = THREADS / 64;
constexpr int PL = 4;
constexpr uint32_t OOB = 0x80000000u;
constexpr int BUF_WORD3 = 0x00020000;
constexpr int LDS_LIMIT = 64 * 1024;

struct WaveArgs {
    const float *X;
    const float *w;
    const float *bias;
    float *Y;
    int64_t HW;
    int C, H, W, Ho, Wo, ph, pw;
    int tasks;          // planes * bands
    int bands;          // wave tasks per plane
    int G;              // row groups per wave
    int UPR;            // 16-byte units per padded row
    int NRW;            // padded rows per region
    int NI;             // load instructions per wave
    int xcd_stride;     // grid / 8 to map workgroups to slots by XCD, else 0
    FastDiv div_bands, div_upr, div_wo, div_c;
};

template <int KH, int KW, int S, int RT, int EXACT>
__global__ __launch_bounds__(THREADS) void dw_waves_kernel(WaveArgs a)
{
#pragma clang fp contract(off)
    extern __shared__ __align__(16) float lds[];
    const int lane = threadIdx.x & 63;
    // Uniform across the wave (scalar registers: the buffer descriptor and
    // the LDS address of the loads must be).
    const int wave = with_args_loaded(__builtin_amdgcn_readfirstlane(threadIdx.x >> 6), a);
    // With xcd_stride = grid / 8, workgroup b (which runs on XCD b % 8:
    // workgroups are dealt to the 8 XCDs round robin) takes slot (b % 8) *
    // xcd_stride + b / 8, so consecutive slots, hence the bands of one plane
    // and the halo rows they share, meet in one XCD's L2. (The grid size
    // comes in the argument block rather than from the dispatch's hidden
    // arguments: a second, dependent argument load at the start of every
    // wave cost 0.35 us on the 72-channel layer.)
    const int b = (int)blockIdx.x;
    const int slot = a.xcd_stride ? (b & 7) * a.xcd_stride + (b >> 3) : b;
    const int task = slot * WAVES + wave;
    if (task >= a.tasks)
        return;                                     // the whole wave
    const int q = (int)fdiv((uint32_t)task, a.div_bands);
    const int band = task - q * a.bands;
    const int r0 = band * (a.G * RT);
    const int iy0 = r0 * S - a.ph;
    float *reg = lds + wave * (a.NI * 256);       // the wave's region

    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float *>(a.X + (int64_t)q * a.HW), 0, (int)(a.HW * 4), BUF_WORD3);
    // Unit u = 64 i + lane is padded row u / UPR, 16-byte column u % UPR;
    // both step by fixed amounts from one instruction to the next, so the
    // addresses take a few full-rate operations each (the loads go out
    // back to back).
    int row = (int)fdiv((uint32_t)lane, a.div_upr);
    int c4 = lane - row * a.UPR;
    const int q64 = (int)fdiv(64u, a.div_upr), r64 = 64 - q64 * a.UPR;
    for (int i = 0; i < a.NI; ++i) {
        const int iy = iy0 + row;
        const int ix = 4 * c4 - PL;
        const bool ok = (row < a.NRW) & ((unsigned)iy < (unsigned)a.H) & ((unsigned)ix < (unsigned)a.W);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            xr, (__attribute__((address_space(3))) void *)(reg + i * 256), 16,
            ok ? (uint32_t)(__mul24(iy, a.W) + ix) * 4u : OOB, 0, 0, 0);
        c4 += r64;
        row += q64;
        const bool wrap = c4 >= a.UPR;
        c4 -= wrap ? a.UPR : 0;
        row += wrap ? 1 : 0;
    }

    constexpr int KK = KH * KW;
    const int oc = q - (int)fdiv((uint32_t)q, a.div_c) * a.C;
    float wv[KK];
#pragma unroll
    for (int k = 0; k < KK; ++k)
        wv[k] = a.w[oc * KK + k];
    const float bv = a.bias ? a.bias[oc] : 0.0f;

    int g = (int)fdiv((uint32_t)lane, a.div_wo);
    const int ox = lane - g * a.Wo;
    const bool active = g < a.G;
    if (!active)
        g = 0;
    // The loads into LDS are outside the compiler's dependency tracking:
    // wait for all of this wave's loads before reading its region.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    const float *tb = reg + g * RT * S * (4 * a.UPR) + PL - a.pw + ox * S;
    const int WP = 4 * a.UPR;
    float acc[RT];
#pragma unroll
    for (int t = 0; t < RT; ++t)
        acc[t] = +0.0f;
    constexpr int NIR = (RT - 1) * S + KH;
#pragma unroll
    for (int ir = 0; ir < NIR; ++ir) {
        const float *rp = tb + ir * WP;
        float xv[KW];
#pragma unroll
        for (int kx = 0; kx < KW; ++kx)
            xv[kx] = rp[kx];
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
#pragma unroll
        for (int t = 0; t < RT; ++t)
            asm volatile("" : "+v"(acc[t]));
    }

    if (!active)
        return;
    float *yp = a.Y + (int64_t)q * a.Ho * a.Wo + ox;
#pragma unroll
    for (int t = 0; t < RT; ++t) {
        const int oy = r0 + g * RT + t;
        if (oy < a.Ho) {
            float r = acc[t];
            if (a.bias)
                r = r + bv;
            if (EXACT && __builtin_isnan(r))
                r = __uint_as_float(0x7FC00000u);
            __builtin_nontemporal_store(r, &yp[(int64_t)oy * a.Wo]);
        }
    }
}

struct WavePlan {
    int RT, G, bands, UPR, NRW, NI, region;
};

bool wave_plan_for(const DwProblem &p, int RT, WavePlan &t)
{
    t.RT = RT;
    t.G = 64 / p.Wo;
    const int RW = t.G * RT;
    t.bands = (p.Ho + RW - 1) / RW;
    const int cols = std::max(PL + p.W, PL - p.pw + (p.Wo - 1) * p.sw + p.KW);
    t.UPR = (cols + 3) / 4;
    t.NRW = (RW - 1) * p.sh + p.KH;
    t.NI = (t.NRW * t.UPR + 63) / 64;
    t.region = t.NI * 256;
    return (int64_t)t.region * 4 * WAVES <= LDS_LIMIT;
}

// Output rows per lane: two for 5x5 windows (the 72-channel exact layer:
// 4.89 us against 5.17 with one row and 5.55 with four), four for 3x3
// windows (the 64-channel stride-2 layer: 23.2 us with three or four, 23.8
// with two).
int rt_choice(const DwProblem &p) { return p.KH == 5 ? 2 : 4; }

bool wave_plan(const DwProblem &p, WavePlan &t)
{
    if (!((p.KH == 3 && p.KW == 3) || (p.KH == 5 && p.KW == 5)))
        return false;
    // Stride 2 only: at stride 1 the padded-row kernel (depthwise_pad.hip)
    // was faster on the 28-wide 5x5 layer (7.5 against 7.8 us).
    if (p.mult != 1 || p.sh != 2 || p.sw != 2 || p.dh != 1 || p.dw != 1)
        return false;
    if (p.pw > PL || p.Wo > 64 || p.W % 4 != 0 || (reinterpret_cast<uintptr_t>(p.X) & 15) != 0)
        return false;
    const int64_t planes = (int64_t)p.N * p.C;
    if ((int64_t)p.H * p.W * 4 >= (1ll << 31) || (int64_t)p.C * p.KH * p.KW >= (1ll << 31))
        return false;
    if (!wave_plan_for(p, rt_choice(p), t))
        return false;
    return planes * t.bands < (1ll << 31) - WAVES;
}

template <int KH, int KW, int S, int RT>
hipError_t launch_waves_rt(const WaveArgs &a, unsigned grid, size_t lds, bool exact, hipStream_t s)
{
    if (exact)
        hipLaunchKernelGGL((dw_waves_kernel<KH, KW, S, RT, 1>), dim3(grid), dim3(THREADS), lds, s, a);
    else
        hipLaunchKernelGGL((dw_waves_kernel<KH, KW, S, RT, 0>), dim3(grid), dim3(THREADS), lds, s, a);
    return hipGetLastError();
}

template <int KH, int KW, int S>
hipError_t launch_waves_s(const WaveArgs &a, int RT, unsigned grid, size_t lds, bool exact, hipStream_t s)
{
    switch (RT) {
    case 2: return launch_waves_rt<KH, KW, S, 2>(a, grid, lds, exact, s);
    default: return launch_waves_rt<KH, KW, S, 4>(a, grid, lds, exact, s);
    }
}

}  // namespace

bool dw_waves_supports(const DwProblem &p)
{
    WavePlan t;
    return wave_plan(p, t);
}

hipError_t launch_dw_waves(const DwProblem &p, hipStream_t s)
{
    WavePlan t;
    if (!wave_plan(p, t))
        return hipErrorNotSupported;
    WaveArgs a;
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
    a.bands = t.bands;
    a.tasks = (int)((int64_t)p.N * p.C * t.bands);
    a.G = t.G;
    a.UPR = t.UPR;
    a.NRW = t.NRW;
    a.NI = t.NI;
    a.div_bands = make_fastdiv((uint32_t)t.bands);
    a.div_upr = make_fastdiv((uint32_t)t.UPR);
    a.div_wo = make_fastdiv((uint32_t)p.Wo);
    a.div_c = make_fastdiv((uint32_t)p.C);
    // Small layers (every workgroup resident at once) keep each plane's bands
    // on one XCD: the 72-channel 5x5 exact layer reads 9 % fewer bytes from
    // HBM and takes 4.59 us instead of 4.89. Layers that run in many rounds
    // keep the plain order (the 64-channel 112-wide layer: 23.3 us plain,
    // 23.9 by XCD).
    const int64_t wgs = (a.tasks + WAVES - 1) / WAVES;
    const bool by_xcd = wgs <= 2048;
    const unsigned grid = (unsigned)(by_xcd ? (wgs + 7) / 8 * 8 : wgs);
    a.xcd_stride = by_xcd ? (int)(grid / 8) : 0;
    const size_t lds = (size_t)t.region * 4 * WAVES;
    const bool exact = p.mode == CONV_DW_EXACT;
    if (p.KH == 3)
        return launch_waves_s<3, 3, 2>(a, t.RT, grid, lds, exact, s);
    return launch_waves_s<5, 5, 2>(a, t.RT, grid, lds, exact, s);
}

}  // namespace convfwd
