// Dense NHWC cross-correlation with fp32 operands on CDNA4 matrix cores.
//
// Contract: "CMU DLSys Lecture 14: Convolutional Network Implementation",
// section 1 (Y[n,y,x,o] = sum over i,j,c of X[n,y+i,x+j,c] * F[i,j,c,o]), the
// implicit form of the patch-matrix product of section 5 (no patch matrix is
// ever built: patch fragments are LDS reads at per-tap offsets).
//
// The organisation follows the bf16 kernel (dense_mfma.hip): a workgroup of
// 512 threads owns a band of output rows of one image and 64 output
// channels, walks its input rows top to bottom through two LDS row buffers
// with the next rows' loads in flight, and lets each X fragment feed every
// output row that uses it. What changes with fp32 operands:
//  * The instruction is v_mfma_f32_16x16x4_f32: 4 channels per step, one
//    fp32 value per lane per operand. A lane reads 4 consecutive channels of
//    one pixel (16 bytes) and feeds them to 4 consecutive MFMAs, so a
//    16-channel step is 4 MFMAs with k-group g = lane / 16 covering channels
//    4g..4g+3 of the step (the k order is permuted the same way on both
//    operands, which leaves the sum unchanged).
//  * The filter fragments (4 values per 16-channel step and lane) are loaded
//    straight from global memory: lane (g, r) of wave w needs
//    F[tap][c0 + 4g + s][o0 + 16*(w % 4) + r], and the 16 lanes of a group
//    read 64 contiguous bytes. No LDS staging is needed.
//  * Wave w owns the 16-channel column block w % 4 and the pixel-block
//    group w / 4 (blocks g and g + 2 of the row: rows are at most 64 pixels).
//  * fp32 MFMA is the bottleneck (1/16 of the bf16 rate), so every output
//    block keeps enough partial sums in flight for 4 independent
//    accumulation chains per wave; the partials are added in a fixed order.
//
// LDS pixel pitch is Cin_padded + 8 floats (32 bytes of padding, the pitch
// class that keeps 16-byte reads of 16 consecutive pixels conflict-free).
// All global accesses are raw buffer operations; out-of-range offsets are
// dropped (loads return zeros).
#include <type_traits>

#include "common.h"
#include "internal.h"

namespace convfwd {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int THREADS = 512;
constexpr int COUT_TILE = 64;      // 4 column blocks of 16 output channels
constexpr int LDS_BYTES_MAX = 160 * 1024;
constexpr uint32_t OOB = 0x80000000u;           // buffer offset beyond every range: access dropped
constexpr int BUF_WORD3 = 0x00020000;           // raw buffer descriptor word 3 (gfx9 family)

struct RowArgsF {
    const float *X;
    const float *F;
    const float *bias;
    float *Y;
    int64_t xs0, xs1, xs2, ys0, ys1, ys2;
    int H, W, Cin, Cout, Ho, Wo;
    int R;              // output rows per band
    int bands_per_img;
    int bands;          // N * bands_per_img (the grid may hold more: those exit)
    int tiles;          // 64-channel output tiles
    int row_elems;      // LDS floats per staged input row (W * pitch)
    int chunks_per_row; // 16-byte chunks per input row (W * Cin_padded / 4)
    int otile_off;      // LDS byte offset of the output tiles
    uint32_t x_records; // bytes addressable from one image's base in X
    uint32_t y_records; // bytes addressable from one image's base in Y
};

// Byte offset of 16-byte chunk q (pixel q / CG, channels 4*(q % CG)..+3) of
// input row r, or OOB for padding channels and rows outside the band.
template <int CINP>
__device__ __forceinline__ uint32_t chunk_off_f32(const RowArgsF &a, int r, int q, int rows_end)
{
    constexpr int CG = CINP / 4;
    const int px = q / CG;
    const int cg = q - px * CG;
    const bool ok = q < a.chunks_per_row && r < rows_end && cg * 4 < a.Cin;
    return ok ? (uint32_t)(((int64_t)r * a.xs1 + (int64_t)px * a.xs2 + cg * 4) * 4) : OOB;
}

template <int CINP>
__device__ __forceinline__ void put_chunk_f32(float *lds_row, int q, u32x4 v)
{
    constexpr int CG = CINP / 4;
    constexpr int PITCH = CINP + 8;
    const int px = q / CG;
    const int cg = q - px * CG;
    *reinterpret_cast<u32x4 *>(lds_row + px * PITCH + cg * 4) = v;
}

template <int U, int N, class Fn>
__device__ __forceinline__ void static_for_f32(Fn &&fn)
{
    if constexpr (U < N) {
        fn(std::integral_constant<int, U>{});
        static_for_f32<U + 1, N>(fn);
    }
}

template <int KH, int KW, int CS, int BPW, int MAXC, int NR>
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
void dense_rows_mfma_f32(RowArgsF a)
{
    constexpr int CINP = 16 * CS;
    constexpr int PITCH = CINP + 8;
    constexpr int KSTEPS = KH * KW * CS;
    // Output tile: one row of results (32 pixels per block slot x 64
    // channels), double buffered, pitch 32 mod 64 bytes.
    constexpr int OPITCH = COUT_TILE * 4 + 32;
    constexpr int OTILE_BYTES = 32 * BPW * OPITCH;
    constexpr int OCH = COUT_TILE * 4 / 16;                           // 16-byte chunks per pixel
    constexpr int OSTORE = (32 * BPW * OCH + THREADS - 1) / THREADS;  // store instructions per row
    // Partial sums per output block: at least 4 independent chains per wave.
    constexpr int CHAINS = KH * BPW >= 4 ? 1 : (4 + KH * BPW - 1) / (KH * BPW);

    extern __shared__ __align__(16) float smem[];
    float *rows = smem;
    uint8_t *otile = reinterpret_cast<uint8_t *>(smem) + a.otile_off;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int cb = wave & 3;            // 16-channel column block of the tile
    const int pg = wave >> 2;           // pixel-block group 0..1
    // Slot s runs on XCD s % 8; all tiles of a band and neighbouring bands
    // share an XCD (same map as the bf16 kernel).
    const int bid = with_args_loaded((int)blockIdx.x, a);
    const int slot_in_xcd = bid >> 3;
    const int band = (bid & 7) * (int)(gridDim.x >> 3) / a.tiles + slot_in_xcd / a.tiles;
    const int o0 = (slot_in_xcd % a.tiles) * COUT_TILE;
    if (band >= a.bands)
        return;
    const int n = band / a.bands_per_img;
    const int y0 = (band - n * a.bands_per_img) * a.R;
    if (y0 >= a.Ho)
        return;
    const int y1 = min(y0 + a.R, a.Ho);
    const int rows_end = y1 + KH - 1;

    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float *>(a.X + (int64_t)n * a.xs0), 0, (int)a.x_records, BUF_WORD3);
    const __amdgpu_buffer_rsrc_t yr = __builtin_amdgcn_make_buffer_rsrc(
        a.Y + (int64_t)n * a.ys0, 0, (int)a.y_records, BUF_WORD3);

    // 1. Filter fragments and bias. Lane (g = lane / 16, r = lane % 16) holds
    //    F[tap][cs*16 + 4g + s][o] for its output channel o and s = 0..3.
    const int g = lane >> 4;
    const int o = o0 + cb * 16 + (lane & 15);
    const __amdgpu_buffer_rsrc_t fr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float *>(a.F), 0, KH * KW * a.Cin * a.Cout * 4, BUF_WORD3);
    float wf[KSTEPS][4];
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
        const int tap = ks / CS;
        const int cs = ks % CS;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int c = cs * 16 + 4 * g + s;
            const bool ok = c < a.Cin && o < a.Cout;
            wf[ks][s] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                fr, ok ? (uint32_t)((((int64_t)tap * a.Cin + c) * a.Cout + o) * 4) : OOB, 0, 0));
        }
    }
    // Bias of the 4 output channels this lane's results belong to.
    const __amdgpu_buffer_rsrc_t br = __builtin_amdgcn_make_buffer_rsrc(
        a.bias ? (void *)a.bias : (void *)a.F, 0, a.bias ? a.Cout * 4 : 0, BUF_WORD3);
    const u32x4 bq = __builtin_amdgcn_raw_buffer_load_b128(br, (uint32_t)((o0 + cb * 16 + g * 4) * 4), 0, 0);

    // 2. The first D input rows of the band (the loop keeps D rows ahead).
    __builtin_amdgcn_sched_barrier(0);
    constexpr int DW = MAXC == 1 ? 4 : 2;
    constexpr int D = NR < DW ? NR : DW;
    u32x4 xin[D][MAXC];
#pragma unroll
    for (int i = 0; i < D; ++i)
#pragma unroll
        for (int k = 0; k < MAXC; ++k)
            xin[i][k] = __builtin_amdgcn_raw_buffer_load_b128(
                xr, chunk_off_f32<CINP>(a, y0 + i, tid + k * THREADS, rows_end), 0, 0);

    // 3. Input row 0 into LDS buffer 0.
#pragma unroll
    for (int k = 0; k < MAXC; ++k) {
        const int q = tid + k * THREADS;
        if (q < a.chunks_per_row)
            put_chunk_f32<CINP>(rows, q, xin[0][k]);
    }
    __syncthreads();

    auto store_row = [&](const int t) __attribute__((always_inline)) {
        const uint8_t *obuf = otile + (t & 1) * OTILE_BYTES;
        const int yo = y0 + t;
#pragma unroll
        for (int k = 0; k < OSTORE; ++k) {
            const int q = tid + k * THREADS;
            const int px = q / OCH;
            const int cc = q - px * OCH;
            const int ch = o0 + cc * 4;
            const bool ok = px < a.Wo && ch < a.Cout && yo < y1;
            const u32x4 v = *reinterpret_cast<const u32x4 *>(obuf + (px < 32 * BPW ? px : 0) * OPITCH + cc * 16);
            const uint32_t off = ok ? (uint32_t)(((int64_t)yo * a.ys1 + (int64_t)px * a.ys2 + ch) * 4) : OOB;
            __builtin_amdgcn_raw_buffer_store_b128(v, yr, off, 0, 18);   // sc1 | nt: drains faster (1x1 fp32: 66.2 -> 63.9 us)
        }
    };

    // 4. Slide down the band: input row r feeds output rows r - i (filter
    //    row i). Output row t accumulates in slot t % KH and is complete at
    //    step t + KH - 1; it leaves at step t + KH, after the barrier.
    f32x4 acc[KH][BPW][CHAINS];
#pragma unroll
    for (int s2 = 0; s2 < KH; ++s2)
#pragma unroll
        for (int qb = 0; qb < BPW; ++qb)
#pragma unroll
            for (int p = 0; p < CHAINS; ++p)
                acc[s2][qb][p] = f32x4{0.f, 0.f, 0.f, 0.f};

    static_for_f32<0, NR>([&](auto RR) {
        constexpr int r = decltype(RR)::value;
        if constexpr (r >= KH)
            store_row(r - KH);
        if constexpr (r + D < NR) {
#pragma unroll
            for (int k = 0; k < MAXC; ++k)
                xin[(r + D) % D][k] = __builtin_amdgcn_raw_buffer_load_b128(
                    xr, chunk_off_f32<CINP>(a, y0 + r + D, tid + k * THREADS, rows_end), 0, 0);
        }
        const float *rowp = rows + (r & 1) * a.row_elems;
#pragma unroll
        for (int qb = 0; qb < BPW; ++qb) {
            const int x = (pg + 2 * qb) * 16 + (lane & 15);
            const int xl = min(x, a.Wo - 1);
            f32x4 xb[KW * CS];
#pragma unroll
            for (int jc = 0; jc < KW * CS; ++jc) {
                const int j = jc / CS;
                const int cs = jc % CS;
                xb[jc] = *reinterpret_cast<const f32x4 *>(rowp + (xl + j) * PITCH + cs * 16 + g * 4);
            }
#pragma unroll
            for (int i = 0; i < KH; ++i) {
                const int t = r - i;
                if (t >= 0 && t <= NR - KH && y0 + t < y1) {
#pragma unroll
                    for (int jc = 0; jc < KW * CS; ++jc) {
                        const int ks = i * KW * CS + jc;
#pragma unroll
                        for (int s = 0; s < 4; ++s) {
                            const int p = (jc * 4 + s) % CHAINS;
                            acc[(t + KH) % KH][qb][p] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                                wf[ks][s], xb[jc][s], acc[(t + KH) % KH][qb][p], 0, 0, 0);
                        }
                    }
                }
            }
            if constexpr (r >= KH - 1) {
                // Output row t is complete: lane holds channels
                // 16*cb + 4*g + {0..3} of pixel x.
                constexpr int t = r - KH + 1;
                f32x4 v = acc[t % KH][qb][0];
#pragma unroll
                for (int p = 1; p < CHAINS; ++p)
                    v = v + acc[t % KH][qb][p];
                const f32x4 out = {v[0] + __uint_as_float(bq[0]), v[1] + __uint_as_float(bq[1]),
                                   v[2] + __uint_as_float(bq[2]), v[3] + __uint_as_float(bq[3])};
                *reinterpret_cast<f32x4 *>(otile + (t & 1) * OTILE_BYTES + x * OPITCH + (cb * 16 + g * 4) * 4) = out;
#pragma unroll
                for (int p = 0; p < CHAINS; ++p)
                    acc[t % KH][qb][p] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
        if constexpr (r + 1 < NR) {
#pragma unroll
            for (int k = 0; k < MAXC; ++k) {
                const int q = tid + k * THREADS;
                if (q < a.chunks_per_row)
                    put_chunk_f32<CINP>(rows + ((r + 1) & 1) * a.row_elems, q, xin[(r + 1) % D][k]);
            }
        }
        __syncthreads();
    });
    store_row(NR - KH);
}

// --- host side -------------------------------------------------------------

int cin_steps16(int Cin)
{
    const int cs = (Cin + 15) / 16;
    for (int c : {1, 2, 4, 8, 16})
        if (cs <= c)
            return c;
    return 0;
}

bool taps_instantiated_f32(int KH, int KW, int CS)
{
    if (KH == 1 && KW == 1)
        return CS == 1 || CS == 2 || CS == 4 || CS == 8 || CS == 16;
    if (KH == 3 && KW == 3)
        return CS == 1 || CS == 2 || CS == 4;
    return false;
}

constexpr int band_rows_f32(int KH) { return KH == 1 ? 25 : 9; }

struct PlanF {
    int CS, BPW, MAXC, NR, R;
    size_t otile_off, lds;
};

int64_t extent_f32(const int64_t *s, int rows, int cols, int ch)
{
    return ((int64_t)(rows - 1) * s[1] + (int64_t)(cols - 1) * s[2] + ch) * 4;
}

bool plan_rows_f32(const DenseProblem &p, PlanF *plan)
{
    if (p.xdt != CONV_F32 || p.ydt != CONV_F32 || p.Cin % 4 != 0 || p.Cout % 4 != 0)
        return false;
    if ((uintptr_t)p.X % 16 != 0 || p.xs[0] % 4 != 0 || p.xs[1] % 4 != 0 || p.xs[2] % 4 != 0)
        return false;
    if ((uintptr_t)p.Y % 16 != 0 || p.ys[0] % 4 != 0 || p.ys[1] % 4 != 0 || p.ys[2] % 4 != 0)
        return false;
    if ((uintptr_t)p.F % 4 != 0 || (int64_t)p.KH * p.KW * p.Cin * p.Cout * 4 >= (int64_t(1) << 31))
        return false;
    if (extent_f32(p.xs, p.H, p.W, p.Cin) >= (int64_t(1) << 31) ||
        extent_f32(p.ys, p.Ho, p.Wo, p.Cout) >= (int64_t(1) << 31))
        return false;
    PlanF pl;
    pl.CS = cin_steps16(p.Cin);
    if (pl.CS == 0 || !taps_instantiated_f32(p.KH, p.KW, pl.CS))
        return false;
    const int blocks = (p.Wo + 15) / 16;
    pl.BPW = (blocks + 1) / 2;
    if (pl.BPW > 2)
        return false;
    const int64_t chunks = (int64_t)p.W * 16 * pl.CS / 4;
    pl.MAXC = chunks <= THREADS ? 1 : chunks <= 2 * THREADS ? 2 : chunks <= 4 * THREADS ? 4 : 0;
    if (pl.MAXC == 0 || (p.KH == 3 && pl.CS == 4 && pl.MAXC == 4))
        return false;       // (that combination does not fit the register file)
    pl.NR = band_rows_f32(p.KH);
    const int rmax = pl.NR - p.KH + 1;
    const int tiles = (p.Cout + COUT_TILE - 1) / COUT_TILE;
    int want = (int)((256 + (int64_t)p.N * tiles - 1) / ((int64_t)p.N * tiles));
    want = want < 1 ? 1 : want > p.Ho ? p.Ho : want;
    const int R = (p.Ho + want - 1) / want;
    pl.R = R < rmax ? R : rmax;
    const size_t pitch = (size_t)16 * pl.CS + 8;
    pl.otile_off = (size_t)2 * p.W * pitch * 4;
    pl.lds = pl.otile_off + 2 * (size_t)32 * pl.BPW * (COUT_TILE * 4 + 32);
    if (pl.lds > (size_t)LDS_BYTES_MAX)
        return false;
    *plan = pl;
    return true;
}

// As for bf16: a 1x1 filter over pixel-contiguous data is regrouped into
// rows of 32 pixels (or another width that divides the pixel count).
DenseProblem regroup_pointwise_f32(const DenseProblem &p)
{
    if (p.KH != 1 || p.KW != 1)
        return p;
    if (p.xs[1] != (int64_t)p.W * p.xs[2] || p.ys[1] != (int64_t)p.Wo * p.ys[2])
        return p;
    const bool batch = p.xs[0] == (int64_t)p.H * p.xs[1] && p.ys[0] == (int64_t)p.Ho * p.ys[1];
    const int64_t pixels = batch ? (int64_t)p.N * p.H * p.W : (int64_t)p.H * p.W;
    int best = 0;
    double best_score = 0;
    for (int w = 16; w <= 64; ++w) {
        if (pixels % w != 0)
            continue;
        const double fill = (double)w / (16.0 * ((w + 15) / 16));
        const double score = fill * (w >= 32 ? 1.0 : (double)w / 32.0) + (w == 32 ? 1e-3 : 0.0);
        if (score > best_score) {
            best_score = score;
            best = w;
        }
    }
    if (best == 0 || pixels / best >= (int64_t(1) << 31))
        return p;
    DenseProblem q = p;
    q.N = batch ? 1 : p.N;
    q.W = q.Wo = best;
    q.H = q.Ho = (int)(pixels / best);
    q.xs[1] = (int64_t)best * p.xs[2];
    q.ys[1] = (int64_t)best * p.ys[2];
    if (batch) {
        q.xs[0] = q.H * q.xs[1];
        q.ys[0] = q.Ho * q.ys[1];
    }
    PlanF a, b;
    if (!plan_rows_f32(q, &a))
        return p;
    if (plan_rows_f32(p, &b) && p.Wo % 16 == 0 && p.Wo >= 32)
        return p;
    return q;
}

template <int KH, int KW, int CS, int BPW, int MAXC>
hipError_t launch_inst_f32(const RowArgsF &a, dim3 grid, size_t lds, hipStream_t s)
{
    constexpr int NR = band_rows_f32(KH);
    auto kern = dense_rows_mfma_f32<KH, KW, CS, BPW, MAXC, NR>;
    const hipError_t attr = allow_lds<dense_rows_mfma_f32<KH, KW, CS, BPW, MAXC, NR>>(LDS_BYTES_MAX);
    if (attr != hipSuccess)
        return attr;
    hipLaunchKernelGGL(kern, grid, dim3(THREADS), lds, s, a);
    return hipGetLastError();
}

// Loads per thread for one input row, at most, for rows that fit the
// kernel (32 * BPW output pixels plus the halo).
constexpr int max_chunks_f32(int KW, int CS, int BPW) { return ((32 * BPW + KW - 1) * 4 * CS + THREADS - 1) / THREADS; }

template <int KH, int KW, int CS, int BPW>
hipError_t launch_bpw_f32(const RowArgsF &a, dim3 grid, size_t lds, int MAXC, hipStream_t s)
{
    constexpr int CMAX = max_chunks_f32(KW, CS, BPW);
    if (MAXC == 1)
        return launch_inst_f32<KH, KW, CS, BPW, 1>(a, grid, lds, s);
    if constexpr (CMAX >= 2) {
        if (MAXC == 2)
            return launch_inst_f32<KH, KW, CS, BPW, 2>(a, grid, lds, s);
    }
    if constexpr (CMAX >= 3 && !(KH == 3 && CS == 4)) {
        if (MAXC == 4)
            return launch_inst_f32<KH, KW, CS, BPW, 4>(a, grid, lds, s);
    }
    return hipErrorNotSupported;
}

template <int KH, int KW, int CS>
hipError_t launch_cs_f32(const RowArgsF &a, dim3 grid, const PlanF &plan, hipStream_t s)
{
    if (plan.BPW == 1)
        return launch_bpw_f32<KH, KW, CS, 1>(a, grid, plan.lds, plan.MAXC, s);
    return launch_bpw_f32<KH, KW, CS, 2>(a, grid, plan.lds, plan.MAXC, s);
}

}  // namespace

bool dense_mfma_f32_supports(const DenseProblem &p)
{
    PlanF plan;
    return plan_rows_f32(regroup_pointwise_f32(p), &plan);
}

hipError_t launch_dense_mfma_f32(const DenseProblem &p0, hipStream_t s)
{
    const DenseProblem p = regroup_pointwise_f32(p0);
    PlanF plan;
    if (!plan_rows_f32(p, &plan))
        return hipErrorNotSupported;
    RowArgsF a;
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
    a.row_elems = p.W * (16 * plan.CS + 8);
    a.chunks_per_row = p.W * 16 * plan.CS / 4;
    a.otile_off = (int)plan.otile_off;
    a.x_records = (uint32_t)extent_f32(p.xs, p.H, p.W, p.Cin);
    a.y_records = (uint32_t)extent_f32(p.ys, p.Ho, p.Wo, p.Cout);
    a.R = plan.R;
    a.bands_per_img = (p.Ho + a.R - 1) / a.R;
    a.bands = p.N * a.bands_per_img;
    a.tiles = (p.Cout + COUT_TILE - 1) / COUT_TILE;
    const int64_t slots = (int64_t)((a.bands + 7) / 8 * 8) * a.tiles;
    if (slots >= (int64_t(1) << 31))
        return hipErrorNotSupported;
    const dim3 grid((unsigned)slots);

    if (p.KH == 1) {
        switch (plan.CS) {
        case 1: return launch_cs_f32<1, 1, 1>(a, grid, plan, s);
        case 2: return launch_cs_f32<1, 1, 2>(a, grid, plan, s);
        case 4: return launch_cs_f32<1, 1, 4>(a, grid, plan, s);
        case 8: return launch_cs_f32<1, 1, 8>(a, grid, plan, s);
        case 16: return launch_cs_f32<1, 1, 16>(a, grid, plan, s);
        }
    } else {
        switch (plan.CS) {
        case 1: return launch_cs_f32<3, 3, 1>(a, grid, plan, s);
        case 2: return launch_cs_f32<3, 3, 2>(a, grid, plan, s);
        case 4: return launch_cs_f32<3, 3, 4>(a, grid, plan, s);
        }
    }
    return hipErrorNotSupported;
}

}  // namespace convfwd
