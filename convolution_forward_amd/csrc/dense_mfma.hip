// Dense NHWC cross-correlation as an implicit GEMM on CDNA4 matrix cores.
//
// Contract: "CMU DLSys Lecture 14: Convolutional Network Implementation",
// section 1 (Y[n,y,x,o] = sum over i,j,c of X[n,y+i,x+j,c] * F[i,j,c,o]).
// Section 5 writes it as a product of the (N*Ho*Wo) x (K*K*Cin) patch matrix
// with F reshaped to (K*K*Cin) x Cout; section 6 prices the copy that builds
// the patch matrix. This kernel never builds it: input rows are staged once
// in LDS and every patch fragment is read from there with a per-tap offset
// (the 6-axis patch view of section 5 turned into LDS addressing).
//
// Work decomposition (one workgroup = 8 waves = 512 threads, 2 per SIMD):
//  * A workgroup owns a band of R consecutive output rows of one image and a
//    tile of 64 output channels.
//  * The filter slice F[:, :, :, tile] is loaded once, transposed through LDS,
//    and then held in registers (A operand of v_mfma_f32_16x16x32_bf16) for
//    the whole band. Wave w keeps the 32-channel half (w & 1) of the tile:
//    KH*KW*ceil(Cin/32) k-steps x 2 column blocks x 4 registers.
//  * Input rows flow through an LDS ring of KH+1 rows. Row y+KH is written
//    while output row y is computed; global loads for the next PF rows sit
//    in registers, so HBM latency overlaps the matrix work.
//  * Output row y is cut into 16-pixel blocks; wave pair (2g, 2g+1) takes
//    blocks g, g+4. Per k-step a lane reads 8 channels of one pixel (16
//    bytes, B operand) and issues one MFMA per 16-channel column block of its
//    half. The two waves sharing a SIMD hide each other's LDS latency.
//  * The product is computed transposed (rows = output channels, columns =
//    pixels), so each lane ends with 4 consecutive channels of one pixel and
//    stores them with one vector write.
//
// LDS pixel pitch is Cin_padded + 8 bf16 (16 bytes of padding): eight lanes
// reading eight consecutive pixels hit eight distinct bank groups.
// Channels beyond Cin (up to the multiple of 32) are zero in LDS.
#include <type_traits>

#include "common.h"
#include "internal.h"

namespace convfwd {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int THREADS = 512;
constexpr int COUT_TILE = 64;      // 4 column blocks of 16 output channels
constexpr int NBW = 2;             // column blocks per wave (its half of the tile)
constexpr int PF = 3;              // input rows in registers ahead of the ring
constexpr int LDS_BYTES_MAX = 160 * 1024;
constexpr uint32_t OOB = 0x80000000u;           // buffer offset beyond every range: access dropped
constexpr int BUF_WORD3 = 0x00020000;           // raw buffer descriptor word 3 (gfx9 family)

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

struct RowArgs {
    const uint16_t *X;
    const uint16_t *F;
    const float *bias;
    void *Y;
    int64_t xs0, xs1, xs2, ys0, ys1, ys2;
    int H, W, Cin, Cout, Ho, Wo;
    int R;              // output rows per band
    int bands_per_img;
    int row_elems;      // LDS elements per ring row (W * pitch)
    int chunks_per_row; // 16-byte chunks per staged input row (W * Cin_padded / 8)
    uint32_t x_records; // bytes addressable from one image's base in X
    uint32_t y_records; // bytes addressable from one image's base in Y
};

// Byte offset of 16-byte chunk q (pixel q / CG, channel group q % CG) of
// input row r inside the image, or OOB when the chunk is padding or outside
// the band: the buffer load then returns zeros without touching memory.
template <int CINP>
__device__ __forceinline__ uint32_t chunk_off(const RowArgs &a, int r, int q, int rows_end)
{
    constexpr int CG = CINP / 8;
    const int px = q / CG;
    const int cg = q - px * CG;
    const bool ok = q < a.chunks_per_row && r < rows_end && cg * 8 < a.Cin;
    return ok ? (uint32_t)(((int64_t)r * a.xs1 + (int64_t)px * a.xs2 + cg * 8) * 2) : OOB;
}

template <int CINP>
__device__ __forceinline__ void put_chunk(uint16_t *ring_row, int q, u32x4 v)
{
    constexpr int CG = CINP / 8;
    constexpr int PITCH = CINP + 8;
    const int px = q / CG;
    const int cg = q - px * CG;
    *reinterpret_cast<u32x4 *>(ring_row + px * PITCH + cg * 8) = v;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    // v_cvt_pk_bf16_f32: round to nearest even, NaN stays NaN.
    return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)lo) |
           ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)hi) << 16);
}

template <int U, int N, class Fn>
__device__ __forceinline__ void static_for(Fn &&fn)
{
    if constexpr (U < N) {
        fn(std::integral_constant<int, U>{});
        static_for<U + 1, N>(fn);
    }
}

template <int KH, int KW, int CS, int BPW, int MAXC, bool OUT_BF16>
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
void dense_rows_mfma(RowArgs a)
{
    constexpr int CINP = 32 * CS;
    constexpr int PITCH = CINP + 8;
    constexpr int KSTEPS = KH * KW * CS;
    constexpr int NSLOT = KH + 1;
    constexpr int ESZ = OUT_BF16 ? 2 : 4;

    extern __shared__ __align__(16) uint16_t smem[];
    uint16_t *ring = smem;
    uint16_t *ft = smem + NSLOT * a.row_elems;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int half = wave & 1;          // which 32 output channels of the tile
    const int pg = wave >> 1;           // pixel-block group 0..3
    const int o0 = blockIdx.y * COUT_TILE;
    const int band = blockIdx.x;
    const int n = band / a.bands_per_img;
    const int y0 = (band - n * a.bands_per_img) * a.R;
    if (y0 >= a.Ho)
        return;
    const int y1 = min(y0 + a.R, a.Ho);
    const int rows_end = y1 + KH - 1;           // one past the last input row this band reads

    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(a.X + (int64_t)n * a.xs0), 0, (int)a.x_records, BUF_WORD3);
    const __amdgpu_buffer_rsrc_t yr = __builtin_amdgcn_make_buffer_rsrc(
        static_cast<char *>(a.Y) + (int64_t)n * a.ys0 * ESZ, 0, (int)a.y_records, BUF_WORD3);

    // 1. Input rows y0 .. y0+KH-1, the filter slice and the bias: issue every
    //    global load first, then write LDS, so the latencies overlap.
    u32x4 pro[KH][MAXC];
#pragma unroll
    for (int i = 0; i < KH; ++i)
#pragma unroll
        for (int k = 0; k < MAXC; ++k)
            pro[i][k] = __builtin_amdgcn_raw_buffer_load_b128(xr, chunk_off<CINP>(a, y0 + i, tid + k * THREADS, rows_end), 0, 0);

    // Filter: item it -> (c fastest, then 8-channel output group, then tap),
    // so the 2-byte transposed LDS writes of a wave hit consecutive addresses.
    // Padding channels and output channels past Cout load as zeros.
    constexpr int FITEMS = (KH * KW * CINP * 8 + THREADS - 1) / THREADS;
    const __amdgpu_buffer_rsrc_t fr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(a.F), 0, KH * KW * a.Cin * a.Cout * 2, BUF_WORD3);
    u32x4 fv[FITEMS];
#pragma unroll
    for (int t = 0; t < FITEMS; ++t) {
        const int it = tid + t * THREADS;
        const int c = it % CINP;
        const int og = (it / CINP) & 7;
        const int tap = it / (CINP * 8);
        const int o = o0 + og * 8;
        const bool ok = tap < KH * KW && c < a.Cin && o < a.Cout;
        fv[t] = __builtin_amdgcn_raw_buffer_load_b128(
            fr, ok ? (uint32_t)((((int64_t)tap * a.Cin + c) * a.Cout + o) * 2) : OOB, 0, 0);
    }
    // Bias of this lane's 8 output channels (zeros without bias).
    const __amdgpu_buffer_rsrc_t br = __builtin_amdgcn_make_buffer_rsrc(
        a.bias ? (void *)a.bias : (void *)a.F, 0, a.bias ? a.Cout * 4 : 0, BUF_WORD3);
    u32x4 bq[NBW];
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb)
        bq[nb] = __builtin_amdgcn_raw_buffer_load_b128(
            br, (uint32_t)((o0 + half * 32 + nb * 16 + (lane >> 4) * 4) * 4), 0, 0);
    // Next PF-1 rows into the register queue.
    u32x4 stage[PF][MAXC];
#pragma unroll
    for (int p = 0; p < PF - 1; ++p)
#pragma unroll
        for (int k = 0; k < MAXC; ++k)
            stage[p][k] = __builtin_amdgcn_raw_buffer_load_b128(
                xr, chunk_off<CINP>(a, y0 + KH + p, tid + k * THREADS, rows_end), 0, 0);

#pragma unroll
    for (int i = 0; i < KH; ++i)
#pragma unroll
        for (int k = 0; k < MAXC; ++k) {
            const int q = tid + k * THREADS;
            if (q < a.chunks_per_row)
                put_chunk<CINP>(ring + i * a.row_elems, q, pro[i][k]);
        }
#pragma unroll
    for (int t = 0; t < FITEMS; ++t) {
        const int it = tid + t * THREADS;
        const int c = it % CINP;
        const int og = (it / CINP) & 7;
        const int tap = it / (CINP * 8);
        if (tap < KH * KW) {
            const uint32_t w4[4] = {fv[t][0], fv[t][1], fv[t][2], fv[t][3]};
#pragma unroll
            for (int e = 0; e < 8; ++e)
                ft[(tap * COUT_TILE + og * 8 + e) * PITCH + c] = (uint16_t)(w4[e >> 1] >> ((e & 1) * 16));
        }
    }
    __syncthreads();

    // 2. Filter fragments into registers: lane holds F^T[o = 32*half + 16nb + lane%16][8 channels].
    bf16x8 wf[KSTEPS][NBW];
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
        const int tap = ks / CS;
        const int cs = ks % CS;
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb)
            wf[ks][nb] = *reinterpret_cast<const bf16x8 *>(
                ft + (tap * COUT_TILE + half * 32 + nb * 16 + (lane & 15)) * PITCH + cs * 32 + (lane >> 4) * 8);
    }

    // 3. One output row: prefetch, matrix work, store, commit, barrier. Every
    //    global memory operation here is unconditional (invalid lanes use
    //    out-of-range buffer offsets), so the compiler can count outstanding
    //    loads exactly and keep PF rows in flight.
    auto row_step = [&](const int y, auto U) {
        constexpr int u = decltype(U)::value;
#pragma unroll
        for (int k = 0; k < MAXC; ++k)
            stage[(u + PF - 1) % PF][k] = __builtin_amdgcn_raw_buffer_load_b128(
                xr, chunk_off<CINP>(a, y + KH + PF - 1, tid + k * THREADS, rows_end), 0, 0);

        const uint16_t *rowp[KH];
#pragma unroll
        for (int i = 0; i < KH; ++i)
            rowp[i] = ring + ((y - y0 + i) % NSLOT) * a.row_elems;

#pragma unroll
        for (int qb = 0; qb < BPW; ++qb) {
            const int x = (pg + 4 * qb) * 16 + (lane & 15);
            const int xl = min(x, a.Wo - 1);
            f32x4 acc[NBW];
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb)
                acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) {
                const int tap = ks / CS;
                const int i = tap / KW;
                const int j = tap % KW;
                const int cs = ks % CS;
                const bf16x8 xb = *reinterpret_cast<const bf16x8 *>(
                    rowp[i] + (xl + j) * PITCH + cs * 32 + (lane >> 4) * 8);
#pragma unroll
                for (int nb = 0; nb < NBW; ++nb)
                    acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[ks][nb], xb, acc[nb], 0, 0, 0);
            }
            // Lane holds channels o0+32*half+16nb+4*(lane/16)+{0..3} of pixel x.
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb) {
                const int ch0 = o0 + half * 32 + nb * 16 + (lane >> 4) * 4;
                const bool ok = x < a.Wo && ch0 < a.Cout;
                const uint32_t off = ok ? (uint32_t)(((int64_t)y * a.ys1 + (int64_t)x * a.ys2 + ch0) * ESZ) : OOB;
                const float v0 = acc[nb][0] + __uint_as_float(bq[nb][0]);
                const float v1 = acc[nb][1] + __uint_as_float(bq[nb][1]);
                const float v2 = acc[nb][2] + __uint_as_float(bq[nb][2]);
                const float v3 = acc[nb][3] + __uint_as_float(bq[nb][3]);
                if constexpr (OUT_BF16) {
                    const u32x2 w = {pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
                    __builtin_amdgcn_raw_buffer_store_b64(w, yr, off, 0, 0);
                } else {
                    const u32x4 w = {__float_as_uint(v0), __float_as_uint(v1), __float_as_uint(v2), __float_as_uint(v3)};
                    __builtin_amdgcn_raw_buffer_store_b128(w, yr, off, 0, 0);
                }
            }
        }

        // Commit input row y+KH (loaded PF-1 rows ago) into the ring slot of
        // row y-1, which no wave reads any more.
        const int r = y + KH;
        if (r < rows_end) {
            uint16_t *dst = ring + ((r - y0) % NSLOT) * a.row_elems;
#pragma unroll
            for (int k = 0; k < MAXC; ++k) {
                const int q = tid + k * THREADS;
                if (q < a.chunks_per_row)
                    put_chunk<CINP>(dst, q, stage[u][k]);
            }
        }
        __syncthreads();
    };

    int y = y0;
    for (; y + PF <= y1; y += PF)
        static_for<0, PF>([&](auto U) { row_step(y + decltype(U)::value, U); });
    static_for<0, PF - 1>([&](auto U) {
        if (y + decltype(U)::value < y1)
            row_step(y + decltype(U)::value, U);
    });
}

// --- host side -------------------------------------------------------------

int cin_steps(int Cin)
{
    const int cs = (Cin + 31) / 32;
    for (int c : {1, 2, 4, 8, 16})
        if (cs <= c)
            return c;
    return 0;
}

bool taps_instantiated(int KH, int KW, int CS)
{
    if (KH == 1 && KW == 1)
        return CS == 1 || CS == 2 || CS == 4 || CS == 8 || CS == 16;
    if (KH == 2 && KW == 2)
        return CS == 1 || CS == 2 || CS == 4;
    if (KH == 3 && KW == 3)
        return CS == 1 || CS == 2;
    return false;
}

size_t lds_bytes(const DenseProblem &p, int CS)
{
    const int cinp = 32 * CS;
    const size_t pitch = (size_t)cinp + 8;
    return ((size_t)(p.KH + 1) * p.W * pitch + (size_t)p.KH * p.KW * COUT_TILE * pitch) * 2;
}

struct Plan {
    int CS, BPW, MAXC;
    size_t lds;
};

// Bytes addressable from one image's base: the extent of the last element.
int64_t image_extent(const int64_t *s, int rows, int cols, int ch, int esz)
{
    return ((int64_t)(rows - 1) * s[1] + (int64_t)(cols - 1) * s[2] + ch) * esz;
}

bool plan_rows(const DenseProblem &p, Plan *plan)
{
    if (p.xdt != CONV_BF16 || p.Cin % 8 != 0 || p.Cout % 8 != 0)
        return false;
    if ((uintptr_t)p.F % 16 != 0 || (int64_t)p.KH * p.KW * p.Cin * p.Cout * 2 >= (int64_t(1) << 31))
        return false;
    if ((uintptr_t)p.X % 16 != 0 || p.xs[0] % 8 != 0 || p.xs[1] % 8 != 0 || p.xs[2] % 8 != 0)
        return false;
    const int yesz = p.ydt == CONV_BF16 ? 2 : 4;
    if ((uintptr_t)p.Y % (4 * yesz) != 0 || p.ys[0] % 4 != 0 || p.ys[1] % 4 != 0 || p.ys[2] % 4 != 0)
        return false;
    // Buffer offsets are 32-bit: one image of X and of Y must stay below 2 GB.
    if (image_extent(p.xs, p.H, p.W, p.Cin, 2) >= (int64_t(1) << 31) ||
        image_extent(p.ys, p.Ho, p.Wo, p.Cout, yesz) >= (int64_t(1) << 31))
        return false;
    const int CS = cin_steps(p.Cin);
    if (CS == 0 || !taps_instantiated(p.KH, p.KW, CS))
        return false;
    const int blocks = (p.Wo + 15) / 16;
    const int BPW = (blocks + 3) / 4;
    if (BPW > 2)
        return false;
    const int64_t chunks = (int64_t)p.W * 32 * CS / 8;
    const int MAXC = chunks <= THREADS ? 1 : chunks <= 2 * THREADS ? 2 : chunks <= 4 * THREADS ? 4 : 0;
    if (MAXC == 0)
        return false;
    const size_t lds = lds_bytes(p, CS);
    if (lds > (size_t)LDS_BYTES_MAX)
        return false;
    plan->CS = CS;
    plan->BPW = BPW;
    plan->MAXC = MAXC;
    plan->lds = lds;
    return true;
}

template <int KH, int KW, int CS, int BPW, int MAXC, bool OB>
hipError_t launch_inst(const RowArgs &a, dim3 grid, size_t lds, hipStream_t s)
{
    auto kern = dense_rows_mfma<KH, KW, CS, BPW, MAXC, OB>;
    // Allow the full LDS once per instantiation (first launch, before any
    // graph capture a caller may start later).
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES_MAX);
    if (attr != hipSuccess)
        return attr;
    hipLaunchKernelGGL(kern, grid, dim3(THREADS), lds, s, a);
    return hipGetLastError();
}

template <int KH, int KW, int CS, int BPW>
hipError_t launch_bpw(const RowArgs &a, dim3 grid, size_t lds, int MAXC, bool ob, hipStream_t s)
{
    switch (MAXC) {
    case 1: return ob ? launch_inst<KH, KW, CS, BPW, 1, true>(a, grid, lds, s) : launch_inst<KH, KW, CS, BPW, 1, false>(a, grid, lds, s);
    case 2: return ob ? launch_inst<KH, KW, CS, BPW, 2, true>(a, grid, lds, s) : launch_inst<KH, KW, CS, BPW, 2, false>(a, grid, lds, s);
    default: return ob ? launch_inst<KH, KW, CS, BPW, 4, true>(a, grid, lds, s) : launch_inst<KH, KW, CS, BPW, 4, false>(a, grid, lds, s);
    }
}

template <int KH, int KW, int CS>
hipError_t launch_cs(const RowArgs &a, dim3 grid, const Plan &plan, bool ob, hipStream_t s)
{
    if (plan.BPW == 1)
        return launch_bpw<KH, KW, CS, 1>(a, grid, plan.lds, plan.MAXC, ob, s);
    return launch_bpw<KH, KW, CS, 2>(a, grid, plan.lds, plan.MAXC, ob, s);
}

}  // namespace

bool dense_tiled_supports(const DenseProblem &p)
{
    Plan plan;
    return plan_rows(p, &plan);
}

hipError_t launch_dense_tiled(const DenseProblem &p, hipStream_t s)
{
    Plan plan;
    if (!plan_rows(p, &plan))
        return hipErrorNotSupported;
    RowArgs a;
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
    a.Cin = p.Cin;
    a.Cout = p.Cout;
    a.Ho = p.Ho;
    a.Wo = p.Wo;
    a.row_elems = p.W * (32 * plan.CS + 8);
    a.chunks_per_row = p.W * 32 * plan.CS / 8;
    a.x_records = (uint32_t)image_extent(p.xs, p.H, p.W, p.Cin, 2);
    a.y_records = (uint32_t)image_extent(p.ys, p.Ho, p.Wo, p.Cout, p.ydt == CONV_BF16 ? 2 : 4);

    // Bands: aim for one workgroup per compute unit (256) in total.
    const int tiles = (p.Cout + COUT_TILE - 1) / COUT_TILE;
    int want = (int)((256 + (int64_t)p.N * tiles - 1) / ((int64_t)p.N * tiles));
    if (want < 1)
        want = 1;
    if (want > p.Ho)
        want = p.Ho;
    a.R = (p.Ho + want - 1) / want;
    a.bands_per_img = (p.Ho + a.R - 1) / a.R;
    const dim3 grid((unsigned)(p.N * a.bands_per_img), (unsigned)tiles);
    const bool ob = p.ydt == CONV_BF16;

    switch (p.KH * 100 + p.KW * 10) {
    case 110:
        switch (plan.CS) {
        case 1: return launch_cs<1, 1, 1>(a, grid, plan, ob, s);
        case 2: return launch_cs<1, 1, 2>(a, grid, plan, ob, s);
        case 4: return launch_cs<1, 1, 4>(a, grid, plan, ob, s);
        case 8: return launch_cs<1, 1, 8>(a, grid, plan, ob, s);
        case 16: return launch_cs<1, 1, 16>(a, grid, plan, ob, s);
        }
        break;
    case 220:
        switch (plan.CS) {
        case 1: return launch_cs<2, 2, 1>(a, grid, plan, ob, s);
        case 2: return launch_cs<2, 2, 2>(a, grid, plan, ob, s);
        case 4: return launch_cs<2, 2, 4>(a, grid, plan, ob, s);
        }
        break;
    case 330:
        switch (plan.CS) {
        case 1: return launch_cs<3, 3, 1>(a, grid, plan, ob, s);
        case 2: return launch_cs<3, 3, 2>(a, grid, plan, ob, s);
        }
        break;
    }
    return hipErrorNotSupported;
}

}  // namespace convfwd
