// Dense NHWC cross-correlation, any window, as an implicit GEMM on matrix
// cores with both operands staged through LDS.
//
// Contract: "CMU DLSys Lecture 14: Convolutional Network Implementation",
// sections 1 and 5 (Y = patch matrix times F.reshape(K*K*Cin, Cout), the
// patch matrix never built), with the window of "Convolution Is Wx+b Moving
// Across a Signal" (section "Why 1D? Why 2D?": output (y, x) reads input
// row y*sh + i*dh - pt and column x*sw + j*dw - pl, zero outside) and its
// groups (section "Find the same sum in CKE's C kernels").
//
// This kernel takes strided windows whose groups fill its 64-channel tiles,
// and what the row kernel (dense_mfma.hip) declines: more than 64 input
// channels under a 3x3 window, 5x5 and larger windows, dilation, unequal
// strides, and 1D sequences longer than a row tile. It holds nothing per
// band: the GEMM's M axis is the flat output pixel index
// m = (n*Ho + y)*Wo + x, so any output shape tiles evenly.
//
// Work decomposition (one workgroup = 12 waves = 768 threads, three per
// SIMD):
//  * A tile is 64*BPW output pixels x 64 output channels of one group.
//  * Eight waves only load: each issues its share of every stage's loads,
//    waits for them and meets the others at the stage's barrier. Issuing a
//    stage's loads holds a wave for about as long as the stage's MFMAs take
//    (timestamps: 0.9 us a stage with four issuing waves, whether each load
//    gathers 16 pixels x 64 bytes or 8 pixels x 128 bytes), so a wave that
//    both loads and computes leaves the matrix pipe idle that long, and
//    more issuing waves shorten it.
//  * Four waves only compute: computing wave w owns the tile's 16-pixel
//    blocks w*BPW .. w*BPW + BPW - 1 and all 64 channels (four 16-channel
//    column blocks): 4*BPW accumulators. BPW (2 to 5) is chosen per launch
//    so the tiles fill the compute units in as few rounds as possible.
//  * The K axis runs over stages (64-channel slice, tap i, tap j): the taps
//    of one slice follow each other, so they read input lines still in the
//    caches (the sum is the same; only the fp32 rounding order differs from
//    the lecture's (i, j, c)). A stage is two MFMA k-steps of 32 channels.
//    Its operands are staged in LDS: the patch slice (the tile's pixels x 64
//    channels, one whole 128-byte line a pixel: the address unit's time goes
//    by lines touched, so 8 pixels x 128 bytes per load cost about half of
//    16 pixels x 64 bytes) and the filter slice F[i, j, c:c+64, o0:o0+64]
//    (8 KB), both with loads that write LDS directly (each wave instruction
//    fills 1 KB contiguously; taps in the padding, pixels past the end and
//    channels past Cin load zeros).
//  * Stages go through a ring of three: stage t + 2 is requested as stage t
//    starts, so two stages are in flight while one is used. The waits are
//    explicit counts: every memory instruction in the loop is unconditional
//    (stages past the end load zeros into a free slot), so the number issued
//    after stage t is a constant.
//  * Filter fragments are read with the gfx950 transpose read, patch
//    fragments with 16-byte reads; both are placed with an XOR swizzle so the
//    16 lanes of a read hit distinct banks. All of a stage's fragment reads
//    go out from one asm block that ends in its own wait (as intrinsics the
//    transpose reads would be preceded by a wait for every load in flight).
//  * bf16 results are regrouped through LDS (by then idle): each wave parks
//    its pixels x 64 channels there, then eight lanes store each pixel's
//    128-byte row whole. fp32 results leave straight from the accumulators,
//    16 bytes per lane in 64-byte runs.
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

constexpr int LOADERS = 8;              // waves that only issue loads
constexpr int GT = 64 * (LOADERS + 4);  // threads per workgroup: the loading and 4 computing waves
constexpr int GN = 64;                  // output channels per tile
constexpr int NB = 4;                   // 16-channel column blocks per wave
constexpr int NSTAGE = 3;               // stages in the LDS ring
constexpr int FSTAGE = 64 * GN * 2;     // filter bytes per stage (64 rows of 128 bytes)
constexpr int OPITCH = GN * 2 + 16;     // LDS pitch of one pixel of a wave's bf16 output patch (bytes)
constexpr uint32_t OOB = 0x80000000u;
constexpr int BUF_WORD3 = 0x00020000;
constexpr int LDS_MAX = 160 * 1024;

template <int BPW>
struct GShape {
    static constexpr int M = 64 * BPW;                  // pixels per tile
    static constexpr int XSTAGE = M * 128;              // patch bytes per stage
    static constexpr int STAGE = XSTAGE + FSTAGE;
    static constexpr int LDS = NSTAGE * STAGE;
    static constexpr int XLOADS = XSTAGE / (LOADERS * 64 * 16);   // patch loads per loading lane: 2 * BPW
    static constexpr int FLOADS = FSTAGE / (LOADERS * 64 * 16);   // filter loads per loading lane: 1
    static constexpr int LOADS = XLOADS + FLOADS;       // loads per loading lane per stage
    static_assert(LDS <= LDS_MAX, "LDS");
    static_assert(4 * 16 * BPW * OPITCH <= LDS, "output patches fit in the ring");
    static_assert(XLOADS * LOADERS * 64 * 16 == XSTAGE && FLOADS * LOADERS * 64 * 16 == FSTAGE, "whole loads");
    static_assert(LOADS < 64, "vmcnt holds 6 bits");
};

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

template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt holds 6 bits");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Physical 16-byte chunk of logical chunk c in row k of a staged filter
// slice (rows of 128 bytes): the 8 rows that one half-wave's transpose read
// touches fall in 8 distinct pairs of bank groups. (Patch pixels P, also
// 128 bytes, keep logical chunk c at c ^ ((P >> 1) & 7): the 16 pixels of a
// fragment read fall in 16 distinct bank groups.)
__host__ __device__ constexpr int fswz(int k) { return (((k >> 1) & 1) << 1) | (((k >> 3) & 1) << 2); }

// Every fragment read of one stage: for each k-step s the four filter
// fragments (two transposed 8-byte reads each, at +0 and +512 bytes from the
// column block's base, k-step 1 another 4 KB on) and the BPW patch
// fragments (16-byte reads 2 KB apart from k-step s's base). Outputs are
// early-clobber so no read lands in an address register still to be used.
template <int BPW>
__device__ __forceinline__ void stage_reads(const uint32_t (&abase)[4], const uint32_t (&xbase)[2],
                                            i16x4 (&a)[2][4][2], u32x4 (&b)[2][BPW]);

template <>
__device__ __forceinline__ void stage_reads<2>(const uint32_t (&abase)[4], const uint32_t (&xbase)[2],
                                                 i16x4 (&a)[2][4][2], u32x4 (&b)[2][2])
{
    asm volatile("ds_read_b64_tr_b16 %0, %20 offset:0\n\t"
                 "ds_read_b64_tr_b16 %1, %20 offset:512\n\t"
                 "ds_read_b64_tr_b16 %2, %21 offset:0\n\t"
                 "ds_read_b64_tr_b16 %3, %21 offset:512\n\t"
                 "ds_read_b64_tr_b16 %4, %22 offset:0\n\t"
                 "ds_read_b64_tr_b16 %5, %22 offset:512\n\t"
                 "ds_read_b64_tr_b16 %6, %23 offset:0\n\t"
                 "ds_read_b64_tr_b16 %7, %23 offset:512\n\t"
                 "ds_read_b128 %16, %24 offset:0\n\t"
                 "ds_read_b128 %17, %24 offset:2048\n\t"
                 "ds_read_b64_tr_b16 %8, %20 offset:4096\n\t"
                 "ds_read_b64_tr_b16 %9, %20 offset:4608\n\t"
                 "ds_read_b64_tr_b16 %10, %21 offset:4096\n\t"
                 "ds_read_b64_tr_b16 %11, %21 offset:4608\n\t"
                 "ds_read_b64_tr_b16 %12, %22 offset:4096\n\t"
                 "ds_read_b64_tr_b16 %13, %22 offset:4608\n\t"
                 "ds_read_b64_tr_b16 %14, %23 offset:4096\n\t"
                 "ds_read_b64_tr_b16 %15, %23 offset:4608\n\t"
                 "ds_read_b128 %18, %25 offset:0\n\t"
                 "ds_read_b128 %19, %25 offset:2048\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(a[0][0][0]), "=&v"(a[0][0][1]), "=&v"(a[0][1][0]), "=&v"(a[0][1][1]), "=&v"(a[0][2][0]), "=&v"(a[0][2][1]), "=&v"(a[0][3][0]), "=&v"(a[0][3][1]), "=&v"(a[1][0][0]), "=&v"(a[1][0][1]), "=&v"(a[1][1][0]), "=&v"(a[1][1][1]), "=&v"(a[1][2][0]), "=&v"(a[1][2][1]), "=&v"(a[1][3][0]), "=&v"(a[1][3][1]), "=&v"(b[0][0]), "=&v"(b[0][1]), "=&v"(b[1][0]), "=&v"(b[1][1])
                 : "v"(abase[0]), "v"(abase[1]), "v"(abase[2]), "v"(abase[3]), "v"(xbase[0]), "v"(xbase[1])
                 : "memory");
}

template <>
__device__ __forceinline__ void stage_reads<3>(const uint32_t (&abase)[4], const uint32_t (&xbase)[2],
                                                 i16x4 (&a)[2][4][2], u32x4 (&b)[2][3])
{
    asm volatile("ds_read_b64_tr_b16 %0, %22 offset:0\n\t"
                 "ds_read_b64_tr_b16 %1, %22 offset:512\n\t"
                 "ds_read_b64_tr_b16 %2, %23 offset:0\n\t"
                 "ds_read_b64_tr_b16 %3, %23 offset:512\n\t"
                 "ds_read_b64_tr_b16 %4, %24 offset:0\n\t"
                 "ds_read_b64_tr_b16 %5, %24 offset:512\n\t"
                 "ds_read_b64_tr_b16 %6, %25 offset:0\n\t"
                 "ds_read_b64_tr_b16 %7, %25 offset:512\n\t"
                 "ds_read_b128 %16, %26 offset:0\n\t"
                 "ds_read_b128 %17, %26 offset:2048\n\t"
                 "ds_read_b128 %18, %26 offset:4096\n\t"
                 "ds_read_b64_tr_b16 %8, %22 offset:4096\n\t"
                 "ds_read_b64_tr_b16 %9, %22 offset:4608\n\t"
                 "ds_read_b64_tr_b16 %10, %23 offset:4096\n\t"
                 "ds_read_b64_tr_b16 %11, %23 offset:4608\n\t"
                 "ds_read_b64_tr_b16 %12, %24 offset:4096\n\t"
                 "ds_read_b64_tr_b16 %13, %24 offset:4608\n\t"
                 "ds_read_b64_tr_b16 %14, %25 offset:4096\n\t"
                 "ds_read_b64_tr_b16 %15, %25 offset:4608\n\t"
                 "ds_read_b128 %19, %27 offset:0\n\t"
                 "ds_read_b128 %20, %27 offset:2048\n\t"
                 "ds_read_b128 %21, %27 offset:4096\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(a[0][0][0]), "=&v"(a[0][0][1]), "=&v"(a[0][1][0]), "=&v"(a[0][1][1]), "=&v"(a[0][2][0]), "=&v"(a[0][2][1]), "=&v"(a[0][3][0]), "=&v"(a[0][3][1]), "=&v"(a[1][0][0]), "=&v"(a[1][0][1]), "=&v"(a[1][1][0]), "=&v"(a[1][1][1]), "=&v"(a[1][2][0]), "=&v"(a[1][2][1]), "=&v"(a[1][3][0]), "=&v"(a[1][3][1]), "=&v"(b[0][0]), "=&v"(b[0][1]), "=&v"(b[0][2]), "=&v"(b[1][0]), "=&v"(b[1][1]), "=&v"(b[1][2])
                 : "v"(abase[0]), "v"(abase[1]), "v"(abase[2]), "v"(abase[3]), "v"(xbase[0]), "v"(xbase[1])
                 : "memory");
}

template <>
__device__ __forceinline__ void stage_reads<4>(const uint32_t (&abase)[4], const uint32_t (&xbase)[2],
                                                 i16x4 (&a)[2][4][2], u32x4 (&b)[2][4])
{
    asm volatile("ds_read_b64_tr_b16 %0, %24 offset:0\n\t"
                 "ds_read_b64_tr_b16 %1, %24 offset:512\n\t"
                 "ds_read_b64_tr_b16 %2, %25 offset:0\n\t"
                 "ds_read_b64_tr_b16 %3, %25 offset:512\n\t"
                 "ds_read_b64_tr_b16 %4, %26 offset:0\n\t"
                 "ds_read_b64_tr_b16 %5, %26 offset:512\n\t"
                 "ds_read_b64_tr_b16 %6, %27 offset:0\n\t"
                 "ds_read_b64_tr_b16 %7, %27 offset:512\n\t"
                 "ds_read_b128 %16, %28 offset:0\n\t"
                 "ds_read_b128 %17, %28 offset:2048\n\t"
                 "ds_read_b128 %18, %28 offset:4096\n\t"
                 "ds_read_b128 %19, %28 offset:6144\n\t"
                 "ds_read_b64_tr_b16 %8, %24 offset:4096\n\t"
                 "ds_read_b64_tr_b16 %9, %24 offset:4608\n\t"
                 "ds_read_b64_tr_b16 %10, %25 offset:4096\n\t"
                 "ds_read_b64_tr_b16 %11, %25 offset:4608\n\t"
                 "ds_read_b64_tr_b16 %12, %26 offset:4096\n\t"
                 "ds_read_b64_tr_b16 %13, %26 offset:4608\n\t"
                 "ds_read_b64_tr_b16 %14, %27 offset:4096\n\t"
                 "ds_read_b64_tr_b16 %15, %27 offset:4608\n\t"
                 "ds_read_b128 %20, %29 offset:0\n\t"
                 "ds_read_b128 %21, %29 offset:2048\n\t"
                 "ds_read_b128 %22, %29 offset:4096\n\t"
                 "ds_read_b128 %23, %29 offset:6144\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(a[0][0][0]), "=&v"(a[0][0][1]), "=&v"(a[0][1][0]), "=&v"(a[0][1][1]), "=&v"(a[0][2][0]), "=&v"(a[0][2][1]), "=&v"(a[0][3][0]), "=&v"(a[0][3][1]), "=&v"(a[1][0][0]), "=&v"(a[1][0][1]), "=&v"(a[1][1][0]), "=&v"(a[1][1][1]), "=&v"(a[1][2][0]), "=&v"(a[1][2][1]), "=&v"(a[1][3][0]), "=&v"(a[1][3][1]), "=&v"(b[0][0]), "=&v"(b[0][1]), "=&v"(b[0][2]), "=&v"(b[0][3]), "=&v"(b[1][0]), "=&v"(b[1][1]), "=&v"(b[1][2]), "=&v"(b[1][3])
                 : "v"(abase[0]), "v"(abase[1]), "v"(abase[2]), "v"(abase[3]), "v"(xbase[0]), "v"(xbase[1])
                 : "memory");
}

template <>
__device__ __forceinline__ void stage_reads<5>(const uint32_t (&abase)[4], const uint32_t (&xbase)[2],
                                                 i16x4 (&a)[2][4][2], u32x4 (&b)[2][5])
{
    asm volatile("ds_read_b64_tr_b16 %0, %26 offset:0\n\t"
                 "ds_read_b64_tr_b16 %1, %26 offset:512\n\t"
                 "ds_read_b64_tr_b16 %2, %27 offset:0\n\t"
                 "ds_read_b64_tr_b16 %3, %27 offset:512\n\t"
                 "ds_read_b64_tr_b16 %4, %28 offset:0\n\t"
                 "ds_read_b64_tr_b16 %5, %28 offset:512\n\t"
                 "ds_read_b64_tr_b16 %6, %29 offset:0\n\t"
                 "ds_read_b64_tr_b16 %7, %29 offset:512\n\t"
                 "ds_read_b128 %16, %30 offset:0\n\t"
                 "ds_read_b128 %17, %30 offset:2048\n\t"
                 "ds_read_b128 %18, %30 offset:4096\n\t"
                 "ds_read_b128 %19, %30 offset:6144\n\t"
                 "ds_read_b128 %20, %30 offset:8192\n\t"
                 "ds_read_b64_tr_b16 %8, %26 offset:4096\n\t"
                 "ds_read_b64_tr_b16 %9, %26 offset:4608\n\t"
                 "ds_read_b64_tr_b16 %10, %27 offset:4096\n\t"
                 "ds_read_b64_tr_b16 %11, %27 offset:4608\n\t"
                 "ds_read_b64_tr_b16 %12, %28 offset:4096\n\t"
                 "ds_read_b64_tr_b16 %13, %28 offset:4608\n\t"
                 "ds_read_b64_tr_b16 %14, %29 offset:4096\n\t"
                 "ds_read_b64_tr_b16 %15, %29 offset:4608\n\t"
                 "ds_read_b128 %21, %31 offset:0\n\t"
                 "ds_read_b128 %22, %31 offset:2048\n\t"
                 "ds_read_b128 %23, %31 offset:4096\n\t"
                 "ds_read_b128 %24, %31 offset:6144\n\t"
                 "ds_read_b128 %25, %31 offset:8192\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(a[0][0][0]), "=&v"(a[0][0][1]), "=&v"(a[0][1][0]), "=&v"(a[0][1][1]), "=&v"(a[0][2][0]), "=&v"(a[0][2][1]), "=&v"(a[0][3][0]), "=&v"(a[0][3][1]), "=&v"(a[1][0][0]), "=&v"(a[1][0][1]), "=&v"(a[1][1][0]), "=&v"(a[1][1][1]), "=&v"(a[1][2][0]), "=&v"(a[1][2][1]), "=&v"(a[1][3][0]), "=&v"(a[1][3][1]), "=&v"(b[0][0]), "=&v"(b[0][1]), "=&v"(b[0][2]), "=&v"(b[0][3]), "=&v"(b[0][4]), "=&v"(b[1][0]), "=&v"(b[1][1]), "=&v"(b[1][2]), "=&v"(b[1][3]), "=&v"(b[1][4])
                 : "v"(abase[0]), "v"(abase[1]), "v"(abase[2]), "v"(abase[3]), "v"(xbase[0]), "v"(xbase[1])
                 : "memory");
}

struct GemmArgs {
    const uint16_t *X;
    const uint16_t *F;
    const float *bias;
    void *Y;
    int64_t xs0, xs1, xs2, ys0, ys1, ys2;
    int H, W, Ho, Wo, KH, KW;
    int Cin, Cout;          // channels of one group
    int f_ld;               // F row length (output channels of all groups)
    int sh, sw, pt, pl, dh, dw;
    int nstages;            // KH * KW * (64-channel slices)
    int taps;               // KH * KW
    int m_total;            // N * Ho * Wo
    int n_tiles;            // 64-channel tiles per group
    int nt_all;             // n_tiles * groups: channel tiles per pixel tile
    int tiles;              // pixel tiles * nt_all
    uint32_t x_records, f_records, b_records;
    FastDivG div_wo, div_ho;
};

template <int BPW, bool OUT_BF16>
__global__ __launch_bounds__(GT) void dense_gemm_mfma(GemmArgs a)
{
    using S = GShape<BPW>;
    constexpr int ESZ = OUT_BF16 ? 2 : 4;
    extern __shared__ __align__(16) uint8_t ring[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int g = lane >> 4;                 // k-group of the lane
    const int r = lane & 15;
    // Slot s runs on XCD s % 8; consecutive tiles (the channel tiles of one
    // pixel tile first) go to one XCD so the X rows they share meet in its L2.
    const int bid = with_args_loaded((int)blockIdx.x, a);
    const int tile = (bid & 7) * (int)(gridDim.x >> 3) + (bid >> 3);
    if (tile >= a.tiles)
        return;
    const int mt = tile / a.nt_all;
    const int nt = tile - mt * a.nt_all;
    const int grp = nt / a.n_tiles;
    const int o0 = (nt - grp * a.n_tiles) * GN;
    const int xc0 = grp * a.Cin, oc0 = grp * a.Cout;
    const int m0 = mt * S::M;

    if (wave < LOADERS) {
        // ---- Loader wave p: issues its share of every stage's loads and
        // waits for them; the barrier then publishes the stage.
        // The wave index as a scalar: every LDS destination below is then
        // computed on the scalar unit (M0), not moved out of a vector
        // register per load.
        const int pw = __builtin_amdgcn_readfirstlane(wave);
        const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t *>(a.X), 0, (int)a.x_records, BUF_WORD3);
        const __amdgpu_buffer_rsrc_t fr = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t *>(a.F), 0, (int)a.f_records, BUF_WORD3);
        // Patch loads: load v of loader p fills tile pixels
        // 8*(LOADERS*v + p) ..+7, lane L taking pixel P = 8*(LOADERS*v + p) + L/8
        // and stored chunk L % 8, which holds logical chunk
        // (L % 8) ^ ((P >> 1) % 8) (8 channels): the same for every v.
        constexpr int XL = S::XLOADS;
        const int xchunk = (lane & 7) ^ ((4 * (pw & 1) + (lane >> 4)) & 7);
        int xb0[XL], iy0[XL], ix0[XL];
        bool mok[XL];
#pragma unroll
        for (int v = 0; v < XL; ++v) {
            const int m = m0 + 8 * (LOADERS * v + pw) + (lane >> 3);
            mok[v] = m < a.m_total;
            const uint32_t mm = mok[v] ? (uint32_t)m : 0u;
            const uint32_t ny = fdiv_g(mm, a.div_wo);
            const int x = (int)(mm - ny * (uint32_t)a.Wo);
            const uint32_t n = fdiv_g(ny, a.div_ho);
            const int y = (int)(ny - n * (uint32_t)a.Ho);
            xb0[v] = (int)(n * (uint32_t)a.xs0) + xc0 + 8 * xchunk;
            iy0[v] = y * a.sh - a.pt;
            ix0[v] = x * a.sw - a.pl;
        }
        // Filter loads: loader p fills rows 8p .. 8p+7 of the slice's 64, lane
        // L row 8p + L/8, stored chunk L % 8 (logical chunk (L % 8) ^
        // fswz(row)).
        const int frow = 8 * pw + (lane >> 3);
        const int fcol = o0 + 8 * ((lane & 7) ^ fswz(frow));
        const bool fcol_ok = fcol < a.Cout;

        // The stage whose loads go out next: tap (li, lj), channel slice lcs.
        int lst = 0, lcs = 0, li = 0, lj = 0;
        auto issue_stage = [&](int t) __attribute__((always_inline)) {
            uint8_t *dst = ring + (t % NSTAGE) * S::STAGE;
            const bool kok = lst < a.nstages;
            const int c = lcs * 64;
#pragma unroll
            for (int v = 0; v < XL; ++v) {
                const int iy = iy0[v] + li * a.dh;
                const int ix = ix0[v] + lj * a.dw;
                const bool ok = kok && mok[v] && (unsigned)iy < (unsigned)a.H && (unsigned)ix < (unsigned)a.W &&
                                c + 8 * xchunk < a.Cin;
                const uint32_t off =
                    ok ? ((uint32_t)xb0[v] + (uint32_t)iy * (uint32_t)a.xs1 + (uint32_t)ix * (uint32_t)a.xs2 + (uint32_t)c) * 2u
                       : OOB;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    xr, (__attribute__((address_space(3))) void *)(dst + 1024 * (LOADERS * v + pw)), 16, off, 0, 0, 0);
            }
            {
                const int tap = li * a.KW + lj;
                const int row = c + frow;
                const bool ok = kok && fcol_ok && row < a.Cin;
                const uint32_t off = ok ? (uint32_t)((((int64_t)tap * a.Cin + row) * a.f_ld + oc0 + fcol) * 2) : OOB;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    fr, (__attribute__((address_space(3))) void *)(dst + S::XSTAGE + 1024 * pw), 16, off, 0, 0, 0);
            }
            // Next stage: tap column, then tap row, then channel slice (the
            // taps of one slice read neighbouring input lines while they are
            // cached).
            ++lst;
            if (++lj == a.KW) {
                lj = 0;
                if (++li == a.KH) {
                    li = 0;
                    ++lcs;
                }
            }
        };

        issue_stage(0);
        issue_stage(1);
        for (int t = 0; t < a.nstages; ++t) {
            // Stage t landed for this loader (issued after it: stage t + 1);
            // at the barrier, for every loader. Past the barrier the
            // computing waves have read stage t - 1: its slot takes stage
            // t + 2.
            wait_vmcnt<S::LOADS>();
            lds_barrier();
            __builtin_amdgcn_sched_barrier(0);
            issue_stage(t + 2);
            __builtin_amdgcn_sched_barrier(0);
        }
        // The stages past the end (zeros into free slots) land before the
        // ring is reused for the output.
        wait_vmcnt<0>();
        lds_barrier();
        return;
    }

    // ---- Computing wave w: MFMAs on the stage published by the barrier.
    const int cw = wave - LOADERS;
    // Fragment addresses within a stage. Filter, k-step s: lane (g, r) reads
    // row 32s + 8g + 4h + r/4 (h = 0, 1), logical chunk 2nb + (r%4)/2, half
    // r%2. Patch, k-step s: block b of the wave, pixel
    // P = 16*(cw*BPW + b) + r, logical chunk 4s + g.
    const int arow = 8 * g + (r >> 2);
    const int asw = fswz(arow) >> 1;
    uint32_t abase0[4];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
        abase0[nb] = (uint32_t)(S::XSTAGE + 128 * arow + 32 * (nb ^ asw) + 16 * ((r & 3) >> 1) + 8 * (r & 1));
    uint32_t xbase0[2];
#pragma unroll
    for (int st = 0; st < 2; ++st)
        xbase0[st] = (uint32_t)(128 * (16 * cw * BPW + r) + 16 * ((4 * st + g) ^ ((r >> 1) & 7)));
    const uint32_t ring_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t *)ring;

    f32x4 acc[BPW][NB];
#pragma unroll
    for (int b = 0; b < BPW; ++b)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
            acc[b][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int t = 0; t < a.nstages; ++t) {
        // Stage t is in LDS for every loader; stage t - 1's reads are done.
        lds_barrier();
        __builtin_amdgcn_sched_barrier(0);
        const uint32_t sb = ring_lds + (uint32_t)((t % NSTAGE) * S::STAGE);
        uint32_t ab[4], xbs[2];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
            ab[nb] = sb + abase0[nb];
        xbs[0] = sb + xbase0[0];
        xbs[1] = sb + xbase0[1];
        i16x4 fa[2][4][2];
        u32x4 xv[2][BPW];
        stage_reads<BPW>(ab, xbs, fa, xv);
        // A slice of at most 32 channels (the last, when Cin is not a
        // multiple of 64) has nothing in its second k-step.
        const bool two = (t / a.taps) * 64 + 32 < a.Cin;
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            if (st == 1 && !two)
                break;
            bf16x8 wf[NB];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const i16x4 lo = fa[st][nb][0], hi = fa[st][nb][1];
                const i16x8 both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                wf[nb] = __builtin_bit_cast(bf16x8, both);
            }
#pragma unroll
            for (int b = 0; b < BPW; ++b)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    acc[b][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[nb], __builtin_bit_cast(bf16x8, xv[st][b]),
                                                                         acc[b][nb], 0, 0, 0);
        }
    }
    // Every loader's stages past the end have landed: the ring is free.
    lds_barrier();

    // Epilogue: lane holds channels o0 + 16nb + 4g + {0..3} of pixel
    // m0 + 16*(cw*BPW + b) + r.
    const __amdgpu_buffer_rsrc_t br = __builtin_amdgcn_make_buffer_rsrc(
        a.bias ? (void *)(a.bias + oc0) : (void *)a.F, 0, a.bias ? (int)a.b_records : 0, BUF_WORD3);
    u32x4 bq[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
        bq[nb] = __builtin_amdgcn_raw_buffer_load_b128(br, (uint32_t)((o0 + nb * 16 + g * 4) * 4), 0, 0);
    const int mw = m0 + 16 * cw * BPW;       // the wave's first pixel
    if constexpr (OUT_BF16) {
        uint8_t *patch = ring + cw * 16 * BPW * OPITCH;
#pragma unroll
        for (int b = 0; b < BPW; ++b)
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
        // 8i + L/8 of the wave's, channels 8*(L%8)..+7.
        const int ch = o0 + (lane & 7) * 8;
#pragma unroll
        for (int i = 0; i < 2 * BPW; ++i) {
            const int pp = i * 8 + (lane >> 3);
            const u32x4 w = *reinterpret_cast<const u32x4 *>(patch + pp * OPITCH + (lane & 7) * 16);
            const int m = mw + pp;
            if (m < a.m_total && ch < a.Cout) {
                const uint32_t ny = fdiv_g((uint32_t)m, a.div_wo);
                const int x = (int)((uint32_t)m - ny * (uint32_t)a.Wo);
                const uint32_t n = fdiv_g(ny, a.div_ho);
                const int y = (int)(ny - n * (uint32_t)a.Ho);
                char *yp = static_cast<char *>(a.Y) +
                           ((int64_t)n * a.ys0 + (int64_t)y * a.ys1 + (int64_t)x * a.ys2 + oc0 + ch) * 2;
                __builtin_nontemporal_store(w, reinterpret_cast<u32x4 *>(yp));
            }
        }
    } else {
#pragma unroll
        for (int b = 0; b < BPW; ++b) {
            const int m = mw + 16 * b + r;
            if (m >= a.m_total)
                continue;
            const uint32_t ny = fdiv_g((uint32_t)m, a.div_wo);
            const int x = (int)((uint32_t)m - ny * (uint32_t)a.Wo);
            const uint32_t n = fdiv_g(ny, a.div_ho);
            const int y = (int)(ny - n * (uint32_t)a.Ho);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const int ch = o0 + nb * 16 + g * 4;
                if (ch >= a.Cout)
                    continue;
                const f32x4 v = acc[b][nb];
                char *yp = static_cast<char *>(a.Y) +
                           ((int64_t)n * a.ys0 + (int64_t)y * a.ys1 + (int64_t)x * a.ys2 + oc0 + ch) * ESZ;
                *reinterpret_cast<f32x4 *>(yp) = f32x4{v[0] + __uint_as_float(bq[nb][0]), v[1] + __uint_as_float(bq[nb][1]),
                                                       v[2] + __uint_as_float(bq[nb][2]), v[3] + __uint_as_float(bq[nb][3])};
            }
        }
    }
}

// Pixel blocks per wave: the fewest rounds of at most 256 resident tiles
// (one per compute unit), weighted by the per-tile work BPW.
int pick_bpw(int64_t m_total, int64_t nt_all)
{
    int best = 4;
    int64_t best_cost = -1;
    for (int bpw = 2; bpw <= 5; ++bpw) {
        const int64_t tiles = (m_total + 64 * bpw - 1) / (64 * bpw) * nt_all;
        const int64_t cost = (tiles + 255) / 256 * bpw;
        if (best_cost < 0 || cost < best_cost || (cost == best_cost && bpw == 4)) {
            best = bpw;
            best_cost = cost;
        }
    }
    return best;
}

template <int BPW, bool OB>
hipError_t launch_gemm(const GemmArgs &a, unsigned grid, hipStream_t s)
{
    constexpr int lds = GShape<BPW>::LDS;
    const hipError_t attr = allow_lds<dense_gemm_mfma<BPW, OB>>(lds);
    if (attr != hipSuccess)
        return attr;
    hipLaunchKernelGGL((dense_gemm_mfma<BPW, OB>), dim3(grid), dim3(GT), lds, s, a);
    return hipGetLastError();
}

template <bool OB>
hipError_t launch_gemm_ob(const GemmArgs &a, int bpw, unsigned grid, hipStream_t s)
{
    switch (bpw) {
    case 2: return launch_gemm<2, OB>(a, grid, s);
    case 3: return launch_gemm<3, OB>(a, grid, s);
    case 5: return launch_gemm<5, OB>(a, grid, s);
    default: return launch_gemm<4, OB>(a, grid, s);
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
    const int64_t tiles = (m_total + 127) / 128 * ((cout_g + GN - 1) / GN) * p.groups;   // the smallest tile
    return m_total < (int64_t(1) << 31) - 320 && tiles * 8 < (int64_t(1) << 31);
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
    a.KH = p.KH;
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
    a.taps = p.KH * p.KW;
    a.nstages = a.taps * ((a.Cin + 63) / 64);
    a.m_total = p.N * p.Ho * p.Wo;
    a.n_tiles = (a.Cout + GN - 1) / GN;
    a.nt_all = a.n_tiles * p.groups;
    const int bpw = pick_bpw(a.m_total, a.nt_all);
    const int m_tiles = (a.m_total + 64 * bpw - 1) / (64 * bpw);
    a.tiles = m_tiles * a.nt_all;
    a.x_records = (uint32_t)(((int64_t)(p.N - 1) * p.xs[0] + (int64_t)(p.H - 1) * p.xs[1] +
                              (int64_t)(p.W - 1) * p.xs[2] + p.Cin) * 2);
    a.f_records = (uint32_t)((int64_t)p.KH * p.KW * a.Cin * p.Cout * 2);
    a.b_records = (uint32_t)(a.Cout * 4);
    a.div_wo = make_fastdiv_g((uint32_t)p.Wo);
    a.div_ho = make_fastdiv_g((uint32_t)p.Ho);
    const unsigned grid = (unsigned)((a.tiles + 7) / 8 * 8);
    return p.ydt == CONV_BF16 ? launch_gemm_ob<true>(a, bpw, grid, s) : launch_gemm_ob<false>(a, bpw, grid, s);
}

}  // namespace convfwd
