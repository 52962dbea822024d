// Dense NHWC cross-correlation, unit stride, bf16 operands, bf16 or fp32 output:
// an implicit GEMM on CDNA4 matrix cores whose whole band of input rows is
// requested from memory at the start and lands in LDS without passing
// through registers.
//
// Contract: "CMU DLSys Lecture 14: Convolutional Network Implementation",
// section 1 (Y[n,y,x,o] = sum over i,j,c of X[n,y+i,x+j,c] * F[i,j,c,o]);
// section 5 writes it as the patch matrix times F reshaped to
// (K*K*Cin) x Cout, and section 6 prices the copy that builds the patch
// matrix. Nothing here builds it: every patch fragment is an LDS read of a
// staged input row at a per-tap offset. Zero padding and groups follow
// "Convolution Is Wx+b Moving Across a Signal" ("Why 1D? Why 2D?" and "Find
// the same sum in CKE's C kernels").
//
// Why this shape of kernel. A workgroup owns a band of R output rows x 64
// output channels, one per compute unit, so each unit must pull the whole
// filter slice (K*K*Cin x 64) and R + K - 1 input rows before it is done.
// Time spent waiting for the filter is time in which memory sits idle
// unless the input rows are already on their way. So:
//  * every input row of the band is requested within the first two steps,
//    with buffer loads that write straight into LDS (no registers held, no
//    commit instructions); each step waits only for the row it is about to
//    read;
//  * the filter slice is requested one filter row (K taps) at a time: row 0
//    and input rows 0-1 first (a barrier then makes every wave put these in
//    the memory pipeline before any wave asks for more), then input row 2
//    and the other filter rows, input rows 3-5 at the start of step 0 and
//    the last rows at the start of step 1, so that the memory system serves
//    the rows needed first ahead of the later ones (all at once, they land
//    together at the end). The first step needs only filter row 0 and input
//    rows 0-1, so
//    the matrix cores start after about a third of the filter has arrived
//    instead of all of it. Filter row i is staged in LDS at step i - 1 and
//    read into registers (gfx950 transpose read) at step i; two staging
//    areas alternate.
//
// Work decomposition (one workgroup = 8 waves = 512 threads, 2 per SIMD):
//  * Wave w keeps the 32-channel half (w & 1) of the tile's filter as A
//    operands of v_mfma_f32_16x16x32_bf16 and the 16-pixel block w >> 1 of
//    every output row (rows are at most 64 pixels wide).
//  * Step r reads input row r's X fragments (8 channels of one pixel per
//    lane, 16 bytes) once and feeds them to every output row that uses that
//    input row: K output rows accumulate at once, 2K independent chains per
//    wave. The next row's fragments are read during the current row's
//    MFMAs.
//  * For bf16 outputs the tile's output channels are staged in LDS in an
//    order that gives each lane 8 consecutive channels of one pixel across
//    its two 16-row MFMA blocks: MFMA row 4g + k of block nb is channel
//    8g + 4nb + k of the wave's 32. A finished output row is converted to
//    bf16 (round to nearest even) and stored straight from the accumulators
//    as 16 bytes per lane, with no trip through LDS: the four lanes of a
//    pixel write one 64-byte run (half a cache line; the other half is the
//    other wave's). fp32 outputs keep the plain order (row m of block nb is
//    channel 16nb + m), so that each store instruction writes 64-byte runs
//    (4 channels per lane); with the bf16 order each would leave gaps and
//    write partial lines, measured 1.6x slower. Stores carry the sc1 and
//    nt cache policies (device scope, streaming): on the 3x3 layers 12%
//    faster than the default policy and 2-4% faster than sc1 alone; 32-byte
//    runs (8 bytes per lane) take 1.6x as long as whole lines.
//  * Only the first few steps end with a barrier (filter rows staged, input
//    rows published); the last of them waits for every input row, after
//    which the waves run to the end without synchronising.
//
// LDS layout of a staged input row: 512 units of 16 bytes (8 channels), one
// per thread of the loading instruction. Pixel slot p holds its channel
// chunk c in unit p*CG + (c ^ ((p >> SH) & (CG - 1))), CG = Cin_padded / 8.
// The XOR swizzle gives the 16 lanes that read one chunk of 16 consecutive
// pixels 16 distinct 16-byte bank groups (all 64 banks), with no padding
// between pixels, so the loading instruction can write 1 KB contiguously.
// Slots left or right of the image and channels past Cin load as zeros.
//
// Memory-count bookkeeping. Loads into LDS are not visible to the
// compiler's dependency tracking once issued, so the steps that publish
// input rows wait with an explicit vmcnt: the number of memory instructions
// this wave issued after that row's load (later rows, later filter rows,
// output stores so far), all known at compile time because every memory
// instruction is unconditional (out-of-range lanes use an offset the
// hardware drops).
// Barriers are plain s_barrier after lgkmcnt(0): a workgroup fence would
// wait for every load still in flight.
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

constexpr int BT = 512;                  // threads per workgroup
constexpr int TILE_O = 64;               // output channels per tile
constexpr int NBW = 2;                   // 16-channel column blocks per wave
static_assert(NBW == 2, "a lane's two blocks hold the 8 channels of one 16-byte store");
constexpr int ROW_UNITS = 512;           // 16-byte units per staged input row
constexpr int ROW_BYTES = ROW_UNITS * 16;
constexpr int FPITCH = TILE_O + 8;       // LDS pitch of a staged filter row of 64 outputs (elements)
constexpr int LDS_MAX = 160 * 1024;
constexpr uint32_t OOB = 0x80000000u;    // buffer offset past every range: access dropped
constexpr int BUF_WORD3 = 0x00020000;    // raw buffer descriptor word 3 (gfx9 family)

struct BandArgs {
    const uint16_t *X;
    const uint16_t *F;
    const float *bias;
    void *Y;            // bf16 or fp32 (the kernel's OUT_BF16)
    int64_t xs0, xs1, xs2, ys0, ys1, ys2;
    int H, W, Ho, Wo;
    int Cin, Cout;      // channels of one group (input, output)
    int f_ld;           // F row length: output channels of all groups
    int gpack;          // 0, or the channels of one true group packed into a tile
    int pt, pl;         // zero rows / columns before the input
    int R;              // output rows per band
    int bands_per_img;
    int bands;          // N * bands_per_img (the grid may hold more: those exit)
    int tiles;          // 64-channel output tiles per group
    int groups;
    int row_slots;      // pixel slots of a staged row (zero padding included)
    uint32_t x_records; // bytes addressable from one image's base in X
    uint32_t y_records; // bytes addressable from one image's base in Y
};

// Explicit waits. "memory" keeps the compiler from moving LDS accesses
// across them.
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt holds 6 bits");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

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

template <int KH, int KW, int CS, int NR, int LS, bool OUT_BF16, int LR, int LT, bool GS>
struct BandShape {
    static constexpr int CINP = 32 * CS;
    // Small groups packed block-diagonally into a 64-channel tile (GS): the
    // 32 output channels of wave half h belong to the groups whose inputs are
    // channels 32h..32h+31, so the wave runs only that channel step of each
    // tap; the other step's filter entries are all zero.
    static_assert(!GS || CS == 2, "packed groups fill a 64-channel tile");
    static constexpr int CSW = GS ? 1 : CS;                 // channel steps per tap a wave runs
    static constexpr int CG = CINP / 8;                     // 16-byte units per pixel
    static constexpr int SH = CS == 2 ? 1 : 2;              // log2(pixels per 256 bytes)
    static constexpr int FROW = KW * CINP * FPITCH;         // elements of one staged filter row
    static constexpr int FITEMS = (KW * CINP * 8 + BT - 1) / BT;  // 16-byte filter loads per thread per filter row
    static constexpr int KSR = KW * CSW;                    // k-steps per filter row and wave
    static constexpr int TRN = KSR * NBW * 2;               // transposed reads per filter row
    static constexpr int RMAX = NR - KH + 1;                // output rows a band holds
    static constexpr int EARLY = NR < 3 ? NR : 3;           // input rows requested before filter rows 1..KH-1
    static constexpr int OSTORE = OUT_BF16 ? 1 : NBW;       // store instructions per output row and wave
    static constexpr int LAST_SYNC = LS;                    // last step that ends with a barrier
    static_assert(LS >= KH - 1 && LS + 2 < NR, "filter rows are staged at barriers; rows past LS + 1 exist");
    // Late rows LR..NR-1 go out at the start of step LT: each must be
    // requested before the step that waits for it.
    static_assert(LR == NR || (LR >= EARLY && LT >= 1 && LT <= LR - 2 && LT <= LS),
                  "a late row is waited for before it is requested");
    // Step at whose start input row q is requested (-1: the prologue).
    static constexpr int issue_step(int q) { return q < EARLY ? -1 : q < LR ? 0 : LT; }
    static constexpr size_t LDS = (size_t)2 * FROW * 2 + (size_t)NR * ROW_BYTES;

    // Output rows stored by the end of step r: row t completes (and is
    // stored) at step t + KH - 1.
    static constexpr int stores_by(int r)
    {
        const int s = r - KH + 2;
        return s < 0 ? 0 : s > RMAX ? RMAX : s;
    }
    // Memory instructions a wave has issued after input row q's load, by
    // the end of step r (r >= 0), or in the prologue (r = -1). Issue order:
    // bias, filter row 0, input rows 0 and 1, a barrier (every wave's first
    // loads reach the memory pipeline before any wave's later ones), input
    // rows 2..EARLY-1, filter rows 1..KH-1; input rows EARLY..LR-1 at the
    // start of step 0 and rows LR..NR-1 at the start of step LT; one output
    // row's stores (OSTORE instructions) at each step from KH-1 on.
    static constexpr int after_row(int q, int r)
    {
        int n = 0;
        for (int k = q + 1; k < NR; ++k)                    // later rows requested by then
            n += issue_step(k) <= r ? 1 : 0;
        if (q < EARLY)
            n += FITEMS * (KH - 1);                         // filter rows 1..KH-1
        if (r >= 0) {                                       // stores of the steps from q's request on
            const int s0 = issue_step(q);
            n += OSTORE * (stores_by(r) - (s0 <= 0 ? 0 : stores_by(s0 - 1)));
        }
        return n;
    }
};

// The transposed reads of filter row i (TRN of them, 8 bytes each) in one
// asm block that ends with a wait for all of them. The compiler cannot tell
// that these LDS reads never touch the input rows still being loaded into
// LDS, and would wait for every one of those loads before a transposed-read
// intrinsic; issued from asm, they wait only for themselves. Read q =
// (kk * NBW + nb) * 2 + h is at byte offset tr_off(q) from the lane's base.
// The outputs are early-clobber: a read that returns while later reads of
// the block are still to issue must not land in the address register.
template <class B, int I>
struct TrOff {
    static constexpr int at(int q)
    {
        const int h = q & 1, nb = (q >> 1) % NBW, kk = q / (2 * NBW);
        const int j = kk / B::CSW, cs = kk % B::CSW;
        return (I & 1) * B::FROW * 2 + ((j * B::CINP + cs * 32 + h * 4) * FPITCH + nb * 16) * 2;
    }
};

#define CF_TR(o, f) "ds_read_b64_tr_b16 %" #o ", %[a] offset:%" #f "\n\t"

template <class B, int I>
__device__ __forceinline__ void tr_reads(uint32_t base, i16x4 (&p)[B::TRN])
{
    using T = TrOff<B, I>;
    static_assert(T::at(B::TRN - 1) < 65536, "ds offsets are 16 bits");
    if constexpr (B::TRN == 24) {
        asm volatile(CF_TR(0, 25) CF_TR(1, 26) CF_TR(2, 27) CF_TR(3, 28) CF_TR(4, 29) CF_TR(5, 30)
                     CF_TR(6, 31) CF_TR(7, 32) CF_TR(8, 33) CF_TR(9, 34) CF_TR(10, 35) CF_TR(11, 36)
                     CF_TR(12, 37) CF_TR(13, 38) CF_TR(14, 39) CF_TR(15, 40) CF_TR(16, 41) CF_TR(17, 42)
                     CF_TR(18, 43) CF_TR(19, 44) CF_TR(20, 45) CF_TR(21, 46) CF_TR(22, 47) CF_TR(23, 48)
                     "s_waitcnt lgkmcnt(0)"
                     : "=&v"(p[0]), "=&v"(p[1]), "=&v"(p[2]), "=&v"(p[3]), "=&v"(p[4]), "=&v"(p[5]), "=&v"(p[6]),
                       "=&v"(p[7]), "=&v"(p[8]), "=&v"(p[9]), "=&v"(p[10]), "=&v"(p[11]), "=&v"(p[12]), "=&v"(p[13]),
                       "=&v"(p[14]), "=&v"(p[15]), "=&v"(p[16]), "=&v"(p[17]), "=&v"(p[18]), "=&v"(p[19]),
                       "=&v"(p[20]), "=&v"(p[21]), "=&v"(p[22]), "=&v"(p[23])
                     : [a] "v"(base), "n"(T::at(0)), "n"(T::at(1)), "n"(T::at(2)), "n"(T::at(3)), "n"(T::at(4)),
                       "n"(T::at(5)), "n"(T::at(6)), "n"(T::at(7)), "n"(T::at(8)), "n"(T::at(9)), "n"(T::at(10)),
                       "n"(T::at(11)), "n"(T::at(12)), "n"(T::at(13)), "n"(T::at(14)), "n"(T::at(15)),
                       "n"(T::at(16)), "n"(T::at(17)), "n"(T::at(18)), "n"(T::at(19)), "n"(T::at(20)),
                       "n"(T::at(21)), "n"(T::at(22)), "n"(T::at(23))
                     : "memory");
    } else {
        static_assert(B::TRN == 12, "filter rows of 3 taps by 1 or 2 channel steps");
        asm volatile(CF_TR(0, 13) CF_TR(1, 14) CF_TR(2, 15) CF_TR(3, 16) CF_TR(4, 17) CF_TR(5, 18)
                     CF_TR(6, 19) CF_TR(7, 20) CF_TR(8, 21) CF_TR(9, 22) CF_TR(10, 23) CF_TR(11, 24)
                     "s_waitcnt lgkmcnt(0)"
                     : "=&v"(p[0]), "=&v"(p[1]), "=&v"(p[2]), "=&v"(p[3]), "=&v"(p[4]), "=&v"(p[5]), "=&v"(p[6]),
                       "=&v"(p[7]), "=&v"(p[8]), "=&v"(p[9]), "=&v"(p[10]), "=&v"(p[11])
                     : [a] "v"(base), "n"(T::at(0)), "n"(T::at(1)), "n"(T::at(2)), "n"(T::at(3)), "n"(T::at(4)),
                       "n"(T::at(5)), "n"(T::at(6)), "n"(T::at(7)), "n"(T::at(8)), "n"(T::at(9)), "n"(T::at(10)),
                       "n"(T::at(11))
                     : "memory");
    }
}

#undef CF_TR

template <int KH, int KW, int CS, int NR, int SAUX, int LS, bool OUT_BF16, int LR, int LT, bool GS>
__global__ __launch_bounds__(BT) __attribute__((amdgpu_waves_per_eu(2, 2)))
void dense_band_mfma(BandArgs a)
{
    using B = BandShape<KH, KW, CS, NR, LS, OUT_BF16, LR, LT, GS>;
    constexpr int ESZ = OUT_BF16 ? 2 : 4;
    constexpr int CINP = B::CINP;
    constexpr int CG = B::CG;
    constexpr int KSR = B::KSR;
    constexpr int RMAX = B::RMAX;
    static_assert(KH == 3 && KW == 3, "filter rows alternate between two staging areas");
    static_assert(B::LDS <= (size_t)LDS_MAX, "band does not fit in LDS");

    extern __shared__ __align__(16) uint8_t smem[];
    uint16_t *farea = reinterpret_cast<uint16_t *>(smem);        // two staged filter rows
    uint8_t *xrows = smem + 2 * B::FROW * 2;                       // NR staged input rows

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int half = wave & 1;
    const int pg = wave >> 1;
    // Workgroups are dealt to the 8 XCDs round robin by launch order (slot s
    // runs on XCD s % 8). Slot s takes band (s % 8) * (bands/8) + (s/8) /
    // tiles and tile (s/8) % tiles, so all tiles of a band and neighbouring
    // bands of an image share one XCD's L2 (the halo rows meet there).
    const int bid = with_args_loaded((int)blockIdx.x, a);
    const int tiles_all = a.tiles * a.groups;
    const int slot_in_xcd = bid >> 3;
    const int band = (bid & 7) * (int)(gridDim.x >> 3) / tiles_all + slot_in_xcd / tiles_all;
    const int tile = slot_in_xcd % tiles_all;
    const int grp = tile / a.tiles;
    const int o0 = (tile - grp * a.tiles) * TILE_O;
    const int xc0 = grp * a.Cin;
    const int oc0 = grp * a.Cout;
    if (band >= a.bands)
        return;
    const int n = band / a.bands_per_img;
    const int y0 = (band - n * a.bands_per_img) * a.R;
    if (y0 >= a.Ho)
        return;
    const int y1 = min(y0 + a.R, a.Ho);
    const int iy0 = y0 - a.pt;                         // input row of step 0
    const int iy_end = min(a.H, y1 - 1 - a.pt + KH);   // one past the last input row the band reads

    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(a.X + (int64_t)n * a.xs0 + xc0), 0, (int)(a.x_records - xc0 * 2), BUF_WORD3);
    const __amdgpu_buffer_rsrc_t yr = __builtin_amdgcn_make_buffer_rsrc(
        static_cast<char *>(a.Y) + ((int64_t)n * a.ys0 + oc0) * ESZ, 0, (int)(a.y_records - oc0 * ESZ), BUF_WORD3);
    const int fcin = a.gpack ? a.gpack : a.Cin;        // F rows per tap
    const __amdgpu_buffer_rsrc_t fr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(a.F), 0, KH * KW * fcin * a.f_ld * 2, BUF_WORD3);

    // Filter row i: load item it = tid + t*BT -> (8-output group og
    // fastest, then input channel c, then tap column j), eight lanes per
    // 128-byte row of F. Everything but the tap is fixed per thread: item t
    // reads tap column fj0 + t*JSTEP, channel fc, outputs o0 + 8*(tid & 7).
    // With small groups packed into the tile (gpack = G), entries between
    // different true groups are the zeros of the block-diagonal filter.
    constexpr int JSTEP = (BT / 8) / CINP;
    static_assert(JSTEP >= 1 && (BT / 8) % CINP == 0, "an item round covers whole taps");
    const int fog = tid & 7;
    const int fc = (tid >> 3) % CINP;
    const int fj0 = (tid >> 3) / CINP;
    const int fo = o0 + fog * 8;
    const bool fok = fc < a.Cin && fo < a.Cout && (a.gpack == 0 || fc / a.gpack == fo / a.gpack);
    const uint32_t fgoff = (uint32_t)(((a.gpack ? fc % a.gpack : fc) * a.f_ld + oc0 + fo) * 2);
    const uint32_t ftap = (uint32_t)(fcin * a.f_ld * 2);      // bytes per tap
    u32x4 fv[KH][B::FITEMS];
    auto issue_frow = [&](const int i) __attribute__((always_inline)) {
#pragma unroll
        for (int t = 0; t < B::FITEMS; ++t) {
            const int j = fj0 + t * JSTEP;
            fv[i][t] = __builtin_amdgcn_raw_buffer_load_b128(
                fr, (fok && j < KW) ? fgoff + (uint32_t)(i * KW + j) * ftap : OOB, 0, 0);
        }
    };
    // bf16 outputs: channels 8g + 4nb + k of a 32-channel half (g = fog % 4)
    // sit in staged column 16nb + 4g + k of that half, which the MFMA blocks
    // read as row 4g + k of block nb: the item's two 4-channel halves go to
    // columns 4g and 16 + 4g. fp32 outputs: columns in channel order.
    const int fcol = OUT_BF16 ? (fog >> 2) * 32 + (fog & 3) * 4 : fog * 8;
    auto commit_frow = [&](const int i) __attribute__((always_inline)) {
        uint16_t *ft = farea + (i & 1) * B::FROW;
#pragma unroll
        for (int t = 0; t < B::FITEMS; ++t) {
            const int j = fj0 + t * JSTEP;
            if (j < KW) {
                uint16_t *at = ft + (j * CINP + fc) * FPITCH + fcol;
                if constexpr (OUT_BF16) {
                    *reinterpret_cast<u32x2 *>(at) = u32x2{fv[i][t][0], fv[i][t][1]};
                    *reinterpret_cast<u32x2 *>(at + 16) = u32x2{fv[i][t][2], fv[i][t][3]};
                } else {
                    *reinterpret_cast<u32x4 *>(at) = fv[i][t];
                }
            }
        }
    };
    // A fragments of filter row i (k-steps i*KSR ..). Within each 16-lane
    // group of ds_read_b64_tr_b16, output lane i gets element i % 4 of the
    // 8-byte chunk addressed by lane 4j + i/4: lane r addresses row r/4,
    // columns 4*(r%4)..+3 of a 4-row block and receives four consecutive
    // input channels of output channel r % 16 (the A-operand layout); two
    // reads give the lane's 8 channels. All reads of a filter row go out in
    // one block with one wait (see tr_reads). With packed groups the wave's
    // channel step (32 * half) is part of the base.
    bf16x8 wf[KH * KSR][NBW];
    const uint32_t fbase = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint16_t *)farea +
                           (uint32_t)((((lane >> 4) * 8 + ((lane & 15) >> 2) + (GS ? half * 32 : 0)) * FPITCH +
                                       half * 32 + 4 * (lane & 3)) * 2);
    auto read_frow = [&](auto I) __attribute__((always_inline)) {
        constexpr int i = decltype(I)::value;
        i16x4 p[B::TRN];
        tr_reads<B, i>(fbase, p);
#pragma unroll
        for (int kk = 0; kk < KSR; ++kk)
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb) {
                const i16x4 lo = p[(kk * NBW + nb) * 2];
                const i16x4 hi = p[(kk * NBW + nb) * 2 + 1];
                const i16x8 both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                wf[i * KSR + kk][nb] = __builtin_bit_cast(bf16x8, both);
            }
    };

    // Input row r into LDS: thread tid moves unit tid of the row (pixel slot
    // tid / CG, swizzled chunk); the instruction of wave w writes bytes
    // [1024 w, 1024 w + 1024) of the row. The offset is a select, never a
    // branch, so every wave issues exactly one instruction per row.
    const int dpx = tid / CG;
    const int dc = (tid % CG) ^ ((dpx >> B::SH) & (CG - 1));
    const int dix = dpx - a.pl;
    const bool col_ok = dpx < a.row_slots && dix >= 0 && dix < a.W && dc * 8 < a.Cin;
    const uint32_t col_off = col_ok ? (uint32_t)(((int64_t)dix * a.xs2 + dc * 8) * 2) : 0u;
    auto dma_row = [&](const int r) __attribute__((always_inline)) {
        const int iy = iy0 + r;
        const bool row_ok = iy >= 0 && iy < iy_end;
        const uint32_t row_off = row_ok ? (uint32_t)((int64_t)iy * a.xs1 * 2) : 0u;
        const uint32_t off = (col_ok && row_ok) ? row_off + col_off : OOB;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            xr, (__attribute__((address_space(3))) void *)(xrows + r * ROW_BYTES + wave * 1024), 16, off, 0, 0, 0);
    };

    // Bias of the 4 output channels of each MFMA block a lane's results
    // belong to (zeros without bias): 32*half + 8*(lane/16) + 4*nb + {0..3}
    // for bf16 outputs, 32*half + 16*nb + 4*(lane/16) + {0..3} for fp32.
    u32x4 bq[NBW];
    auto issue_bias = [&]() __attribute__((always_inline)) {
        const __amdgpu_buffer_rsrc_t br = __builtin_amdgcn_make_buffer_rsrc(
            a.bias ? (void *)(a.bias + oc0) : (void *)a.F, 0, a.bias ? a.Cout * 4 : 0, BUF_WORD3);
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb)
            bq[nb] = __builtin_amdgcn_raw_buffer_load_b128(
                br, (uint32_t)((o0 + half * 32 + (OUT_BF16 ? (lane >> 4) * 8 + nb * 4 : nb * 16 + (lane >> 4) * 4)) * 4),
                0, 0);
    };

    // Issue order (the vmcnt bookkeeping in BandShape::after_row depends on
    // it; the scheduling fences keep the compiler from reordering).
    issue_bias();
    issue_frow(0);
    __builtin_amdgcn_sched_barrier(0);
    static_for<0, 2>([&](auto R) { dma_row(decltype(R)::value); });
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_barrier" ::: "memory");
    static_for<2, B::EARLY>([&](auto R) { dma_row(decltype(R)::value); });
    __builtin_amdgcn_sched_barrier(0);
    static_for<1, KH>([&](auto I) { issue_frow(decltype(I)::value); });
    __builtin_amdgcn_sched_barrier(0);

    // Filter row 0 into LDS, input rows 0 and 1 landed, then the first
    // fragments.
    commit_frow(0);
    wait_vmcnt<B::after_row(NR > 1 ? 1 : 0, -1)>();
    lds_barrier();
    read_frow(std::integral_constant<int, 0>{});

    // X fragments of staged row r for this wave's 16-pixel block: for each
    // tap column j and 32-channel step, lane (g, p) reads chunk 4*cs + g of
    // pixel slot x + j (x = its output pixel, clamped into the row). With
    // packed groups the wave's one step is cs = half.
    const int x = pg * 16 + (lane & 15);
    const int xl = min(x, a.Wo - 1);
    auto read_x = [&](const int r, bf16x8 (&xb)[KSR]) __attribute__((always_inline)) {
        const uint8_t *row = xrows + r * ROW_BYTES;
#pragma unroll
        for (int jc = 0; jc < KSR; ++jc) {
            const int j = jc / B::CSW;
            const int cs = GS ? half : jc % B::CSW;
            const int p = xl + j;
            const int c = cs * 4 + (lane >> 4);
            const int unit = p * CG + (c ^ ((p >> B::SH) & (CG - 1)));
            xb[jc] = *reinterpret_cast<const bf16x8 *>(row + unit * 16);
        }
    };
    bf16x8 xn[KSR];
    read_x(0, xn);

    // Store target of this lane: pixel pg*16 + lane % 16, channels
    // 32*half + 8*(lane/16) .. +7 (block nb holds the 4 from 4*nb).
    const int xs_px = pg * 16 + (lane & 15);
    const int xs_ch = o0 + half * 32 + (lane >> 4) * 8;
    const bool xs_ok = xs_px < a.Wo && xs_ch < a.Cout;
    const int64_t xs_off = (int64_t)xs_px * a.ys2 + xs_ch;

    f32x4 acc[KH][NBW];
#pragma unroll
    for (int s = 0; s < KH; ++s)
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb)
            acc[s][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Output row t is complete: bias, conversion, store; its accumulators
    // are cleared for the row that reuses the slot.
    auto store_row = [&](auto TT) __attribute__((always_inline)) {
        constexpr int t = decltype(TT)::value;
        const int yo = y0 + t;
        if constexpr (!OUT_BF16) {
            // Channels 32*half + 16*nb + 4*(lane/16) + {0..3} of pixel x, 16
            // fp32 bytes: the four lanes of a pixel write one 64-byte run.
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb) {
                const f32x4 v = acc[t % KH][nb];
                const u32x4 w = {__float_as_uint(v[0] + __uint_as_float(bq[nb][0])),
                                 __float_as_uint(v[1] + __uint_as_float(bq[nb][1])),
                                 __float_as_uint(v[2] + __uint_as_float(bq[nb][2])),
                                 __float_as_uint(v[3] + __uint_as_float(bq[nb][3]))};
                const int ch = o0 + half * 32 + nb * 16 + (lane >> 4) * 4;
                const bool okc = x < a.Wo && ch < a.Cout && yo < y1;
                const uint32_t off =
                    okc ? (uint32_t)(((int64_t)yo * a.ys1 + (int64_t)x * a.ys2 + ch) * 4) : OOB;
                __builtin_amdgcn_raw_buffer_store_b128(w, yr, off, 0, SAUX);
                acc[t % KH][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        } else {
            // 8 bf16 channels, one 16-byte store.
            const bool ok = xs_ok && yo < y1;
            u32x4 w;
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb) {
                const f32x4 v = acc[t % KH][nb];
                w[2 * nb] = pack_bf16x2(v[0] + __uint_as_float(bq[nb][0]), v[1] + __uint_as_float(bq[nb][1]));
                w[2 * nb + 1] = pack_bf16x2(v[2] + __uint_as_float(bq[nb][2]), v[3] + __uint_as_float(bq[nb][3]));
                acc[t % KH][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
            const uint32_t off = ok ? (uint32_t)(((int64_t)yo * a.ys1 + xs_off) * 2) : OOB;
            __builtin_amdgcn_raw_buffer_store_b128(w, yr, off, 0, SAUX);
        }
    };

    // Step r: input row r feeds output rows t = r - i for filter rows i;
    // output row t accumulates in slot t % KH (taps in ascending i, then j,
    // then channel step) and is complete at step t + KH - 1. The MFMAs of a
    // step run with the tap column outermost, so the KH output rows' 2*KH
    // accumulation chains interleave. Rows past the end of a short band are
    // computed from zero rows and never stored.
    //
    // Steps up to LAST_SYNC end with a barrier: filter rows 1..KH-1 are
    // staged there, and each step publishes the input row the next step
    // reads. The last of them waits for every input row, so the remaining
    // steps need no barrier at all and the waves run freely to the end.
    static_for<0, NR>([&](auto RR) {
        constexpr int r = decltype(RR)::value;
        if constexpr (r == 0) {
            __builtin_amdgcn_sched_barrier(0);
            static_for<B::EARLY, LR>([&](auto R) { dma_row(decltype(R)::value); });
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (LR < NR && r == LT) {
            __builtin_amdgcn_sched_barrier(0);
            static_for<LR, NR>([&](auto R) { dma_row(decltype(R)::value); });
            __builtin_amdgcn_sched_barrier(0);
        }
        bf16x8 xb[KSR];
#pragma unroll
        for (int jc = 0; jc < KSR; ++jc)
            xb[jc] = xn[jc];
        if constexpr (r + 1 < NR)
            read_x(r + 1, xn);
        // Filter rows already in registers first (all of them from step
        // KH on; rows 0..r-1 at step r < KH, row 0 at step 0), then, at
        // steps 1..KH-1, filter row r once its fragments are read.
        constexpr int IA = r < 1 ? 1 : r < KH ? r : KH;
#pragma unroll
        for (int jc = 0; jc < KSR; ++jc)
#pragma unroll
            for (int i = 0; i < IA; ++i) {
                const int t = r - i;
                if (t >= 0 && t < RMAX) {
#pragma unroll
                    for (int nb = 0; nb < NBW; ++nb)
                        acc[t % KH][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            wf[i * KSR + jc][nb], xb[jc], acc[t % KH][nb], 0, 0, 0);
                }
            }
        if constexpr (r >= 1 && r < KH) {
            read_frow(std::integral_constant<int, r>{});
            // Filter row r feeds output row 0 only.
#pragma unroll
            for (int jc = 0; jc < KSR; ++jc)
#pragma unroll
                for (int nb = 0; nb < NBW; ++nb)
                    acc[0][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        wf[r * KSR + jc][nb], xb[jc], acc[0][nb], 0, 0, 0);
        }
        if constexpr (r + 1 < KH)
            commit_frow(r + 1);
        if constexpr (r >= KH - 1 && r - (KH - 1) < RMAX)
            store_row(std::integral_constant<int, r - (KH - 1)>{});
        if constexpr (r < B::LAST_SYNC) {
            // Row r + 2 is read (as the next row's fragments) during step r + 1.
            wait_vmcnt<B::after_row(r + 2, r)>();
            lds_barrier();
        } else if constexpr (r == B::LAST_SYNC) {
            wait_vmcnt<B::after_row(NR - 1, r)>();
            lds_barrier();
        }
    });
}

// Defaults measured on the 3x3 layers: rows 6..8 requested at step 1 (so
// that rows 3..5 reach the memory system first), barriers through step 3,
// stores with the sc1 and nt policies (SAUX = 16 | 2).
template <int KH, int KW, int CS, int NR, bool OB, bool GS = false, int SAUX = 18, int LS = 3, int LR = 6, int LT = 1>
hipError_t launch_band(const BandArgs &a, dim3 grid, hipStream_t s)
{
    auto kern = dense_band_mfma<KH, KW, CS, NR, SAUX, LS, OB, LR, LT, GS>;
    constexpr size_t lds = BandShape<KH, KW, CS, NR, LS, OB, LR, LT, GS>::LDS;
    const hipError_t attr = allow_lds<dense_band_mfma<KH, KW, CS, NR, SAUX, LS, OB, LR, LT, GS>>((int)lds);
    if (attr != hipSuccess)
        return attr;
    hipLaunchKernelGGL(kern, grid, dim3(BT), lds, s, a);
    return hipGetLastError();
}

constexpr int BAND_NR = 9;   // input rows per band (R <= 7 output rows for a 3-row filter)

struct BandPlan {
    int CS, R, slots;
};

bool plan_band(const DenseProblem &p, BandPlan *plan)
{
    if (p.xdt != CONV_BF16)
        return false;
    const int yesz = p.ydt == CONV_BF16 ? 2 : 4;
    if (p.sh != 1 || p.sw != 1 || p.dh != 1 || p.dw != 1)
        return false;
    if (p.KH != 3 || p.KW != 3)
        return false;
    const int cin_g = p.Cin / p.groups, cout_g = p.Cout / p.groups;
    if (cin_g % 8 != 0 || cout_g % 8 != 0 || cin_g > 64)
        return false;
    if ((uintptr_t)p.X % 16 != 0 || p.xs[0] % 8 != 0 || p.xs[1] % 8 != 0 || p.xs[2] % 8 != 0)
        return false;
    if ((uintptr_t)p.F % 16 != 0 || (int64_t)p.KH * p.KW * cin_g * p.Cout * 2 >= (int64_t(1) << 31))
        return false;
    // Output pieces are 16 bytes: 8 bf16 or 4 fp32 channels.
    const int yvec = 16 / yesz;
    if ((uintptr_t)p.Y % 16 != 0 || p.ys[0] % yvec != 0 || p.ys[1] % yvec != 0 || p.ys[2] % yvec != 0)
        return false;
    // Buffer offsets are 32-bit: one image of X and of Y must stay below 2 GB.
    auto extent = [](const int64_t *s, int rows, int cols, int ch, int esz) {
        return ((int64_t)(rows - 1) * s[1] + (int64_t)(cols - 1) * s[2] + ch) * esz;
    };
    if (extent(p.xs, p.H, p.W, p.Cin, 2) >= (int64_t(1) << 31) ||
        extent(p.ys, p.Ho, p.Wo, p.Cout, yesz) >= (int64_t(1) << 31))
        return false;
    if (p.Wo > 64)
        return false;
    const int CS = cin_g <= 32 ? 1 : 2;
    const int need = p.Wo - 1 + p.KW;
    const int slots = need > p.pl + p.W ? need : p.pl + p.W;
    if (slots * 4 * CS > ROW_UNITS)
        return false;
    const int rmax = BAND_NR - p.KH + 1;
    const int tiles = (cout_g + TILE_O - 1) / TILE_O * p.groups;
    int want = (int)((256 + (int64_t)p.N * tiles - 1) / ((int64_t)p.N * tiles));
    want = want < 1 ? 1 : want > p.Ho ? p.Ho : want;
    const int R = (p.Ho + want - 1) / want;
    plan->CS = CS;
    plan->R = R < rmax ? R : rmax;
    plan->slots = slots;
    return true;
}

}  // namespace

bool dense_band_supports(const DenseProblem &p)
{
    BandPlan plan;
    return plan_band(p, &plan);
}

hipError_t launch_dense_band(const DenseProblem &p, int gpack, hipStream_t s)
{
    BandPlan plan;
    if (!plan_band(p, &plan))
        return hipErrorNotSupported;
    BandArgs a;
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
    a.Cin = p.Cin / p.groups;
    a.Cout = p.Cout / p.groups;
    a.f_ld = p.Cout;
    a.gpack = gpack;
    a.pt = p.pt;
    a.pl = p.pl;
    a.R = plan.R;
    a.bands_per_img = (p.Ho + a.R - 1) / a.R;
    a.bands = p.N * a.bands_per_img;
    a.tiles = (a.Cout + TILE_O - 1) / TILE_O;
    a.groups = p.groups;
    a.row_slots = plan.slots;
    a.x_records = (uint32_t)(((int64_t)(p.H - 1) * p.xs[1] + (int64_t)(p.W - 1) * p.xs[2] + p.Cin) * 2);
    const int yesz = p.ydt == CONV_BF16 ? 2 : 4;
    a.y_records = (uint32_t)(((int64_t)(p.Ho - 1) * p.ys[1] + (int64_t)(p.Wo - 1) * p.ys[2] + p.Cout) * yesz);
    const int64_t slots = (int64_t)((a.bands + 7) / 8 * 8) * a.tiles * a.groups;
    if (slots >= (int64_t(1) << 31))
        return hipErrorNotSupported;
    const dim3 grid((unsigned)slots);
    if (gpack != 0) {
        // pack_groups makes 64-channel tiles: two channel steps per tap.
        if (plan.CS != 2 || a.Cin != 64 || a.Cout != 64)
            return hipErrorNotSupported;
        return p.ydt == CONV_BF16 ? launch_band<3, 3, 2, BAND_NR, true, true>(a, grid, s)
                                  : launch_band<3, 3, 2, BAND_NR, false, true>(a, grid, s);
    }
    if (p.ydt == CONV_BF16)
        return plan.CS == 1 ? launch_band<3, 3, 1, BAND_NR, true>(a, grid, s)
                            : launch_band<3, 3, 2, BAND_NR, true>(a, grid, s);
    return plan.CS == 1 ? launch_band<3, 3, 1, BAND_NR, false>(a, grid, s)
                        : launch_band<3, 3, 2, BAND_NR, false>(a, grid, s);
}

}  // namespace convfwd
