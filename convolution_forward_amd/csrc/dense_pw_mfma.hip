// Pointwise (1x1) dense convolution as a plain GEMM on CDNA4 matrix cores:
// Y[p, o] = sum over c of X[p, c] * F[0, 0, c, o] for every pixel p of the
// batch, bf16 operands, fp32 accumulation, bf16 or fp32 output.
//
// Contract: "CMU DLSys Lecture 14: Convolutional Network Implementation",
// section 2: with a 1x1 filter the convolution is one matrix product of the
// (pixels x Cin) input with the Cin x Cout filter, the degenerate case of
// the patch matrix of section 5 (no patch is ever formed).
//
// Why a kernel of its own. In the row kernel a wave owns 32 output channels,
// so every 16-byte X fragment it reads from LDS feeds two MFMAs: LDS reads
// then run at 256 bytes per clock per compute unit, above what LDS serves,
// and each input pixel is pulled into eight workgroups (one per 64-channel
// tile). Here:
//  * A workgroup owns a contiguous range of 16-pixel blocks and 128 output
//    channels. Its 8 waves split the work: 4 only load, 4 only compute.
//    Issuing loads holds a wave for ~150 clocks per instruction, and a wave
//    that both loaded and computed spent about a fifth of each round issuing
//    and much of the rest waiting at the round's barrier for the slower one
//    (per-round timestamps: 1.65 us a round against 0.5 us of MFMAs).
//  * Computing wave w keeps the filter of the 64 channels (w & 1) of the
//    tile in registers (A operands, all of Cin) and takes pixel groups
//    2*(w >> 1) and 2*(w >> 1) + 1: each X fragment feeds four MFMAs, and
//    every pixel is pulled into Cout / 128 workgroups.
//  * Blocks arrive in rounds of four (one per pixel group) through a ring
//    of three LDS slots, written by buffer loads with the LDS bit (no
//    registers held); the loading waves request round k + 2 as round k
//    starts. Within a block, pixel p keeps channel chunk c (8 channels, 16
//    bytes) in unit p*CG + (c ^ (p >> SH)): the 16 lanes reading one chunk of
//    16 pixels hit 16 distinct bank groups.
//  * The loading waves stage the filter slice F[:, tile] in LDS in two
//    halves of Cin; the computing waves read it into registers with the
//    gfx950 transpose read (each element read by two waves, not four).
//  * bf16 results are regrouped through a small LDS patch private to the
//    wave so that eight consecutive lanes store one whole 128-byte pixel row
//    (64 channels); fp32 results leave straight from the accumulators (four
//    lanes write 64 contiguous bytes). Stores carry the device-scope policy
//    (sc1).
// Memory-count bookkeeping as in dense_band_mfma.hip: every load of the
// loading waves is unconditional (out-of-range lanes use an offset the
// hardware drops), so the number issued after each round's loads is a
// compile-time constant and the waits are explicit vmcnt values.
#include <algorithm>
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

constexpr int COMPUTERS = 4;             // waves that compute
constexpr int LOADERS = 4;               // waves that stage the filter and issue the input loads
constexpr int PC = 64 * COMPUTERS;       // computing threads
constexpr int PT = PC + 64 * LOADERS;    // threads per workgroup
constexpr int SLOTS = 3;                 // input rounds in the LDS ring
constexpr int CT = 128;                  // output channels per tile
constexpr int NB = 4;                    // 16-channel blocks per wave
constexpr int FPITCH = CT + 8;           // LDS pitch of a staged filter row (elements)
constexpr int OPP = 144;                 // LDS pitch of one pixel of a wave's bf16 output patch (bytes)
constexpr int SAUX = 18;                 // store cache policy: sc1 | nt (1x1 bf16: 15.4 -> 15.2 us against sc1)
constexpr uint32_t OOB = 0x80000000u;
constexpr int BUF_WORD3 = 0x00020000;
constexpr int LDS_MAX = 160 * 1024;

struct PwArgs {
    const uint16_t *X;
    const uint16_t *F;
    const float *bias;
    void *Y;
    int64_t xs, ys;        // pixel strides of X and Y (elements)
    int Cin, Cout;
    int nblocks;           // 16-pixel blocks of the batch (the last one may be partial)
    int npix;              // pixels of the batch
    int mtiles;            // pixel tiles (a multiple of 8; tiles past the blocks exit)
    int mreal;             // pixel tiles that hold blocks
    int ctiles;            // 128-channel tiles
    uint32_t x_records, y_records;
};

template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt holds 6 bits");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
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

// Sixteen transposed 8-byte reads at immediate offsets from one base, in one
// asm block ending in a wait (the compiler would otherwise wait for every
// LDS-bound load in flight before each transposed-read intrinsic). Outputs
// are early-clobber so no read lands in the address register while later
// reads are still to issue.
#define CF_TR(o, f) "ds_read_b64_tr_b16 %" #o ", %[a] offset:%" #f "\n\t"
template <int O0, int O1, int O2, int O3, int O4, int O5, int O6, int O7, int O8, int O9, int O10, int O11, int O12,
          int O13, int O14, int O15>
__device__ __forceinline__ void tr16(uint32_t base, i16x4 (&p)[16])
{
    asm volatile(CF_TR(0, 17) CF_TR(1, 18) CF_TR(2, 19) CF_TR(3, 20) CF_TR(4, 21) CF_TR(5, 22) CF_TR(6, 23)
                     CF_TR(7, 24) CF_TR(8, 25) CF_TR(9, 26) CF_TR(10, 27) CF_TR(11, 28) CF_TR(12, 29) CF_TR(13, 30)
                         CF_TR(14, 31) CF_TR(15, 32) "s_waitcnt lgkmcnt(0)"
                 : "=&v"(p[0]), "=&v"(p[1]), "=&v"(p[2]), "=&v"(p[3]), "=&v"(p[4]), "=&v"(p[5]), "=&v"(p[6]),
                   "=&v"(p[7]), "=&v"(p[8]), "=&v"(p[9]), "=&v"(p[10]), "=&v"(p[11]), "=&v"(p[12]), "=&v"(p[13]),
                   "=&v"(p[14]), "=&v"(p[15])
                 : [a] "v"(base), "n"(O0), "n"(O1), "n"(O2), "n"(O3), "n"(O4), "n"(O5), "n"(O6), "n"(O7), "n"(O8),
                   "n"(O9), "n"(O10), "n"(O11), "n"(O12), "n"(O13), "n"(O14), "n"(O15)
                 : "memory");
}
#undef CF_TR

template <int CS, bool OUT_BF16>
struct PwShape {
    static constexpr int CINP = 32 * CS;
    static constexpr int CG = CINP / 8;                          // 16-byte units per pixel
    static constexpr int SH = CG >= 16 ? 0 : CG == 8 ? 1 : 2;    // pixels per 256 bytes, log2
    static constexpr int BLOCK_BYTES = 16 * CINP * 2;            // one 16-pixel block
    static constexpr int ROUND_BYTES = 4 * BLOCK_BYTES;          // one block per pixel group
    static constexpr int DMA = ROUND_BYTES / (LOADERS * 64 * 16);   // loads into LDS per loading lane per round
    static constexpr int STAGE = CINP / 2;                       // filter rows staged at a time (two halves)
    static constexpr int NSTAGE = CINP / STAGE;
    static constexpr int FITEMS = STAGE * (CT / 8) / (LOADERS * 64);   // 16-byte filter loads per loading lane per stage
    static constexpr int RING = SLOTS * ROUND_BYTES;
    static constexpr int FSTAGE = STAGE * FPITCH * 2;
    // bf16 output patches: one round's (two blocks per computing wave) in
    // each of two buffers; the filter staging area, idle after the
    // prologue, serves as one of them when it is large enough.
    static constexpr int PSET = 2 * COMPUTERS * 16 * OPP;
    static constexpr bool PSET_IN_FSTAGE = STAGE * FPITCH * 2 >= PSET;
    static constexpr int PATCH = OUT_BF16 ? (PSET_IN_FSTAGE ? PSET : 2 * PSET) : 0;
    static constexpr size_t LDS = (size_t)RING + FSTAGE + PATCH;
    static_assert(CS % 4 == 0 && DMA >= 1 && DMA * LOADERS * 64 * 16 == ROUND_BYTES, "whole loads per loading wave");
    static_assert(FITEMS * LOADERS * 64 == STAGE * (CT / 8) && NSTAGE == 2, "whole filter loads per loading lane");
    static_assert(LDS <= (size_t)LDS_MAX, "LDS");
    // Memory instructions a loading wave has issued after round k's loads
    // when it waits for them, counted over its issue order: the filter, rounds
    // 0 .. SLOTS-2; then per round j: round j + SLOTS - 1, and (bf16 output)
    // the stores of round j - 1.
    static constexpr int NSTO = OUT_BF16 ? 4 : 0;
    static constexpr int after_round(int k)
    {
        int pos = 0, last = -1;
        for (int r = 0; r <= SLOTS - 2; ++r) {
            pos += DMA;
            if (r == k)
                last = pos;
        }
        for (int j = 0; j < k; ++j) {
            pos += DMA;
            if (j + SLOTS - 1 == k)
                last = pos;
            if (j > 0)
                pos += NSTO;
        }
        return pos - last;
    }
    static_assert(after_round(8) < 64, "vmcnt holds 6 bits");
};

template <int CS, int ROUNDS, bool OUT_BF16>
__global__ __launch_bounds__(PT) __attribute__((amdgpu_waves_per_eu(2, 2)))
void dense_pw_mfma(PwArgs a)
{
    using B = PwShape<CS, OUT_BF16>;
    constexpr int CG = B::CG;
    extern __shared__ __align__(16) uint8_t smem[];
    uint8_t *ring = smem;
    uint16_t *fst = reinterpret_cast<uint16_t *>(smem + B::RING);
    uint8_t *patch_all = smem + B::RING + B::FSTAGE;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    // Slot s runs on XCD s % 8; the channel tiles of one pixel range share
    // an XCD, so their common input meets in that XCD's L2.
    const int bid = with_args_loaded((int)blockIdx.x, a);
    const int slot_in_xcd = bid >> 3;
    const int mt = (bid & 7) * (a.mtiles >> 3) + slot_in_xcd / a.ctiles;
    const int ct = slot_in_xcd % a.ctiles;
    if (mt >= a.mreal)
        return;
    const int b0 = (int)((int64_t)mt * a.nblocks / a.mreal);
    const int b1 = (int)((int64_t)(mt + 1) * a.nblocks / a.mreal);
    const int o_tile = ct * CT;
    const __amdgpu_buffer_rsrc_t yr = __builtin_amdgcn_make_buffer_rsrc(a.Y, 0, (int)a.y_records, BUF_WORD3);
    // Round r's bf16 output patches.
    auto pbuf = [&](const int r) __attribute__((always_inline)) {
        return (r & 1) ? patch_all + (B::PSET_IN_FSTAGE ? 0 : B::PSET)
                       : (B::PSET_IN_FSTAGE ? reinterpret_cast<uint8_t *>(fst) : patch_all);
    };

    if (wave >= COMPUTERS) {
        // ---- Loading wave lw: stages the filter (through registers, into
        // the padded staging area) and issues its share of every round's
        // loads, waits for them and meets the computing waves at the round's
        // barrier.
        const int lw = __builtin_amdgcn_readfirstlane(wave - COMPUTERS);
        const int lt = tid - PC;
        const __amdgpu_buffer_rsrc_t xr =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(a.X), 0, (int)a.x_records, BUF_WORD3);
        const __amdgpu_buffer_rsrc_t fr = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t *>(a.F), 0, a.Cin * a.Cout * 2, BUF_WORD3);
        // Filter stage h: item it = lt + t*256 -> 8-output group (it & 15) of
        // the tile, input channel h*STAGE + (it >> 4).
        u32x4 fv[B::NSTAGE][B::FITEMS];
        auto issue_fstage = [&](const int h) __attribute__((always_inline)) {
#pragma unroll
            for (int t = 0; t < B::FITEMS; ++t) {
                const int it = lt + t * (LOADERS * 64);
                const int og = it & 15;
                const int c = h * B::STAGE + (it >> 4);
                const int o = o_tile + og * 8;
                const bool ok = c < a.Cin && o < a.Cout;
                fv[h][t] = __builtin_amdgcn_raw_buffer_load_b128(fr, ok ? (uint32_t)(c * a.Cout + o) * 2 : OOB, 0, 0);
            }
        };
        auto commit_fstage = [&](const int h) __attribute__((always_inline)) {
#pragma unroll
            for (int t = 0; t < B::FITEMS; ++t) {
                const int it = lt + t * (LOADERS * 64);
                *reinterpret_cast<u32x4 *>(fst + (it >> 4) * FPITCH + (it & 15) * 8) = fv[h][t];
            }
        };
        // Round k: block pg + 4k of the tile for each pixel group pg, into
        // ring slot k % SLOTS. Unit u of a round (16 bytes) is block
        // u / (16*CG), pixel (u / CG) % 16, stored chunk u % CG, loaded from
        // chunk (u % CG) ^ (p >> SH).
        auto dma_round = [&](const int k) __attribute__((always_inline)) {
            uint8_t *dst = ring + (k % SLOTS) * B::ROUND_BYTES;
#pragma unroll
            for (int i = 0; i < B::DMA; ++i) {
                const int u = (lw * B::DMA + i) * 64 + lane;
                const int blk = u / (16 * CG);
                const int p = (u / CG) % 16;
                const int c = (u % CG) ^ ((p >> B::SH) & (CG - 1));
                const int b = b0 + blk + 4 * k;
                const int pix = b * 16 + p;
                const bool ok = b < b1 && pix < a.npix && c * 8 < a.Cin;
                const uint32_t off = ok ? (uint32_t)(((int64_t)pix * a.xs + c * 8) * 2) : OOB;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    xr, (__attribute__((address_space(3))) void *)(dst + (lw * B::DMA + i) * 1024), 16, off, 0, 0, 0);
            }
        };

        // Round r's bf16 results, parked in LDS by the computing waves:
        // loading wave lw stores computing wave lw's two blocks (channels
        // 64*(lw & 1).., pixel groups 2*(lw >> 1) + hb). Store i: lane L takes
        // 16 bytes of pixel 8*(i % 2) + L/8 of block i / 2, chunk L % 8: eight
        // lanes write a whole 128-byte pixel row.
        auto store_round = [&](const int r) __attribute__((always_inline)) {
            const uint8_t *pb = pbuf(r) + lw * 2 * 16 * OPP;
            const int ch = o_tile + (lw & 1) * 64 + (lane & 7) * 8;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int hb = i >> 1;
                const int pq = 8 * (i & 1) + (lane >> 3);
                const int b = b0 + 2 * (lw >> 1) + hb + 4 * r;
                const u32x4 w = *reinterpret_cast<const u32x4 *>(pb + (hb * 16 + pq) * OPP + (lane & 7) * 16);
                const int pix = b * 16 + pq;
                const bool ok = b < b1 && pix < a.npix && ch < a.Cout;
                __builtin_amdgcn_raw_buffer_store_b128(w, yr, ok ? (uint32_t)(((int64_t)pix * a.ys + ch) * 2) : OOB,
                                                       0, SAUX);
            }
        };

        // The filter first (shared by every workgroup of the XCD, so mostly
        // L2 hits), then the first rounds.
        issue_fstage(0);
        issue_fstage(1);
        __builtin_amdgcn_sched_barrier(0);
        static_for<0, SLOTS - 1>([&](auto R) { dma_round(decltype(R)::value); });
        __builtin_amdgcn_sched_barrier(0);
        commit_fstage(0);
        lds_barrier();           // stage 0 published
        lds_barrier();           // the computing waves have read stage 0: the area is free
        commit_fstage(1);
        lds_barrier();           // stage 1 published
        static_for<0, ROUNDS>([&](auto K) {
            constexpr int k = decltype(K)::value;
            // Round k landed for this wave (issued after it: the rounds up
            // to k + SLOTS - 2); at the barrier, for every loading wave.
            // Past it the computing waves are done with round k - 1: its
            // slot takes round k + SLOTS - 1.
            wait_vmcnt<B::after_round(k)>();
            lds_barrier();
            __builtin_amdgcn_sched_barrier(0);
            dma_round(k + SLOTS - 1);
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (OUT_BF16 && k > 0)
                store_round(k - 1);
        });
        if constexpr (OUT_BF16) {
            lds_barrier();       // the last round's patches are written
            store_round(ROUNDS - 1);
        }
        return;
    }

    // ---- Computing wave w: 64 output channels (w & 1) of the tile, pixel
    // groups 2*(w >> 1) and 2*(w >> 1) + 1: two blocks a round.
    const int cg = wave & 1;
    const int pp = wave >> 1;
    // Bias of the 4 channels of each column block the lane's results belong to.
    u32x4 bq[NB];
    {
        const __amdgpu_buffer_rsrc_t br = __builtin_amdgcn_make_buffer_rsrc(
            a.bias ? (void *)a.bias : (void *)a.F, 0, a.bias ? a.Cout * 4 : 0, BUF_WORD3);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int o = o_tile + cg * 64 + nb * 16 + (lane >> 4) * 4;
            bq[nb] = __builtin_amdgcn_raw_buffer_load_b128(br, o < a.Cout ? (uint32_t)o * 4 : OOB, 0, 0);
        }
    }

    // A fragments: wf[k-step][nb], 8 consecutive input channels of one
    // output channel per lane (see dense_band_mfma.hip for the transposed
    // read's lane layout).
    bf16x8 wf[CS][NB];
    const uint32_t fbase = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint16_t *)fst +
                           (uint32_t)((((lane >> 4) * 8 + ((lane & 15) >> 2)) * FPITCH + cg * 64 + 4 * (lane & 3)) * 2);
    auto read_fstage = [&](auto H) __attribute__((always_inline)) {
        constexpr int h = decltype(H)::value;
        // Two k-steps (32 channels each) per asm block: reads
        // q = (kk*NB + nb)*2 + half4.
        static_for<0, B::STAGE / 64>([&](auto P) {
            constexpr int pr = decltype(P)::value;
            i16x4 q[16];
            constexpr int E = 2 * FPITCH;              // bytes per staged filter row
            constexpr int k0 = 2 * pr, k1 = 2 * pr + 1;
            tr16<(k0 * 32 + 0) * E + 0, (k0 * 32 + 4) * E + 0, (k0 * 32 + 0) * E + 32, (k0 * 32 + 4) * E + 32,
                 (k0 * 32 + 0) * E + 64, (k0 * 32 + 4) * E + 64, (k0 * 32 + 0) * E + 96, (k0 * 32 + 4) * E + 96,
                 (k1 * 32 + 0) * E + 0, (k1 * 32 + 4) * E + 0, (k1 * 32 + 0) * E + 32, (k1 * 32 + 4) * E + 32,
                 (k1 * 32 + 0) * E + 64, (k1 * 32 + 4) * E + 64, (k1 * 32 + 0) * E + 96, (k1 * 32 + 4) * E + 96>(fbase, q);
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    const i16x4 lo = q[(kk * NB + nb) * 2], hi = q[(kk * NB + nb) * 2 + 1];
                    const i16x8 both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                    wf[h * (B::STAGE / 32) + 2 * pr + kk][nb] = __builtin_bit_cast(bf16x8, both);
                }
        });
    };
    lds_barrier();               // stage 0 published
    read_fstage(std::integral_constant<int, 0>{});
    lds_barrier();               // done with stage 0
    lds_barrier();               // stage 1 published
    read_fstage(std::integral_constant<int, 1>{});

    const int p16 = lane & 15;
    const int g = lane >> 4;

    static_for<0, ROUNDS>([&](auto K) {
        constexpr int k = decltype(K)::value;
        lds_barrier();           // round k landed for every loading wave; round k - 1 is no longer read
        __builtin_amdgcn_sched_barrier(0);
        // Both blocks' fragments first and no branches: one straight run the
        // compiler can interleave (block 0's epilogue under block 1's
        // MFMAs). A block past the tile's end computes on stale LDS data;
        // its stores go to the dropped offset.
        bf16x8 xb[2][CS];
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
            const uint8_t *src = ring + (k % SLOTS) * B::ROUND_BYTES + (2 * pp + hb) * B::BLOCK_BYTES;
#pragma unroll
            for (int cs = 0; cs < CS; ++cs) {
                const int c = cs * 4 + g;
                xb[hb][cs] = *reinterpret_cast<const bf16x8 *>(src + (p16 * CG + (c ^ ((p16 >> B::SH) & (CG - 1)))) * 16);
            }
        }
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
            const int b = b0 + 2 * pp + hb + 4 * k;
            f32x4 acc[NB];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
                acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int cs = 0; cs < CS; ++cs)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[cs][nb], xb[hb][cs], acc[nb], 0, 0, 0);
            // The lane holds channels o_tile + 64*cg + 16*nb + 4*g + {0..3}
            // of pixel b*16 + p16.
            if constexpr (OUT_BF16) {
                // Parked in LDS; a loading wave stores it next round (a
                // store holds the issuing wave as long as a load does).
                uint8_t *patch = pbuf(k) + (wave * 2 + hb) * 16 * OPP;
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    const f32x4 v = acc[nb];
                    *reinterpret_cast<u32x2 *>(patch + p16 * OPP + (nb * 16 + g * 4) * 2) =
                        u32x2{pack_bf16x2(v[0] + __uint_as_float(bq[nb][0]), v[1] + __uint_as_float(bq[nb][1])),
                              pack_bf16x2(v[2] + __uint_as_float(bq[nb][2]), v[3] + __uint_as_float(bq[nb][3]))};
                }
            } else {
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    const f32x4 v = acc[nb];
                    const u32x4 w = {__float_as_uint(v[0] + __uint_as_float(bq[nb][0])),
                                     __float_as_uint(v[1] + __uint_as_float(bq[nb][1])),
                                     __float_as_uint(v[2] + __uint_as_float(bq[nb][2])),
                                     __float_as_uint(v[3] + __uint_as_float(bq[nb][3]))};
                    const int ch = o_tile + cg * 64 + nb * 16 + g * 4;
                    const int pix = b * 16 + p16;
                    const bool ok = b < b1 && pix < a.npix && ch < a.Cout;
                    __builtin_amdgcn_raw_buffer_store_b128(w, yr, ok ? (uint32_t)(((int64_t)pix * a.ys + ch) * 4) : OOB,
                                                           0, SAUX);
                }
            }
        }
    });
    if constexpr (OUT_BF16)
        lds_barrier();           // the last round's patches are written
}

template <int CS, int ROUNDS, bool OB>
hipError_t launch_pw(const PwArgs &a, dim3 grid, hipStream_t s)
{
    auto kern = dense_pw_mfma<CS, ROUNDS, OB>;
    constexpr size_t lds = PwShape<CS, OB>::LDS;
    const hipError_t attr = allow_lds<dense_pw_mfma<CS, ROUNDS, OB>>((int)lds);
    if (attr != hipSuccess)
        return attr;
    hipLaunchKernelGGL(kern, grid, dim3(PT), lds, s, a);
    return hipGetLastError();
}

constexpr int PW_ROUNDS = 7;    // rounds of four blocks: up to 28 blocks (448 pixels) per tile

struct PwPlan {
    int CS, mtiles, mreal, ctiles, nblocks;
    int64_t npix, xs, ys;
};

bool plan_pw(const DenseProblem &p, PwPlan *pl)
{
    if (p.KH != 1 || p.KW != 1 || !plain_window(p) || p.xdt != CONV_BF16)
        return false;
    if (p.Cin % 128 != 0 || p.Cin > 256 || p.Cout % 8 != 0)
        return false;       // two filter stages of whole pairs of 32-channel steps
    // Every pixel of the batch at one stride, in X and in Y.
    if (p.xs[1] != (int64_t)p.W * p.xs[2] || p.xs[0] != (int64_t)p.H * p.xs[1] ||
        p.ys[1] != (int64_t)p.Wo * p.ys[2] || p.ys[0] != (int64_t)p.Ho * p.ys[1])
        return false;
    const int yesz = p.ydt == CONV_BF16 ? 2 : 4;
    if ((uintptr_t)p.X % 16 || (uintptr_t)p.F % 16 || (uintptr_t)p.Y % 16 || p.xs[2] % 8 || p.ys[2] % (16 / yesz))
        return false;
    const int64_t npix = (int64_t)p.N * p.H * p.W;
    if (((npix - 1) * p.xs[2] + p.Cin) * 2 >= (int64_t(1) << 31) ||
        ((npix - 1) * p.ys[2] + p.Cout) * yesz >= (int64_t(1) << 31) || (int64_t)p.Cin * p.Cout * 2 >= (1ll << 31))
        return false;
    const int64_t nblocks = (npix + 15) / 16;
    const int ctiles = (p.Cout + CT - 1) / CT;
    // About one workgroup per compute unit, each with at most 4 * PW_ROUNDS blocks.
    int64_t mreal = std::max<int64_t>(1, 256 / ctiles);
    mreal = std::max<int64_t>(mreal, (nblocks + 4 * PW_ROUNDS - 1) / (4 * PW_ROUNDS));
    mreal = std::min<int64_t>(mreal, nblocks);
    if (mreal * ctiles >= (1 << 30))
        return false;
    pl->CS = p.Cin / 32;
    pl->mreal = (int)mreal;
    pl->mtiles = (int)((mreal + 7) / 8 * 8);
    pl->ctiles = ctiles;
    pl->nblocks = (int)nblocks;
    pl->npix = npix;
    pl->xs = p.xs[2];
    pl->ys = p.ys[2];
    return true;
}

}  // namespace

bool dense_pw_supports(const DenseProblem &p)
{
    PwPlan pl;
    return plan_pw(p, &pl);
}

hipError_t launch_dense_pw(const DenseProblem &p, hipStream_t s)
{
    PwPlan pl;
    if (!plan_pw(p, &pl))
        return hipErrorNotSupported;
    PwArgs a;
    a.X = static_cast<const uint16_t *>(p.X);
    a.F = static_cast<const uint16_t *>(p.F);
    a.bias = p.bias;
    a.Y = p.Y;
    a.xs = pl.xs;
    a.ys = pl.ys;
    a.Cin = p.Cin;
    a.Cout = p.Cout;
    a.nblocks = pl.nblocks;
    a.npix = (int)pl.npix;
    a.mtiles = pl.mtiles;
    a.mreal = pl.mreal;
    a.ctiles = pl.ctiles;
    const int yesz = p.ydt == CONV_BF16 ? 2 : 4;
    a.x_records = (uint32_t)(((pl.npix - 1) * pl.xs + p.Cin) * 2);
    a.y_records = (uint32_t)(((pl.npix - 1) * pl.ys + p.Cout) * yesz);
    const dim3 grid((unsigned)(pl.mtiles * pl.ctiles));
    const bool ob = p.ydt == CONV_BF16;
    switch (pl.CS) {
    case 4: return ob ? launch_pw<4, PW_ROUNDS, true>(a, grid, s) : launch_pw<4, PW_ROUNDS, false>(a, grid, s);
    case 8: return ob ? launch_pw<8, PW_ROUNDS, true>(a, grid, s) : launch_pw<8, PW_ROUNDS, false>(a, grid, s);
    }
    return hipErrorNotSupported;
}

}  // namespace convfwd
