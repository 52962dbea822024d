// Dense NHWC cross-correlation as an implicit GEMM on CDNA4 matrix cores.
//
// Contract: "CMU DLSys Lecture 14: Convolutional Network Implementation",
// section 1 (Y[n,y,x,o] = sum over i,j,c of X[n,y+i,x+j,c] * F[i,j,c,o]).
// Section 5 writes it as a product of the (N*Ho*Wo) x (K*K*Cin) patch matrix
// with F reshaped to (K*K*Cin) x Cout; section 6 prices the copy that builds
// the patch matrix. This kernel never builds it: a band's input rows are
// staged once in LDS and every patch fragment is read from there with a
// per-tap offset (the 6-axis patch view of section 5 turned into LDS
// addressing).
//
// Work decomposition (one workgroup = 8 waves = 512 threads, 2 per SIMD):
//  * A workgroup owns a band of R output rows of one image and a tile of 64
//    output channels. It walks its R + KH - 1 input rows (at most NR) top to
//    bottom, keeping the loads of the next two to four rows in flight in
//    registers. A 1x1 filter makes pixels independent: pixel-contiguous
//    inputs are regrouped into rows of 64 pixels first.
//  * The filter slice F[:, :, :, tile] is transposed through LDS and then held
//    in registers as the A operand of v_mfma_f32_16x16x32_bf16 for the whole
//    band. Wave w keeps the 32-channel half (w & 1) of the tile:
//    KH*KW*ceil(Cin/32) k-steps x 2 column blocks x 4 registers.
//  * Each input row is committed to LDS once, and every X fragment read
//    from it feeds all KH output rows that use that input row (one
//    accumulator set per output row in flight), so LDS traffic per output
//    row is KW*CS fragment reads rather than KH*KW*CS.
//  * Output row y is cut into 16-pixel blocks; wave pair (2g, 2g+1) takes
//    blocks g, g+4. Per fragment a lane reads 8 channels of one pixel (16
//    bytes, B operand) and issues one MFMA per 16-channel column block of its
//    half into each output row in flight: KH*2 independent accumulation
//    chains per wave.
//  * The product is computed transposed (rows = output channels, columns =
//    pixels). Each row of results is parked in an LDS tile and leaves as
//    16-byte chunks, so every store instruction writes whole cache lines.
//
// LDS pixel pitch is Cin_padded + 16 bf16 (32 bytes of padding). Measured on
// gfx950, 16-byte LDS reads whose 16 lanes step through consecutive pixels
// run conflict-free only when the pitch is 32 modulo 64 bytes (96, 160, 288,
// 544 B all reach ~190 B/clk per CU; pitches of 16, 48 or 0 modulo 64 lose
// about 40%). Channels beyond Cin (up to the multiple of 32) are zero.
//
// All global accesses are raw buffer operations: out-of-range offsets are
// dropped by the hardware (loads return zeros), which masks ragged edges
// without branches around memory operations.
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

constexpr int THREADS = 512;
constexpr int COUT_TILE = 64;      // 4 column blocks of 16 output channels
constexpr int NBW = 2;             // column blocks per wave (its half of the tile)
constexpr int LDS_BYTES_MAX = 160 * 1024;
constexpr uint32_t OOB = 0x80000000u;           // buffer offset beyond every range: access dropped
constexpr int BUF_WORD3 = 0x00020000;           // raw buffer descriptor word 3 (gfx9 family)

struct RowArgs {
    const uint16_t *X;
    const uint16_t *F;
    const float *bias;
    void *Y;
    int64_t xs0, xs1, xs2, ys0, ys1, ys2;
    int H, W, Ho, Wo;
    int Cin, Cout;      // channels of one group (input, output)
    int f_ld;           // F row length: output channels of all groups
    int gpack;          // 0, or the channels of one true group when several small
                        // groups share a 64-channel tile (block-diagonal filter)
    int pt, pl;         // zero rows / columns before the input
    int R;              // output rows per band
    int bands_per_img;
    int bands;          // N * bands_per_img (the grid may hold more: those exit)
    int tiles;          // 64-channel output tiles per group
    int groups;
    int row_slots;      // pixel slots of a staged input row (zero padding included)
    int row_elems;      // LDS elements per staged input row (row_slots * pitch)
    int chunks_per_row; // 16-byte chunks of real input per row (W * Cin_padded / 8)
    int otile_off;      // LDS byte offset of the output tiles
    int rows_off;       // LDS element offset of the row buffers: 0 (they reuse the
                        // filter staging area) or past the staging area
    uint32_t x_records; // bytes addressable from one image's base in X
    uint32_t y_records; // bytes addressable from one image's base in Y
};

// LDS pixel pitch of a staged row, in bf16 elements. Lanes read pixels S
// slots apart, and 16-byte reads of 16 lanes are conflict-free when the lane
// step is 32 modulo 64 bytes: Cin_padded + 16 for S = 1 (CINP*2 + 32 bytes),
// Cin_padded + 8 for S = 2 (twice CINP*2 + 16 bytes).
template <int CINP, int S>
constexpr int row_pitch() { return S == 1 ? CINP + 16 : CINP + 8; }

// Byte offset (from the image's base) of 16-byte chunk q (pixel q / CG,
// channel group q % CG) of input row iy, or OOB when the chunk is padding,
// outside the image or past the rows the band reads: the buffer load then
// returns zeros without touching memory.
template <int CINP>
__device__ __forceinline__ uint32_t chunk_off(const RowArgs &a, int iy, int q, int iy_end)
{
    constexpr int CG = CINP / 8;
    const int px = q / CG;
    const int cg = q - px * CG;
    const bool ok = q < a.chunks_per_row && iy >= 0 && iy < iy_end && cg * 8 < a.Cin;
    return ok ? (uint32_t)(((int64_t)iy * a.xs1 + (int64_t)px * a.xs2 + cg * 8) * 2) : OOB;
}

// Chunk q of a row lands in pixel slot (q / CG) + pl: the first pl slots and
// those past the input hold the zero padding.
template <int CINP, int S>
__device__ __forceinline__ void put_chunk(uint16_t *lds_row, int pl, int q, u32x4 v)
{
    constexpr int CG = CINP / 8;
    constexpr int PITCH = row_pitch<CINP, S>();
    const int px = q / CG;
    const int cg = q - px * CG;
    *reinterpret_cast<u32x4 *>(lds_row + (px + pl) * PITCH + cg * 8) = v;
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

// Filter slice F[:, :, :, o0:o0+64] of a workgroup, in three steps shared
// by both kernels: issue the loads, write the slice to LDS in its natural
// layout ft[tap][c][o] (rows of 64 outputs padded to 72 elements), then read
// the A fragments back with the gfx950 transpose read.
//
// Load item it -> (8-channel output group og fastest, then input channel c,
// then tap): eight lanes cover one 128-byte row of F, so the loads are
// coalesced. Padding channels and outputs past Cout load as zeros.
template <int KH, int KW, int CS>
struct FilterSlice {
    static constexpr int CINP = 32 * CS;
    static constexpr int FPITCH = COUT_TILE + 8;
    static constexpr int KSTEPS = KH * KW * CS;
    static constexpr int ITEMS = (KH * KW * CINP * 8 + THREADS - 1) / THREADS;
    static constexpr size_t LDS_BYTES = (size_t)KH * KW * CINP * FPITCH * 2;

    u32x4 fv[ITEMS];

    // o0: first output channel of the tile within its group; oc0: first
    // output channel of the group (F rows hold all groups' outputs).
    //
    // With small groups packed into the tile (a.gpack = G), tile input
    // channel c and output channel o belong to true groups c / G and o / G;
    // F holds G input channels per tap, and entries between different groups
    // are the zeros of the block-diagonal filter (eight consecutive outputs
    // never straddle a group: G is a multiple of 8).
    __device__ __forceinline__ void issue(const RowArgs &a, int o0, int oc0, int tid)
    {
        const int fcin = a.gpack ? a.gpack : a.Cin;          // F rows per tap
        const __amdgpu_buffer_rsrc_t fr = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t *>(a.F), 0, KH * KW * fcin * a.f_ld * 2, BUF_WORD3);
#pragma unroll
        for (int t = 0; t < ITEMS; ++t) {
            const int it = tid + t * THREADS;
            const int og = it & 7;
            const int c = (it >> 3) % CINP;
            const int tap = (it >> 3) / CINP;
            const int o = o0 + og * 8;
            bool ok = tap < KH * KW && c < a.Cin && o < a.Cout;
            int cf = c;
            if (a.gpack) {
                ok = ok && c / a.gpack == o / a.gpack;
                cf = c % a.gpack;
            }
            fv[t] = __builtin_amdgcn_raw_buffer_load_b128(
                fr, ok ? (uint32_t)((((int64_t)tap * fcin + cf) * a.f_ld + oc0 + o) * 2) : OOB, 0, 0);
        }
    }

    __device__ __forceinline__ void commit(uint16_t *ft, int tid) const
    {
#pragma unroll
        for (int t = 0; t < ITEMS; ++t) {
            const int it = tid + t * THREADS;
            const int og = it & 7;
            const int c = (it >> 3) % CINP;
            const int tap = (it >> 3) / CINP;
            if (tap < KH * KW)
                *reinterpret_cast<u32x4 *>(ft + (tap * CINP + c) * FPITCH + og * 8) = fv[t];
        }
    }

    // Within each 16-lane group of ds_read_b64_tr_b16, output lane i gets
    // element i % 4 of the 8-byte chunk addressed by lane 4j + i/4, for
    // j = 0..3. Lane r of the group therefore addresses row r/4, columns
    // 4*(r%4)..+3 of a 4-row block of ft, and receives F[c0+j][o0+i]: four
    // consecutive input channels of one output channel, which is the
    // A-operand layout (lane holds 8 consecutive k of row o = lane % 16).
    // Two reads give the 8 channels of the lane's k-group.
    template <int I0 = 0, int I1 = KH>
    static __device__ __forceinline__ void fragments(const uint16_t *ft, int lane, int half, bf16x8 (&wf)[KSTEPS][NBW])
    {
        const int g = lane >> 4;           // k-group: channels 8g..8g+7 of a 32-channel step
        const int r = lane & 15;
#pragma unroll
        for (int ks = I0 * KW * CS; ks < I1 * KW * CS; ++ks) {
            const int tap = ks / CS;
            const int cs = ks % CS;
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb) {
                i16x4 part[2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int c = cs * 32 + g * 8 + h * 4 + (r >> 2);
                    const int o = half * 32 + nb * 16 + 4 * (r & 3);
                    part[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) i16x4 *)(ft + (tap * CINP + c) * FPITCH + o));
                }
                const i16x8 both = {part[0][0], part[0][1], part[0][2], part[0][3],
                                    part[1][0], part[1][1], part[1][2], part[1][3]};
                wf[ks][nb] = __builtin_bit_cast(bf16x8, both);
            }
        }
    }
};

// Bias of the 4 output channels of each column block a lane's results
// belong to (zeros without bias).
__device__ __forceinline__ void bias_issue(const RowArgs &a, int o0, int oc0, int half, int lane, u32x4 (&bq)[NBW])
{
    const __amdgpu_buffer_rsrc_t br = __builtin_amdgcn_make_buffer_rsrc(
        a.bias ? (void *)(a.bias + oc0) : (void *)a.F, 0, a.bias ? a.Cout * 4 : 0, BUF_WORD3);
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb)
        bq[nb] = __builtin_amdgcn_raw_buffer_load_b128(
            br, (uint32_t)((o0 + half * 32 + nb * 16 + (lane >> 4) * 4) * 4), 0, 0);
}

// S is the stride along both axes (1 or 2). A band of output rows
// t = 0..R-1 reads input rows y0*S - pt + r for r = 0..(R-1)*S + KH - 1;
// output row t uses rows r = t*S + i (filter row i). NR bounds that count.
// Whether the row kernel prefetches the next row's X fragments (three LDS
// row buffers instead of two): one block per wave, and either one chunk per
// thread per row with at most six fragments (the 3x3 layers, whose filter
// fills most registers) or a 1x1 filter (whose filter registers are few).
constexpr bool prefetch_rows(int KW, int CS, int BPW, int MAXC)
{
    return BPW == 1 && ((MAXC == 1 && KW * CS <= 6) || (KW == 1 && CS <= 8));
}

template <int KH, int KW, int S>
struct Window {
    static constexpr int INFLIGHT = (KH + S - 1) / S;    // output rows summing at once
    // Output row t of a band of at most RMAX rows completes at step t*S + KH - 1.
    static constexpr bool completes(int r, int RMAX) { return r >= KH - 1 && (r - (KH - 1)) % S == 0 && (r - (KH - 1)) / S < RMAX; }
};

template <int KH, int KW, int CS, int BPW, int MAXC, int NR, int S, bool OUT_BF16>
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
void dense_rows_mfma(RowArgs a)
{
    constexpr int CINP = 32 * CS;
    constexpr int PITCH = row_pitch<CINP, S>();
    constexpr int CG = CINP / 8;
    constexpr int KSTEPS = KH * KW * CS;
    constexpr int ESZ = OUT_BF16 ? 2 : 4;
    constexpr int RMAX = (NR - KH) / S + 1;          // output rows a band can hold
    constexpr int T = Window<KH, KW, S>::INFLIGHT;
    // Output tile: one row of results (64 pixels per block slot x 64
    // channels), double buffered, padded to a pitch of 32 mod 64 bytes.
    constexpr int OPITCH = COUT_TILE * ESZ + 32;
    constexpr int OTILE_BYTES = 64 * BPW * OPITCH;
    constexpr int OCH = COUT_TILE * ESZ / 16;                        // 16-byte chunks per pixel
    constexpr int OSTORE = (64 * BPW * OCH + THREADS - 1) / THREADS;  // store instructions per row
    // Store cache policy: sc1 | nt drains whole-line stores faster on
    // gfx950 (measured: fp32 outputs and windowed layers 3-6% faster with
    // sc1, nt adds a little); the 1x1 bf16 layer, whose stores interleave
    // with a long X stream, keeps the default.
    constexpr int SAUX = (KH == 1 && OUT_BF16) ? 0 : 18;

    // LDS: [filter staging] [two input-row buffers] [output tiles], or, when
    // that does not fit, [filter staging, later the row buffers] [output
    // tiles]: the staging area is dead once the fragments are in registers.
    // Input row r lives in buffer r & 1.
    extern __shared__ __align__(16) uint16_t smem[];
    uint16_t *ft = smem;
    uint16_t *rows = smem + a.rows_off;
    const bool rows_apart = a.rows_off != 0;
    uint8_t *otile = reinterpret_cast<uint8_t *>(smem) + a.otile_off;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int half = wave & 1;          // which 32 output channels of the tile
    const int pg = wave >> 1;           // pixel-block group 0..3
    // Workgroups are dealt to the 8 XCDs round robin by launch order (slot s
    // runs on XCD s % 8). The grid holds a multiple of 8 bands times the
    // output tiles; slot s takes band (s % 8) * (bands/8) + (s/8) / tiles and
    // tile (s/8) % tiles. All tiles of a band and consecutive bands of one
    // image then run on one XCD, so the input rows they share (the whole band
    // across tiles, the halo rows across bands) meet in that XCD's L2.
    const int tiles_all = a.tiles * a.groups;
    const int bid = with_args_loaded((int)blockIdx.x, a);
    const int slot_in_xcd = bid >> 3;
    const int band = (bid & 7) * (int)(gridDim.x >> 3) / tiles_all + slot_in_xcd / tiles_all;
    const int tile = slot_in_xcd % tiles_all;
    const int grp = tile / a.tiles;
    const int o0 = (tile - grp * a.tiles) * COUT_TILE;   // within the group
    const int xc0 = grp * a.Cin;                          // group's first input channel
    const int oc0 = grp * a.Cout;                         // group's first output channel
    if (band >= a.bands)
        return;
    const int n = band / a.bands_per_img;
    const int y0 = (band - n * a.bands_per_img) * a.R;
    if (y0 >= a.Ho)
        return;
    const int y1 = min(y0 + a.R, a.Ho);
    const int iy0 = y0 * S - a.pt;                        // input row of step 0
    const int iy_end = min(a.H, (y1 - 1) * S - a.pt + KH);  // one past the last input row the band reads

    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(a.X + (int64_t)n * a.xs0 + xc0), 0, (int)(a.x_records - xc0 * 2), BUF_WORD3);
    const __amdgpu_buffer_rsrc_t yr = __builtin_amdgcn_make_buffer_rsrc(
        static_cast<char *>(a.Y) + ((int64_t)n * a.ys0 + oc0) * ESZ, 0, (int)(a.y_records - oc0 * ESZ), BUF_WORD3);

    // 1. Filter slice and bias first.
    FilterSlice<KH, KW, CS> filt;
    filt.issue(a, o0, oc0, tid);
    u32x4 bq[NBW];
    bias_issue(a, o0, oc0, half, lane, bq);

    // 2. The first D input rows of the band; the loop below keeps loading D
    //    rows ahead of use. The fence keeps the scheduler from hoisting these
    //    above the filter loads (the counter is in order, so the filter wait
    //    would then also wait for the rows).
    __builtin_amdgcn_sched_barrier(0);
    // When prefetch_rows allows it, the next row's X fragments are read
    // during the current row's MFMAs: rows then rotate through three LDS
    // buffers (row r in buffer r % 3; row r + 2 is committed during step r),
    // and three rows of loads are in flight. Otherwise those registers are
    // not there (the compiler would spill) and two buffers suffice.
    constexpr bool PF = prefetch_rows(KW, CS, BPW, MAXC);
    constexpr int NBUF = PF ? 3 : 2;
    constexpr int DW = PF ? 3 : MAXC == 1 ? 4 : 2;    // rows of loads in flight (register budget)
    constexpr int D = NR < DW ? NR : DW;
    static_assert(!PF || D >= 3, "the prefetching ring loads three rows ahead");
    u32x4 xin[D][MAXC];
#pragma unroll
    for (int i = 0; i < D; ++i)
#pragma unroll
        for (int k = 0; k < MAXC; ++k)
            xin[i][k] = __builtin_amdgcn_raw_buffer_load_b128(
                xr, chunk_off<CINP>(a, iy0 + i, tid + k * THREADS, iy_end), 0, 0);

    // 3. Filter slice into LDS; 4. zero the padding slots of every row
    //    buffer (never overwritten afterwards) and commit the first input
    //    rows (row 0, and row 1 when prefetching); 5. the A fragments into
    //    registers. With the rows apart from the staging area, 3 and 4 share
    //    one barrier and the loop can start right after 5; otherwise 4 waits
    //    until every wave has read its fragments.
    auto commit_first_row = [&]() __attribute__((always_inline)) {
        const int zslots = a.row_slots - a.W;
        for (int q = tid; q < NBUF * zslots * CG; q += THREADS) {
            const int b = q / (zslots * CG);
            const int zq = q - b * zslots * CG;
            const int zi = zq / CG;
            const int slot = zi < a.pl ? zi : zi + a.W;
            *reinterpret_cast<u32x4 *>(rows + b * a.row_elems + slot * PITCH + (zq - zi * CG) * 8) = u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int k = 0; k < MAXC; ++k) {
            const int q = tid + k * THREADS;
            if (q < a.chunks_per_row)
                put_chunk<CINP, S>(rows, a.pl, q, xin[0][k]);
        }
        if constexpr (PF && NR > 1) {
#pragma unroll
            for (int k = 0; k < MAXC; ++k) {
                const int q = tid + k * THREADS;
                if (q < a.chunks_per_row)
                    put_chunk<CINP, S>(rows + a.row_elems, a.pl, q, xin[1][k]);
            }
        }
    };
    // With the rows apart from the staging area, the staged filter stays in
    // LDS during the loop: only filter row 0's fragments are read now, and
    // those of filter row i at the start of step i (the first step to use
    // them), under the first steps' few MFMAs. (With fp32 outputs or stride
    // 2 the longer register live ranges would spill: those read them all
    // here.)
    constexpr bool LAZY = PF && S == 1 && OUT_BF16;
    bf16x8 wf[KSTEPS][NBW];
    auto stage_eager = [&]() __attribute__((always_inline)) {
        filt.commit(ft, tid);
        if (rows_apart)
            commit_first_row();
        __syncthreads();
        FilterSlice<KH, KW, CS>::fragments(ft, lane, half, wf);
        if (!rows_apart) {
            __syncthreads();      // the staging area becomes the input-row area
            commit_first_row();
            __syncthreads();
        }
    };
    bool lazy = false;
    if constexpr (LAZY) {
        lazy = rows_apart;
        if (lazy) {
            filt.commit(ft, tid);
            commit_first_row();
            __syncthreads();
            FilterSlice<KH, KW, CS>::template fragments<0, 1>(ft, lane, half, wf);
        } else {
            stage_eager();
        }
    } else {
        stage_eager();
    }

    // A finished output row leaves as 16-byte chunks from its LDS tile:
    // consecutive lanes write consecutive bytes of consecutive pixels, so
    // every store instruction writes whole cache lines. Rows past the band
    // and lanes past the row use out-of-range offsets (dropped).
    auto store_row = [&](const int t) __attribute__((always_inline)) {
        const uint8_t *obuf = otile + (t & 1) * OTILE_BYTES;
        const int yo = y0 + t;
#pragma unroll
        for (int k = 0; k < OSTORE; ++k) {
            const int q = tid + k * THREADS;
            const int px = q / OCH;               // pixel
            const int cc = q - px * OCH;          // 16-byte chunk within the pixel's tile row
            const int ch = o0 + cc * (16 / ESZ);
            const bool ok = px < a.Wo && ch < a.Cout && yo < y1;
            const u32x4 v = *reinterpret_cast<const u32x4 *>(obuf + (px < 64 * BPW ? px : 0) * OPITCH + cc * 16);
            const uint32_t off = ok ? (uint32_t)(((int64_t)yo * a.ys1 + (int64_t)px * a.ys2 + ch) * ESZ) : OOB;
            __builtin_amdgcn_raw_buffer_store_b128(v, yr, off, 0, SAUX);
        }
    };

    // 6. Slide down the band one input row at a time. Input row r feeds
    //    output rows t = (r - i) / S for the filter rows i with r - i a
    //    multiple of S, so each X fragment read from LDS serves every output
    //    row that uses that input row. Output row t accumulates in slot t % T
    //    (taps in ascending i, then j, then channel step); it is complete at
    //    step t*S + KH - 1, goes to output tile t & 1, and leaves at the next
    //    step, after the barrier.
    //    The loop is fully unrolled (NR steps, all indices static) and every
    //    global operation in it is unconditional, so the waits the compiler
    //    places for prefetched rows never include the stores.
    using Win = Window<KH, KW, S>;
    f32x4 acc[T][BPW][NBW];
#pragma unroll
    for (int s2 = 0; s2 < T; ++s2)
#pragma unroll
        for (int qb = 0; qb < BPW; ++qb)
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb)
                acc[s2][qb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

    // X fragments of input row r for block qb (eight channels of one pixel
    // per lane, for each tap column j and channel step).
    auto read_frags = [&](const uint16_t *rowp, int qb, bf16x8 (&xb)[KW * CS]) __attribute__((always_inline)) {
        const int x = (pg + 4 * qb) * 16 + (lane & 15);
        const int xl = min(x, a.Wo - 1);
#pragma unroll
        for (int jc = 0; jc < KW * CS; ++jc) {
            const int j = jc / CS;
            const int cs = jc % CS;
            xb[jc] = *reinterpret_cast<const bf16x8 *>(rowp + (xl * S + j) * PITCH + cs * 32 + (lane >> 4) * 8);
        }
    };
    bf16x8 xn[KW * CS];          // prefetched fragments of the next row (PF)
    if constexpr (PF)
        read_frags(rows, 0, xn);

    static_for<0, NR>([&](auto RR) {
        constexpr int r = decltype(RR)::value;
        if constexpr (LAZY && r >= 1 && r < KH) {
            if (lazy)
                FilterSlice<KH, KW, CS>::template fragments<r, r + 1>(ft, lane, half, wf);
        }
        if constexpr (r >= 1 && Win::completes(r - 1, RMAX))
            store_row((r - KH) / S);
        if constexpr (r + D < NR) {
#pragma unroll
            for (int k = 0; k < MAXC; ++k)
                xin[(r + D) % D][k] = __builtin_amdgcn_raw_buffer_load_b128(
                    xr, chunk_off<CINP>(a, iy0 + r + D, tid + k * THREADS, iy_end), 0, 0);
        }
        const uint16_t *rowp = rows + (r % NBUF) * a.row_elems;
#pragma unroll
        for (int qb = 0; qb < BPW; ++qb) {
            const int x = (pg + 4 * qb) * 16 + (lane & 15);
            bf16x8 xb[KW * CS];
            if constexpr (PF) {
                // Row r was read during the previous step; row r + 1 was
                // committed then too, so its fragments can be read now,
                // under this row's MFMAs.
#pragma unroll
                for (int jc = 0; jc < KW * CS; ++jc)
                    xb[jc] = xn[jc];
                if constexpr (r + 1 < NR)
                    read_frags(rows + ((r + 1) % NBUF) * a.row_elems, 0, xn);
            } else {
                read_frags(rowp, qb, xb);
            }
#pragma unroll
            for (int i = 0; i < KH; ++i) {
                const int d = r - i;                      // t * S for the output row this tap feeds
                const int t = d / S;
                if (d >= 0 && d % S == 0 && t < RMAX && y0 + t < y1) {
#pragma unroll
                    for (int jc = 0; jc < KW * CS; ++jc) {
                        const int ks = i * KW * CS + jc;
#pragma unroll
                        for (int nb = 0; nb < NBW; ++nb)
                            acc[t % T][qb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                wf[ks][nb], xb[jc], acc[t % T][qb][nb], 0, 0, 0);
                    }
                }
            }
            if constexpr (Win::completes(r, RMAX)) {
                // Output row t is complete: lane holds channels
                // 32*half+16nb+4*(lane/16)+{0..3} of pixel x.
                constexpr int t = (r - (KH - 1)) / S;
                uint8_t *orow = otile + (t & 1) * OTILE_BYTES + x * OPITCH;
#pragma unroll
                for (int nb = 0; nb < NBW; ++nb) {
                    const int cl = half * 32 + nb * 16 + (lane >> 4) * 4;
                    const f32x4 v = acc[t % T][qb][nb];
                    const float v0 = v[0] + __uint_as_float(bq[nb][0]);
                    const float v1 = v[1] + __uint_as_float(bq[nb][1]);
                    const float v2 = v[2] + __uint_as_float(bq[nb][2]);
                    const float v3 = v[3] + __uint_as_float(bq[nb][3]);
                    if constexpr (OUT_BF16) {
                        *reinterpret_cast<u32x2 *>(orow + cl * 2) = u32x2{pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
                    } else {
                        *reinterpret_cast<u32x4 *>(orow + cl * 4) =
                            u32x4{__float_as_uint(v0), __float_as_uint(v1), __float_as_uint(v2), __float_as_uint(v3)};
                    }
                    acc[t % T][qb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
            }
        }
        // The input row committed now: r + 2 with prefetching (its buffer
        // last held row r - 1, whose fragments were read during step r - 2),
        // else r + 1 into the other buffer (its previous row was last read
        // before the barrier that ended the previous step). Rows past the
        // band are zeros and never feed a stored output.
        constexpr int rc = PF ? r + 2 : r + 1;
        if constexpr (rc < NR) {
#pragma unroll
            for (int k = 0; k < MAXC; ++k) {
                const int q = tid + k * THREADS;
                if (q < a.chunks_per_row)
                    put_chunk<CINP, S>(rows + (rc % NBUF) * a.row_elems, a.pl, q, xin[rc % D][k]);
            }
        }
        __syncthreads();
    });
    if constexpr (Win::completes(NR - 1, RMAX))
        store_row((NR - KH) / S);
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

bool taps_instantiated(int KH, int KW, int CS, int S)
{
    if (KH == 1 && KW == 1)
        return S == 1 ? (CS == 1 || CS == 2 || CS == 4 || CS == 8 || CS == 16) : (CS == 1 || CS == 2 || CS == 4 || CS == 8);
    if (KH == 2 && KW == 2)
        return S == 1 && (CS == 1 || CS == 2 || CS == 4);
    if (KH == 3 && KW == 3)
        return CS == 1 || CS == 2;
    return false;
}

// Input rows a band walks (the unrolled step count). Only the loads of the
// next few rows are held in registers, so this is bounded by code size, not
// by registers or LDS.
constexpr int rows_in_regs(int MAXC) { return MAXC == 1 ? 9 : MAXC == 2 ? 9 : 13; }

// Loads per thread for one input row, at most, for rows that fit the
// kernel (64 * BPW output pixels at stride S, plus the halo).
constexpr int max_chunks(int KW, int CS, int BPW, int S) { return ((64 * BPW * S + KW - 1) * 4 * CS + THREADS - 1) / THREADS; }

// Four chunks per thread are instantiated only for 1x1 filters: with a
// larger window the row registers no longer fit beside the filter.
constexpr bool wide_rows_ok(int KH) { return KH == 1; }

struct Plan {
    int S, CS, BPW, MAXC, NR, R, slots;
    size_t rows_off, otile_off, lds;
};

// Bytes addressable from one image's base: the extent of the last element.
int64_t image_extent(const int64_t *s, int rows, int cols, int ch, int esz)
{
    return ((int64_t)(rows - 1) * s[1] + (int64_t)(cols - 1) * s[2] + ch) * esz;
}

// The stride the kernel runs with (1 or 2, the same on both axes, no
// dilation), or 0 when the window needs the direct kernel.
int kernel_stride(const DenseProblem &p)
{
    if (p.sh != p.sw || (p.sh != 1 && p.sh != 2) || p.dh != 1 || p.dw != 1)
        return 0;
    return p.sh;
}

bool plan_rows(const DenseProblem &p, Plan *plan)
{
    Plan pl;
    pl.S = kernel_stride(p);
    if (pl.S == 0 || p.xdt != CONV_BF16)
        return false;
    const int cin_g = p.Cin / p.groups, cout_g = p.Cout / p.groups;
    if (cin_g % 8 != 0 || cout_g % 8 != 0)
        return false;
    if ((uintptr_t)p.X % 16 != 0 || p.xs[0] % 8 != 0 || p.xs[1] % 8 != 0 || p.xs[2] % 8 != 0)
        return false;
    if ((uintptr_t)p.F % 16 != 0 || (int64_t)p.KH * p.KW * cin_g * p.Cout * 2 >= (int64_t(1) << 31))
        return false;
    // Output rows leave in 16-byte chunks of 8 (bf16) or 4 (fp32) channels.
    const int yesz = p.ydt == CONV_BF16 ? 2 : 4;
    const int yvec = 16 / yesz;
    if ((uintptr_t)p.Y % 16 != 0 || p.ys[0] % yvec != 0 || p.ys[1] % yvec != 0 || p.ys[2] % yvec != 0)
        return false;
    // Buffer offsets are 32-bit: one image of X and of Y must stay below 2 GB.
    if (image_extent(p.xs, p.H, p.W, p.Cin, 2) >= (int64_t(1) << 31) ||
        image_extent(p.ys, p.Ho, p.Wo, p.Cout, yesz) >= (int64_t(1) << 31))
        return false;
    pl.CS = cin_steps(cin_g);
    if (pl.CS == 0 || !taps_instantiated(p.KH, p.KW, pl.CS, pl.S))
        return false;
    const int blocks = (p.Wo + 15) / 16;
    pl.BPW = (blocks + 3) / 4;
    if (pl.BPW > 2)
        return false;
    const int64_t chunks = (int64_t)p.W * 32 * pl.CS / 8;
    pl.MAXC = chunks <= THREADS ? 1 : chunks <= 2 * THREADS ? 2 : chunks <= 4 * THREADS ? 4 : 0;
    if (pl.MAXC == 0 || (pl.MAXC == 4 && !wide_rows_ok(p.KH)) || pl.MAXC > max_chunks(p.KW, pl.CS, pl.BPW, pl.S))
        return false;
    pl.NR = rows_in_regs(pl.MAXC);
    if (pl.NR < p.KH)
        return false;
    const int rmax = (pl.NR - p.KH) / pl.S + 1;      // output rows a band can hold
    // Bands: aim for about one workgroup per compute unit (256) in total.
    const int tiles = (cout_g + COUT_TILE - 1) / COUT_TILE * p.groups;
    int want = (int)((256 + (int64_t)p.N * tiles - 1) / ((int64_t)p.N * tiles));
    want = want < 1 ? 1 : want > p.Ho ? p.Ho : want;
    const int R = (p.Ho + want - 1) / want;
    pl.R = R < rmax ? R : rmax;
    // A staged row holds the pixels the outputs read and every real pixel.
    const int need = (p.Wo - 1) * pl.S + p.KW;
    pl.slots = need > p.pl + p.W ? need : p.pl + p.W;
    // LDS: [filter staging] [two input rows] [two output tiles] when it
    // fits, else [max(filter staging, two input rows)] [two output tiles].
    const size_t pitch = pl.S == 1 ? (size_t)32 * pl.CS + 16 : (size_t)32 * pl.CS + 8;
    const size_t filt = (size_t)p.KH * p.KW * 32 * pl.CS * (COUT_TILE + 8) * 2;
    const size_t rows = (size_t)(prefetch_rows(p.KW, pl.CS, pl.BPW, pl.MAXC) ? 3 : 2) * pl.slots * pitch * 2;
    const size_t otiles = 2 * (size_t)64 * pl.BPW * (COUT_TILE * yesz + 32);
    if (filt + rows + otiles <= (size_t)LDS_BYTES_MAX) {
        pl.rows_off = filt;
        pl.otile_off = filt + rows;
    } else {
        pl.rows_off = 0;
        pl.otile_off = filt > rows ? filt : rows;
    }
    pl.lds = pl.otile_off + otiles;
    if (pl.lds > (size_t)LDS_BYTES_MAX)
        return false;
    *plan = pl;
    return true;
}

template <int KH, int KW, int CS, int BPW, int MAXC, int S, bool OB>
hipError_t launch_inst(const RowArgs &a, dim3 grid, size_t lds, hipStream_t s)
{
    constexpr int NR = rows_in_regs(MAXC);
    if constexpr (NR < KH) {
        return hipErrorNotSupported;
    } else {
        auto kern = dense_rows_mfma<KH, KW, CS, BPW, MAXC, NR, S, OB>;
        // Allow the full LDS (on the first launch on a device; see allow_lds).
        const hipError_t attr = allow_lds<dense_rows_mfma<KH, KW, CS, BPW, MAXC, NR, S, OB>>(LDS_BYTES_MAX);
        if (attr != hipSuccess)
            return attr;
        hipLaunchKernelGGL(kern, grid, dim3(THREADS), lds, s, a);
        return hipGetLastError();
    }
}

template <int KH, int KW, int CS, int BPW, int S>
hipError_t launch_bpw(const RowArgs &a, dim3 grid, size_t lds, int MAXC, bool ob, hipStream_t s)
{
    constexpr int CMAX = max_chunks(KW, CS, BPW, S);
    if (MAXC == 1)
        return ob ? launch_inst<KH, KW, CS, BPW, 1, S, true>(a, grid, lds, s) : launch_inst<KH, KW, CS, BPW, 1, S, false>(a, grid, lds, s);
    if constexpr (CMAX >= 2) {
        if (MAXC == 2)
            return ob ? launch_inst<KH, KW, CS, BPW, 2, S, true>(a, grid, lds, s) : launch_inst<KH, KW, CS, BPW, 2, S, false>(a, grid, lds, s);
    }
    if constexpr (CMAX >= 3 && wide_rows_ok(KH)) {
        if (MAXC == 4)
            return ob ? launch_inst<KH, KW, CS, BPW, 4, S, true>(a, grid, lds, s) : launch_inst<KH, KW, CS, BPW, 4, S, false>(a, grid, lds, s);
    }
    return hipErrorNotSupported;
}

template <int KH, int KW, int CS>
hipError_t launch_cs(const RowArgs &a, dim3 grid, const Plan &plan, bool ob, hipStream_t s)
{
    if (plan.S == 1)
        return plan.BPW == 1 ? launch_bpw<KH, KW, CS, 1, 1>(a, grid, plan.lds, plan.MAXC, ob, s)
                             : launch_bpw<KH, KW, CS, 2, 1>(a, grid, plan.lds, plan.MAXC, ob, s);
    if constexpr ((KH == 3 && CS <= 2) || (KH == 1 && CS <= 8))
        return plan.BPW == 1 ? launch_bpw<KH, KW, CS, 1, 2>(a, grid, plan.lds, plan.MAXC, ob, s)
                             : launch_bpw<KH, KW, CS, 2, 2>(a, grid, plan.lds, plan.MAXC, ob, s);
    return hipErrorNotSupported;
}

// A 1x1 filter makes every pixel independent: when the pixels of X and Y
// sit at one pixel stride (within each image, or across the whole batch),
// regroup them into rows of 64 (or another width that divides the pixel
// count) so no 16-pixel block of a row is left partly empty. Only for the
// plain window: padding and stride tie outputs to input positions.
DenseProblem regroup_pointwise(const DenseProblem &p)
{
    if (p.KH != 1 || p.KW != 1 || !plain_window(p))
        return p;
    if (p.xs[1] != (int64_t)p.W * p.xs[2] || p.ys[1] != (int64_t)p.Wo * p.ys[2])
        return p;
    const bool batch = p.xs[0] == (int64_t)p.H * p.xs[1] && p.ys[0] == (int64_t)p.Ho * p.ys[1];
    const int64_t pixels = batch ? (int64_t)p.N * p.H * p.W : (int64_t)p.H * p.W;
    int best = 0;
    double best_score = 0;
    for (int w = 16; w <= 128; ++w) {
        if (pixels % w != 0)
            continue;
        const double fill = (double)w / (16.0 * ((w + 15) / 16));
        const double score = fill * (w >= 64 ? 1.0 : (double)w / 64.0) + (w == 64 ? 1e-3 : 0.0);
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
    // Keep the regrouped shape only if the kernel takes it and the original
    // one is worse off (a row of the original already fills its blocks).
    Plan a, b;
    const bool ok_q = plan_rows(q, &a);
    const bool ok_p = plan_rows(p, &b);
    if (!ok_q)
        return p;
    if (ok_p && p.Wo % 16 == 0 && p.Wo >= 64)
        return p;
    return q;
}

}  // namespace

// Small groups (grouped convolution between dense and depthwise, "Convolution
// Is Wx+b Moving Across a Signal", section "Find the same sum in CKE's C
// kernels"): when every group has G = 8, 16 or 32 input and output channels,
// 64 / G groups share one 64-channel tile with a block-diagonal filter. X is
// then read once, in whole 128-byte pixel rows, instead of once per group in
// G-channel slivers; the extra matrix-core work multiplies zeros.
int pack_groups(const DenseProblem &p, DenseProblem *q)
{
    if (p.groups <= 1 || p.Cin != p.Cout || p.Cin % 64 != 0)
        return 0;
    const int g = p.Cin / p.groups;
    if (g != 8 && g != 16 && g != 32)
        return 0;
    *q = p;
    q->groups = p.Cin / 64;
    return g;
}

bool dense_mfma_bf16_supports(const DenseProblem &p)
{
    Plan plan;
    DenseProblem q;
    if (pack_groups(p, &q) && (dense_band_supports(q) || plan_rows(q, &plan)))
        return true;
    return dense_pw_supports(p) || dense_band_supports(p) || plan_rows(regroup_pointwise(p), &plan);
}

hipError_t launch_dense_mfma_bf16(const DenseProblem &p0, hipStream_t s)
{
    Plan plan;
    DenseProblem packed;
    const int gpack = pack_groups(p0, &packed);
    // Unit-stride windows with bf16 output and rows of at most 64 pixels run
    // on the band kernel (dense_band_mfma.hip), which requests the whole
    // band of input rows up front.
    if (gpack != 0 && dense_band_supports(packed))
        return launch_dense_band(packed, gpack, s);
    if (dense_band_supports(p0))
        return launch_dense_band(p0, 0, s);
    // Pointwise layers whose pixels sit at one stride: the GEMM kernel
    // (dense_pw_mfma.hip).
    if (dense_pw_supports(p0))
        return launch_dense_pw(p0, s);
    const bool use_pack = gpack != 0 && plan_rows(packed, &plan);
    const DenseProblem p = use_pack ? packed : regroup_pointwise(p0);
    if (!use_pack && !plan_rows(p, &plan))
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
    a.Ho = p.Ho;
    a.Wo = p.Wo;
    a.Cin = p.Cin / p.groups;
    a.Cout = p.Cout / p.groups;
    a.f_ld = p.Cout;
    a.gpack = use_pack ? gpack : 0;
    a.pt = p.pt;
    a.pl = p.pl;
    a.groups = p.groups;
    a.row_slots = plan.slots;
    a.row_elems = plan.slots * (plan.S == 1 ? 32 * plan.CS + 16 : 32 * plan.CS + 8);
    a.chunks_per_row = p.W * 32 * plan.CS / 8;
    a.otile_off = (int)plan.otile_off;
    a.rows_off = (int)(plan.rows_off / 2);
    a.x_records = (uint32_t)image_extent(p.xs, p.H, p.W, p.Cin, 2);
    a.y_records = (uint32_t)image_extent(p.ys, p.Ho, p.Wo, p.Cout, p.ydt == CONV_BF16 ? 2 : 4);
    a.R = plan.R;
    a.bands_per_img = (p.Ho + a.R - 1) / a.R;
    a.bands = p.N * a.bands_per_img;
    a.tiles = (a.Cout + COUT_TILE - 1) / COUT_TILE;
    // One slot per (band, group, tile), bands padded to a multiple of 8 (the
    // padding slots exit at once) for the XCD-aware slot map.
    const int64_t slots = (int64_t)((a.bands + 7) / 8 * 8) * a.tiles * a.groups;
    if (slots >= (int64_t(1) << 31))
        return hipErrorNotSupported;
    const dim3 grid((unsigned)slots);
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
