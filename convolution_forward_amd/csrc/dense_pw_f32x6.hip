// Dense 1x1 convolution with fp32 operands and fp32 output, computed on the
// bf16 matrix cores.
//
// Contract: "CMU DLSys Lecture 14: Convolutional Network Implementation",
// section 1 (Y[n,y,x,o] = sum over c of X[n,y,x,c] * F[0,0,c,o] for a 1x1
// filter); section 2 notes that K = 1 is a single matrix product of the
// pixels' channel vectors with F. Here it is that product, pixels at one
// stride in X and in Y.
//
// Precision. Each fp32 value v is split exactly into three bf16 parts by
// truncation: vh = v with the low 16 bits cleared, r = v - vh (exact),
// vm = r with the low 16 bits cleared, vl = r - vm (exact, at most 8
// significant bits, so a bf16). Of the nine products of X's and F's parts,
// the six whose size can matter (h*h, h*m, m*h, h*l, m*m, l*h) are summed by
// v_mfma_f32_16x16x32_bf16 with fp32 accumulation; each of the three
// dropped ones is below 2^-24 of |x*w| (the splitting of fp32 into bf16
// parts for fp32-accurate products follows Henry, Tang and Heinecke,
// "Leveraging the bfloat16 Artificial Intelligence Datatype For
// Higher-Precision Computations", 2019). The bf16 matrix rate is 16x the
// fp32 one, so six bf16 products cost 6/16 of one fp32 product. Integer-
// valued inputs up to 2^8 have zero middle and low parts, so their sums
// are exact as in fp32. A NaN input gives NaN outputs; an output that fp32
// arithmetic makes infinite comes out as NaN here (an infinite input's
// middle part is inf - inf). Non-finite outputs stay non-finite and finite
// ones finite.
//
// Work: a workgroup (4 waves) owns 208 pixels (13 blocks of 16) x 128 output
// channels; wave w computes every pixel block x channels 32 w .. +31 as
// 13 x 2 tiles of 16 x 16. At the 1x1 workload that is 121 x 4 = 484
// workgroups, one round at two per compute unit (128-pixel tiles made 784,
// 1.53 rounds). The input channels go in chunks of 32: each chunk of X
// and F is loaded into registers (16-byte loads, one chunk ahead, while
// the current one is multiplied), split, and written to LDS as three bf16
// planes of each: X as [pixel][channel] (B operand, 16-byte reads), F as
// [channel][output] (A operand, gfx950 transposed reads).
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

constexpr int BT = 256;
constexpr int PB = 13;                  // 16-pixel blocks per tile
constexpr int TP = 16 * PB;             // pixel slots per tile (208)
constexpr int TO = 128;                 // output channels per tile
constexpr int KC = 32;                  // input channels per chunk
constexpr int XP = KC + 8;              // LDS pitch of a staged pixel (80 bytes: 16 lanes on distinct banks)
constexpr int FP = TO + 8;              // LDS pitch of a staged filter row (272 bytes)
constexpr int XPART = TP * XP;          // elements of one X plane
constexpr int FPART = KC * FP;          // elements of one F plane
constexpr size_t LDS_BYTES = (size_t)(3 * XPART + 3 * FPART) * 2;
constexpr uint32_t OOB = 0x80000000u;
// Output stores: device-scope write-through with the streaming hint (sc1 |
// nt). Every workgroup finishes its products at about the same time and the
// output (two thirds of the layer's bytes) then drains at once: 47.0 ->
// 42.4 us at the 1x1 workload against the default policy (nt alone 43.5,
// sc1 alone 44.2).
constexpr int SAUX = 18;
constexpr int BUF_WORD3 = 0x00020000;

struct F32x6Args {
    const float *X;
    const float *F;
    const float *bias;
    float *Y;
    int npix;           // pixels of the batch
    int xs, ys;         // pixel strides of X and Y (elements)
    int Cin, Cout;
    int ptiles, otiles;
    int xcd_stride;     // grid / 8: workgroup b takes slot (b % 8) * xcd_stride + b / 8
    uint32_t x_records, y_records;
};

// The three bf16 parts of four fp32 values, packed two per word: four
// vector operations per value (two masks, two exact subtractions) and one
// byte permute per pair and part (the high halves of two words). A NaN
// input leaves NaN in its middle part (NaN - x), so NaN propagates; an
// infinite one leaves infinity in its high part and NaN in its middle part.
__device__ __forceinline__ void split4(const u32x4 v, u32x2 &h, u32x2 &m, u32x2 &l)
{
    uint32_t r1[4], r2[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float x1 = __uint_as_float(v[i]) - __uint_as_float(v[i] & 0xFFFF0000u);
        r1[i] = __float_as_uint(x1);
        r2[i] = __float_as_uint(x1 - __uint_as_float(r1[i] & 0xFFFF0000u));
    }
    constexpr uint32_t HI = 0x07060302u;     // bytes 2, 3 of the first word, then of the second
    h = u32x2{__builtin_amdgcn_perm(v[1], v[0], HI), __builtin_amdgcn_perm(v[3], v[2], HI)};
    m = u32x2{__builtin_amdgcn_perm(r1[1], r1[0], HI), __builtin_amdgcn_perm(r1[3], r1[2], HI)};
    l = u32x2{__builtin_amdgcn_perm(r2[1], r2[0], HI), __builtin_amdgcn_perm(r2[3], r2[2], HI)};
}

__global__ __launch_bounds__(BT) __attribute__((amdgpu_waves_per_eu(2, 2))) void dense_pw_f32x6(F32x6Args a)
{
    extern __shared__ __align__(16) uint16_t lds[];
    uint16_t *xl = lds;                 // [3][TP][XP]
    uint16_t *fl = lds + 3 * XPART;     // [3][KC][FP]
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int bid = with_args_loaded((int)blockIdx.x, a);
    const int slot = (bid & 7) * a.xcd_stride + (bid >> 3);
    const int pt = slot / a.otiles;
    const int ot = slot - pt * a.otiles;
    if (pt >= a.ptiles)
        return;
    const int p0 = pt * TP;
    const int pend = min(a.npix, p0 + TP);     // one past the tile's last pixel
    const int o0 = ot * TO;

    const __amdgpu_buffer_rsrc_t xr =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(a.X), 0, (int)a.x_records, BUF_WORD3);
    const __amdgpu_buffer_rsrc_t fr =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(a.F), 0, a.Cin * a.Cout * 4, BUF_WORD3);
    const __amdgpu_buffer_rsrc_t yr = __builtin_amdgcn_make_buffer_rsrc(a.Y, 0, (int)a.y_records, BUF_WORD3);

    // Chunk loads: X unit u = tid + 256 i (u < 8 TP) is pixel u / 8,
    // channels 4 (u % 8) of the chunk; F unit u is chunk channel u / 32,
    // outputs 4 (u % 32). Chunk k + 1 loads while chunk k is multiplied (a
    // second register set, two chunks ahead, did not fit beside the 104
    // accumulator registers without spilling).
    constexpr int XU = (8 * TP + BT - 1) / BT;      // X loads per thread
    u32x4 xa[XU], fa[4];
    auto load = [&](const int k0, u32x4 (&xv)[XU], u32x4 (&fv)[4]) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < XU; ++i) {
            const int u = tid + BT * i;
            const int px = p0 + (u >> 3);
            const int c = k0 + 4 * (u & 7);
            const bool ok = u < 8 * TP && px < pend && c < a.Cin;
            xv[i] = __builtin_amdgcn_raw_buffer_load_b128(xr, ok ? (uint32_t)(px * a.xs + c) * 4u : OOB, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int u = tid + BT * i;
            const int c = k0 + (u >> 5);
            const int o = o0 + 4 * (u & 31);
            const bool ok = c < a.Cin && o < a.Cout;
            fv[i] = __builtin_amdgcn_raw_buffer_load_b128(fr, ok ? (uint32_t)(c * a.Cout + o) * 4u : OOB, 0, 0);
        }
    };
    auto stage = [&](const u32x4 (&xv)[XU], const u32x4 (&fv)[4]) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < XU; ++i) {
            const int u = tid + BT * i;
            if (u < 8 * TP) {
                u32x2 h, m, l;
                split4(xv[i], h, m, l);
                uint16_t *d = xl + (u >> 3) * XP + 4 * (u & 7);
                *reinterpret_cast<u32x2 *>(d) = h;
                *reinterpret_cast<u32x2 *>(d + XPART) = m;
                *reinterpret_cast<u32x2 *>(d + 2 * XPART) = l;
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int u = tid + BT * i;
            u32x2 h, m, l;
            split4(fv[i], h, m, l);
            uint16_t *d = fl + (u >> 5) * FP + 4 * (u & 31);
            *reinterpret_cast<u32x2 *>(d) = h;
            *reinterpret_cast<u32x2 *>(d + FPART) = m;
            *reinterpret_cast<u32x2 *>(d + 2 * FPART) = l;
        }
    };

    const int oq = wave;                // the wave's 32 output channels: 32 oq .. +31
    const int g = lane >> 4;            // k-group: chunk channels 8g .. 8g + 7
    const int r = lane & 15;
    f32x4 acc[PB][2];
#pragma unroll
    for (int pb = 0; pb < PB; ++pb)
#pragma unroll
        for (int ob = 0; ob < 2; ++ob)
            acc[pb][ob] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute = [&]() __attribute__((always_inline)) {
        // A fragments of output channels 32 oq + 16 ob + (0..15): within each
        // 16-lane group of the transposed read, lane r addresses row r / 4
        // and columns 4 (r % 4) .. +3 of a 4-row block and receives four
        // consecutive chunk channels of output channel r; two reads give
        // the lane's eight.
        bf16x8 wa[2][3];
#pragma unroll
        for (int ob = 0; ob < 2; ++ob)
#pragma unroll
            for (int q = 0; q < 3; ++q) {
                i16x4 part[2];
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int c = g * 8 + hh * 4 + (r >> 2);
                    const int o = oq * 32 + ob * 16 + 4 * (r & 3);
                    part[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) i16x4 *)(fl + q * FPART + c * FP + o));
                }
                const i16x8 both = {part[0][0], part[0][1], part[0][2], part[0][3],
                                    part[1][0], part[1][1], part[1][2], part[1][3]};
                wa[ob][q] = __builtin_bit_cast(bf16x8, both);
            }
#pragma unroll
        for (int pb = 0; pb < PB; ++pb) {
            // B fragments: pixel 16 pb + r of the tile, chunk channels 8g .. 8g + 7.
            bf16x8 xb[3];
#pragma unroll
            for (int q = 0; q < 3; ++q)
                xb[q] = *reinterpret_cast<const bf16x8 *>(xl + q * XPART + (pb * 16 + r) * XP + 8 * g);
#pragma unroll
            for (int ob = 0; ob < 2; ++ob) {
                // Smallest products first.
                f32x4 t = acc[pb][ob];
                t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[ob][2], xb[0], t, 0, 0, 0);   // l * h
                t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[ob][1], xb[1], t, 0, 0, 0);   // m * m
                t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[ob][0], xb[2], t, 0, 0, 0);   // h * l
                t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[ob][1], xb[0], t, 0, 0, 0);   // m * h
                t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[ob][0], xb[1], t, 0, 0, 0);   // h * m
                t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[ob][0], xb[0], t, 0, 0, 0);   // h * h
                acc[pb][ob] = t;
            }
        }
    };
    const int nk = (a.Cin + KC - 1) / KC;
    load(0, xa, fa);
    for (int k = 0; k < nk; ++k) {
        if (k > 0)
            __syncthreads();            // every wave is done with chunk k - 1
        stage(xa, fa);
        __syncthreads();
        if (k + 1 < nk)
            load((k + 1) * KC, xa, fa);
        compute();
    }

    // Lane (g, r) of tile (pb, ob) holds output channels 32 oq + 16 ob + 4 g
    // + (0..3) of pixel 16 pb + r of the tile: one 16-byte store each.
#pragma unroll
    for (int ob = 0; ob < 2; ++ob) {
        const int o = o0 + oq * 32 + ob * 16 + 4 * g;
        f32x4 bv = {0.f, 0.f, 0.f, 0.f};
        if (a.bias && o < a.Cout)
            bv = *reinterpret_cast<const f32x4 *>(a.bias + o);
#pragma unroll
        for (int pb = 0; pb < PB; ++pb) {
            const int px = p0 + pb * 16 + r;
            const f32x4 v = acc[pb][ob];
            const u32x4 w = {__float_as_uint(v[0] + bv[0]), __float_as_uint(v[1] + bv[1]),
                             __float_as_uint(v[2] + bv[2]), __float_as_uint(v[3] + bv[3])};
            const bool ok = px < pend && o < a.Cout;
            __builtin_amdgcn_raw_buffer_store_b128(w, yr, ok ? (uint32_t)(px * a.ys + o) * 4u : OOB, 0, SAUX);
        }
    }
}

struct F32x6Plan {
    int64_t npix;
    int ptiles, otiles;
};

bool plan_f32x6(const DenseProblem &p, F32x6Plan *pl)
{
    if (p.KH != 1 || p.KW != 1 || !plain_window(p) || p.xdt != CONV_F32 || p.ydt != CONV_F32)
        return false;
    if (p.Cin % 4 != 0 || p.Cout % 4 != 0)
        return false;       // whole 16-byte pieces of channels
    // Every pixel of the batch at one stride, in X and in Y.
    if (p.xs[1] != (int64_t)p.W * p.xs[2] || p.xs[0] != (int64_t)p.H * p.xs[1] ||
        p.ys[1] != (int64_t)p.Wo * p.ys[2] || p.ys[0] != (int64_t)p.Ho * p.ys[1])
        return false;
    if ((uintptr_t)p.X % 16 || (uintptr_t)p.F % 16 || (uintptr_t)p.Y % 16 || (p.bias && (uintptr_t)p.bias % 16) ||
        p.xs[2] % 4 || p.ys[2] % 4)
        return false;
    const int64_t npix = (int64_t)p.N * p.H * p.W;
    if (((npix - 1) * p.xs[2] + p.Cin) * 4 >= (int64_t(1) << 31) ||
        ((npix - 1) * p.ys[2] + p.Cout) * 4 >= (int64_t(1) << 31) || (int64_t)p.Cin * p.Cout * 4 >= (1ll << 31))
        return false;
    pl->npix = npix;
    pl->otiles = (p.Cout + TO - 1) / TO;
    pl->ptiles = (int)((npix + TP - 1) / TP);
    return (int64_t)pl->ptiles * pl->otiles + 8 < (1ll << 31);
}

}  // namespace

bool dense_f32x6_supports(const DenseProblem &p)
{
    F32x6Plan pl;
    return plan_f32x6(p, &pl);
}

hipError_t launch_dense_f32x6(const DenseProblem &p, hipStream_t s)
{
    F32x6Plan pl;
    if (!plan_f32x6(p, &pl))
        return hipErrorNotSupported;
    F32x6Args a;
    a.X = static_cast<const float *>(p.X);
    a.F = static_cast<const float *>(p.F);
    a.bias = p.bias;
    a.Y = static_cast<float *>(p.Y);
    a.npix = (int)pl.npix;
    a.xs = (int)p.xs[2];
    a.ys = (int)p.ys[2];
    a.Cin = p.Cin;
    a.Cout = p.Cout;
    a.ptiles = pl.ptiles;
    a.otiles = pl.otiles;
    a.x_records = (uint32_t)(((pl.npix - 1) * p.xs[2] + p.Cin) * 4);
    a.y_records = (uint32_t)(((pl.npix - 1) * p.ys[2] + p.Cout) * 4);
    // Slots (pixel tile, output tile) with the output tiles of one pixel
    // tile on one XCD, so that their common X meets in that XCD's L2.
    const int64_t slots = ((int64_t)pl.ptiles * pl.otiles + 7) / 8 * 8;
    a.xcd_stride = (int)(slots / 8);
    const hipError_t attr = allow_lds<dense_pw_f32x6>((int)LDS_BYTES);
    if (attr != hipSuccess)
        return attr;
    hipLaunchKernelGGL(dense_pw_f32x6, dim3((unsigned)slots), dim3(BT), LDS_BYTES, s, a);
    return hipGetLastError();
}

}  // namespace convfwd
