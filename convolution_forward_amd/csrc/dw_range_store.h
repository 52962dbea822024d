// The last step of the small-plane depthwise kernels: a workgroup's outputs
// are one contiguous range of Y, left in LDS by its threads, and written out
// in aligned 16-byte pieces with streaming stores.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace convfwd {

// Y elements [ostart, ostart + olen) sit at LDS words [lead, lead + olen),
// where lead = ostart mod 4 if Y is 16-byte aligned (else 0), so LDS words
// 4c..4c+3 are one aligned 16-byte piece of Y. MAXWORDS bounds lead + olen.
// Pieces c = tid, tid + NT, ...: all read, then all stored; only the first
// and the last piece can be partial.
template <int NT, int MAXWORDS>
__device__ __forceinline__ void store_range_from_lds(const float *lds, float *Y, int64_t ostart, int olen, int lead,
                                                     bool y_aligned, int tid)
{
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    if (y_aligned) {
        constexpr int NPC = (MAXWORDS + 4 * NT - 1) / (4 * NT);
        float *yb = Y + (ostart - lead);
        const int end = lead + olen;
        f32x4 ov[NPC];
#pragma unroll
        for (int i = 0; i < NPC; ++i) {
            const int e0 = 4 * (tid + i * NT);
            if (e0 < end)
                ov[i] = *reinterpret_cast<const f32x4 *>(lds + e0);
        }
#pragma unroll
        for (int i = 0; i < NPC; ++i) {
            const int e0 = 4 * (tid + i * NT);
            if (e0 >= lead && e0 + 4 <= end) {
                __builtin_nontemporal_store(ov[i], reinterpret_cast<f32x4 *>(yb + e0));
            } else if (e0 < end) {
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    if (e0 + k >= lead && e0 + k < end)
                        yb[e0 + k] = ov[i][k];
            }
        }
    } else {
        for (int e = tid; e < olen; e += NT)
            __builtin_nontemporal_store(lds[e], &Y[ostart + e]);
    }
}

}  // namespace convfwd
