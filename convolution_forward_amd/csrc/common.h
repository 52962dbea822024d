// Small device helpers shared by the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace convfwd {

// bf16 is the upper 16 bits of an IEEE binary32.
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Round a binary32 to bf16, nearest-even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u)
        return (uint16_t)((u >> 16) | 0x0040u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float load_as_f32(const float *p) { return *p; }
__device__ __forceinline__ float load_as_f32(const uint16_t *p) { return bf16_to_f32(*p); }

__device__ __forceinline__ void store_from_f32(float *p, float v) { *p = v; }
__device__ __forceinline__ void store_from_f32(uint16_t *p, float v) { *p = f32_to_bf16_rne(v); }

// Grid size for a grid-stride loop over `total` items: enough blocks to fill
// the chip several times, never more than the work needs.
inline unsigned grid_for(int64_t total, int block, int64_t cap = 256 * 64)
{
    int64_t blocks = (total + block - 1) / block;
    if (blocks > cap)
        blocks = cap;
    if (blocks < 1)
        blocks = 1;
    return (unsigned)blocks;
}

}  // namespace convfwd
