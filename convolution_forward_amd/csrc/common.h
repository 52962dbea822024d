// Small device helpers shared by the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

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

// Raise kernel Kern's dynamic LDS limit to `bytes` on the current device
// before its first launch there. Only a success is remembered (one bit per
// device and kernel), so a failed attempt is made again by the next call;
// later calls (graph capture included) then make no HIP call at all.
// Bring every 64-byte line of a kernel's argument block (up to 256 bytes)
// into the scalar cache with one batch of scalar loads at the kernel's
// start: x passes through an asm that takes one word of each line as input,
// so everything computed from the returned value waits for that one batch.
// Left alone, the compiler loads each argument just before its first use,
// behind the branches that need the earlier ones, so a kernel paid one
// memory round trip per such step before its first global load. The asm is
// not volatile and touches no memory, so loads after it can still be proven
// free of stores (uniform loads then stay scalar loads).
template <class T>
__device__ __forceinline__ int with_args_loaded(int x, const T &a)
{
    static_assert(sizeof(T) <= 256, "four lines at most");
    const uint32_t *p = reinterpret_cast<const uint32_t *>(&a);
    constexpr int L = (int)(sizeof(T) / 4) - 1;
    asm("" : "+s"(x) : "s"(p[0]), "s"(p[16 < L ? 16 : L]), "s"(p[32 < L ? 32 : L]), "s"(p[48 < L ? 48 : L]));
    return x;
}

template <auto Kern>
hipError_t allow_lds(int bytes)
{
    static std::atomic<uint64_t> done{0};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    const uint64_t bit = dev >= 0 && dev < 64 ? uint64_t(1) << dev : 0;
    if (bit && (done.load(std::memory_order_acquire) & bit))
        return hipSuccess;
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(Kern), hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess && bit)
        done.fetch_or(bit, std::memory_order_acq_rel);
    return e;
}

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
