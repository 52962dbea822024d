// Copies that are not part of the convolution. The plain streaming copy
// (16-byte loads and stores, grid-stride) calibrates the memory-traffic
// counters against a known byte count; it and the wide copy below (many
// loads in flight per thread) measure what the memory system delivers at the
// byte counts of one convolution.
#include "common.h"
#include "internal.h"

namespace convfwd {
namespace {

__global__ __launch_bounds__(256) void copy_vec16_kernel(const uint4 *__restrict__ src, uint4 *__restrict__ dst,
                                                         int64_t n16)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
        dst[i] = src[i];
}

__global__ __launch_bounds__(256) void copy_bytes_kernel(const uint8_t *__restrict__ src, uint8_t *__restrict__ dst,
                                                         int64_t n)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        dst[i] = src[i];
}

// The same bytes moved with as much in flight as the chip takes: a thread
// owns U consecutive 16-byte pieces strided by the workgroup's width, issues
// all U loads before the first store, and the grid holds every piece once
// (no grid-stride loop: at the sizes of one convolution all workgroups are
// resident together). Stores carry the device-scope write-through and
// streaming hints (sc1 | nt), the policy measured fastest for whole-line
// stores. Offsets past the end read zeros and store nothing (buffer range).
template <int U>
__global__ __launch_bounds__(256) void copy_wide_kernel(const uint8_t *__restrict__ src, uint8_t *__restrict__ dst,
                                                        int64_t n16)
{
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const int64_t base16 = (int64_t)blockIdx.x * (256 * U);
    const int64_t left = n16 - base16;
    const int records = (int)((left < 256 * U ? left : 256 * U) * 16);
    const __amdgpu_buffer_rsrc_t sr =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(src) + base16 * 16, 0, records, 0x00020000);
    const __amdgpu_buffer_rsrc_t dr = __builtin_amdgcn_make_buffer_rsrc(dst + base16 * 16, 0, records, 0x00020000);
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
        v[u] = __builtin_amdgcn_raw_buffer_load_b128(sr, (uint32_t)((u * 256 + threadIdx.x) * 16), 0, 0);
#pragma unroll
    for (int u = 0; u < U; ++u)
        __builtin_amdgcn_raw_buffer_store_b128(v[u], dr, (uint32_t)((u * 256 + threadIdx.x) * 16), 0, 18);
}

}  // namespace

hipError_t launch_copy_wide(const void *src, void *dst, int64_t bytes, hipStream_t s)
{
    constexpr int U = 8;
    const int64_t n16 = bytes / 16;
    const int64_t blocks = (n16 + 256 * U - 1) / (256 * U);
    if (blocks >= (int64_t(1) << 31))
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(copy_wide_kernel<U>, dim3((unsigned)blocks), dim3(256), 0, s,
                       static_cast<const uint8_t *>(src), static_cast<uint8_t *>(dst), n16);
    return hipGetLastError();
}

hipError_t launch_copy_bytes(const void *src, void *dst, int64_t bytes, hipStream_t s)
{
    const int block = 256;
    const bool aligned = ((uintptr_t)src % 16 == 0) && ((uintptr_t)dst % 16 == 0);
    const int64_t n16 = aligned ? bytes / 16 : 0;
    if (n16 > 0)
        hipLaunchKernelGGL(copy_vec16_kernel, dim3(grid_for(n16, block, 256 * 32)), dim3(block), 0, s,
                           static_cast<const uint4 *>(src), static_cast<uint4 *>(dst), n16);
    const int64_t done = n16 * 16;
    if (bytes > done)
        hipLaunchKernelGGL(copy_bytes_kernel, dim3(grid_for(bytes - done, block)), dim3(block), 0, s,
                           static_cast<const uint8_t *>(src) + done, static_cast<uint8_t *>(dst) + done,
                           bytes - done);
    return hipGetLastError();
}

}  // namespace convfwd
