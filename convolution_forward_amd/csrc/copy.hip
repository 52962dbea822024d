// A plain streaming copy: 16-byte loads and stores, grid-stride. It is not
// part of the convolution; it measures the achievable HBM bandwidth and
// calibrates the memory-traffic counters against a known byte count.
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

}  // namespace

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
