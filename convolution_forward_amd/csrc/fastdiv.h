// Division by a divisor fixed for a whole launch (the depthwise kernels'
// plane, row and channel indexing): n / d for 0 <= n < 2^31 as a multiply-
// high, an add and a shift (Granlund and Montgomery, "Division by invariant
// integers using multiplication", 1994). The host picks m and s once per
// launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace convfwd {

struct FastDiv {
    uint32_t m, s;
};

// s = ceil(log2 d), m = floor(2^32 * (2^s - d) / d) + 1, for 1 <= d < 2^31.
inline FastDiv make_fastdiv(uint32_t d)
{
    uint32_t s = 0;
    while ((1ull << s) < d)
        ++s;
    const uint64_t m = ((1ull << 32) * ((1ull << s) - d)) / d + 1;
    return FastDiv{(uint32_t)m, s};
}

// umulhi(n, m) < n, so the sum stays below 2^32 for n < 2^31.
__device__ __forceinline__ uint32_t fdiv(uint32_t n, FastDiv f) { return (__umulhi(n, f.m) + n) >> f.s; }

}  // namespace convfwd
