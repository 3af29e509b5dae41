// Order-preserving 32-bit image of an fp32 score, shared by the producers of
// the first-digit histogram (indexer) and by the top-k selection: larger
// floats give larger unsigned keys, and -0 maps to the key of +0.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ic {

__device__ __forceinline__ uint32_t ord_key(float x)
{
    uint32_t u = __float_as_uint(x);
    if (u == 0x80000000u)
        u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int kHistBins0 = 2048;      // first radix digit: key bits 31..21
constexpr int kHistShift0 = 21;
constexpr int kHistCopies = 8;        // copies of each query's histogram

}  // namespace ic
