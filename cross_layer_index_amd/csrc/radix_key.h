// Order-preserving 32-bit image of an fp32 score, shared by the producers of
// the first-digit histogram (indexer) and by the top-k selection: larger
// floats give larger unsigned keys, and -0 maps to the key of +0. Also a
// wave-aggregated LDS histogram add.
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

// Adds one count to LDS histogram bin `b` for every lane with `live` set.
// Scores crowd into a few first-digit bins, so the lanes of one LDS atomic
// mostly hit the same address and serialise: the wave adds the bin of its
// first remaining live lane with one atomic for all lanes that share it, twice
// over, then the rest one by one. It uses ballots: lanes that do not execute it
// add nothing.
__device__ __forceinline__ void hist_add_wave(uint32_t *hist, uint32_t b, bool live)
{
    bool rest = live;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const uint64_t pm = __ballot(rest);
        if (pm == 0)
            break;
        const uint32_t lead = __builtin_amdgcn_readlane(b, __builtin_ctzll(pm));
        const bool same = rest && b == lead;
        const uint64_t m = __ballot(same);
        if (same && (m & __lanemask_lt()) == 0)
            atomicAdd(&hist[lead], (uint32_t)__popcll(m));
        rest = rest && !same;
    }
    if (rest)
        atomicAdd(&hist[b], 1u);
}

constexpr int kHistBins0 = 2048;      // first radix digit: key bits 31..21
constexpr int kHistShift0 = 21;
constexpr int kHistCopies = 8;        // copies of each query's histogram

}  // namespace ic
