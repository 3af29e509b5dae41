// LDS DMA fills the compiler does not track, and exact waits for them,
// shared by the kernels that stage global rows in LDS through
// global_load_lds: the sparse MLA's row gathers and the shared-key
// indexer's key tiles.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ic {
namespace {

// s_waitcnt on the vector-memory counter only (expcnt and lgkmcnt left at max)
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// One 64-lane LDS fill (global_load_lds, 16 bytes a lane): lane l's bytes
// base + voff land at LDS byte address lds + 16 l. Written as inline asm so
// that the compiler does not track it: with several buffers in flight its
// own alias bookkeeping for such fills falls back to waiting for all of them
// before a read of any buffer. The fill has no register result; the waits
// for it are the explicit ones in the tile loops (and any wait the compiler
// places for its own loads only waits longer). M0 is written in the same
// block, one wait state before its use.
__device__ __forceinline__ void lds_fill16(const void *base, uint32_t voff, uint32_t lds)
{
    // base and lds are the same in every lane (a wave's fill has one source
    // base and one LDS span); say so to the compiler, which keeps them in
    // scalar registers, M0 for the LDS address
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    const uint64_t bs = (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b) |
                        ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32)) << 32);
    asm volatile("s_nop 0\n\t"
                 "global_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(voff), "s"(bs), "{m0}"(__builtin_amdgcn_readfirstlane((int)lds))
                 : "memory");
}

}  // namespace
}  // namespace ic
