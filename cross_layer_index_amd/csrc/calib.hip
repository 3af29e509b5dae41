// Calibration kernel: one pass of plain coalesced reads over a buffer,
// nothing else. Its time is the floor of a single launch that streams that
// many bytes (the decode indexer streams 16 MiB of keys per query), the
// reference its own roofline figures are read against.
#include "kernels.h"

namespace ic {
namespace {

constexpr int kCalThreads = 256;
constexpr int kCalLoads = 8;                          // 16-byte loads per thread
constexpr int64_t kCalChunk = (int64_t)kCalThreads * kCalLoads * 16;   // bytes per workgroup

// grid: ceil(bytes / kCalChunk); each workgroup reads one contiguous chunk,
// load i of every thread covering a contiguous 4 KiB slab. The loads feed an
// xor that decides a store which never happens for real data, so none of
// them can be dropped.
__global__ __launch_bounds__(kCalThreads) void stream_read_kernel(const uint4 *__restrict__ src, int64_t n16,
                                                                  uint32_t *__restrict__ sink)
{
    const int64_t base = (int64_t)blockIdx.x * (kCalChunk / 16) + threadIdx.x;
    uint4 v[kCalLoads];
#pragma unroll
    for (int i = 0; i < kCalLoads; ++i) {
        const int64_t j = base + (int64_t)i * kCalThreads;
        v[i] = j < n16 ? src[j] : make_uint4(0, 0, 0, 0);
    }
    uint32_t acc = 0;
#pragma unroll
    for (int i = 0; i < kCalLoads; ++i)
        acc ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
    if (acc == 0x9E3779B9u && threadIdx.x == 0)
        sink[blockIdx.x & 63] = acc;
}

}  // namespace

hipError_t launch_stream_read(const void *src, int64_t bytes, uint32_t *sink, hipStream_t stream)
{
    const int64_t n16 = bytes / 16;
    const int64_t grid = (bytes + kCalChunk - 1) / kCalChunk;
    if (grid == 0)
        return hipSuccess;
    if (!trace_skip("stream_read_kernel"))
        hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)grid), dim3(kCalThreads), 0, stream,
                           reinterpret_cast<const uint4 *>(src), n16, sink);
    trace_launch(stream, "stream_read_kernel");
    return hipGetLastError();
}

}  // namespace ic
