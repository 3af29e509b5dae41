// Gated head output on bf16 matrix cores.
//
//   out[t,h,e] = sigmoid(gate[t,h,e]) * sum_c wv_b[h,e,c] * o[t,h,c]
//
// (GitHub issue "rtx6kpro #90", bullet on the elementwise sigmoid gate: the
// gate multiplies the decompressed per-head attention output before o_proj,
// so the latent output o of the sparse attention is first taken through the
// head's value up-projection wv_b; folding wv_b into o_proj would gate in the
// wrong space.)
//
// A workgroup owns one head, a run of 16-query blocks and 64 output columns;
// each of its 4 waves one 16-column tile. v_mfma_f32_16x16x32_bf16 with queries on M and
// output columns on N: A lane l holds o[t0 + l%16][h][32*ks + 8*(l/16) .. +8],
// B lane l holds wv_b[h][e + l%16][32*ks + 8*(l/16) .. +8] -- both contiguous
// 16-byte loads, since the contraction runs along the rows of o and wv_b.
// Accumulator element r of lane l is (query 4*(l/16) + r, column l%16).
// Workgroups of one head share its wv_b rows through one L2: the grid's x
// extent is a multiple of 8, so a head's workgroups stay on one XCD.
#include "kernels.h"

namespace ic {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kGateThreads = 256;
constexpr int kGateRows = 16;          // queries per workgroup
constexpr int kGateCols = 64;          // output columns per workgroup

__device__ __forceinline__ float bf16_to_f32(uint16_t b)
{
    return __uint_as_float((uint32_t)b << 16);
}

__device__ __forceinline__ uint16_t f32_to_bf16(float f)
{
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);                 // round to nearest even
    return (uint16_t)(u >> 16);
}

// grid: (H * D_o / 64, query chunks); a workgroup takes `blocks` consecutive
// 16-query blocks of one head and 64 columns. Each wave keeps its wv_b
// fragments (16 columns x D_v) in registers for the whole chunk and loads the
// next block's o fragments while the current block multiplies.
template <int DV>
__global__ __launch_bounds__(kGateThreads) void gated_output_kernel(const uint16_t *__restrict__ o,
                                                                    const uint16_t *__restrict__ wv_b,
                                                                    const uint16_t *__restrict__ gate, int32_t T,
                                                                    int32_t H, int32_t D_o, int32_t blocks,
                                                                    uint16_t *__restrict__ out)
{
    constexpr int KS = DV / 32;
    const int colblocks = D_o / kGateCols;
    const int h = blockIdx.x / colblocks;
    const int e0 = (blockIdx.x % colblocks) * kGateCols + (threadIdx.x >> 6) * 16;
    const int lane = threadIdx.x & 63;
    const int c = lane & 15;
    const int g = lane >> 4;
    const int tb0 = blockIdx.y * blocks;                          // first 16-query block
    const int nb = min(blocks, (T + kGateRows - 1) / kGateRows - tb0);
    if (nb <= 0)
        return;

    uint4 bv[KS];
    const uint16_t *brow = wv_b + ((int64_t)h * D_o + e0 + c) * DV + 8 * g;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        bv[ks] = *reinterpret_cast<const uint4 *>(brow + 32 * ks);

    // o fragments of block i: lane row t = 16*(tb0 + i) + c (zero past T)
    auto load_a = [&](int i, uint4 (&av)[KS]) {
        const int ta = kGateRows * (tb0 + i) + c;
        const bool ok = ta < T;
        const uint16_t *arow = o + ((int64_t)(ok ? ta : 0) * H + h) * DV + 8 * g;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            av[ks] = ok ? *reinterpret_cast<const uint4 *>(arow + 32 * ks) : make_uint4(0, 0, 0, 0);
    };
    auto block = [&](int i, const uint4 (&av)[KS]) {
        f4 acc[2] = {f4{0.f, 0.f, 0.f, 0.f}, f4{0.f, 0.f, 0.f, 0.f}};   // two chains, summed at the end
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            acc[ks & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av[ks]),
                                                                 __builtin_bit_cast(bf16x8, bv[ks]), acc[ks & 1],
                                                                 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = kGateRows * (tb0 + i) + 4 * g + r;
            if (t < T) {
                const int64_t idx = ((int64_t)t * H + h) * D_o + e0 + c;
                const float x = bf16_to_f32(gate[idx]);
                const float sg = 1.0f / (1.0f + __expf(-x));
                out[idx] = f32_to_bf16((acc[0][r] + acc[1][r]) * sg);
            }
        }
    };
    uint4 a0[KS], a1[KS];
    load_a(0, a0);
    int i = 0;
    for (; i + 1 < nb; i += 2) {
        load_a(i + 1, a1);
        block(i, a0);
        if (i + 2 < nb)
            load_a(i + 2, a0);
        block(i + 1, a1);
    }
    if (i < nb)
        block(i, a0);
}

}  // namespace

bool gated_output_supported(int32_t D_v, int32_t D_o)
{
    return (D_v == 512 || D_v == 64) && D_o >= kGateCols && D_o <= 1024 && D_o % kGateCols == 0;
}

hipError_t launch_gated_output(const uint16_t *o, const uint16_t *wv_b, const uint16_t *gate, int32_t T, int32_t H,
                               int32_t D_v, int32_t D_o, uint16_t *out, hipStream_t stream)
{
    if (!gated_output_supported(D_v, D_o))
        return hipErrorInvalidValue;
    if (T == 0 || H == 0)
        return hipSuccess;
    // query blocks per workgroup: one while the grid is small, up to 16 once
    // there are >= 2048 workgroups of the next size
    const int64_t cols = (int64_t)H * (D_o / kGateCols);
    const int64_t tblocks = (T + kGateRows - 1) / kGateRows;
    int blocks = 1;
    while (blocks < 16 && cols * ((tblocks + 2 * blocks - 1) / (2 * blocks)) >= 2048)
        blocks *= 2;
    const dim3 grid((unsigned)cols, (unsigned)((tblocks + blocks - 1) / blocks));
    if (D_v == 512)
        hipLaunchKernelGGL(gated_output_kernel<512>, grid, dim3(kGateThreads), 0, stream, o, wv_b, gate, T, H, D_o,
                           blocks, out);
    else
        hipLaunchKernelGGL(gated_output_kernel<64>, grid, dim3(kGateThreads), 0, stream, o, wv_b, gate, T, H, D_o,
                           blocks, out);
    return hipGetLastError();
}

}  // namespace ic
