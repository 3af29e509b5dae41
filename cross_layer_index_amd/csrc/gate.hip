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
// A workgroup (8 waves) owns one head, a run of 16-query blocks and up to
// 128 output columns, each wave one 16-column tile. The gate values and the
// results of a block travel as whole 16-byte chunks of their rows through LDS
// (loaded with the block's o, stored after it by the workgroup together),
// rather than as two bytes a lane. v_mfma_f32_16x16x32_bf16
// with queries on M and output columns on N: A lane l holds
// o[t0 + l%16][h][32*ks + 8*(l/16) .. +8], B lane l holds
// wv_b[h][e + l%16][32*ks + 8*(l/16) .. +8] (the contraction runs along the
// rows of o and wv_b). Accumulator element r of lane l is (query
// 4*(l/16) + r, column l%16). A wave keeps its wv_b fragments in registers
// for the whole run; each 16-query block of o is read from memory once per
// workgroup, staged through registers into a padded LDS tile (double
// buffered: the next block's loads are in flight while the current one
// multiplies) and read from there by all eight waves. The gate values of a
// block are loaded with its o. Workgroups of one head share its wv_b rows
// through one L2: the grid's x extent is a multiple of 8 when H is, so a
// head's workgroups stay on one XCD.
#include "kernels.h"

namespace ic {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kGateRows = 16;          // queries per block

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

template <int DV, int NT>
struct GateGeom {
    static constexpr int KS = DV / 32;                         // K-steps of 32
    static constexpr int ROWB = DV * 2 + 16;                   // LDS bytes per o row (16 of padding)
    static constexpr int CH = DV * 2 / 16;                     // 16-byte chunks per o row
    static constexpr int CHUNKS = kGateRows * CH;              // per block
    static constexpr int PER = (CHUNKS + NT - 1) / NT;         // chunks per thread
    static constexpr int COLS = NT / 64 * 16;                  // columns per workgroup
    static constexpr int GROWB = COLS * 2 + 16;                // LDS bytes per gate / output row
    static constexpr int GCH = COLS * 2 / 16;                  // 16-byte chunks per gate / output row
    static constexpr int GCHUNKS = kGateRows * GCH;            // per block (at most one per thread)
    static_assert(GCHUNKS <= NT, "one gate chunk per thread");
};

// grid: (H * ceil(D_o / COLS), query chunks); NT threads (NT/64 waves, one
// 16-column tile each); a workgroup takes `blocks` consecutive 16-query
// blocks of one head; waves whose tile lies past D_o only help stage o.
template <int DV, int NT>
__global__ __launch_bounds__(NT) void gated_output_kernel(const uint16_t *__restrict__ o,
                                                          const uint16_t *__restrict__ wv_b,
                                                          const uint16_t *__restrict__ gate, int32_t T, int32_t H,
                                                          int32_t D_o, int32_t blocks, uint16_t *__restrict__ out)
{
    using GG = GateGeom<DV, NT>;
    constexpr int wcols = GG::COLS;
    __shared__ __attribute__((aligned(16))) unsigned char ob0[kGateRows * GG::ROWB];
    __shared__ __attribute__((aligned(16))) unsigned char ob1[kGateRows * GG::ROWB];
    __shared__ __attribute__((aligned(16))) unsigned char gb0[kGateRows * GG::GROWB];   // gate values
    __shared__ __attribute__((aligned(16))) unsigned char gb1[kGateRows * GG::GROWB];
    __shared__ __attribute__((aligned(16))) unsigned char rb0[kGateRows * GG::GROWB];   // results
    __shared__ __attribute__((aligned(16))) unsigned char rb1[kGateRows * GG::GROWB];
    const int groups = (D_o + wcols - 1) / wcols;
    const int h = blockIdx.x / groups;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: scalar branches
    const int lane = threadIdx.x & 63;
    const int eb = (blockIdx.x % groups) * wcols;             // the workgroup's first column
    const int e0 = eb + wave * 16;
    const bool active = e0 < D_o;                 // D_o is a multiple of 16: whole tiles
    const int c = lane & 15;
    const int g = lane >> 4;
    const int tb0 = blockIdx.y * blocks;          // first 16-query block
    const int nb = min(blocks, (T + kGateRows - 1) / kGateRows - tb0);
    if (nb <= 0)
        return;

    uint4 bv[GG::KS];
    {
        const uint16_t *brow = wv_b + ((int64_t)h * D_o + (active ? e0 : 0) + c) * DV + 8 * g;
#pragma unroll
        for (int ks = 0; ks < GG::KS; ++ks)
            bv[ks] = *reinterpret_cast<const uint4 *>(brow + 32 * ks);
    }

    // o block i: thread chunk q = row q / CH, 16-byte chunk q % CH (zero past
    // T); gate chunk q = threadIdx.x: row q / GCH, chunk q % GCH
    uint4 stg[GG::PER];
    uint4 gstg;
    const int gq = threadIdx.x;
    const int gcol = eb + 8 * (gq % GG::GCH);
    const bool gown = gq < GG::GCHUNKS && gcol < D_o;   // D_o is a multiple of 8: whole chunks
    auto fetch = [&](int i) {
        {
            const int t = kGateRows * (tb0 + i) + gq / GG::GCH;
            gstg = gown && t < T ? *reinterpret_cast<const uint4 *>(gate + ((int64_t)t * H + h) * D_o + gcol)
                                 : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int p = 0; p < GG::PER; ++p) {
            const int q = threadIdx.x + p * NT;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (q < GG::CHUNKS) {
                const int t = kGateRows * (tb0 + i) + q / GG::CH;
                if (t < T)
                    v = *reinterpret_cast<const uint4 *>(o + ((int64_t)t * H + h) * DV + 8 * (q % GG::CH));
            }
            stg[p] = v;
        }
    };
    auto stash = [&](unsigned char *buf, unsigned char *gbuf) {
#pragma unroll
        for (int p = 0; p < GG::PER; ++p) {
            const int q = threadIdx.x + p * NT;
            if (q < GG::CHUNKS)
                *reinterpret_cast<uint4 *>(buf + (q / GG::CH) * GG::ROWB + 16 * (q % GG::CH)) = stg[p];
        }
        if (gq < GG::GCHUNKS)
            *reinterpret_cast<uint4 *>(gbuf + (gq / GG::GCH) * GG::GROWB + 16 * (gq % GG::GCH)) = gstg;
    };
    // the results of block i, rows of 16-byte chunks (chunks past D_o or
    // rows past T are not stored)
    auto store = [&](int i, const unsigned char *rbuf) {
        const int t = kGateRows * (tb0 + i) + gq / GG::GCH;
        if (gown && t < T)
            *reinterpret_cast<uint4 *>(out + ((int64_t)t * H + h) * D_o + gcol) =
                *reinterpret_cast<const uint4 *>(rbuf + (gq / GG::GCH) * GG::GROWB + 16 * (gq % GG::GCH));
    };
    auto compute = [&](int i, const unsigned char *buf, const unsigned char *gbuf, unsigned char *rbuf) {
        if (!active)
            return;
        f4 acc[2] = {f4{0.f, 0.f, 0.f, 0.f}, f4{0.f, 0.f, 0.f, 0.f}};   // two chains, summed at the end
        const unsigned char *arow = buf + c * GG::ROWB + 16 * g;
#pragma unroll
        for (int ks = 0; ks < GG::KS; ++ks) {
            const uint4 av = *reinterpret_cast<const uint4 *>(arow + 64 * ks);
            acc[ks & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av),
                                                                 __builtin_bit_cast(bf16x8, bv[ks]), acc[ks & 1],
                                                                 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 4 * g + r;
            const uint16_t gv = *reinterpret_cast<const uint16_t *>(gbuf + row * GG::GROWB + 2 * (e0 - eb + c));
            const float sg = 1.0f / (1.0f + __expf(-bf16_to_f32(gv)));
            *reinterpret_cast<uint16_t *>(rbuf + row * GG::GROWB + 2 * (e0 - eb + c)) =
                f32_to_bf16((acc[0][r] + acc[1][r]) * sg);
        }
    };

    fetch(0);
    stash(ob0, gb0);
    if (nb > 1)
        fetch(1);
    __syncthreads();
    // block i (o and gate) is in LDS and its successor's in registers; the
    // multiply leaves block i's results in its result buffer, the successor
    // goes to the other buffers and block i+2 is fetched; after the barrier
    // block i's results go out while block i+1 multiplies into the other
    // result buffer
    auto iter = [&](int i, const unsigned char *cur, unsigned char *nxt, const unsigned char *gcur,
                    unsigned char *gnxt, unsigned char *rcur, const unsigned char *rprev) {
        if (i > 0)
            store(i - 1, rprev);
        compute(i, cur, gcur, rcur);
        if (i + 1 < nb)
            stash(nxt, gnxt);
        if (i + 2 < nb)
            fetch(i + 2);
        __syncthreads();
    };
    for (int i = 0; i < nb; i += 2) {
        iter(i, ob0, ob1, gb0, gb1, rb0, rb1);
        if (i + 1 < nb)
            iter(i + 1, ob1, ob0, gb1, gb0, rb1, rb0);
    }
    store(nb - 1, (nb - 1) & 1 ? rb1 : rb0);
}

}  // namespace

bool gated_output_supported(int32_t D_v, int32_t D_o)
{
    return (D_v == 512 || D_v == 64) && D_o >= 64 && D_o <= 1024 && D_o % 64 == 0;
}

hipError_t launch_gated_output(const uint16_t *o, const uint16_t *wv_b, const uint16_t *gate, int32_t T, int32_t H,
                               int32_t D_v, int32_t D_o, uint16_t *out, hipStream_t stream)
{
    if (!gated_output_supported(D_v, D_o))
        return hipErrorInvalidValue;
    if (T == 0 || H == 0)
        return hipSuccess;
    // Few queries (decode): 4-wave workgroups of 64 columns, so that the
    // wv_b stream spreads over twice as many workgroups; otherwise 8-wave
    // workgroups of 128 columns, which read each o block once for more
    // columns. Query blocks per workgroup: one while the grid is small, up to
    // 16 once there are >= 2048 workgroups of the next size.
    const int64_t tblocks = (T + kGateRows - 1) / kGateRows;
    const bool narrow = (int64_t)H * ((D_o + 127) / 128) * tblocks < 256;
    const int wcols = narrow ? 64 : 128;
    const int64_t cols = (int64_t)H * ((D_o + wcols - 1) / wcols);
    int blocks = 1;
    while (blocks < 16 && cols * ((tblocks + 2 * blocks - 1) / (2 * blocks)) >= 2048)
        blocks *= 2;
    const dim3 grid((unsigned)cols, (unsigned)((tblocks + blocks - 1) / blocks));
#define IC_GATE_LAUNCH(DVV, NTT)                                                                                  \
    hipLaunchKernelGGL((gated_output_kernel<DVV, NTT>), grid, dim3(NTT), 0, stream, o, wv_b, gate, T, H, D_o,     \
                       blocks, out)
    if (!trace_skip("gated_output_kernel")) {
        if (D_v == 512) {
            if (narrow)
                IC_GATE_LAUNCH(512, 256);
            else
                IC_GATE_LAUNCH(512, 512);
        } else {
            if (narrow)
                IC_GATE_LAUNCH(64, 256);
            else
                IC_GATE_LAUNCH(64, 512);
        }
    }
#undef IC_GATE_LAUNCH
    trace_launch(stream, "gated_output_kernel");
    return hipGetLastError();
}

}  // namespace ic
