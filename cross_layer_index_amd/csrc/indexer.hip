// Lightning-indexer scores on gfx950 fp8 matrix cores.
//
//   I[t, s] = sum_h w[t,h] * max(0, q[t,h,:] . k[base_t + s, :])
//
// (explainer "Hy4 IndexCache cross-layer index reuse", Jargon "Indexer" and
// "DSA": one cheap score per cached position per query). The q.k contraction
// over d runs on v_mfma_f32_32x32x64_f8f6f4 with OCP e4m3fn operands and fp32
// accumulation; heads sit on the M side of the tile and cached tokens on the
// N side, so the ReLU / weight / head-sum epilogue stays inside each lane plus
// one exchange between the two half-waves.
//
// Operand placement (32x32x64, 8 VGPRs = 32 fp8 per lane per operand):
//   A lane l holds row (l % 32), B lane l holds column (l % 32); both take 32
//   K-values from the half-wave g = l / 32. Which physical d sits in which K
//   slot is irrelevant to a dot product as long as A and B agree, so each
//   lane takes one contiguous run of D_I/2 bytes of its row: d in
//   [g*D_I/2, (g+1)*D_I/2), split into 32-byte K-steps (zero-padded when
//   D_I/2 < 32). That keeps every key-row load a contiguous 16-byte vector.
//   Accumulator element r of lane l is (row 8*(r/4) + 4*(l/32) + r%4,
//   column l % 32).
#include "kernels.h"
#include "lds_dma.h"
#include "radix_key.h"

namespace ic {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ v16f mfma_fp8_32x32x64(const v8i &a, const v8i &b, const v16f &c)
{
    // Format selectors 0/0 = fp8 e4m3 for both operands; zero scale operands
    // select the unscaled instruction.
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// ReLU of a matrix-core result as a signed-integer max on its bits: a
// negative float is a negative integer and -0 becomes +0, in one VALU op
// (fmaxf adds a NaN-quieting step per element). The inputs are finite
// e4m3fn codes, so every accumulator is finite.
__device__ __forceinline__ float relu_bits(float x)
{
    return __int_as_float(max(__float_as_int(x), 0));
}

// Sum over the two half-waves: v_permlane32_swap exchanges lanes 32..63 of
// one copy with lanes 0..31 of the other inside the VGPRs, so the first
// result holds x[l % 32] and the second x[l % 32 + 32] on every lane l.
__device__ __forceinline__ float half_sum(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int DI>
struct IdxGeom {
    static constexpr int HALF = DI / 2;                 // bytes per lane per row
    static constexpr int KS = (HALF + 31) / 32;         // 32-byte K-steps
    static constexpr int VEC = HALF / 16;               // 16-byte loads per lane
    static_assert(DI == 32 || DI == 64 || DI == 128, "D_I");
};

// Load one lane's run of a row into K-step fragments (zero beyond the run).
template <int DI>
__device__ __forceinline__ void load_run(const uint8_t *p, v8i (&frag)[IdxGeom<DI>::KS])
{
    using G = IdxGeom<DI>;
    uint4 v[G::KS * 2];
#pragma unroll
    for (int i = 0; i < G::KS * 2; ++i) {
        if (i < G::VEC)
            v[i] = *reinterpret_cast<const uint4 *>(p + 16 * i);
        else
            v[i] = make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int ks = 0; ks < G::KS; ++ks) {
        frag[ks] = v8i{(int)v[2 * ks].x, (int)v[2 * ks].y, (int)v[2 * ks].z, (int)v[2 * ks].w,
                       (int)v[2 * ks + 1].x, (int)v[2 * ks + 1].y, (int)v[2 * ks + 1].z,
                       (int)v[2 * ks + 1].w};
    }
}

constexpr int kIdxWaves = 4;
constexpr int kIdxThreads = kIdxWaves * 64;
constexpr int kIdxStep = kIdxWaves * 32 * 2;                  // tokens per WG step of two groups
constexpr int kIdxMaxChunk = 1024;                             // tokens per WG, upper bound
constexpr int64_t kIdxResident = 2 * 256;                      // resident WGs: 2 per CU x 256 CUs

// One wave step's key fragments: U groups of 32 tokens, each lane holding its
// run of one token row (rows past the query's end are clamped to its last
// row; their scores are never stored).
template <int DI, int U>
struct KeyStep {
    v8i b[U][IdxGeom<DI>::KS];
};

template <int DI, int U>
__device__ __forceinline__ void load_step(KeyStep<DI, U> &ks, const uint8_t *krows, int64_t s0, int j, int64_t nt)
{
#pragma unroll
    for (int u = 0; u < U; ++u) {
        int64_t s = s0 + 32 * u + j;
        s = s < nt ? s : nt - 1;
        load_run<DI>(krows + s * DI, ks.b[u]);
    }
}

// grid: (token chunks, T); block: 256 threads. A workgroup scores `chunk`
// consecutive tokens of one query; each wave takes every fourth step of 32 U
// tokens and keeps the next step's key rows in flight while it scores the
// current one. Head weights come from LDS as float4 (four consecutive heads
// per accumulator quad), q fragments stay in registers. With `hist0` set the
// workgroup also counts the first radix digit of its scores and adds its
// counts to copy (blockIdx.x mod kHistCopies) of the query's histogram.
template <int DI, int MT, int U>
__global__ __launch_bounds__(kIdxThreads) void indexer_decode_kernel(
    const uint8_t *__restrict__ q_idx, const float *__restrict__ w, const uint8_t *__restrict__ k_idx,
    const int64_t *__restrict__ base, const int32_t *__restrict__ n, int32_t H_I,
    float *__restrict__ scores, int64_t ld, int64_t chunk, uint32_t *__restrict__ hist0)
{
    using G = IdxGeom<DI>;
    __shared__ uint32_t hist[kHistBins0];
    __shared__ __attribute__((aligned(16))) float wsh[MT * 32];
    const int t = blockIdx.y;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: scalar branches
    const int g = lane >> 5;
    const int j = lane & 31;

    // the query's extent and first row (scalar loads) first: a workgroup
    // past the query's end (ragged batches launch the longest query's grid
    // for every query) leaves before it issues any vector load, which would
    // hold its slot until the data returned; the q fragments and weights go
    // out together with the first key rows
    const int64_t nt = n[t];
    const int64_t bt = base[t];
    asm volatile("" ::"s"(nt), "s"(bt));   // both loads complete here, not one after the other
    const int64_t s_begin = (int64_t)blockIdx.x * chunk;
    if (s_begin >= nt)
        return;
    v8i a[MT][G::KS];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int h = 32 * mt + j;
        if (h < H_I) {
            load_run<DI>(q_idx + ((int64_t)t * H_I + h) * DI + g * G::HALF, a[mt]);
        } else {
#pragma unroll
            for (int ks = 0; ks < G::KS; ++ks)
                a[mt][ks] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
        }
    }
    float wv = 0.0f;
    if (threadIdx.x < MT * 32 && (int)threadIdx.x < H_I)
        wv = w[(int64_t)t * H_I + threadIdx.x];
    const int64_t s_end = min(nt, s_begin + chunk);
    const uint8_t *krows = k_idx + (bt * DI) + g * G::HALF;
    float *srow = scores + (int64_t)t * ld;

    // the wave's first key rows go out before the weights are staged (the
    // LDS store waits for the weight load; the key loads need not)
    constexpr int64_t WS = kIdxWaves * 32 * U;    // tokens per workgroup step
    int64_t s0 = s_begin + (int64_t)wave * 32 * U;
    KeyStep<DI, U> x, y;
    load_step<DI, U>(x, krows, s0 < s_end ? s0 : s_begin, j, nt);
    if (threadIdx.x < MT * 32)
        wsh[threadIdx.x] = wv;
    if (hist0)
        for (int i = threadIdx.x; i < kHistBins0; i += kIdxThreads)
            hist[i] = 0;
    __syncthreads();
    const float4 *w4 = reinterpret_cast<const float4 *>(wsh);

    auto score_step = [&](const KeyStep<DI, U> &ks, int64_t s0) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float sum = 0.0f;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                v16f acc = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int k = 0; k < G::KS; ++k)
                    acc = mfma_fp8_32x32x64(a[mt][k], ks.b[u][k], acc);
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    // accumulator quad q4 holds heads 32*mt + 8*q4 + 4*g + (0..3)
                    const float4 wq = w4[8 * mt + 2 * q4 + g];
                    sum = fmaf(wq.x, relu_bits(acc[4 * q4 + 0]), sum);
                    sum = fmaf(wq.y, relu_bits(acc[4 * q4 + 1]), sum);
                    sum = fmaf(wq.z, relu_bits(acc[4 * q4 + 2]), sum);
                    sum = fmaf(wq.w, relu_bits(acc[4 * q4 + 3]), sum);
                }
            }
            sum = half_sum(sum);
            const int64_t s = s0 + 32 * u + j;
            if (g == 0 && s < s_end) {
                srow[s] = sum;
                if (hist0)
                    atomicAdd(&hist[ord_key(sum) >> kHistShift0], 1u);
            }
        }
    };

    // two register buffers alternated by an unrolled pair of steps: the next
    // step's loads are always issued before the current step is scored, and
    // every load in the loop is unconditional so the compiler's wait counts
    // stay exact (a conditional load makes it wait for everything)
    const int nsteps = s0 < s_end ? (int)((s_end - s0 + WS - 1) / WS) : 0;
    int i = 0;
    for (; i + 2 < nsteps; i += 2, s0 += 2 * WS) {
        load_step<DI, U>(y, krows, s0 + WS, j, nt);
        __builtin_amdgcn_sched_barrier(0);
        score_step(x, s0);
        load_step<DI, U>(x, krows, s0 + 2 * WS, j, nt);
        __builtin_amdgcn_sched_barrier(0);
        score_step(y, s0 + WS);
    }
    if (nsteps - i == 2) {
        load_step<DI, U>(y, krows, s0 + WS, j, nt);
        __builtin_amdgcn_sched_barrier(0);
        score_step(x, s0);
        score_step(y, s0 + WS);
    } else if (nsteps - i == 1) {
        score_step(x, s0);
    }
    if (hist0) {
        __syncthreads();
        uint32_t *h = hist0 + ((int64_t)t * kHistCopies + (blockIdx.x % kHistCopies)) * kHistBins0;
        for (int i = threadIdx.x; i < kHistBins0; i += kIdxThreads)
            if (hist[i])
                atomicAdd(&h[i], hist[i]);
    }
}

template <int DI>
hipError_t launch_decode_di(const uint8_t *q_idx, const float *w, const uint8_t *k_idx,
                            const int64_t *base, const int32_t *n, int32_t T, int64_t max_n,
                            int32_t H_I, float *scores, int64_t ld, uint32_t *hist0, hipStream_t stream)
{
    // one WG step per workgroup while the whole grid fits on the chip at
    // once (two workgroups per CU at this kernel's register use); beyond
    // that, longer chunks whose steps are pipelined inside each wave
    int64_t chunk = kIdxStep;
    while (chunk < kIdxMaxChunk && chunk < max_n && T * ((max_n + chunk - 1) / chunk) > kIdxResident)
        chunk *= 2;
    const int64_t nchunks = (max_n + chunk - 1) / chunk;
    if (nchunks == 0 || T == 0)
        return hipSuccess;
    dim3 grid((unsigned)nchunks, (unsigned)T);
    // A workgroup that holds a single step of two groups per wave (the whole
    // grid in one round) takes it as two pipelined one-group steps instead:
    // each wave scores its first 32 tokens while the next 32 arrive, which
    // shortens the tail after the last bytes land. Longer chunks keep
    // two-group steps.
    const bool one = chunk == kIdxStep;
    auto go = [&](auto kern) {
        if (!trace_skip("indexer_decode_kernel"))
            hipLaunchKernelGGL(kern, grid, dim3(kIdxThreads), 0, stream, q_idx, w, k_idx, base, n, H_I, scores, ld, chunk,
                           hist0);
    };
    if (H_I <= 32)
        one ? go(indexer_decode_kernel<DI, 1, 1>) : go(indexer_decode_kernel<DI, 1, 2>);
    else
        one ? go(indexer_decode_kernel<DI, 2, 1>) : go(indexer_decode_kernel<DI, 2, 2>);
    trace_launch(stream, "indexer_decode_kernel");
    return hipGetLastError();
}

// ---- shared-sequence form ----------------------------------------------------
// Queries that read one sequence share its key stream: causal prefill (every
// query on one sequence; query t sees tokens 0..n_t-1) and draft/verify
// decode (groups of G consecutive queries per sequence). A workgroup takes G
// queries (G <= 2P) of one sequence and a chunk of its tokens; a key tile
// staged in LDS serves all of them. Wave w takes query pair w % P (q
// fragments and head weights in registers) and token split w / P of the
// tile's S = 8 / P splits (P = 8 for prefill: every wave covers the whole
// tile; smaller groups split the tokens instead).
//
// Tiles of 256 tokens go straight from memory into LDS (global_load_lds, no
// registers), three buffers deep. Within a tile, 32-token group gi occupies
// 4 KB as four 1 KB slabs; slot i (16 bytes) of slab v holds token
// 32*gi + i%32, bytes 16*(4*(i/32) + v) .. +16 of its row. Lane i of a wave
// reads slot i of each slab, so the four conflict-free 16-byte reads hand lane
// (j = i%32, g = i/32) bytes 64g .. 64g+63 of token j: its B fragments for
// both K-steps, in the K-slot order the q fragments use. Wave w fills group w.
//
// The work of a tile is 16 units (group, query). Unit u+1's four MFMAs are
// interleaved with unit u's ReLU / weight / head-sum epilogue on the VALU, so
// the matrix cores and the vector ALUs of a wave run side by side.
constexpr int kPfWaves = 8;
constexpr int kPfThreads = kPfWaves * 64;
constexpr int kPfQW = 2;                                  // queries per wave
constexpr int kPfQ = kPfWaves * kPfQW;                    // most queries per workgroup
constexpr int kPfTile = 256;                              // tokens per LDS tile
constexpr int kPfGroups = kPfTile / 32;                   // 32-token groups per tile
constexpr int kPfDI = 128;
constexpr int kPfSlab = 1024;                             // bytes per fill instruction
constexpr int kPfGroupBytes = 32 * kPfDI;                 // 4 slabs
static_assert(kPfGroups == kPfWaves, "wave w fills group w of each tile");

// What a launch of the shared-key kernel produces (causal prefill uses all
// three, see the collecting top-k in topk.hip):
//   kPfScores   the score rows;
//   kPfSample   the score rows of a strided sample of the keys: sample row i
//               is key row kPfSampleStride * i, and query t sees
//               ceil(n_t / kPfSampleStride) of them;
//   kPfCollect  no score rows: each score whose order key is at or above the
//               query's bound goes, as (key << 32 | position), into the
//               query's slice for this token chunk, in position order, and
//               the slice's count is stored (beyond `cap` entries only counted).
enum { kPfScores = 0, kPfSample = 1, kPfCollect = 2 };

// The collecting mode's outputs. Slice (t, c) of query t and token chunk c
// (blockIdx.x) holds `cap` entries from (t * gridDim.x + c) * cap.
struct PfCollect {
    const uint32_t *bound;       // [T] order-key bound per query
    uint64_t *slices;
    uint32_t *counts;            // [T, gridDim.x]
    int32_t cap;
};

template <int P, int MODE>
__global__ __launch_bounds__(kPfThreads, 1) void indexer_prefill_kernel(
    const uint8_t *__restrict__ q_idx, const float *__restrict__ w, const uint8_t *__restrict__ k_idx,
    const int64_t *__restrict__ base, const int32_t *__restrict__ n, int32_t T, int32_t grp,
    float *__restrict__ scores, int64_t ld, int64_t chunk, const uint32_t *__restrict__ need, PfCollect col)
{
    static_assert(P == 1 || P == 2 || P == 4 || P == 8, "query pairs per workgroup");
    constexpr int S = kPfWaves / P;                       // token splits of a tile
    constexpr int kUnits = 2 * P;                         // (group, query) units per wave per tile
    // collecting keeps each query's survivors in position order in one wave
    static_assert(MODE != kPfCollect || S == 1, "one wave per query");
    using G = IdxGeom<kPfDI>;
    // three separate LDS objects (not one array): a read of one buffer is then
    // known not to alias the fills in flight into the others, and the
    // compiler need not wait for those fills before reading
    __shared__ __attribute__((aligned(16))) uint8_t tile0[kPfTile * kPfDI];
    __shared__ __attribute__((aligned(16))) uint8_t tile1[kPfTile * kPfDI];
    __shared__ __attribute__((aligned(16))) uint8_t tile2[kPfTile * kPfDI];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5;
    const int j = lane & 31;
    const int t_base = blockIdx.y * grp;
    const int qp = wave % P;                              // this wave's query pair
    const int ts = wave / P;                              // and token split

    // visible rows of query t (sample rows in the sampling mode)
    auto n_of = [&](int t) -> int64_t {
        const int64_t v = n[t];
        return MODE == kPfSample ? (v + kPfSampleStride - 1) / kPfSampleStride : v;
    };
    // a gated launch (need non-null) serves only groups with a query marked
    if (need) {
        bool any = false;
        for (int i = 0; i < grp; ++i)
            if (t_base + i < T)
                any = any || need[t_base + i] != 0u;
        if (!any)
            return;
    }
    // extent of the group: the largest n among its queries
    int64_t nmax = 0;
    for (int i = 0; i < grp; ++i)
        if (t_base + i < T)
            nmax = max(nmax, n_of(t_base + i));
    const int64_t s_begin = (int64_t)blockIdx.x * chunk;
    if (s_begin >= nmax)
        return;
    const int64_t s_end = min(nmax, s_begin + chunk);
    const uint8_t *krows = k_idx + base[t_base] * kPfDI;

    int tq[kPfQW];
    int64_t nq[kPfQW];
    uint32_t bq[kPfQW];                                   // collecting: bound and running count
    uint32_t run[kPfQW];
    v8i a[kPfQW][2][G::KS];
    float wr[kPfQW][2][16];
#pragma unroll
    for (int i = 0; i < kPfQW; ++i) {
        tq[i] = t_base + qp * kPfQW + i;
        const bool ok = qp * kPfQW + i < grp && tq[i] < T;
        nq[i] = ok ? n_of(tq[i]) : 0;
        bq[i] = MODE == kPfCollect && ok ? col.bound[tq[i]] : 0xFFFFFFFFu;
        run[i] = 0;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            const int h = 32 * mt + j;
            if (ok)
                load_run<kPfDI>(q_idx + ((int64_t)tq[i] * 64 + h) * kPfDI + g * G::HALF, a[i][mt]);
            else
#pragma unroll
                for (int ks = 0; ks < G::KS; ++ks)
                    a[i][mt][ks] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int hh = 32 * mt + 8 * (r >> 2) + 4 * g + (r & 3);
                wr[i][mt][r] = ok ? w[(int64_t)tq[i] * 64 + hh] : 0.0f;
            }
        }
    }

    // fills of this wave's group: row 32*wave + lane%32 of the tile (clamped
    // to the group's extent), bytes 64*(lane/32) + 16*v for slab v; four fill
    // instructions per wave per tile, by 32-bit offsets from the sequence's
    // first key row (the rows of one sequence span less than 4 GiB)
    const int64_t frow = 32 * wave + j;
    const int fcol = 64 * g;
    auto issue = [&](uint8_t *buf, int64_t tile) {
        int64_t row = tile + frow;
        row = row < s_end ? row : s_end - 1;
        if (MODE == kPfSample)
            row *= kPfSampleStride;
        const uint32_t off = (uint32_t)(row * kPfDI + fcol);
        const uint32_t dst = (uint32_t)(uintptr_t)(lds_void *)buf + wave * kPfGroupBytes;
#pragma unroll
        for (int v = 0; v < 4; ++v)
            lds_fill16(krows, off + 16 * v, dst + v * kPfSlab);
    };

    auto bfrag = [&](const uint8_t *tb, int gi, v8i (&b)[G::KS]) {
        const uint8_t *p = tb + gi * kPfGroupBytes + 16 * lane;
#pragma unroll
        for (int ks = 0; ks < G::KS; ++ks) {
            const uint4 lo = *reinterpret_cast<const uint4 *>(p + (2 * ks) * kPfSlab);
            const uint4 hi = *reinterpret_cast<const uint4 *>(p + (2 * ks + 1) * kPfSlab);
            b[ks] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        }
    };

    // this wave's k-th 32-token group of a tile
    auto gidx = [&](int kk) { return S == 1 ? kk : ts + S * kk; };
    auto compute = [&](const uint8_t *tb, int64_t tile) {
        v8i b[2][G::KS];
        v16f acc[2][2];
        auto mfmas = [&](int u) {
            const int i = u & 1;
            const v8i(&bb)[G::KS] = b[(u >> 1) & 1];
            v16f(&c)[2] = acc[u & 1];
            const v16f z = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            c[0] = mfma_fp8_32x32x64(a[i][0][0], bb[0], z);
            c[1] = mfma_fp8_32x32x64(a[i][1][0], bb[0], z);
            c[0] = mfma_fp8_32x32x64(a[i][0][1], bb[1], c[0]);
            c[1] = mfma_fp8_32x32x64(a[i][1][1], bb[1], c[1]);
        };
        bfrag(tb, gidx(0), b[0]);
        mfmas(0);
#pragma unroll
        for (int u = 0; u < kUnits; ++u) {
            const int kk = u >> 1, i = u & 1;
            if (i == 0 && kk + 1 < P)
                bfrag(tb, gidx(kk + 1), b[(kk + 1) & 1]);
            if (u + 1 < kUnits)
                mfmas(u + 1);
            const v16f(&c)[2] = acc[u & 1];
            float sum = 0.0f;
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    sum = fmaf(wr[i][mt][r], relu_bits(c[mt][r]), sum);
            if (u + 1 < kUnits) {
                // one MFMA, then a quarter of the epilogue, four times over
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, 16, 0);
                }
            }
            sum = half_sum(sum);
            const int64_t s = tile + 32 * gidx(kk) + j;
            if (MODE == kPfCollect) {
                // scores at or above the bound, in position order (lanes in
                // order, units of a query in token order)
                const uint32_t key = ord_key(sum);
                const bool keep = g == 0 && s < nq[i] && key >= bq[i];
                const uint64_t m = __ballot(keep);
                if (m) {
                    const uint32_t o = run[i] + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                                          __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
                    if (keep && o < (uint32_t)col.cap)
                        col.slices[((int64_t)tq[i] * gridDim.x + blockIdx.x) * col.cap + o] =
                            ((uint64_t)key << 32) | (uint32_t)s;
                    run[i] += (uint32_t)__popcll(m);
                }
            } else if (g == 0 && s < nq[i]) {
                scores[(int64_t)tq[i] * ld + s] = sum;
            }
        }
    };

    // ring of three tiles: tile it+2 is issued at the top of iteration it and
    // tiles it+1 and it+2 stay in flight while tile it is scored. The score
    // stores share the vector-memory counter with the fills, but loads
    // complete in order among themselves: with at most four operations
    // outstanding, and tile it+1's four fills issued after tile it's, tile
    // it's fills are complete whatever the stores do. The barrier then orders
    // LDS only (a full one would also wait for the fills in flight).
    const int ntiles = (int)((s_end - s_begin + kPfTile - 1) / kPfTile);
    issue(tile0, s_begin);
    if (ntiles > 1)
        issue(tile1, s_begin + kPfTile);
    // the ring unrolled by three so that every access names its buffer
    auto step = [&](int it, uint8_t *cur, uint8_t *ahead) {
        if (it + 1 < ntiles)
            wait_vmcnt<4>();
        else
            wait_vmcnt<0>();
        // tile it is in LDS for every wave; `ahead` is free
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        if (it + 2 < ntiles)
            issue(ahead, s_begin + (int64_t)(it + 2) * kPfTile);
        compute(cur, s_begin + (int64_t)it * kPfTile);
    };
    for (int it = 0; it < ntiles; it += 3) {
        step(it, tile0, tile2);
        if (it + 1 < ntiles)
            step(it + 1, tile1, tile0);
        if (it + 2 < ntiles)
            step(it + 2, tile2, tile1);
    }
    if (MODE == kPfCollect && lane == 0)
#pragma unroll
        for (int i = 0; i < kPfQW; ++i)
            if (qp * kPfQW + i < grp && tq[i] < T)
                col.counts[(int64_t)tq[i] * gridDim.x + blockIdx.x] = run[i];
}

}  // namespace

hipError_t launch_indexer_decode(const uint8_t *q_idx, const float *w, const uint8_t *k_idx,
                                 const int64_t *base, const int32_t *n, int32_t T, int64_t max_n,
                                 int32_t H_I, int32_t D_I, float *scores, int64_t ld,
                                 uint32_t *hist0, hipStream_t stream)
{
    switch (D_I) {
    case 32: return launch_decode_di<32>(q_idx, w, k_idx, base, n, T, max_n, H_I, scores, ld, hist0, stream);
    case 64: return launch_decode_di<64>(q_idx, w, k_idx, base, n, T, max_n, H_I, scores, ld, hist0, stream);
    case 128: return launch_decode_di<128>(q_idx, w, k_idx, base, n, T, max_n, H_I, scores, ld, hist0, stream);
    default: return hipErrorInvalidValue;
    }
}

bool indexer_prefill_supported(int32_t H_I, int32_t D_I) { return H_I == 64 && D_I == kPfDI; }

int64_t indexer_prefill_chunk(int32_t T, int32_t G, int64_t max_n)
{
    const int64_t groups = (T + G - 1) / G;
    const int P = G <= 2 ? 1 : (G <= 4 ? 2 : (G <= 8 ? 4 : 8));
    // token chunks: at least 64 units per wave per workgroup (32 / P tiles),
    // which keeps the tile ring's fill latency hidden and, for draft/verify
    // groups, the grid within one round of workgroups (8 groups of 4 queries
    // over 131,072 tokens: 256 workgroups, 5% faster than two rounds of
    // 512); at most 16384 workgroups (prefill: 16384-token chunks)
    int64_t chunk = (int64_t)kPfTile * (32 / P);
    while (chunk < max_n && groups * ((max_n + chunk - 1) / chunk) > 16384)
        chunk *= 2;
    return chunk;
}

namespace {
template <int MODE>
void launch_pf(int P, dim3 grid, hipStream_t stream, const uint8_t *q_idx, const float *w, const uint8_t *k_idx,
               const int64_t *base, const int32_t *n, int32_t T, int32_t G, float *scores, int64_t ld,
               int64_t chunk, const uint32_t *need, const PfCollect &col)
{
    if constexpr (MODE != kPfScores)     // groups of 16 queries: eight pairs, one per wave
        hipLaunchKernelGGL((indexer_prefill_kernel<8, MODE>), grid, dim3(kPfThreads), 0, stream, q_idx, w, k_idx,
                           base, n, T, G, scores, ld, chunk, need, col);
    else if (P == 1)
        hipLaunchKernelGGL((indexer_prefill_kernel<1, MODE>), grid, dim3(kPfThreads), 0, stream, q_idx, w, k_idx,
                           base, n, T, G, scores, ld, chunk, need, col);
    else if (P == 2)
        hipLaunchKernelGGL((indexer_prefill_kernel<2, MODE>), grid, dim3(kPfThreads), 0, stream, q_idx, w, k_idx,
                           base, n, T, G, scores, ld, chunk, need, col);
    else if (P == 4)
        hipLaunchKernelGGL((indexer_prefill_kernel<4, MODE>), grid, dim3(kPfThreads), 0, stream, q_idx, w, k_idx,
                           base, n, T, G, scores, ld, chunk, need, col);
    else
        hipLaunchKernelGGL((indexer_prefill_kernel<8, MODE>), grid, dim3(kPfThreads), 0, stream, q_idx, w, k_idx,
                           base, n, T, G, scores, ld, chunk, need, col);
}
}  // namespace

hipError_t launch_indexer_prefill(const uint8_t *q_idx, const float *w, const uint8_t *k_idx,
                                  const int64_t *base, const int32_t *n, int32_t T, int64_t max_n,
                                  int32_t H_I, int32_t D_I, int32_t G, float *scores, int64_t ld,
                                  hipStream_t stream, const uint32_t *need)
{
    if (!indexer_prefill_supported(H_I, D_I) || G < 1 || G > kPfQ)
        return hipErrorInvalidValue;
    if (T == 0 || max_n == 0)
        return hipSuccess;
    const int64_t groups = (T + G - 1) / G;
    const int P = G <= 2 ? 1 : (G <= 4 ? 2 : (G <= 8 ? 4 : 8));
    const int64_t chunk = indexer_prefill_chunk(T, G, max_n);
    const int64_t nchunks = (max_n + chunk - 1) / chunk;
    if (groups > 65535)
        return hipErrorInvalidValue;
    if (!trace_skip("indexer_prefill_kernel"))
        launch_pf<kPfScores>(P, dim3((unsigned)nchunks, (unsigned)groups), stream, q_idx, w, k_idx, base, n, T, G,
                             scores, ld, chunk, need, PfCollect{});
    trace_launch(stream, "indexer_prefill_kernel");
    return hipGetLastError();
}

hipError_t launch_indexer_prefill_sample(const uint8_t *q_idx, const float *w, const uint8_t *k_idx,
                                         const int64_t *base, const int32_t *n, int32_t T, int64_t max_n,
                                         float *scores, int64_t ld, hipStream_t stream)
{
    if (T == 0 || max_n == 0)
        return hipSuccess;
    const int64_t max_s = (max_n + kPfSampleStride - 1) / kPfSampleStride;
    const int64_t groups = (T + kPfQ - 1) / kPfQ;
    const int64_t chunk = indexer_prefill_chunk(T, kPfQ, max_s);
    const int64_t nchunks = (max_s + chunk - 1) / chunk;
    if (groups > 65535)
        return hipErrorInvalidValue;
    if (!trace_skip("indexer_prefill_sample"))
        launch_pf<kPfSample>(8, dim3((unsigned)nchunks, (unsigned)groups), stream, q_idx, w, k_idx, base, n, T, kPfQ,
                             scores, ld, chunk, nullptr, PfCollect{});
    trace_launch(stream, "indexer_prefill_sample");
    return hipGetLastError();
}

hipError_t launch_indexer_prefill_collect(const uint8_t *q_idx, const float *w, const uint8_t *k_idx,
                                          const int64_t *base, const int32_t *n, int32_t T, int64_t max_n,
                                          const uint32_t *bound, uint64_t *slices, uint32_t *counts, int32_t cap,
                                          hipStream_t stream)
{
    if (T == 0 || max_n == 0)
        return hipSuccess;
    const int64_t groups = (T + kPfQ - 1) / kPfQ;
    const int64_t chunk = indexer_prefill_chunk(T, kPfQ, max_n);
    const int64_t nchunks = (max_n + chunk - 1) / chunk;
    if (groups > 65535)
        return hipErrorInvalidValue;
    if (!trace_skip("indexer_prefill_collect"))
        launch_pf<kPfCollect>(8, dim3((unsigned)nchunks, (unsigned)groups), stream, q_idx, w, k_idx, base, n, T, kPfQ,
                              nullptr, 0, chunk, nullptr, PfCollect{bound, slices, counts, cap});
    trace_launch(stream, "indexer_prefill_collect");
    return hipGetLastError();
}

}  // namespace ic
