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
#include "radix_key.h"

namespace ic {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

__device__ __forceinline__ v16f mfma_fp8_32x32x64(const v8i &a, const v8i &b, const v16f &c)
{
    // Format selectors 0/0 = fp8 e4m3 for both operands; zero scale operands
    // select the unscaled instruction.
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
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
constexpr int kIdxUnroll = 2;                                  // 32-token groups per wave step
constexpr int kIdxStep = kIdxWaves * 32 * kIdxUnroll;          // tokens per WG step

// grid: (token chunks, T); block: 256 threads. Each wave scores groups of 32
// consecutive tokens; a WG covers `chunk` tokens of one query.
template <int DI, int MT>
__global__ __launch_bounds__(256) void indexer_decode_kernel(
    const uint8_t *__restrict__ q_idx, const float *__restrict__ w, const uint8_t *__restrict__ k_idx,
    const int64_t *__restrict__ base, const int32_t *__restrict__ n, int32_t H_I,
    float *__restrict__ scores, int64_t ld, int64_t chunk, uint32_t *__restrict__ hist0)
{
    using G = IdxGeom<DI>;
    __shared__ uint32_t hist[kHistBins0];
    const int t = blockIdx.y;
    const int64_t nt = n[t];
    const int64_t s_begin = (int64_t)blockIdx.x * chunk;
    if (s_begin >= nt)
        return;
    const int64_t s_end = min(nt, s_begin + chunk);
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int g = lane >> 5;
    const int j = lane & 31;
    if (hist0) {
        for (int i = threadIdx.x; i < kHistBins0; i += 256)
            hist[i] = 0;
        __syncthreads();
    }

    // q fragments for all heads of this query, kept in registers
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
    // head weight of every accumulator element this lane holds
    float wr[MT][16];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int h = 32 * mt + 8 * (r >> 2) + 4 * g + (r & 3);
            wr[mt][r] = h < H_I ? w[(int64_t)t * H_I + h] : 0.0f;
        }

    const uint8_t *krows = k_idx + (base[t] * DI) + g * G::HALF;
    float *srow = scores + (int64_t)t * ld;

    for (int64_t s0 = s_begin + (int64_t)wave * 32 * kIdxUnroll; s0 < s_end; s0 += kIdxStep) {
        v8i b[kIdxUnroll][G::KS];
#pragma unroll
        for (int u = 0; u < kIdxUnroll; ++u) {
            int64_t s = s0 + 32 * u + j;
            s = s < nt ? s : nt - 1;       // stay inside this query's rows
            load_run<DI>(krows + s * DI, b[u]);
        }
#pragma unroll
        for (int u = 0; u < kIdxUnroll; ++u) {
            float sum = 0.0f;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                v16f acc = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < G::KS; ++ks)
                    acc = mfma_fp8_32x32x64(a[mt][ks], b[u][ks], acc);
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    sum = fmaf(wr[mt][r], fmaxf(acc[r], 0.0f), sum);
            }
            sum += __shfl_xor(sum, 32);
            const int64_t s = s0 + 32 * u + j;
            if (g == 0 && s < s_end) {
                srow[s] = sum;
                if (hist0)
                    atomicAdd(&hist[ord_key(sum) >> kHistShift0], 1u);
            }
        }
    }
    if (hist0) {
        __syncthreads();
        uint32_t *h = hist0 + ((int64_t)t * kHistCopies + (blockIdx.x % kHistCopies)) * kHistBins0;
        for (int i = threadIdx.x; i < kHistBins0; i += 256)
            if (hist[i])
                atomicAdd(&h[i], hist[i]);
    }
}

template <int DI>
hipError_t launch_decode_di(const uint8_t *q_idx, const float *w, const uint8_t *k_idx,
                            const int64_t *base, const int32_t *n, int32_t T, int64_t max_n,
                            int32_t H_I, float *scores, int64_t ld, uint32_t *hist0, hipStream_t stream)
{
    // aim for >= 2048 workgroups over the whole call, chunks of >= one WG step
    int64_t total = max_n * (int64_t)T;
    int64_t chunk = kIdxStep;
    while (chunk < max_n && total / chunk > 2048 && chunk < (1 << 16))
        chunk *= 2;
    const int64_t nchunks = (max_n + chunk - 1) / chunk;
    if (nchunks == 0 || T == 0)
        return hipSuccess;
    dim3 grid((unsigned)nchunks, (unsigned)T);
    if (H_I <= 32)
        hipLaunchKernelGGL((indexer_decode_kernel<DI, 1>), grid, dim3(256), 0, stream, q_idx, w, k_idx,
                           base, n, H_I, scores, ld, chunk, hist0);
    else
        hipLaunchKernelGGL((indexer_decode_kernel<DI, 2>), grid, dim3(256), 0, stream, q_idx, w, k_idx,
                           base, n, H_I, scores, ld, chunk, hist0);
    return hipGetLastError();
}

// ---- prefill form ------------------------------------------------------------
// All queries read one sequence (causal prefill: query t sees tokens
// 0..n_t-1 of the shared cache), so a key tile staged in LDS serves a group of
// 16 queries: 8 waves x 2 queries, each wave holding its queries' q fragments
// and head weights in registers. Per 32-token group a wave reads the key
// fragments from LDS once and runs 4 MFMAs per query. Key rows sit in LDS with
// a 144-byte stride so the fragment reads (64 contiguous bytes per lane, lanes
// on consecutive rows) hit distinct banks. The next tile is loaded into
// registers while the current one is scored.
constexpr int kPfWaves = 8;
constexpr int kPfThreads = kPfWaves * 64;
constexpr int kPfQW = 2;                                  // queries per wave
constexpr int kPfQ = kPfWaves * kPfQW;                    // queries per workgroup
constexpr int kPfTile = 256;                              // tokens per LDS tile
constexpr int kPfRow = 144;                               // LDS bytes per key row
constexpr int kPfDI = 128;
constexpr int kPfLoads = kPfTile * kPfDI / 16 / kPfThreads;   // 16-byte loads per thread per tile

__global__ __launch_bounds__(kPfThreads, 1) void indexer_prefill_kernel(
    const uint8_t *__restrict__ q_idx, const float *__restrict__ w, const uint8_t *__restrict__ k_idx,
    const int64_t *__restrict__ base, const int32_t *__restrict__ n, int32_t T, float *__restrict__ scores,
    int64_t ld, int64_t chunk)
{
    using G = IdxGeom<kPfDI>;
    __shared__ __attribute__((aligned(16))) uint8_t keys[2][kPfTile * kPfRow];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int g = lane >> 5;
    const int j = lane & 31;
    const int t_base = blockIdx.y * kPfQ;

    // causal extent of the group: the largest n among its queries
    int64_t nmax = 0;
    for (int i = 0; i < kPfQ; ++i)
        if (t_base + i < T)
            nmax = max(nmax, (int64_t)n[t_base + i]);
    const int64_t s_begin = (int64_t)blockIdx.x * chunk;
    if (s_begin >= nmax)
        return;
    const int64_t s_end = min(nmax, s_begin + chunk);
    const uint8_t *krows = k_idx + base[t_base] * kPfDI;

    int tq[kPfQW];
    int64_t nq[kPfQW];
    v8i a[kPfQW][2][G::KS];
    float wr[kPfQW][2][16];
#pragma unroll
    for (int i = 0; i < kPfQW; ++i) {
        tq[i] = t_base + wave * kPfQW + i;
        const bool ok = tq[i] < T;
        nq[i] = ok ? n[tq[i]] : 0;
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

    // tile loads: chunk c of the tile = (row c / 8, 16-byte column c % 8)
    uint4 pre[kPfLoads];
    auto fetch = [&](int64_t tile) {
#pragma unroll
        for (int u = 0; u < kPfLoads; ++u) {
            const int c = tid + u * kPfThreads;
            int64_t row = tile + (c >> 3);
            row = row < s_end ? row : s_end - 1;
            pre[u] = *reinterpret_cast<const uint4 *>(krows + row * kPfDI + (c & 7) * 16);
        }
    };
    auto stage = [&](int buf) {
#pragma unroll
        for (int u = 0; u < kPfLoads; ++u) {
            const int c = tid + u * kPfThreads;
            *reinterpret_cast<uint4 *>(&keys[buf][(c >> 3) * kPfRow + (c & 7) * 16]) = pre[u];
        }
    };

    fetch(s_begin);
    int buf = 0;
    for (int64_t tile = s_begin; tile < s_end; tile += kPfTile, buf ^= 1) {
        stage(buf);
        __syncthreads();
        if (tile + kPfTile < s_end)
            fetch(tile + kPfTile);
        const int groups = (int)min((int64_t)(kPfTile / 32), (s_end - tile + 31) / 32);
        for (int grp = 0; grp < groups; ++grp) {
            const uint8_t *kr = &keys[buf][(32 * grp + j) * kPfRow + g * G::HALF];
            v8i b[G::KS];
#pragma unroll
            for (int ks = 0; ks < G::KS; ++ks) {
                const uint4 lo = *reinterpret_cast<const uint4 *>(kr + 32 * ks);
                const uint4 hi = *reinterpret_cast<const uint4 *>(kr + 32 * ks + 16);
                b[ks] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            }
            const int64_t s = tile + 32 * grp + j;
#pragma unroll
            for (int i = 0; i < kPfQW; ++i) {
                float sum = 0.0f;
#pragma unroll
                for (int mt = 0; mt < 2; ++mt) {
                    v16f acc = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < G::KS; ++ks)
                        acc = mfma_fp8_32x32x64(a[i][mt][ks], b[ks], acc);
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        sum = fmaf(wr[i][mt][r], fmaxf(acc[r], 0.0f), sum);
                }
                sum += __shfl_xor(sum, 32);
                if (g == 0 && s < nq[i])
                    scores[(int64_t)tq[i] * ld + s] = sum;
            }
        }
        // no barrier here: buffer `buf` is next written two tiles on, after the
        // barrier that follows the other buffer's staging
    }
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

hipError_t launch_indexer_prefill(const uint8_t *q_idx, const float *w, const uint8_t *k_idx,
                                  const int64_t *base, const int32_t *n, int32_t T, int64_t max_n,
                                  int32_t H_I, int32_t D_I, float *scores, int64_t ld, hipStream_t stream)
{
    if (!indexer_prefill_supported(H_I, D_I))
        return hipErrorInvalidValue;
    if (T == 0 || max_n == 0)
        return hipSuccess;
    const int64_t groups = (T + kPfQ - 1) / kPfQ;
    // token chunks: enough workgroups to fill the chip several times over
    int64_t chunk = kPfTile;
    while (chunk < max_n && groups * ((max_n + chunk - 1) / chunk) > 16384)
        chunk *= 2;
    const int64_t nchunks = (max_n + chunk - 1) / chunk;
    if (groups > 65535)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(indexer_prefill_kernel, dim3((unsigned)nchunks, (unsigned)groups), dim3(kPfThreads), 0,
                       stream, q_idx, w, k_idx, base, n, T, scores, ld, chunk);
    return hipGetLastError();
}

}  // namespace ic
