// Exact per-query top-k selection (explainer "Hy4 IndexCache cross-layer
// index reuse", Jargon "Top-k selection"; k = 2048 on the GitHub issue
// "rtx6kpro #90"): keep the k largest scores of positions 0..n_t-1, the lower
// position winning among equal scores, emitted in ascending position order.
//
// Method: radix select over an order-preserving 32-bit image of the fp32
// score, in three digits (bits 31..21, 20..10, 9..0). Each digit's histogram
// finds the bin holding the k-th largest key; after the last digit the k-th
// key `thr` is known, with `need` = how many keys equal to thr are kept. A
// final ordered compaction walks the keys in position order: a key above thr
// is kept, a key equal to thr is kept while fewer than `need` equal keys came
// before it, and its output slot is (#kept keys above thr before it) +
// min(#equal keys before it, need) -- a prefix sum of packed (above, equal)
// counts.
//
// Only keys at or above a bound on the k-th largest key (about k of them)
// take part in the digits, in LDS:
//   * split path (few queries, long rows): P workgroups per query each read
//     a fixed sample of the row (blocks of 32 scores spread over it), derive
//     from it the same two-digit bound, which at least k keys reach with high
//     probability, and copy their chunk's keys at or above it, in position
//     order, into their own slice of the workspace (topk_collect_kernel); one
//     workgroup per query gathers those into LDS and finishes there
//     (topk_finish_kernel), or over the whole row when fewer than k keys
//     reached the bound. The kernel boundary orders the two phases.
//     Scores spanning less than a factor of two share a handful of
//     first-digit bins (the digit holds two mantissa bits), so a bound from
//     the first digit alone could keep half a row.
//   * row path (many queries): one workgroup per query. Rows of at least
//     kSampleMinN scores take the same kind of bound from 1/16 of the row;
//     shorter ones, and rows whose sampled bound fails, take the first digit's
//     histogram (built while the scores were produced -- the indexer kernel can
//     add into it -- or by one pass here), then stream the row once more to
//     collect its survivors into LDS and finish there. When those exceed the
//     LDS list (the threshold fell into a dense first-digit bin), the second
//     digit's histogram over the survivors kept in global memory keeps only
//     those at or above the second-digit threshold.
// Only ties spanning more than a list fall back to digit passes over the
// full row.
// The first-digit histogram a producer fills is kept in kHistCopies copies per
// query (adders pick a copy by workgroup index, which spreads atomic traffic);
// the caller clears them before the producer runs (clear_hist0_kernel) and
// the row kernel returns them to zero after reading them, so the next producer
// in the same call finds them clear.
#include <algorithm>

#include "kernels.h"
#include "radix_key.h"
#include "select.h"

namespace ic {
namespace {

constexpr int kSplitThreads = 1024;
constexpr int kSplitRuns = 2;                      // groups of 4 consecutive scores per survivors thread
constexpr int kSplitChunk = kSplitThreads * 4 * kSplitRuns;   // scores per split workgroup
constexpr int kRowThreads = 1024;
constexpr int kFinishThreads = 1024;
constexpr int kListCap = 18432;         // survivors held in LDS (split path)
constexpr int kRowListCap = 8192;       // survivors held in LDS (row path: two workgroups per CU)
constexpr int kRowRuns = 2;             // consecutive groups of 4 scores per thread per collect round
constexpr int kMaxSplit = 1024;         // workgroups per query on the split path
constexpr int kSpec = 8;                // slice entries per finishing thread loaded ahead of the counts
constexpr int kRowSurvCap = 32768;      // survivors kept in global memory per query (row path)

// Finish from a survivor list `src` (keys with first digit >= d0, position
// order, `total` entries) that does not fit the LDS list: histogram the second
// digit over the first-digit bin, keep only keys at or above the second-digit
// threshold (they fit unless ties span the list), finish from the third digit.
template <int NT, class Src, class Fallback>
__device__ void finish_from_overflow(const Src &src, const Fallback &row, Shared &sh, uint64_t *list,
                                     uint32_t list_cap, uint32_t d0, uint32_t need0, int32_t k,
                                     int32_t *__restrict__ out)
{
    const uint32_t p0 = d0 << 21;
    for (int i = threadIdx.x; i < kBins0; i += NT)
        sh.hist[i] = 0;
    __syncthreads();
    for_each_key<NT>(src, [&](uint32_t key, bool ok) {
        hist_add_wave(sh.hist, (key >> 10) & 2047, ok && (key & 0xFFE00000u) == p0);
    });
    __syncthreads();
    uint32_t d1, above1;
    find_digit<NT>(sh, 2048, need0, d1, above1);
    const uint32_t bound = p0 | (d1 << 10);
    const uint32_t cnt = collect<NT>(src, bound, sh, list, list_cap, nullptr, 0);
    if (cnt <= list_cap)
        finish_select<NT>(ListSrc{list, cnt}, sh, 2, bound, 0xFFFFFC00u, need0 - above1, k, out);
    else
        finish_select<NT>(row, sh, 2, bound, 0xFFFFFC00u, need0 - above1, k, out);
}

template <int NT>
__device__ void write_all(int32_t *out, int64_t nt, int32_t k)
{
    for (int i = threadIdx.x; i < k; i += NT)
        out[i] = i < nt ? i : -1;
}

// Sum the histogram copies of one query into LDS.
template <int NT>
__device__ void load_hist0(Shared &sh, const uint32_t *h)
{
    for (int i = threadIdx.x * 4; i < kBins0; i += NT * 4) {
        uint4 acc = *reinterpret_cast<const uint4 *>(h + i);
#pragma unroll
        for (int c = 1; c < kHistCopies; ++c) {
            const uint4 v = *reinterpret_cast<const uint4 *>(h + c * kBins0 + i);
            acc.x += v.x, acc.y += v.y, acc.z += v.z, acc.w += v.w;
        }
        *reinterpret_cast<uint4 *>(&sh.hist[i]) = acc;
    }
    __syncthreads();
}

template <int NT>
__device__ void zero_hist0(uint32_t *h)
{
    for (int i = threadIdx.x * 4; i < kBins0 * kHistCopies; i += NT * 4)
        *reinterpret_cast<uint4 *>(h + i) = make_uint4(0, 0, 0, 0);
}

// ---- split path -------------------------------------------------------------
// The row's sample for the bound: blocks of kSplitSampleBlock consecutive
// scores, one every G blocks, G = ceil(n / kSplitSamples): the whole row when
// n <= kSplitSamples, otherwise between kSplitSamples / 2 and kSplitSamples
// scores spread over all of it.
constexpr int kSplitSampleBlock = 32;
constexpr int kSplitSamples = 4096;
static_assert(kSplitSamples % (kSplitThreads * 4) == 0, "whole groups of four samples per thread");
static_assert(kSplitSampleBlock % 4 == 0, "groups of four stay inside a sampled block");

// The sample's slots of this thread: geometry from `n_geo` (the longest row of
// the call, known before the row's own length arrives), loads bounded by the
// row's capacity `cap` (a multiple of 4, at least 4); split_bound masks them
// by the row's length.
template <int NT>
struct SplitSample {
    static constexpr int G = kSplitSamples / (NT * 4);     // groups of four samples per thread
    uint32_t key[G][4];
    int64_t pos[G][4];
    bool ok[G][4];
    __device__ void load(const float *row, int64_t cap, int64_t n_geo)
    {
        const int64_t sb = (n_geo + kSplitSamples - 1) / kSplitSamples * kSplitSampleBlock;   // block spacing
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int64_t s = ((int64_t)threadIdx.x + (int64_t)NT * g) * 4;     // first sample slot
            row_get4u(row, cap, s / kSplitSampleBlock * sb + s % kSplitSampleBlock, key[g], pos[g], ok[g]);
        }
    }
};

// Two-digit key bound that at least k keys of the row reach with high
// probability: the bound of the key whose rank among the samples is 1.5 times
// the k-th largest key's expected rank, plus 16 (the finishing workgroup
// checks the count). 0 (every key) when the sample is too small for that.
template <int NT>
__device__ uint32_t split_bound(SplitSample<NT> &sp, int64_t n, int32_t k, Shared &sh)
{
    constexpr int G = SplitSample<NT>::G;
    auto &key = sp.key;
    auto &ok = sp.ok;
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            ok[g][e] = ok[g][e] && sp.pos[g][e] < n;
    for (int i = threadIdx.x; i < kBins0; i += NT)
        sh.hist[i] = 0;
    __syncthreads();
    uint32_t mine = 0;
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            mine += ok[g][e];
            hist_add_wave(sh.hist, key[g][e] >> 21, ok[g][e]);
        }
    uint32_t ns;
    block_scan<NT>(mine, sh.waves, &ns);          // its barriers also close the histogram
    const uint64_t tgt = ((uint64_t)k * ns * 3 + (uint64_t)n * 2 - 1) / ((uint64_t)n * 2) + 16;
    if (tgt > ns)
        return 0u;
    uint32_t b, above;
    find_digit<NT>(sh, kBins0, (uint32_t)tgt, b, above);
    for (int i = threadIdx.x; i < kBins0; i += NT)
        sh.hist[i] = 0;
    __syncthreads();
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (ok[g][e] && (key[g][e] >> 21) == b)
                atomicAdd(&sh.hist[(key[g][e] >> 10) & (kBins0 - 1)], 1u);
    __syncthreads();
    uint32_t d1, above1;
    find_digit<NT>(sh, kBins0, (uint32_t)tgt - above, d1, above1);
    return (b << 21) | (d1 << 10);
}

// Phase 1. grid: (P, T); block: kSplitThreads; kSplitChunk scores per
// workgroup. Every workgroup of a query derives the same bound from the same
// sample, then copies its chunk's keys at or above it, in position order,
// into its slice of `regions`, and their count to counts; workgroup 0
// publishes the bound.
__global__ __launch_bounds__(kSplitThreads) void topk_collect_kernel(const float *__restrict__ scores, int64_t ld,
                                                                     const int32_t *__restrict__ n, int64_t max_n,
                                                                     int32_t k, uint32_t *__restrict__ counts,
                                                                     uint64_t *__restrict__ regions,
                                                                     uint32_t *__restrict__ bounds)
{
    constexpr int NT = kSplitThreads;
    __shared__ Shared sh;
    const int t = blockIdx.y;
    const int w = blockIdx.x;
    const int P = gridDim.x;
    const int tid = threadIdx.x;
    const float *row = scores + (int64_t)t * ld;
    // this chunk's scores and the sample, issued before the row's length
    // arrives (loads stay inside the row's capacity ld; positions at or past
    // the length are dropped once it is known)
    const int64_t s = (int64_t)w * kSplitChunk + (int64_t)tid * 4 * kSplitRuns;
    uint32_t key[kSplitRuns][4];
    int64_t pos[kSplitRuns][4];
    bool ok[kSplitRuns][4];
#pragma unroll
    for (int r = 0; r < kSplitRuns; ++r)
        row_get4u(row, ld, s + 4 * r, key[r], pos[r], ok[r]);
    SplitSample<NT> sp;
    sp.load(row, ld, max_n);
    const int64_t nt = n[t];
    if (nt <= k)
        return;                                   // the finish kernel keeps everything
    const uint32_t bound = split_bound<NT>(sp, nt, k, sh);
    uint32_t ls = 0;
#pragma unroll
    for (int r = 0; r < kSplitRuns; ++r)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            ok[r][e] = ok[r][e] && pos[r][e] < nt && key[r][e] >= bound;
            ls += ok[r][e];
        }
    uint32_t tot;
    uint32_t o = block_scan<NT>(ls, sh.waves, &tot) - ls;
    uint64_t *reg = regions + ((int64_t)t * P + w) * kSplitChunk;
#pragma unroll
    for (int r = 0; r < kSplitRuns; ++r)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (ok[r][e])
                reg[o++] = ((uint64_t)key[r][e] << 32) | (uint32_t)pos[r][e];
    if (tid == 0) {
        counts[(int64_t)t * P + w] = tot;
        if (w == 0)
            bounds[t] = bound;                    // every workgroup found the same bound
    }
}

// Phase 2. grid: T; block: kFinishThreads. The first C = min(kSpec * NT / P,
// kSplitChunk) entries of every slice are loaded together with the slice
// counts, before these are known (one round trip, instead of a second one
// once the counts are scanned). Each key is stored at its rank in the LDS
// list (slice order = position order), slices longer than C adding the rest.
// If at least k keys reached the bound, the k-th largest key and all its ties
// are among them and the three digits finish from the list; with fewer, or
// more than the list holds, they finish from the whole row. The kernel reads
// back none of its global stores, so its barriers order LDS traffic only.
__global__ __launch_bounds__(kFinishThreads) void topk_finish_kernel(
    const float *__restrict__ scores, int64_t ld, const int32_t *__restrict__ n, int32_t k,
    int32_t *__restrict__ idx, const uint32_t *__restrict__ counts,
    const uint64_t *__restrict__ regions, int32_t P, const uint32_t *__restrict__ bounds)
{
    constexpr int NT = kFinishThreads;
    constexpr bool LB = true;
    __shared__ Shared sh;
    __shared__ __align__(16) uint64_t list[kListCap];
    __shared__ uint32_t offs[kMaxSplit + 1];
    __shared__ uint32_t long_slice;
    const int t = blockIdx.x;
    const int tid = threadIdx.x;
    int32_t *out = idx + (int64_t)t * k;
    // loads first (slice counts, slice prefixes: inside the workspace whatever
    // the row's length, which they do not wait for)
    static_assert(kMaxSplit <= NT, "one scan over the slices");
    static_assert((NT * kSpec) / kMaxSplit >= 1 && kSplitChunk <= 8192 && NT * kSpec <= 8192,
                  "C >= 1; slice and entry fit 13 bits each");
    const uint32_t c0 = tid < P ? counts[(int64_t)t * P + tid] : 0u;
    const uint32_t bound = bounds[t];
    const uint64_t *reg_t = regions + (int64_t)t * P * kSplitChunk;
    const uint32_t C = min((uint32_t)(NT * kSpec) / (uint32_t)P, (uint32_t)kSplitChunk);
    uint64_t sv[kSpec];
    uint32_t slot[kSpec];                         // slice << 13 | entry
#pragma unroll
    for (int e = 0; e < kSpec; ++e) {
        const uint32_t f = (uint32_t)tid + (uint32_t)NT * e;
        const uint32_t sl = f / C, j = f - sl * C;
        slot[e] = (sl << 13) | j;
        sv[e] = sl < (uint32_t)P ? reg_t[(int64_t)sl * kSplitChunk + j] : 0ull;
    }
    const int64_t nt = n[t];
    if (nt <= k) {
        write_all<NT>(out, nt, k);
        return;
    }
    // slice offsets (P <= NT: one scan)
    if (tid == 0)
        long_slice = 0;
    wg_barrier<LB>();
    if (tid < P && c0 > C)
        long_slice = 1;
    uint32_t total;
    const uint32_t excl = block_scan<NT, LB>(c0, sh.waves, &total) - c0;
    if (tid < P)
        offs[tid] = excl;
    if (tid == 0)
        offs[P] = total;
    wg_barrier<LB>();
    if (total < (uint32_t)k || total > (uint32_t)kListCap) {
        finish_select<NT, LB>(RowSrc{scores + (int64_t)t * ld, nt}, sh, 0, 0u, 0u, (uint32_t)k, k, out);
        return;
    }
#pragma unroll
    for (int e = 0; e < kSpec; ++e) {
        const uint32_t sl = slot[e] >> 13, j = slot[e] & 0x1FFFu;
        if (sl < (uint32_t)P) {
            const uint32_t o = offs[sl];
            if (j < offs[sl + 1] - o)
                list[o + j] = sv[e];
        }
    }
    if (long_slice) {
        // the entries past C of the longer slices, by rank among them; their
        // offsets go to sh.hist, free until the first digit
        const uint32_t rem = tid < P && c0 > C ? c0 - C : 0u;
        uint32_t rtot;
        const uint32_t rex = block_scan<NT, LB>(rem, sh.waves, &rtot) - rem;
        if (tid < P)
            sh.hist[tid] = rex;
        wg_barrier<LB>();
        for (uint32_t r0 = 0; r0 < rtot; r0 += (uint32_t)NT * 4) {
            uint64_t v[4];
            uint32_t dst[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const uint32_t r = r0 + (uint32_t)tid + (uint32_t)NT * u;
                dst[u] = 0xFFFFFFFFu;
                if (r < rtot) {
                    int lo = 0, hi = P;                   // last slice whose rest starts at or before r
                    while (hi - lo > 1) {
                        const int mid = (lo + hi) >> 1;
                        if (sh.hist[mid] <= r)
                            lo = mid;
                        else
                            hi = mid;
                    }
                    const uint32_t j = C + (r - sh.hist[lo]);
                    dst[u] = offs[lo] + j;
                    v[u] = reg_t[(int64_t)lo * kSplitChunk + j];
                }
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (dst[u] != 0xFFFFFFFFu)
                    list[dst[u]] = v[u];
        }
    }
    wg_barrier<LB>();
    // The listed keys' top 22 bits, less the bound's, rarely span 2048 bins:
    // one histogram of that difference (the last bin taking everything from
    // 2047 up) gives the k-th key's two leading digits, unless it lands in
    // the last bin; then the digits run from the first.
    const ListSrc src{list, total};
    const uint32_t b22 = bound >> 10;
    for (int i = tid; i < kBins0; i += NT)
        sh.hist[i] = 0;
    wg_barrier<LB>();
    for_each_key<NT>(src, [&](uint32_t key, bool ok) {
        if (ok)
            atomicAdd(&sh.hist[min((key >> 10) - b22, (uint32_t)kBins0 - 1)], 1u);
    });
    wg_barrier<LB>();
    uint32_t rel, above;
    find_digit<NT, LB>(sh, kBins0, (uint32_t)k, rel, above);
    const uint32_t in_bin = sh.count;
    const uint32_t pre = (b22 + rel) << 10;
    if (rel == (uint32_t)kBins0 - 1)
        finish_select<NT, LB>(src, sh, 0, 0u, 0u, (uint32_t)k, k, out);
    else if (in_bin == (uint32_t)k - above && pre != 0u)
        // every key of the k-th key's bin is kept: the selection is the keys
        // at or above the bin's lowest key, no last digit needed
        finish_select<NT, LB>(src, sh, 3, pre - 1u, 0xFFFFFFFFu, 0u, k, out);
    else
        finish_select<NT, LB>(src, sh, 2, pre, 0xFFFFFC00u, (uint32_t)k - above, k, out);
}

// ---- row path ---------------------------------------------------------------
// Long rows skip the full histogram pass: blocks of kSampleBlock scores at
// every kSampleStride-th block (1/16 of the row) are read twice -- the first
// digit's histogram, then the second digit's inside the bin that holds the
// target rank -- and give a two-digit key bound with, among the samples, a
// quarter more keys at or above it than the k-th largest key is expected to
// have. One pass then collects every key of the row at or above the bound; if
// there are at least k of them, the k-th largest key and all its ties are
// among them, and the selection finishes from that list. Otherwise (or when
// they exceed the global list) the row takes the exact two-pass path.
constexpr int kSampleBlock = 256;          // consecutive scores per sampled block
constexpr int kSampleStride = 16;          // one block in kSampleStride is sampled
constexpr int64_t kSampleMinN = 65536;     // shorter rows take the two-pass path
static_assert(kSampleBlock % 4 == 0, "groups of four stay inside a sampled block");

// Returns the bound, or 0 when the samples cannot give one.
template <int NT>
__device__ uint32_t sampled_bound(const RowSrc &src, int32_t k, Shared &sh)
{
    const int64_t nblocks = (src.n + kSampleBlock - 1) / kSampleBlock;
    const int64_t slots = (nblocks + kSampleStride - 1) / kSampleStride * kSampleBlock;
    auto at = [](int64_t s) {                      // row position of sample slot s
        return s / kSampleBlock * (int64_t)(kSampleBlock * kSampleStride) + s % kSampleBlock;
    };
    for (int i = threadIdx.x; i < kBins0; i += NT)
        sh.hist[i] = 0;
    __syncthreads();
    uint32_t mine = 0;
    for (int64_t s0 = (int64_t)threadIdx.x * 4; s0 < slots; s0 += (int64_t)NT * 4) {
        uint32_t key[4];
        int64_t pos[4];
        bool ok[4];
        src.get4(at(s0), key, pos, ok);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            mine += ok[e];
            hist_add_wave(sh.hist, key[e] >> 21, ok[e]);
        }
    }
    uint32_t ns;
    block_scan<NT>(mine, sh.waves, &ns);           // its barriers also close the histogram
    // the k-th largest key's expected rank among the samples, plus a quarter and 16
    const uint64_t tgt = ((uint64_t)k * ns * 5 + (uint64_t)src.n * 4 - 1) / ((uint64_t)src.n * 4) + 16;
    if (tgt > ns)
        return 0u;
    uint32_t b, above;
    find_digit<NT>(sh, kBins0, (uint32_t)tgt, b, above);
    for (int i = threadIdx.x; i < kBins0; i += NT)
        sh.hist[i] = 0;
    __syncthreads();
    for (int64_t s0 = (int64_t)threadIdx.x * 4; s0 < slots; s0 += (int64_t)NT * 4) {
        uint32_t key[4];
        int64_t pos[4];
        bool ok[4];
        src.get4(at(s0), key, pos, ok);
#pragma unroll
        for (int e = 0; e < 4; ++e)
            hist_add_wave(sh.hist, (key[e] >> 10) & (kBins0 - 1), ok[e] && (key[e] >> 21) == b);
    }
    __syncthreads();
    uint32_t d1, above1;
    find_digit<NT>(sh, kBins0, (uint32_t)tgt - above, d1, above1);
    return (b << 21) | (d1 << 10);
}


// grid: T; block: 1024. With `hist0` non-null the first digit's histogram is
// taken from it (and zeroed); otherwise it is built here.
__global__ __launch_bounds__(kRowThreads) void topk_row_kernel(const float *__restrict__ scores, int64_t ld,
                                                               const int32_t *__restrict__ n, int32_t k,
                                                               int32_t *__restrict__ idx,
                                                               uint32_t *__restrict__ hist0,
                                                               uint64_t *__restrict__ surv,
                                                               const uint32_t *__restrict__ gate)
{
    __shared__ Shared sh;
    __shared__ __align__(16) uint64_t list[kRowListCap];
    const int t = blockIdx.x;
    if (gate && gate[t] == 0u)                    // a gated launch serves the marked queries only
        return;
    const int tid = threadIdx.x;
    const int64_t nt = n[t];
    int32_t *out = idx + (int64_t)t * k;
    const float *row = scores + (int64_t)t * ld;
    const RowSrc src{row, nt};
    uint32_t *h0 = hist0 ? hist0 + (int64_t)t * kHistCopies * kBins0 : nullptr;

    if (nt <= k) {
        write_all<kRowThreads>(out, nt, k);
        if (h0)
            zero_hist0<kRowThreads>(h0);
        return;
    }
    uint64_t *gl = surv + (int64_t)t * kRowSurvCap;
    if (h0) {
        load_hist0<kRowThreads>(sh, h0);
        zero_hist0<kRowThreads>(h0);
    } else {
        if (nt >= kSampleMinN) {
            const uint32_t bound = sampled_bound<kRowThreads>(src, k, sh);
            if (bound != 0u) {
                const uint32_t c = collect<kRowThreads, kRowRuns>(src, bound, sh, list, (uint32_t)kRowListCap, gl,
                                                                  (uint32_t)kRowSurvCap);
                if (c >= (uint32_t)k && c <= (uint32_t)kRowListCap) {
                    finish_select<kRowThreads>(ListSrc{list, c}, sh, 0, 0u, 0u, (uint32_t)k, k, out);
                    return;
                }
                if (c >= (uint32_t)k && c <= (uint32_t)kRowSurvCap) {
                    finish_select<kRowThreads>(GListSrc{gl, c}, sh, 0, 0u, 0u, (uint32_t)k, k, out);
                    return;
                }
            }
        }
        for (int i = tid; i < kBins0; i += kRowThreads)
            sh.hist[i] = 0;
        __syncthreads();
        for (int64_t i = (int64_t)tid * 4; i < nt; i += (int64_t)kRowThreads * 4) {
            uint32_t key[4];
            int64_t pos[4];
            bool ok[4];
            src.get4(i, key, pos, ok);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                hist_add_wave(sh.hist, key[e] >> 21, ok[e]);
        }
        __syncthreads();
    }
    uint32_t d0, above0;
    find_digit<kRowThreads>(sh, kBins0, (uint32_t)k, d0, above0);
    const uint32_t need = (uint32_t)k - above0;
    // survivors in position order: into LDS, and into this query's global list
    const uint32_t total = collect<kRowThreads, kRowRuns>(src, d0 << 21, sh, list, (uint32_t)kRowListCap, gl,
                                                           (uint32_t)kRowSurvCap);
    if (total <= (uint32_t)kRowListCap)
        finish_select<kRowThreads>(ListSrc{list, total}, sh, 1, d0 << 21, 0xFFE00000u, need, k, out);
    else if (total <= (uint32_t)kRowSurvCap)
        finish_from_overflow<kRowThreads>(GListSrc{gl, total}, src, sh, list, (uint32_t)kRowListCap, d0, need, k,
                                          out);
    else
        finish_select<kRowThreads>(src, sh, 1, d0 << 21, 0xFFE00000u, need, k, out);
}

// ---- causal prefill with bounded collection ---------------------------------
// The prefill indexer first scores a strided sample of the keys (one in
// kPfSampleStride). Per query, prefill_bound_kernel takes from the sample
// scores a two-digit key bound at a sample rank of twice the k-th largest
// key's expected rank plus 16; the collecting indexer then keeps every score
// at or above the bound, per (query, token chunk) slice in position order,
// and prefill_select_kernel finishes the selection from the slices. When at
// least k scores reach the bound, the k-th largest key and all its ties are
// among them, so the result is exact. A query with fewer than k, a slice
// past its capacity, or more than fit the LDS list is marked in `need`;
// the scores path (indexer and row top-k, gated by `need`) then serves it.
constexpr int kPfSelMaxChunks = 1024;      // token chunks per query the selection reads

// grid: T; block: kRowThreads. bound[t] = 0xFFFFFFFF when n_t <= k (nothing
// to collect: every position is kept) or when `none` is set (nothing
// collected: every longer query takes the score rows), 0 when the sample
// cannot bound the k-th key (everything is collected).
__global__ __launch_bounds__(kRowThreads) void prefill_bound_kernel(const float *__restrict__ sample, int64_t ld,
                                                                    const int32_t *__restrict__ n, int32_t k,
                                                                    uint32_t *__restrict__ bound, int32_t none)
{
    __shared__ Shared sh;
    const int t = blockIdx.x;
    const int64_t nt = n[t];
    if (nt <= k || none) {
        if (threadIdx.x == 0)
            bound[t] = 0xFFFFFFFFu;
        return;
    }
    const int64_t ns = (nt + kPfSampleStride - 1) / kPfSampleStride;
    const uint64_t tgt = 2 * (((uint64_t)k * ns + nt - 1) / nt) + 16;
    if (tgt > (uint64_t)ns) {
        if (threadIdx.x == 0)
            bound[t] = 0u;
        return;
    }
    const RowSrc src{sample + (int64_t)t * ld, ns};
    uint32_t b = 0, above = 0, d1 = 0, above1 = 0;
    for (int pass = 0; pass < 2; ++pass) {
        for (int i = threadIdx.x; i < kBins0; i += kRowThreads)
            sh.hist[i] = 0;
        __syncthreads();
        for (int64_t i = (int64_t)threadIdx.x * 4; i < ns; i += (int64_t)kRowThreads * 4) {
            uint32_t key[4];
            int64_t pos[4];
            bool ok[4];
            src.get4(i, key, pos, ok);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (pass == 0)
                    hist_add_wave(sh.hist, key[e] >> 21, ok[e]);
                else if (ok[e] && (key[e] >> 21) == b)
                    atomicAdd(&sh.hist[(key[e] >> 10) & (kBins0 - 1)], 1u);
            }
        }
        __syncthreads();
        if (pass == 0)
            find_digit<kRowThreads>(sh, kBins0, (uint32_t)tgt, b, above);
        else
            find_digit<kRowThreads>(sh, kBins0, (uint32_t)tgt - above, d1, above1);
        __syncthreads();
    }
    if (threadIdx.x == 0)
        bound[t] = (b << 21) | (d1 << 10);
}

// grid: T; block: kRowThreads. Query t's slices are those of the token
// chunks its n_t rows reach; idx row t is written unless the query is marked.
__global__ __launch_bounds__(kRowThreads) void prefill_select_kernel(const uint64_t *__restrict__ slices,
                                                                     const uint32_t *__restrict__ counts,
                                                                     int32_t nchunks, int64_t chunk, int32_t cap,
                                                                     const int32_t *__restrict__ n, int32_t k,
                                                                     int32_t *__restrict__ idx,
                                                                     uint32_t *__restrict__ need)
{
    __shared__ Shared sh;
    __shared__ __align__(16) uint64_t list[kRowListCap];
    __shared__ uint32_t offs[kPfSelMaxChunks + 1];
    __shared__ uint32_t bad;
    const int t = blockIdx.x;
    const int tid = threadIdx.x;
    const int64_t nt = n[t];
    int32_t *out = idx + (int64_t)t * k;
    if (nt <= k) {
        write_all<kRowThreads>(out, nt, k);
        if (tid == 0)
            need[t] = 0u;
        return;
    }
    const int64_t nch = (nt + chunk - 1) / chunk;
    if (nch > kPfSelMaxChunks) {
        if (tid == 0)
            need[t] = 1u;
        return;
    }
    if (tid == 0)
        bad = 0u;
    __syncthreads();
    // chunk counts, their running offsets and the total
    uint32_t total = 0;
    for (int64_t j0 = 0; j0 < nch; j0 += kRowThreads) {
        const int64_t j = j0 + tid;
        const uint32_t c = j < nch ? counts[(int64_t)t * nchunks + j] : 0u;
        if (c > (uint32_t)cap)
            bad = 1u;
        uint32_t tot;
        const uint32_t incl = block_scan<kRowThreads>(c, sh.waves, &tot);
        if (j < nch)
            offs[j + 1] = total + incl;
        total += tot;
    }
    if (tid == 0)
        offs[0] = 0u;
    __syncthreads();
    if (bad || total < (uint32_t)k || total > (uint32_t)kRowListCap) {
        if (tid == 0)
            need[t] = 1u;
        return;
    }
    // gather the slices into one position-ordered list
    const uint64_t *sl = slices + (int64_t)t * nchunks * cap;
    for (uint32_t f = tid; f < total; f += kRowThreads) {
        int lo = 0, hi = (int)nch - 1;                // chunk j with offs[j] <= f < offs[j + 1]
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (offs[mid] <= f)
                lo = mid;
            else
                hi = mid - 1;
        }
        list[f] = sl[(int64_t)lo * cap + (f - offs[lo])];
    }
    __syncthreads();
    finish_select<kRowThreads>(ListSrc{list, total}, sh, 0, 0u, 0u, (uint32_t)k, k, out);
    if (tid == 0)
        need[t] = 0u;
}

// grid-stride fill of the first-digit histograms with zeros (a kernel, not a
// memset: calls are captured into HIP graphs)
__global__ __launch_bounds__(256) void clear_hist0_kernel(uint4 *__restrict__ h, int64_t n4)
{
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256)
        h[i] = make_uint4(0, 0, 0, 0);
}

struct TopkLayout {
    bool split;
    int64_t P;
    size_t hist_off, counts_off, bounds_off, regions_off, total;
};

size_t up256(size_t x) { return (x + 255) / 256 * 256; }

TopkLayout topk_layout(int32_t T, int64_t max_n)
{
    TopkLayout L{};
    L.P = (max_n + kSplitChunk - 1) / kSplitChunk;
    if (L.P < 1)
        L.P = 1;
    // split when the queries alone cannot fill the chip and the survivor
    // slices stay small
    L.split = T < 256 && (int64_t)T * L.P * kSplitChunk <= ((int64_t)1 << 26) && L.P <= kMaxSplit;
    // first-digit histogram copies (counters that start and end at zero)
    L.hist_off = 0;
    L.counts_off = up256((size_t)T * kHistCopies * kBins0 * 4);
    if (L.split) {
        L.bounds_off = L.counts_off + up256((size_t)T * L.P * 4);
        L.regions_off = L.bounds_off + up256((size_t)T * 4);
        L.total = L.regions_off + up256((size_t)T * L.P * kSplitChunk * 8);
    } else {
        L.regions_off = L.counts_off;
        L.total = L.regions_off + up256((size_t)T * kRowSurvCap * 8);
    }
    return L;
}

}  // namespace

size_t topk_workspace_bytes(int32_t T, int64_t max_n, int32_t) { return topk_layout(T, max_n).total; }

uint32_t *topk_hist0(void *ws) { return reinterpret_cast<uint32_t *>(ws); }

bool topk_reads_hist0(int32_t T, int64_t max_n) { return !topk_layout(T, max_n).split; }

hipError_t launch_clear_hist0(void *ws, int32_t T, hipStream_t stream)
{
    const int64_t n4 = (int64_t)T * kHistCopies * kBins0 / 4;
    if (n4 == 0)
        return hipSuccess;
    const int64_t blocks = std::min<int64_t>((n4 + 255) / 256, 1024);
    if (!trace_skip("clear_hist0_kernel"))
        hipLaunchKernelGGL(clear_hist0_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       reinterpret_cast<uint4 *>(ws), n4);
    trace_launch(stream, "clear_hist0_kernel");
    return hipGetLastError();
}

bool topk_split_view(void *ws, int32_t T, int64_t max_n, TopkSplitView *v)
{
    const TopkLayout L = topk_layout(T, max_n);
    if (!L.split)
        return false;
    char *base = static_cast<char *>(ws);
    v->counts = reinterpret_cast<const uint32_t *>(base + L.counts_off);
    v->regions = reinterpret_cast<const uint64_t *>(base + L.regions_off);
    v->bounds = reinterpret_cast<const uint32_t *>(base + L.bounds_off);
    v->P = (int32_t)L.P;
    v->stride = kSplitChunk;
    return true;
}

hipError_t launch_topk_collect(const float *scores, int64_t ld, const int32_t *n, int32_t T, int64_t max_n,
                               int32_t k, void *ws, hipStream_t stream)
{
    const TopkLayout L = topk_layout(T, max_n);
    if (T == 0)
        return hipSuccess;
    if (!L.split || ld < 4)
        return hipErrorInvalidValue;              // (its loads need rows of at least 4 scores)
    char *base = static_cast<char *>(ws);
    if (!trace_skip("topk_collect_kernel"))
        hipLaunchKernelGGL(topk_collect_kernel, dim3((unsigned)L.P, (unsigned)T), dim3(kSplitThreads), 0, stream,
                           scores, ld, n, max_n, k, reinterpret_cast<uint32_t *>(base + L.counts_off),
                           reinterpret_cast<uint64_t *>(base + L.regions_off),
                           reinterpret_cast<uint32_t *>(base + L.bounds_off));
    trace_launch(stream, "topk_collect_kernel");
    return hipGetLastError();
}

hipError_t launch_prefill_bound(const float *sample, int64_t ld, const int32_t *n, int32_t T, int32_t k,
                                uint32_t *bound, bool none, hipStream_t stream)
{
    if (T == 0)
        return hipSuccess;
    if (!trace_skip("prefill_bound_kernel"))
        hipLaunchKernelGGL(prefill_bound_kernel, dim3((unsigned)T), dim3(kRowThreads), 0, stream, sample, ld, n, k,
                           bound, (int32_t)none);
    trace_launch(stream, "prefill_bound_kernel");
    return hipGetLastError();
}

hipError_t launch_prefill_select(const uint64_t *slices, const uint32_t *counts, int32_t nchunks, int64_t chunk,
                                 int32_t cap, const int32_t *n, int32_t T, int32_t k, int32_t *idx, uint32_t *need,
                                 hipStream_t stream)
{
    if (T == 0)
        return hipSuccess;
    if (!trace_skip("prefill_select_kernel"))
        hipLaunchKernelGGL(prefill_select_kernel, dim3((unsigned)T), dim3(kRowThreads), 0, stream, slices, counts,
                           nchunks, chunk, cap, n, k, idx, need);
    trace_launch(stream, "prefill_select_kernel");
    return hipGetLastError();
}

hipError_t launch_topk(const float *scores, int64_t ld, const int32_t *n, int32_t T, int64_t max_n, int32_t k,
                       int32_t *idx, void *ws, bool hist_ready, hipStream_t stream, const uint32_t *need)
{
    if (T == 0)
        return hipSuccess;
    const TopkLayout L = topk_layout(T, max_n);
    char *base = static_cast<char *>(ws);
    uint32_t *hist0 = reinterpret_cast<uint32_t *>(base + L.hist_off);
    if (L.split && need)
        return hipErrorInvalidValue;              // gating is a row-path feature
    if (L.split) {
        uint32_t *counts = reinterpret_cast<uint32_t *>(base + L.counts_off);
        uint64_t *regions = reinterpret_cast<uint64_t *>(base + L.regions_off);
        uint32_t *bounds = reinterpret_cast<uint32_t *>(base + L.bounds_off);
        // (ld < 4: every row is empty, the finishing kernel writes them
        // without the collected keys; the collect kernel's loads need ld >= 4)
        if (ld >= 4 && !trace_skip("topk_collect_kernel"))
            hipLaunchKernelGGL(topk_collect_kernel, dim3((unsigned)L.P, (unsigned)T), dim3(kSplitThreads), 0, stream,
                           scores, ld, n, max_n, k, counts, regions, bounds);
        trace_launch(stream, "topk_collect_kernel");
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
        // (the split path builds no first-digit histogram: a producer fills none)
        if (!trace_skip("topk_finish_kernel"))
            hipLaunchKernelGGL(topk_finish_kernel, dim3((unsigned)T), dim3(kFinishThreads), 0, stream, scores, ld, n,
                           k, idx, counts, regions, (int32_t)L.P, bounds);
        trace_launch(stream, "topk_finish_kernel");
    } else {
        if (!trace_skip("topk_row_kernel"))
            hipLaunchKernelGGL(topk_row_kernel, dim3((unsigned)T), dim3(kRowThreads), 0, stream, scores, ld, n, k, idx,
                           hist_ready ? hist0 : nullptr, reinterpret_cast<uint64_t *>(base + L.regions_off), need);
        trace_launch(stream, "topk_row_kernel");
    }
    return hipGetLastError();
}

}  // namespace ic
