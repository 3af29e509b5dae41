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
// The first digit's histogram is built while the scores are produced (the
// indexer kernel can add into it) or by topk_hist_kernel. Only keys whose
// first digit is >= the threshold digit ("survivors", about k plus one bin)
// take part in the later digits:
//   * split path (few queries, long rows): P workgroups per query each copy
//     their chunk's survivors, in position order, into their own slice of the
//     workspace and add the second digit's histogram of the threshold bin
//     (topk_survivors_kernel); one workgroup per query then reads the second
//     digit, gathers in order into LDS only the survivors at or above the
//     two-digit bound, and finishes the selection there (topk_finish_kernel).
//     The kernel boundary orders the two phases.
//   * row path (many queries): one workgroup per query streams its row once
//     more to collect survivors into LDS and finishes there. When they exceed
//     the LDS list (the threshold fell into a dense first-digit bin), it
//     histograms the second digit over the survivors kept in global memory and
//     keeps only those at or above the second-digit threshold.
// Only ties spanning more than the list at 21 bits of the key fall back to
// digit passes over the full row.
// The first-digit histogram is kept in kHistCopies copies per query (adders
// pick a copy by workgroup index, which spreads atomic traffic); the workspace
// holds them zeroed on entry and the finishing workgroup zeroes them again.
#include "kernels.h"
#include "radix_key.h"

namespace ic {
namespace {

constexpr int kBins0 = kHistBins0;      // first digit: bits 31..21
constexpr int kSplitThreads = 256;
constexpr int kSplitRuns = 2;                      // groups of 4 consecutive scores per survivors thread
constexpr int kSplitChunk = kSplitThreads * 4 * kSplitRuns;   // scores per split workgroup
constexpr int kRowThreads = 1024;
constexpr int kFinishThreads = 1024;
constexpr int kListCap = 18432;         // survivors held in LDS (split path)
constexpr int kRowListCap = 8192;       // survivors held in LDS (row path: two workgroups per CU)
constexpr int kRowRuns = 2;             // consecutive groups of 4 scores per thread per collect round
constexpr int kMaxSplit = 1024;         // workgroups per query on the split path
constexpr int kGatherPer = 20;          // survivors per finishing thread and gather round
constexpr int kRowSurvCap = 32768;      // survivors kept in global memory per query (row path)

// Block-wide inclusive scan of one uint32 per thread.
template <int NT>
__device__ __forceinline__ uint32_t block_scan(uint32_t v, uint32_t *lds_waves, uint32_t *total)
{
    constexpr int NW = NT / 64;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t o = __shfl_up(v, off);
        if (lane >= off)
            v += o;
    }
    if (lane == 63)
        lds_waves[wave] = v;
    __syncthreads();
    if (wave == 0) {
        uint32_t x = lane < NW ? lds_waves[lane] : 0u;
#pragma unroll
        for (int off = 1; off < NW; off <<= 1) {
            const uint32_t o = __shfl_up(x, off);
            if (lane >= off)
                x += o;
        }
        if (lane < NW)
            lds_waves[lane] = x;
    }
    __syncthreads();
    const uint32_t before = wave ? lds_waves[wave - 1] : 0u;
    if (total)
        *total = lds_waves[NW - 1];
    __syncthreads();
    return v + before;
}

struct Shared {
    uint32_t hist[kBins0];
    uint32_t waves[16];
    uint32_t digit, above;
};

// Given a histogram of `nb` bins (in LDS), find the digit of the bin holding
// the need-th largest key; returns it with the count of keys in higher bins.
template <int NT>
__device__ __forceinline__ void find_digit(Shared &sh, int nb, uint32_t need, uint32_t &digit, uint32_t &above)
{
    constexpr int PER = kBins0 / NT;             // bins per thread (descending)
    uint32_t c[PER];
    uint32_t local = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int b = nb - 1 - (PER * (int)threadIdx.x + i);
        c[i] = b >= 0 ? sh.hist[b] : 0u;
        local += c[i];
    }
    const uint32_t incl = block_scan<NT>(local, sh.waves, nullptr);
    uint32_t run = incl - local;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int b = nb - 1 - (PER * (int)threadIdx.x + i);
        if (b >= 0 && run < need && run + c[i] >= need) {
            sh.digit = (uint32_t)b;
            sh.above = run;
        }
        run += c[i];
    }
    __syncthreads();
    digit = sh.digit;
    above = sh.above;
    __syncthreads();
}

// Key sources: a row of fp32 scores (position = index) or an LDS list of
// (key << 32 | position) entries in position order.
struct RowSrc {
    const float *row;
    int64_t n;
    __device__ void get4(int64_t i, uint32_t (&key)[4], int64_t (&pos)[4], bool (&ok)[4]) const
    {
        if (i + 3 < n) {
            const float4 v = *reinterpret_cast<const float4 *>(row + i);
            key[0] = ord_key(v.x), key[1] = ord_key(v.y), key[2] = ord_key(v.z), key[3] = ord_key(v.w);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                pos[e] = i + e, ok[e] = true;
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                ok[e] = i + e < n;
                key[e] = ok[e] ? ord_key(row[i + e]) : 0u;
                pos[e] = i + e;
            }
        }
    }
};

struct ListSrc {
    const uint64_t *list;
    int64_t n;
    __device__ void get4(int64_t i, uint32_t (&key)[4], int64_t (&pos)[4], bool (&ok)[4]) const
    {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            ok[e] = i + e < n;
            const uint64_t v = ok[e] ? list[i + e] : 0ull;
            key[e] = (uint32_t)(v >> 32);
            pos[e] = (int64_t)(uint32_t)v;
        }
    }
};

// A contiguous (key << 32 | position) list in global memory, position order.
struct GListSrc {
    const uint64_t *list;
    int64_t n;
    __device__ void get4(int64_t i, uint32_t (&key)[4], int64_t (&pos)[4], bool (&ok)[4]) const
    {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            ok[e] = i + e < n;
            const uint64_t v = ok[e] ? list[i + e] : 0ull;
            key[e] = (uint32_t)(v >> 32);
            pos[e] = (int64_t)(uint32_t)v;
        }
    }
};

// Ordered compaction of the entries with key >= bound into an LDS list (the
// first lcap) and, if given, a global list (the first gcap). Returns the count.
// A thread takes R groups of 4 consecutive entries per round (all their loads
// in flight before the round's one scan).
template <int NT, int R = 1, class Src>
__device__ uint32_t collect(const Src &src, uint32_t bound, Shared &sh, uint64_t *lds, uint32_t lcap,
                            uint64_t *glist, uint32_t gcap)
{
    uint32_t total = 0;
    for (int64_t c0 = 0; c0 < src.n; c0 += (int64_t)NT * 4 * R) {
        uint32_t key[R][4];
        int64_t pos[R][4];
        bool ok[R][4];
        const int64_t i0 = c0 + (int64_t)threadIdx.x * 4 * R;
#pragma unroll
        for (int r = 0; r < R; ++r)
            src.get4(i0 + 4 * r, key[r], pos[r], ok[r]);
        uint32_t ls = 0;
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                ok[r][e] = ok[r][e] && key[r][e] >= bound;
                ls += ok[r][e];
            }
        uint32_t tot;
        uint32_t o = total + block_scan<NT>(ls, sh.waves, &tot) - ls;
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (ok[r][e]) {
                    const uint64_t v = ((uint64_t)key[r][e] << 32) | (uint32_t)pos[r][e];
                    if (o < lcap)
                        lds[o] = v;
                    if (glist && o < gcap)
                        glist[o] = v;
                    ++o;
                }
            }
        total += tot;
    }
    __syncthreads();
    return total;
}

// Digit passes `first`..2 over `src`, then the ordered compaction into out[0..k).
template <int NT, class Src>
__device__ void finish_select(const Src &src, Shared &sh, int first, uint32_t prefix, uint32_t pmask,
                              uint32_t need, int32_t k, int32_t *__restrict__ out)
{
    const int tid = threadIdx.x;
    for (int pass = first; pass < 3; ++pass) {
        const int shf = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
        const int nb = pass == 2 ? 1024 : 2048;
        for (int i = tid; i < nb; i += NT)
            sh.hist[i] = 0;
        __syncthreads();
        for (int64_t i = (int64_t)tid * 4; i < src.n; i += (int64_t)NT * 4) {
            uint32_t key[4];
            int64_t pos[4];
            bool ok[4];
            src.get4(i, key, pos, ok);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (ok[e] && (key[e] & pmask) == prefix)
                    atomicAdd(&sh.hist[(key[e] >> shf) & (nb - 1)], 1u);
        }
        __syncthreads();
        uint32_t digit, above;
        find_digit<NT>(sh, nb, need, digit, above);
        prefix |= digit << shf;
        pmask |= (uint32_t)(nb - 1) << shf;
        need -= above;
    }
    const uint32_t thr = prefix;
    uint32_t run_gt = 0, run_eq = 0;
    for (int64_t c0 = 0; c0 < src.n; c0 += (int64_t)NT * 4) {
        uint32_t key[4];
        int64_t pos[4];
        bool ok[4];
        src.get4(c0 + (int64_t)tid * 4, key, pos, ok);
        uint32_t gt[4], eq[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            gt[e] = ok[e] && key[e] > thr;
            eq[e] = ok[e] && key[e] == thr;
        }
        const uint32_t lg = gt[0] + gt[1] + gt[2] + gt[3];
        const uint32_t le = eq[0] + eq[1] + eq[2] + eq[3];
        uint32_t tot;
        const uint32_t incl = block_scan<NT>(lg | (le << 16), sh.waves, &tot);
        const uint32_t excl = incl - (lg | (le << 16));
        uint32_t gb = run_gt + (excl & 0xFFFFu);
        uint32_t eb = run_eq + (excl >> 16);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            // slots are < k by construction; the check keeps any inconsistent
            // input (NaN scores) from writing outside the row
            if (gt[e]) {
                const uint32_t slot = gb + min(eb, need);
                if (slot < (uint32_t)k)
                    out[slot] = (int32_t)pos[e];
            } else if (eq[e] && eb < need) {
                if (gb + eb < (uint32_t)k)
                    out[gb + eb] = (int32_t)pos[e];
            }
            gb += gt[e];
            eb += eq[e];
        }
        run_gt += tot & 0xFFFFu;
        run_eq += tot >> 16;
        if (run_gt + min(run_eq, need) >= (uint32_t)k)
            break;
    }
}

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
    for (int64_t i = (int64_t)threadIdx.x * 4; i < src.n; i += (int64_t)NT * 4) {
        uint32_t key[4];
        int64_t pos[4];
        bool ok[4];
        src.get4(i, key, pos, ok);
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (ok[e] && (key[e] & 0xFFE00000u) == p0)
                atomicAdd(&sh.hist[(key[e] >> 10) & 2047], 1u);
    }
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

// ---- first-digit histogram of a score row (standalone top-k) -------------
// grid: (chunks, T); block: 256.
__global__ __launch_bounds__(256) void topk_hist_kernel(const float *__restrict__ scores, int64_t ld,
                                                        const int32_t *__restrict__ n, int64_t chunk,
                                                        uint32_t *__restrict__ hist0)
{
    __shared__ uint32_t h[kBins0];
    const int t = blockIdx.y;
    const int64_t nt = n[t];
    const int64_t s0 = (int64_t)blockIdx.x * chunk;
    if (s0 >= nt)
        return;
    const int64_t s1 = min(nt, s0 + chunk);
    for (int i = threadIdx.x; i < kBins0; i += 256)
        h[i] = 0;
    __syncthreads();
    const float *row = scores + (int64_t)t * ld;
    for (int64_t i = s0 + (int64_t)threadIdx.x * 4; i < s1; i += 256 * 4) {
        if (i + 3 < s1) {
            const float4 v = *reinterpret_cast<const float4 *>(row + i);
            atomicAdd(&h[ord_key(v.x) >> 21], 1u);
            atomicAdd(&h[ord_key(v.y) >> 21], 1u);
            atomicAdd(&h[ord_key(v.z) >> 21], 1u);
            atomicAdd(&h[ord_key(v.w) >> 21], 1u);
        } else {
            for (int64_t e = i; e < s1; ++e)
                atomicAdd(&h[ord_key(row[e]) >> 21], 1u);
        }
    }
    __syncthreads();
    uint32_t *g = hist0 + ((int64_t)t * kHistCopies + (blockIdx.x % kHistCopies)) * kBins0;
    for (int i = threadIdx.x; i < kBins0; i += 256)
        if (h[i])
            atomicAdd(&g[i], h[i]);
}

// ---- split path -------------------------------------------------------------
// First digit from the query's histogram copies, read from the top bin down
// NT bins at a time (the threshold sits in the highest bins, so one round
// usually suffices). Falls back to digit 0 (everything survives) if the
// counts never reach `need`.
template <int NT>
__device__ void find_digit0_topdown(Shared &sh, const uint32_t *h, uint32_t need, uint32_t &digit, uint32_t &above)
{
    uint32_t run = 0;
    digit = 0;
    above = 0;
    for (int top = kBins0; top > 0; top -= NT) {
        const int b = top - 1 - (int)threadIdx.x;          // thread 0 takes the highest bin
        uint32_t c = 0;
        if (b >= 0) {
#pragma unroll
            for (int cp = 0; cp < kHistCopies; ++cp)
                c += h[cp * kBins0 + b];
        }
        uint32_t tot;
        const uint32_t incl = block_scan<NT>(c, sh.waves, &tot);
        if (run + tot >= need) {                           // uniform: the bin is in this round
            if (b >= 0 && run + incl - c < need && run + incl >= need) {
                sh.digit = (uint32_t)b;
                sh.above = run + incl - c;
            }
            __syncthreads();
            digit = sh.digit;
            above = sh.above;
            __syncthreads();
            return;
        }
        run += tot;
    }
}

// Phase 1. grid: (P, T); block: 256; kSplitChunk scores per workgroup. Copies
// the chunk's survivors (first digit >= the threshold digit), in position
// order, into the workgroup's slice of `regions`, and their count to counts;
// adds the second-digit histogram of its threshold-bin keys to hist1.
__global__ __launch_bounds__(kSplitThreads) void topk_survivors_kernel(
    const float *__restrict__ scores, int64_t ld, const int32_t *__restrict__ n, int32_t k,
    const uint32_t *__restrict__ hist0, uint32_t *__restrict__ hist1, uint32_t *__restrict__ counts,
    uint64_t *__restrict__ regions, uint32_t *__restrict__ digit0)
{
    __shared__ Shared sh;
    const int t = blockIdx.y;
    const int w = blockIdx.x;
    const int P = gridDim.x;
    const int tid = threadIdx.x;
    const int64_t nt = n[t];
    if (nt <= k)
        return;                                   // the finish kernel keeps everything
    const float *row = scores + (int64_t)t * ld;
    // this chunk's scores, issued before the histogram is read
    const int64_t s = (int64_t)w * kSplitChunk + (int64_t)tid * 4 * kSplitRuns;
    uint32_t key[kSplitRuns][4];
    int64_t pos[kSplitRuns][4];
    bool ok[kSplitRuns][4];
#pragma unroll
    for (int r = 0; r < kSplitRuns; ++r)
        RowSrc{row, nt}.get4(s + 4 * r, key[r], pos[r], ok[r]);
    for (int i = tid; i < kBins0; i += kSplitThreads)
        sh.hist[i] = 0;

    uint32_t d0, above0;
    find_digit0_topdown<kSplitThreads>(sh, hist0 + (int64_t)t * kHistCopies * kBins0, (uint32_t)k, d0, above0);
    uint32_t ls = 0;
#pragma unroll
    for (int r = 0; r < kSplitRuns; ++r)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const bool sv = ok[r][e] && (key[r][e] >> 21) >= d0;
            ls += sv;
            if (ok[r][e] && (key[r][e] >> 21) == d0)
                atomicAdd(&sh.hist[(key[r][e] >> 10) & (kBins0 - 1)], 1u);
            ok[r][e] = sv;
        }
    uint32_t tot;
    uint32_t o = block_scan<kSplitThreads>(ls, sh.waves, &tot) - ls;   // its barriers also close the histogram
    uint64_t *reg = regions + ((int64_t)t * P + w) * kSplitChunk;
#pragma unroll
    for (int r = 0; r < kSplitRuns; ++r)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (ok[r][e])
                reg[o++] = ((uint64_t)key[r][e] << 32) | (uint32_t)pos[r][e];
    uint32_t *h1 = hist1 + (int64_t)t * kBins0;
    for (int i = tid; i < kBins0; i += kSplitThreads)
        if (sh.hist[i])
            atomicAdd(&h1[i], sh.hist[i]);
    if (tid == 0) {
        counts[(int64_t)t * P + w] = tot;
        if (w == 0) {                             // every workgroup found the same digit
            digit0[2 * t] = d0;
            digit0[2 * t + 1] = above0;
        }
    }
}

// Phase 2. grid: T; block: kFinishThreads. The second digit comes from hist1;
// the survivors of all P slices at or above the two-digit bound (about k of
// them) are gathered in slice order (= position order) into LDS, and the last
// digit finishes the selection. Zeroes the query's histograms.
__global__ __launch_bounds__(kFinishThreads) void topk_finish_kernel(
    const float *__restrict__ scores, int64_t ld, const int32_t *__restrict__ n, int32_t k,
    int32_t *__restrict__ idx, uint32_t *__restrict__ hist0, uint32_t *__restrict__ hist1,
    const uint32_t *__restrict__ counts, const uint64_t *__restrict__ regions, int32_t P,
    const uint32_t *__restrict__ digit0)
{
    constexpr int NT = kFinishThreads;
    __shared__ Shared sh;
    __shared__ uint64_t list[kListCap];
    __shared__ uint32_t offs[kMaxSplit + 1];
    __shared__ uint32_t wave_cnt[kFinishThreads / 64];
    const int t = blockIdx.x;
    const int tid = threadIdx.x;
    const int64_t nt = n[t];
    int32_t *out = idx + (int64_t)t * k;
    uint32_t *h0 = hist0 + (int64_t)t * kHistCopies * kBins0;
    uint32_t *h1 = hist1 + (int64_t)t * kBins0;
    if (nt <= k) {
        zero_hist0<NT>(h0);                       // no reader of this query's copies remains
        write_all<NT>(out, nt, k);                // hist1 was not touched for this query
        return;
    }
    // the second-digit histogram, the slice counts and the first digit are
    // all loaded at once (one round trip), then the first-digit copies cleared
    static_assert(kBins0 % NT == 0 && kMaxSplit <= NT, "one pass over bins and slices");
    uint32_t hv[kBins0 / NT];
#pragma unroll
    for (int i = 0; i < kBins0 / NT; ++i)
        hv[i] = h1[tid + i * NT];
    const uint32_t c0 = tid < P ? counts[(int64_t)t * P + tid] : 0u;
    const uint32_t d0 = digit0[2 * t], above0 = digit0[2 * t + 1];
    zero_hist0<NT>(h0);                           // no reader of this query's copies remains
    const uint32_t need0 = (uint32_t)k - above0;
    // second digit over the first-digit bin
#pragma unroll
    for (int i = 0; i < kBins0 / NT; ++i) {
        sh.hist[tid + i * NT] = hv[i];
        h1[tid + i * NT] = 0;
    }
    __syncthreads();
    uint32_t d1, above1;
    find_digit<NT>(sh, kBins0, need0, d1, above1);
    const uint32_t bound = (d0 << 21) | (d1 << 10);
    // slice offsets (P <= NT: one scan)
    uint32_t total;
    const uint32_t excl = block_scan<NT>(c0, sh.waves, &total) - c0;
    if (tid < P)
        offs[tid] = excl;
    if (tid == 0)
        offs[P] = total;
    __syncthreads();
    // Gather, in slice order (= position order), only the survivors at or
    // above the two-digit bound: about k of them, plus the ties of the bound's
    // bin. Per round each wave takes a contiguous segment, its lanes
    // interleaved so that one load covers 512 contiguous bytes of a slice; a
    // lane finds the slice of its first entry by binary search, then walks
    // forward with the next slice's offset in a register. All loads of a round
    // are in flight before the compaction: ballot prefix counts inside the
    // wave, then one exchange of the 16 wave counts.
    constexpr int NW = NT / 64;
    const int wv = tid >> 6, lane = tid & 63;
    const uint64_t *reg_t = regions + (int64_t)t * P * kSplitChunk;
    uint32_t cnt = 0;
    for (uint32_t r0 = 0; r0 < total; r0 += (uint32_t)NT * kGatherPer) {
        const uint32_t part = min(total - r0, (uint32_t)NT * kGatherPer);
        const uint32_t seg = (part + NW - 1) / NW;            // <= 64 * kGatherPer
        const uint32_t s0 = r0 + (uint32_t)wv * seg;
        const uint32_t s1 = min(s0 + seg, r0 + part);
        const uint32_t x0 = s0 + (uint32_t)lane;
        int lo = 0;
        if (x0 < s1) {
            int hi = P;
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if (offs[mid] <= x0)
                    lo = mid;
                else
                    hi = mid;
            }
        }
        uint32_t next = offs[lo + 1];
        uint64_t v[kGatherPer];
#pragma unroll
        for (int e = 0; e < kGatherPer; ++e) {
            const uint32_t x = x0 + 64u * e;
            v[e] = 0;
            if (x < s1) {
                while (next <= x) {               // offs[P] = total > x ends the walk
                    ++lo;
                    next = offs[lo + 1];
                }
                v[e] = reg_t[(int64_t)lo * kSplitChunk + (x - offs[lo])];
            }
        }
        uint32_t loc[kGatherPer];
        bool keep[kGatherPer];
        uint32_t wcount = 0;
#pragma unroll
        for (int e = 0; e < kGatherPer; ++e) {
            keep[e] = x0 + 64u * e < s1 && (uint32_t)(v[e] >> 32) >= bound;
            const uint64_t m = __ballot(keep[e]);
            loc[e] = wcount + (uint32_t)__popcll(m & __lanemask_lt());
            wcount += (uint32_t)__popcll(m);
        }
        if (lane == 0)
            wave_cnt[wv] = wcount;
        __syncthreads();
        uint32_t woff = 0, tot = 0;
#pragma unroll
        for (int j = 0; j < NW; ++j) {
            const uint32_t c = wave_cnt[j];
            woff += j < wv ? c : 0u;
            tot += c;
        }
#pragma unroll
        for (int e = 0; e < kGatherPer; ++e) {
            const uint32_t o = cnt + woff + loc[e];
            if (keep[e] && o < (uint32_t)kListCap)
                list[o] = v[e];
        }
        cnt += tot;
        __syncthreads();                          // wave_cnt is rewritten next round
    }
    if (cnt <= (uint32_t)kListCap)
        finish_select<NT>(ListSrc{list, cnt}, sh, 2, bound, 0xFFFFFC00u, need0 - above1, k, out);
    else                                          // more than kListCap keys share the top two digits
        finish_select<NT>(RowSrc{scores + (int64_t)t * ld, nt}, sh, 2, bound, 0xFFFFFC00u, need0 - above1, k, out);
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
                                                               uint64_t *__restrict__ surv)
{
    __shared__ Shared sh;
    __shared__ uint64_t list[kRowListCap];
    const int t = blockIdx.x;
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

struct TopkLayout {
    bool split;
    int64_t P;
    size_t hist_off, hist1_off, counts_off, digit_off, regions_off, total;
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
    // counters that start and end at zero: first-digit histogram copies and
    // the second-digit histogram of the split path
    L.hist_off = 0;
    L.hist1_off = up256((size_t)T * kHistCopies * kBins0 * 4);
    L.counts_off = L.hist1_off + up256((size_t)T * kBins0 * 4);
    if (L.split) {
        L.digit_off = L.counts_off + up256((size_t)T * L.P * 4);
        L.regions_off = L.digit_off + up256((size_t)T * 8);
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

hipError_t launch_topk(const float *scores, int64_t ld, const int32_t *n, int32_t T, int64_t max_n, int32_t k,
                       int32_t *idx, void *ws, bool hist_ready, hipStream_t stream)
{
    if (T == 0)
        return hipSuccess;
    const TopkLayout L = topk_layout(T, max_n);
    char *base = static_cast<char *>(ws);
    uint32_t *hist0 = reinterpret_cast<uint32_t *>(base + L.hist_off);
    if (L.split) {
        uint32_t *counts = reinterpret_cast<uint32_t *>(base + L.counts_off);
        uint64_t *regions = reinterpret_cast<uint64_t *>(base + L.regions_off);
        if (!hist_ready && max_n > 0) {
            const int64_t chunk = 8192;
            hipLaunchKernelGGL(topk_hist_kernel, dim3((unsigned)((max_n + chunk - 1) / chunk), (unsigned)T),
                               dim3(256), 0, stream, scores, ld, n, chunk, hist0);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess)
                return e;
        }
        uint32_t *digit0 = reinterpret_cast<uint32_t *>(base + L.digit_off);
        uint32_t *hist1 = reinterpret_cast<uint32_t *>(base + L.hist1_off);
        hipLaunchKernelGGL(topk_survivors_kernel, dim3((unsigned)L.P, (unsigned)T), dim3(kSplitThreads), 0,
                           stream, scores, ld, n, k, hist0, hist1, counts, regions, digit0);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
        hipLaunchKernelGGL(topk_finish_kernel, dim3((unsigned)T), dim3(kFinishThreads), 0, stream, scores, ld, n,
                           k, idx, hist0, hist1, counts, regions, (int32_t)L.P, digit0);
    } else {
        hipLaunchKernelGGL(topk_row_kernel, dim3((unsigned)T), dim3(kRowThreads), 0, stream, scores, ld, n, k, idx,
                           hist_ready ? hist0 : nullptr, reinterpret_cast<uint64_t *>(base + L.regions_off));
    }
    return hipGetLastError();
}

}  // namespace ic
