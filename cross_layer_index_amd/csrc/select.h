// Radix-select building blocks shared by the top-k kernels and the sparse-MLA
// kernel that selects its own rows: workgroup barriers, DPP prefix sums, the
// one-wave digit search, key sources and the digit passes with the ordered
// compaction (see topk.hip for the method).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "radix_key.h"


namespace ic {
namespace {

constexpr int kBins0 = kHistBins0;      // first digit: bits 31..21

// Workgroup barrier. The full form is __syncthreads, whose release fence
// also waits for every global store and load in flight; the LDS form (this
// wave's LDS operations complete, then s_barrier) orders LDS traffic only and
// serves kernels that read back none of their own global stores. The memory
// clobber keeps the compiler from moving memory operations across it.
template <bool LdsOnly>
__device__ __forceinline__ void wg_barrier()
{
    if constexpr (LdsOnly)
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else
        __syncthreads();
}

// Inclusive prefix sum over the 64 lanes of a wave, in registers (DPP): row
// shifts by 1, 2, 4 and 8 scan each row of 16 lanes, then the last lane of row
// 0 is added to row 1 and that of row 2 to row 3, and the last lane of row 1
// to rows 2 and 3. Lanes without a source add 0.
__device__ __forceinline__ uint32_t wave_scan(uint32_t v)
{
    int x = (int)v;
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);   // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);   // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);   // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);   // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);   // row_bcast:15, rows 1 and 3
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);   // row_bcast:31, rows 2 and 3
    return (uint32_t)x;
}

// Block-wide inclusive scan of one uint32 per thread.
template <int NT, bool LB = false>
__device__ __forceinline__ uint32_t block_scan(uint32_t v, uint32_t *lds_waves, uint32_t *total)
{
    constexpr int NW = NT / 64;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    v = wave_scan(v);
    if (lane == 63)
        lds_waves[wave] = v;
    wg_barrier<LB>();
    if (wave == 0) {
        const uint32_t x = wave_scan(lane < NW ? lds_waves[lane] : 0u);
        if (lane < NW)
            lds_waves[lane] = x;
    }
    wg_barrier<LB>();
    const uint32_t before = wave ? lds_waves[wave - 1] : 0u;
    if (total)
        *total = lds_waves[NW - 1];
    wg_barrier<LB>();
    return v + before;
}

// Block-wide inclusive scans of R values per thread at once (R columns):
// incl[c] is the sum of column c over threads 0..tid, total[c] over all
// threads. `lds` holds R * NT / 64 words. Three barriers for all columns.
template <int NT, int R, bool LB = false>
__device__ __forceinline__ void block_scan_n(uint32_t (&v)[R], uint32_t *lds, uint32_t (&total)[R])
{
    constexpr int NW = NT / 64;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
#pragma unroll
    for (int c = 0; c < R; ++c) {
        v[c] = wave_scan(v[c]);
        if (lane == 63)
            lds[c * NW + wave] = v[c];
    }
    wg_barrier<LB>();
    if (wave == 0) {
#pragma unroll
        for (int c = 0; c < R; ++c) {
            const uint32_t x = wave_scan(lane < NW ? lds[c * NW + lane] : 0u);
            if (lane < NW)
                lds[c * NW + lane] = x;
        }
    }
    wg_barrier<LB>();
#pragma unroll
    for (int c = 0; c < R; ++c) {
        v[c] += wave ? lds[c * NW + wave - 1] : 0u;
        total[c] = lds[c * NW + NW - 1];
    }
    wg_barrier<LB>();
}

struct Shared {
    uint32_t hist[kBins0];
    uint32_t waves[16];
    uint32_t digit, above, count;
    uint32_t list_n;                 // entries of a short key list kept in hist
};

// Given a histogram of `nb` (1024 or 2048) bins in LDS, complete before the
// call, find the digit of the bin holding the need-th largest key; returns it
// with the count of keys in higher bins (and, in sh.count, the bin's own
// count). One wave scans: lane l owns nb/64
// consecutive bins, lane 0 the highest; a wave prefix sum of their totals
// names the lane whose range holds the need-th key, and a second one over
// that range, one bin per lane from the top, names the bin. One barrier
// publishes the result (a barrier before the next call separates these reads
// from its writes). Digit 0 and 0 when the counts never reach `need`.
template <int NT, bool LB = false>
__device__ __forceinline__ void find_digit(Shared &sh, int nb, uint32_t need, uint32_t &digit, uint32_t &above)
{
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        const int per = nb >> 6;                       // bins per lane: 32 or 16
        const int quads = per >> 2;
        const uint4 *h4 = reinterpret_cast<const uint4 *>(&sh.hist[nb - (lane + 1) * per]);
        uint32_t local = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (j < quads) {
                const uint4 c = h4[j];
                local += c.x + c.y + c.z + c.w;
            }
        const uint32_t incl = wave_scan(local);
        const uint64_t hit = __ballot(incl - local < need && incl >= need);
        if (hit == 0) {
            if (lane == 0) {
                sh.digit = 0;
                sh.above = 0;
                sh.count = 0;
            }
        } else {
            const int L = __builtin_ctzll(hit);
            const uint32_t run = __builtin_amdgcn_readlane(incl - local, L);
            const int b = nb - L * per - 1 - lane;     // lane i takes the range's i-th bin from the top
            const uint32_t x = lane < per ? sh.hist[b] : 0u;
            const uint32_t in2 = run + wave_scan(x);
            if (lane < per && in2 - x < need && in2 >= need) {
                sh.digit = (uint32_t)b;
                sh.above = in2 - x;
                sh.count = x;
            }
        }
    }
    wg_barrier<LB>();
    digit = sh.digit;
    above = sh.above;
}

// Key sources: a row of fp32 scores (position = index) or an LDS list of
// (key << 32 | position) entries in position order.
struct RowSrc {
    static constexpr bool kLds = false;
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

// Four consecutive scores from one unconditional 16-byte load, the address
// clamped into a row of capacity cap (a multiple of 4, at least 4; i a
// multiple of 4); positions at or past cap come back not ok. A branch around
// the load (RowSrc::get4) makes the compiler wait for each such load before
// the next is issued; these go out back to back.
__device__ __forceinline__ void row_get4u(const float *row, int64_t cap, int64_t i, uint32_t (&key)[4],
                                          int64_t (&pos)[4], bool (&ok)[4])
{
    const float4 v = *reinterpret_cast<const float4 *>(row + min(i, cap - 4));
    key[0] = ord_key(v.x), key[1] = ord_key(v.y), key[2] = ord_key(v.z), key[3] = ord_key(v.w);
#pragma unroll
    for (int e = 0; e < 4; ++e)
        pos[e] = i + e, ok[e] = i + e < cap;
}

struct ListSrc {
    static constexpr bool kLds = true;
    const uint64_t *list;                          // 16-byte aligned
    int64_t n;
    // i is a multiple of 4: two 16-byte reads
    __device__ void get4(int64_t i, uint32_t (&key)[4], int64_t (&pos)[4], bool (&ok)[4]) const
    {
        uint64_t v[4] = {0ull, 0ull, 0ull, 0ull};
        if (i + 3 < n) {
            const uint4 a = *reinterpret_cast<const uint4 *>(list + i);
            const uint4 b = *reinterpret_cast<const uint4 *>(list + i + 2);
            v[0] = a.x | ((uint64_t)a.y << 32), v[1] = a.z | ((uint64_t)a.w << 32);
            v[2] = b.x | ((uint64_t)b.y << 32), v[3] = b.z | ((uint64_t)b.w << 32);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (i + e < n)
                    v[e] = list[i + e];
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            ok[e] = i + e < n;
            key[e] = (uint32_t)(v[e] >> 32);
            pos[e] = (int64_t)(uint32_t)v[e];
        }
    }
};

// A contiguous (key << 32 | position) list in global memory, position order.
struct GListSrc {
    static constexpr bool kLds = false;
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

// The split phase's slices in global memory as one list: slice s (P of them,
// each in position order, the slices in chunk order) holds off[s + 1] - off[s]
// entries from reg + s * stride; off (P + 1 words) is in LDS.
struct SliceSrc {
    static constexpr bool kLds = false;
    const uint64_t *reg;
    int64_t stride;
    const uint32_t *off;
    int32_t P;
    int64_t n;
    __device__ void get4(int64_t i, uint32_t (&key)[4], int64_t (&pos)[4], bool (&ok)[4]) const
    {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t j = (uint32_t)(i + e);
            ok[e] = i + e < n;
            uint64_t v = 0ull;
            if (ok[e]) {
                int lo = 0, hi = P - 1;               // the slice s with off[s] <= j < off[s + 1]
                while (lo < hi) {
                    const int mid = (lo + hi + 1) >> 1;
                    if (off[mid] <= j)
                        lo = mid;
                    else
                        hi = mid - 1;
                }
                v = reg[(int64_t)lo * stride + (j - off[lo])];
            }
            key[e] = (uint32_t)(v >> 32);
            pos[e] = (int64_t)(uint32_t)v;
        }
    }
};

// Calls f(key, live) once for every entry of `src`, in no particular order,
// with every lane of the wave taking part in each call (f may use ballots).
// An LDS list is read interleaved (lane i takes entry i, i + NT, ...), which
// keeps the lanes of one read on distinct banks; other sources are read four
// consecutive entries per thread.
template <int NT, class Src, class F>
__device__ __forceinline__ void for_each_key(const Src &src, F f)
{
    if constexpr (Src::kLds) {
        for (int64_t i0 = 0; i0 < src.n; i0 += (int64_t)NT * 4) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t i = i0 + threadIdx.x + (int64_t)NT * e;
                const bool ok = i < src.n;
                const uint64_t v = ok ? src.list[i] : 0ull;
                f((uint32_t)(v >> 32), ok);
            }
        }
    } else {
        for (int64_t i = (int64_t)threadIdx.x * 4; i < src.n; i += (int64_t)NT * 4) {
            uint32_t key[4];
            int64_t pos[4];
            bool ok[4];
            src.get4(i, key, pos, ok);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                f(key[e], ok[e]);
        }
    }
}

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

// Digit passes `first`..2 over `src` (none when first is 3: then `prefix` is
// the threshold key itself), then the ordered compaction: emit(slot, position)
// for every selected key, slot in [0, k) in position order.
template <int NT, bool LB = false, class Src, class Emit>
__device__ void select_emit(const Src &src, Shared &sh, int first, uint32_t prefix, uint32_t pmask,
                            uint32_t need, int32_t k, Emit emit)
{
    const int tid = threadIdx.x;
    for (int pass = first; pass < 3; ++pass) {
        const int shf = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
        const int nb = pass == 2 ? 1024 : 2048;
        for (int i = tid; i < nb; i += NT)
            sh.hist[i] = 0;
        wg_barrier<LB>();
        // first digits crowd into a few bins (aggregated adds); later ones
        // spread out (plain adds)
        for_each_key<NT>(src, [&](uint32_t key, bool ok) {
            const bool live = ok && (key & pmask) == prefix;
            const uint32_t b = (key >> shf) & (nb - 1);
            if (pass == 0)
                hist_add_wave(sh.hist, b, live);
            else if (live)
                atomicAdd(&sh.hist[b], 1u);
        });
        wg_barrier<LB>();
        uint32_t digit, above;
        find_digit<NT, LB>(sh, nb, need, digit, above);
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
        const uint32_t incl = block_scan<NT, LB>(lg | (le << 16), sh.waves, &tot);
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
                    emit(slot, (int32_t)pos[e]);
            } else if (eq[e] && eb < need) {
                if (gb + eb < (uint32_t)k)
                    emit(gb + eb, (int32_t)pos[e]);
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

// The same, into out[0..k).
template <int NT, bool LB = false, class Src>
__device__ void finish_select(const Src &src, Shared &sh, int first, uint32_t prefix, uint32_t pmask,
                              uint32_t need, int32_t k, int32_t *__restrict__ out)
{
    select_emit<NT, LB>(src, sh, first, prefix, pmask, need, k, [out](uint32_t slot, int32_t p) { out[slot] = p; });
}


// One query's top k from the split path's collected keys, by one workgroup
// that holds them in registers. Slice s keeps count[s] keys (all at or above
// `bound`, position order) from entry s * stride. Rank f of the concatenation
// of the slices' first C entries (C = NT * E / P rounded down to a multiple of
// 4, at most stride) is entry f mod C of slice f / C; thread tid holds ranks
// NT * 4 * r + 4 * tid + (0..3) for r < E / 4: groups of four consecutive ranks,
// loaded as two 16-byte vectors with the lanes of a load contiguous, and
// ordered by (r, tid), so one block scan per round orders the output. load()
// issues the loads before the counts are known (clamped, unconditional);
// select() calls emit(slot, position) for every selected key (slot in
// [0, k)). A slice longer than C takes the digits over the slices in global
// memory (every key at or above the bound is there, in position order); fewer
// than k keys at the bound take them over the whole row. The caller handles
// rows of at most k keys.
template <int NT, int E>
struct SplitSel {
    static_assert(E % 4 == 0, "groups of four");
    static constexpr int R = E / 4;
    uint32_t key[E], pos[E];
    uint32_t C;
    const uint64_t *reg;
    int64_t stride;

    // (both members inline into the caller: called, they would keep the
    // arrays in memory behind `this`)
    __device__ __forceinline__ void load(const uint64_t *reg_t, int64_t stride_, int32_t P)
    {
        reg = reg_t;
        stride = stride_;
        C = min((uint32_t)(NT * E) / (uint32_t)P, (uint32_t)stride) & ~3u;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const uint32_t f = (uint32_t)(NT * 4 * r) + 4u * threadIdx.x;
            const uint32_t sl = min(f / C, (uint32_t)P - 1u), j = f - (f / C) * C;
            const uint4 *src = reinterpret_cast<const uint4 *>(reg_t + (int64_t)sl * stride + j);
            const uint4 a = src[0], b = src[1];
            key[4 * r + 0] = a.y, pos[4 * r + 0] = a.x;
            key[4 * r + 1] = a.w, pos[4 * r + 1] = a.z;
            key[4 * r + 2] = b.y, pos[4 * r + 2] = b.x;
            key[4 * r + 3] = b.w, pos[4 * r + 3] = b.z;
        }
    }

    // cnt: P + 1 + R * NT / 64 + P + 1 words of LDS (the slice counts, an
    // overflow flag, the scan's wave totals, the slice offsets)
    // Only slots in [s0, s1) are emitted (a group whose slots lie outside
    // skips the per-key work).
    template <class Emit>
    __device__ __forceinline__ void select(const RowSrc &row, int32_t k, uint32_t c0, uint32_t bound, int32_t P, Shared &sh,
                           uint32_t *cnt, uint32_t s0, uint32_t s1, Emit emit)
    {
        constexpr bool LB = true;
        const int tid = threadIdx.x;
        if (tid == 0)
            cnt[P] = 0;
        wg_barrier<LB>();
        if (tid < P) {
            cnt[tid] = c0;
            if (c0 > C)
                cnt[P] = 1;
        }
        uint32_t total;
        const uint32_t incl = block_scan<NT, LB>(c0, sh.waves, &total);     // its barriers publish cnt
        auto in_split = [&](uint32_t slot, int32_t p) {
            if (slot >= s0 && slot < s1)
                emit(slot, p);
        };
        if (total < (uint32_t)k) {
            select_emit<NT, LB>(row, sh, 0, 0u, 0u, (uint32_t)k, k, in_split);
            return;
        }
        uint32_t valid = 0;
        if (__builtin_expect(cnt[P] != 0, 0)) {
            uint32_t *off = cnt + P + 1 + R * NT / 64;
            if (tid < P)
                off[tid + 1] = incl;
            if (tid == 0)
                off[0] = 0u;
            wg_barrier<LB>();
            if (total > (uint32_t)(NT * E)) {
                // more keys than the registers hold: digit passes over the
                // slices in global memory
                select_emit<NT, LB>(SliceSrc{reg, stride, off, P, (int64_t)total}, sh, 0, 0u, 0u, (uint32_t)k, k,
                                    in_split);
                return;
            }
            // A slice holds more than its share, but every key fits the
            // registers: reload them by their rank in the concatenated slices
            // (position order; rank f in register 4r + e of thread
            // (f / 4) % NT, as below) and go on in registers. A group's first
            // rank finds its slice by a binary search over the offsets, the
            // next three step forward from it; ranks past the last key read
            // the last key again, so every load is unconditional.
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const uint32_t f0 = min((uint32_t)(NT * 4 * r) + 4u * tid, total - 1u);
                int lo = 0, hi = P - 1;
                while (lo < hi) {
                    const int mid = (lo + hi + 1) >> 1;
                    if (off[mid] <= f0)
                        lo = mid;
                    else
                        hi = mid - 1;
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t f = (uint32_t)(NT * 4 * r) + 4u * tid + (uint32_t)e;
                    const uint32_t fc = min(f, total - 1u);
                    while (lo + 1 < P && off[lo + 1] <= fc)
                        ++lo;
                    const uint64_t v = reg[(int64_t)lo * stride + (fc - off[lo])];
                    key[4 * r + e] = (uint32_t)(v >> 32);
                    pos[4 * r + e] = (uint32_t)v;
                    if (f < total)
                        valid |= 1u << (4 * r + e);
                }
            }
        } else {
            // which entries hold keys (a group of four lies in one slice)
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const uint32_t f = (uint32_t)(NT * 4 * r) + 4u * tid;
                const uint32_t sl = f / C, j = f - sl * C;
                const uint32_t have = sl < (uint32_t)P ? cnt[sl] : 0u;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (j + e < have)
                        valid |= 1u << (4 * r + e);
            }
        }
        // the keys' top 22 bits relative to the bound's, the last bin taking
        // everything from 2047 up (the same pass as the finishing kernel's)
        const uint32_t b22 = bound >> 10;
        for (int i = tid; i < kBins0; i += NT)
            sh.hist[i] = 0;
        if (tid == 0)
            sh.list_n = 0;
        wg_barrier<LB>();
#pragma unroll
        for (int e = 0; e < E; ++e)
            if (valid >> e & 1u)
                atomicAdd(&sh.hist[min((key[e] >> 10) - b22, (uint32_t)kBins0 - 1)], 1u);
        wg_barrier<LB>();
        uint32_t rel, above;
        find_digit<NT, LB>(sh, kBins0, (uint32_t)k, rel, above);
        const uint32_t in_bin = __builtin_amdgcn_readfirstlane(sh.count);
        const uint32_t pre = (b22 + rel) << 10;
        uint32_t thr, need;
        if (rel < (uint32_t)kBins0 - 1 && in_bin == (uint32_t)k - above && pre != 0u) {
            thr = pre - 1u;                           // every key of the bin is kept
            need = 0;
        } else if (rel < (uint32_t)kBins0 - 1 && in_bin <= 64u) {
            // A bin of at most a wave's width: its keys go to a list (the
            // histogram's words, read by no one any more) and wave 0 ranks
            // them. The threshold is the key with fewer than k - above
            // greater keys in the bin and at least k - above greater or
            // equal ones; of the keys equal to it, the first k - above -
            // (greater ones) in position order are kept.
            const uint32_t want = (uint32_t)k - above;  // in [1, in_bin]
#pragma unroll
            for (int e = 0; e < E; ++e)
                if ((valid >> e & 1u) && (key[e] >> 10) - b22 == rel)
                    sh.hist[atomicAdd(&sh.list_n, 1u)] = key[e];
            wg_barrier<LB>();
            if (tid < 64) {
                const uint32_t kv = (uint32_t)tid < in_bin ? sh.hist[tid] : 0u;
                uint32_t gt = 0, eq = 0;
                for (uint32_t j = 0; j < in_bin; ++j) {
                    const uint32_t o = (uint32_t)__builtin_amdgcn_readlane((int)kv, (int)j);
                    gt += o > kv;
                    eq += o == kv;
                }
                if ((uint32_t)tid < in_bin && gt < want && gt + eq >= want) {
                    sh.digit = kv;                    // every lane holding the key writes the same
                    sh.above = want - gt;
                }
            }
            wg_barrier<LB>();
            thr = sh.digit;
            need = sh.above;
        } else {
            uint32_t prefix = 0, pmask = 0;
            int first = 0;
            need = (uint32_t)k;
            if (rel < (uint32_t)kBins0 - 1) {
                prefix = pre;
                pmask = 0xFFFFFC00u;
                first = 2;
                need = (uint32_t)k - above;
            }
            for (int pass = first; pass < 3; ++pass) {
                const int shf = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
                const int nb = pass == 2 ? 1024 : 2048;
                for (int i = tid; i < nb; i += NT)
                    sh.hist[i] = 0;
                wg_barrier<LB>();
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const bool live = (valid >> e & 1u) && (key[e] & pmask) == prefix;
                    if (pass == 0)
                        hist_add_wave(sh.hist, key[e] >> 21, live);
                    else if (live)
                        atomicAdd(&sh.hist[(key[e] >> shf) & (nb - 1)], 1u);
                }
                wg_barrier<LB>();
                uint32_t digit, ab;
                find_digit<NT, LB>(sh, nb, need, digit, ab);
                prefix |= digit << shf;
                pmask |= (uint32_t)(nb - 1) << shf;
                need -= ab;
            }
            thr = prefix;
        }
        // ordered compaction: packed (above, equal) counts over each group of
        // the thread, scanned for all rounds at once
        uint32_t cv[R], tot[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            uint32_t lg = 0, le = 0;
#pragma unroll
            for (int e = 4 * r; e < 4 * r + 4; ++e)
                if (valid >> e & 1u) {
                    lg += key[e] > thr;
                    le += key[e] == thr;
                }
            cv[r] = lg | (le << 16);
        }
        uint32_t cnt_r[R];
#pragma unroll
        for (int r = 0; r < R; ++r)
            cnt_r[r] = cv[r];
        block_scan_n<NT, R, LB>(cv, cnt + P + 1, tot);
        uint32_t run_gt = 0, run_eq = 0;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const uint32_t excl = cv[r] - cnt_r[r];
            uint32_t gb = run_gt + (excl & 0xFFFFu), eb = run_eq + (excl >> 16);
            // the group's slots: [lo, lo + above + kept equal)
            const uint32_t lo = gb + min(eb, need);
            const uint32_t hi = gb + (cnt_r[r] & 0xFFFFu) + min(eb + (cnt_r[r] >> 16), need);
            if (lo < s1 && hi > s0) {
#pragma unroll
                for (int e = 4 * r; e < 4 * r + 4; ++e) {
                    const bool v = valid >> e & 1u;
                    const bool gt = v && key[e] > thr, eq = v && key[e] == thr;
                    const uint32_t slot = gt ? gb + min(eb, need) : gb + eb;
                    if ((gt || (eq && eb < need)) && slot >= s0 && slot < s1 && slot < (uint32_t)k)
                        emit(slot, (int32_t)pos[e]);
                    gb += gt;
                    eb += eq;
                }
            }
            run_gt += tot[r] & 0xFFFFu;
            run_eq += tot[r] >> 16;
        }
    }
};

}  // namespace
}  // namespace ic
