// Sparse MLA with a per-head softmax sink over selected latent rows.
//
// For query t, head h and the selected positions j (explainer "Hy4 IndexCache
// cross-layer index reuse", Jargon "DSA"; GitHub issue "rtx6kpro #90":
// 576-wide latent rows = 512 latent + 64 RoPE, learnable per-head sink that
// biases the softmax denominator):
//   s_j = scale * <q[t,h,:], kv[row_j,:]>,  o = sum_j e^{s_j} v_j / (e^{sink_h} + sum_j e^{s_j})
// with v_j the leading D_v entries of the same row (absorbed-MLA form).
//
// Work split: a workgroup (8 waves) owns 64 heads of one query and a range of
// the index list; a wave owns 16 heads and one half of the dims (the partner
// wave with the other half adds its partial scores through LDS). Selected rows
// are gathered 32 at a time straight from HBM into a row-major LDS tile by
// global_load_lds_dwordx4 (no registers, no VALU; a ring of three tiles, the
// next ones filling while one is used).
// Both products run on v_mfma_f32_16x16x32_bf16:
//   S^T[j,h] = sum_d K[j,d] Q[h,d]      (A = gathered rows, B = q in registers)
//   O[h,v]  += sum_j P[h,j] V[j,v]      (A = P straight from the S^T
//                                         accumulators, B = V read from the
//                                         same tile by ds_read_b64_tr_b16)
// The accumulator of S^T puts (row 4*(l/16)+r, head l%16) in lane l, element
// r; using that as P's K-slot order (slot 4*b + r <-> row 16*b + 4*(l/16) + r)
// and letting the transposing LDS read deliver V in the same order lets P feed
// the second product without any data movement. Softmax runs online in fp32
// in log2 units.
// When one query's list is split over several workgroups, each writes its
// partial (m, l, and o normalised by l, in fp16) with streaming stores, and a
// combine kernel merges them and adds the sink once.
#include "kernels.h"
#include "select.h"

namespace ic {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kMlaThreads = 512;
constexpr int kHeadsPerWave = 16;
constexpr int kHeadsPerWG = 64;
constexpr int kTile = 32;                 // gathered rows per LDS tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kMInit = -1.0e30f;        // finite "minus infinity" for partials
constexpr int kMaxRowsPerSplit = 2048;    // index entries one workgroup handles
// Rescale slack (log2 units). Zero keeps the running maximum exact, so the
// dominant key's P is exactly 1 and its bf16 rounding is error-free; a larger
// slack would skip more rescales but lets every P carry bf16 rounding.
constexpr float kSlack = 0.0f;

__device__ __forceinline__ f4 mfma_bf16_16x16x32(const bf16x8 &a, const bf16x8 &b, const f4 &c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v)
{
    return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

template <int DQK, int DV>
struct MlaGeom {
    static constexpr int KS = (DQK + 31) / 32;   // K-steps of QK^T
    static constexpr int DQKP = KS * 32;         // padded row length
    static constexpr int KROW = DQKP + 8;        // LDS row stride (bf16)
    static constexpr int NCH = DQK / 8;          // 16-byte chunks per row
    static constexpr int NTV = DV / 16;          // value column tiles
    static_assert(DQK % 8 == 0 && DV % 16 == 0 && DV <= DQK, "shape");
};

typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;
typedef __attribute__((address_space(3))) void lds_void;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Reductions over the four 16-lane rows of a wave (lanes c, c+16, c+32, c+48)
// inside the VGPRs: v_permlane16_swap pairs rows (0,1) and (2,3),
// v_permlane32_swap pairs rows (0,2) and (1,3); each swap of a value with
// itself leaves one partner's copy in each result.
__device__ __forceinline__ float rows_max(float x)
{
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float rows_sum(float x)
{
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Two fp32 -> two bf16 (round to nearest even) in one instruction.
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2{lo, hi}), bf16x2));
}

// LDS tile: kTile gathered rows, row-major, each row padded to ROWCH 16-byte
// chunks (one spare chunk). The pad shifts consecutive rows by 4 banks, so
// lanes reading the same column of 16 consecutive rows hit distinct banks, and
// every operand address is a per-lane base plus a compile-time offset. The tile
// is filled by global_load_lds_dwordx4 instructions that each place 64 lanes x
// 16 bytes contiguously; which (row, chunk) a lane fills in a given
// instruction is the same for every tile and is computed once.
template <int DQK, int DV>
struct TileGeom {
    using G = MlaGeom<DQK, DV>;
    static constexpr int ROWCH = G::KROW * 2 / 16;             // chunks per LDS row
    static constexpr int INSTR = (kTile * ROWCH + 63) / 64;    // fill instructions per tile
    static constexpr int ELEMS = INSTR * 64 * 8;               // bf16 slots per buffer
    static_assert((G::KROW * 2) % 16 == 0, "row stride");
};

constexpr int kBuffers = 3;                 // tiles in flight per workgroup
constexpr int kWaves = kMlaThreads / 64;
constexpr int kFillPerWave = 5;             // >= ceil(fill instructions / waves)
constexpr int kQkBatch = 5;                 // QK^T K-steps whose fragments are read together
constexpr int kPvBatch = 4;                 // PV value tiles whose fragments are read together

// Workgroup barrier that orders LDS traffic only: this wave's LDS operations
// complete, then s_barrier. (__syncthreads carries a release fence that also
// waits for every load in flight, including the ring's LDS fills of later
// tiles, which the barriers of the tile loop do not need: before the barrier
// at the top of a step each wave has waited for its own fills of the tile
// about to be read.) The memory clobber keeps the compiler from moving memory
// operations across it.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// s_waitcnt on the vector-memory counter only (expcnt and lgkmcnt left at max)
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// grid: splits * ceil(H/64) * T workgroups (1-D; the work unit comes from the
// linear id, see below); block: 512 = 4 head groups x 2 halves.
// Wave w owns heads 16*(w%4) .. +16 of the workgroup's 64 and half h = w/4:
// QK^T over its half of the 576 dims (partial scores are summed with the
// partner wave's through LDS), then PV over its half of the 512 value dims.
// Halving the q fragments and the O accumulators per wave lets two waves share
// each SIMD, which hides LDS latency.
// The selection fused into the kernel (SEL): the split phase's view, the
// score rows (for the whole-row fallback) and the index list to write.
struct SelArgs {
    TopkSplitView v;
    const float *scores;
    int64_t ld;
    int32_t *idx_out;
};
constexpr int kSelPerThread = 16;           // collected keys per thread (512 threads: 8192 per query)

template <int DQK, int DV, bool SEL>
__global__ __launch_bounds__(kMlaThreads, 1) void sparse_mla_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ kv, const int64_t *__restrict__ base,
    const int32_t *__restrict__ n_valid, const int32_t *__restrict__ idx, int32_t k, int32_t H,
    const float *__restrict__ sink, float scale_log2,
    int32_t rows_per_split, int32_t splits, void *__restrict__ out, int32_t out_f32,
    uint16_t *__restrict__ part_o, float *__restrict__ part_ml, int32_t direct_parts, const SelArgs sa)
{
    using G = MlaGeom<DQK, DV>;
    using TG = TileGeom<DQK, DV>;
    constexpr int KSH = (G::KS + 1) / 2;          // K-steps per half
    constexpr int NTH = G::NTV / 2;               // value tiles per half
    static_assert(TG::INSTR <= kWaves * kFillPerWave, "fill instructions per wave");
    // the ring's buffers are separate LDS objects (not one array): a read of
    // one buffer is then known not to alias the fills in flight into the
    // others, so the compiler does not wait for those fills before reading
    static_assert(kBuffers == 3, "the ring below is unrolled for three buffers");
    __shared__ __attribute__((aligned(16))) uint16_t tile0[TG::ELEMS];
    __shared__ __attribute__((aligned(16))) uint16_t tile1[TG::ELEMS];
    __shared__ __attribute__((aligned(16))) uint16_t tile2[TG::ELEMS];
    __shared__ __attribute__((aligned(16))) f4 sx[2][kWaves][2][64];   // partial S^T per wave, by tile parity
    __shared__ __attribute__((aligned(16))) int32_t rowid[kMaxRowsPerSplit + kTile];

    // Workgroups are dispatched round-robin over the 8 XCDs (linear id mod 8).
    // Consecutive ids on one XCD take the head groups of the same (query,
    // split), so they gather the same rows through the same L2.
    const int nhg = (H + kHeadsPerWG - 1) / kHeadsPerWG;
    int split, hg, t;
    {
        const int L = blockIdx.x;
        const int xcd = L & 7, slot = L >> 3;
        const int unit_in_xcd = slot / nhg;
        hg = slot - unit_in_xcd * nhg;
        int unit = unit_in_xcd * 8 + xcd;
        // the tail (ids beyond the last full group of 8 x nhg) maps linearly
        const int full = (int)(gridDim.x / (8 * nhg)) * (8 * nhg);
        if (L >= full) {
            unit = full / nhg + (L - full) / nhg;
            hg = (L - full) % nhg;
        }
        split = unit % splits;
        t = unit / splits;
    }
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int hgrp = wave & 3;
    const int half = wave >> 2;
    const int c = lane & 15;
    const int g = lane >> 4;
    const int h0 = hg * kHeadsPerWG + hgrp * kHeadsPerWave;
    const int hc = h0 + c;                        // head of this lane's S^T column
    // this query's latent rows: row j is at byte 2*DQK*j from kvq (a
    // workgroup-uniform base, so fills address by 32-bit offsets)
    const char *kvq = reinterpret_cast<const char *>(kv + base[t] * DQK);
    const int j_begin = split * rows_per_split;
    const int j_end = min(k, j_begin + rows_per_split);
    const int nrows = j_end - j_begin;
    const int ks0 = half * KSH;
    const int nt0 = half * NTH;
    // the split's index list in LDS, padded with empty slots to whole tiles;
    // an entry outside [0, n_valid[t]) counts as empty (it never addresses memory)
    const int padded = (nrows + kTile - 1) / kTile * kTile;
    // with SEL, the split phase's loads go out first: this thread's slice
    // count, the bound and its share of the collected keys
    uint32_t sel_c0 = 0, sel_bound = 0;
    SplitSel<kMlaThreads, kSelPerThread> sel;
    if constexpr (SEL) {
        sel_c0 = tid < sa.v.P ? sa.v.counts[(int64_t)t * sa.v.P + tid] : 0u;
        sel_bound = sa.v.bounds[t];
        sel.load(sa.v.regions + (int64_t)t * sa.v.P * sa.v.stride, sa.v.stride, sa.v.P);
    }
    const int32_t nt = n_valid[t];
    int any_valid = 0;
    if constexpr (!SEL) {
        for (int i = tid; i < padded; i += kMlaThreads) {
            int r = i < nrows ? idx[(int64_t)t * k + j_begin + i] : -1;
            r = (r >= 0 && r < nt) ? r : -1;
            rowid[i] = r;
            any_valid |= r >= 0;
        }
    }

    // q fragments of this half: lane (head hc, group g) holds d = 32*ks + 8*g .. +8
    bf16x8 qf[KSH];
#pragma unroll
    for (int i = 0; i < KSH; ++i) {
        const int d0 = 32 * (ks0 + i) + 8 * g;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (hc < H && ks0 + i < G::KS && d0 < DQK)
            v = *reinterpret_cast<const uint4 *>(q + ((int64_t)t * H + hc) * DQK + d0);
        qf[i] = as_bf16x8(v);
    }

    // (row, chunk) this lane fills in each of this wave's fill instructions
    int fill_row[kFillPerWave], fill_ch[kFillPerWave];
#pragma unroll
    for (int i = 0; i < kFillPerWave; ++i) {
        const int chunk = (wave + kWaves * i) * 64 + lane;
        fill_row[i] = chunk / TG::ROWCH;
        fill_ch[i] = chunk - fill_row[i] * TG::ROWCH;
    }
    // A split with no valid entry skips the tile loop (its result is the
    // empty one: zero output, or m = kMInit and l = 0). Otherwise the query
    // has at least one row, row 0 exists, and empty slots (and the spare
    // chunk of each LDS row) read row 0: finite data the math never uses.
    bool has_rows;
    if constexpr (SEL) {
        // this split's rows are the slots [j_begin, j_end) of the query's
        // selection (position order); the selection's LDS (histograms, slice
        // counts) borrows the score-exchange buffer, unused until the tile loop
        // Shared, then P + 1 slice counts (P <= kMlaThreads) and the scan's
        // wave totals
        static_assert(sizeof(Shared) + 4 * (kMlaThreads + 1 + (kSelPerThread / 4) * kWaves) <= sizeof(sx),
                      "the selection's LDS fits the exchange buffer");
        Shared &sh = *reinterpret_cast<Shared *>(&sx[0][0][0][0]);
        uint32_t *cnt = reinterpret_cast<uint32_t *>(&sh + 1);
        int32_t *iout = hg == 0 && sa.idx_out ? sa.idx_out + (int64_t)t * k : nullptr;
        if (nt <= k) {                            // every position, in order
            for (int i = tid; i < padded; i += kMlaThreads) {
                const int j = j_begin + i;
                rowid[i] = i < nrows && j < nt ? j : -1;
            }
        } else {
            for (int i = nrows + tid; i < padded; i += kMlaThreads)
                rowid[i] = -1;
            auto emit = [&](uint32_t slot, int32_t p) {
                const uint32_t i = slot - (uint32_t)j_begin;
                if (i < (uint32_t)nrows)
                    rowid[i] = p;
            };
            sel.select(RowSrc{sa.scores + (int64_t)t * sa.ld, nt}, k, sel_c0, sel_bound, sa.v.P, sh, cnt,
                       (uint32_t)j_begin, (uint32_t)j_end, emit);
        }
        __syncthreads();                          // rowid complete, sx free
        // the slots of this split go to the layer's index list in one
        // coalesced pass (stores per selected key would each cost a vector
        // memory instruction for a handful of lanes)
        if (iout)
            for (int i = tid; i < nrows; i += kMlaThreads)
                iout[j_begin + i] = rowid[i];
        has_rows = nrows > 0 && j_begin < min(nt, k);
    } else {
        has_rows = __syncthreads_or(any_valid);
    }
    // byte offset of each fill's 16-byte chunk within its row
    int fill_boff[kFillPerWave];
#pragma unroll
    for (int i = 0; i < kFillPerWave; ++i)
        fill_boff[i] = fill_ch[i] < G::NCH ? 16 * fill_ch[i] : 0;

    auto issue = [&](uint16_t *tile, int j0) {
#pragma unroll
        for (int i = 0; i < kFillPerWave; ++i) {
            const int m = wave + kWaves * i;
            if (m < TG::INSTR) {
                const int r = fill_row[i];
                const int rid = r < kTile ? rowid[j0 + r] : -1;
                const uint32_t off = (uint32_t)max(rid, 0) * (uint32_t)(2 * DQK) + (uint32_t)fill_boff[i];
                __builtin_amdgcn_global_load_lds(kvq + off, (lds_void *)(tile + m * 64 * 8), 16, 0, 0);
            }
        }
    };

    float m_run, l_run;
    if (splits == 1) {
        m_run = (hc < H ? sink[hc] : 0.0f) * kLog2e;   // the sink joins as a value-less logit
        l_run = 1.0f;
    } else {
        m_run = kMInit;
        l_run = 0.0f;
    }
    f4 o[NTH];
#pragma unroll
    for (int i = 0; i < NTH; ++i)
        o[i] = f4{0.f, 0.f, 0.f, 0.f};

    // Matrix row m of a 16-row block is tile row perm(m) of that block:
    // perm(4a + j) = 8*(a/2) + 2*j + a%2. The S^T operand reads (8 lanes on 8
    // rows, 16 bytes each) and the transposing V reads (16 lanes on 4 rows x
    // 4 column quads) then both spread over all LDS banks; with plain row
    // order the V reads of neighbouring rows collide.
    auto perm = [](int m) { return 8 * (m >> 3) + 2 * (m & 3) + ((m >> 2) & 1); };
    // per-lane operand bases (element offsets within a tile)
    const int kb0 = perm(c) * G::KROW + 32 * ks0 + 8 * g;    // matrix row c, this half's first K-step
    const int kb1 = kb0 + 16 * G::KROW;                       // matrix row 16 + c
    const int vb0 = perm(4 * g + (c >> 2)) * G::KROW + 16 * nt0 + 4 * (c & 3);
    const int vb1 = vb0 + 16 * G::KROW;
    // rows of this lane's S^T elements r = 0..3: perm(4g + r) = rb8 + 2r + odd
    const int rb8 = 8 * (g >> 1);
    const bool odd = g & 1;

    // partial S^T of one tile over this half's K-steps; fragments are read in
    // batches of kQkBatch steps ahead of their MFMAs
    auto qk = [&](const uint16_t *K, f4 &st0, f4 &st1) {
        // both halves have KSH steps when KS is even (the 576-wide rows); an
        // odd KS leaves the second half one step short
        const int nks = (G::KS % 2 == 0) ? KSH : min(KSH, G::KS - ks0);
        // even and odd K-steps accumulate separately: four independent
        // matrix-instruction chains instead of two dependent ones
        f4 acc[2][2];
#pragma unroll
        for (int a = 0; a < 2; ++a)
            acc[a][0] = acc[a][1] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i0 = 0; i0 < KSH; i0 += kQkBatch) {
            uint4 fa[kQkBatch][2];
#pragma unroll
            for (int i = 0; i < kQkBatch; ++i) {
                if (i0 + i < nks) {
                    fa[i][0] = *reinterpret_cast<const uint4 *>(K + kb0 + 32 * (i0 + i));
                    fa[i][1] = *reinterpret_cast<const uint4 *>(K + kb1 + 32 * (i0 + i));
                }
            }
#pragma unroll
            for (int i = 0; i < kQkBatch; ++i) {
                if (i0 + i < nks) {
                    f4(&c)[2] = acc[(i0 + i) & 1];
                    c[0] = mfma_bf16_16x16x32(as_bf16x8(fa[i][0]), qf[i0 + i], c[0]);
                    c[1] = mfma_bf16_16x16x32(as_bf16x8(fa[i][1]), qf[i0 + i], c[1]);
                }
            }
        }
        st0 = acc[0][0] + acc[1][0];
        st1 = acc[0][1] + acc[1][1];
    };

    // softmax of one tile (this wave's half of the scores plus the partner
    // wave's, exchanged through sx[par]) and its PV product
    auto softmax_pv = [&](const uint16_t *K, int j0, const f4 st0, const f4 st1, int par) {
        // add the partner wave's half of the dims
        const int *rp = &rowid[j0 + rb8 + odd];
        int va[4], vbv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            va[r] = rp[2 * r];
            vbv[r] = rp[16 + 2 * r];
        }
        const f4 o0 = sx[par][wave ^ 4][0][lane];
        const f4 o1 = sx[par][wave ^ 4][1][lane];
        float s[8];
        float mt = -INFINITY;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            // a two-term fp32 sum is commutative, so both waves of the pair
            // get identical scores
            const float t0 = st0[r] + o0[r];
            const float t1 = st1[r] + o1[r];
            s[r] = va[r] >= 0 ? t0 * scale_log2 : -INFINITY;
            s[4 + r] = vbv[r] >= 0 ? t1 * scale_log2 : -INFINITY;
            mt = fmaxf(mt, fmaxf(s[r], s[4 + r]));
        }
        mt = rows_max(mt);
        // The reference point m_run moves only when a column's maximum exceeds
        // it by more than kSlack; tiles that do not raise any maximum skip the
        // O rescale.
        const bool grow = mt > m_run + kSlack;
        float al[4] = {1.0f, 1.0f, 1.0f, 1.0f};
        const bool rescale = __any(grow);
        if (rescale) {
            const float m_new = grow ? mt : m_run;
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            l_run *= alpha;
            m_run = m_new;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                al[r] = __shfl(alpha, 4 * g + r);   // O rows are heads 4*g + r
        }
        float p[8];
        float ps = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            p[i] = __builtin_amdgcn_exp2f(s[i] - m_run);
            ps += p[i];
        }
        ps = rows_sum(ps);
        l_run += ps;
        const uint4 pw = make_uint4(cvt_pk_bf16(p[0], p[1]), cvt_pk_bf16(p[2], p[3]), cvt_pk_bf16(p[4], p[5]),
                                    cvt_pk_bf16(p[6], p[7]));
        const bf16x8 pa = as_bf16x8(pw);
        if (__builtin_amdgcn_readfirstlane(rescale)) {   // rare: a branch, not selects
#pragma unroll
            for (int i = 0; i < NTH; ++i)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    o[i][r] *= al[r];
        }
        // V operand by transposing reads of the row-major tile: per 16-lane
        // group, lane p addresses matrix row 16*b + 4*g + p/4 (tile row
        // 16*b + perm(4*g + p/4)), columns v0 + 4*(p%4) .. +4; lane i then
        // receives column v0 + i of those 4 rows, which is P's slot order
        // (slot 4*b + e <-> matrix row 16*b + 4*g + e).
        auto vfrag = [&](int i) -> bf16x8 {
            const v4s v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(K + vb0 + 16 * i));
            const v4s v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(K + vb1 + 16 * i));
            return __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
        };
#pragma unroll
        for (int i0 = 0; i0 < NTH; i0 += kPvBatch) {
            bf16x8 vb[kPvBatch];
#pragma unroll
            for (int i = 0; i < kPvBatch; ++i)
                if (i0 + i < NTH)
                    vb[i] = vfrag(i0 + i);
#pragma unroll
            for (int i = 0; i < kPvBatch; ++i)
                if (i0 + i < NTH)
                    o[i0 + i] = mfma_bf16_16x16x32(pa, vb[i], o[i0 + i]);
        }
    };

    // Ring of three tiles, tile i in buffer i % 3, software-pipelined by one
    // tile: step i finishes tile i (softmax and PV over the scores exchanged
    // at the end of the previous step), then computes the partial scores of
    // tile i+1 and writes them to sx for the partner wave; tile i+2 fills
    // meanwhile into the buffer tile i-1 left. One barrier per step orders it
    // all: the next tile's partial scores are in sx, its successor's fills
    // have landed, and the oldest buffer is free. The only LDS writes come at
    // the end of a step, so the fills in flight never wait behind them. The
    // ring is unrolled by three so that every access names its buffer.
    const int ntiles = has_rows ? padded / kTile : 0;
    // fill loads a wave issues per tile (the smallest count over the waves)
    constexpr int kPerWave = TG::INSTR / kWaves;
    f4 sc0, sc1;                                  // partial scores of the tile to finish
    if (ntiles > 0) {
        issue(tile0, 0);
        if (ntiles > 1) {
            issue(tile1, kTile);
            wait_vmcnt<kPerWave>();               // tile 0's fills; tile 1's may stay in flight
        } else {
            wait_vmcnt<0>();
        }
        lds_barrier();
        qk(tile0, sc0, sc1);
        sx[0][wave][0][lane] = sc0;
        sx[0][wave][1][lane] = sc1;
        wait_vmcnt<0>();                          // tile 1's fills
        lds_barrier();
    }
    // The two waves of a pair share a SIMD (waves w and w + 4); they take the
    // step's two halves in opposite orders, so that one's matrix products
    // overlap the other's LDS reads and exponentials. (Both orders are
    // legal: tile i+1's scores go to the other sx buffer than tile i's.)
    auto step = [&](int i, const uint16_t *cur, const uint16_t *nxt, uint16_t *ahead) {
        if (i + 2 < ntiles)
            issue(ahead, (i + 2) * kTile);
        if (half == 0) {
            softmax_pv(cur, i * kTile, sc0, sc1, i & 1);
            qk(nxt, sc0, sc1);
        } else {
            f4 n0, n1;
            qk(nxt, n0, n1);
            softmax_pv(cur, i * kTile, sc0, sc1, i & 1);
            sc0 = n0;
            sc1 = n1;
        }
        sx[(i + 1) & 1][wave][0][lane] = sc0;
        sx[(i + 1) & 1][wave][1][lane] = sc1;
        wait_vmcnt<0>();                          // tile i+2's fills
        lds_barrier();
    };
    // (a for loop with guarded steps: a loop with early exits here made the
    // register allocator spill)
    for (int i = 0; i + 1 < ntiles; i += 3) {
        step(i, tile0, tile1, tile2);
        if (i + 2 < ntiles)
            step(i + 1, tile1, tile2, tile0);
        if (i + 3 < ntiles)
            step(i + 2, tile2, tile0, tile1);
    }
    if (ntiles > 0) {                             // the last tile has no successor
        const int last = ntiles - 1;
        const int b = last % 3;
        softmax_pv(b == 0 ? tile0 : (b == 1 ? tile1 : tile2), last * kTile, sc0, sc1, last & 1);
    }

    if (splits == 1) {
        float inv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r)
            inv[r] = 1.0f / __shfl(l_run, 4 * g + r);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int h = h0 + 4 * g + r;
            if (h >= H)
                continue;
            const int64_t orow = ((int64_t)t * H + h) * DV;
#pragma unroll
            for (int i = 0; i < NTH; ++i) {
                const float val = o[i][r] * inv[r];
                const int v = 16 * (nt0 + i) + c;
                if (out_f32)
                    reinterpret_cast<float *>(out)[orow + v] = val;
                else
                    reinterpret_cast<uint16_t *>(out)[orow + v] = (uint16_t)f32_to_bf16_rne(val);
            }
        }
    } else {
        // The split's partial, normalised by its own denominator: a convex
        // combination of value rows, stored as fp16 (2^-11 relative, finer
        // than the bf16 output). Values are scaled by 2^-e per (head, half),
        // e > 0 only when the half's largest magnitude reaches 2^14, so that
        // none leaves the fp16 range; (m, l, e_half0, e_half1) go beside it.
        // Partials go out with streaming stores: dirty L2 lines would
        // otherwise be written back at the kernel boundary, on the critical
        // path. A small set (direct_parts: one short round of workgroups,
        // where the epilogue's latency counts) is stored from the registers,
        // a large one is first staged into whole rows.
        const int64_t prow = ((int64_t)t * splits + split) * H;
        float inv4[4], mx4[4];
        bool big = false;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float l = __shfl(l_run, 4 * g + r);   // O rows are heads 4*g + r
            inv4[r] = l > 0.0f ? 1.0f / l : 0.0f;
            float mx = 0.0f;
#pragma unroll
            for (int i = 0; i < NTH; ++i)
                mx = fmaxf(mx, fabsf(o[i][r] * inv4[r]));
            mx4[r] = mx;
            big |= !(mx < 16384.0f);
        }
        // the maximum over the row group's 16 lanes only where some value of
        // the wave reaches the scaled range (otherwise every e is 0)
        const bool any_big = __any(big);
        float scl4[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float mx = mx4[r];
            if (any_big) {
#pragma unroll
                for (int off = 8; off > 0; off >>= 1)  // over the 16 lanes of the row group
                    mx = fmaxf(mx, __shfl_xor(mx, off));
            }
            const int e = mx >= 16384.0f ? ilogbf(mx) - 13 : 0;
            scl4[r] = ldexpf(inv4[r], -e);
            const int h = h0 + 4 * g + r;
            if (c == 0 && h < H)
                part_ml[(prow + h) * 4 + 2 + half] = (float)e;
        }
        if (direct_parts) {
            // a small partial set: straight from the registers
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if (h0 + 4 * g + r >= H)
                    continue;
                uint16_t *po = part_o + (prow + h0 + 4 * g + r) * DV + 16 * nt0 + c;
#pragma unroll
                for (int i = 0; i < NTH; ++i)
                    __builtin_nontemporal_store(
                        __builtin_bit_cast(uint16_t, static_cast<_Float16>(o[i][r] * scl4[r])), po + 16 * i);
            }
        } else {
            // A large one: the wave's 16 x DV/2 block goes through LDS (the tile
            // buffers, free once every wave has left the tile loop) and leaves in
            // whole rows, 16-byte stores, 32 lanes per 512-byte row.
            constexpr int SROW = DV / 2 + 16;          // staging row stride (elements)
            static_assert(4 * 16 * SROW <= TG::ELEMS, "staging fits a tile buffer");
            lds_barrier();
            uint16_t *stg = (half == 0 ? tile0 : tile1) + hgrp * 16 * SROW;
#pragma unroll
            for (int i = 0; i < NTH; ++i)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    stg[(4 * g + r) * SROW + 16 * i + c] =
                        __builtin_bit_cast(uint16_t, static_cast<_Float16>(o[i][r] * scl4[r]));
            constexpr int RCH = DV / 16;               // 16-byte chunks per staged row
#pragma unroll
            for (int j = 0; j < DV / 64; ++j) {
                const int q = lane + 64 * j;
                const int row = q / RCH, ch = q - row * RCH;
                const u32x4 v = *reinterpret_cast<const u32x4 *>(stg + row * SROW + 8 * ch);
                u32x4 *dst = reinterpret_cast<u32x4 *>(part_o + (prow + h0 + row) * DV + (DV / 2) * half + 8 * ch);
                if (h0 + row < H)
                    __builtin_nontemporal_store(v, dst);
            }
        }
        if (half == 0 && g == 0 && hc < H) {
            part_ml[(prow + hc) * 4 + 0] = m_run;
            part_ml[(prow + hc) * 4 + 1] = l_run;
        }
    }
}

// grid: (H, T); block: DV/4 threads, four value columns each. Merges the
// per-split partials (fp16, normalised by the split's own denominator and
// scaled by 2^-e) and adds the sink:
//   out = sum_s 2^(m_s - m) l_s 2^e_s p_s / (2^(sink - m) + sum_s 2^(m_s - m) l_s)
constexpr int kMaxSplits = 256;
// partial loads in flight per thread: 32 where a head has more than 16
// splits (one round trip instead of two), else 16 (fewer registers)
constexpr int kCombineBatchMax = 32;
constexpr int64_t kResidentWGs = 256;       // one per CU (the tile ring's LDS)
constexpr size_t kDirectPartsMax = (size_t)8 << 20;   // partial sets stored straight from the registers

// Max / sum over the first n lanes of a wave (n = 16 or 64), in registers
// (DPP): row shifts by 1, 2, 4 and 8 reduce each row of 16 lanes into its last
// lane, the row broadcasts carry rows 0 and 2 into rows 1 and 3 and row 1 into
// rows 2 and 3; lane n-1 then holds the result, read back as a scalar.
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_max_step(float v)
{
    constexpr int kNegInf = (int)0xFF800000u;   // lanes without a source take -inf
    return fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(kNegInf, __float_as_int(v), CTRL, ROWS, 0xf, false)));
}

template <int N>
__device__ __forceinline__ float wave_max(float v)
{
    v = dpp_max_step<0x111, 0xf>(v);            // row_shr:1
    v = dpp_max_step<0x112, 0xf>(v);            // row_shr:2
    v = dpp_max_step<0x114, 0xf>(v);            // row_shr:4
    v = dpp_max_step<0x118, 0xf>(v);            // row_shr:8
    if (N > 16) {
        v = dpp_max_step<0x142, 0xa>(v);        // row_bcast:15 into rows 1 and 3
        v = dpp_max_step<0x143, 0xc>(v);        // row_bcast:31 into rows 2 and 3
    }
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), N - 1));
}

template <int N>
__device__ __forceinline__ float wave_sum(float v)
{
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x111, 0xf, 0xf, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x112, 0xf, 0xf, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x114, 0xf, 0xf, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x118, 0xf, 0xf, false));
    if (N > 16) {
        v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xa, 0xf, false));
        v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xc, 0xf, false));
    }
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), N - 1));
}

template <int DV, int CB>
__global__ __launch_bounds__(DV / 4) void mla_combine_kernel(const uint16_t *__restrict__ part_o,
                                                             const float *__restrict__ part_ml,
                                                             const float *__restrict__ sink, int32_t H,
                                                             int32_t splits, void *__restrict__ out,
                                                             int32_t out_f32)
{
    constexpr int NT = DV / 4;
    constexpr int NL = NT < 64 ? NT : 64;       // lanes of the first wave
    static_assert(NL == 16 || NL == 64, "one row or one full wave");
    __shared__ float wgt[2][kMaxSplits];        // per half of the value columns
    __shared__ float inv_den;
    const int h = blockIdx.x;
    const int t = blockIdx.y;
    const int tid = threadIdx.x;
    const int hf = 4 * tid >= DV / 2;           // the half this thread's columns lie in
    const int64_t pr0 = (int64_t)t * splits * H + h;          // row of split 0
    // this thread's four columns of the first CB splits: they do
    // not depend on the weights, so they travel with the (m, l) loads
    const uint2 *p = reinterpret_cast<const uint2 *>(part_o + pr0 * DV) + tid;
    const int64_t stride = (int64_t)H * DV / 4;               // uint2s between splits
    uint2 x[CB];
#pragma unroll
    for (int u = 0; u < CB; ++u)
        if (u < splits)
            x[u] = p[(int64_t)u * stride];
    // the first wave: (m, l, e0, e1) of splits tid, tid + NL, ... in one
    // round trip; the maximum over them and the sink, the weights into LDS,
    // the denominator
    if (tid < NL) {
        constexpr int R = kMaxSplits / NL;
        const float ms = sink[h] * kLog2e;
        float4 ml[R];
        float m = ms;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int s = tid + NL * r;
            ml[r] = s < splits ? *reinterpret_cast<const float4 *>(part_ml + (pr0 + (int64_t)s * H) * 4)
                               : make_float4(-INFINITY, 0.f, 0.f, 0.f);
            m = fmaxf(m, ml[r].x);
        }
        m = wave_max<NL>(m);
        float d = tid == 0 ? exp2f(ms - m) : 0.0f;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int s = tid + NL * r;
            if (s < splits) {
                const float wl = exp2f(ml[r].x - m) * ml[r].y;
                wgt[0][s] = ldexpf(wl, (int)ml[r].z);
                wgt[1][s] = ldexpf(wl, (int)ml[r].w);
                d += wl;
            }
        }
        d = wave_sum<NL>(d);
        if (tid == 0)
            inv_den = 1.0f / d;
    }
    __syncthreads();
    const float inv = inv_den;
    // every split's columns, CB loads in flight
    auto h2f = [](uint32_t b) { return (float)__builtin_bit_cast(_Float16, (uint16_t)b); };
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s0 = 0; s0 < splits; s0 += CB) {
        if (s0 > 0) {
#pragma unroll
            for (int u = 0; u < CB; ++u)
                if (s0 + u < splits)
                    x[u] = p[(int64_t)(s0 + u) * stride];
        }
#pragma unroll
        for (int u = 0; u < CB; ++u)
            if (s0 + u < splits) {
                const float wv = wgt[hf][s0 + u];
                acc.x = fmaf(h2f(x[u].x & 0xFFFFu), wv, acc.x);
                acc.y = fmaf(h2f(x[u].x >> 16), wv, acc.y);
                acc.z = fmaf(h2f(x[u].y & 0xFFFFu), wv, acc.z);
                acc.w = fmaf(h2f(x[u].y >> 16), wv, acc.w);
            }
    }
    const int64_t oi = ((int64_t)t * H + h) * DV + 4 * tid;
    if (out_f32) {
        *reinterpret_cast<float4 *>(reinterpret_cast<float *>(out) + oi) =
            make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
    } else {
        const uint2 v = make_uint2(pack_bf16x2(acc.x * inv, acc.y * inv), pack_bf16x2(acc.z * inv, acc.w * inv));
        *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(out) + oi) = v;
    }
}

template <int DQK, int DV, bool SEL>
hipError_t launch_shape(const uint16_t *q, const uint16_t *kv, const int64_t *base, const int32_t *n_valid,
                        const int32_t *idx,
                        int32_t T, int32_t H, int32_t k, const float *sink, float scale, void *out,
                        int32_t out_f32, const MlaPlan &plan, void *ws, const SelArgs &sa, hipStream_t stream)
{
    const int hg = (H + kHeadsPerWG - 1) / kHeadsPerWG;
    uint16_t *part_o = nullptr;
    float *part_ml = nullptr;
    if (plan.splits > 1) {
        part_o = reinterpret_cast<uint16_t *>(ws);
        part_ml = reinterpret_cast<float *>(part_o + (size_t)T * plan.splits * H * DV);
    }
    hipLaunchKernelGGL((sparse_mla_kernel<DQK, DV, SEL>), dim3(plan.splits * hg * T), dim3(kMlaThreads), 0, stream,
                       q, kv, base, n_valid, idx, k, H, sink, scale * kLog2e, plan.rows_per_split, plan.splits, out,
                       out_f32, part_o, part_ml, (int32_t)plan.direct_parts, sa);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || plan.splits == 1)
        return e;
    if (plan.splits > kCombineBatchMax / 2)
        hipLaunchKernelGGL((mla_combine_kernel<DV, kCombineBatchMax>), dim3(H, T), dim3(DV / 4), 0, stream, part_o,
                           part_ml, sink, H, plan.splits, out, out_f32);
    else
        hipLaunchKernelGGL((mla_combine_kernel<DV, kCombineBatchMax / 2>), dim3(H, T), dim3(DV / 4), 0, stream, part_o,
                           part_ml, sink, H, plan.splits, out, out_f32);
    return hipGetLastError();
}

}  // namespace

bool sparse_mla_supported(int32_t D_qk, int32_t D_v)
{
    return (D_qk == 576 && D_v == 512) || (D_qk == 80 && D_v == 64);
}

MlaPlan plan_sparse_mla(int32_t T, int32_t H, int32_t k, int32_t D_v)
{
    MlaPlan p;
    const int64_t hg = (H + kHeadsPerWG - 1) / kHeadsPerWG;
    const int64_t base_wgs = (int64_t)T * hg;
    int64_t max_splits = (k + 4 * kTile - 1) / (4 * kTile);   // >= 4 tiles per split
    if (max_splits > kMaxSplits)
        max_splits = kMaxSplits;
    int64_t s = base_wgs > 0 ? (512 + base_wgs - 1) / base_wgs : 1;
    s = s < 1 ? 1 : s;
    s = s > max_splits ? max_splits : s;
    s = s < 1 ? 1 : s;
    if (s < (k + kMaxRowsPerSplit - 1) / kMaxRowsPerSplit)
        s = (k + kMaxRowsPerSplit - 1) / kMaxRowsPerSplit;
    // a grid that needs two rounds of workgroups takes one round instead
    // while its splits stay within 16 tiles (one round pays the prologue and
    // epilogue once per CU and lets the layer stack select rows inside it)
    if (base_wgs * s > kResidentWGs && base_wgs <= kResidentWGs) {
        const int64_t s1 = kResidentWGs / base_wgs;
        if (s1 >= 1 && (k + s1 - 1) / s1 <= 16 * kTile)
            s = s1;
    }
    // a small grid takes twice the splits (two tiles each at least) while
    // they still fit on the chip at once (one workgroup per CU): shorter
    // tile loops outweigh the larger partials there, not once a second
    // round of workgroups is needed
    const int64_t max_splits2 = (k + 2 * kTile - 1) / (2 * kTile);
    if (base_wgs * 2 * s <= kResidentWGs && 2 * s <= max_splits2 && 2 * s <= kMaxSplits)
        s *= 2;
    int64_t rps = (k + s - 1) / s;
    rps = (rps + kTile - 1) / kTile * kTile;
    s = (k + rps - 1) / rps;
    if (s < 1)
        s = 1;
    p.splits = (int32_t)s;
    p.rows_per_split = (int32_t)rps;
    p.ws_bytes = s > 1 ? (size_t)T * s * H * ((size_t)D_v * 2 + 4 * sizeof(float)) : 0;
    p.direct_parts = p.ws_bytes <= kDirectPartsMax;
    return p;
}

hipError_t launch_sparse_mla(const uint16_t *q, const uint16_t *kv, const int64_t *base, const int32_t *n_valid,
                             const int32_t *idx, int32_t T, int32_t H, int32_t k, int32_t D_qk, int32_t D_v, const float *sink,
                             float scale, void *out, int32_t out_f32, const MlaPlan &plan, void *ws,
                             hipStream_t stream)
{
    if (T == 0 || H == 0)
        return hipSuccess;
    const SelArgs none{};
    if (D_qk == 576 && D_v == 512)
        return launch_shape<576, 512, false>(q, kv, base, n_valid, idx, T, H, k, sink, scale, out, out_f32, plan, ws,
                                             none, stream);
    if (D_qk == 80 && D_v == 64)
        return launch_shape<80, 64, false>(q, kv, base, n_valid, idx, T, H, k, sink, scale, out, out_f32, plan, ws,
                                           none, stream);
    return hipErrorInvalidValue;
}

bool sparse_mla_selecting_supported(const MlaPlan &plan, int32_t T, int32_t H, const TopkSplitView &v)
{
    const int64_t wgs = (int64_t)plan.splits * ((H + kHeadsPerWG - 1) / kHeadsPerWG) * T;
    return wgs <= kResidentWGs && v.P >= 1 && v.P <= kMlaThreads;
}

hipError_t launch_sparse_mla_selecting(const uint16_t *q, const uint16_t *kv, const int64_t *base,
                                       const int32_t *n_valid, int32_t T, int32_t H, int32_t k, int32_t D_qk,
                                       int32_t D_v, const float *sink, float scale, void *out, int32_t out_f32,
                                       const MlaPlan &plan, void *ws, const float *scores, int64_t ld,
                                       const TopkSplitView &v, int32_t *idx_out, hipStream_t stream)
{
    if (T == 0 || H == 0)
        return hipSuccess;
    const SelArgs sa{v, scores, ld, idx_out};
    if (D_qk == 576 && D_v == 512)
        return launch_shape<576, 512, true>(q, kv, base, n_valid, nullptr, T, H, k, sink, scale, out, out_f32, plan,
                                            ws, sa, stream);
    if (D_qk == 80 && D_v == 64)
        return launch_shape<80, 64, true>(q, kv, base, n_valid, nullptr, T, H, k, sink, scale, out, out_f32, plan,
                                          ws, sa, stream);
    return hipErrorInvalidValue;
}

}  // namespace ic
