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
#include <cstdlib>
#include <cstring>

#include "kernels.h"
#include "lds_dma.h"
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
    static constexpr int KROW = DQKP + 16;       // LDS row stride (bf16), see the tile below
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
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

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

// Sum of the two bf16 values of a packed pair. The softmax denominators add
// the probabilities as rounded for the value product, so that the weights
// the product applies are normalised exactly (a single dominant row then
// passes its value through unchanged, whatever its probability's rounding).
__device__ __forceinline__ float bf16x2_sum(uint32_t w)
{
    return __uint_as_float(w << 16) + __uint_as_float(w & 0xFFFF0000u);
}

// LDS tile: kTile gathered rows, row-major, each row padded to ROWCH 16-byte
// chunks (two spare chunks), and every operand address is a per-lane base plus
// a compile-time offset. The LDS has 64 banks of 4 bytes; a 16-byte read is
// served in four phases of 16 lanes (lanes 0-7 with 24-31, 8-15 with 16-23,
// 32-39 with 56-63, 40-47 with 48-55) and an 8-byte or transposing read in two
// phases of 32 consecutive lanes (found with the bank-conflict counter on
// reads of known addresses). A row stride of 296 words (40 banks mod 64) keeps
// every phase of both fragment reads below on distinct banks; the earlier
// 292-word stride, right for 32 banks, doubled both. The tile is filled by
// global_load_lds_dwordx4 instructions that each place 64 lanes x 16 bytes
// contiguously; which (row, chunk) a lane fills in a given instruction is the
// same for every tile and is computed once.
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

template <int DQK, int DV, bool SEL, bool TR>
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
        // Shared, then P + 1 slice counts (P <= kMlaThreads), the scan's wave
        // totals and P + 1 slice offsets
        static_assert(sizeof(Shared) + 4 * (2 * (kMlaThreads + 1) + (kSelPerThread / 4) * kWaves) <= sizeof(sx),
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
                const int rid = rowid[j0 + min(fill_row[i], kTile - 1)];
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
    // perm(4a + j) = 8*(a/2) + 2*j + a%2, which puts the four rows of each
    // 16-lane group of the transposing V reads 2 rows apart.
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
        // (through readfirstlane: the compiler then knows the count is the
        // same in every lane, so the steps past it are skipped by a scalar
        // branch. Under an EXEC mask instead, a skipped matrix instruction
        // would still run -- they ignore EXEC -- on operand registers that
        // were never loaded.)
        const int nks = __builtin_amdgcn_readfirstlane((G::KS % 2 == 0) ? KSH : min(KSH, G::KS - ks0));
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
        float alpha = 1.0f;                       // this lane's head hc
        float al[4] = {1.0f, 1.0f, 1.0f, 1.0f};   // heads 4*g + r (O's rows, untransposed)
        const bool rescale = __any(grow);
        if (rescale) {
            const float m_new = grow ? mt : m_run;
            alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            l_run *= alpha;
            m_run = m_new;
            if constexpr (!TR) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    al[r] = __shfl(alpha, 4 * g + r);
            }
        }
        float p[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            p[i] = __builtin_amdgcn_exp2f(s[i] - m_run);
        const uint4 pw = make_uint4(cvt_pk_bf16(p[0], p[1]), cvt_pk_bf16(p[2], p[3]), cvt_pk_bf16(p[4], p[5]),
                                    cvt_pk_bf16(p[6], p[7]));
        float ps = (bf16x2_sum(pw.x) + bf16x2_sum(pw.y)) + (bf16x2_sum(pw.z) + bf16x2_sum(pw.w));
        ps = rows_sum(ps);
        l_run += ps;
        const bf16x8 pa = as_bf16x8(pw);
        if (__builtin_amdgcn_readfirstlane(rescale)) {   // rare: a branch, not selects
#pragma unroll
            for (int i = 0; i < NTH; ++i)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    o[i][r] *= TR ? alpha : al[r];
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
                    o[i0 + i] = TR ? mfma_bf16_16x16x32(vb[i], pa, o[i0 + i])
                                   : mfma_bf16_16x16x32(pa, vb[i], o[i0 + i]);
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

    if constexpr (TR) {
    // O is held transposed: element r of o[i] in lane (c, g) is value column
    // 16*(nt0 + i) + 4*g + r of head hc, four consecutive columns per lane
    auto pack_f16x4 = [](const f4 &v, float sc) {
        typedef _Float16 h4 __attribute__((ext_vector_type(4)));
        const h4 x = {static_cast<_Float16>(v[0] * sc), static_cast<_Float16>(v[1] * sc),
                      static_cast<_Float16>(v[2] * sc), static_cast<_Float16>(v[3] * sc)};
        return __builtin_bit_cast(u32x2, x);
    };
    if (splits == 1) {
        const float inv = 1.0f / l_run;           // the sink is in l_run
        if (hc < H) {
            const int64_t orow = ((int64_t)t * H + hc) * DV;
#pragma unroll
            for (int i = 0; i < NTH; ++i) {
                const int v = 16 * (nt0 + i) + 4 * g;
                if (out_f32)
                    *reinterpret_cast<float4 *>(reinterpret_cast<float *>(out) + orow + v) =
                        make_float4(o[i][0] * inv, o[i][1] * inv, o[i][2] * inv, o[i][3] * inv);
                else
                    *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(out) + orow + v) =
                        make_uint2(pack_bf16x2(o[i][0] * inv, o[i][1] * inv), pack_bf16x2(o[i][2] * inv, o[i][3] * inv));
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
        // four columns to a store; a large one is first staged into whole rows.
        const int64_t prow = ((int64_t)t * splits + split) * H;
        const float inv = l_run > 0.0f ? 1.0f / l_run : 0.0f;
        float mx = 0.0f;
#pragma unroll
        for (int i = 0; i < NTH; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                mx = fmaxf(mx, fabsf(o[i][r] * inv));
        // the head's half spans the four 16-lane row groups; their maximum
        // only where some value of the wave reaches the scaled range
        // (otherwise every e is 0)
        if (__any(!(mx < 16384.0f)))
            mx = rows_max(mx);
        const int e = mx >= 16384.0f ? ilogbf(mx) - 13 : 0;
        const float scl = ldexpf(inv, -e);
        if (g == 0 && hc < H)
            part_ml[(prow + hc) * 4 + 2 + half] = (float)e;
        if (direct_parts) {
            // a small partial set: straight from the registers, 8 bytes a store
            if (hc < H) {
                u32x2 *po = reinterpret_cast<u32x2 *>(part_o + (prow + hc) * DV + 16 * nt0 + 4 * g);
#pragma unroll
                for (int i = 0; i < NTH; ++i)
                    __builtin_nontemporal_store(pack_f16x4(o[i], scl), po + 4 * i);
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
                *reinterpret_cast<u32x2 *>(stg + c * SROW + 16 * i + 4 * g) = pack_f16x4(o[i], scl);
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
    } else {
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
}

// ---- wide form -------------------------------------------------------------
// 128 heads per workgroup: 4 waves of 32 heads, each over the whole 576-wide
// row (no split of the dims, so no partial scores cross waves and the tile
// loop writes no LDS), on v_mfma_f32_32x32x16_bf16:
//   S^T[j,h] = sum_d K[j,d] Q[h,d]   (A = 32 gathered rows x 16 dims from LDS,
//                                     B = q of the wave's 32 heads in registers)
//   O[h,v]  += sum_j P[h,j] V[j,v]    (A = P straight from the S^T accumulator,
//                                     B = V by transposing LDS reads)
// The S^T accumulator holds (row 8*(r/4) + 4*(l/32) + r%4, head l%32) in lane
// l, element r. Read as P's K slots (slot e of K-step s <-> row
// 16s + 4*(l/32) + e for e < 4, 16s + 8 + 4*(l/32) + (e-4) after), it feeds the
// second product as is: the transposing V reads deliver those rows in the same
// slots. Every selected row is gathered once for all 128 heads, into a ring of
// four tiles: three gathers stay in flight while one tile is used, and one
// barrier per tile orders it all.
constexpr int kWThreads = 256;
constexpr int kWWaves = kWThreads / 64;
constexpr int kWHeadsPerWave = 32;
constexpr int kWHeadsPerWG = kWWaves * kWHeadsPerWave;     // 128
constexpr int kWQkDepth = 4;                               // QK^T fragment reads in flight
constexpr int kWPvDepth = 4;                               // PV fragment reads in flight
constexpr float kHeadroom = 32.0f;                         // log2 of the largest probability before a second pass

typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ v16f mfma_bf16_32x32x16(const bf16x8 &a, const bf16x8 &b, const v16f &c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Max / sum of a value over the two half-waves (lanes l and l ^ 32): the
// swap of a value with itself leaves one copy of each half in each result.
__device__ __forceinline__ float halves_max(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int DQK, int DV>
struct WideGeom {
    static constexpr int KS = DQK / 16;                     // 32x32x16 K-steps of QK^T
    static constexpr int NT = DV / 32;                      // 32-column value tiles
    static constexpr int KROW = DQK + 16;                   // LDS row stride (bf16): rows 40 banks apart
    static constexpr int ROWCH = KROW * 2 / 16;             // 16-byte chunks per LDS row
    static constexpr int NCH = DQK / 8;                     // of which hold data
    static constexpr int INSTR = (kTile * ROWCH + 63) / 64; // fill instructions per tile
    static constexpr int ELEMS = INSTR * 64 * 8;            // bf16 slots per buffer
    static constexpr int FPW = (INSTR + kWWaves - 1) / kWWaves;   // fill instructions per wave, most
    static constexpr int FPW_MIN = INSTR / kWWaves;               // and fewest
    static constexpr int SROW = DV + 8;                     // partial staging row stride (fp16)
    static_assert(DQK % 16 == 0 && DV % 32 == 0 && DV <= DQK, "shape");
    static_assert((KROW / 2) % 64 == 40, "consecutive LDS rows 40 banks apart");
    static_assert(NCH % 2 == 0, "the chunk swizzle stays inside the row's data");
    static_assert(kWHeadsPerWave * SROW <= ELEMS, "a wave's partial fits one tile buffer");
};

template <int DQK, int DV>
__global__ __launch_bounds__(kWThreads, 1) void sparse_mla_wide_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ kv, const int64_t *__restrict__ base,
    const int32_t *__restrict__ n_valid, const int32_t *__restrict__ idx, int32_t k, int32_t H,
    const float *__restrict__ sink, float scale_log2,
    int32_t rows_per_split, int32_t splits, void *__restrict__ out, int32_t out_f32,
    uint16_t *__restrict__ part_o, float *__restrict__ part_ml, int32_t n_units)
{
    using G = WideGeom<DQK, DV>;
    // the ring's buffers are separate LDS objects: a read of one is known not
    // to alias the fills in flight into the others
    __shared__ __attribute__((aligned(16))) uint16_t tile0[G::ELEMS];
    __shared__ __attribute__((aligned(16))) uint16_t tile1[G::ELEMS];
    __shared__ __attribute__((aligned(16))) uint16_t tile2[G::ELEMS];
    __shared__ __attribute__((aligned(16))) uint16_t tile3[G::ELEMS];
    __shared__ __attribute__((aligned(16))) int32_t rowid[kMaxRowsPerSplit + kTile];

    // Workgroups go round-robin over the 8 XCDs (linear id mod 8). Work unit
    // u = (query, split, head group), in that order of significance from
    // the left, is taken by slot u mod per of XCD u / per: each XCD takes a
    // contiguous block of units, so the splits of a query share its q
    // fragments (and the head groups its rows) through one L2. The grid is
    // 8 * per; ids past the last unit return at once.
    const int nhg = H / kWHeadsPerWG;
    int split, hg, t;
    {
        const int per = (int)(gridDim.x >> 3);
        const int u = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
        if (u >= n_units)
            return;
        hg = u % nhg;
        split = (u / nhg) % splits;
        t = u / (nhg * splits);
    }
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = lane & 31;
    const int g = lane >> 5;
    const int h0 = hg * kWHeadsPerWG + wave * kWHeadsPerWave;
    const int hc = h0 + c;                        // this lane's S^T column (and P row)
    const char *kvq = reinterpret_cast<const char *>(kv + base[t] * DQK);
    const int j_begin = split * rows_per_split;
    const int j_end = min(k, j_begin + rows_per_split);
    const int nrows = j_end - j_begin;
    const int padded = (nrows + kTile - 1) / kTile * kTile;
    const int32_t nt = n_valid[t];
    int any_valid = 0;
    for (int i = tid; i < padded; i += kWThreads) {
        int r = i < nrows ? idx[(int64_t)t * k + j_begin + i] : -1;
        r = (r >= 0 && r < nt) ? r : -1;
        rowid[i] = r;
        any_valid |= r >= 0;
    }
    const bool has_rows = __syncthreads_or(any_valid);

    bf16x8 qf[G::KS];                             // loaded with the first fills, below

    // fill instruction m places 64 lanes x 16 bytes contiguously: lane's chunk
    // m * 64 + lane is chunk ch of tile row r (the spare chunks of each row
    // read chunk 0, and slots past the tile's rows repeat its last row: finite
    // data the math never uses; the row id loads stay unconditional, so they
    // go out together rather than each behind its own branch and wait). The
    // lane index passes through an empty asm so that the per-fill offsets are
    // recomputed here (a few VALU ops) instead of being hoisted out of the
    // tile loop into registers it does not have; the row ids are read all
    // at once, without branches, before the fills go out.
    // LDS byte addresses of the four buffers (constants once LDS is laid out)
    const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_void *)tile0, lds1 = (uint32_t)(uintptr_t)(lds_void *)tile1;
    const uint32_t lds2 = (uint32_t)(uintptr_t)(lds_void *)tile2, lds3 = (uint32_t)(uintptr_t)(lds_void *)tile3;
    auto issue = [&](uint32_t lds_tile, int j0) __attribute__((always_inline)) {
        int ln = lane;
        asm volatile("" : "+v"(ln));
        int rid[G::FPW];
        uint32_t coff[G::FPW];
#pragma unroll
        for (int i = 0; i < G::FPW; ++i) {
            const int chunk = (wave + kWWaves * i) * 64 + ln;
            const int r = chunk / G::ROWCH;
            const int ch = chunk - r * G::ROWCH;
            rid[i] = max(rowid[j0 + min(r, kTile - 1)], 0);
            coff[i] = ch < G::NCH ? 16u * (uint32_t)(ch ^ ((r >> 3) & 1)) : 0u;
        }
#pragma unroll
        for (int i = 0; i < G::FPW; ++i) {
            const int m = wave + kWWaves * i;
            if (m < G::INSTR)
                lds_fill16(kvq, (uint32_t)rid[i] * (uint32_t)(2 * DQK) + coff[i], lds_tile + m * 1024);
        }
    };

    // Softmax state of head hc (log2 units), the same in both half-waves.
    // O is never rescaled inside the tile loop (that would take the
    // accumulators through the VALU): each head's reference m_run moves
    // freely only while its O is still empty, and afterwards stays put while
    // the logits stay within kHeadroom above it, probabilities of up to
    // 2^kHeadroom being exact in bf16 and far from overflow in the fp32
    // sums. A logit beyond that marks the pass void; a second pass then runs
    // with every head's reference at its largest logit, found by the first.
    const float sink_l2 = splits == 1 ? sink[hc] * kLog2e : -INFINITY;   // the sink, a value-less logit
    float m_run, l_run, m_top;
    bool o_nz;                                    // head hc has terms in O
    int overflow = 0;
    auto reset = [&](float m0) __attribute__((always_inline)) {
        m_run = m0;
        l_run = splits == 1 ? __builtin_amdgcn_exp2f(sink_l2 - m0) : 0.0f;
        m_top = m0;
        o_nz = false;
    };
    reset(splits == 1 ? sink_l2 : kMInit);
    v16f o[G::NT];
#pragma unroll
    for (int i = 0; i < G::NT; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            o[i][r] = 0.0f;

    // Matrix row m of the tile is tile row perm(m) = 8(m/8) + 2(m%4) + (m/4)%2.
    // Rows are 40 banks apart and tile rows whose bit 3 is set hold their
    // 16-byte chunks in swapped pairs (chunk ch at ch ^ 1; the fills place
    // them so). With the LDS phases of 16-byte reads (lanes 0-7 with 24-31,
    // 8-15 with 16-23, and so on) and of 8-byte transposing reads (32
    // consecutive lanes), every phase of the K reads (32 rows, 16 bytes each)
    // and of the V reads (4 rows x 64 bytes per phase) lands on distinct banks.
    auto perm = [](int m) { return 8 * (m >> 3) + 2 * (m & 3) + ((m >> 2) & 1); };
    const int kb = perm(c) * G::KROW + 8 * (g ^ ((c >> 3) & 1));    // K: matrix row c, dims 8g..
    const int p16 = lane & 15;
    const int vcol = 16 * ((lane >> 4) & 1) + 4 * (p16 & 3);
    const int vb = perm(4 * g + (p16 >> 2)) * G::KROW + vcol;      // rows 0..7 of each 16: unswapped
    const int vb8 = vb + 8 * G::KROW + ((vcol ^ 8) - vcol);         // rows 8..15: chunk pairs swapped

    auto compute = [&](const uint16_t *K, int j0) __attribute__((always_inline)) {
        // S^T over the 36 K-steps (one accumulation chain: a dependent
        // matrix op takes its predecessor's result by forwarding)
        v16f acc[1];
#pragma unroll
        for (int r = 0; r < 16; ++r)
            acc[0][r] = 0.0f;
        // fragments read kWQkDepth K-steps ahead: each step's read goes into
        // the slot the step kWQkDepth before it has just consumed
        uint4 fa[kWQkDepth];
#pragma unroll
        for (int i = 0; i < kWQkDepth; ++i)
            fa[i] = *reinterpret_cast<const uint4 *>(K + kb + 16 * i);
#pragma unroll
        for (int s = 0; s < G::KS; ++s) {
            acc[0] = mfma_bf16_32x32x16(as_bf16x8(fa[s % kWQkDepth]), qf[s], acc[0]);
            if (s + kWQkDepth < G::KS)
                fa[s % kWQkDepth] = *reinterpret_cast<const uint4 *>(K + kb + 16 * (s + kWQkDepth));
        }
        // validity of this lane's 16 rows: matrix row 8a + 4g + b is index
        // entry j0 + perm(.) = j0 + 8a + 2b + g
        float s[16];
        float mt = -INFINITY;
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const int4 x0 = *reinterpret_cast<const int4 *>(&rowid[j0 + 8 * a]);
            const int4 x1 = *reinterpret_cast<const int4 *>(&rowid[j0 + 8 * a + 4]);
            const int v[4] = {g ? x0.y : x0.x, g ? x0.w : x0.z, g ? x1.y : x1.x, g ? x1.w : x1.z};
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const int r = 4 * a + b;
                const float sum = acc[0][r];
                s[r] = v[b] >= 0 ? sum * scale_log2 : -INFINITY;
                mt = fmaxf(mt, s[r]);
            }
        }
        mt = halves_max(mt);                      // all 32 rows of head hc
        m_top = fmaxf(m_top, mt);
        if (!o_nz) {
            if (mt > m_run) {                     // only the sink's term to carry over
                l_run *= __builtin_amdgcn_exp2f(m_run - mt);
                m_run = mt;
            }
        } else if (mt > m_run + kHeadroom) {
            overflow = 1;
        }
        o_nz = o_nz || mt > -INFINITY;
        float p[16];
#pragma unroll
        for (int r = 0; r < 16; ++r)
            p[r] = __builtin_amdgcn_exp2f(fminf(s[r] - m_run, kHeadroom));
        bf16x8 pa[2];
        float ps = 0.0f;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint4 pw = make_uint4(cvt_pk_bf16(p[8 * h + 0], p[8 * h + 1]), cvt_pk_bf16(p[8 * h + 2], p[8 * h + 3]),
                                        cvt_pk_bf16(p[8 * h + 4], p[8 * h + 5]), cvt_pk_bf16(p[8 * h + 6], p[8 * h + 7]));
            ps += (bf16x2_sum(pw.x) + bf16x2_sum(pw.y)) + (bf16x2_sum(pw.z) + bf16x2_sum(pw.w));
            pa[h] = as_bf16x8(pw);
        }
        l_run += halves_sum(ps);
        // V operand of value tile i, K-step h: rows 16h + 4g + 0..3 and
        // 16h + 8 + 4g + 0..3 of column 32 i + (lane % 32)
        auto vfrag = [&](int i, int h) -> bf16x8 {
            const v4s v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(K + vb + 16 * h * G::KROW + 32 * i));
            const v4s v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(K + vb8 + 16 * h * G::KROW + 32 * i));
            return __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
        };
        // product s: value tile 2(s/4) + s%2, K-half (s/2)%2 (a tile's two
        // products one apart, not back to back), its fragment read
        // kWPvDepth products ahead into the slot just consumed
        constexpr int NS = 2 * G::NT;
        bf16x8 vf[kWPvDepth];
#pragma unroll
        for (int s = 0; s < kWPvDepth; ++s)
            vf[s] = vfrag(2 * (s / 4) + (s % 2), (s / 2) % 2);
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            o[2 * (s / 4) + (s % 2)] = mfma_bf16_32x32x16(pa[(s / 2) % 2], vf[s % kWPvDepth], o[2 * (s / 4) + (s % 2)]);
            if (s + kWPvDepth < NS)
                vf[s % kWPvDepth] = vfrag(2 * ((s + kWPvDepth) / 4) + ((s + kWPvDepth) % 2), ((s + kWPvDepth) / 2) % 2);
        }
    };

    // Ring of four tiles, tile i in buffer i % 4: step i waits for its own
    // fills of tile i (those of tiles i+1 and i+2 stay in flight), and after
    // the barrier -- tile i complete for every wave, tile i-1's buffer free --
    // issues tile i+3 into that buffer, then uses tile i. The loop writes no
    // LDS, so no fill in flight is waited for before its time. The first
    // three tiles and the q fragments go out together and are waited for
    // before the loop (the compiler then has no load of its own pending in
    // it). Unrolled by four so that every access names its buffer.
    const int ntiles = has_rows ? padded / kTile : 0;
    auto step = [&](int i, const uint16_t *cur, uint32_t ahead) __attribute__((always_inline)) {
        // fills issued after tile i's: those of tiles i+1 and i+2 that exist
        // (each wave issues at least FPW_MIN per tile)
        if (i + 2 < ntiles)
            wait_vmcnt<2 * G::FPW_MIN>();
        else if (i + 1 < ntiles)
            wait_vmcnt<G::FPW_MIN>();
        else
            wait_vmcnt<0>();
        lds_barrier();
        if (i + 3 < ntiles)
            issue(ahead, (i + 3) * kTile);
        compute(cur, i * kTile);
    };
    auto issue3 = [&]() __attribute__((always_inline)) {
        issue(lds0, 0);
        if (ntiles > 1)
            issue(lds1, kTile);
        if (ntiles > 2)
            issue(lds2, 2 * kTile);
    };
    if (ntiles > 0)
        issue3();
    // q fragments: K-step i, lane (head c, half g) holds d = 16 i + 8 g .. + 8
#pragma unroll
    for (int i = 0; i < G::KS; ++i)
        qf[i] = as_bf16x8(*reinterpret_cast<const uint4 *>(q + ((int64_t)t * H + hc) * DQK + 16 * i + 8 * g));
    for (int pass = 0; ntiles > 0; ++pass) {
        if (pass > 0)
            issue3();
        wait_vmcnt<0>();
        for (int i = 0; i < ntiles; i += 4) {
            step(i, tile0, lds3);
            if (i + 1 < ntiles)
                step(i + 1, tile1, lds0);
            if (i + 2 < ntiles)
                step(i + 2, tile2, lds1);
            if (i + 3 < ntiles)
                step(i + 3, tile3, lds2);
        }
        wait_vmcnt<0>();                          // the fills past the last tile
        // (the barrier also frees every buffer for a second pass)
        if (pass > 0 || !__syncthreads_or(overflow))
            break;
        reset(m_top);
        o_nz = true;                              // the reference is final
#pragma unroll
        for (int i = 0; i < G::NT; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                o[i][r] = 0.0f;
    }

    // Element r of lane l is head 8(r/4) + 4g + r%4 of the wave, column
    // 32 i + c of value tile i. The output (no split) is staged per wave in
    // one tile buffer (all free once every wave has left the loop) and goes
    // out as whole rows, 16 bytes a lane; a split's partial goes out from
    // the registers (below). A scheduling barrier after each value tile
    // keeps the accumulator reads from crowding the registers.
    auto head_of = [&](int r) { return 8 * (r >> 2) + 4 * g + (r & 3); };
    uint16_t *stg = wave == 0 ? tile0 : (wave == 1 ? tile1 : (wave == 2 ? tile2 : tile3));
    // rows of the staged block to global memory: row j of `bytes` bytes at
    // stg + j * stride bytes goes to dst(j)
    auto store_rows = [&](auto bytes_c, int stride, auto dst) {
        constexpr int chunks = decltype(bytes_c)::value / 16;
        static_assert(kWHeadsPerWave * chunks % 64 == 0, "whole rounds of the wave");
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // the wave's own staging writes
#pragma unroll 8
        for (int it = 0; it < kWHeadsPerWave * chunks / 64; ++it) {
            const int q = lane + 64 * it;
            const int j = q / chunks, ch = q - j * chunks;
            const u32x4 v = *reinterpret_cast<const u32x4 *>(reinterpret_cast<const char *>(stg) + j * stride + 16 * ch);
            __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(dst(j)) + ch);
        }
    };
    using RowBytes = std::integral_constant<int, DV * 2>;       // a bf16 or fp16 row; an fp32 half row
    float inv[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const float l = __shfl(l_run, head_of(r));
        inv[r] = l > 0.0f ? 1.0f / l : 0.0f;
    }
    if (splits == 1) {
        lds_barrier();                            // every wave has left the tile loop
        const int64_t orow = (int64_t)t * H + h0;
        if (out_f32) {
            // fp32 rows in two halves of 256 columns (33 KB of staging each)
            constexpr int SW = DV / 2 + 4;
            float *st = reinterpret_cast<float *>(stg);
            static_assert(kWHeadsPerWave * SW * 4 <= G::ELEMS * 2, "a half fits a tile buffer");
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
                for (int i = hf * G::NT / 2; i < (hf + 1) * G::NT / 2; ++i) {
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        st[head_of(r) * SW + 32 * (i - hf * G::NT / 2) + c] = o[i][r] * inv[r];
                    __builtin_amdgcn_sched_barrier(0);
                }
                store_rows(RowBytes{}, SW * 4, [&](int j) {
                    return reinterpret_cast<float *>(out) + (orow + j) * DV + hf * (DV / 2);
                });
            }
        } else {
#pragma unroll
            for (int i = 0; i < G::NT; ++i) {
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    stg[head_of(r) * G::SROW + 32 * i + c] = (uint16_t)f32_to_bf16_rne(o[i][r] * inv[r]);
                __builtin_amdgcn_sched_barrier(0);
            }
            store_rows(RowBytes{}, G::SROW * 2, [&](int j) {
                return reinterpret_cast<uint16_t *>(out) + (orow + j) * DV;
            });
        }
    } else {
        // The split's partial, normalised by its own denominator, goes out
        // straight from the accumulators in their own order (the wide combine
        // reads that order): per (32-head block, value tile i) 64 lanes x 16
        // fp16, elements 8 hh .. 8 hh + 7 of lane l at ((i * 2 + hh) * 64 + l)
        // * 8, so each store instruction writes 1 KB contiguously. Values
        // are scaled by 2^-e per (head, half of the value columns), e > 0
        // only when that half reaches 2^14; (m, l, e0, e1) go beside them.
        const int64_t prow = ((int64_t)t * splits + split) * H;
        u32x4 *pw = reinterpret_cast<u32x4 *>(part_o + (prow + h0) * DV) + lane;
        auto store_tile = [&](int i, auto scale_of) __attribute__((always_inline)) {
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                uint32_t w4[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 8 * hh + 2 * e;
                    w4[e] = __builtin_bit_cast(uint32_t, f16x2{static_cast<_Float16>(o[i][r] * scale_of(r)),
                                                                static_cast<_Float16>(o[i][r + 1] * scale_of(r + 1))});
                }
                __builtin_nontemporal_store(u32x4{w4[0], w4[1], w4[2], w4[3]}, pw + (i * 2 + hh) * 64);
            }
        };
        // optimistic pass at the plain scale (e = 0), tracking |o| per
        // (element, half)
        float mxr[16][2];
#pragma unroll
        for (int r = 0; r < 16; ++r)
            mxr[r][0] = mxr[r][1] = 0.0f;
#pragma unroll
        for (int i = 0; i < G::NT; ++i) {
#pragma unroll
            for (int r = 0; r < 16; ++r)
                mxr[r][i >= G::NT / 2] = fmaxf(mxr[r][i >= G::NT / 2], fabsf(o[i][r]));
            store_tile(i, [&](int r) { return inv[r]; });
            __builtin_amdgcn_sched_barrier(0);
        }
        bool big = false;
#pragma unroll
        for (int r = 0; r < 16; ++r)
            big |= !(mxr[r][0] * inv[r] < 16384.0f) || !(mxr[r][1] * inv[r] < 16384.0f);
        if (__builtin_amdgcn_readfirstlane(__any(big))) {
            // rare: a half reaches 2^14 somewhere in the wave; exponents per
            // (head, half) over the half-wave's 32 lanes, stored again (a
            // lane's later stores to the same address land last)
            float scl[16][2];
#pragma unroll
            for (int r = 0; r < 16; ++r)
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    float m = mxr[r][hf] * inv[r];
#pragma unroll
                    for (int off = 16; off > 0; off >>= 1)
                        m = fmaxf(m, __shfl_xor(m, off));
                    const int e = m >= 16384.0f ? ilogbf(m) - 13 : 0;
                    scl[r][hf] = ldexpf(inv[r], -e);
                    if (c == 0)
                        part_ml[(prow + h0 + head_of(r)) * 4 + 2 + hf] = (float)e;
                }
#pragma unroll
            for (int i = 0; i < G::NT; ++i)
                store_tile(i, [&](int r) { return scl[r][i >= G::NT / 2]; });
            if (g == 0) {
                part_ml[(prow + hc) * 4 + 0] = m_run;
                part_ml[(prow + hc) * 4 + 1] = l_run;
            }
        } else if (g == 0) {
            *reinterpret_cast<float4 *>(part_ml + (prow + hc) * 4) = make_float4(m_run, l_run, 0.0f, 0.0f);
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

// The same merge for 512 value columns, one wave per head: lane l merges
// columns 8l .. 8l + 7 (16 bytes of every split's partial row) and the wave
// loads its head's (m, l, e0, e1) itself, so no workgroup barrier is needed:
// each wave's split weights stay in its own LDS words, written and read back
// by that wave alone. grid: (ceil(H / HPW), T); block: 64 * HPW threads.
template <int CB, int HPW>
__global__ __launch_bounds__(64 * HPW) void mla_combine512_kernel(const uint16_t *__restrict__ part_o,
                                                                  const float *__restrict__ part_ml,
                                                                  const float *__restrict__ sink, int32_t H,
                                                                  int32_t splits, void *__restrict__ out,
                                                                  int32_t out_f32)
{
    constexpr int DV = 512;
    static_assert(kMaxSplits % CB == 0, "every batch of weights lies inside the array");
    __shared__ float wgt[HPW][2][kMaxSplits];
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int h = blockIdx.x * HPW + wave;
    const int t = blockIdx.y;
    if (h >= H)
        return;                                   // the whole wave; no barrier follows
    const int hf = lane >= 32;                    // columns 8 * lane lie in the second half
    const int64_t pr0 = (int64_t)t * splits * H + h;           // row of split 0
    const uint4 *p = reinterpret_cast<const uint4 *>(part_o + pr0 * DV) + lane;
    const int64_t stride = (int64_t)H * DV / 8;               // uint4s between splits
    uint4 x[CB];
#pragma unroll
    for (int u = 0; u < CB; ++u)
        if (u < splits)
            x[u] = p[(int64_t)u * stride];
    constexpr int R = kMaxSplits / 64;
    const float ms = sink[h] * kLog2e;
    float4 ml[R];
    float m = ms;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int s = lane + 64 * r;
        ml[r] = s < splits ? *reinterpret_cast<const float4 *>(part_ml + (pr0 + (int64_t)s * H) * 4)
                           : make_float4(-INFINITY, 0.f, 0.f, 0.f);
        m = fmaxf(m, ml[r].x);
    }
    m = wave_max<64>(m);
    float d = lane == 0 ? exp2f(ms - m) : 0.0f;
    float *wg = &wgt[wave][0][0];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int s = lane + 64 * r;
        if (s < splits) {
            const float wl = exp2f(ml[r].x - m) * ml[r].y;
            wg[s] = ldexpf(wl, (int)ml[r].z);
            wg[kMaxSplits + s] = ldexpf(wl, (int)ml[r].w);
            d += wl;
        }
    }
    const float inv = 1.0f / wave_sum<64>(d);
    __builtin_amdgcn_wave_barrier();
    const float *wh = wg + kMaxSplits * hf;
    auto h2f = [](uint32_t b) { return (float)__builtin_bit_cast(_Float16, (uint16_t)b); };
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
        acc[e] = 0.0f;
    for (int s0 = 0; s0 < splits; s0 += CB) {
        if (s0 > 0) {
#pragma unroll
            for (int u = 0; u < CB; ++u)
                if (s0 + u < splits)
                    x[u] = p[(int64_t)(s0 + u) * stride];
        }
        // the batch's weights in one go (inside the array whatever the split
        // count: s0 + CB <= kMaxSplits), so the LDS reads are not waited for
        // one by one behind the per-split branches
        float wv4[CB];
#pragma unroll
        for (int u = 0; u < CB; ++u)
            wv4[u] = wh[s0 + u];
#pragma unroll
        for (int u = 0; u < CB; ++u)
            if (s0 + u < splits) {
                const float wv = wv4[u];
                const uint32_t v4[4] = {x[u].x, x[u].y, x[u].z, x[u].w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    acc[2 * e] = fmaf(h2f(v4[e] & 0xFFFFu), wv, acc[2 * e]);
                    acc[2 * e + 1] = fmaf(h2f(v4[e] >> 16), wv, acc[2 * e + 1]);
                }
            }
    }
    const int64_t oi = ((int64_t)t * H + h) * DV + 8 * lane;
    if (out_f32) {
        float4 *o = reinterpret_cast<float4 *>(reinterpret_cast<float *>(out) + oi);
        o[0] = make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
        o[1] = make_float4(acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv);
    } else {
        *reinterpret_cast<uint4 *>(reinterpret_cast<uint16_t *>(out) + oi) =
            make_uint4(pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv),
                       pack_bf16x2(acc[4] * inv, acc[5] * inv), pack_bf16x2(acc[6] * inv, acc[7] * inv));
    }
}

// Merges the wide form's split partials (register order, see its epilogue)
// and adds the sink:
//   out = sum_s 2^(m_s - m) l_s 2^e_s p_s / (2^(sink - m) + sum_s 2^(m_s - m) l_s)
// grid: (value tiles x 32-head blocks, T); block: 64 threads, thread l the
// lane whose 16 values it merges: heads 8(r/4) + 4(l/32) + r%4 of the block,
// column 32 i + l%32. Weights go through LDS; the merged block goes out as
// rows through an LDS transpose.
template <int DV>
__global__ __launch_bounds__(64) void mla_combine_wide_kernel(const uint16_t *__restrict__ part_o,
                                                              const float *__restrict__ part_ml,
                                                              const float *__restrict__ sink, int32_t H,
                                                              int32_t splits, void *__restrict__ out,
                                                              int32_t out_f32)
{
    constexpr int NT = DV / 32;
    extern __shared__ float wgt_dyn[];                       // [splits][33]: weight of (split, head)
    auto wgt = [&](int s_, int h_) -> float & { return wgt_dyn[s_ * 33 + h_]; };
    __shared__ float inv_den[32];
    __shared__ float ot[32][33];
    const int i = blockIdx.x % NT;
    const int wb = blockIdx.x / NT;
    const int t = blockIdx.y;
    const int lane = threadIdx.x;
    const int hf = i >= NT / 2;
    const int64_t pr0 = (int64_t)t * splits * H;             // row of split 0, head 0
    const uint4 *p = reinterpret_cast<const uint4 *>(part_o + (pr0 + 32 * wb) * DV) + (i * 2) * 64 + lane;
    const int64_t stride = (int64_t)H * DV / 8;               // uint4s between splits
    constexpr int CB = 8;                                     // splits in flight
    uint4 x[CB][2];
    auto load_batch = [&](int s0) {
#pragma unroll
        for (int u = 0; u < CB; ++u)
            if (s0 + u < splits) {
                x[u][0] = p[(int64_t)(s0 + u) * stride];
                x[u][1] = p[(int64_t)(s0 + u) * stride + 64];
            }
    };
    // the first batch of partials does not depend on the weights: its loads
    // go out first, so their round trip overlaps the (m, l) phase
    load_batch(0);
    if (lane < 32) {
        // head 32 wb + lane: the maximum over the splits and the sink, then
        // the weights and the denominator
        const int h = 32 * wb + lane;
        const float ms = sink[h] * kLog2e;
        float m = ms;
#pragma unroll 8
        for (int s = 0; s < splits; ++s)
            m = fmaxf(m, part_ml[(pr0 + (int64_t)s * H + h) * 4]);
        float d = exp2f(ms - m);
#pragma unroll 8
        for (int s = 0; s < splits; ++s) {
            const float4 ml = *reinterpret_cast<const float4 *>(part_ml + (pr0 + (int64_t)s * H + h) * 4);
            const float wl = exp2f(ml.x - m) * ml.y;
            wgt(s, lane) = ldexpf(wl, (int)(hf ? ml.w : ml.z));
            d += wl;
        }
        inv_den[lane] = 1.0f / d;
    }
    __syncthreads();
    const int g = lane >> 5;
    auto head_of = [&](int r) { return 8 * (r >> 2) + 4 * g + (r & 3); };
    auto h2f = [](uint32_t b) { return (float)__builtin_bit_cast(_Float16, (uint16_t)b); };
    float acc[16];
#pragma unroll
    for (int r = 0; r < 16; ++r)
        acc[r] = 0.0f;
    for (int s0 = 0; s0 < splits; s0 += CB) {
        if (s0 > 0)
            load_batch(s0);
#pragma unroll
        for (int u = 0; u < CB; ++u)
            if (s0 + u < splits) {
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const uint32_t wv[4] = {x[u][hh].x, x[u][hh].y, x[u][hh].z, x[u][hh].w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = 8 * hh + 2 * e;
                        acc[r] = fmaf(h2f(wv[e] & 0xFFFFu), wgt(s0 + u, head_of(r)), acc[r]);
                        acc[r + 1] = fmaf(h2f(wv[e] >> 16), wgt(s0 + u, head_of(r + 1)), acc[r + 1]);
                    }
                }
            }
    }
    const int c = lane & 31;
#pragma unroll
    for (int r = 0; r < 16; ++r)
        ot[head_of(r)][c] = acc[r] * inv_den[head_of(r)];
    __syncthreads();
    // rows out: head j of the block, columns 32 i .. 32 i + 31
    const int64_t orow = (int64_t)t * H + 32 * wb;
    if (out_f32) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {                        // 32 rows x 8 float4s
            const int k = lane + 64 * q, j = k >> 3, ch = k & 7;
            const float4 v = make_float4(ot[j][4 * ch], ot[j][4 * ch + 1], ot[j][4 * ch + 2], ot[j][4 * ch + 3]);
            *reinterpret_cast<float4 *>(reinterpret_cast<float *>(out) + (orow + j) * DV + 32 * i + 4 * ch) = v;
        }
    } else {
#pragma unroll
        for (int q = 0; q < 2; ++q) {                        // 32 rows x 4 chunks of 8 bf16
            const int k = lane + 64 * q, j = k >> 2, ch = k & 3;
            const uint4 v = make_uint4(pack_bf16x2(ot[j][8 * ch], ot[j][8 * ch + 1]),
                                       pack_bf16x2(ot[j][8 * ch + 2], ot[j][8 * ch + 3]),
                                       pack_bf16x2(ot[j][8 * ch + 4], ot[j][8 * ch + 5]),
                                       pack_bf16x2(ot[j][8 * ch + 6], ot[j][8 * ch + 7]));
            *reinterpret_cast<uint4 *>(reinterpret_cast<uint16_t *>(out) + (orow + j) * DV + 32 * i + 8 * ch) = v;
        }
    }
}

template <int DQK, int DV, bool SEL>
hipError_t launch_shape(const uint16_t *q, const uint16_t *kv, const int64_t *base, const int32_t *n_valid,
                        const int32_t *idx,
                        int32_t T, int32_t H, int32_t k, const float *sink, float scale, void *out,
                        int32_t out_f32, const MlaPlan &plan, void *ws, const SelArgs &sa, hipStream_t stream)
{
    const int hg = (H + plan.heads_per_wg - 1) / plan.heads_per_wg;
    uint16_t *part_o = nullptr;
    float *part_ml = nullptr;
    if (plan.splits > 1) {
        part_o = reinterpret_cast<uint16_t *>(ws);
        part_ml = reinterpret_cast<float *>(part_o + (size_t)T * plan.splits * H * DV);
    }
    if (trace_skip(SEL ? "sparse_mla_kernel<selecting>" : "sparse_mla_kernel")) {
    } else if (plan.heads_per_wg == kWHeadsPerWG) {
        // the wide form: 576/512 rows from a finished list only
        if (SEL || DQK != 576 || DV != 512)
            return hipErrorInvalidValue;
        const int32_t n_units = plan.splits * hg * T;   // eight slots of ceil(n_units / 8) each
        hipLaunchKernelGGL((sparse_mla_wide_kernel<576, 512>), dim3((n_units + 7) / 8 * 8), dim3(kWThreads), 0,
                           stream, q, kv, base, n_valid, idx, k, H, sink, scale * kLog2e, plan.rows_per_split,
                           plan.splits, out, out_f32, part_o, part_ml, n_units);
    } else {
        auto go = [&](auto kern) {
            hipLaunchKernelGGL(kern, dim3(plan.splits * hg * T), dim3(kMlaThreads), 0, stream, q, kv, base, n_valid,
                               idx, k, H, sink, scale * kLog2e, plan.rows_per_split, plan.splits, out, out_f32, part_o,
                               part_ml, (int32_t)plan.direct_parts, sa);
        };
        if (plan.o_trans)
            go(sparse_mla_kernel<DQK, DV, SEL, true>);
        else
            go(sparse_mla_kernel<DQK, DV, SEL, false>);
    }
    trace_launch(stream, SEL ? "sparse_mla_kernel<selecting>" : "sparse_mla_kernel");
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || plan.splits == 1)
        return e;
    if (trace_skip("mla_combine_kernel"))
        ;
    else if (plan.heads_per_wg == kWHeadsPerWG)
        hipLaunchKernelGGL((mla_combine_wide_kernel<512>), dim3((512 / 32) * (H / 32), T), dim3(64),
                           (size_t)plan.splits * 33 * sizeof(float), stream, part_o, part_ml, sink, H, plan.splits,
                           out, out_f32);
    else if (DV == 512) {
        // four heads to a workgroup once that still leaves a workgroup per CU
        const bool four = (int64_t)T * ((H + 3) / 4) >= kResidentWGs;
        auto go = [&](auto kern, int hpw) {
            hipLaunchKernelGGL(kern, dim3((H + hpw - 1) / hpw, T), dim3(64 * hpw), 0, stream, part_o, part_ml, sink, H,
                               plan.splits, out, out_f32);
        };
        if (plan.splits > kCombineBatchMax / 2)
            four ? go(mla_combine512_kernel<kCombineBatchMax, 4>, 4) : go(mla_combine512_kernel<kCombineBatchMax, 1>, 1);
        else
            four ? go(mla_combine512_kernel<kCombineBatchMax / 2, 4>, 4)
                 : go(mla_combine512_kernel<kCombineBatchMax / 2, 1>, 1);
    } else if (plan.splits > kCombineBatchMax / 2)
        hipLaunchKernelGGL((mla_combine_kernel<DV, kCombineBatchMax>), dim3(H, T), dim3(DV / 4), 0, stream, part_o,
                           part_ml, sink, H, plan.splits, out, out_f32);
    else
        hipLaunchKernelGGL((mla_combine_kernel<DV, kCombineBatchMax / 2>), dim3(H, T), dim3(DV / 4), 0, stream, part_o,
                           part_ml, sink, H, plan.splits, out, out_f32);
    trace_launch(stream, "mla_combine_kernel");
    return hipGetLastError();
}

}  // namespace

int32_t sparse_mla_max_k() { return kMaxSplits * kMaxRowsPerSplit; }

bool sparse_mla_supported(int32_t D_qk, int32_t D_v)
{
    return (D_qk == 576 && D_v == 512) || (D_qk == 80 && D_v == 64);
}

MlaPlan plan_sparse_mla(int32_t T, int32_t H, int32_t k, int32_t D_v)
{
    MlaPlan p;
    // The wide form (128 heads per workgroup: each row gathered once, four
    // tiles in flight) serves the 576/512 rows when the heads come in whole
    // groups of 128 and the batch holds at least 16 tiles of rows per CU;
    // smaller batches are latency-bound, where the narrow form's eight
    // waves per workgroup finish each unit of work sooner.
    // IC_MLA_FORM=wide or =narrow overrides the choice where both apply
    // (so that tests reach either form at any size).
    const int64_t wide_tiles = (int64_t)T * (H / kWHeadsPerWG) * ((k + kTile - 1) / kTile);
    const bool wide_ok = D_v == 512 && H % kWHeadsPerWG == 0;
    bool wide = wide_ok && wide_tiles >= 16 * kResidentWGs;
    if (const char *f = getenv("IC_MLA_FORM")) {
        if (!strcmp(f, "wide"))
            wide = wide_ok;
        else if (!strcmp(f, "narrow"))
            wide = false;
    }
    p.heads_per_wg = wide ? kWHeadsPerWG : kHeadsPerWG;
    const int64_t hg = (H + p.heads_per_wg - 1) / p.heads_per_wg;
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
    // The narrow form holds O transposed where its partials are staged
    // through LDS (one 8-byte write per value tile instead of four 2-byte
    // ones: stack_78 2.28 -> 2.19 ms); small sets stored straight from the
    // registers keep the untransposed layout, whose 2-byte stores drain
    // sooner (decode 36.2 us transposed, 34.7 us not). IC_MLA_OTRANS=0|1
    // overrides (both layouts stay testable on every path).
    p.o_trans = p.splits > 1 && !p.direct_parts;
    if (const char *f = getenv("IC_MLA_OTRANS"))
        p.o_trans = !strcmp(f, "1");
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
    const int64_t wgs = (int64_t)plan.splits * ((H + plan.heads_per_wg - 1) / plan.heads_per_wg) * T;
    // The wide form's four waves would select 8192 keys at 32 a thread,
    // slower than the separate finishing pass it saves: it takes its rows
    // from a finished list. (The narrow form keeps one slice count per
    // thread: at most 512 slices.)
    if (plan.heads_per_wg == kWHeadsPerWG)
        return false;
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
