// Sparse MLA with a per-head softmax sink over selected latent rows.
//
// For query t, head h and the selected positions j (explainer "Hy4 IndexCache
// cross-layer index reuse", Jargon "DSA"; GitHub issue "rtx6kpro #90":
// 576-wide latent rows = 512 latent + 64 RoPE, learnable per-head sink that
// biases the softmax denominator):
//   s_j = scale * <q[t,h,:], kv[row_j,:]>,  o = sum_j e^{s_j} v_j / (e^{sink_h} + sum_j e^{s_j})
// with v_j the leading D_v entries of the same row (absorbed-MLA form).
//
// Work split: a workgroup (4 waves) owns 64 heads of one query and a range of
// the index list; each wave owns 16 heads. Selected rows are gathered 32 at a
// time into LDS twice: row-major (the K operand of QK^T, d contiguous) and
// transposed over the value dims (the V operand of PV, rows contiguous).
// Both products run on v_mfma_f32_16x16x32_bf16:
//   S^T[j,h] = sum_d K[j,d] Q[h,d]      (A = gathered rows, B = q in registers)
//   O[h,v]  += sum_j P[h,j] V[j,v]      (A = P straight from the S^T
//                                         accumulators, B = transposed V)
// The accumulator of S^T puts (row 4*(l/16)+r, head l%16) in lane l, element
// r; using that as P's K-slot order (slot 4*b + r <-> row 16*b + 4*(l/16) + r)
// and reading V^T in the same order lets P feed the second product without
// any data movement. Softmax runs online in fp32 in log2 units.
// When one query's list is split over several workgroups, each writes its
// unnormalised partial (m, l, o) and a combine kernel merges them and adds the
// sink once.
#include "kernels.h"

namespace ic {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kMlaThreads = 256;
constexpr int kHeadsPerWave = 16;
constexpr int kHeadsPerWG = 64;
constexpr int kTile = 32;                 // gathered rows per LDS tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kMInit = -1.0e30f;        // finite "minus infinity" for partials
constexpr int kMaxRowsPerSplit = 2048;    // index entries one workgroup handles
constexpr float kSlack = 8.0f;            // lazy-rescale slack, log2 units

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
    static constexpr int VROW = kTile + 4;       // transposed-V row stride (bf16): 72 B keeps
                                                 // the transposing writes conflict-free
    static_assert(DQK % 8 == 0 && DV % 16 == 0 && DV <= DQK, "shape");
};

// Rows of the KV cache a thread copies per tile: items of (row quad, 16-byte
// chunk); the tile's loads are all issued before any is used.
template <int DQK>
struct Gather {
    static constexpr int NCH = DQK / 8;
    static constexpr int ITEMS = (kTile / 4) * NCH;
    static constexpr int PER = (ITEMS + kMlaThreads - 1) / kMlaThreads;
};

// grid: (splits, ceil(H/64), T); block: 256.
template <int DQK, int DV>
__global__ __launch_bounds__(kMlaThreads, 1) void sparse_mla_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ kv, const int64_t *__restrict__ base,
    const int32_t *__restrict__ idx, int32_t k, int32_t H, const float *__restrict__ sink, float scale_log2,
    int32_t rows_per_split, int32_t splits, void *__restrict__ out, int32_t out_f32,
    float *__restrict__ part_o, float *__restrict__ part_ml)
{
    using G = MlaGeom<DQK, DV>;
    using GA = Gather<DQK>;
    __shared__ __attribute__((aligned(16))) uint16_t Ks[kTile * G::KROW];
    __shared__ __attribute__((aligned(16))) uint16_t Vt[DV * G::VROW];
    __shared__ int32_t rowid[kMaxRowsPerSplit];

    const int split = blockIdx.x;
    const int t = blockIdx.z;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int c = lane & 15;
    const int g = lane >> 4;
    const int h0 = blockIdx.y * kHeadsPerWG + wave * kHeadsPerWave;
    const int hc = h0 + c;                        // head of this lane's S^T column
    const int64_t b_t = base[t];
    const int j_begin = split * rows_per_split;
    const int j_end = min(k, j_begin + rows_per_split);
    const int nrows = j_end - j_begin;
    // a row every thread may always read: this query's own q row (used in place
    // of empty index slots, whose data is then replaced by zeros)
    const uint16_t *safe_row = q + (int64_t)t * H * DQK;

    // the split's index list, kept in LDS
    for (int i = tid; i < nrows; i += kMlaThreads)
        rowid[i] = idx[(int64_t)t * k + j_begin + i];

    // q fragments: lane (head hc, group g) holds d = 32*ks + 8*g .. +8
    bf16x8 qf[G::KS];
#pragma unroll
    for (int ks = 0; ks < G::KS; ++ks) {
        const int d0 = 32 * ks + 8 * g;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (hc < H && d0 < DQK)
            v = *reinterpret_cast<const uint4 *>(q + ((int64_t)t * H + hc) * DQK + d0);
        qf[ks] = as_bf16x8(v);
    }
    // padded K columns (d >= DQK) stay zero for the whole kernel
    if (G::DQKP > DQK) {
        for (int i = tid; i < kTile * (G::DQKP - DQK) / 8; i += kMlaThreads) {
            const int r = i / ((G::DQKP - DQK) / 8);
            const int ch = i % ((G::DQKP - DQK) / 8);
            *reinterpret_cast<uint4 *>(&Ks[r * G::KROW + DQK + 8 * ch]) = make_uint4(0, 0, 0, 0);
        }
    }
    __syncthreads();

    // row id of tile-local row j of the tile starting at list offset j0 (-1 = empty)
    auto rid_of = [&](int j0, int j) -> int { return j0 + j < nrows ? rowid[j0 + j] : -1; };

    uint4 pre[GA::PER][4];
    auto prefetch = [&](int j0) {
#pragma unroll
        for (int it = 0; it < GA::PER; ++it) {
            const int item = tid + it * kMlaThreads;
            const int rq = item & 7;
            const int ch = min(item >> 3, GA::NCH - 1);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int rid = rid_of(j0, 4 * rq + r);
                const uint16_t *p = rid >= 0 ? kv + (b_t + rid) * DQK : safe_row;
                pre[it][r] = *reinterpret_cast<const uint4 *>(p + 8 * ch);
            }
        }
    };
    // write the prefetched tile: row-major K, transposed V (zeros for empty slots)
    auto commit = [&](int j0) {
#pragma unroll
        for (int it = 0; it < GA::PER; ++it) {
            const int item = tid + it * kMlaThreads;
            if (item >= GA::ITEMS)
                continue;
            const int rq = item & 7;
            const int ch = item >> 3;
            uint4 v[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                v[r] = rid_of(j0, 4 * rq + r) >= 0 ? pre[it][r] : make_uint4(0, 0, 0, 0);
                *reinterpret_cast<uint4 *>(&Ks[(4 * rq + r) * G::KROW + 8 * ch]) = v[r];
            }
            if (8 * ch < DV) {
                // element e of the 4 rows -> V^T[8*ch + e][4*rq .. 4*rq+3]; a byte
                // permute packs two rows' 16-bit elements per dword
                const uint32_t w0[4] = {v[0].x, v[0].y, v[0].z, v[0].w};
                const uint32_t w1[4] = {v[1].x, v[1].y, v[1].z, v[1].w};
                const uint32_t w2[4] = {v[2].x, v[2].y, v[2].z, v[2].w};
                const uint32_t w3[4] = {v[3].x, v[3].y, v[3].z, v[3].w};
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
                    *reinterpret_cast<uint2 *>(&Vt[(8 * ch + e) * G::VROW + 4 * rq]) =
                        make_uint2(__builtin_amdgcn_perm(w1[e >> 1], w0[e >> 1], sel),
                                   __builtin_amdgcn_perm(w3[e >> 1], w2[e >> 1], sel));
                }
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
    f4 o[G::NTV];
#pragma unroll
    for (int nt = 0; nt < G::NTV; ++nt)
        o[nt] = f4{0.f, 0.f, 0.f, 0.f};

    if (nrows > 0)
        prefetch(0);
    for (int j0 = 0; j0 < nrows; j0 += kTile) {
        __syncthreads();                          // previous tile fully consumed
        commit(j0);
        __syncthreads();

        // S^T = K Q^T for this wave's 16 heads, rows 16*b + (0..15)
        f4 st[2] = {f4{0.f, 0.f, 0.f, 0.f}, f4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int ks = 0; ks < G::KS; ++ks) {
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                const uint4 a = *reinterpret_cast<const uint4 *>(&Ks[(16 * b + c) * G::KROW + 32 * ks + 8 * g]);
                st[b] = mfma_bf16_16x16x32(as_bf16x8(a), qf[ks], st[b]);
            }
        }
        if (j0 + kTile < nrows)
            prefetch(j0 + kTile);                 // in flight during softmax and PV
        float s[8];
        float mt = -INFINITY;
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const bool ok = rid_of(j0, 16 * b + 4 * g + r) >= 0;
                s[4 * b + r] = ok ? st[b][r] * scale_log2 : -INFINITY;
                mt = fmaxf(mt, s[4 * b + r]);
            }
        mt = fmaxf(mt, __shfl_xor(mt, 16));
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        // Lazy rescaling: the reference point m_run only moves when a column's
        // maximum exceeds it by more than kSlack (log2 units), so most tiles
        // skip the O rescale; exponents stay <= 2^kSlack, exact in fp32/bf16 range.
        const bool grow = mt > m_run + kSlack;
        float al[4] = {1.0f, 1.0f, 1.0f, 1.0f};
        const bool rescale = __any(grow);
        if (rescale) {
            const float m_new = grow ? mt : m_run;
            const float alpha = exp2f(m_run - m_new);
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
            p[i] = exp2f(s[i] - m_run);
            ps += p[i];
        }
        ps += __shfl_xor(ps, 16);
        ps += __shfl_xor(ps, 32);
        l_run += ps;
        const uint4 pw = make_uint4(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                                    pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7]));
        const bf16x8 pa = as_bf16x8(pw);
        if (__builtin_amdgcn_readfirstlane(rescale)) {   // rare: a branch, not selects
#pragma unroll
            for (int nt = 0; nt < G::NTV; ++nt)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    o[nt][r] *= al[r];
        }
#pragma unroll
        for (int nt = 0; nt < G::NTV; ++nt) {
            const uint16_t *vr = &Vt[(16 * nt + c) * G::VROW + 4 * g];
            const uint2 v0 = *reinterpret_cast<const uint2 *>(vr);
            const uint2 v1 = *reinterpret_cast<const uint2 *>(vr + 16);
            const bf16x8 vb = as_bf16x8(make_uint4(v0.x, v0.y, v1.x, v1.y));
            o[nt] = mfma_bf16_16x16x32(pa, vb, o[nt]);
        }
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
            for (int nt = 0; nt < G::NTV; ++nt) {
                const float val = o[nt][r] * inv[r];
                if (out_f32)
                    reinterpret_cast<float *>(out)[orow + 16 * nt + c] = val;
                else
                    reinterpret_cast<uint16_t *>(out)[orow + 16 * nt + c] = (uint16_t)f32_to_bf16_rne(val);
            }
        }
    } else {
        const int64_t prow = ((int64_t)t * splits + split) * H;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int h = h0 + 4 * g + r;
            if (h >= H)
                continue;
#pragma unroll
            for (int nt = 0; nt < G::NTV; ++nt)
                part_o[(prow + h) * DV + 16 * nt + c] = o[nt][r];
        }
        if (g == 0 && hc < H) {
            part_ml[(prow + hc) * 2 + 0] = m_run;
            part_ml[(prow + hc) * 2 + 1] = l_run;
        }
    }
}

// grid: (H, T); block: 256. Merges the per-split partials and adds the sink.
constexpr int kMaxSplits = 256;

template <int DV>
__global__ __launch_bounds__(256) void mla_combine_kernel(const float *__restrict__ part_o,
                                                          const float *__restrict__ part_ml,
                                                          const float *__restrict__ sink, int32_t H,
                                                          int32_t splits, void *__restrict__ out,
                                                          int32_t out_f32)
{
    __shared__ float wgt[kMaxSplits];
    __shared__ float red[4];
    const int h = blockIdx.x;
    const int t = blockIdx.y;
    const int tid = threadIdx.x;
    const float ms = sink[h] * kLog2e;
    // global maximum over the sink and the partial maxima
    float m = tid == 0 ? ms : -INFINITY;
    for (int s = tid; s < splits; s += 256)
        m = fmaxf(m, part_ml[(((int64_t)t * splits + s) * H + h) * 2]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        m = fmaxf(m, __shfl_xor(m, off));
    if ((tid & 63) == 0)
        red[tid >> 6] = m;
    __syncthreads();
    m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    // per-split weights and the denominator
    float dsum = tid == 0 ? exp2f(ms - m) : 0.0f;
    for (int s = tid; s < splits; s += 256) {
        const int64_t pr = ((int64_t)t * splits + s) * H + h;
        const float wv = exp2f(part_ml[pr * 2] - m);
        wgt[s] = wv;
        dsum += part_ml[pr * 2 + 1] * wv;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        dsum += __shfl_xor(dsum, off);
    if ((tid & 63) == 0)
        red[tid >> 6] = dsum;
    __syncthreads();
    const float inv = 1.0f / (red[0] + red[1] + red[2] + red[3]);
    const int64_t stride = (int64_t)H * DV;
    for (int v = tid; v < DV; v += 256) {
        const float *p = part_o + ((int64_t)t * splits * H + h) * DV + v;
        float acc = 0.0f;
        int s = 0;
        for (; s + 8 <= splits; s += 8) {
            float x[8];
#pragma unroll
            for (int u = 0; u < 8; ++u)
                x[u] = p[(int64_t)(s + u) * stride];
#pragma unroll
            for (int u = 0; u < 8; ++u)
                acc = fmaf(x[u], wgt[s + u], acc);
        }
        for (; s < splits; ++s)
            acc = fmaf(p[(int64_t)s * stride], wgt[s], acc);
        const int64_t oi = ((int64_t)t * H + h) * DV + v;
        if (out_f32)
            reinterpret_cast<float *>(out)[oi] = acc * inv;
        else
            reinterpret_cast<uint16_t *>(out)[oi] = (uint16_t)f32_to_bf16_rne(acc * inv);
    }
}

template <int DQK, int DV>
hipError_t launch_shape(const uint16_t *q, const uint16_t *kv, const int64_t *base, const int32_t *idx,
                        int32_t T, int32_t H, int32_t k, const float *sink, float scale, void *out,
                        int32_t out_f32, const MlaPlan &plan, void *ws, hipStream_t stream)
{
    const int hg = (H + kHeadsPerWG - 1) / kHeadsPerWG;
    float *part_o = nullptr, *part_ml = nullptr;
    if (plan.splits > 1) {
        part_o = reinterpret_cast<float *>(ws);
        part_ml = part_o + (size_t)T * plan.splits * H * DV;
    }
    hipLaunchKernelGGL((sparse_mla_kernel<DQK, DV>), dim3(plan.splits, hg, T), dim3(kMlaThreads), 0, stream,
                       q, kv, base, idx, k, H, sink, scale * kLog2e, plan.rows_per_split, plan.splits, out,
                       out_f32, part_o, part_ml);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || plan.splits == 1)
        return e;
    hipLaunchKernelGGL((mla_combine_kernel<DV>), dim3(H, T), dim3(256), 0, stream, part_o, part_ml, sink, H,
                       plan.splits, out, out_f32);
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
    int64_t rps = (k + s - 1) / s;
    rps = (rps + kTile - 1) / kTile * kTile;
    s = (k + rps - 1) / rps;
    if (s < 1)
        s = 1;
    p.splits = (int32_t)s;
    p.rows_per_split = (int32_t)rps;
    p.ws_bytes = s > 1 ? (size_t)T * s * H * (D_v + 2) * sizeof(float) : 0;
    return p;
}

hipError_t launch_sparse_mla(const uint16_t *q, const uint16_t *kv, const int64_t *base, const int32_t *idx,
                             int32_t T, int32_t H, int32_t k, int32_t D_qk, int32_t D_v, const float *sink,
                             float scale, void *out, int32_t out_f32, const MlaPlan &plan, void *ws,
                             hipStream_t stream)
{
    if (T == 0 || H == 0)
        return hipSuccess;
    if (D_qk == 576 && D_v == 512)
        return launch_shape<576, 512>(q, kv, base, idx, T, H, k, sink, scale, out, out_f32, plan, ws, stream);
    if (D_qk == 80 && D_v == 64)
        return launch_shape<80, 64>(q, kv, base, idx, T, H, k, sink, scale, out, out_f32, plan, ws, stream);
    return hipErrorInvalidValue;
}

}  // namespace ic
