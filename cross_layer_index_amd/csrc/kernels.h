// Internal launch interface between the C-ABI layer (ic_api.cpp) and the HIP
// kernels. Every launcher enqueues on `stream` and returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ic {

// Tracing hook (a profiling aid): after a kernel launch, records the next of
// the caller's trace events on `stream` when tracing is armed on the calling
// thread (ic_trace_start in ic.h), and keeps the kernel's name.
void trace_launch(hipStream_t stream, const char *kernel);
// Whether launches of `kernel` are left out on the calling thread
// (ic_trace_skip; a profiling aid: the step's time without that kernel).
bool trace_skip(const char *kernel);

// ---- indexer --------------------------------------------------------------
// Decode form: each query streams its own key rows (no reuse across queries).
// With `hist0` non-null, also adds each score's first radix digit (bits 31..21
// of its order-preserving key) into hist0[t][copy][2048] (copy = workgroup
// index mod kHistCopies) for the top-k that follows.
hipError_t launch_indexer_decode(const uint8_t *q_idx, const float *w, const uint8_t *k_idx,
                                 const int64_t *base, const int32_t *n, int32_t T, int64_t max_n,
                                 int32_t H_I, int32_t D_I, float *scores, int64_t ld,
                                 uint32_t *hist0, hipStream_t stream);
// Prefill form: all queries read one sequence; key tiles are shared by a
// group of queries through LDS.
// Shared-sequence indexer: groups of G (<= 16) consecutive queries, each
// group reading one sequence (every base[t] equal within a group).
// With `need` non-null only groups holding a query with need[t] != 0 run.
hipError_t launch_indexer_prefill(const uint8_t *q_idx, const float *w, const uint8_t *k_idx,
                                  const int64_t *base, const int32_t *n, int32_t T, int64_t max_n,
                                  int32_t H_I, int32_t D_I, int32_t G, float *scores, int64_t ld,
                                  hipStream_t stream, const uint32_t *need = nullptr);
bool indexer_prefill_supported(int32_t H_I, int32_t D_I);
// Token chunk per workgroup of the shared-key launch for these sizes.
int64_t indexer_prefill_chunk(int32_t T, int32_t G, int64_t max_n);
// Causal prefill with the bounded collection (H_I = 64, D_I = 128, groups of
// 16): scores of the sampled keys (sample row i = key row
// kPfSampleStride * i; query t sees ceil(n_t / kPfSampleStride) of them) into
// scores [T, ld]; and the collection of every score at or above bound[t]
// (order keys) into the slices [T, nchunks, cap] with their counts [T, nchunks]
// (nchunks from indexer_prefill_chunk(T, 16, max_n)).
constexpr int64_t kPfSampleStride = 64;
hipError_t launch_indexer_prefill_sample(const uint8_t *q_idx, const float *w, const uint8_t *k_idx,
                                         const int64_t *base, const int32_t *n, int32_t T, int64_t max_n,
                                         float *scores, int64_t ld, hipStream_t stream);
hipError_t launch_indexer_prefill_collect(const uint8_t *q_idx, const float *w, const uint8_t *k_idx,
                                          const int64_t *base, const int32_t *n, int32_t T, int64_t max_n,
                                          const uint32_t *bound, uint64_t *slices, uint32_t *counts, int32_t cap,
                                          hipStream_t stream);

// ---- top-k ------------------------------------------------------------------
// The workspace starts with the first-digit histograms [T][copies][2048]
// (uint32) that a producer may fill; topk_hist0() points at them.
// launch_clear_hist0 zeroes them (before the first producer of a call); the
// row path returns them to zero after reading them.
size_t topk_workspace_bytes(int32_t T, int64_t max_n, int32_t k);
uint32_t *topk_hist0(void *ws);
// Whether the selection for this shape reads those histograms (a producer
// need not fill them otherwise).
bool topk_reads_hist0(int32_t T, int64_t max_n);
hipError_t launch_clear_hist0(void *ws, int32_t T, hipStream_t stream);
// hist_ready: the histograms were filled while the scores were produced.
// With `need` non-null (row path only) only queries with need[t] != 0 run.
hipError_t launch_topk(const float *scores, int64_t ld, const int32_t *n, int32_t T, int64_t max_n,
                       int32_t k, int32_t *idx, void *ws, bool hist_ready, hipStream_t stream,
                       const uint32_t *need = nullptr);
// Causal prefill with bounded collection: per-query key bounds from the
// sample scores [T, ld]; then the selection from the collected slices
// (writes idx row t and need[t] = 0, or only need[t] = 1 when the scores
// path must serve query t).
hipError_t launch_prefill_bound(const float *sample, int64_t ld, const int32_t *n, int32_t T, int32_t k,
                                uint32_t *bound, bool none, hipStream_t stream);
hipError_t launch_prefill_select(const uint64_t *slices, const uint32_t *counts, int32_t nchunks, int64_t chunk,
                                 int32_t cap, const int32_t *n, int32_t T, int32_t k, int32_t *idx, uint32_t *need,
                                 hipStream_t stream);

// Split path in two launches around a consumer that selects itself: the
// first phase (the collected keys at or above a sampled bound, per query, in
// position-ordered slices) and where it leaves them in the workspace.
struct TopkSplitView {
    const uint32_t *counts;   // [T][P] keys per slice
    const uint64_t *regions;  // [T][P][stride] (key << 32 | position)
    const uint32_t *bounds;   // [T] key bound
    int32_t P;
    int64_t stride;
};
// false when this shape takes the row path (no split phase to share)
bool topk_split_view(void *ws, int32_t T, int64_t max_n, TopkSplitView *v);
hipError_t launch_topk_collect(const float *scores, int64_t ld, const int32_t *n, int32_t T, int64_t max_n,
                               int32_t k, void *ws, hipStream_t stream);

// ---- sparse MLA -----------------------------------------------------------
struct MlaPlan {
    int32_t heads_per_wg;    // heads per workgroup: 128 (wide form) or 64
    int32_t splits;          // k-splits per (query, head group)
    int32_t rows_per_split;  // multiple of the row tile
    size_t ws_bytes;         // partial results when splits > 1
    bool direct_parts;       // partials few enough to store straight from the registers
    bool o_trans;            // narrow form: O held transposed (four value columns of one head per lane)
};
bool sparse_mla_supported(int32_t D_qk, int32_t D_v);
// Largest index list one query may carry: the combine merges at most
// kMaxSplits splits of at most kMaxRowsPerSplit entries.
int32_t sparse_mla_max_k();
MlaPlan plan_sparse_mla(int32_t T, int32_t H, int32_t k, int32_t D_v);
hipError_t launch_sparse_mla(const uint16_t *q, const uint16_t *kv, const int64_t *base,
                             const int32_t *n_valid, const int32_t *idx, int32_t T, int32_t H, int32_t k, int32_t D_qk,
                             int32_t D_v, const float *sink, float scale, void *out, int32_t out_f32,
                             const MlaPlan &plan, void *ws, hipStream_t stream);

// Sparse MLA whose workgroups select their own rows from the split phase's
// collected keys (each the slots of its split; workgroups of head group 0
// also write the query's index list to idx_out [T, k]). Only for grids that
// fit on the chip at once.
bool sparse_mla_selecting_supported(const MlaPlan &plan, int32_t T, int32_t H, const TopkSplitView &v);
hipError_t launch_sparse_mla_selecting(const uint16_t *q, const uint16_t *kv, const int64_t *base,
                                       const int32_t *n_valid, int32_t T, int32_t H, int32_t k, int32_t D_qk,
                                       int32_t D_v, const float *sink, float scale, void *out, int32_t out_f32,
                                       const MlaPlan &plan, void *ws, const float *scores, int64_t ld,
                                       const TopkSplitView &v, int32_t *idx_out, hipStream_t stream);

// Gated head output: out = sigmoid(gate) * (wv_b @ o) per head.
bool gated_output_supported(int32_t D_v, int32_t D_o);
hipError_t launch_gated_output(const uint16_t *o, const uint16_t *wv_b, const uint16_t *gate, int32_t T, int32_t H,
                               int32_t D_v, int32_t D_o, uint16_t *out, hipStream_t stream);

// Cache write of new tokens: indexer key (LayerNorm with bias, optional
// interleaved RoPE on its trailing span, fp8 cast) and latent row (copy plus
// interleaved RoPE on the trailing span). k_pre == nullptr skips the key,
// kv_pre == nullptr the latent row.
hipError_t launch_write_cache(const int64_t *row, const int32_t *pos, int32_t T, int64_t rows, const float *rope,
                              int64_t n_pos, int32_t D_rope, int32_t key_rope, const uint16_t *k_pre,
                              const float *ln_w, const float *ln_b, float eps, int32_t D_I, uint8_t *k_idx,
                              const uint16_t *kv_pre, int32_t D_qk, uint16_t *kv, hipStream_t stream);

// Calibration: one pass of plain coalesced 16-byte reads over `bytes` of src
// (sink: 64 words that are never written for real data).
hipError_t launch_stream_read(const void *src, int64_t bytes, uint32_t *sink, hipStream_t stream);

}  // namespace ic
