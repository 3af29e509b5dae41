/*
 * ic.h -- C ABI of libic.so: DeepSeek-style sparse attention with IndexCache
 * cross-layer index reuse, on MI355X (gfx950).
 *
 * Sources of the operations (web pages; cited by title and section):
 *  [E]  explainer "Hy4 IndexCache cross-layer index reuse" (learnaivisually.com):
 *       FAQ, TL;DR, Jargon ("Sparse index", "Indexer", "Top-k selection",
 *       "DSA"), the scheme table, and "Where the saving actually lands".
 *  [G]  GitHub issue "local-inference-lab/rtx6kpro #90": the MLA shape
 *       (RoPE-64, head 576, top-k 2048; first paragraph), the learnable
 *       per-head sink bullet, and the "Indexer:" bullet (shared layers reuse
 *       the last preceding full layer's top-k; 21 full of 78).
 *  [B]  catalogue record "Bai et al.: IndexCache cross-layer sparse-index
 *       reuse" (summary and boundary fields).
 *
 * Conventions shared by every call
 *  - All tensors are row-major and contiguous. Device pointers must be 16-byte
 *    aligned. Element types: indexer q/k are OCP fp8 e4m3fn bytes; head
 *    weights, scores and sinks are fp32; attention q and the latent KV cache
 *    are bf16 bit patterns (uint16_t); index lists are int32 (-1 = empty
 *    slot); cache offsets are int64.
 *  - Every device buffer, workspace included, is allocated by the caller. The
 *    library never allocates or frees device memory.
 *  - Workspaces hold no state between calls: their contents on entry are
 *    ignored (any bytes will do), and a call leaves nothing in them that a
 *    later call reads. One workspace therefore serves any sequence of calls
 *    whose sizes it covers. Calls that overlap in time must use distinct
 *    workspaces.
 *  - Every call enqueues kernels on `stream` (a hipStream_t; NULL = default
 *    stream) and returns without synchronising; no call issues memsets or
 *    host<->device copies, so calls may be captured into a HIP graph.
 *  - Errors: arguments are validated on the host before any launch; on a
 *    validation failure nothing is enqueued and the status says why
 *    (ic_last_error() gives the detail, per thread). IC_ERR_HIP means a launch
 *    failed. Faults inside kernels surface at the caller's next synchronisation.
 *  - Values that live in device memory (n_valid, base, idx) cannot be checked
 *    on the host. Contract: 0 <= n_valid[t] <= max_n, base[t] >= 0,
 *    base[t] + n_valid[t] <= rows, and every idx entry is -1 or in
 *    [0, n_valid[t]).
 */
#ifndef IC_H
#define IC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t ic_status;
enum {
    IC_OK = 0,
    IC_ERR_NULL = 1,        /* a required pointer is NULL                      */
    IC_ERR_SHAPE = 2,       /* sizes are inconsistent or out of range          */
    IC_ERR_UNSUPPORTED = 3, /* valid, but no kernel is built for this shape    */
    IC_ERR_ALIGN = 4,       /* a device pointer or stride is misaligned        */
    IC_ERR_WORKSPACE = 5,   /* workspace missing or smaller than required      */
    IC_ERR_REUSE_MAP = 6,   /* reuse map violates the full/shared rule          */
    IC_ERR_HIP = 7          /* a HIP launch failed                             */
};

enum { IC_OUT_BF16 = 0, IC_OUT_F32 = 1 };

/* Which cache rows each query sees. Query t sees the rows
 * base[t] .. base[t] + n_valid[t] - 1 of the key and latent caches, and
 * positions are sequence-local: position s means row base[t] + s.
 * Decode: each query's cache is its own, n_valid[t] = its length.
 * Causal prefill: all queries read one sequence (same_seq = 1, every base[t]
 * equal) and n_valid[t] = position_t + 1 (a query sees itself).
 * Draft/verify decode ([E] Jargon "MTP": a draft layer proposes several next
 * tokens that one verify pass checks): group = m >= 2 says that queries
 * g*m .. g*m + m - 1 read one sequence (every base[t] equal within a group),
 * typically with n_valid growing by one from query to query. Queries of a
 * group then share the indexer's key stream. */
typedef struct {
    const int64_t *base;     /* device [T]                                     */
    const int32_t *n_valid;  /* device [T]                                     */
    int32_t T;               /* number of queries, >= 0                        */
    int32_t same_seq;        /* nonzero: every query reads the same rows       */
    int64_t max_n;           /* host: upper bound of n_valid[t]                */
    int64_t rows;            /* host: rows in the key and latent caches        */
    int32_t group;           /* 0 or 1: no grouping; m >= 2: T % m == 0 and
                                each run of m queries shares a sequence        */
    int32_t reserved;        /* must be 0                                      */
} ic_queries;

/* Shapes. Indexer: H_I heads of dim D_I (D_I in {32, 64, 128}, 1 <= H_I <= 64).
 * Attention: H heads over rows of D_qk bf16 (latent + RoPE); the value is the
 * leading D_v entries of the same row. Built (D_qk, D_v): (576, 512) -- the
 * MLA shape of [G] -- and (80, 64). */
typedef struct {
    int32_t H_I, D_I;
    int32_t k;               /* top-k, >= 1                                     */
    int32_t H, D_qk, D_v;
    int32_t out_dtype;       /* IC_OUT_BF16 or IC_OUT_F32                       */
} ic_dims;

/* Lightning-indexer scores ([E] Jargon "Indexer" and "DSA": a cheap pass that
 * scores every cached position for a query):
 *   scores[t, s] = sum_h w[t,h] * max(0, sum_d q_idx[t,h,d] * k_idx[base_t+s, d])
 * for 0 <= s < n_valid[t]; entries s >= n_valid[t] of a row are not written.
 *   q_idx  [T, H_I, D_I] fp8 e4m3fn     w      [T, H_I] fp32
 *   k_idx  [rows, D_I]   fp8 e4m3fn     scores [T, ld] fp32, ld >= max_n, ld % 4 == 0
 * Products accumulate in fp32 on the matrix cores; with integer-valued inputs
 * whose partial sums stay below 2^24 the result is exact. q_idx and k_idx
 * hold finite codes: the two NaN codes (0x7F, 0xFF) are outside the domain
 * and the scores they reach are unspecified (top-k takes no NaN scores). */
ic_status ic_indexer_score(const uint8_t *q_idx, const float *w, const uint8_t *k_idx,
                           const ic_queries *qs, int32_t H_I, int32_t D_I,
                           float *scores, int64_t ld, void *stream);

/* Top-k selection ([E] Jargon "Top-k selection" and "Sparse index"; k = 2048
 * in [G]): for each query, the min(k, n_valid[t]) positions s < n_valid[t]
 * with the largest scores[t, s]; among equal scores the lower position wins,
 * so exactly one set is correct. idx [T, k] int32 receives the set in
 * ascending position order followed by -1 padding. Scores are compared as
 * fp32 values (-0 equals +0); NaN scores are not allowed. */
size_t ic_topk_workspace_size(const ic_queries *qs, int32_t k);
ic_status ic_topk(const float *scores, int64_t ld, const ic_queries *qs, int32_t k,
                  int32_t *idx, void *ws, size_t ws_bytes, void *stream);

/* Sparse MLA with a per-head softmax sink ([E] Jargon "DSA": each query
 * attends to its selected tokens only; [G]: 576-wide latent rows, learnable
 * per-head sink acting as a bias in the softmax denominator). For each query
 * t and head h, over the valid entries j of idx[t] (-1 entries are skipped):
 *   s_j = scale * <q[t,h,:], kv[base_t + idx[t,j], :]>
 *   out[t,h,:] = sum_j e^{s_j} kv[base_t + idx[t,j], :D_v] / (e^{sink_h} + sum_j e^{s_j})
 *   q   [T, H, D_qk] bf16     kv  [rows, D_qk] bf16     idx [T, k] int32
 *   sink [H] fp32 (a logit in the units of the scaled scores)
 *   out [T, H, D_v] bf16 (round to nearest even) or fp32, per dims->out_dtype.
 * An all-empty selection gives zeros. Entries outside [0, n_valid[t]) are
 * treated as -1 on the device (they never address memory). QK^T and PV run on bf16 matrix cores
 * with fp32 accumulation and an fp32 softmax; P is rounded to bf16 and the
 * denominators sum the rounded values. Two kernel forms (64 heads per
 * workgroup, or 128 for large grids with D_v = 512 and H a multiple of 128)
 * are chosen by size; IC_MLA_FORM=narrow|wide in the environment overrides
 * the choice, and IC_MLA_OTRANS=0|1 the accumulator layout of the narrow form
 * (chosen by how its partials are stored; the results are the same within the
 * stated bound). Long rows are split over workgroups whose partials a second
 * kernel merges (the workspace holds them). */
size_t ic_sparse_mla_workspace_size(const ic_queries *qs, const ic_dims *d);
ic_status ic_sparse_mla(const uint16_t *q, const uint16_t *kv, const ic_queries *qs,
                        const int32_t *idx, const float *sink, float scale, const ic_dims *d,
                        void *out, void *ws, size_t ws_bytes, void *stream);

/* Gated head output, the step after the sparse attention ([G] bullet on the
 * elementwise sigmoid gate: it multiplies the decompressed per-head output
 * before o_proj, so the value up-projection wv_b must be applied first rather
 * than folded into o_proj):
 *   out[t,h,e] = sigmoid(gate[t,h,e]) * sum_c wv_b[h,e,c] * o[t,h,c]
 *   o    [T, H, D_v] bf16  the latent per-head output of ic_sparse_mla
 *   wv_b [H, D_o, D_v] bf16 the per-head value up-projection
 *   gate [T, H, D_o] bf16  the gate's pre-activation (linear_gate's output)
 *   out  [T, H, D_o] bf16 (round to nearest even)
 * Products run on bf16 matrix cores with fp32 accumulation; sigmoid in fp32.
 * Built: D_v in {512, 64}; D_o a multiple of 64 in [64, 1024]. o_proj itself
 * and linear_gate are plain GEMMs outside this library. */
ic_status ic_gated_output(const uint16_t *o, const uint16_t *wv_b, const uint16_t *gate, int32_t T, int32_t H,
                          int32_t D_v, int32_t D_o, uint16_t *out, void *stream);

/* New tokens for ic_write_cache: where each is stored and the rotary table. */
typedef struct {
    const int64_t *row;      /* device [T]: cache row token t is written to;
                                rows of one call must be distinct             */
    const int32_t *pos;      /* device [T]: token t's position (a table row)  */
    int32_t T;               /* number of tokens, >= 0                        */
    int32_t D_rope;          /* entries per rotated span: even, 0..128; 0 = no
                                rotation                                      */
    int64_t rows;            /* host: rows in the caches that are written     */
    const float *rope;       /* device [n_pos, D_rope] fp32: cos of pair i's
                                angle at [p, i], its sin at [p, D_rope/2 + i] */
    int64_t n_pos;           /* rows of the rotary table                      */
    int32_t key_rope;        /* nonzero: the key's trailing D_rope entries
                                rotate too                                    */
    int32_t reserved;        /* must be 0                                     */
} ic_tokens;

/* Cache write, the step before the path ([G] "Indexer:" bullet: the indexer
 * key passes through a LayerNorm with bias, eps being the model's RMS-norm
 * eps; [G] RoPE bullet: the rotary embedding is interleaved, pairing entries
 * 2i and 2i+1; [G] first paragraph: the latent row is 512 latent entries then
 * 64 RoPE entries). For every token t with row r = row[t] and position
 * p = pos[t]:
 *   indexer key  y = (x - mean x) / sqrt(var x + eps) * ln_w + ln_b over the D_I
 *                entries of x = k_pre[t] (var: mean squared deviation); if
 *                key_rope, the trailing D_rope entries of y rotate at p; then
 *                k_idx[r, :] = fp8 e4m3fn of y (nearest, ties to even,
 *                saturating at +-448; no scale, as ic_indexer_score reads it);
 *   latent row   kv[r, :D_qk - D_rope] = kv_pre[t, :D_qk - D_rope] (bit copy);
 *                the trailing D_rope entries of kv_pre[t] rotate at p and are
 *                rounded to bf16 (nearest even).
 *   Rotation of pair i (entries 2i, 2i+1) with c = rope[p, i], s = rope[p, D_rope/2 + i]:
 *                (a, b) -> (a c - b s, b c + a s).
 *   k_pre [T, D_I] bf16, ln_w and ln_b [D_I] fp32, k_idx [rows, D_I] fp8
 *   kv_pre [T, D_qk] bf16, kv [rows, D_qk] bf16
 * Either part may be skipped: k_pre, ln_w, ln_b and k_idx all NULL (a shared
 * layer, whose indexer never runs), or kv_pre and kv both NULL. Arithmetic in
 * fp32. Built: D_I in {32, 64, 128}; D_qk a multiple of 8 up to 4096 with
 * D_qk - D_rope a multiple of 8. A token whose row lies outside [0, rows) or
 * whose position lies outside [0, n_pos) (when D_rope > 0) writes nothing;
 * rows not named by row[] are never touched. T = 0 is a no-op (IC_OK) whatever
 * the pointers. */
ic_status ic_write_cache(const ic_tokens *tk, const uint16_t *k_pre, const float *ln_w, const float *ln_b,
                         float eps, int32_t D_I, uint8_t *k_idx, const uint16_t *kv_pre, int32_t D_qk, uint16_t *kv,
                         void *stream);

/* One attention layer's tensors for ic_layer_stack. q_idx, w and k_idx are
 * read only on full layers and may be NULL on shared ones. */
typedef struct {
    const uint8_t *q_idx;
    const float *w;
    const uint8_t *k_idx;
    const uint16_t *q;
    const uint16_t *kv;
    const float *sink;
    void *out;
} ic_layer;

/* IndexCache reuse map ([G] "Indexer:" bullet; [E] FAQ and TL;DR: the index
 * is computed once and later layers read it): reuse_map[l] = l when is_full[l]
 * is nonzero, else the last full layer before l. Host arrays of n_layers
 * entries. IC_ERR_REUSE_MAP when layer 0 is not full. */
ic_status ic_reuse_map_last_full(int32_t n_layers, const uint8_t *is_full, int32_t *reuse_map);

/* Layer stack ([E] "Where the saving actually lands": the per-layer indexer
 * pass is what IndexCache removes; [G] "Indexer:" bullet). For l = 0..n_layers-1:
 *   full layer   (reuse_map[l] == l): indexer -> top-k, stored in index_cache
 *                slot = rank of l among the full layers;
 *   shared layer (reuse_map[l] <  l): reads the slot of layer reuse_map[l],
 *                which must be a full layer;
 *   every layer: sparse MLA with its own q, kv, sink over that index into
 *                layers[l].out.
 *   layers      host [n_layers]        reuse_map host [n_layers]
 *   index_cache device [n_full, T, k] int32 (kept: the caller may read it)
 *   indexer_passes (host, may be NULL): receives the number of full layers.
 * Validation of the map: reuse_map[0] == 0, and for l > 0 either
 * reuse_map[l] == l or reuse_map[l] < l with reuse_map[reuse_map[l]] equal to
 * reuse_map[l].
 * A full layer of causal prefill (same_seq, at least 256 queries, max_n at
 * least 65,536; indexer 64 x 128) takes its top-k from the scores at or
 * above a per-query bound drawn from a strided sample of its keys instead of
 * from whole score rows, with the score rows as the fallback for any query
 * the collection cannot serve: the index sets are the same; the workspace
 * size covers both. The environment variable IC_PREFILL_TOPK=scores|collect|
 * fallback overrides that choice, and IC_MLA_FORM=narrow|wide the sparse-MLA
 * form (both for testing and measurement; results are the same within the
 * stated bounds). */
size_t ic_layer_stack_workspace_size(const ic_queries *qs, const ic_dims *d);
ic_status ic_layer_stack(int32_t n_layers, const ic_layer *layers, const int32_t *reuse_map,
                         const ic_queries *qs, const ic_dims *d, float scale,
                         int32_t *index_cache, int32_t *indexer_passes,
                         void *ws, size_t ws_bytes, void *stream);

/* ic_layer_stack for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation, but the workspace is the library's own scratch -- a
 * device array of 32 MiB per GPU, resident while the library is loaded --
 * instead of a caller buffer. The call allocates nothing (device or host);
 * the first call on a device looks up that device's copy of the array once.
 * The caller still provides every input and output, the index cache included.
 * Sizes whose workspace (ic_layer_stack_workspace_size) exceeds 32 MiB return
 * IC_ERR_WORKSPACE before any launch (batch 1 fits up to about 700K cached
 * tokens; batch 8 at 32K fits). All calls on one GPU share its scratch: calls
 * that overlap in time on one GPU (two streams, two threads) race and must be
 * serialised by the caller. Nothing needs clearing between calls: the scratch
 * holds no state a later call reads. */
ic_status ic_layer_stack_static(int32_t n_layers, const ic_layer *layers, const int32_t *reuse_map,
                                const ic_queries *qs, const ic_dims *d, float scale,
                                int32_t *index_cache, int32_t *indexer_passes, void *stream);

/* Tracing, a profiling aid outside the computation. A trace owns timing
 * HIP events: ic_trace_create makes one with room for `capacity` launches
 * (host memory and capacity + 1 events; not under stream capture).
 * ic_trace_start records the start mark on `stream` and arms the calling
 * thread: from then on, right after the i-th kernel the library launches (in
 * any call on this thread, i counting from 0, while i < capacity) it records
 * the trace's event i + 1 on that launch's stream and keeps the kernel's name.
 * Under HIP graph capture the records are made as external event nodes of
 * the graph (each replay timestamps them) where the HIP runtime in use
 * supports that; otherwise ic_trace_start returns IC_ERR_HIP. ic_trace_stop disarms and returns
 * the number of launches seen (which may exceed capacity), or -1 if an event
 * record failed (ic_last_error() says why). Once the stream has reached the
 * last event, ic_trace_read gives the time of launches 0..n-1 in
 * microseconds (event i to event i + 1: the kernel's time on its stream) and,
 * if `names` is not NULL, their kernel names in names + 48 * i
 * (NUL-terminated). Tracing never changes what a call computes. */
#define IC_TRACE_NAME_LEN 48
typedef struct ic_trace ic_trace;
ic_status ic_trace_create(int32_t capacity, ic_trace **trace);
void ic_trace_destroy(ic_trace *trace);
ic_status ic_trace_start(ic_trace *trace, void *stream);
int32_t ic_trace_stop(void);
ic_status ic_trace_read(const ic_trace *trace, float *us, char *names, int32_t n);
/* Leave out every launch of the named kernel (one of the names the trace
 * reports) on the calling thread until called again (NULL: launch all). A
 * profiling aid only: the calls then compute wrong results; timing a step
 * with and without a kernel gives that kernel's cost in the step. */
ic_status ic_trace_skip(const char *kernel);

/* Calibration, a measurement aid outside the computation: one launch that
 * reads `bytes` (a multiple of 16) of device memory at src once, in plain
 * coalesced 16-byte loads, and does nothing else (sink: 64 device words, 16-byte
 * aligned, never written for real data). Its time is the floor of a single
 * launch that streams that many bytes, e.g. the decode indexer's keys. */
ic_status ic_stream_read(const void *src, int64_t bytes, uint32_t *sink, void *stream);

/* Human-readable name of a status, and the detail of the last failure on the
 * calling thread (empty string if none). Both return static storage. */
const char *ic_status_str(ic_status s);
const char *ic_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* IC_H */
