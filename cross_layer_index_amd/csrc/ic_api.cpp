// C ABI of libic.so: host-side validation, workspace layout and dispatch to
// the HIP kernels. Semantics of every entry point are documented in ic.h.
#include "ic.h"

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <algorithm>
#include <array>
#include <mutex>
#include <new>
#include <vector>

#include "kernels.h"

#define IC_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

thread_local char g_last_error[512] = "";

// Tracing state of the calling thread (ic_trace_start / ic_trace_stop).
constexpr int kTraceNameLen = IC_TRACE_NAME_LEN;
struct Trace {
    ic_trace *tr = nullptr;          // armed trace; null = disarmed
    int32_t count = 0;               // launches seen since ic_trace_start
    hipError_t error = hipSuccess;
};
thread_local Trace g_trace;
thread_local char g_trace_skip[IC_TRACE_NAME_LEN] = "";   // kernel left out ("" = none)

// Scratch memory of ic_layer_stack_static: a file-scope device array, one copy
// per GPU, resident while the library is loaded. Host code never uses the
// array's name as an address: the device address of each GPU's copy is taken
// once per device with hipGetSymbolAddress and kept in g_scratch_dev.
constexpr size_t kScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_dev[kMaxDevices] = {};

ic_status fail(ic_status s, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return s;
}

ic_status ok()
{
    g_last_error[0] = '\0';
    return IC_OK;
}

ic_status hip_status(hipError_t e, const char *what)
{
    if (e != hipSuccess)
        return fail(IC_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

// Device address of the current GPU's scratch copy (resolved on first use).
ic_status scratch_address(void **out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return fail(IC_ERR_HIP, "static layer stack: hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(IC_ERR_UNSUPPORTED, "static layer stack: device %d beyond the %d supported", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(IC_ERR_HIP, "static layer stack: hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
        g_scratch_dev[dev] = p;
    }
    *out = g_scratch_dev[dev];
    return IC_OK;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

constexpr int32_t kMaxT = 65535;          // grid dimension limit for the query axis
constexpr int64_t kMaxN = (int64_t)1 << 30;

ic_status check_queries(const ic_queries *qs)
{
    if (!qs)
        return fail(IC_ERR_NULL, "queries descriptor is NULL");
    if (qs->T < 0 || qs->T > kMaxT)
        return fail(IC_ERR_SHAPE, "T=%d outside [0, %d]", qs->T, kMaxT);
    if (qs->T > 0 && (!qs->base || !qs->n_valid))
        return fail(IC_ERR_NULL, "queries base/n_valid is NULL");
    if (qs->max_n < 0 || qs->max_n > kMaxN)
        return fail(IC_ERR_SHAPE, "max_n=%lld outside [0, 2^30]", (long long)qs->max_n);
    if (qs->rows < 0)
        return fail(IC_ERR_SHAPE, "rows=%lld is negative", (long long)qs->rows);
    if (qs->max_n > qs->rows && qs->T > 0)
        return fail(IC_ERR_SHAPE, "max_n=%lld exceeds rows=%lld", (long long)qs->max_n, (long long)qs->rows);
    if (qs->T > 0 && (!aligned16(qs->base) || !aligned16(qs->n_valid)))
        return fail(IC_ERR_ALIGN, "queries base/n_valid not 16-byte aligned");
    if (qs->group < 0 || qs->reserved != 0)
        return fail(IC_ERR_SHAPE, "queries group=%d must be >= 0 and reserved=%d must be 0", qs->group,
                    qs->reserved);
    if (qs->group > 1 && qs->T % qs->group != 0)
        return fail(IC_ERR_SHAPE, "T=%d is not a multiple of group=%d", qs->T, qs->group);
    return IC_OK;
}

ic_status check_indexer(const uint8_t *q_idx, const float *w, const uint8_t *k_idx, const ic_queries *qs,
                        int32_t H_I, int32_t D_I, const float *scores, int64_t ld)
{
    if (ic_status s = check_queries(qs))
        return s;
    if (qs->T == 0)
        return IC_OK;
    if (!q_idx || !w || !k_idx || !scores)
        return fail(IC_ERR_NULL, "indexer: q_idx, w, k_idx and scores are required");
    if (H_I < 1 || H_I > 64)
        return fail(IC_ERR_UNSUPPORTED, "indexer: H_I=%d outside [1, 64]", H_I);
    if (D_I != 32 && D_I != 64 && D_I != 128)
        return fail(IC_ERR_UNSUPPORTED, "indexer: D_I=%d not in {32, 64, 128}", D_I);
    if (ld < qs->max_n || ld % 4 != 0)
        return fail(IC_ERR_SHAPE, "indexer: ld=%lld must be >= max_n=%lld and a multiple of 4", (long long)ld,
                    (long long)qs->max_n);
    if (!aligned16(q_idx) || !aligned16(w) || !aligned16(k_idx) || !aligned16(scores))
        return fail(IC_ERR_ALIGN, "indexer: device pointers must be 16-byte aligned");
    return IC_OK;
}

ic_status check_topk(const float *scores, int64_t ld, const ic_queries *qs, int32_t k, const int32_t *idx,
                     const void *ws, size_t ws_bytes)
{
    if (ic_status s = check_queries(qs))
        return s;
    if (k < 1 || k > (1 << 20))
        return fail(IC_ERR_SHAPE, "topk: k=%d outside [1, 2^20]", k);
    if (qs->T == 0)
        return IC_OK;
    if (!scores || !idx)
        return fail(IC_ERR_NULL, "topk: scores and idx are required");
    if (ld < qs->max_n || ld % 4 != 0)
        return fail(IC_ERR_SHAPE, "topk: ld=%lld must be >= max_n and a multiple of 4", (long long)ld);
    if (!aligned16(scores) || !aligned16(idx))
        return fail(IC_ERR_ALIGN, "topk: device pointers must be 16-byte aligned");
    const size_t need = ic::topk_workspace_bytes(qs->T, qs->max_n, k);
    if (need > 0 && (!ws || ws_bytes < need))
        return fail(IC_ERR_WORKSPACE, "topk: workspace of %zu bytes required, %zu given", need, ws_bytes);
    if (need > 0 && !aligned16(ws))
        return fail(IC_ERR_ALIGN, "topk: workspace not 16-byte aligned");
    return IC_OK;
}

ic_status check_dims_mla(const ic_dims *d)
{
    if (!d)
        return fail(IC_ERR_NULL, "dims descriptor is NULL");
    if (d->k < 1 || d->k > (1 << 20))
        return fail(IC_ERR_SHAPE, "k=%d outside [1, 2^20]", d->k);
    if (d->H < 1 || d->H > 4096)
        return fail(IC_ERR_SHAPE, "H=%d outside [1, 4096]", d->H);
    if (d->k > ic::sparse_mla_max_k())
        return fail(IC_ERR_UNSUPPORTED, "sparse MLA: k=%d exceeds the %d index entries one query is built for",
                    d->k, ic::sparse_mla_max_k());
    if (!ic::sparse_mla_supported(d->D_qk, d->D_v))
        return fail(IC_ERR_UNSUPPORTED, "sparse MLA: (D_qk, D_v)=(%d, %d) not built; built: (576, 512), (80, 64)",
                    d->D_qk, d->D_v);
    if (d->out_dtype != IC_OUT_BF16 && d->out_dtype != IC_OUT_F32)
        return fail(IC_ERR_SHAPE, "out_dtype=%d unknown", d->out_dtype);
    return IC_OK;
}

ic_status check_mla(const uint16_t *q, const uint16_t *kv, const ic_queries *qs, const int32_t *idx,
                    const float *sink, const ic_dims *d, const void *out, const void *ws, size_t ws_bytes)
{
    if (ic_status s = check_queries(qs))
        return s;
    if (ic_status s = check_dims_mla(d))
        return s;
    if (qs->T == 0)
        return IC_OK;
    if (!q || !kv || !idx || !sink || !out)
        return fail(IC_ERR_NULL, "sparse MLA: q, kv, idx, sink and out are required");
    if (!aligned16(q) || !aligned16(kv) || !aligned16(idx) || !aligned16(sink) || !aligned16(out))
        return fail(IC_ERR_ALIGN, "sparse MLA: device pointers must be 16-byte aligned");
    // a query's latent rows are addressed by 32-bit byte offsets from its first row
    if ((uint64_t)qs->max_n * (uint64_t)d->D_qk * 2u >= (1ull << 32))
        return fail(IC_ERR_UNSUPPORTED, "sparse MLA: max_n=%lld rows of %d bf16 exceed 4 GiB per sequence",
                    (long long)qs->max_n, d->D_qk);
    const ic::MlaPlan plan = ic::plan_sparse_mla(qs->T, d->H, d->k, d->D_v);
    if (plan.ws_bytes > 0 && (!ws || ws_bytes < plan.ws_bytes))
        return fail(IC_ERR_WORKSPACE, "sparse MLA: workspace of %zu bytes required, %zu given", plan.ws_bytes,
                    ws_bytes);
    if (plan.ws_bytes > 0 && !aligned16(ws))
        return fail(IC_ERR_ALIGN, "sparse MLA: workspace not 16-byte aligned");
    return IC_OK;
}

ic_status check_reuse_map(int32_t n_layers, const int32_t *m)
{
    if (n_layers < 1)
        return fail(IC_ERR_SHAPE, "n_layers=%d must be >= 1", n_layers);
    if (!m)
        return fail(IC_ERR_NULL, "reuse_map is NULL");
    if (m[0] != 0)
        return fail(IC_ERR_REUSE_MAP, "layer 0 must be a full layer (reuse_map[0]=%d)", m[0]);
    for (int32_t l = 1; l < n_layers; ++l) {
        const int32_t s = m[l];
        if (s == l)
            continue;
        if (s < 0 || s > l)
            return fail(IC_ERR_REUSE_MAP, "layer %d: source %d is not an earlier layer", l, s);
        if (m[s] != s)
            return fail(IC_ERR_REUSE_MAP, "layer %d: source %d is itself a shared layer", l, s);
    }
    return IC_OK;
}

int64_t score_ld(const ic_queries *qs) { return (int64_t)round_up((size_t)(qs->max_n > 0 ? qs->max_n : 1), 4); }

// layer-stack workspace: [scores][top-k][sparse MLA], each 256-byte aligned
// Causal prefill over long rows selects from a bounded collection of the
// scores instead of whole score rows (see topk.hip); the score rows stay in
// the layout for the queries the collection cannot serve.
struct Collect {
    bool on;
    int64_t sample_ld, chunk, nchunks;
    int32_t cap;
    size_t sample_off, bound_off, slices_off, counts_off, need_off;
};

int prefill_collect_mode(const ic_queries *qs, const ic_dims *d);

struct StackLayout {
    size_t scores_off, topk_off, mla_off, total;
    int64_t ld;
    Collect col;
};

StackLayout stack_layout(const ic_queries *qs, const ic_dims *d)
{
    StackLayout L;
    L.ld = score_ld(qs);
    L.scores_off = 0;
    L.topk_off = round_up((size_t)qs->T * L.ld * sizeof(float), 256);
    L.mla_off = L.topk_off + round_up(ic::topk_workspace_bytes(qs->T, qs->max_n, d->k), 256);
    size_t end = L.mla_off + round_up(ic::plan_sparse_mla(qs->T, d->H, d->k, d->D_v).ws_bytes, 256);
    Collect &c = L.col;
    c = Collect{};
    c.on = prefill_collect_mode(qs, d) > 0;
    if (c.on) {
        const int64_t T = qs->T, n = qs->max_n;
        c.sample_ld = ((n + ic::kPfSampleStride - 1) / ic::kPfSampleStride + 3) / 4 * 4;
        c.chunk = ic::indexer_prefill_chunk(qs->T, 16, n);
        c.nchunks = (n + c.chunk - 1) / c.chunk;
        // twice a chunk's expected share of the survivors (about 2k + 16 x the
        // sample stride per query), plus 64
        const int64_t expect = (2 * (int64_t)d->k + 16 * ic::kPfSampleStride) * c.chunk / n;
        c.cap = (int32_t)std::min<int64_t>(c.chunk, (2 * expect + 64 + 63) / 64 * 64);
        c.sample_off = end;
        c.bound_off = c.sample_off + round_up((size_t)T * c.sample_ld * sizeof(float), 256);
        c.slices_off = c.bound_off + round_up((size_t)T * 4, 256);
        c.counts_off = c.slices_off + round_up((size_t)T * c.nchunks * c.cap * 8, 256);
        c.need_off = c.counts_off + round_up((size_t)T * c.nchunks * 4, 256);
        end = c.need_off + round_up((size_t)T * 4, 256);
    }
    L.total = end;
    return L;
}

// Queries that share a sequence (prefill, or draft/verify groups of 2..16)
// use the key-sharing GEMM form when it is built for the shape; everything
// else streams keys per query. Returns the queries per workgroup, 0 for none.
int32_t shared_key_group(const ic_queries *qs, int32_t H_I, int32_t D_I)
{
    if (!ic::indexer_prefill_supported(H_I, D_I))
        return 0;
    if (qs->same_seq && qs->T > 1)
        return 16;
    if (qs->group >= 2 && qs->group <= 16)
        return qs->group;
    return 0;
}

bool use_prefill_indexer(const ic_queries *qs, int32_t H_I, int32_t D_I)
{
    return shared_key_group(qs, H_I, D_I) > 0;
}

// 0: score rows; 1: bounded collection; 2: bounded collection with nothing
// collected, so that every query takes the score rows (a test of that path).
// Causal prefill of at least 256 queries over rows of at least 65,536 tokens
// collects; IC_PREFILL_TOPK=scores|collect|fallback overrides the length rule.
int prefill_collect_mode(const ic_queries *qs, const ic_dims *d)
{
    if (!qs->same_seq || qs->T < 256 || shared_key_group(qs, d->H_I, d->D_I) != 16 || qs->max_n < 1)
        return 0;
    if (const char *f = getenv("IC_PREFILL_TOPK")) {
        if (!strcmp(f, "scores"))
            return 0;
        if (!strcmp(f, "collect"))
            return 1;
        if (!strcmp(f, "fallback"))
            return 2;
    }
    return qs->max_n >= 65536 ? 1 : 0;
}

hipError_t launch_indexer(const uint8_t *q_idx, const float *w, const uint8_t *k_idx, const ic_queries *qs,
                          int32_t H_I, int32_t D_I, float *scores, int64_t ld, uint32_t *hist0, hipStream_t st)
{
    if (const int32_t G = shared_key_group(qs, H_I, D_I))
        return ic::launch_indexer_prefill(q_idx, w, k_idx, qs->base, qs->n_valid, qs->T, qs->max_n, H_I, D_I, G,
                                          scores, ld, st);
    return ic::launch_indexer_decode(q_idx, w, k_idx, qs->base, qs->n_valid, qs->T, qs->max_n, H_I, D_I, scores, ld,
                                     hist0, st);
}

}  // namespace

// A trace: its events (the start mark, then one per launch) and the names.
struct ic_trace {
    std::vector<hipEvent_t> events;
    std::vector<std::array<char, kTraceNameLen>> names;
    int32_t recorded = 0;            // launches of the last armed period with an event
};

namespace {
// An event record that stays a timestamp under stream capture (an external
// event node in the graph), a plain record otherwise.
hipError_t trace_record(hipEvent_t ev, hipStream_t stream)
{
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    hipError_t e = hipStreamIsCapturing(stream, &cs);
    if (e != hipSuccess)
        return e;
    return cs == hipStreamCaptureStatusActive ? hipEventRecordWithFlags(ev, stream, hipEventRecordExternal)
                                              : hipEventRecord(ev, stream);
}
}  // namespace

void ic::trace_launch(hipStream_t stream, const char *kernel)
{
    Trace &st = g_trace;
    if (!st.tr)
        return;
    ic_trace &tr = *st.tr;
    if ((size_t)st.count + 1 < tr.events.size()) {
        const hipError_t e = trace_record(tr.events[st.count + 1], stream);
        if (e != hipSuccess && st.error == hipSuccess)
            st.error = e;
        snprintf(tr.names[st.count].data(), kTraceNameLen, "%s", kernel);
        tr.recorded = st.count + 1;
    }
    ++st.count;
}

bool ic::trace_skip(const char *kernel)
{
    return g_trace_skip[0] != '\0' && strcmp(g_trace_skip, kernel) == 0;
}

IC_EXPORT ic_status ic_stream_read(const void *src, int64_t bytes, uint32_t *sink, void *stream)
{
    if (bytes < 0 || bytes % 16)
        return fail(IC_ERR_SHAPE, "stream read: bytes=%lld must be a non-negative multiple of 16", (long long)bytes);
    if (bytes == 0)
        return ok();
    if (!src || !sink)
        return fail(IC_ERR_NULL, "stream read: src and sink are required");
    if (!aligned16(src) || !aligned16(sink))
        return fail(IC_ERR_ALIGN, "stream read: pointers must be 16-byte aligned");
    return hip_status(ic::launch_stream_read(src, bytes, sink, reinterpret_cast<hipStream_t>(stream)),
                      "stream read launch");
}

IC_EXPORT ic_status ic_trace_skip(const char *kernel)
{
    if (kernel && strlen(kernel) >= sizeof g_trace_skip)
        return fail(IC_ERR_SHAPE, "trace: kernel name longer than %d", IC_TRACE_NAME_LEN - 1);
    snprintf(g_trace_skip, sizeof g_trace_skip, "%s", kernel ? kernel : "");
    return ok();
}

IC_EXPORT ic_status ic_trace_create(int32_t capacity, ic_trace **out)
{
    if (!out)
        return fail(IC_ERR_NULL, "trace: no output pointer");
    if (capacity < 1 || capacity > (1 << 20))
        return fail(IC_ERR_SHAPE, "trace: capacity=%d outside [1, 2^20]", capacity);
    *out = nullptr;
    ic_trace *tr = new (std::nothrow) ic_trace;
    if (!tr)
        return fail(IC_ERR_HIP, "trace: out of host memory");
    tr->names.resize(capacity);
    for (int32_t i = 0; i <= capacity; ++i) {
        hipEvent_t ev = nullptr;
        const hipError_t e = hipEventCreate(&ev);
        if (e != hipSuccess) {
            ic_trace_destroy(tr);
            return fail(IC_ERR_HIP, "trace: hipEventCreate: %s", hipGetErrorString(e));
        }
        tr->events.push_back(ev);
    }
    *out = tr;
    return ok();
}

IC_EXPORT void ic_trace_destroy(ic_trace *tr)
{
    if (!tr)
        return;
    if (g_trace.tr == tr)
        g_trace = Trace{};
    for (hipEvent_t ev : tr->events)
        (void)hipEventDestroy(ev);
    delete tr;
}

IC_EXPORT ic_status ic_trace_start(ic_trace *tr, void *stream)
{
    if (!tr)
        return fail(IC_ERR_NULL, "trace: no trace");
    const hipError_t e = trace_record(tr->events[0], reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return fail(IC_ERR_HIP, "trace: start mark: %s", hipGetErrorString(e));
    tr->recorded = 0;
    g_trace = Trace{tr, 0, hipSuccess};
    return ok();
}

IC_EXPORT int32_t ic_trace_stop(void)
{
    const int32_t n = g_trace.count;
    const hipError_t e = g_trace.error;
    g_trace = Trace{};
    if (e != hipSuccess) {
        fail(IC_ERR_HIP, "trace: hipEventRecord: %s", hipGetErrorString(e));
        return -1;
    }
    return n;
}

IC_EXPORT ic_status ic_trace_read(const ic_trace *tr, float *us, char *names, int32_t n)
{
    if (!tr || !us)
        return fail(IC_ERR_NULL, "trace: trace and us are required");
    if (n < 0 || n > tr->recorded)
        return fail(IC_ERR_SHAPE, "trace: %d launches asked, %d recorded", n, tr->recorded);
    for (int32_t i = 0; i < n; ++i) {
        float ms = 0.0f;
        const hipError_t e = hipEventElapsedTime(&ms, tr->events[i], tr->events[i + 1]);
        if (e != hipSuccess)
            return fail(IC_ERR_HIP, "trace: launch %d: hipEventElapsedTime: %s", i, hipGetErrorString(e));
        us[i] = ms * 1000.0f;
        if (names)
            memcpy(names + (size_t)i * kTraceNameLen, tr->names[i].data(), kTraceNameLen);
    }
    return ok();
}

IC_EXPORT const char *ic_status_str(ic_status s)
{
    switch (s) {
    case IC_OK: return "IC_OK";
    case IC_ERR_NULL: return "IC_ERR_NULL";
    case IC_ERR_SHAPE: return "IC_ERR_SHAPE";
    case IC_ERR_UNSUPPORTED: return "IC_ERR_UNSUPPORTED";
    case IC_ERR_ALIGN: return "IC_ERR_ALIGN";
    case IC_ERR_WORKSPACE: return "IC_ERR_WORKSPACE";
    case IC_ERR_REUSE_MAP: return "IC_ERR_REUSE_MAP";
    case IC_ERR_HIP: return "IC_ERR_HIP";
    default: return "IC_ERR_UNKNOWN";
    }
}

IC_EXPORT const char *ic_last_error(void) { return g_last_error; }

IC_EXPORT ic_status ic_indexer_score(const uint8_t *q_idx, const float *w, const uint8_t *k_idx,
                                     const ic_queries *qs, int32_t H_I, int32_t D_I, float *scores, int64_t ld,
                                     void *stream)
{
    if (ic_status s = check_indexer(q_idx, w, k_idx, qs, H_I, D_I, scores, ld))
        return s;
    if (qs->T == 0 || qs->max_n == 0)
        return ok();
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    return hip_status(launch_indexer(q_idx, w, k_idx, qs, H_I, D_I, scores, ld, nullptr, st), "indexer launch");
}

IC_EXPORT size_t ic_topk_workspace_size(const ic_queries *qs, int32_t k)
{
    if (!qs || qs->T < 0)
        return 0;
    return ic::topk_workspace_bytes(qs->T, qs->max_n, k);
}

IC_EXPORT ic_status ic_topk(const float *scores, int64_t ld, const ic_queries *qs, int32_t k, int32_t *idx,
                            void *ws, size_t ws_bytes, void *stream)
{
    if (ic_status s = check_topk(scores, ld, qs, k, idx, ws, ws_bytes))
        return s;
    if (qs->T == 0)
        return ok();
    return hip_status(ic::launch_topk(scores, ld, qs->n_valid, qs->T, qs->max_n, k, idx, ws, false,
                                      reinterpret_cast<hipStream_t>(stream)),
                      "top-k launch");
}

IC_EXPORT size_t ic_sparse_mla_workspace_size(const ic_queries *qs, const ic_dims *d)
{
    if (!qs || !d || qs->T < 0 || d->H < 1 || d->k < 1)
        return 0;
    return ic::plan_sparse_mla(qs->T, d->H, d->k, d->D_v).ws_bytes;
}

IC_EXPORT ic_status ic_sparse_mla(const uint16_t *q, const uint16_t *kv, const ic_queries *qs, const int32_t *idx,
                                  const float *sink, float scale, const ic_dims *d, void *out, void *ws,
                                  size_t ws_bytes, void *stream)
{
    if (ic_status s = check_mla(q, kv, qs, idx, sink, d, out, ws, ws_bytes))
        return s;
    if (qs->T == 0)
        return ok();
    const ic::MlaPlan plan = ic::plan_sparse_mla(qs->T, d->H, d->k, d->D_v);
    return hip_status(ic::launch_sparse_mla(q, kv, qs->base, qs->n_valid, idx, qs->T, d->H, d->k, d->D_qk, d->D_v, sink, scale,
                                            out, d->out_dtype == IC_OUT_F32, plan, ws,
                                            reinterpret_cast<hipStream_t>(stream)),
                      "sparse MLA launch");
}

IC_EXPORT ic_status ic_gated_output(const uint16_t *o, const uint16_t *wv_b, const uint16_t *gate, int32_t T,
                                    int32_t H, int32_t D_v, int32_t D_o, uint16_t *out, void *stream)
{
    if (T < 0 || T > (1 << 20))
        return fail(IC_ERR_SHAPE, "gated output: T=%d outside [0, 2^20]", T);
    if (H < 1 || H > 4096)
        return fail(IC_ERR_SHAPE, "gated output: H=%d outside [1, 4096]", H);
    if (!ic::gated_output_supported(D_v, D_o))
        return fail(IC_ERR_UNSUPPORTED, "gated output: (D_v, D_o)=(%d, %d) not built; D_v in {512, 64}, D_o a "
                    "multiple of 64 in [64, 1024]", D_v, D_o);
    if (T == 0)
        return ok();
    if (!o || !wv_b || !gate || !out)
        return fail(IC_ERR_NULL, "gated output: o, wv_b, gate and out are required");
    if (!aligned16(o) || !aligned16(wv_b) || !aligned16(gate) || !aligned16(out))
        return fail(IC_ERR_ALIGN, "gated output: device pointers must be 16-byte aligned");
    return hip_status(ic::launch_gated_output(o, wv_b, gate, T, H, D_v, D_o, out,
                                              reinterpret_cast<hipStream_t>(stream)),
                      "gated output launch");
}

IC_EXPORT ic_status ic_write_cache(const ic_tokens *tk, const uint16_t *k_pre, const float *ln_w, const float *ln_b,
                                   float eps, int32_t D_I, uint8_t *k_idx, const uint16_t *kv_pre, int32_t D_qk,
                                   uint16_t *kv, void *stream)
{
    if (!tk)
        return fail(IC_ERR_NULL, "write cache: the tokens descriptor is required");
    if (tk->T < 0 || tk->T > (1 << 24))
        return fail(IC_ERR_SHAPE, "write cache: T=%d outside [0, 2^24]", tk->T);
    if (tk->rows < 1)
        return fail(IC_ERR_SHAPE, "write cache: rows=%lld must be >= 1", (long long)tk->rows);
    if (tk->reserved != 0)
        return fail(IC_ERR_SHAPE, "write cache: reserved field must be 0");
    if (tk->D_rope < 0 || tk->D_rope > 128 || (tk->D_rope & 1))
        return fail(IC_ERR_SHAPE, "write cache: D_rope=%d must be even and in [0, 128]", tk->D_rope);
    if (tk->T == 0)
        return ok();                                   // nothing to write
    const bool key = k_pre || ln_w || ln_b || k_idx;
    const bool lat = kv_pre || kv;
    if (!key && !lat)
        return fail(IC_ERR_NULL, "write cache: neither the key nor the latent row is given");
    if (key && (!k_pre || !ln_w || !ln_b || !k_idx))
        return fail(IC_ERR_NULL, "write cache: k_pre, ln_w, ln_b and k_idx go together");
    if (lat && (!kv_pre || !kv))
        return fail(IC_ERR_NULL, "write cache: kv_pre and kv go together");
    if (key) {
        if (D_I != 32 && D_I != 64 && D_I != 128)
            return fail(IC_ERR_UNSUPPORTED, "write cache: D_I=%d not built (32, 64, 128)", D_I);
        if (!(eps > 0.0f) || !std::isfinite(eps))
            return fail(IC_ERR_SHAPE, "write cache: eps must be finite and > 0");
        if (tk->key_rope && tk->D_rope > D_I)
            return fail(IC_ERR_SHAPE, "write cache: D_rope=%d exceeds D_I=%d", tk->D_rope, D_I);
    }
    if (lat && (D_qk < 8 || D_qk > 4096 || D_qk % 8 || tk->D_rope > D_qk || (D_qk - tk->D_rope) % 8))
        return fail(IC_ERR_UNSUPPORTED, "write cache: D_qk=%d with D_rope=%d not built (D_qk and D_qk - D_rope "
                    "multiples of 8, D_qk <= 4096)", D_qk, tk->D_rope);
    const bool rotates = tk->D_rope > 0 && (lat || tk->key_rope);
    if (rotates && (!tk->rope || tk->n_pos < 1))
        return fail(IC_ERR_NULL, "write cache: D_rope > 0 needs the rotary table (n_pos >= 1)");
    if (!tk->row || !tk->pos)
        return fail(IC_ERR_NULL, "write cache: row and pos are required");
    const void *ptrs[] = {tk->row, tk->pos, rotates ? tk->rope : nullptr, k_pre, ln_w, ln_b, k_idx, kv_pre, kv};
    for (const void *p : ptrs)
        if (p && !aligned16(p))
            return fail(IC_ERR_ALIGN, "write cache: device pointers must be 16-byte aligned");
    // a shared layer without key rotation reads no table: pass D_rope only where it is used
    const int32_t D_rope = rotates ? tk->D_rope : 0;
    return hip_status(ic::launch_write_cache(tk->row, tk->pos, tk->T, tk->rows, rotates ? tk->rope : nullptr,
                                             tk->n_pos, D_rope, key && tk->key_rope ? 1 : 0, key ? k_pre : nullptr,
                                             ln_w, ln_b, eps, D_I, k_idx, lat ? kv_pre : nullptr, D_qk, kv,
                                             reinterpret_cast<hipStream_t>(stream)),
                      "write cache launch");
}

IC_EXPORT ic_status ic_reuse_map_last_full(int32_t n_layers, const uint8_t *is_full, int32_t *reuse_map)
{
    if (n_layers < 1)
        return fail(IC_ERR_SHAPE, "n_layers=%d must be >= 1", n_layers);
    if (!is_full || !reuse_map)
        return fail(IC_ERR_NULL, "is_full and reuse_map are required");
    if (!is_full[0])
        return fail(IC_ERR_REUSE_MAP, "layer 0 must be a full layer");
    int32_t last = 0;
    for (int32_t l = 0; l < n_layers; ++l) {
        if (is_full[l])
            last = l;
        reuse_map[l] = last;
    }
    return ok();
}

IC_EXPORT size_t ic_layer_stack_workspace_size(const ic_queries *qs, const ic_dims *d)
{
    if (!qs || !d || qs->T < 0 || d->H < 1 || d->k < 1 || qs->max_n < 0)
        return 0;
    return stack_layout(qs, d).total;
}

IC_EXPORT ic_status ic_layer_stack(int32_t n_layers, const ic_layer *layers, const int32_t *reuse_map,
                                   const ic_queries *qs, const ic_dims *d, float scale, int32_t *index_cache,
                                   int32_t *indexer_passes, void *ws, size_t ws_bytes, void *stream)
{
    if (ic_status s = check_reuse_map(n_layers, reuse_map))
        return s;
    if (!layers)
        return fail(IC_ERR_NULL, "layers is NULL");
    if (ic_status s = check_queries(qs))
        return s;
    if (ic_status s = check_dims_mla(d))
        return s;
    int32_t n_full = 0;
    for (int32_t l = 0; l < n_layers; ++l)
        n_full += reuse_map[l] == l;
    if (qs->T > 0) {
        if (!index_cache)
            return fail(IC_ERR_NULL, "index_cache is NULL");
        if (!aligned16(index_cache))
            return fail(IC_ERR_ALIGN, "index_cache not 16-byte aligned");
        const StackLayout L = stack_layout(qs, d);
        if (!ws || ws_bytes < L.total)
            return fail(IC_ERR_WORKSPACE, "layer stack: workspace of %zu bytes required, %zu given", L.total,
                        ws_bytes);
        if (!aligned16(ws))
            return fail(IC_ERR_ALIGN, "layer stack: workspace not 16-byte aligned");
        for (int32_t l = 0; l < n_layers; ++l) {
            const ic_layer &y = layers[l];
            if (reuse_map[l] == l) {
                if (ic_status s = check_indexer(y.q_idx, y.w, y.k_idx, qs, d->H_I, d->D_I,
                                                reinterpret_cast<float *>(ws), L.ld)) {
                    char msg[512];
                    snprintf(msg, sizeof msg, "%s", g_last_error);
                    return fail(s, "layer %d: %s", l, msg);
                }
            }
            if (ic_status s = check_mla(y.q, y.kv, qs, index_cache, y.sink, d, y.out,
                                        static_cast<char *>(ws) + L.mla_off, ws_bytes - L.mla_off)) {
                char msg[512];
                snprintf(msg, sizeof msg, "%s", g_last_error);
                return fail(s, "layer %d: %s", l, msg);
            }
        }
    }
    if (indexer_passes)
        *indexer_passes = n_full;
    if (qs->T == 0)
        return ok();

    const StackLayout L = stack_layout(qs, d);
    float *scores = reinterpret_cast<float *>(static_cast<char *>(ws) + L.scores_off);
    void *topk_ws = static_cast<char *>(ws) + L.topk_off;
    void *mla_ws = static_cast<char *>(ws) + L.mla_off;
    const ic::MlaPlan plan = ic::plan_sparse_mla(qs->T, d->H, d->k, d->D_v);
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    // slot of a full layer = its rank among the full layers (counted where
    // needed: the call allocates nothing, host memory included)
    auto slot_of = [&](int32_t f) {
        int32_t r = 0;
        for (int32_t i = 0; i < f; ++i)
            r += reuse_map[i] == i;
        return r;
    };
    const size_t slot_elems = (size_t)qs->T * d->k;
    // When the top-k takes its split path and the MLA grid fits on the chip at
    // once, a full layer's MLA workgroups finish the selection themselves
    // from the split phase's collected keys (one launch and one round trip
    // fewer) and write the layer's index list for the shared layers.
    ic::TopkSplitView view{};
    const bool selecting = qs->max_n > 0 && ic::topk_split_view(topk_ws, qs->T, qs->max_n, &view) &&
                           ic::sparse_mla_selecting_supported(plan, qs->T, d->H, view);
    // the per-query key stream also fills the top-k's first-digit histogram
    // when the selection reads it; the workspace carries nothing from earlier
    // calls, so the histograms are cleared once here (the row kernel leaves
    // them clear for the next full layer)
    const bool fused_hist = qs->max_n > 0 && n_full > 0 && !use_prefill_indexer(qs, d->H_I, d->D_I) &&
                            ic::topk_reads_hist0(qs->T, qs->max_n);
    if (fused_hist) {
        hipError_t e = ic::launch_clear_hist0(topk_ws, qs->T, st);
        if (e != hipSuccess)
            return hip_status(e, "layer stack: histogram clear launch");
    }
    for (int32_t l = 0; l < n_layers; ++l) {
        const ic_layer &y = layers[l];
        const bool full = reuse_map[l] == l;
        if (full && L.col.on) {
            // bounded collection: sample scores, bounds, collection, selection;
            // then the score rows and the row top-k for the queries marked
            int32_t *idx = index_cache + slot_of(l) * slot_elems;
            char *w8 = static_cast<char *>(ws);
            const Collect &c = L.col;
            float *sample = reinterpret_cast<float *>(w8 + c.sample_off);
            uint32_t *bound = reinterpret_cast<uint32_t *>(w8 + c.bound_off);
            uint64_t *slices = reinterpret_cast<uint64_t *>(w8 + c.slices_off);
            uint32_t *counts = reinterpret_cast<uint32_t *>(w8 + c.counts_off);
            uint32_t *need = reinterpret_cast<uint32_t *>(w8 + c.need_off);
            hipError_t e = ic::launch_indexer_prefill_sample(y.q_idx, y.w, y.k_idx, qs->base, qs->n_valid, qs->T,
                                                             qs->max_n, sample, c.sample_ld, st);
            if (e == hipSuccess)
                e = ic::launch_prefill_bound(sample, c.sample_ld, qs->n_valid, qs->T, d->k, bound,
                                             prefill_collect_mode(qs, d) == 2, st);
            if (e == hipSuccess)
                e = ic::launch_indexer_prefill_collect(y.q_idx, y.w, y.k_idx, qs->base, qs->n_valid, qs->T,
                                                       qs->max_n, bound, slices, counts, c.cap, st);
            if (e == hipSuccess)
                e = ic::launch_prefill_select(slices, counts, (int32_t)c.nchunks, c.chunk, c.cap, qs->n_valid,
                                              qs->T, d->k, idx, need, st);
            if (e == hipSuccess)
                e = ic::launch_indexer_prefill(y.q_idx, y.w, y.k_idx, qs->base, qs->n_valid, qs->T, qs->max_n,
                                               d->H_I, d->D_I, 16, scores, L.ld, st, need);
            if (e == hipSuccess)
                e = ic::launch_topk(scores, L.ld, qs->n_valid, qs->T, qs->max_n, d->k, idx, topk_ws, false, st,
                                    need);
            if (e != hipSuccess)
                return hip_status(e, "layer stack: prefill indexer and top-k launches");
        } else if (full) {
            int32_t *idx = index_cache + slot_of(l) * slot_elems;
            if (qs->max_n > 0) {
                hipError_t e = launch_indexer(y.q_idx, y.w, y.k_idx, qs, d->H_I, d->D_I, scores, L.ld,
                                              fused_hist ? ic::topk_hist0(topk_ws) : nullptr, st);
                if (e != hipSuccess)
                    return hip_status(e, "layer stack: indexer launch");
            }
            hipError_t e = selecting ? ic::launch_topk_collect(scores, L.ld, qs->n_valid, qs->T, qs->max_n, d->k,
                                                               topk_ws, st)
                                     : ic::launch_topk(scores, L.ld, qs->n_valid, qs->T, qs->max_n, d->k, idx,
                                                       topk_ws, fused_hist, st);
            if (e != hipSuccess)
                return hip_status(e, "layer stack: top-k launch");
        }
        int32_t *idx = index_cache + slot_of(reuse_map[l]) * slot_elems;
        const int32_t f32 = d->out_dtype == IC_OUT_F32;
        hipError_t e = full && selecting
                           ? ic::launch_sparse_mla_selecting(y.q, y.kv, qs->base, qs->n_valid, qs->T, d->H, d->k,
                                                             d->D_qk, d->D_v, y.sink, scale, y.out, f32, plan, mla_ws,
                                                             scores, L.ld, view, idx, st)
                           : ic::launch_sparse_mla(y.q, y.kv, qs->base, qs->n_valid, idx, qs->T, d->H, d->k, d->D_qk,
                                                   d->D_v, y.sink, scale, y.out, f32, plan, mla_ws, st);
        if (e != hipSuccess)
            return hip_status(e, "layer stack: sparse MLA launch");
    }
    return ok();
}

IC_EXPORT ic_status ic_layer_stack_static(int32_t n_layers, const ic_layer *layers, const int32_t *reuse_map,
                                          const ic_queries *qs, const ic_dims *d, float scale,
                                          int32_t *index_cache, int32_t *indexer_passes, void *stream)
{
    if (ic_status s = check_reuse_map(n_layers, reuse_map))
        return s;
    if (ic_status s = check_queries(qs))
        return s;
    if (ic_status s = check_dims_mla(d))
        return s;
    const size_t need = qs->T > 0 ? stack_layout(qs, d).total : 0;
    if (need > kScratchBytes)
        return fail(IC_ERR_WORKSPACE,
                    "static layer stack: these sizes need %zu bytes of scratch, beyond the library's %zu; "
                    "use ic_layer_stack with a workspace", need, kScratchBytes);
    void *ws = nullptr;
    if (qs->T > 0)
        if (ic_status s = scratch_address(&ws))
            return s;
    return ic_layer_stack(n_layers, layers, reuse_map, qs, d, scale, index_cache, indexer_passes, ws,
                          qs->T > 0 ? kScratchBytes : 0, stream);
}
