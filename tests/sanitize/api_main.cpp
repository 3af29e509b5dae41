// Host-side exercise of the C ABI's validation and planning code, built with
// AddressSanitizer and UndefinedBehaviorSanitizer on the host side only (no
// device code is built, and no call here passes validation: nothing ever
// reaches a launch, whatever device is or is not present).
// Exit status 0 when every expectation holds; a sanitizer report aborts.
#include <cstdio>
#include <cstdint>
#include <cstring>
#include <initializer_list>

#include "ic.h"

static int failures = 0;

static void expect(bool ok, const char *what)
{
    if (!ok) {
        std::printf("FAIL: %s (last error: %s)\n", what, ic_last_error());
        ++failures;
    }
}

static void expect_status(ic_status got, ic_status want, const char *what)
{
    if (got != want) {
        std::printf("FAIL: %s: got %d (%s), want %d (%s); last error: %s\n", what, got, ic_status_str(got), want,
                    ic_status_str(want), ic_last_error());
        ++failures;
    }
}

int main()
{
    // status strings, including codes outside the enum
    for (int s = -2; s < 12; ++s)
        expect(ic_status_str(s) != nullptr && std::strlen(ic_status_str(s)) > 0, "status string");

    // fake, aligned, never-dereferenced device addresses
    auto dev = [](uintptr_t a) { return reinterpret_cast<void *>(a << 8); };
    const int64_t *base = static_cast<const int64_t *>(dev(1));
    const int32_t *n_valid = static_cast<const int32_t *>(dev(2));

    ic_queries dec{base, n_valid, 1, 0, 131072, 131072, 0, 0};
    ic_queries rag{base, n_valid, 64, 0, 65536, 64 * 65536, 0, 0};
    ic_queries pre{base, n_valid, 4096, 1, 1048576, 1048576, 0, 0};
    ic_queries grp{base, n_valid, 32, 0, 131072, 8 * 131072, 4, 0};
    ic_dims mla{64, 128, 2048, 128, 576, 512, IC_OUT_BF16};
    ic_dims tiny{4, 32, 64, 4, 80, 64, IC_OUT_F32};

    // planning: workspace sizes over the workloads' shapes
    for (const ic_queries *q : {&dec, &rag, &pre, &grp}) {
        expect(ic_topk_workspace_size(q, 2048) > 0, "top-k workspace");
        expect(ic_sparse_mla_workspace_size(q, &mla) > 0 || q == &pre, "MLA workspace");
        expect(ic_layer_stack_workspace_size(q, &mla) > 0, "stack workspace");
        (void)ic_sparse_mla_workspace_size(q, &tiny);
        (void)ic_layer_stack_workspace_size(q, &tiny);
    }
    // sizes that the calls reject plan to zero or to a finite size, never trap
    ic_dims huge = mla;
    huge.k = 1 << 20;
    (void)ic_sparse_mla_workspace_size(&dec, &huge);
    (void)ic_layer_stack_workspace_size(&dec, &huge);
    (void)ic_topk_workspace_size(&dec, 0);
    (void)ic_topk_workspace_size(&dec, -5);

    // validation failures of every entry point
    float *scores = static_cast<float *>(dev(3));
    int32_t *idx = static_cast<int32_t *>(dev(4));
    void *ws = dev(5);
    expect_status(ic_indexer_score(nullptr, nullptr, nullptr, &dec, 64, 128, scores, 131072, nullptr), IC_ERR_NULL,
                  "indexer NULL");
    expect_status(ic_indexer_score(static_cast<uint8_t *>(dev(6)), scores, static_cast<uint8_t *>(dev(7)), &dec,
                                   64, 48, scores, 131072, nullptr),
                  IC_ERR_UNSUPPORTED, "indexer D_I=48");
    expect_status(ic_indexer_score(static_cast<uint8_t *>(dev(6)), scores, static_cast<uint8_t *>(dev(7)), &dec,
                                   64, 128, scores, 131071, nullptr),
                  IC_ERR_SHAPE, "indexer ld below max_n");
    ic_queries bad = dec;
    bad.reserved = 1;
    expect_status(ic_topk(scores, 131072, &bad, 2048, idx, ws, 1 << 20, nullptr), IC_ERR_SHAPE, "reserved field");
    bad = grp;
    bad.T = 30;
    expect_status(ic_topk(scores, 131072, &bad, 2048, idx, ws, 1 << 20, nullptr), IC_ERR_SHAPE, "group");
    expect_status(ic_topk(scores, 131072, &dec, 0, idx, ws, 1 << 20, nullptr), IC_ERR_SHAPE, "top-k k=0");
    expect_status(ic_topk(scores, 131072, &dec, 2048, idx, ws, 16, nullptr), IC_ERR_WORKSPACE, "top-k workspace");
    expect_status(ic_topk(scores, 131072, &dec, 2048, idx, nullptr, 0, nullptr), IC_ERR_WORKSPACE,
                  "top-k no workspace");
    ic_dims odd = mla;
    odd.D_qk = 600;
    expect_status(ic_sparse_mla(static_cast<uint16_t *>(dev(8)), static_cast<uint16_t *>(dev(9)), &dec, idx,
                                scores, 0.04f, &odd, dev(10), ws, 1 << 30, nullptr),
                  IC_ERR_UNSUPPORTED, "MLA shape");
    expect_status(ic_sparse_mla(static_cast<uint16_t *>(dev(8)), static_cast<uint16_t *>(dev(9)), &dec, idx,
                                scores, 0.04f, &huge, dev(10), ws, 1 << 30, nullptr),
                  IC_ERR_UNSUPPORTED, "MLA k beyond the combine");
    odd = mla;
    odd.out_dtype = 7;
    expect_status(ic_sparse_mla(static_cast<uint16_t *>(dev(8)), static_cast<uint16_t *>(dev(9)), &dec, idx,
                                scores, 0.04f, &odd, dev(10), ws, 1 << 30, nullptr),
                  IC_ERR_SHAPE, "MLA out dtype");
    expect_status(ic_gated_output(nullptr, nullptr, nullptr, 1, 128, 512, 128, nullptr, nullptr), IC_ERR_NULL,
                  "gate NULL");
    ic_tokens tk{static_cast<int64_t *>(dev(11)), static_cast<int32_t *>(dev(12)), 4, 3, 100, scores, 10, 1, 0};
    expect_status(ic_write_cache(&tk, static_cast<uint16_t *>(dev(13)), scores, scores, 1e-6f, 128,
                                 static_cast<uint8_t *>(dev(14)), static_cast<uint16_t *>(dev(15)), 576,
                                 static_cast<uint16_t *>(dev(16)), nullptr),
                  IC_ERR_SHAPE, "write: odd D_rope");

    // reuse maps
    uint8_t full[78];
    int32_t rmap[78];
    for (int l = 0; l < 78; ++l)
        full[l] = (l < 3 || (l - 2) % 4 == 0) ? 1 : 0;
    expect_status(ic_reuse_map_last_full(78, full, rmap), IC_OK, "reuse map");
    int nf = 0;
    for (int l = 0; l < 78; ++l) {
        nf += rmap[l] == l;
        expect(rmap[l] <= l && full[rmap[l]], "reuse map points at a full layer at or before");
    }
    expect(nf == 21, "21 full layers");
    full[0] = 0;
    expect_status(ic_reuse_map_last_full(78, full, rmap), IC_ERR_REUSE_MAP, "first layer shared");
    expect_status(ic_reuse_map_last_full(0, full, rmap), IC_ERR_SHAPE, "no layers");

    // the stack rejects a map that violates the rule before anything else
    ic_layer lay[3];
    for (auto &y : lay)
        y = ic_layer{static_cast<uint8_t *>(dev(20)), scores, static_cast<uint8_t *>(dev(21)),
                     static_cast<uint16_t *>(dev(22)), static_cast<uint16_t *>(dev(23)), scores, dev(24)};
    int32_t passes = -1;
    int32_t badmap[3] = {0, 2, 1};
    expect_status(ic_layer_stack(3, lay, badmap, &dec, &mla, 0.04f, idx, &passes, ws, 1 << 30, nullptr),
                  IC_ERR_REUSE_MAP, "stack map");
    int32_t okmap[3] = {0, 0, 0};
    expect_status(ic_layer_stack(3, lay, okmap, &dec, &mla, 0.04f, idx, &passes, ws, 16, nullptr),
                  IC_ERR_WORKSPACE, "stack workspace");
    expect_status(ic_layer_stack_static(3, lay, okmap, &pre, &huge, 0.04f, idx, &passes, nullptr),
                  IC_ERR_UNSUPPORTED, "static stack beyond its scratch");

    // tracing and the calibration read
    ic_trace *tr = nullptr;
    expect_status(ic_trace_create(0, &tr), IC_ERR_SHAPE, "trace capacity 0");
    expect_status(ic_trace_create(4, nullptr), IC_ERR_NULL, "trace NULL out");
    expect_status(ic_trace_read(nullptr, nullptr, nullptr, 0), IC_ERR_NULL, "trace read NULL");
    ic_trace_destroy(nullptr);
    expect_status(ic_trace_skip("sparse_mla_kernel"), IC_OK, "skip set");
    expect_status(ic_trace_skip(nullptr), IC_OK, "skip cleared");
    expect(ic_trace_stop() == 0, "no trace running");
    expect_status(ic_stream_read(nullptr, 1 << 20, nullptr, nullptr), IC_ERR_NULL, "stream read NULL");
    expect_status(ic_stream_read(dev(30), 1000, static_cast<uint32_t *>(dev(31)), nullptr), IC_ERR_SHAPE,
                  "stream read size");

    std::printf("%s: %d failure(s)\n", failures ? "FAILED" : "ok", failures);
    return failures ? 1 : 0;
}
