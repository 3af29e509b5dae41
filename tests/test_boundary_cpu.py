"""The C-ABI library on the CPU: it loads, exports every entry point that
include/ic.h declares, and its host-side validation rejects bad arguments
before anything is launched. Nothing here enqueues GPU work: every call either
fails validation or has T = 0."""
import ctypes
import os
import re

import pytest
import torch

from cross_layer_index_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def ic():
    from cross_layer_index_amd import ic as m
    return m


def declared_entry_points():
    src = open(os.path.join(ROOT, "include", "ic.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ic_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_symbol(ic):
    names = declared_entry_points()
    assert len(names) == 20
    for n in names:
        assert hasattr(ic._lib, n), n
    assert sorted(ic.EXPORTED) == names


def test_status_strings(ic):
    assert ic._lib.ic_status_str(0) == b"IC_OK"
    assert ic._lib.ic_status_str(6) == b"IC_ERR_REUSE_MAP"
    assert ic._lib.ic_status_str(99) == b"IC_ERR_UNKNOWN"


FAKE = 0x100000   # an aligned non-null address; never dereferenced: validation fails first


def Q(ic, T=1, max_n=16, rows=16, base=FAKE, n=FAKE):
    return ic.ic_queries(base, n, T, 0, max_n, rows)


def call_indexer(ic, qs, H_I=64, D_I=128, ld=16, q=FAKE, w=FAKE, k=FAKE, s=FAKE):
    return ic._lib.ic_indexer_score(q, w, k, ctypes.byref(qs) if qs is not None else None, H_I, D_I, s, ld, None)


def test_indexer_validation(ic):
    assert call_indexer(ic, None) == ic.IC_ERR_NULL
    assert call_indexer(ic, Q(ic), q=None) == ic.IC_ERR_NULL
    assert call_indexer(ic, Q(ic), D_I=96) == ic.IC_ERR_UNSUPPORTED
    assert call_indexer(ic, Q(ic), H_I=65) == ic.IC_ERR_UNSUPPORTED
    assert call_indexer(ic, Q(ic), ld=8) == ic.IC_ERR_SHAPE          # ld < max_n
    assert call_indexer(ic, Q(ic, max_n=16), ld=18) == ic.IC_ERR_SHAPE  # ld not a multiple of 4
    assert call_indexer(ic, Q(ic), k=FAKE + 4) == ic.IC_ERR_ALIGN
    assert call_indexer(ic, Q(ic, T=-1)) == ic.IC_ERR_SHAPE
    assert call_indexer(ic, Q(ic, T=70000)) == ic.IC_ERR_SHAPE
    assert call_indexer(ic, Q(ic, max_n=32, rows=16), ld=32) == ic.IC_ERR_SHAPE   # more tokens than rows
    assert b"D_I" in ic._lib.ic_last_error() or True
    assert call_indexer(ic, Q(ic, T=0)) == ic.IC_OK                  # nothing to do, nothing launched


def test_query_group_validation(ic):
    """Draft/verify groups: T must be a multiple of the group size, the group
    is non-negative and the reserved field zero; rejected before any launch."""
    def G(group, T=4, reserved=0):
        q = Q(ic, T=T)
        q.group, q.reserved = group, reserved
        return q
    assert call_indexer(ic, G(-1)) == ic.IC_ERR_SHAPE
    assert call_indexer(ic, G(3, T=4)) == ic.IC_ERR_SHAPE          # 4 queries are not groups of 3
    assert call_indexer(ic, G(2, reserved=1)) == ic.IC_ERR_SHAPE
    assert call_indexer(ic, G(3, T=0)) == ic.IC_OK                  # no queries: nothing to check


def test_topk_validation(ic):
    qs = Q(ic)
    f = ic._lib.ic_topk
    assert f(FAKE, 16, ctypes.byref(qs), 0, FAKE, None, 0, None) == ic.IC_ERR_SHAPE
    assert f(None, 16, ctypes.byref(qs), 8, FAKE, None, 0, None) == ic.IC_ERR_NULL
    assert f(FAKE, 6, ctypes.byref(qs), 8, FAKE, None, 0, None) == ic.IC_ERR_SHAPE
    assert f(FAKE + 8, 16, ctypes.byref(qs), 8, FAKE, None, 0, None) == ic.IC_ERR_ALIGN
    assert f(FAKE, 16, ctypes.byref(Q(ic, T=0)), 8, None, None, 0, None) == ic.IC_OK


def test_mla_validation(ic):
    qs = Q(ic)
    f = ic._lib.ic_sparse_mla
    good = ic.dims(64, 128, 2048, 128, 576, 512)
    bad_shape = ic.dims(64, 128, 2048, 128, 512, 512)
    assert f(FAKE, FAKE, ctypes.byref(qs), FAKE, FAKE, 0.1, ctypes.byref(bad_shape), FAKE, None, 0, None) \
        == ic.IC_ERR_UNSUPPORTED
    assert f(FAKE, FAKE, ctypes.byref(qs), FAKE, FAKE, 0.1, None, FAKE, None, 0, None) == ic.IC_ERR_NULL
    assert f(FAKE, FAKE, ctypes.byref(qs), FAKE, None, 0.1, ctypes.byref(good), FAKE, None, 0, None) \
        == ic.IC_ERR_NULL
    bad_out = ic.dims(64, 128, 2048, 128, 576, 512)
    bad_out.out_dtype = 7
    assert f(FAKE, FAKE, ctypes.byref(qs), FAKE, FAKE, 0.1, ctypes.byref(bad_out), FAKE, None, 0, None) \
        == ic.IC_ERR_SHAPE
    # batch 1 at k = 2048 splits the index list: a workspace is required
    need = ic._lib.ic_sparse_mla_workspace_size(ctypes.byref(qs), ctypes.byref(good))
    assert need > 0
    assert f(FAKE, FAKE, ctypes.byref(qs), FAKE, FAKE, 0.1, ctypes.byref(good), FAKE, None, 0, None) \
        == ic.IC_ERR_WORKSPACE
    assert f(FAKE, FAKE, ctypes.byref(qs), FAKE, FAKE, 0.1, ctypes.byref(good), FAKE, FAKE, need - 1, None) \
        == ic.IC_ERR_WORKSPACE


def test_mla_rejects_lists_beyond_the_combine(ic):
    """The split combine merges at most 256 splits of 2048 entries: an index
    list of 524,289 entries is rejected before any launch (it would need 257
    splits), 524,288 passes validation up to the workspace check."""
    qs = Q(ic, max_n=1 << 20, rows=1 << 20)
    f = ic._lib.ic_sparse_mla
    over = ic.dims(64, 128, 524289, 128, 576, 512)
    assert f(FAKE, FAKE, ctypes.byref(qs), FAKE, FAKE, 0.1, ctypes.byref(over), FAKE, FAKE, 1 << 40, None) \
        == ic.IC_ERR_UNSUPPORTED
    assert b"524289" in ic._lib.ic_last_error()
    edge = ic.dims(64, 128, 524288, 128, 576, 512)
    assert f(FAKE, FAKE, ctypes.byref(qs), FAKE, FAKE, 0.1, ctypes.byref(edge), FAKE, None, 0, None) \
        == ic.IC_ERR_WORKSPACE
    stack = ic._lib.ic_layer_stack
    lay = (ic.ic_layer * 1)(ic.ic_layer(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE))
    rmap = (ctypes.c_int32 * 1)(0)
    assert stack(1, lay, rmap, ctypes.byref(qs), ctypes.byref(over), 0.1, FAKE, None, FAKE, 1 << 40, None) \
        == ic.IC_ERR_UNSUPPORTED


def test_static_stack_rejects_oversized_workspace(ic):
    """ic_layer_stack_static serves sizes whose workspace fits its 32 MiB
    scratch; larger ones (64 queries over 64K tokens) fail with
    IC_ERR_WORKSPACE before anything is launched or looked up."""
    qs = Q(ic, T=64, max_n=65536, rows=64 * 65536)
    d = ic.dims(64, 128, 2048, 128, 576, 512)
    assert ic._lib.ic_layer_stack_workspace_size(ctypes.byref(qs), ctypes.byref(d)) > (32 << 20)
    lay = (ic.ic_layer * 1)(ic.ic_layer(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE))
    rmap = (ctypes.c_int32 * 1)(0)
    st = ic._lib.ic_layer_stack_static(1, lay, rmap, ctypes.byref(qs), ctypes.byref(d), 0.1, FAKE, None, None)
    assert st == ic.IC_ERR_WORKSPACE
    assert b"32" in ic._lib.ic_last_error() or b"33554432" in ic._lib.ic_last_error()
    bad = (ctypes.c_int32 * 2)(1, 1)
    assert ic._lib.ic_layer_stack_static(2, lay, bad, ctypes.byref(qs), ctypes.byref(d), 0.1, FAKE, None, None) \
        == ic.IC_ERR_REUSE_MAP


def test_stream_read_validation(ic):
    """The calibration read rejects sizes that are not whole 16-byte vectors
    and null or misaligned pointers before any launch; zero bytes is a no-op."""
    f = ic._lib.ic_stream_read
    assert f(FAKE, 24, FAKE, None) == ic.IC_ERR_SHAPE
    assert f(FAKE, -16, FAKE, None) == ic.IC_ERR_SHAPE
    assert f(None, 32, FAKE, None) == ic.IC_ERR_NULL
    assert f(FAKE + 8, 32, FAKE, None) == ic.IC_ERR_ALIGN
    assert f(None, 0, None, None) == ic.IC_OK


def test_reuse_map_matches_oracle_rule(ic):
    import oracle
    for pattern in (W.WORKLOADS["stack_78"].is_full(), [True] * 78, [True] + [False] * 77,
                    [l % 6 == 0 for l in range(78)], [True, False, True, True, False]):
        assert ic.reuse_map_last_full(pattern) == oracle.reuse_map_last_full(pattern)
    with pytest.raises(ic.ICError) as e:
        ic.reuse_map_last_full([False, True])
    assert e.value.status == ic.IC_ERR_REUSE_MAP


def stack_call(ic, rmap, T=0):
    n = len(rmap)
    layers = (ic.ic_layer * n)()
    m = (ctypes.c_int32 * n)(*rmap)
    qs = Q(ic, T=T)
    d = ic.dims(64, 128, 2048, 128, 576, 512)
    passes = ctypes.c_int32(-1)
    st = ic._lib.ic_layer_stack(n, layers, m, ctypes.byref(qs), ctypes.byref(d), 0.04, None,
                                ctypes.byref(passes), None, 0, None)
    return st, passes.value


def test_layer_stack_counts_indexer_passes(ic):
    """Through the C ABI with no queries: the pass counter reproduces the
    explainer's per-token index-build counts (78, 1, 13) and the issue's 21."""
    for pattern, want in ((W.WORKLOADS["stack_78"].is_full(), 21), ([True] * 78, 78),
                          ([True] + [False] * 77, 1), ([l % 6 == 0 for l in range(78)], 13)):
        st, passes = stack_call(ic, ic.reuse_map_last_full(pattern))
        assert st == ic.IC_OK and passes == want


@pytest.mark.parametrize("bad", [[1, 1], [0, 2, 2], [0, 0, 1], [0, 1, 1, 2], [0, -1]])
def test_layer_stack_rejects_bad_maps(ic, bad):
    st, passes = stack_call(ic, bad)
    assert st == ic.IC_ERR_REUSE_MAP and passes == -1


def test_layer_stack_needs_workspace_and_cache(ic):
    st, _ = stack_call(ic, [0, 0], T=1)
    assert st == ic.IC_ERR_NULL     # index_cache missing


def test_binding_rejects_short_caches():
    """The library sees pointers only; the binding checks every tensor's shape
    against the query descriptor before any launch (a cache drawn for other
    lengths than the descriptor's must never reach a kernel)."""
    from cross_layer_index_amd import ic
    kv = torch.empty((100, 576), dtype=torch.bfloat16)
    ic._shape(kv, ((">=", 100), 576), "kv")
    ic._shape(kv, ((">=", 99), 576), "kv")
    with pytest.raises(ValueError):
        ic._shape(kv, ((">=", 101), 576), "kv")
    with pytest.raises(ValueError):
        ic._shape(kv, ((">=", 100), 512), "kv")
    with pytest.raises(ValueError):
        ic._shape(kv[0], ((">=", 1), 576), "kv")


def test_variant_draws_keep_geometry():
    """Input sets drawn with another variant share the workload's lengths and
    row count and differ in values."""
    wl = W.scaled(W.WORKLOADS["ragged_64"], T=5, len_range=(10, 300))
    a = W.layer_inputs(wl, 0)
    b = W.layer_inputs(wl, 0, variant=3)
    for f in ("q_idx", "w", "k_idx", "q", "kv", "sink"):
        x, y = getattr(a, f), getattr(b, f)
        assert x.shape == y.shape and x.dtype == y.dtype
    assert not torch.equal(a.kv, b.kv) and not torch.equal(a.k_idx, b.k_idx)
    assert a.kv.shape[0] == wl.rows()


def test_reuse_patterns_match_the_pages_counts(orc):
    """The full-layer sets the reuse-pattern measurement compares give the
    index-build counts the pages print (tests/golden/index_score_counts.txt),
    and under each of them every shared layer reads the last full layer
    before it (library and oracle agree)."""
    from cross_layer_index_amd import ic
    golden = {}
    for line in open(os.path.join(os.path.dirname(__file__), "golden", "index_score_counts.txt")):
        if line.strip() and not line.startswith("#"):
            k, v = line.split()
            golden[k] = v
    L = int(golden["layers"])
    want = {"hy4_21": int(golden["hy4_full_layers"]), "every6_13": int(golden["refresh_every_index_builds"]),
            "first_only_1": 1, "all_78": L}
    assert set(W.REUSE_PATTERNS) == set(want)
    for name, fl in W.REUSE_PATTERNS.items():
        flags = [l in set(fl) for l in range(L)]
        assert sum(flags) == want[name], name
        m = ic.reuse_map_last_full(flags)
        assert m == orc.reuse_map_last_full(flags)
        for l in range(L):
            assert m[l] == max(f for f in fl if f <= l)
    assert "".join("F" if l in set(W.REUSE_PATTERNS["hy4_21"]) else "S" for l in range(6)) == \
        golden["hy4_pattern_prefix"]


def test_gated_output_validation(ic):
    f = ic._lib.ic_gated_output
    assert f(FAKE, FAKE, FAKE, -1, 128, 512, 128, FAKE, None) == ic.IC_ERR_SHAPE
    assert f(FAKE, FAKE, FAKE, 1, 0, 512, 128, FAKE, None) == ic.IC_ERR_SHAPE
    assert f(FAKE, FAKE, FAKE, 1, 128, 576, 128, FAKE, None) == ic.IC_ERR_UNSUPPORTED
    assert f(FAKE, FAKE, FAKE, 1, 128, 512, 96, FAKE, None) == ic.IC_ERR_UNSUPPORTED
    assert f(None, FAKE, FAKE, 1, 128, 512, 128, FAKE, None) == ic.IC_ERR_NULL
    assert f(FAKE, FAKE + 4, FAKE, 1, 128, 512, 128, FAKE, None) == ic.IC_ERR_ALIGN
    assert f(None, None, None, 0, 128, 512, 128, None, None) == ic.IC_OK          # nothing to do


def test_write_cache_validation(ic):
    f = ic._lib.ic_write_cache

    def tk(T=4, D_rope=64, rows=100, rope=FAKE, n_pos=10, key_rope=1, reserved=0, row=FAKE, pos=FAKE):
        return ctypes.byref(ic.ic_tokens(row, pos, T, D_rope, rows, rope, n_pos, key_rope, reserved))

    key = (FAKE, FAKE, FAKE, 1e-6, 128, FAKE)
    lat = (FAKE, 576, FAKE)
    assert f(None, *key, *lat, None) == ic.IC_ERR_NULL
    assert f(tk(T=0, row=None, pos=None), None, None, None, 1e-6, 128, None, None, 576, None, None) == ic.IC_OK
    assert f(tk(T=-1), *key, *lat, None) == ic.IC_ERR_SHAPE
    assert f(tk(rows=0), *key, *lat, None) == ic.IC_ERR_SHAPE
    assert f(tk(reserved=1), *key, *lat, None) == ic.IC_ERR_SHAPE
    assert f(tk(D_rope=63), *key, *lat, None) == ic.IC_ERR_SHAPE
    assert f(tk(D_rope=130), *key, *lat, None) == ic.IC_ERR_SHAPE
    assert f(tk(), None, None, None, 1e-6, 128, None, None, 576, None, None) == ic.IC_ERR_NULL  # nothing
    assert f(tk(), FAKE, None, FAKE, 1e-6, 128, FAKE, *lat, None) == ic.IC_ERR_NULL             # ln_w missing
    assert f(tk(), *key, FAKE, 576, None, None) == ic.IC_ERR_NULL                              # kv missing
    assert f(tk(), FAKE, FAKE, FAKE, 1e-6, 96, FAKE, *lat, None) == ic.IC_ERR_UNSUPPORTED
    assert f(tk(), FAKE, FAKE, FAKE, 0.0, 128, FAKE, *lat, None) == ic.IC_ERR_SHAPE
    assert f(tk(), FAKE, FAKE, FAKE, float("nan"), 128, FAKE, *lat, None) == ic.IC_ERR_SHAPE
    assert f(tk(D_rope=64), FAKE, FAKE, FAKE, 1e-6, 32, FAKE, None, 0, None, None) == ic.IC_ERR_SHAPE
    assert f(tk(), *key, FAKE, 572, FAKE, None) == ic.IC_ERR_UNSUPPORTED
    assert f(tk(D_rope=60), *key, FAKE, 576, FAKE, None) == ic.IC_ERR_UNSUPPORTED             # 516 not % 8
    assert f(tk(rope=None), *key, *lat, None) == ic.IC_ERR_NULL
    assert f(tk(n_pos=0), *key, *lat, None) == ic.IC_ERR_NULL
    assert f(tk(row=None), *key, *lat, None) == ic.IC_ERR_NULL
    assert f(tk(row=FAKE + 8), *key, *lat, None) == ic.IC_ERR_ALIGN
    assert f(tk(), FAKE, FAKE, FAKE, 1e-6, 128, FAKE, FAKE + 2, 576, FAKE, None) == ic.IC_ERR_ALIGN
    assert f(tk(T=0, row=None, pos=None), *key, *lat, None) == ic.IC_OK                        # nothing to do
    # a key without rotation reads no table
    assert f(tk(T=3, rope=None, n_pos=0, key_rope=0, row=FAKE + 1), *key, None, 0, None, None) == ic.IC_ERR_ALIGN


def test_prefill_collection_workspace(ic, monkeypatch):
    """Causal prefill of at least 256 queries over rows of at least 65,536
    tokens selects from a bounded collection of the scores: its workspace
    adds the sample scores, bounds, survivor slices and marks to the score
    rows (kept for queries the collection cannot serve). Shorter rows, fewer
    queries, queries that do not share one sequence, and IC_PREFILL_TOPK=scores
    keep the plain layout; IC_PREFILL_TOPK=collect or =fallback takes the
    collection at any length."""
    d = ic.dims(64, 128, 2048, 128, 576, 512)
    size = lambda qs: ic._lib.ic_layer_stack_workspace_size(ctypes.byref(qs), ctypes.byref(d))

    def prefill(T, n):
        return ic.ic_queries(FAKE, FAKE, T, 1, n, n)

    monkeypatch.delenv("IC_PREFILL_TOPK", raising=False)
    long_, short = prefill(4096, 1 << 20), prefill(4096, 65535)
    plain = {}
    monkeypatch.setenv("IC_PREFILL_TOPK", "scores")
    for name, qs in (("long", long_), ("short", short)):
        plain[name] = size(qs)
    monkeypatch.delenv("IC_PREFILL_TOPK")
    assert size(short) == plain["short"]
    extra = size(long_) - plain["long"]
    T, n = 4096, 1 << 20
    sample = T * ((n + 63) // 64) * 4              # one key in 64, fp32
    assert extra > sample + 2 * T * 4              # sample scores, bounds, marks and the slices
    # slices: per chunk twice its expected share of the survivors plus 64,
    # rounded to 64 entries: a few times the ~2k + 1024 expected per query
    assert extra < sample + T * 8 * (2 * 2048 + 16 * 64) * 8
    monkeypatch.setenv("IC_PREFILL_TOPK", "scores")
    few_plain = size(prefill(255, 1 << 20))
    own = ic.ic_queries(FAKE, FAKE, 4096, 0, 1 << 20, 4096 << 20)   # every query its own cache
    own_plain = size(own)
    monkeypatch.setenv("IC_PREFILL_TOPK", "collect")
    assert size(prefill(255, 1 << 20)) == few_plain   # fewer than 256 queries: never collects
    assert size(own) == own_plain                      # no shared sequence: never collects
    forced = size(short)
    assert forced > plain["short"]                     # collects at any length when asked
    monkeypatch.setenv("IC_PREFILL_TOPK", "fallback")
    assert size(short) == forced
