"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Integer work (scores of integer-valued fp8 inputs, top-k index sets) must match
bit for bit; attention outputs must be within max-abs 5e-3 of the oracle's
fp64 result. Inputs come from the seeded generator only."""
import ctypes
import math
import sys

import numpy as np
import pytest
import torch

from checks import check_topk_invariants, report
from cross_layer_index_amd import workloads as W

pytestmark = pytest.mark.gpu
ATOL = 5e-3


def max_abs(got, ref):
    return float(np.abs(got - ref).max()) if np.size(ref) else 0.0


def assert_close(got, ref, what=""):
    """Max-abs error within the flat 5e-3 bar, whatever the output type."""
    err = max_abs(got, ref)
    report(what, err)
    assert err <= ATOL, f"{what} max abs error {err:.3e} > {ATOL}"


def bf16_rne(x):
    """Round to the nearest bf16 value, ties to even (torch's cast)."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).float().numpy()


def assert_bf16_output(got_bf16, got_f32, ref, what=""):
    """A bf16 output: bit for bit the round-to-nearest-even image of the fp32
    output of the same launch (which assert_close holds to 5e-3), and itself
    within the flat 5e-3 wherever the format can hold the exact value: when
    some exact value lies more than 2.5e-3 from every bf16 number (|o| >= 1
    in the single-key edge cases, where o = v * sigmoid(s - sink)), no bf16
    output can meet 5e-3 there and the fp32 check carries the bar."""
    assert np.array_equal(got_bf16, bf16_rne(got_f32)), f"{what}: bf16 output is not the rounded fp32 output"
    fmt = max_abs(bf16_rne(ref), ref)
    if fmt <= ATOL / 2:
        assert_close(got_bf16, ref, what + " [bf16]")
    else:
        report(what + f" [bf16; format rounding alone {fmt:.3e}, bar carried by fp32]", max_abs(got_bf16, ref))


def dev(li):
    return W.LayerInputs(*[None if x is None else x.cuda() for x in (li.q_idx, li.w, li.k_idx, li.q, li.kv,
                                                                       li.sink)])


def qs_of(ic, wl):
    return ic.make_queries(wl.base(), wl.n_valid(), wl.rows(), wl.same_seq, group=wl.group)


SMALL = {
    "tiny": W.WORKLOADS["tiny_2layer"],
    "decode_5000": W.scaled(W.WORKLOADS["decode_128k"], lengths=[5000]),
    "ragged": W.scaled(W.WORKLOADS["ragged_64"], T=6, len_range=(1, 3000)),
    "edges": W.scaled(W.WORKLOADS["edge_lengths"], T=8, lengths=[0, 1, 31, 33, 255, 257, 700, 2049]),
    "hi40_di64": W.scaled(W.WORKLOADS["decode_128k"], H_I=40, D_I=64, T=3, lengths=[1000, 77, 1300]),
    "di32_hi64": W.scaled(W.WORKLOADS["decode_128k"], H_I=64, D_I=32, T=2, lengths=[513, 999]),
    # causal prefill over one shared cache (the key-sharing kernel)
    "prefill_tail": W.scaled(W.WORKLOADS["prefill_1m"], T=37, prefill_first_pos=2900, prefill_rows=3000),
    "prefill_diag": W.scaled(W.WORKLOADS["prefill_1m"], T=300, prefill_first_pos=0, prefill_rows=300),
    "prefill_long": W.scaled(W.WORKLOADS["prefill_1m"], T=20, prefill_first_pos=70000, prefill_rows=70100),
    # draft/verify groups sharing a sequence (one workgroup per group; waves
    # split the tokens when the group has fewer than 16 queries)
    "mtp_g2": W.scaled(W.WORKLOADS["mtp_verify"], T=6, group=2, seq_lengths=[3000, 1, 700]),
    "mtp_g3": W.scaled(W.WORKLOADS["mtp_verify"], T=9, group=3, seq_lengths=[2, 2049, 513]),
    "mtp_g4": W.scaled(W.WORKLOADS["mtp_verify"], T=8, group=4, seq_lengths=[5000, 257]),
    "mtp_g5": W.scaled(W.WORKLOADS["mtp_verify"], T=10, group=5, seq_lengths=[1500, 4]),
    "mtp_g8": W.scaled(W.WORKLOADS["mtp_verify"], T=16, group=8, seq_lengths=[2500, 40]),
    "mtp_g16": W.scaled(W.WORKLOADS["mtp_verify"], T=32, group=16, seq_lengths=[1000, 3333]),
}


# ----------------------------------------------------------------- indexer --
@pytest.mark.parametrize("case", sorted(SMALL))
def test_indexer_scores_exact(gpu, orc, case):
    wl = SMALL[case]
    li = W.layer_inputs(wl, 0)
    n = wl.n_valid().numpy()
    d = dev(li)
    sc = gpu.indexer_score(d.q_idx, d.w, d.k_idx, qs_of(gpu, wl)).cpu().numpy()
    ref = orc.indexer_scores(li.q_idx, li.w, li.k_idx, wl.base(), wl.n_valid())
    for t in range(wl.T):
        r = ref[t, :n[t]].astype(np.float32)
        assert np.array_equal(r.astype(np.float64), ref[t, :n[t]])      # exact in fp32
        bad = np.nonzero(sc[t, :n[t]] != r)[0]
        assert bad.size == 0, f"t={t}: {bad.size} mismatches, first at {bad[:5]}: {sc[t, bad[:5]]} vs {r[bad[:5]]}"


# ------------------------------------------------------------------- top-k --
def topk_case(name):
    rng = np.random.default_rng(sum(map(ord, name)))
    if name == "ties_int":
        n = np.array([10000, 9999, 4097], np.int32)
        s = rng.integers(0, 50, size=(3, 10000)).astype(np.float32)
        return s, n, 2048
    if name == "ties_pm1":
        n = np.array([5000, 130, 101], np.int32)
        return rng.integers(-1, 2, size=(3, 5000)).astype(np.float32), n, 100
    if name == "normal":
        n = np.array([131072], np.int32)
        return rng.standard_normal((1, 131072)).astype(np.float32), n, 2048
    if name == "signed_zero":
        n = np.array([64, 64], np.int32)
        s = np.where(rng.integers(0, 2, size=(2, 64)) == 0, -0.0, 0.0).astype(np.float32)
        s[1, ::5] = -1.5
        return s, n, 7
    if name == "edges":
        n = np.array([0, 1, 63, 64, 65, 2047, 2048, 2049, 4095], np.int32)
        return rng.integers(0, 300, size=(9, 4096)).astype(np.float32), n, 2048
    if name == "k1":
        n = np.array([1000, 3], np.int32)
        s = rng.integers(-5, 5, size=(2, 1000)).astype(np.float32)
        return s, n, 1
    # every score in one first-digit bin: the survivor list overflows and the
    # second digit must thin it (split path: few queries; row path: many)
    if name == "dense_bin_split":
        n = np.array([131072, 100000], np.int32)
        return rng.integers(24576, 28672, size=(2, 131072)).astype(np.float32), n, 2048
    if name == "dense_bin_row":
        n = np.full(300, 12000, np.int32)
        n[::7] = 11999
        return rng.integers(24576, 28672, size=(300, 12000)).astype(np.float32), n, 2048
    # more ties at the two-digit bound than the finishing workgroup's list
    # holds: the split path falls back to digit passes over the whole row
    if name == "all_equal_split":
        n = np.array([131072, 50000], np.int32)
        s = np.full((2, 131072), 7.0, np.float32)
        s[:, ::977] = 8.0
        s[1, 3::1201] = 9.0
        return s, n, 2048
    # long rows on the row path: the k-th key is bounded from 1/16 of the row
    # (every 16th block of 256 scores), then one pass collects the keys above
    if name == "sampled_row":
        n = rng.integers(65536, 70001, size=260).astype(np.int32)
        return rng.integers(0, 4000, size=(260, 70000)).astype(np.float32), n, 2048
    # the sampled blocks hold the largest scores: fewer than k keys reach the
    # bound, so the exact two-pass path runs
    if name == "sampled_row_fallback":
        n = np.full(260, 65536, np.int32)
        s = rng.integers(0, 1000, size=(260, 65536)).astype(np.float32)
        blk = (np.arange(65536) // 256) % 16 == 0
        s[:, blk] = 1000.0
        return s, n, 8192
    # every sample equal: all keys reach the bound and overflow the list
    if name == "sampled_all_equal_row":
        n = np.full(256, 66000, np.int32)
        s = np.full((256, 66000), 7.0, np.float32)
        s[:, 5::997] = 8.0
        return s, n, 2048
    # split path, every slice holding more keys at or above the bound than the
    # finishing workgroup loads ahead of the counts (four values, so the bound
    # keeps half the row: 1024 of 2048 per slice), all of them together still
    # fitting its list; the second row is ragged
    if name == "long_slices_split":
        n = np.array([32768, 30001], np.int32)
        return rng.integers(0, 4, size=(2, 32768)).astype(np.float32), n, 5000
    # split path, the sampled positions (32 of every 1024) hold the largest
    # scores: fewer than k keys reach the sampled bound and the selection
    # finishes from the whole row
    if name == "sampled_split_fallback":
        n = np.array([131072], np.int32)
        s = rng.integers(0, 1000, size=(1, 131072)).astype(np.float32)
        s[:, (np.arange(131072) % 1024) < 32] = 1000.0
        return s, n, 8192
    # split path, the winners clustered in the first two slices
    if name == "clustered_split":
        n = np.array([131072], np.int32)
        s = rng.standard_normal((1, 131072)).astype(np.float32)
        s[0, 100:3100] += 10.0
        return s, n, 2048
    if name == "all_equal_row":
        n = np.full(260, 9000, np.int32)
        s = np.full((260, 9000), 7.0, np.float32)
        s[:, ::1000] = 8.0
        return s, n, 2048
    raise KeyError(name)


def test_topk_workspace_reuse(gpu, orc):
    """Workspaces carry no state: one workspace, filled with arbitrary bytes
    before every call, serves repeated top-k calls of several shapes (split
    path and row path) with new scores each time."""
    rng = np.random.default_rng(77)
    shapes = [(1, 131072, 2048), (3, 5000, 2048), (300, 3000, 64), (5, 300, 7), (2, 70000, 2048)]
    need = 0
    for T, L, k in shapes:
        qs = gpu.make_queries(torch.zeros(T, dtype=torch.int64), torch.full((T,), L, dtype=torch.int32), L)
        need = max(need, gpu._lib.ic_topk_workspace_size(ctypes.byref(qs.c()), k))
    ws = gpu.workspace(need)
    for T, L, k in shapes:
        n = rng.integers(max(1, L // 2), L + 1, size=T).astype(np.int32)
        qs = gpu.make_queries(torch.zeros(T, dtype=torch.int64), torch.from_numpy(n), L)
        for rep in range(3):
            ws.fill_(int(rng.integers(0, 256)))
            s = rng.integers(0, 4000, size=(T, L)).astype(np.float32)
            buf = np.zeros((T, gpu.score_ld(L)), np.float32)
            buf[:, :L] = s
            got = gpu.topk(torch.from_numpy(buf).cuda(), qs, k, ws=ws).cpu().numpy()
            assert np.array_equal(got, orc.topk(s, n, k)), f"shape {(T, L, k)}, call {rep}"


def test_layer_stack_workspace_garbage(gpu, orc):
    """A layer stack whose workspace holds arbitrary bytes on entry gives the
    same index sets and outputs as one with a zeroed workspace, on the path
    that fills the first-digit histogram in the indexer (300 queries: the
    row path) and on the split path (2 queries)."""
    for T, L in ((300, 3000), (2, 20000)):
        wl = W.scaled(W.WORKLOADS["decode_128k"], T=T, lengths=[L] * T, n_layers=3, full_layers=[0, 2], H=8)
        rmap = gpu.reuse_map_last_full(wl.is_full())
        lays = []
        for l in range(wl.n_layers):
            y = dev(W.layer_inputs(wl, l, with_indexer=rmap[l] == l))
            lays.append(dict(q_idx=y.q_idx, w=y.w, k_idx=y.k_idx, q=y.q, kv=y.kv, sink=y.sink,
                             out=torch.empty((wl.T, wl.H, wl.D_v), dtype=torch.float32, device="cuda")))
        d = gpu.dims(wl.H_I, wl.D_I, wl.k, wl.H, wl.D_qk, wl.D_v, out_f32=True)
        st = gpu.LayerStack(lays, rmap, qs_of(gpu, wl), d, wl.scale)
        results = []
        for fill in (0, 0xA5, 0xFF, 0x3C):
            st.ws.fill_(fill)
            st()
            torch.cuda.synchronize()
            results.append(([y["out"].clone() for y in lays], st.index_cache.clone()))
        for outs, cache in results[1:]:
            assert torch.equal(cache, results[0][1]), f"T={T}: index cache depends on workspace contents"
            for a, b in zip(outs, results[0][0]):
                assert torch.equal(a, b), f"T={T}: outputs depend on workspace contents"


@pytest.mark.parametrize("name", ["ties_int", "ties_pm1", "normal", "signed_zero", "edges", "k1",
                                  "dense_bin_split", "dense_bin_row", "all_equal_split", "all_equal_row",
                                  "sampled_row", "sampled_row_fallback", "sampled_all_equal_row",
                                  "long_slices_split", "clustered_split", "sampled_split_fallback"])
def test_topk_exact(gpu, orc, name):
    s, n, k = topk_case(name)
    T, L = s.shape
    ld = gpu.score_ld(L)
    buf = np.zeros((T, ld), np.float32)
    buf[:, :L] = s
    qs = gpu.make_queries(torch.zeros(T, dtype=torch.int64), torch.from_numpy(n), L)
    got = gpu.topk(torch.from_numpy(buf).cuda(), qs, k).cpu().numpy()
    ref = orc.topk(s, n, k)
    assert np.array_equal(got, ref)
    check_topk_invariants(s, n, k, got)


def test_topk_all_rows_empty_zero_stride(gpu):
    """Split top-k over rows that hold no scores, with the zero row stride the
    boundary allows then (ld = 0): the collection launch, whose loads need
    rows of at least four scores, is skipped and every index row is all -1."""
    import ctypes
    T, k = 3, 16
    buf = torch.zeros(16, dtype=torch.float32, device="cuda")       # never read
    qs = gpu.make_queries(torch.zeros(T, dtype=torch.int64), torch.zeros(T, dtype=torch.int32), 0)
    assert qs.max_n == 0
    qc = qs.c()
    need = gpu._lib.ic_topk_workspace_size(ctypes.byref(qc), k)
    ws = gpu.workspace(need, buf.device)
    idx = torch.full((T, k), 5, dtype=torch.int32, device="cuda")
    gpu._check(gpu._lib.ic_topk(gpu._ptr(buf), 0, ctypes.byref(qc), k, gpu._ptr(idx), gpu._ptr(ws), ws.numel(),
                                gpu._stream(None)))
    torch.cuda.synchronize()
    assert bool((idx == -1).all())


# ---------------------------------------------------------------- sparse MLA --
@pytest.fixture(params=["narrow", "wide"])
def mla_form(request, monkeypatch):
    """Both forms of the sparse MLA kernel, whatever the library would pick
    for the size (the wide one takes the heads 128 to a workgroup)."""
    monkeypatch.setenv("IC_MLA_FORM", request.param)
    return request.param


@pytest.fixture(params=["0", "1"])
def o_layout(request, monkeypatch, mla_form):
    """Both layouts of the narrow form's O accumulators (untransposed: four
    heads of one value column per lane; transposed: four value columns of one
    head), forced on every path whatever the plan would pick."""
    if mla_form == "wide" and request.param == "1":
        pytest.skip("the layout is the narrow form's")
    monkeypatch.setenv("IC_MLA_OTRANS", request.param)
    return request.param


def needs_form(form, H):
    if form == "wide" and H % 128:
        pytest.skip("the wide form takes whole groups of 128 heads")


def mla_case(name):
    """(workload, idx [T, k] int32 with sequence-local positions)."""
    rng = np.random.default_rng(7)
    if name == "tiny":
        wl = W.WORKLOADS["tiny_2layer"]
        idx = np.sort(rng.choice(4096, 64, replace=False)).astype(np.int32)[None]
        return wl, idx
    if name == "decode_split":
        wl = W.scaled(W.WORKLOADS["decode_128k"], lengths=[5000])
        idx = rng.choice(5000, 2048, replace=False).astype(np.int32)[None]     # unsorted
        return wl, idx
    if name == "decode_k8192":
        # 8192 entries: 128 splits of 64 rows, so the combine takes its
        # partials in several batches of loads
        wl = W.scaled(W.WORKLOADS["decode_128k"], lengths=[10000], k=8192)
        idx = rng.choice(10000, 8192, replace=False).astype(np.int32)[None]
        return wl, idx
    if name == "batch_k64":
        wl = W.scaled(W.WORKLOADS["decode_128k"], T=8, k=64, lengths=[300, 64, 65, 1, 0, 100, 200, 90])
        idx = np.full((8, 64), -1, np.int32)
        for t, nt in enumerate(wl.lengths):
            sel = rng.choice(nt, min(nt, 64), replace=False) if nt else np.zeros(0, np.int32)
            idx[t, :sel.size] = sel
            rng.shuffle(idx[t])                                                 # -1 anywhere
        return wl, idx
    if name == "padded_split":
        wl = W.scaled(W.WORKLOADS["decode_128k"], T=2, lengths=[1500, 0])
        idx = np.full((2, 2048), -1, np.int32)
        idx[0, :1500] = rng.permutation(1500)
        rng.shuffle(idx[0])
        return wl, idx
    if name == "many_queries":
        # enough queries that every (query, head group) takes one workgroup
        # and no split: the sink enters inside the kernel
        lengths = [int(x) for x in rng.integers(1, 200, 512)]
        wl = W.scaled(W.WORKLOADS["decode_128k"], T=512, k=64, lengths=lengths)
        idx = np.full((512, 64), -1, np.int32)
        for t, nt in enumerate(lengths):
            sel = rng.choice(nt, min(nt, 64), replace=False)
            idx[t, :sel.size] = sel
        return wl, idx
    raise KeyError(name)


@pytest.mark.parametrize("name", ["tiny", "decode_split", "decode_k8192", "batch_k64", "padded_split", "many_queries"])
def test_sparse_mla_close(gpu, orc, name, mla_form, o_layout):
    """fp32 output within 5e-3 of the fp64 oracle; the bf16 output of the same
    launch is its rounded image (and within 5e-3 where bf16 can be)."""
    wl, idx = mla_case(name)
    needs_form(mla_form, wl.H)
    li = W.layer_inputs(wl, 0, with_indexer=False)
    d = dev(li)
    qs = qs_of(gpu, wl)
    i = torch.from_numpy(idx).cuda()
    ref = orc.sparse_mla(li.q, li.kv, wl.base(), idx, li.sink, wl.scale, wl.D_v)
    f32 = gpu.sparse_mla(d.q, d.kv, qs, i, d.sink, wl.scale, wl.D_v, out_f32=True).cpu().numpy()
    b16 = gpu.sparse_mla(d.q, d.kv, qs, i, d.sink, wl.scale, wl.D_v).float().cpu().numpy()
    assert_close(f32, ref, f"sparse MLA {name} {mla_form}/o{o_layout} [fp32]")
    assert_bf16_output(b16, f32, ref, f"sparse MLA {name} {mla_form}")
    for got in (f32, b16):
        assert np.all(got[idx.max(1) < 0] == 0)                                  # empty rows are zero


def test_sparse_mla_large_values(gpu, orc, mla_form, o_layout):
    """Latent rows scaled by 1e5 (and q by 1e-5, so the scores stay as they
    were): the split partials, stored in fp16 with a per-(head, half)
    power-of-two scale, must stay in range; the fp32 output holds the bar
    scaled with the values, and the bf16 output is its rounded image."""
    wl, idx = mla_case("decode_split")
    li = W.layer_inputs(wl, 0, with_indexer=False)
    big = 1.0e5
    kv = (li.kv.float() * big).to(torch.bfloat16)
    q = (li.q.float() / big).to(torch.bfloat16)
    qs = qs_of(gpu, wl)
    i = torch.from_numpy(idx).cuda()
    f32 = gpu.sparse_mla(q.cuda(), kv.cuda(), qs, i, li.sink.cuda(), wl.scale, wl.D_v, out_f32=True).cpu().numpy()
    b16 = gpu.sparse_mla(q.cuda(), kv.cuda(), qs, i, li.sink.cuda(), wl.scale, wl.D_v).float().cpu().numpy()
    ref = orc.sparse_mla(q, kv, wl.base(), idx, li.sink, wl.scale, wl.D_v)
    assert np.isfinite(f32).all()
    assert np.abs(ref).max() > 16384.0                                          # the scaled range is in use
    err = max_abs(f32, ref)
    report(f"sparse MLA large values {mla_form} [fp32, bar 5e-3 x 1e5]", err)
    assert err <= ATOL * big, f"max abs error {err} (scaled bar {ATOL * big})"
    assert np.array_equal(b16, bf16_rne(f32))


@pytest.mark.parametrize("name", ["decode_split", "many_queries"])
def test_sparse_mla_logit_range(gpu, orc, name, mla_form, o_layout):
    """q scaled by a power of two until the logits of a head spread over
    hundreds of units: later rows then beat the first rows' maximum by far
    (the narrow form rescales its sums; the wide form, whose probabilities
    may grow only so far above its first reference, takes a second pass over
    the rows with every reference at its final maximum). The output must
    still match the oracle's softmax to the bar."""
    wl, idx = mla_case(name)
    li = W.layer_inputs(wl, 0, with_indexer=False)
    t0 = int(np.argmax((idx >= 0).sum(1)))
    rows = idx[t0][idx[t0] >= 0] + int(wl.base()[t0])
    logits = wl.scale * (li.q[t0].double().numpy() @ li.kv[rows].double().numpy().T)
    f = 2.0 ** math.ceil(math.log2(300.0 / logits.std(axis=1).mean()))
    q = (li.q.float() * f).to(torch.bfloat16)
    assert torch.equal(q.float() / f, li.q.float())                             # exact scaling
    qs = qs_of(gpu, wl)
    i = torch.from_numpy(idx).cuda()
    ref = orc.sparse_mla(q, li.kv, wl.base(), idx, li.sink, wl.scale, wl.D_v)
    f32 = gpu.sparse_mla(q.cuda(), li.kv.cuda(), qs, i, li.sink.cuda(), wl.scale, wl.D_v,
                         out_f32=True).cpu().numpy()
    assert np.isfinite(f32).all()
    assert_close(f32, ref, f"sparse MLA {name} {mla_form}/o{o_layout} logits x{f:g} [fp32]")


def test_sparse_mla_deterministic(gpu, mla_form):
    wl, idx = mla_case("decode_split")
    d = dev(W.layer_inputs(wl, 0, with_indexer=False))
    qs = qs_of(gpu, wl)
    i = torch.from_numpy(idx).cuda()
    a = gpu.sparse_mla(d.q, d.kv, qs, i, d.sink, wl.scale, wl.D_v)
    b = gpu.sparse_mla(d.q, d.kv, qs, i, d.sink, wl.scale, wl.D_v)
    assert torch.equal(a, b)


# --------------------------------------------------------------- layer stack --
@pytest.mark.parametrize("case", ["decode_3layer", "ragged_2layer"])
def test_layer_stack_graph_replay(gpu, case, mla_form):
    """The stack captured in a HIP graph and replayed several times, with eager
    work and synchronisations between the replays, gives the eager result bit
    for bit every time: the calls enqueue no memsets or copies, and the
    workspace holds no state between calls."""
    wl = {"decode_3layer": W.scaled(W.WORKLOADS["decode_128k"], lengths=[20000], n_layers=3, full_layers=[0, 2]),
          "ragged_2layer": W.scaled(W.WORKLOADS["ragged_64"], T=5, len_range=(100, 9000), n_layers=2,
                                    full_layers=[0])}[case]
    rmap = gpu.reuse_map_last_full(wl.is_full())
    lays = []
    for l in range(wl.n_layers):
        y = dev(W.layer_inputs(wl, l, with_indexer=rmap[l] == l))
        lays.append(dict(q_idx=y.q_idx, w=y.w, k_idx=y.k_idx, q=y.q, kv=y.kv, sink=y.sink,
                         out=torch.empty((wl.T, wl.H, wl.D_v), dtype=torch.bfloat16, device="cuda")))
    d = gpu.dims(wl.H_I, wl.D_I, wl.k, wl.H, wl.D_qk, wl.D_v)
    st = gpu.LayerStack(lays, rmap, qs_of(gpu, wl), d, wl.scale)
    st()
    torch.cuda.synchronize()
    ref_out = [y["out"].clone() for y in lays]
    ref_cache = st.index_cache.clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        st()                                      # once on the capture stream first
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        st()
    for rep in range(3):
        for y in lays:
            y["out"].zero_()
        st.index_cache.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for l, y in enumerate(lays):
            assert torch.equal(y["out"], ref_out[l]), f"replay {rep}: layer {l} output differs from eager"
        assert torch.equal(st.index_cache, ref_cache), f"replay {rep}: index cache differs from eager"
        x = torch.randn(4096, device="cuda")
        assert float((x * 0).sum().item()) == 0.0       # eager work between replays


def run_stack(ic, wl, layers_dev, rmap, out_f32=False):
    T = wl.T
    outs = []
    lays = []
    for y in layers_dev:
        o = torch.empty((T, wl.H, wl.D_v), dtype=torch.float32 if out_f32 else torch.bfloat16, device="cuda")
        outs.append(o)
        lays.append(dict(q_idx=y.q_idx, w=y.w, k_idx=y.k_idx, q=y.q, kv=y.kv, sink=y.sink, out=o))
    d = ic.dims(wl.H_I, wl.D_I, wl.k, wl.H, wl.D_qk, wl.D_v, out_f32)
    cache, passes = ic.layer_stack(lays, rmap, qs_of(ic, wl), d, wl.scale)
    return outs, cache, passes


@pytest.mark.parametrize("case", ["tiny", "small_5layer", "every6_13layer", "first_only_4layer", "ties_3layer",
                                  "clustered_2layer"])
def test_layer_stack_small(gpu, orc, case, mla_form, o_layout):
    if case == "tiny":
        wl = W.WORKLOADS["tiny_2layer"]
    elif case == "clustered_2layer":
        # key rows 0..4999 all equal to +-8 along the weighted sum of the
        # query's heads: those positions tie above every other score and all
        # fall in the first chunk of the split path, more than a workgroup's
        # share of one slice when the sparse MLA selects its own rows (then
        # the keys are reloaded into registers by their rank over the slices)
        wl = W.scaled(W.WORKLOADS["decode_128k"], n_layers=2, full_layers=[0], T=1, lengths=[20000])
    elif case == "ties_3layer":
        # every key row equal: a query's scores all tie, every key reaches the
        # bound and the lowest positions win (past 8192 keys the selection
        # runs over the slices in memory; at 5000 they are reloaded into
        # registers by rank)
        wl = W.scaled(W.WORKLOADS["decode_128k"], n_layers=3, full_layers=[0, 2], T=3, lengths=[20000, 5000, 2049])
    elif case == "small_5layer":
        wl = W.scaled(W.WORKLOADS["decode_128k"], n_layers=5, full_layers=[0, 3], T=3, lengths=[3000, 2048, 100])
    elif case == "every6_13layer":
        # an index refreshed every sixth layer, on small shapes
        wl = W.scaled(W.WORKLOADS["decode_128k"], n_layers=13, full_layers=[0, 6, 12], T=2, k=64,
                      lengths=[700, 65], H=8)
    else:
        wl = W.scaled(W.WORKLOADS["decode_128k"], n_layers=4, full_layers=[0], T=2, k=64, lengths=[300, 50], H=8)
    needs_form(mla_form, wl.H)
    host = [W.layer_inputs(wl, l) for l in range(wl.n_layers)]
    if case == "ties_3layer":
        for x in host:
            x.k_idx.copy_(x.k_idx[0:1].expand_as(x.k_idx))
    if case == "clustered_2layer":
        for x in host:
            v = (x.w[0, :, None].double() * x.q_idx[0].view(torch.float8_e4m3fn).double()).sum(0)
            x.k_idx[:5000] = torch.where(v >= 0, 0x50, 0xD0).to(torch.uint8)    # e4m3fn codes of +8, -8
    rmap = gpu.reuse_map_last_full(wl.is_full())
    outs, cache, passes = run_stack(gpu, wl, [dev(x) for x in host], rmap, out_f32=True)
    base, n = wl.base().numpy(), wl.n_valid().numpy()
    r_outs, r_index, r_passes = orc.layer_stack(host, rmap, base, n, wl.k, wl.scale, wl.D_v)
    assert passes == r_passes == sum(wl.is_full())
    slots = {l: i for i, l in enumerate(l for l in range(wl.n_layers) if rmap[l] == l)}
    for l in range(wl.n_layers):
        got_idx = cache[slots[rmap[l]]].cpu().numpy()
        assert np.array_equal(got_idx, r_index[l])
        assert_close(outs[l].cpu().numpy(), r_outs[l], f"layer stack {case} {mla_form}/o{o_layout} layer {l} [fp32]")


def test_sparse_mla_odd_k_steps_after_graph_replays(gpu, orc, monkeypatch):
    """80-wide rows make an odd count of 32-wide K-steps, so the two halves of
    a head group run different numbers of matrix steps. The vector registers
    a kernel's waves start with hold whatever earlier work left there; after
    the ragged graph-replay test below, a matrix step that ran on never-loaded
    operands (matrix instructions ignore EXEC masks) made every output NaN.
    Several launches after that same work, each checked against the oracle."""
    monkeypatch.setenv("IC_MLA_FORM", "narrow")
    test_layer_stack_graph_replay(gpu, "ragged_2layer", "narrow")
    wl, idx = mla_case("tiny")
    li = W.layer_inputs(wl, 0, with_indexer=False)
    d = dev(li)
    qs = qs_of(gpu, wl)
    i = torch.from_numpy(idx).cuda()
    ref = orc.sparse_mla(li.q, li.kv, wl.base(), idx, li.sink, wl.scale, wl.D_v)
    for rep in range(4):
        got = gpu.sparse_mla(d.q, d.kv, qs, i, d.sink, wl.scale, wl.D_v, out_f32=True).cpu().numpy()
        assert np.isfinite(got).all(), f"launch {rep}: non-finite output"
        assert_close(got, ref, f"sparse MLA tiny after graph replays, launch {rep} [fp32]")


def test_sparse_mla_out_of_range_entries_are_empty(gpu, orc, mla_form):
    """Index entries outside [0, n_valid[t]) (a list that breaks the contract)
    are treated as empty on the device: the output equals the oracle's on the
    same list with those entries replaced by -1, and no latent row outside the
    query's range is read."""
    wl = W.scaled(W.WORKLOADS["decode_128k"], T=3, k=64, lengths=[200, 90, 130])
    rng = np.random.default_rng(11)
    n = wl.n_valid().numpy()
    idx = np.stack([rng.choice(int(x), 64, replace=False) for x in n]).astype(np.int32)
    idx[0, 5] = n[0]                     # one past the query's rows
    idx[0, 9] = n[0] + n[1]              # a row of the next query
    idx[1, :8] = 2_000_000_000           # far outside the cache
    idx[2, -3:] = -7                     # negative but not -1
    clean = np.where((idx >= 0) & (idx < n[:, None]), idx, -1).astype(np.int32)
    li = W.layer_inputs(wl, 0, with_indexer=False)
    d = dev(li)
    qs = qs_of(gpu, wl)
    got = gpu.sparse_mla(d.q, d.kv, qs, torch.from_numpy(idx).cuda(), d.sink, wl.scale, wl.D_v,
                         out_f32=True).float().cpu().numpy()
    ref = orc.sparse_mla(li.q, li.kv, wl.base(), clean, li.sink, wl.scale, wl.D_v)
    assert_close(got, ref, f"sparse MLA out-of-range entries {mla_form} [fp32]")


# ------------------------------------------------------------ gated output --
def assert_gated(got, ref, what):
    """The gated output is bf16 only and its values reach |4| (sigmoid times a
    decompressed N(0, 1) entry), where bf16 spacing alone exceeds 5e-3: its
    bar is 5e-3 of max(1, |ref|) -- the flat 5e-3 below 1, the same relative
    precision above."""
    err = np.abs(got - ref) / np.maximum(1.0, np.abs(ref))
    m = float(err.max())
    report(what + " [relative above 1]", m)
    assert m <= ATOL, f"{what}: error {m:.3e} of max(1, |ref|) > {ATOL}"


@pytest.mark.parametrize("T,H,D_v,D_o", [(1, 128, 512, 128), (5, 3, 512, 64), (17, 2, 512, 192),
                                         (33, 4, 64, 64), (40, 1, 512, 1024),
                                         (250, 8, 512, 192), (253, 16, 64, 64), (600, 4, 512, 1024),
                                         (630, 128, 512, 128)])
def test_gated_output_close(gpu, orc, T, H, D_v, D_o):
    """sigmoid(gate) * (wv_b @ o) per head against the fp64 oracle: partial
    query blocks (T % 16), several column blocks, both built latent widths,
    both workgroup shapes (64 columns for few query blocks, 128 otherwise,
    with a partial last column group at D_o = 192) and runs of several query
    blocks per workgroup."""
    wl = W.scaled(W.WORKLOADS["decode_128k"], T=T, H=H, D_v=D_v)
    gi = W.gate_inputs(wl, 0, D_o)
    got = gpu.gated_output(gi.o.cuda(), gi.wv_b.cuda(), gi.gate.cuda()).float().cpu().numpy()
    ref = orc.gated_output(gi.o, gi.wv_b, gi.gate)
    assert_gated(got, ref, f"gated output T={T} H={H} D_v={D_v} D_o={D_o}")


def test_gated_output_prefill_sampled(gpu, orc):
    """4096 queries x 128 heads (the prefill shape), oracle on sampled queries."""
    wl = W.scaled(W.WORKLOADS["prefill_1m"], T=4096)
    gi = W.gate_inputs(wl, 1, 128, device="cuda")
    got = gpu.gated_output(gi.o, gi.wv_b, gi.gate).float().cpu().numpy()
    for t in (0, 15, 16, 2047, 4095):
        ref = orc.gated_output(gi.o[t:t + 1].cpu(), gi.wv_b.cpu(), gi.gate[t:t + 1].cpu())
        assert_gated(got[t:t + 1], ref, f"gated output prefill query {t}")


def test_trace_records_every_launch(gpu):
    """Tracing (ic_trace_start) names and times every kernel of a layer stack
    and leaves its results unchanged; leaving a kernel out (ic_trace_skip,
    the per-kernel cost measurement) still reports its launches, and the
    stack computes the reference again once the switch is cleared."""
    wl = W.scaled(W.WORKLOADS["decode_128k"], lengths=[20000], n_layers=3, full_layers=[0, 2])
    rmap = gpu.reuse_map_last_full(wl.is_full())
    lays = []
    for l in range(wl.n_layers):
        y = dev(W.layer_inputs(wl, l, with_indexer=rmap[l] == l))
        lays.append(dict(q_idx=y.q_idx, w=y.w, k_idx=y.k_idx, q=y.q, kv=y.kv, sink=y.sink,
                         out=torch.empty((wl.T, wl.H, wl.D_v), dtype=torch.bfloat16, device="cuda")))
    st = gpu.LayerStack(lays, rmap, qs_of(gpu, wl), gpu.dims(wl.H_I, wl.D_I, wl.k, wl.H, wl.D_qk, wl.D_v),
                        wl.scale)
    st()
    torch.cuda.synchronize()
    ref = [y["out"].clone() for y in lays]
    tr = gpu.Trace(32)
    with tr:
        st()
    torch.cuda.synchronize()
    ks = tr.read()
    names = [k[0] for k in ks]
    assert tr.count == len(names) >= wl.n_layers
    assert names.count("indexer_decode_kernel") == 2
    assert sum(n.startswith("sparse_mla_kernel") for n in names) == 3
    assert all(k[1] > 0 for k in ks)
    for l, y in enumerate(lays):
        assert torch.equal(y["out"], ref[l])
    tr2 = gpu.Trace(32)
    with gpu.SkipKernel("mla_combine_kernel"), tr2:
        st()
    torch.cuda.synchronize()
    assert [k[0] for k in tr2.read()] == names
    st()
    torch.cuda.synchronize()
    for l, y in enumerate(lays):
        assert torch.equal(y["out"], ref[l]), f"layer {l} after the skip switch was cleared"
