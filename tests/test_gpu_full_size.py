"""Parity at the workloads' full sizes, in the launch configuration the
benchmark uses (ic_layer_stack, bf16 outputs). The oracle recomputes sampled
queries (and sampled layers of the 78-layer stack) one by one; every query's
index row is also checked against the top-k invariants where its scores are
known. Inputs of the large workloads are drawn on the device by the seeded
generator and copied back for the oracle."""
import sys

import numpy as np
import pytest
import torch

from checks import check_topk_invariants, report
from cross_layer_index_amd import workloads as W

pytestmark = pytest.mark.gpu
ATOL = 5e-3


def assert_close(got, ref, what):
    """Flat max-abs 5e-3 against the fp64 oracle."""
    err = float(np.abs(got - ref).max())
    report(what, err)
    assert err <= ATOL, f"{what}: max abs error {err:.3e} > {ATOL}"
    return err


def bf16_rne(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).float().numpy()


def build_stack(ic, wl, rmap, device_gen, out_f32=False):
    lays, host = [], []
    for l in range(wl.n_layers):
        full = rmap[l] == l
        li = W.layer_inputs(wl, l, device="cuda" if device_gen else "cpu", with_indexer=full)
        d = W.LayerInputs(*[None if x is None else x.cuda() for x in (li.q_idx, li.w, li.k_idx, li.q, li.kv,
                                                                       li.sink)])
        out = torch.empty((wl.T, wl.H, wl.D_v), dtype=torch.float32 if out_f32 else torch.bfloat16, device="cuda")
        lays.append(dict(q_idx=d.q_idx, w=d.w, k_idx=d.k_idx, q=d.q, kv=d.kv, sink=d.sink, out=out))
        host.append(li)
    return lays, host


def query_slice(li, wl, base, n, ts):
    """Host copies of what the oracle needs for queries ts (their own rows)."""
    out = []
    for t in ts:
        b, nt = int(base[t]), int(n[t])
        rows = slice(b, b + nt)
        out.append(dict(
            q_idx=None if li.q_idx is None else li.q_idx[t:t + 1].cpu(),
            w=None if li.w is None else li.w[t:t + 1].cpu(),
            k_idx=None if li.k_idx is None else li.k_idx[rows].cpu(),
            q=li.q[t:t + 1].cpu(), kv=li.kv[rows].cpu(), n=np.array([nt], np.int32)))
    return out


def oracle_query(orc, wl, qd, idx_src=None):
    """Oracle index row and output for one query (base 0 within its rows)."""
    base0 = np.array([0], np.int64)
    if idx_src is None:
        I = orc.indexer_scores(qd["q_idx"], qd["w"], qd["k_idx"], base0, qd["n"])
        idx = orc.topk(I.astype(np.float32), qd["n"], wl.k)
    else:
        I, idx = None, idx_src
    return I, idx


def run_case(gpu, orc, wl, sample_t, sample_layers=None, device_gen=True, out_f32=False, pairs=None):
    """The stack at full size; sampled (layer, query) outputs against the
    oracle at the flat 5e-3. With out_f32 and a dict `pairs`, the fp32
    outputs of every layer are also returned in it (for the bf16 pairing)."""
    rmap = gpu.reuse_map_last_full(wl.is_full())
    lays, host = build_stack(gpu, wl, rmap, device_gen, out_f32)
    qs = gpu.make_queries(wl.base(), wl.n_valid(), wl.rows(), wl.same_seq, group=wl.group)
    d = gpu.dims(wl.H_I, wl.D_I, wl.k, wl.H, wl.D_qk, wl.D_v, out_f32)
    st = gpu.LayerStack(lays, rmap, qs, d, wl.scale)
    passes = st()
    torch.cuda.synchronize()
    assert passes == sum(1 for l in range(wl.n_layers) if rmap[l] == l)
    base, n = wl.base().numpy(), wl.n_valid().numpy()
    slots = {l: i for i, l in enumerate(l for l in range(wl.n_layers) if rmap[l] == l)}
    layers = range(wl.n_layers) if sample_layers is None else sample_layers
    ref_idx = {}
    worst = 0.0
    for l in layers:
        src = rmap[l]
        got_idx = st.index_cache[slots[src]].cpu().numpy()
        for t in sample_t:
            key = (src, t)
            if key not in ref_idx:
                qd = query_slice(host[src], wl, base, n, [t])[0]
                I, idx = oracle_query(orc, wl, qd)
                ref_idx[key] = idx
                check_topk_invariants(I.astype(np.float32), qd["n"], wl.k, got_idx[t:t + 1])
            assert np.array_equal(got_idx[t], ref_idx[key][0]), f"layer {l} query {t}: index set differs"
            qd = query_slice(host[l], wl, base, n, [t])[0]
            sink = host[l].sink.cpu()
            ref = orc.sparse_mla(qd["q"], qd["kv"], np.array([0], np.int64), ref_idx[key], sink, wl.scale, wl.D_v)
            got = lays[l]["out"][t:t + 1].float().cpu().numpy()
            worst = max(worst, assert_close(got, ref, f"{wl.name} layer {l} query {t} "
                                                      f"[{'fp32' if out_f32 else 'bf16'}]"))
    if pairs is not None:
        pairs.update({l: lays[l]["out"].float().cpu().numpy() for l in range(wl.n_layers)})
    return st, worst


def test_decode_128k_full(gpu, orc):
    wl = W.WORKLOADS["decode_128k"]
    run_case(gpu, orc, wl, [0], device_gen=False)


def test_decode_128k_recency_full(gpu, orc):
    """Scores rising with position: the top-k lies in the row's last chunks,
    so a slice of the split top-k holds more keys than its share of the
    selecting sparse MLA's registers and the keys are reloaded by their rank
    over the slices."""
    wl = W.WORKLOADS["decode_128k_recency"]
    run_case(gpu, orc, wl, [0], device_gen=False)


def test_ragged_64_full(gpu, orc):
    wl = W.WORKLOADS["ragged_64"]
    n = wl.n_valid().numpy()
    ts = sorted({0, 31, 63, int(np.argmin(n)), int(np.argmax(n))})
    run_case(gpu, orc, wl, ts)


def test_edge_lengths_full(gpu, orc):
    """The edge set (n = 0, 1, 63, 64, 65, 2047, 2048, 2049, 4095). Its short
    rows give outputs near 3 (one key: o = v * sigmoid(s - sink)), where bf16
    spacing alone is 2^-6: the fp32 stack holds the flat 5e-3 on every query,
    and the bf16 stack's outputs are the rounded fp32 outputs bit for bit."""
    wl = W.WORKLOADS["edge_lengths"]
    f32 = {}
    run_case(gpu, orc, wl, list(range(wl.T)), device_gen=False, out_f32=True, pairs=f32)
    rmap = gpu.reuse_map_last_full(wl.is_full())
    lays, _ = build_stack(gpu, wl, rmap, False)
    qs = gpu.make_queries(wl.base(), wl.n_valid(), wl.rows())
    st = gpu.LayerStack(lays, rmap, qs, gpu.dims(wl.H_I, wl.D_I, wl.k, wl.H, wl.D_qk, wl.D_v), wl.scale)
    st()
    torch.cuda.synchronize()
    for l in range(wl.n_layers):
        assert np.array_equal(lays[l]["out"].float().cpu().numpy(), bf16_rne(f32[l])), f"layer {l}"


def test_mtp_verify_full(gpu, orc):
    """Draft/verify decode at full size: 8 sequences x 4 queries sharing each
    cache (the grouped key-sharing indexer); first and last query of three
    groups checked against the oracle."""
    wl = W.WORKLOADS["mtp_verify"]
    run_case(gpu, orc, wl, [0, 3, 12, 15, 28, 31])


def test_stack_78_full(gpu, orc):
    wl = W.WORKLOADS["stack_78"]
    layers = [0, 1, 2, 3, 5, 6, 9, 10, 41, 74, 77]
    st, _ = run_case(gpu, orc, wl, [0, 7], sample_layers=layers)
    assert st.passes.value == 21


def test_stack_78_all_full_passes(gpu):
    """The same stack with every layer full runs 78 indexer passes (the
    comparison configuration); checked for the pass count and index rows of a
    few layers against the IndexCache run's full layers (same inputs)."""
    wl = W.scaled(W.WORKLOADS["stack_78"], n_layers=6, full_layers=list(range(6)))
    rmap = list(range(6))
    lays, _ = build_stack(gpu, wl, rmap, device_gen=True)
    qs = gpu.make_queries(wl.base(), wl.n_valid(), wl.rows())
    d = gpu.dims(wl.H_I, wl.D_I, wl.k, wl.H, wl.D_qk, wl.D_v)
    st = gpu.LayerStack(lays, rmap, qs, d, wl.scale)
    assert st() == 6
    # the Hy4 map over the same 6 layers reuses slot 2 for layers 3..5
    m = gpu.reuse_map_last_full(W.WORKLOADS["stack_78"].is_full()[:6])
    st2 = gpu.LayerStack(lays, m, qs, d, wl.scale)
    assert st2() == 3
    torch.cuda.synchronize()
    for l in range(3):
        assert torch.equal(st.index_cache[l], st2.index_cache[l])


def test_prefill_1m_full(gpu, orc):
    wl = W.WORKLOADS["prefill_1m"]
    rmap = gpu.reuse_map_last_full(wl.is_full())
    lays, host = build_stack(gpu, wl, rmap, device_gen=True)
    qs = gpu.make_queries(wl.base(), wl.n_valid(), wl.rows(), same_seq=True)
    d = gpu.dims(wl.H_I, wl.D_I, wl.k, wl.H, wl.D_qk, wl.D_v)
    st = gpu.LayerStack(lays, rmap, qs, d, wl.scale)
    assert st() == 1
    torch.cuda.synchronize()
    n = wl.n_valid().numpy()
    k_host = host[0].k_idx.cpu()
    kv_host = [host[l].kv.cpu() for l in range(2)]
    idx_all = st.index_cache[0].cpu().numpy()
    for t in (0, 1, 2047, 4095):
        nt = np.array([n[t]], np.int32)
        I = orc.indexer_scores(host[0].q_idx[t:t + 1].cpu(), host[0].w[t:t + 1].cpu(), k_host[:n[t]],
                               np.array([0], np.int64), nt)
        ref_idx = orc.topk(I.astype(np.float32), nt, wl.k)
        assert np.array_equal(idx_all[t], ref_idx[0]), f"query {t}"
        for l in range(2):
            ref = orc.sparse_mla(host[l].q[t:t + 1].cpu(), kv_host[l], np.array([0], np.int64), ref_idx,
                                 host[l].sink.cpu(), wl.scale, wl.D_v)
            got = lays[l]["out"][t:t + 1].float().cpu().numpy()
            assert_close(got, ref, f"prefill_1m layer {l} query {t} [bf16]")
    # every row: a valid index set of the right size
    assert (idx_all >= 0).all() and (np.diff(idx_all, axis=1) > 0).all()
    assert (idx_all < n[:, None]).all()
    # every row against its own scores (recomputed by the indexer, exact):
    # no unselected score above a selected one, ties at the threshold taken
    # in position order
    sc = gpu.indexer_score(lays[0]["q_idx"], lays[0]["w"], lays[0]["k_idx"], qs)
    topk_invariants_gpu(sc, torch.from_numpy(n).cuda(), st.index_cache[0].long())


def topk_invariants_gpu(sc, n, idx, rows=256):
    """Row-by-row (in chunks) check of a top-k index set on the device."""
    T, ld = sc.shape
    pos = torch.arange(ld, device=sc.device)
    for r0 in range(0, T, rows):
        r1 = min(T, r0 + rows)
        s = sc[r0:r1]
        valid = pos[None, :] < n[r0:r1, None]
        sel = torch.zeros_like(valid)
        sel.scatter_(1, idx[r0:r1], True)
        assert not bool((sel & ~valid).any()), f"rows {r0}..{r1}: index outside the visible tokens"
        lo_sel = torch.where(sel, s, torch.full_like(s, float("inf"))).amin(1)
        hi_rest = torch.where(valid & ~sel, s, torch.full_like(s, float("-inf"))).amax(1)
        assert bool((lo_sel >= hi_rest).all()), f"rows {r0}..{r1}: an unselected score exceeds a selected one"
        tie = lo_sel == hi_rest
        if bool(tie.any()):
            at = s == lo_sel[:, None]
            last_sel = torch.where(sel & at, pos[None, :], torch.full_like(pos[None, :], -1)).amax(1)
            first_rest = torch.where(valid & ~sel & at, pos[None, :], torch.full_like(pos[None, :], ld)).amin(1)
            assert bool((last_sel[tie] < first_rest[tie]).all()), f"rows {r0}..{r1}: tie rule violated"
