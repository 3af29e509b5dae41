"""Causal prefill with the bounded collection: the top-k of each query taken
from the scores at or above a bound drawn from a strided sample of its keys,
with whole score rows and the row top-k serving any query the collection
cannot (fewer than k scores at the bound, a chunk's slice past capacity).
The index rows must equal, bit for bit, those of the score-row path (itself
held to the oracle by the parity tests) and the oracle's on sampled queries,
on the collected path, on the forced fallback, and where the sample cannot
bound the k-th key (everything collected)."""
import numpy as np
import pytest
import torch

from checks import report
from cross_layer_index_amd import workloads as W
from test_gpu_full_size import build_stack, topk_invariants_gpu

pytestmark = pytest.mark.gpu

CASES = {
    # 512 queries over ~200K rows: the collection serves every query
    "mid": W.scaled(W.WORKLOADS["prefill_1m"], T=512, prefill_first_pos=199488, prefill_rows=200000),
    # 256 queries over ~3K rows: the sample cannot bound the k-th key, so the
    # collection takes every score
    "short": W.scaled(W.WORKLOADS["prefill_1m"], T=256, prefill_first_pos=3000, prefill_rows=3256),
}


def index_rows(gpu, wl, lays, mode, monkeypatch):
    if mode is None:
        monkeypatch.delenv("IC_PREFILL_TOPK", raising=False)
    else:
        monkeypatch.setenv("IC_PREFILL_TOPK", mode)
    rmap = gpu.reuse_map_last_full(wl.is_full())
    qs = gpu.make_queries(wl.base(), wl.n_valid(), wl.rows(), same_seq=True)
    d = gpu.dims(wl.H_I, wl.D_I, wl.k, wl.H, wl.D_qk, wl.D_v)
    st = gpu.LayerStack(lays, rmap, qs, d, wl.scale)
    assert st() == 1
    torch.cuda.synchronize()
    return st.index_cache[0].clone(), [y["out"].clone() for y in lays], qs


@pytest.mark.parametrize("case", list(CASES))
@pytest.mark.parametrize("mode", ["collect", "fallback"])
def test_prefill_collect_equals_score_rows(gpu, orc, monkeypatch, case, mode):
    wl = CASES[case]
    print(f"[case] prefill collect {case} mode={mode} T={wl.T} rows={wl.rows()}", flush=True)
    rmap = gpu.reuse_map_last_full(wl.is_full())
    lays, host = build_stack(gpu, wl, rmap, device_gen=True)
    ref_idx, ref_out, qs = index_rows(gpu, wl, lays, "scores", monkeypatch)
    got_idx, got_out, _ = index_rows(gpu, wl, lays, mode, monkeypatch)
    diff = int((got_idx != ref_idx).sum().item())
    report(f"prefill {case} {mode}: index entries differing from the score-row path", float(diff))
    assert diff == 0
    for l in range(len(lays)):
        assert torch.equal(got_out[l], ref_out[l]), f"layer {l} output differs"
    n = wl.n_valid().numpy()
    # every row a valid index set, checked against its own scores
    sc = gpu.indexer_score(lays[0]["q_idx"], lays[0]["w"], lays[0]["k_idx"], qs)
    topk_invariants_gpu(sc, torch.from_numpy(n).cuda(), got_idx.long())
    # and the oracle on the first and last query
    k_host = host[0].k_idx.cpu()
    for t in (0, wl.T - 1):
        nt = np.array([n[t]], np.int32)
        I = orc.indexer_scores(host[0].q_idx[t:t + 1].cpu(), host[0].w[t:t + 1].cpu(), k_host[:n[t]],
                               np.array([0], np.int64), nt)
        ref = orc.topk(I.astype(np.float32), nt, wl.k)
        assert np.array_equal(got_idx[t].cpu().numpy(), ref[0]), f"query {t}"
