"""ic_layer_stack_static (the library's own scratch, no allocation in the
call) against ic_layer_stack with a caller workspace: the same index sets and
outputs bit for bit, on two calls in a row, the second with a smaller input,
through the C ABI."""
import ctypes

import numpy as np
import pytest
import torch

from cross_layer_index_amd import workloads as W

pytestmark = pytest.mark.gpu


def stack_for(ic, wl, out_f32):
    rmap = ic.reuse_map_last_full(wl.is_full())
    lays = []
    for l in range(wl.n_layers):
        li = W.layer_inputs(wl, l, device="cuda", with_indexer=rmap[l] == l)
        lays.append(dict(q_idx=li.q_idx, w=li.w, k_idx=li.k_idx, q=li.q, kv=li.kv, sink=li.sink,
                         out=torch.empty((wl.T, wl.H, wl.D_v), dtype=torch.float32 if out_f32 else torch.bfloat16,
                                         device="cuda")))
    qs = ic.make_queries(wl.base(), wl.n_valid(), wl.rows(), wl.same_seq, group=wl.group)
    d = ic.dims(wl.H_I, wl.D_I, wl.k, wl.H, wl.D_qk, wl.D_v, out_f32)
    return ic.LayerStack(lays, rmap, qs, d, wl.scale), lays


def run_both(ic, wl, out_f32):
    st, lays = stack_for(ic, wl, out_f32)
    assert st() == sum(wl.is_full())
    torch.cuda.synchronize()
    ref_out = [y["out"].clone() for y in lays]
    ref_idx = st.index_cache.clone()
    for y in lays:
        y["out"].fill_(float("nan"))
    st.index_cache.fill_(-7)
    torch.cuda.synchronize()
    assert st.call_static() == sum(wl.is_full())
    torch.cuda.synchronize()
    assert torch.equal(st.index_cache, ref_idx), f"{wl.name}: index cache differs"
    for l, y in enumerate(lays):
        assert torch.equal(y["out"], ref_out[l]), f"{wl.name}: layer {l} output differs"


def test_static_stack_matches_workspace_stack(gpu):
    """decode_128k (one full layer, batch 1, 131,072 tokens), then a smaller
    3-layer stack (batch 2, 20,000 and 7,000 tokens, shared layer in the
    middle), both against the workspace entry point."""
    run_both(gpu, W.WORKLOADS["decode_128k"], out_f32=False)
    small = W.scaled(W.WORKLOADS["decode_128k"], T=2, lengths=[20000, 7000], n_layers=3, full_layers=[0, 2])
    run_both(gpu, small, out_f32=True)
