"""Pins for the layer-stack rule (O4) and the counts the pages print.

The explainer page ("Hy4 IndexCache cross-layer index reuse", section "Where
the saving actually lands") prints index-score counts per decoded token; the
GitHub issue ("rtx6kpro #90", "Indexer:" bullet) gives the reuse rule and the
21-of-78 pattern. Those figures live in tests/golden/index_score_counts.txt."""
import os

import numpy as np
import pytest

from cross_layer_index_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "index_score_counts.txt")


def golden():
    d = {}
    for line in open(GOLDEN):
        line = line.strip()
        if line and not line.startswith("#"):
            k, v = line.split()
            d[k] = v
    return d


def test_printed_counts(orc):
    g = golden()
    L, ctx = int(g["layers"]), int(g["context_tokens"])
    per_layer = orc.reuse_map_last_full([True] * L)
    one_index = orc.reuse_map_last_full([True] + [False] * (L - 1))
    every = int(g["refresh_every"])
    every_map = orc.reuse_map_last_full([l % every == 0 for l in range(L)])
    assert orc.indexer_passes(per_layer) * ctx == int(g["per_layer_index_scores"])
    assert orc.indexer_passes(one_index) * ctx == int(g["one_shared_index_scores"])
    assert orc.indexer_passes(every_map) == int(g["refresh_every_index_builds"])
    hy4 = orc.reuse_map_last_full(W.WORKLOADS["stack_78"].is_full())
    assert orc.indexer_passes(hy4) == int(g["hy4_full_layers"])
    pat = "".join("F" if hy4[l] == l else "S" for l in range(L))
    assert pat.startswith(g["hy4_pattern_prefix"])


def test_hy4_map_sources():
    import oracle
    m = oracle.reuse_map_last_full(W.WORKLOADS["stack_78"].is_full())
    full = [l for l in range(78) if m[l] == l]
    assert full == [0, 1, 2] + list(range(6, 75, 4))
    for l in range(78):
        assert m[l] == max(f for f in full if f <= l)
    assert m[77] == 74 and m[5] == 2 and m[3] == 2 and m[9] == 6


@pytest.mark.parametrize("bad", [[1], [0, 2], [0, 0, 1], [0, 1, 1, 2], [0, -1]])
def test_invalid_maps(orc, bad):
    with pytest.raises(orc.ReuseMapError):
        orc.check_reuse_map(bad)


def test_first_layer_must_be_full(orc):
    with pytest.raises(orc.ReuseMapError):
        orc.reuse_map_last_full([False, True])


def test_stack_shared_layers_inherit(orc):
    """Shared layers carry their source's index unchanged and attend with it;
    full layers select from their own scores."""
    wl = W.scaled(W.WORKLOADS["tiny_2layer"], n_layers=5, full_layers=[0, 3], T=2, lengths=[300, 257])
    layers = [W.layer_inputs(wl, l) for l in range(5)]
    rmap = orc.reuse_map_last_full(wl.is_full())
    base, n = wl.base().numpy(), wl.n_valid().numpy()
    outs, index_of, passes = orc.layer_stack(layers, rmap, base, n, wl.k, wl.scale, wl.D_v)
    assert passes == 2 and rmap == [0, 0, 0, 3, 3]
    for l in range(5):
        src = rmap[l]
        assert np.array_equal(index_of[l], index_of[src])
        own = orc.topk(orc.indexer_scores(layers[src].q_idx, layers[src].w, layers[src].k_idx, base, n)
                       .astype(np.float32), n, wl.k)
        assert np.array_equal(index_of[l], own)
        ref = orc.sparse_mla(layers[l].q, layers[l].kv, base, index_of[src], layers[l].sink, wl.scale, wl.D_v)
        assert np.array_equal(outs[l], ref)
    # a shared layer's own indexer would generally choose differently: the
    # inherited set is the source's, not a recomputation
    own2 = orc.topk(orc.indexer_scores(layers[1].q_idx, layers[1].w, layers[1].k_idx, base, n)
                    .astype(np.float32), n, wl.k)
    assert not np.array_equal(own2, index_of[1])
