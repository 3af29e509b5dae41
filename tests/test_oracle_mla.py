"""Pins for the oracle's sparse MLA with sink (O3).

Independent checks: a torch float64 softmax over [scores, sink] with the sink
column dropped from the value sum, torch's scaled_dot_product_attention when
the sink vanishes, and closed forms (zero query, single key, empty selection,
permutation of the index list, linearity in the value part)."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F


def bf16(x):
    return torch.as_tensor(x, dtype=torch.float32).to(torch.bfloat16)


def torch_sink_softmax(q, kv, sink, scale, D_v):
    """q [H, D], kv [n, D] (float64): softmax over the n scores plus one sink
    logit per head, sink column dropped from P·V."""
    s = scale * (q @ kv.T)                       # [H, n]
    logits = torch.cat([s, sink[:, None]], 1)    # [H, n+1]
    p = torch.softmax(logits, 1)[:, :-1]
    return p @ kv[:, :D_v]


def make(seed, T=2, H=3, D_qk=40, D_v=32, rows=70):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(T, H, D_qk, generator=g).to(torch.bfloat16)
    kv = torch.randn(rows, D_qk, generator=g).to(torch.bfloat16)
    sink = torch.randn(H, generator=g)
    return q, kv, sink


@pytest.mark.parametrize("seed", range(3))
def test_dense_equals_torch_sink_softmax(orc, seed):
    q, kv, sink = make(seed)
    base = np.array([0, 30], np.int64)
    n = np.array([30, 40], np.int32)
    scale = 1 / math.sqrt(40)
    got = orc.dense_mla(q, kv, base, n, sink, scale, 32)
    for t in range(2):
        rows = kv[base[t]:base[t] + n[t]].double()
        ref = torch_sink_softmax(q[t].double(), rows, sink.double(), scale, 32).numpy()
        np.testing.assert_allclose(got[t], ref, rtol=1e-12, atol=1e-13)


def test_vanishing_sink_is_sdpa(orc):
    q, kv, _ = make(5, T=1, H=4, D_qk=48, D_v=48, rows=33)
    sink = torch.full((4,), -3.0e38)
    scale = 0.17
    got = orc.dense_mla(q, kv, np.array([0]), np.array([33], np.int32), sink, scale, 48)
    Q = q.double()[0][None, :, None, :]                      # [1, H, 1, D]
    K = kv.double()[None, None].expand(1, 4, 33, 48).contiguous()
    ref = F.scaled_dot_product_attention(Q, K, K, scale=scale)[0, :, 0]   # [H, D]
    np.testing.assert_allclose(got[0], ref.numpy(), rtol=1e-12, atol=1e-13)


def test_zero_query_is_mean_with_sink(orc):
    _, kv, sink = make(2, H=2, D_qk=24, D_v=16, rows=10)
    q = torch.zeros(1, 2, 24, dtype=torch.bfloat16)
    got = orc.dense_mla(q, kv, np.array([0]), np.array([10], np.int32), sink, 0.3, 16)
    v = kv.double()[:, :16].sum(0).numpy()
    for h in range(2):
        np.testing.assert_allclose(got[0, h], v / (10 + math.exp(float(sink[h]))), rtol=1e-13)


def test_single_key_is_sigmoid(orc):
    q, kv, sink = make(3, T=1, H=3, D_qk=24, D_v=16, rows=5)
    idx = np.array([[-1, 3, -1]], np.int32)
    got = orc.sparse_mla(q, kv, np.array([0]), idx, sink, 0.2, 16)
    for h in range(3):
        s = 0.2 * float(q[0, h].double() @ kv[3].double())
        sig = 1 / (1 + math.exp(float(sink[h]) - s))
        np.testing.assert_allclose(got[0, h], kv[3, :16].double().numpy() * sig, rtol=1e-12)


def test_empty_selection_is_zero(orc):
    q, kv, sink = make(4, T=1)
    got = orc.sparse_mla(q, kv, np.array([0]), np.full((1, 6), -1, np.int32), sink, 0.1, 32)
    assert np.all(got == 0)


def test_permutation_and_padding_invariant(orc):
    q, kv, sink = make(6, T=1, H=2, rows=64)
    rng = np.random.default_rng(0)
    sel = rng.choice(64, 20, replace=False).astype(np.int32)
    a = np.concatenate([np.sort(sel), -np.ones(5, np.int32)])[None]
    b = np.insert(rng.permutation(sel), [3, 3, 10, 20, 20], -1).astype(np.int32)[None]
    oa = orc.sparse_mla(q, kv, np.array([0]), a, sink, 0.15, 32)
    ob = orc.sparse_mla(q, kv, np.array([0]), b, sink, 0.15, 32)
    np.testing.assert_allclose(oa, ob, rtol=1e-13, atol=1e-15)


def test_value_is_leading_part_and_linear(orc):
    """With the query zero on the value dims, scores ignore them; scaling the
    value dims by 2 (exact in bf16) scales the output by 2."""
    q, kv, sink = make(7, T=1, H=2, D_qk=40, D_v=32, rows=12)
    q[..., :32] = 0
    kv2 = (kv.float() * torch.cat([torch.full((32,), 2.0), torch.ones(8)])).to(torch.bfloat16)
    n = np.array([12], np.int32)
    o1 = orc.dense_mla(q, kv, np.array([0]), n, sink, 0.2, 32)
    o2 = orc.dense_mla(q, kv2, np.array([0]), n, sink, 0.2, 32)
    np.testing.assert_allclose(o2, 2 * o1, rtol=1e-13)
    ref = torch_sink_softmax(q[0].double(), kv.double(), sink.double(), 0.2, 32).numpy()
    np.testing.assert_allclose(o1[0], ref, rtol=1e-12)


def test_rows_offset_by_base(orc):
    q, kv, sink = make(8, T=2, rows=70)
    idx = np.array([[0, 1, 2, -1], [0, 1, 2, -1]], np.int32)
    base = np.array([10, 50], np.int64)
    got = orc.sparse_mla(q, kv, base, idx, sink, 0.1, 32)
    for t in range(2):
        ref = torch_sink_softmax(q[t].double(), kv[base[t]:base[t] + 3].double(), sink.double(), 0.1, 32)
        np.testing.assert_allclose(got[t], ref.numpy(), rtol=1e-12)
