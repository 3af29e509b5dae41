"""Pins for the oracle's indexer scores (O1).

Independent checks: numpy int64 einsum on integer inputs (library routine),
closed forms with constant inputs, and the placement of each query's rows."""
import numpy as np
import pytest
import torch

from cross_layer_index_amd import workloads as W


def fp8_bytes(vals):
    return torch.as_tensor(np.array(vals, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def int_ref(q_int, w, k_int, base, n):
    """numpy int64 reference: per-head dots as exact integers, then weights."""
    T = q_int.shape[0]
    out = np.full((T, int(n.max())), np.nan)
    for t in range(T):
        rows = k_int[base[t]:base[t] + n[t]].astype(np.int64)
        dots = np.einsum("hd,sd->hs", q_int[t].astype(np.int64), rows)
        out[t, :n[t]] = (w[t][:, None].astype(np.float64) * np.maximum(dots, 0)).sum(0)
    return out


@pytest.mark.parametrize("name", ["tiny_2layer", "decode_128k"])
def test_against_int64_einsum(orc, name):
    wl = W.WORKLOADS[name]
    if name == "decode_128k":
        wl = W.scaled(wl, lengths=[3000])
    li = W.layer_inputs(wl, 0)
    n = wl.n_valid().numpy()
    base = wl.base().numpy()
    q_int = li.q_idx.view(torch.float8_e4m3fn).to(torch.float32).numpy().astype(np.int64)
    k_int = li.k_idx.view(torch.float8_e4m3fn).to(torch.float32).numpy().astype(np.int64)
    got = orc.indexer_scores(li.q_idx, li.w, li.k_idx, base, n)
    ref = int_ref(q_int, li.w.numpy(), k_int, base, n)
    assert np.array_equal(got, ref)
    # every partial sum is an integer well inside fp32's exact range
    assert np.abs(got).max() < 2 ** 24


@pytest.mark.parametrize("c", [-3.0, 0.0, 2.0, 0.5])
def test_closed_form_constant(orc, c):
    H_I, D_I, L = 4, 32, 40
    q = fp8_bytes(np.ones((1, H_I, D_I)))
    k = fp8_bytes(np.full((L, D_I), c))
    w = np.array([[1.0, 2.0, 3.0, 0.5]], np.float32)
    got = orc.indexer_scores(q, w, k, np.array([0]), np.array([L], np.int32))
    assert np.all(got == D_I * max(c, 0.0) * w.sum())


def test_closed_form_signed_heads(orc):
    """Heads whose dot is negative contribute nothing (ReLU before the weight)."""
    H_I, D_I, L = 6, 64, 10
    sign = np.array([1, -1, 1, -1, 1, -1], np.float32)
    q = fp8_bytes(np.broadcast_to(sign[None, :, None], (1, H_I, D_I)))
    w = np.array([[1, 2, 3, 4, 5, 6]], np.float32)
    for c in (3.0, -2.0):
        k = fp8_bytes(np.full((L, D_I), c))
        got = orc.indexer_scores(q, w, k, np.array([0]), np.array([L], np.int32))
        pos_heads = (sign * c) > 0
        assert np.all(got == D_I * abs(c) * w[0][pos_heads].sum())


def test_rows_follow_base_and_length(orc):
    """Query t scores rows base_t .. base_t+n_t-1 in order, nothing else."""
    H_I, D_I = 2, 32
    vals = np.array([(r % 7) - 3 for r in range(50)], np.float32)   # row r holds constant vals[r]
    k = fp8_bytes(np.repeat(vals[:, None], D_I, 1))
    q = fp8_bytes(np.ones((3, H_I, D_I)))
    w = np.ones((3, H_I), np.float32)
    base = np.array([0, 17, 30], np.int64)
    n = np.array([17, 13, 20], np.int32)
    got = orc.indexer_scores(q, w, k, base, n, ld=24)
    for t in range(3):
        exp = D_I * H_I * np.maximum(vals[base[t]:base[t] + n[t]], 0)
        assert np.array_equal(got[t, :n[t]], exp)
        assert np.all(np.isnan(got[t, n[t]:]))


def test_nan_codes_rejected(orc):
    """The fp8 NaN codes lie outside the indexer's input domain."""
    q = np.zeros((1, 1, 32), np.uint8)
    w = np.ones((1, 1), np.float32)
    k = np.zeros((4, 32), np.uint8)
    for bad in (0x7F, 0xFF):
        kk = k.copy()
        kk[2, 5] = bad
        with pytest.raises(ValueError):
            orc.indexer_scores(q, w, kk, np.array([0], np.int64), np.array([4], np.int32))
        qq = q.copy()
        qq[0, 0, 3] = bad
        with pytest.raises(ValueError):
            orc.indexer_scores(qq, w, k, np.array([0], np.int64), np.array([4], np.int32))
