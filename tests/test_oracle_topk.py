"""Pins for the oracle's top-k selection (O2).

Brute force by rank on tiny, tie-heavy inputs: a position is kept exactly when
fewer than k positions beat it (a larger score, or an equal score at a lower
position). That definition is independent of the oracle's sort."""
import numpy as np
import pytest

from checks import check_topk_invariants


def brute_force(scores, n, k):
    T = scores.shape[0]
    out = np.full((T, k), -1, np.int32)
    for t in range(T):
        sel = []
        for s in range(n[t]):
            beats = sum(1 for u in range(n[t])
                        if scores[t, u] > scores[t, s] or (scores[t, u] == scores[t, s] and u < s))
            if beats < k:
                sel.append(s)
        out[t, :len(sel)] = sel
    return out


@pytest.mark.parametrize("seed", range(6))
def test_brute_force_ties(orc, seed):
    rng = np.random.default_rng(seed)
    T = 5
    n = np.array([0, 1, 7, 40, 200], np.int32)
    scores = rng.integers(-1, 2, size=(T, 200)).astype(np.float32)
    for k in (1, 3, 7, 8, 39, 64, 250):
        got = orc.topk(scores, n, k)
        assert np.array_equal(got, brute_force(scores, n, k)), k
        check_topk_invariants(scores, n, k, got)


@pytest.mark.parametrize("seed", range(3))
def test_brute_force_real_values(orc, seed):
    rng = np.random.default_rng(100 + seed)
    n = np.array([120, 300], np.int32)
    scores = rng.standard_normal((2, 300)).astype(np.float32)
    scores[:, ::9] = 0.25   # a block of equal values
    for k in (5, 64, 119, 120, 121, 299):
        got = orc.topk(scores, n, k)
        assert np.array_equal(got, brute_force(scores, n, k))


def test_short_rows_keep_everything(orc):
    n = np.array([0, 1, 5], np.int32)
    got = orc.topk(np.zeros((3, 8), np.float32), n, 6)
    assert got.tolist() == [[-1] * 6, [0] + [-1] * 5, [0, 1, 2, 3, 4, -1]]


def test_signed_zero_is_one_value(orc):
    scores = np.array([[-0.0, 0.0, -0.0, 0.0]], np.float32)
    assert orc.topk(scores, np.array([4], np.int32), 2).tolist() == [[0, 1]]


def test_large_row_invariants(orc):
    rng = np.random.default_rng(7)
    n = np.array([131072], np.int32)
    scores = rng.integers(0, 40000, size=(1, 131072)).astype(np.float32)
    idx = orc.topk(scores, n, 2048)
    check_topk_invariants(scores, n, 2048, idx)
