"""Checks shared by the CPU and GPU tests (no method arithmetic)."""
import numpy as np

# (case, achieved error) of every tolerance check in the run, printed in the
# terminal summary (outside pytest's output capture) by conftest.py
ERRORS = []


def report(what, err):
    ERRORS.append((what, float(err)))


def check_topk_invariants(scores, n, k, idx):
    """Full-size invariant: |S| = min(k, n), distinct, in range, ascending, and
    every kept (score, -pos) key beats every dropped one."""
    for t in range(idx.shape[0]):
        nt = int(n[t])
        kp = min(k, nt)
        row = idx[t]
        sel = row[:kp]
        assert np.all(row[kp:] == -1)
        assert np.all(sel >= 0) and np.all(sel < nt)
        assert np.all(np.diff(sel) > 0)
        if kp < nt:
            sc = scores[t, :nt].astype(np.float32)
            mask = np.zeros(nt, bool)
            mask[sel] = True
            ks, kd = sc[mask], sc[~mask]
            worst_kept = ks.min()
            best_dropped = kd.max()
            assert worst_kept >= best_dropped
            if worst_kept == best_dropped:
                # among the tied score, kept positions all precede dropped ones
                tied_kept = np.nonzero(mask & (sc == worst_kept))[0]
                tied_drop = np.nonzero(~mask & (sc == worst_kept))[0]
                assert tied_kept.max() < tied_drop.min()
