"""IC_DEBUG=1: the binding reads back the device-resident values that the C
library cannot validate (n_valid, base, index lists; include/ic.h, "Values
that live in device memory") and rejects a contract violation before any
launch. These run on the CPU: the check works on host copies."""
import pytest
import torch

from cross_layer_index_amd import ic


def queries(base, n, rows, same_seq=False, group=1, max_n=None):
    n = torch.tensor(n, dtype=torch.int32)
    return ic.Queries(torch.tensor(base, dtype=torch.int64), n, int(n.max()) if max_n is None else max_n, rows,
                      same_seq, group)


def test_valid_queries_pass():
    ic.check_contract(queries([0, 100, 250], [100, 150, 6], rows=256))
    ic.check_contract(queries([0, 0, 0], [10, 11, 12], rows=12, same_seq=True))
    ic.check_contract(queries([0, 0, 50, 50], [5, 6, 7, 8], rows=58, group=2))
    idx = torch.tensor([[0, 99, -1], [149, -1, 3], [5, 4, -1]], dtype=torch.int32)
    ic.check_contract(queries([0, 100, 250], [100, 150, 6], rows=256), idx)


@pytest.mark.parametrize("case, pattern", [
    (dict(base=[0, 100], n=[100, 200], rows=256), "base \\+ n_valid > rows"),
    (dict(base=[0, -1], n=[10, 10], rows=256), "base < 0"),
    (dict(base=[0, 10], n=[10, -3], rows=256, max_n=10), "n_valid < 0"),
    (dict(base=[0, 10], n=[10, 30], rows=256, max_n=20), "n_valid > max_n"),
    (dict(base=[0, 1], n=[1, 2], rows=4, same_seq=True), "same_seq with unequal bases"),
    (dict(base=[0, 0, 5, 6], n=[1, 2, 1, 1], rows=8, group=2), "unequal bases within a group"),
])
def test_query_violations_rejected(case, pattern):
    with pytest.raises(ic.ICError, match=pattern) as e:
        ic.check_contract(queries(**case))
    assert e.value.status == ic.IC_ERR_SHAPE


@pytest.mark.parametrize("bad", [100, -7, 2_000_000_000])
def test_index_violations_rejected(bad):
    qs = queries([0, 100], [100, 50], rows=150)
    idx = torch.tensor([[0, 1, 2], [3, 4, 5]], dtype=torch.int32)
    idx[0, 2] = bad
    with pytest.raises(ic.ICError, match=r"idx\[0, 2\]"):
        ic.check_contract(qs, idx)


def test_debug_mode_rejects_before_launch(monkeypatch):
    """A call in debug mode rejects a bad list before anything else; without
    debug mode the same (host-resident) arguments fail the binding's device
    check instead, so the contract check is the debug mode's doing."""
    qs = queries([0], [10], rows=10)
    q = torch.zeros(1, 128, 576, dtype=torch.bfloat16)
    kv = torch.zeros(10, 576, dtype=torch.bfloat16)
    idx = torch.tensor([[0, 10]], dtype=torch.int32)          # 10 == n_valid: out of range
    sink = torch.zeros(128)
    monkeypatch.setenv("IC_DEBUG", "1")
    with pytest.raises(ic.ICError, match="contract violated"):
        ic.sparse_mla(q, kv, qs, idx, sink, 0.04, 512)
    monkeypatch.delenv("IC_DEBUG")
    with pytest.raises(TypeError):
        ic.sparse_mla(q, kv, qs, idx, sink, 0.04, 512)
