"""Host logic of the binding's prepared calls (no GPU): a PreparedCall issues its function
with the arguments it was given, again on every call, runs its pre-issue hook first, and
turns a non-zero status into Csa2Error; _issue issues at once unless asked to prepare."""
import pytest

import compressed_sparse_kv_csa2_amd as csa2
from compressed_sparse_kv_csa2_amd import PreparedCall, _issue


def test_prepared_call_reissues_the_same_arguments():
    seen = []
    call = PreparedCall(lambda *a: seen.append(a) or 0, (1, "x", 2.5))
    call()
    call()
    assert seen == [(1, "x", 2.5), (1, "x", 2.5)]


def test_prepared_call_runs_its_hook_before_each_issue():
    order = []
    call = PreparedCall(lambda: order.append("call") or 0, (), pre=lambda: order.append("pre"))
    call()
    call()
    assert order == ["pre", "call", "pre", "call"]


def test_hook_failure_stops_the_issue():
    issued = []

    def bad():
        raise csa2.Csa2Error("list out of range")

    call = PreparedCall(lambda: issued.append(1) or 0, (), pre=bad)
    with pytest.raises(csa2.Csa2Error):
        call()
    assert issued == []


def test_issue_prepares_or_issues():
    seen = []
    fn = lambda *a: seen.append(a) or 0
    assert _issue(fn, (7,), prepare=False) is None and seen == [(7,)]
    p = _issue(fn, (8,), prepare=True)
    assert isinstance(p, PreparedCall) and seen == [(7,)]
    p()
    assert seen == [(7,), (8,)]
