"""Plant plausible mistakes in the oracle (on the CPU) and check that at least
one pin in test_oracle_rkv.py / test_oracle_refreekv.py fails for each.

This is what makes the pins worth trusting: a dropped term, a wrong sign, a
wrong index or a transposed operand anywhere in the oracle must be caught.
"""

import inspect

import numpy as np
import pytest

from oracle import refreekv as rf
from oracle import rkv
from tests import test_oracle_refreekv as pins_rf
from tests import test_oracle_rkv as pins_rkv


def _run_pins(module):
    """Call every pin of ``module``; return how many raised."""
    failures = 0
    for name, fn in inspect.getmembers(module, inspect.isfunction):
        if not name.startswith("test_") or fn.__module__ != module.__name__:
            continue
        params = [m for m in getattr(fn, "pytestmark", []) if m.name == "parametrize"]
        calls = [{}]
        if params:
            argname, values = params[0].args[0], list(params[0].args[1])
            calls = [{argname: v} for v in values[:6]]
        for kw in calls:
            try:
                with np.errstate(all="ignore"):
                    fn(**kw)
            except Exception:
                failures += 1
    return failures


def _softmax_rows(s):
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    return p / p.sum(axis=1, keepdims=True)


def _imp_no_scale(q, k):
    return _softmax_rows(np.asarray(q, float) @ np.asarray(k, float).T).mean(axis=0)


def _imp_max_pool(q, k):
    d = np.asarray(k).shape[1]
    p = _softmax_rows(np.asarray(q, float) @ np.asarray(k, float).T / np.sqrt(d))
    return p.max(axis=0)


def _imp_wrong_axis(q, k):
    d = np.asarray(k).shape[1]
    s = (np.asarray(q, float) @ np.asarray(k, float).T / np.sqrt(d)).T
    return _softmax_rows(s).T.mean(axis=0)


def _red_with_diag(k):
    u = rkv.unit_keys(k)
    n = len(u)
    return (u @ u.T).sum(axis=0) / max(n - 1, 1)


def _red_over_n(k):
    u = rkv.unit_keys(k)
    n = len(u)
    c = u @ u.T
    c[np.arange(n), np.arange(n)] = 0
    return c.sum(axis=0) / n


def _red_unnormalised(k):
    k = np.asarray(k, float)
    n = len(k)
    c = k @ k.T
    c[np.arange(n), np.arange(n)] = 0
    return c.sum(axis=0) / max(n - 1, 1)


def _combine_plus(i, r, lam):
    return lam * np.asarray(i) + (1 - lam) * np.asarray(r)


def _combine_swapped(i, r, lam):
    return (1 - lam) * np.asarray(i) - lam * np.asarray(r)


def _top_ties_high(z, budget):
    z = np.asarray(z, float)
    n = len(z)
    if n <= budget:
        return np.arange(n)
    order = np.lexsort((-np.arange(n), -z))
    return np.sort(order[:budget])


def _top_unsorted(z, budget):
    z = np.asarray(z, float)
    n = len(z)
    if n <= budget:
        return np.arange(n)
    return np.lexsort((np.arange(n), -z))[:budget]


def _rank_no_sinks(n, m):
    return np.arange(n - 1, -1, -1)


def _rank_sinks_last(n, m):
    s = min(m, n)
    return np.concatenate([np.arange(n - 1, s - 1, -1), np.arange(s)]).astype(np.int64)


def _energy_linear(a):
    return np.asarray(a, float).sum(axis=0)


def _cut_off_by_one(e, m, T):
    e = np.asarray(e, float)
    n = len(e)
    if n == 0:
        return 0
    c = np.cumsum(e[rf.rank_order(n, m)])
    p = int(np.argmax(c >= (1 - T) * c[-1]))
    return max(min(m, n), p)


def _cut_wrong_threshold(e, m, T):
    e = np.asarray(e, float)
    n = len(e)
    if n == 0:
        return 0
    c = np.cumsum(e[rf.rank_order(n, m)])
    p = int(np.argmax(c >= T * c[-1])) + 1
    return max(min(m, n), p)


def _attn_no_scale(q, k):
    return _softmax_rows(np.asarray(q, float) @ np.asarray(k, float).T)


MUTANTS = [
    (rkv, "importance", _imp_no_scale, pins_rkv),
    (rkv, "importance", _imp_max_pool, pins_rkv),
    (rkv, "importance", _imp_wrong_axis, pins_rkv),
    (rkv, "redundancy", _red_with_diag, pins_rkv),
    (rkv, "redundancy", _red_over_n, pins_rkv),
    (rkv, "redundancy", _red_unnormalised, pins_rkv),
    (rkv, "combine", _combine_plus, pins_rkv),
    (rkv, "combine", _combine_swapped, pins_rkv),
    (rkv, "top_budget", _top_ties_high, pins_rkv),
    (rkv, "top_budget", _top_unsorted, pins_rkv),
    (rf, "rank_order", _rank_no_sinks, pins_rf),
    (rf, "rank_order", _rank_sinks_last, pins_rf),
    (rf, "energies", _energy_linear, pins_rf),
    (rf, "cut_length", _cut_off_by_one, pins_rf),
    (rf, "cut_length", _cut_wrong_threshold, pins_rf),
    (rf, "last_row_attention", _attn_no_scale, pins_rf),
]


def test_unmutated_oracle_passes_every_pin():
    assert _run_pins(pins_rkv) == 0
    assert _run_pins(pins_rf) == 0


@pytest.mark.parametrize("mod,attr,mutant,pins", MUTANTS,
                         ids=[f"{m[1]}:{m[2].__name__}" for m in MUTANTS])
def test_each_mutant_fails_a_pin(monkeypatch, mod, attr, mutant, pins):
    monkeypatch.setattr(mod, attr, mutant)
    assert _run_pins(pins) > 0, f"no pin catches {mutant.__name__}"
