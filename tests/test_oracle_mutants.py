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
            names = [a.strip() for a in params[0].args[0].split(",")]
            values = list(params[0].args[1])[:6]
            calls = [dict(zip(names, v if len(names) > 1 else (v,))) for v in values]
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


def _cut_strided(q_last, k, lengths, layer, n_full_layers=2, m=4, T=0.01, heads=None):
    # GQA group of KV head h taken as q heads h, h + Hkv, ... (strided, not contiguous)
    q_last = np.asarray(q_last)
    b, hq, d = q_last.shape
    hkv = k.shape[1]
    L = np.zeros((b, hkv), np.int64)
    es = {}
    for bi in range(b):
        for h in range(hkv):
            n = int(lengths[bi])
            if layer < n_full_layers:
                L[bi, h] = n
                continue
            e = rf.energies(rf.last_row_attention(q_last[bi, h::hkv], k[bi, h, :n]))
            es[(bi, h)] = e
            L[bi, h] = rf.cut_length(e, m, T)
    return L, es


def _cut_rows_strided(q_rows, k, lengths, layer, n_full_layers=2, m=4, T=0.01, heads=None):
    q_rows = np.asarray(q_rows)
    b = q_rows.shape[0]
    hkv = k.shape[1]
    L = np.zeros((b, hkv), np.int64)
    es = {}
    for bi in range(b):
        for h in range(hkv):
            n = int(lengths[bi])
            if layer < n_full_layers:
                L[bi, h] = n
                continue
            e = rf.energies(rf.last_rows_attention(q_rows[bi, h::hkv], k[bi, h, :n]))
            es[(bi, h)] = e
            L[bi, h] = rf.cut_length(e, m, T)
    return L, es


def _from_attn_strided(attn32, lengths, hkv, m=4, T=0.01):
    attn32 = np.asarray(attn32, np.float32)
    b = attn32.shape[0]
    L = np.zeros((b, hkv), np.int64)
    for bi in range(b):
        n = int(lengths[bi])
        for h in range(hkv):
            L[bi, h] = rf.cut_length_fixed(rf.energies_fixed(attn32[bi, h::hkv, :n]), m, T)
    return L


def _last_rows_not_causal(q_rows, k):
    # every row attends to all n keys
    q64 = np.asarray(q_rows, np.float64)
    k64 = np.asarray(k, np.float64)
    g, kr, d = q64.shape
    return _softmax_rows(q64.reshape(g * kr, d) @ k64.T / np.sqrt(d)) if len(k64) else np.zeros((g * kr, 0))


def _energies_fixed_linear(a32):
    # the probability itself rounded, not its square
    a32 = np.asarray(a32, np.float32).astype(np.float64)
    return np.floor(a32 * float(1 << rf.FIX_SHIFT)).astype(np.uint64).sum(axis=0, dtype=np.uint64)


def _evict_ties_by_slot(z, budget, pos=None):
    # equal scores split by slot index instead of token position
    z = np.asarray(z, np.float64)
    n = z.shape[0]
    if n <= budget:
        return np.zeros(0, dtype=np.int64)
    order = np.lexsort((np.arange(n), -z))
    keep = np.zeros(n, dtype=bool)
    keep[order[:max(budget, 0)]] = True
    return np.arange(n)[~keep].astype(np.int64)


def _head_budget_unclamped(budgets, h, budget):
    return budget if budgets is None else int(budgets[h])


def _red_keysum_no_self(k):
    u = rkv.unit_keys(k)
    n = len(u)
    if n <= 1:
        return np.zeros(n)
    return (u @ u.sum(axis=0)) / (n - 1)


def _kept_oldest(n, L, m):
    # the oldest L - m positions after the sinks instead of the newest
    s = min(m, n, L)
    return np.concatenate([np.arange(s), np.arange(s, L)]).astype(np.int64)


def _cut_fixed_no_sink_floor(E, m, T):
    # the walk's length without the floor of m sink tokens
    E = np.asarray(E, np.uint64)
    n = E.shape[0]
    if n == 0:
        return 0
    tau = int(np.ceil(float(int(E.sum(dtype=np.uint64))) * (1.0 - float(np.float32(T)))))
    acc = 0
    for pos, j in enumerate(rf.rank_order(n, m)):
        acc += int(E[j])
        if acc >= tau:
            return pos + 1
    return n


def _unit_keys_squared_norm(k):
    # divided by the squared norm instead of the norm
    k64 = np.asarray(k, np.float64)
    nrm2 = (k64 * k64).sum(axis=1)
    out = np.zeros_like(k64)
    nz = nrm2 > 0
    out[nz] = k64[nz] / nrm2[nz, None]
    return out


def _red_rows_with_self(k, rows):
    # the i == j term left in
    u = rkv.unit_keys(k)
    n = len(u)
    rows = np.asarray(rows, dtype=np.int64)
    if n <= 1:
        return np.zeros(len(rows))
    return (u[rows] @ u.T).sum(axis=1) / (n - 1)


_score_evict_orig = rkv.score_evict


def _score_evict_strided(q, k, v, lengths, lam, budget, form="definition", heads=None,
                         budgets=None):
    # query heads grouped by stride (h, h + Hkv, ...) instead of contiguously
    q = np.asarray(q)
    hkv = k.shape[1]
    g = q.shape[1] // hkv
    perm = np.arange(q.shape[1]).reshape(g, hkv).T.reshape(-1)
    return _score_evict_orig(q[:, perm], k, v, lengths, lam, budget, form, heads, budgets)


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
    (rf, "threshold_cut", _cut_strided, pins_rf),
    (rf, "threshold_cut_rows", _cut_rows_strided, pins_rf),
    (rf, "threshold_cut_from_attn", _from_attn_strided, pins_rf),
    (rf, "last_rows_attention", _last_rows_not_causal, pins_rf),
    (rf, "energies_fixed", _energies_fixed_linear, pins_rf),
    (rkv, "evict_slots", _evict_ties_by_slot, pins_rkv),
    (rkv, "head_budget", _head_budget_unclamped, pins_rkv),
    (rkv, "redundancy_keysum", _red_keysum_no_self, pins_rkv),
    (rf, "kept_positions", _kept_oldest, pins_rf),
    (rf, "cut_length_fixed", _cut_fixed_no_sink_floor, pins_rf),
    (rkv, "unit_keys", _unit_keys_squared_norm, pins_rkv),
    (rkv, "redundancy_rows", _red_rows_with_self, pins_rkv),
    (rkv, "score_evict", _score_evict_strided, pins_rkv),
]


def test_unmutated_oracle_passes_every_pin():
    assert _run_pins(pins_rkv) == 0
    assert _run_pins(pins_rf) == 0


@pytest.mark.parametrize("mod,attr,mutant,pins", MUTANTS,
                         ids=[f"{m[1]}:{m[2].__name__}" for m in MUTANTS])
def test_each_mutant_fails_a_pin(monkeypatch, mod, attr, mutant, pins):
    monkeypatch.setattr(mod, attr, mutant)
    assert _run_pins(pins) > 0, f"no pin catches {mutant.__name__}"
