"""Pins for the R-KV oracle (CPU only).

Each test ties oracle.rkv to something other than itself: hand-derived closed
forms (tests/golden/rkv_duplicate_copy.txt), brute-force subset search with
exact rational sums, independent library routines (scipy softmax, sklearn
cosine similarity) and invariants.  test_oracle_mutants.py plants plausible
mistakes in the oracle and checks that one of these pins fails for each.
"""

import itertools
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.special
from sklearn.metrics.pairwise import cosine_similarity

from oracle import rkv

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, val = line.split("=", 1)
            vals[key.strip()] = [float(x) for x in val.split()]
    return vals


# ---------------------------------------------------------------- importance

def test_importance_two_keys_closed_form():
    # d = 4, q = (1,1,1,1), k0 = q, k1 = 0: logits 4/sqrt(4) = 2 and 0,
    # so I0 = e^2/(e^2+1) (the 1/sqrt(d) scale is pinned by the 2).
    q = np.ones((1, 4))
    k = np.stack([np.ones(4), np.zeros(4)])
    got = rkv.importance(q, k)
    want0 = math.exp(2.0) / (math.exp(2.0) + 1.0)
    assert got == pytest.approx([want0, 1.0 - want0], abs=1e-15)


def test_importance_zero_query_is_uniform():
    rng = np.random.default_rng(1)
    k = rng.standard_normal((37, 16))
    got = rkv.importance(np.zeros((8, 16)), k)
    assert np.allclose(got, 1.0 / 37, atol=1e-16, rtol=0)


def test_importance_pools_rows_by_mean():
    # row 0 attends only to key 0, row 1 only to key 1 (logit gap 200): I ~ [.5, .5, 0]
    d = 4
    k = np.array([[100.0, 0, 0, 0], [0, 100.0, 0, 0], [0, 0, 0, 0]])
    q = np.array([[2.0 * math.sqrt(d), 0, 0, 0], [0, 2.0 * math.sqrt(d), 0, 0]])
    got = rkv.importance(q, k)
    assert got == pytest.approx([0.5, 0.5, 0.0], abs=1e-80)


def test_importance_matches_library_softmax():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((32, 64)) * 2
    k = rng.standard_normal((300, 64))
    logits = q @ k.T / 8.0
    want = scipy.special.softmax(logits, axis=1).mean(axis=0)
    assert np.allclose(rkv.importance(q, k), want, rtol=1e-12, atol=0)


def test_importance_is_a_distribution():
    rng = np.random.default_rng(3)
    got = rkv.importance(rng.standard_normal((12, 32)) * 3, rng.standard_normal((500, 32)))
    assert abs(got.sum() - 1.0) < 1e-13 and (got >= 0).all() and (got <= 1).all()


# ---------------------------------------------------------------- redundancy

def test_redundancy_identical_keys_is_one():
    k = np.tile(np.array([[0.3, -1.0, 2.0, 0.5]]), (9, 1)) * np.arange(1, 10)[:, None]
    assert np.allclose(rkv.redundancy(k), 1.0, atol=1e-15)


def test_redundancy_orthonormal_is_zero():
    k = np.eye(8)[:6] * 3.0
    assert np.allclose(rkv.redundancy(k), 0.0, atol=0)


def test_redundancy_planar_triangle():
    # three unit keys 120 degrees apart: every cosine is -1/2, so R = -1/2
    ang = np.array([0, 2 * np.pi / 3, 4 * np.pi / 3])
    k = np.stack([np.cos(ang), np.sin(ang), np.zeros(3)], axis=1) * [[1], [5], [0.2]]
    assert np.allclose(rkv.redundancy(k), -0.5, atol=1e-15)


def test_redundancy_zero_key_counts_in_denominator():
    # keys e0, e0, 0: R[0] = (1 + 0)/2, R[1] = (1 + 0)/2, R[2] = 0
    k = np.array([[1.0, 0], [2.0, 0], [0.0, 0]])
    assert rkv.redundancy(k) == pytest.approx([0.5, 0.5, 0.0], abs=1e-16)


def test_redundancy_single_key():
    assert rkv.redundancy(np.ones((1, 4))).tolist() == [0.0]


def test_redundancy_matches_library_cosine():
    rng = np.random.default_rng(4)
    k = rng.standard_normal((257, 24))
    c = cosine_similarity(k)
    want = (c.sum(axis=0) - np.diag(c)) / 256
    assert np.allclose(rkv.redundancy(k), want, rtol=0, atol=1e-13)


def test_redundancy_keysum_equals_definition():
    rng = np.random.default_rng(5)
    k = rng.standard_normal((400, 64))
    k[7] = 0.0
    k[100:140] = k[20:60] + 0.01 * rng.standard_normal((40, 64))
    assert np.max(np.abs(rkv.redundancy_keysum(k) - rkv.redundancy(k))) < 1e-14


def test_redundancy_rows_equals_definition():
    rng = np.random.default_rng(6)
    k = rng.standard_normal((300, 16))
    rows = [0, 5, 299, 150]
    assert np.allclose(rkv.redundancy_rows(k, rows), rkv.redundancy(k)[rows], atol=1e-15)


def test_redundancy_scale_invariant():
    rng = np.random.default_rng(7)
    k = rng.standard_normal((50, 8))
    scaled = k * rng.uniform(0.1, 10.0, size=(50, 1))
    assert np.allclose(rkv.redundancy(k), rkv.redundancy(scaled), atol=1e-14)


# ---------------------------------------------------------------- combine

def test_combine_values_and_limits():
    i_sc = np.array([0.5, 0.25, 0.25])
    r_sc = np.array([0.1, -0.2, 0.4])
    assert rkv.combine(i_sc, r_sc, 0.25) == pytest.approx([0.05, 0.2125, -0.2375], abs=1e-16)
    assert np.array_equal(rkv.combine(i_sc, r_sc, 1.0), i_sc)
    assert np.array_equal(rkv.combine(i_sc, r_sc, 0.0), -r_sc)


# ---------------------------------------------------------------- selection

def _brute_top(z, budget):
    """Best subset by exact rational sum; ties -> lexicographically smallest."""
    n = len(z)
    zf = [Fraction(float(x)) for x in z]
    best, best_set = None, None
    for sub in itertools.combinations(range(n), min(budget, n)):
        s = sum((zf[i] for i in sub), Fraction(0))
        if best is None or s > best:
            best, best_set = s, sub
    return list(best_set)


@pytest.mark.parametrize("seed", range(40))
def test_top_budget_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(1, 13))
    budget = int(rng.integers(1, 7))
    # few distinct values so that ties are common
    z = rng.integers(-3, 4, size=n) * 0.125 + (rng.random(n) < 0.3) * 1e-3
    assert rkv.top_budget(z, budget).tolist() == _brute_top(z, budget)


def test_top_budget_shape_and_order():
    rng = np.random.default_rng(8)
    z = rng.standard_normal(1000)
    got = rkv.top_budget(z, 100)
    assert len(got) == 100 and len(set(got.tolist())) == 100
    assert (np.diff(got) > 0).all() and got.min() >= 0 and got.max() < 1000
    assert z[got].min() > np.delete(z, got).max()
    assert rkv.top_budget(z[:40], 100).tolist() == list(range(40))


def test_top_budget_permutation_equivariant():
    rng = np.random.default_rng(9)
    z = rng.standard_normal(200)
    perm = rng.permutation(200)
    a = set(rkv.top_budget(z, 30).tolist())
    b = set(perm[rkv.top_budget(z[perm], 30)].tolist())
    assert a == b


@pytest.mark.parametrize("seed", range(12))
def test_per_head_budgets_brute_force(seed):
    # each KV head keeps the best subset of its own (clamped) size, and the
    # head index of the budget row matches the head of the scores
    rng = np.random.default_rng(300 + seed)
    hkv, n, d, w, budget = 3, int(rng.integers(1, 10)), 4, 2, 5
    q = rng.integers(-2, 3, size=(1, hkv, w, d)).astype(np.float64)
    k = rng.integers(-2, 3, size=(1, hkv, n, d)).astype(np.float64)
    budgets = rng.integers(-2, budget + 3, size=hkv)
    out = rkv.score_evict(q, k, k, [n], 0.1, budget, budgets=budgets)
    for h in range(hkv):
        bh = min(max(int(budgets[h]), 0), budget)
        want = _brute_top(out["Z"][0][h], bh)
        got = out["idx"][0, h]
        assert got[:len(want)].tolist() == want
        assert (got[len(want):] == -1).all()


@pytest.mark.parametrize("seed", range(6))
def test_top_budget_nested(seed):
    # with ties going to the lower position, a smaller budget's set lies inside a larger one's
    rng = np.random.default_rng(400 + seed)
    z = rng.integers(-5, 6, size=300) * 0.25
    prev = set()
    for budget in range(0, 301, 7):
        cur = set(rkv.top_budget(z, budget).tolist())
        assert prev <= cur and len(cur) == min(budget, 300)
        prev = cur


@pytest.mark.parametrize("seed", range(30))
def test_evict_slots_brute_force(seed):
    # a slot-ordered cache holding tokens in permuted positions: the kept set is
    # the best subset under the tie rule applied to positions (brute force over
    # subsets in position order), the evicted slots are the rest
    rng = np.random.default_rng(500 + seed)
    n = int(rng.integers(1, 12))
    budget = int(rng.integers(0, 8))
    z = rng.integers(-2, 3, size=n) * 0.25
    pos = rng.permutation(1000)[:n]
    order = np.argsort(pos)                       # slots by token position
    kept = set(order[_brute_top(z[order], budget)].tolist())
    want = [s for s in range(n) if s not in kept]
    assert rkv.evict_slots(z, budget, pos).tolist() == want


def test_evict_slots_identity_positions_complement_top_budget():
    rng = np.random.default_rng(11)
    for n, budget in [(500, 100), (64, 64), (64, 65), (300, 1)]:
        z = rng.integers(-20, 20, size=n) * 0.5
        keep = set(rkv.top_budget(z, budget).tolist())
        assert rkv.evict_slots(z, budget).tolist() == [s for s in range(n) if s not in keep]


def test_duplicate_copy_golden():
    g = _golden("rkv_duplicate_copy.txt")
    d, n, budget = int(g["d"][0]), int(g["n"][0]), int(g["budget"][0])
    k = np.zeros((n, d))
    k[np.arange(5), np.arange(5)] = 1.0
    k[5] = k[2]
    q = np.zeros((1, 1, 1, d))
    out = rkv.score_evict(q, k[None, None], k[None, None], [n], g["lam"][0], budget)
    assert np.allclose(out["I"][0][0], g["I"], atol=1e-16)
    assert np.allclose(out["R"][0][0], g["R"], atol=1e-16)
    assert np.allclose(out["Z"][0][0], g["Z"], atol=1e-16)
    assert out["idx"][0, 0].tolist() == [int(x) for x in g["keep"]]


def test_lambda_one_is_attention_top_b():
    rng = np.random.default_rng(10)
    q = rng.standard_normal((1, 4, 8, 16)) * 2
    k = rng.standard_normal((1, 1, 120, 16))
    out = rkv.score_evict(q, k, k, [120], 1.0, 20)
    attn = scipy.special.softmax(q[0].reshape(32, 16) @ k[0, 0].T / 4.0, axis=1).mean(axis=0)
    want = np.sort(np.argsort(-attn, kind="stable")[:20])
    assert out["idx"][0, 0].tolist() == want.tolist()


def test_lambda_zero_is_least_redundant():
    rng = np.random.default_rng(11)
    k = rng.standard_normal((1, 1, 90, 8))
    out = rkv.score_evict(rng.standard_normal((1, 1, 8, 8)), k, k, [90], 0.0, 15)
    c = cosine_similarity(k[0, 0])
    r = (c.sum(axis=0) - 1.0) / 89
    assert out["idx"][0, 0].tolist() == np.sort(np.argsort(r, kind="stable")[:15]).tolist()


def test_gqa_groups_are_contiguous():
    # Hq = 4, Hkv = 2: q heads 2,3 belong to KV head 1.  Only they point at key 5.
    d = 8
    k = np.zeros((1, 2, 10, d))
    k[0, :, 5, 0] = 10.0
    q = np.zeros((1, 4, 2, d))
    q[0, 2:, :, 0] = 10.0
    out = rkv.score_evict(q, k, k, [10], 1.0, 3)
    assert np.allclose(out["I"][0][0], 0.1, atol=1e-16)         # KV head 0: uniform
    assert out["I"][0][1][5] > 0.99                               # KV head 1: key 5


def test_score_evict_compaction_and_padding():
    rng = np.random.default_rng(12)
    b, hq, hkv, w, d, cap, budget = 3, 4, 2, 2, 8, 40, 16
    q = rng.standard_normal((b, hq, w, d))
    k = rng.standard_normal((b, hkv, cap, d)).astype(np.float32)
    v = rng.standard_normal((b, hkv, cap, d)).astype(np.float32)
    lengths = [40, 9, 16]
    out = rkv.score_evict(q, k, v, lengths, 0.1, budget)
    for bi in range(b):
        m = min(lengths[bi], budget)
        for h in range(hkv):
            idx = out["idx"][bi, h]
            assert (idx[:m] >= 0).all() and (idx[m:] == -1).all()
            assert np.array_equal(out["k_out"][bi, h, :m], k[bi, h, idx[:m]])
            assert np.array_equal(out["v_out"][bi, h, :m], v[bi, h, idx[:m]])
