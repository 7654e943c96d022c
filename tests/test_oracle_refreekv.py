"""Pins for the ReFreeKV oracle (CPU only).

Closed forms from tests/golden/refreekv_closed_forms.txt (uniform attention,
spikes, geometric energies), a brute-force linear search with exactly rounded
sums, a library softmax, and invariants (kept energy reaches the threshold,
one token less does not; monotone in T; first two layers whole).
"""

import math
import os

import numpy as np
import pytest
import scipy.special

from oracle import refreekv as rf

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _closed_forms(kind):
    rows = []
    with open(os.path.join(GOLDEN, "refreekv_closed_forms.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line.startswith(kind + " "):
                rows.append({k: float(v) for k, v in (t.split("=") for t in line.split()[1:])})
    assert rows
    return rows


def test_rank_order_closed_form():
    assert rf.rank_order(10, 4).tolist() == [0, 1, 2, 3, 9, 8, 7, 6, 5, 4]
    assert rf.rank_order(3, 4).tolist() == [0, 1, 2]
    assert rf.rank_order(5, 4).tolist() == [0, 1, 2, 3, 4]
    assert rf.rank_order(0, 4).tolist() == []


def test_last_row_attention_two_keys():
    # d = 4: logits (q.k)/2 = 3 and 0 -> a0 = e^3/(e^3+1)
    q = np.array([[1.0, 1.0, 1.0, 1.0]])
    k = np.array([[1.5, 1.5, 1.5, 1.5], [0, 0, 0, 0]])
    a0 = math.exp(3.0) / (math.exp(3.0) + 1.0)
    assert rf.last_row_attention(q, k)[0] == pytest.approx([a0, 1 - a0], abs=1e-15)


def test_last_row_attention_matches_library():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((7, 128)) * 3
    k = rng.standard_normal((333, 128))
    want = scipy.special.softmax(q @ k.T / math.sqrt(128), axis=1)
    assert np.allclose(rf.last_row_attention(q, k), want, rtol=1e-12, atol=0)


def test_energy_is_group_frobenius():
    a = np.array([[0.5, 0.5, 0.0], [0.0, 0.25, 0.75]])
    assert rf.energies(a) == pytest.approx([0.25, 0.3125, 0.5625], abs=1e-16)
    assert rf.energies(a).sum() == pytest.approx(np.linalg.norm(a, "fro") ** 2, abs=1e-15)


@pytest.mark.parametrize("row", _closed_forms("uniform"), ids=lambda r: f"n{int(r['n'])}")
def test_uniform_attention_closed_form(row):
    n, m, T, L = int(row["n"]), int(row["m"]), row["T"], int(row["L"])
    d = 16
    rng = np.random.default_rng(n)
    k = rng.standard_normal((1, 1, n, d))
    got, _ = rf.threshold_cut(np.zeros((1, 1, d)), k, [n], layer=5, m=m, T=T)
    assert int(got[0, 0]) == L


@pytest.mark.parametrize("row", _closed_forms("spike"), ids=lambda r: f"t{int(r['t'])}")
def test_spike_attention_closed_form(row):
    n, m, t, T, L = int(row["n"]), int(row["m"]), int(row["t"]), row["T"], int(row["L"])
    d = 8
    k = np.zeros((1, 1, n, d))
    spikes = list(range(m)) + list(range(n - t, n))
    k[0, 0, spikes, 0] = 30.0 * math.sqrt(d)       # logit 30 with q = e0
    q = np.zeros((1, 1, d))
    q[0, 0, 0] = 1.0
    got, _ = rf.threshold_cut(q, k, [n], layer=2, m=m, T=T)
    assert int(got[0, 0]) == L


@pytest.mark.parametrize("row", _closed_forms("geometric"), ids=lambda r: f"r{r['r']}")
def test_geometric_energy_closed_form(row):
    n, m, r, T, L = int(row["n"]), int(row["m"]), row["r"], row["T"], int(row["L"])
    e = np.zeros(n)
    e[m:] = r ** (n - 1 - np.arange(m, n))
    assert rf.cut_length(e, m, T) == L
    # the fixed-point form reaches the same cut on the same energies
    E = np.floor(e * 2.0 ** 52).astype(np.uint64)
    assert rf.cut_length_fixed(E, m, T) == L


def _linear_search(e, m, T):
    """Independent: for p = 1.. test the exactly rounded energy of the first p ranked."""
    n = len(e)
    if n == 0:
        return 0
    order = list(range(min(m, n))) + list(range(n - 1, min(m, n) - 1, -1))
    total = math.fsum(e)
    for p in range(1, n + 1):
        if math.fsum(e[j] for j in order[:p]) >= (1 - T) * total:
            return max(min(m, n), p)
    return n


@pytest.mark.parametrize("seed", range(25))
def test_cut_matches_linear_search(seed):
    rng = np.random.default_rng(200 + seed)
    n = int(rng.integers(1, 300))
    e = rng.exponential(size=n) * (rng.random(n) < 0.7)
    e[-min(5, n):] *= 20
    T = float(rng.choice([0.001, 0.01, 0.1, 0.3]))
    assert rf.cut_length(e, 4, T) == _linear_search(e, 4, T)


@pytest.mark.parametrize("seed", range(10))
def test_cut_invariants_and_monotone(seed):
    rng = np.random.default_rng(300 + seed)
    n, d, g = int(rng.integers(50, 900)), 32, 4
    q = rng.standard_normal((g, d)) * 2
    k = rng.standard_normal((n, d))
    e = rf.energies(rf.last_row_attention(q, k))
    total = e.sum()
    order = rf.rank_order(n, 4)
    prev = n + 1
    for T in [0.0001, 0.001, 0.01, 0.05, 0.1, 0.5]:
        L = rf.cut_length(e, 4, T)
        kept = e[order[:L]].sum()
        assert kept >= (1 - T) * total * (1 - 1e-12)
        if L > 4:
            assert e[order[:L - 1]].sum() < (1 - T) * total
        assert L <= prev
        prev = L
        pos = rf.kept_positions(n, L, 4)
        assert len(pos) == L and sorted(set(order[:L].tolist())) == pos.tolist()


def test_first_layers_keep_everything_and_edges():
    rng = np.random.default_rng(5)
    k = rng.standard_normal((2, 2, 64, 16))
    q = rng.standard_normal((2, 4, 16))
    for layer in (0, 1):
        L, _ = rf.threshold_cut(q, k, [64, 10], layer=layer)
        assert L.tolist() == [[64, 64], [10, 10]]
    L, _ = rf.threshold_cut(q, k, [0, 3], layer=2)
    assert L.tolist() == [[0, 0], [3, 3]]


def test_fixed_point_energies_exact():
    a = np.array([[0.5, 0.25], [0.5, 0.0]], dtype=np.float32)
    E = rf.energies_fixed(a)
    assert E.tolist() == [2 ** 51, 2 ** 48]          # 0.25+0.25 and 1/16, times 2^52


@pytest.mark.parametrize("seed", range(10))
def test_fixed_point_cut_agrees_with_fp64(seed):
    rng = np.random.default_rng(400 + seed)
    n, d, g = int(rng.integers(100, 3000)), 64, 7
    q = rng.standard_normal((g, d)) * 3
    k = rng.standard_normal((n, d))
    a = rf.last_row_attention(q, k)
    L64 = rf.cut_length(rf.energies(a), 4, 0.01)
    Lfx = rf.cut_length_fixed(rf.energies_fixed(a.astype(np.float32)), 4, 0.01)
    # both are valid cuts of the same energies up to fp32 rounding of a
    assert abs(L64 - Lfx) <= 1


# ---------------------------------------------------------------- last k rows

def test_last_rows_zero_query_closed_form():
    # zero queries: row r (token n-k+r) is uniform over its n-k+r+1 visible keys,
    # so e_j = g * sum over rows that see j of 1/(n-k+r+1)^2; rows of tokens
    # before position 0 add nothing
    g, d = 3, 8
    for n, kr in [(50, 1), (50, 7), (6, 9), (1, 4)]:
        k = np.random.default_rng(n + kr).standard_normal((n, d))
        e = rf.energies(rf.last_rows_attention(np.zeros((g, kr, d)), k))
        want = np.zeros(n)
        for j in range(n):
            for r in range(kr):
                last = n - kr + r
                if last >= j:
                    want[j] += g / (last + 1) ** 2
        assert np.allclose(e, want, rtol=1e-13, atol=0), (n, kr)


def test_last_rows_brute_force_loops():
    # per-row softmax over the visible keys written out with scalar loops
    rng = np.random.default_rng(5)
    g, kr, n, d = 2, 3, 5, 4
    q = rng.integers(-2, 3, size=(g, kr, d)).astype(np.float64)
    k = rng.integers(-2, 3, size=(n, d)).astype(np.float64)
    a = rf.last_rows_attention(q, k)
    for qi in range(g):
        for r in range(kr):
            last = n - kr + r
            logits = [sum(q[qi, r, t] * k[j, t] for t in range(d)) / math.sqrt(d)
                      for j in range(last + 1)]
            mx = max(logits)
            ex = [math.exp(x - mx) for x in logits]
            tot = sum(ex)
            for j in range(n):
                want = ex[j] / tot if j <= last else 0.0
                assert abs(a[qi * kr + r, j] - want) < 1e-15


def test_last_rows_k1_is_last_row():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((4, 1, 16))
    k = rng.standard_normal((40, 16))
    assert np.allclose(rf.last_rows_attention(q, k), rf.last_row_attention(q[:, 0], k), rtol=1e-14)


# ------------------------------------------------- GQA grouping, whole calls
#
# Hq = 4 query heads over Hkv = 2 KV heads (g = 2): query heads 0, 1 form KV
# head 0's group and 2, 3 KV head 1's.  Head 0's queries are zero, so its
# attention is uniform whatever its keys (the uniform closed form); head 1's
# queries are e0 and its keys spike (logit 30) on the sinks and on the old
# positions 100..109, so every row spends ~1/14 on each of those 14 tokens and
# the walk (sinks, then newest first) must reach back to position 100:
#   L = m + (n - 100)   since 13/14 of the energy is below 1 - T.
# Head 0's keys spike on positions 200..209 along e0: a grouping that hands
# head 0 one of head 1's e0 queries (for instance a strided q[h::Hkv]) no
# longer sees uniform attention there and cuts near m + (n - 200).

_GN, _GD, _GM, _GT = 1234, 8, 4, 0.01


def _gqa_case(k_rows=None):
    rng = np.random.default_rng(77)
    k = rng.standard_normal((1, 2, _GN, _GD))
    spike = 30.0 * math.sqrt(_GD)                  # logit 30 against e0
    k[0, 0, 200:210, 0] = spike
    k[0, 1] = 0.0
    k[0, 1, list(range(_GM)) + list(range(100, 110)), 0] = spike
    q = np.zeros((1, 4, _GD))
    q[0, 2:, 0] = 1.0
    if k_rows is not None:
        q = np.repeat(q[:, :, None, :], k_rows, axis=2)
    return q, k


def _uniform_causal_cut(n, kr, g, m, T):
    """Kept length for zero queries over the last kr causal rows: token j's
    energy is g * sum over rows r with n-kr+r >= j of 1/(n-kr+r+1)^2; the cut
    by an exactly rounded linear search down the queue."""
    e = [0.0] * n
    for j in range(n):
        e[j] = g * math.fsum(1.0 / (n - kr + r + 1) ** 2 for r in range(kr) if n - kr + r >= j)
    order = list(range(min(m, n))) + list(range(n - 1, min(m, n) - 1, -1))
    total = math.fsum(e)
    acc = []
    for p in range(1, n + 1):
        acc.append(e[order[p - 1]])
        if math.fsum(acc) >= (1 - T) * total:
            return max(min(m, n), p)
    return n


def test_gqa_groups_whole_call_last_row():
    q, k = _gqa_case()
    L, es = rf.threshold_cut(q, k, [_GN], layer=2, m=_GM, T=_GT)
    assert L.tolist() == [[1222, _GM + _GN - 100]]
    # head 0 uniform: every token carries 2/n^2 (two zero queries)
    assert np.allclose(es[(0, 0)], 2.0 / _GN ** 2, rtol=1e-12, atol=0)


def test_gqa_groups_whole_call_rows_k1():
    q, k = _gqa_case(k_rows=1)
    L, _ = rf.threshold_cut_rows(q, k, [_GN], layer=3, m=_GM, T=_GT)
    assert L.tolist() == [[1222, _GM + _GN - 100]]


def test_gqa_groups_whole_call_rows_causal():
    kr = 3
    q, k = _gqa_case(k_rows=kr)
    L, _ = rf.threshold_cut_rows(q, k, [_GN], layer=2, m=_GM, T=_GT)
    want0 = _uniform_causal_cut(_GN, kr, 2, _GM, _GT)
    assert L.tolist() == [[want0, _GM + _GN - 100]]
    # layers below n_full_layers keep everything for both heads
    L, _ = rf.threshold_cut_rows(q, k, [_GN], layer=1, m=_GM, T=_GT)
    assert L.tolist() == [[_GN, _GN]]


def test_gqa_groups_whole_call_from_attn():
    # the same two groups given as fp32 attention rows: rows 0, 1 uniform,
    # rows 2, 3 equal to 1/14 on the sinks and positions 100..109
    a = np.zeros((1, 4, _GN + 6), np.float32)        # cap above n: slots past n ignored
    a[0, :2, :_GN] = np.float32(1.0 / _GN)
    a[0, 2:, list(range(_GM)) + list(range(100, 110))] = np.float32(1.0 / 14)
    a[0, :, _GN:] = 0.5                               # junk past n
    L = rf.threshold_cut_from_attn(a, [_GN], hkv=2, m=_GM, T=_GT)
    assert L.tolist() == [[1222, _GM + _GN - 100]]


@pytest.mark.parametrize("T,m", [(0.001, 4), (0.1, 4), (0.01, 0), (0.01, 10)])
def test_uniform_cut_other_T_and_sinks(T, m):
    # zero query: L = max(min(m, n), ceil((1 - T) n)) when (1 - T) n is not an integer
    n, d = 1237, 16
    k = np.random.default_rng(5).standard_normal((1, 1, n, d))
    got, _ = rf.threshold_cut(np.zeros((1, 1, d)), k, [n], layer=2, m=m, T=T)
    assert int(got[0, 0]) == max(min(m, n), math.ceil((1 - T) * n))


def test_fixed_cut_zero_energy():
    # all-zero rows: the total is 0, tau = 0, and the first queued token
    # already reaches it, so L = max(min(m, n), 1)
    for m in (0, 4):
        for n in (1, 3, 10):
            assert rf.cut_length_fixed(np.zeros(n, np.uint64), m, 0.01) == max(min(m, n), 1)
    assert rf.cut_length_fixed(np.zeros(0, np.uint64), 4, 0.01) == 0
