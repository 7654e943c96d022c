"""ReFreeKV threshold cut: plain fp64 CPU oracle.

TEST INFRASTRUCTURE ONLY.  Imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py; never by the product path.  It shares no code
with the HIP library.

Source: the review "论文综述：ReFreeKV：迈向无阈值的KV缓存压缩", section 二
(核心方法与创新): first step (Initial Ranking), second step (Uni-Metric), and the
efficiency paragraph after them; section 七 (mind-map, branch 效率优化).
What the review states:
  * ranking: the first m = 4 tokens stay at the head of the queue in their
    original order; every other token follows, nearest to the current
    position first;
  * walking down that queue, tokens are kept until cutting all the remaining
    ones would lose less than T = 1% of the attention matrix's Frobenius energy;
  * the attention matrix is approximated by its last row (k = 1);
  * the first two layers always keep the whole cache;
  * the walk is a cumulative sum (vectorised, batched), not a loop.

Readings where the review is silent or loose:
  * energy = squared Frobenius norm = sum of squared attention probabilities;
    "keep >= 99%" is C_p >= (1 - T) * E_total with C_p the energy of the first
    p ranked tokens;
  * with grouped-query attention the unit is one KV head and its energy is the
    Frobenius energy of the g last-row query heads of the group together;
  * the attention row is the last token's query over all n cached keys,
    softmax with scale 1/sqrt(d);
  * kept length L = max(min(m, n), smallest p >= 1 with C_p >= (1-T)*E_total);
    n = 0 gives L = 0; layers below n_full_layers give L = n;
  * the kept set is the m sinks plus the last L - m positions;
  * the k > 1 ablation (the review's last paragraph on ablations) uses the
    last k rows of the causal attention matrix: row r is token n - k + r's
    query over keys 0 .. n - k + r; the energy sums over all g*k rows.

Bit-exact decision (reading, used where two implementations must reach the
same integer L from the same fp32 attention probabilities): each squared
probability is rounded to fp32 (one IEEE multiply), scaled by 2^52 and
floored to an integer, and all sums are exact integer sums; the threshold is
ceil(double(E_total) * (1 - double(T))) with T taken as its fp32 value.
"""

from __future__ import annotations

import math

import numpy as np

FIX_SHIFT = 52


def rank_order(n: int, m: int) -> np.ndarray:
    """Queue order: positions 0..m-1, then n-1, n-2, ..., m."""
    s = min(m, n)
    return np.concatenate([np.arange(s), np.arange(n - 1, s - 1, -1)]).astype(np.int64)


def last_row_attention(q_rows: np.ndarray, k: np.ndarray) -> np.ndarray:
    """a[q, j] = softmax_j(q_rows[q].k[j] / sqrt(d)) in fp64; q_rows [g, d], k [n, d]."""
    q64 = np.asarray(q_rows, np.float64)
    k64 = np.asarray(k, np.float64)
    n, d = k64.shape
    if n == 0:
        return np.zeros((q64.shape[0], 0))
    s = (q64 @ k64.T) / np.sqrt(d)
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    return p / p.sum(axis=1, keepdims=True)


def last_rows_attention(q_rows: np.ndarray, k: np.ndarray) -> np.ndarray:
    """Causal attention rows of the last k tokens, fp64.

    q_rows [g, k_rows, d]: row r of query head q is the query of token
    n - k_rows + r and sees keys j <= n - k_rows + r (softmax over those,
    scale 1/sqrt(d)); rows of tokens before position 0 see nothing and are 0.
    Returns a [g * k_rows, n] (rows ordered head-major)."""
    q64 = np.asarray(q_rows, np.float64)
    k64 = np.asarray(k, np.float64)
    g, kr, d = q64.shape
    n = k64.shape[0]
    a = np.zeros((g * kr, n))
    for q in range(g):
        for r in range(kr):
            last = n - kr + r                       # position of the row's token
            if last < 0:
                continue
            s = (k64[:last + 1] @ q64[q, r]) / np.sqrt(d)
            s = s - s.max()
            p = np.exp(s)
            a[q * kr + r, :last + 1] = p / p.sum()
    return a


def energies(a: np.ndarray) -> np.ndarray:
    """Per-token Frobenius energy of the g x n last-row block: sum_q a[q, j]^2."""
    a = np.asarray(a, np.float64)
    return (a * a).sum(axis=0)


def cut_length(e: np.ndarray, m: int, T: float) -> int:
    """Kept length for per-token energies e (fp64 decision)."""
    e = np.asarray(e, np.float64)
    n = e.shape[0]
    if n == 0:
        return 0
    c = np.cumsum(e[rank_order(n, m)])             # c[p-1] = energy of the first p
    need = (1.0 - float(T)) * c[-1]
    p = int(np.argmax(c >= need)) + 1              # first p with C_p >= need
    return max(min(m, n), p)


def kept_positions(n: int, L: int, m: int) -> np.ndarray:
    """Ascending positions kept by a cut of length L: sinks + the last L - m."""
    s = min(m, n, L)
    return np.concatenate([np.arange(s), np.arange(n - (L - s), n)]).astype(np.int64)


# --------------------------------------------------------------------------
# fixed-point form of the same decision (exact integer sums)
# --------------------------------------------------------------------------

def energies_fixed(a32: np.ndarray) -> np.ndarray:
    """E[j] = sum_q floor(fl32(a[q,j]*a[q,j]) * 2^52) as uint64.

    a32: fp32 attention probabilities [g, n].  The fp32 square is formed as
    one IEEE multiply; widening to fp64 and scaling by 2^52 are exact."""
    a32 = np.asarray(a32, np.float32)
    sq = (a32 * a32).astype(np.float64)            # fl32 product, widened exactly
    terms = np.floor(sq * float(1 << FIX_SHIFT)).astype(np.uint64)
    return terms.sum(axis=0, dtype=np.uint64)


def cut_length_fixed(E: np.ndarray, m: int, T: float) -> int:
    """Kept length from fixed-point energies: exact integer walk down the queue."""
    E = np.asarray(E, np.uint64)
    n = E.shape[0]
    if n == 0:
        return 0
    total = int(E.sum(dtype=np.uint64))
    t64 = float(np.float32(T))
    tau = math.ceil(float(total) * (1.0 - t64))
    acc = 0
    p = n
    for pos, j in enumerate(rank_order(n, m)):
        acc += int(E[j])
        if acc >= tau:
            p = pos + 1
            break
    return max(min(m, n), p)


def threshold_cut(q_last, k, lengths, layer: int, n_full_layers: int = 2, m: int = 4,
                  T: float = 0.01, heads=None):
    """Whole call: q_last [b][Hq][d], k [b][Hkv][cap][d] (exact input values),
    lengths [b].  Returns (L [b][Hkv] int64, energies dict {(b,h): e})."""
    q_last = np.asarray(q_last)
    b, hq, d = q_last.shape
    hkv = k.shape[1]
    g = hq // hkv
    L = np.zeros((b, hkv), np.int64)
    es = {}
    todo = heads if heads is not None else [(bi, h) for bi in range(b) for h in range(hkv)]
    for bi, h in todo:
        n = int(lengths[bi])
        if layer < n_full_layers:
            L[bi, h] = n
            continue
        a = last_row_attention(q_last[bi, h * g:(h + 1) * g], k[bi, h, :n])
        e = energies(a)
        es[(bi, h)] = e
        L[bi, h] = cut_length(e, m, T)
    return L, es


def threshold_cut_rows(q_rows, k, lengths, layer: int, n_full_layers: int = 2, m: int = 4,
                       T: float = 0.01, heads=None):
    """The cut from the last k rows: q_rows [b][Hq][k_rows][d] (exact input
    values), k [b][Hkv][cap][d], lengths [b].  Energy of token j: the sum of
    a^2 over the g*k_rows causal rows of the group.  Returns (L, energies)."""
    q_rows = np.asarray(q_rows)
    b, hq, kr, d = q_rows.shape
    hkv = k.shape[1]
    g = hq // hkv
    L = np.zeros((b, hkv), np.int64)
    es = {}
    todo = heads if heads is not None else [(bi, h) for bi in range(b) for h in range(hkv)]
    for bi, h in todo:
        n = int(lengths[bi])
        if layer < n_full_layers:
            L[bi, h] = n
            continue
        e = energies(last_rows_attention(q_rows[bi, h * g:(h + 1) * g], k[bi, h, :n]))
        es[(bi, h)] = e
        L[bi, h] = cut_length(e, m, T)
    return L, es


def threshold_cut_from_attn(attn32, lengths, hkv: int, m: int = 4, T: float = 0.01):
    """Fixed-point cut from given fp32 last-row probabilities attn32 [b][Hq][cap]."""
    attn32 = np.asarray(attn32, np.float32)
    b, hq, _ = attn32.shape
    g = hq // hkv
    L = np.zeros((b, hkv), np.int64)
    for bi in range(b):
        n = int(lengths[bi])
        for h in range(hkv):
            E = energies_fixed(attn32[bi, h * g:(h + 1) * g, :n])
            L[bi, h] = cut_length_fixed(E, m, T)
    return L
