"""R-KV joint importance + redundancy selection: plain fp64 CPU oracle.

TEST INFRASTRUCTURE ONLY.  Imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py; never by the product path.  It shares no code
with the HIP library.

Source: the QbitAI R-KV article, section "R-KV三步走：冗余识别+重要性评估+动态淘汰".
That section names four parts of the method and no formulas:
  * compression happens while decoding, before the cache grows;
  * importance of a cached token comes from multi-head attention jointly;
  * redundancy comes from the cosine similarity of key vectors ("repeaters");
  * joint eviction keeps high-importance, low-redundancy tokens within a KV
    budget, with a mixing weight lambda of about 0.1 working best.
The exact formulas below are the plain reading of those four sentences:

  importance  I[j] = mean over the g*w window rows (q, r) of softmax_j(Q[q,r].K[j]/sqrt(d))
  redundancy  R[j] = mean over i != j of cos(K[i], K[j])          (0 when n == 1)
  score       Z[j] = lam*I[j] - (1-lam)*R[j]
  selection   the min(B, n) largest Z; equal Z -> lower position first;
              returned in ascending position order
  compaction  K_out[t] = K[idx[t]], V_out[t] = V[idx[t]]

Readings where the article is silent: scale 1/sqrt(d); no causal mask among the
w window rows; a zero key has cosine 0 with everything; the GQA group of KV
head h is q heads h*g .. h*g+g-1; nothing (sinks, window) is force-kept.

Everything is fp64 on the exact values of the (bf16 or fp32) inputs.
"""

from __future__ import annotations

import numpy as np


def importance(q_rows: np.ndarray, k: np.ndarray) -> np.ndarray:
    """I[j] for one KV head.

    q_rows: [m, d] all query rows of the head's GQA group over the window
            (m = g*w); k: [n, d] valid keys.  Returns [n] fp64.
    Step: attention of every row over all n keys, then the plain mean of the
    m attention rows (the joint multi-head estimate).
    """
    q64 = np.asarray(q_rows, np.float64)
    k64 = np.asarray(k, np.float64)
    n, d = k64.shape
    if n == 0:
        return np.zeros(0)
    s = (q64 @ k64.T) / np.sqrt(d)                 # [m, n] logits
    s = s - s.max(axis=1, keepdims=True)           # stable softmax
    p = np.exp(s)
    p = p / p.sum(axis=1, keepdims=True)           # each row sums to 1
    return p.mean(axis=0)


def unit_keys(k: np.ndarray) -> np.ndarray:
    """k_j / ||k_j||, with the zero vector kept as zero."""
    k64 = np.asarray(k, np.float64)
    nrm = np.sqrt((k64 * k64).sum(axis=1))
    out = np.zeros_like(k64)
    nz = nrm > 0
    out[nz] = k64[nz] / nrm[nz, None]
    return out


def redundancy(k: np.ndarray) -> np.ndarray:
    """R[j] = (1/(n-1)) * sum over i != j of cos(k_i, k_j): the definition,
    through the full n x n cosine matrix.  Memory n*n*8 bytes: for n up to a
    few thousand."""
    kh = unit_keys(k)
    n = kh.shape[0]
    if n <= 1:
        return np.zeros(n)
    c = kh @ kh.T                                  # c[i, j] = cos(k_i, k_j)
    c[np.arange(n), np.arange(n)] = 0.0            # leave out i == j
    return c.sum(axis=0) / (n - 1)


def redundancy_keysum(k: np.ndarray) -> np.ndarray:
    """The same R regrouped: sum over i != j of u_i.u_j = u_j.(sum_i u_i) - u_j.u_j,
    with u the unit keys.  O(n*d); used where n*n is too large for the
    definition above, and cross-checked against it by the tests."""
    kh = unit_keys(k)
    n = kh.shape[0]
    if n <= 1:
        return np.zeros(n)
    s = kh.sum(axis=0)
    return (kh @ s - (kh * kh).sum(axis=1)) / (n - 1)


def redundancy_rows(k: np.ndarray, rows) -> np.ndarray:
    """R[j] by the definition for selected positions j only (O(len(rows)*n*d))."""
    kh = unit_keys(k)
    n = kh.shape[0]
    rows = np.asarray(rows, dtype=np.int64)
    if n <= 1:
        return np.zeros(len(rows))
    c = kh[rows] @ kh.T                            # [len(rows), n]
    c[np.arange(len(rows)), rows] = 0.0
    return c.sum(axis=1) / (n - 1)


def combine(i_scores: np.ndarray, r_scores: np.ndarray, lam: float) -> np.ndarray:
    """Z = lam*I - (1-lam)*R: high importance and low redundancy rank first."""
    lam = float(lam)
    return lam * np.asarray(i_scores, np.float64) - (1.0 - lam) * np.asarray(r_scores, np.float64)


def top_budget(z: np.ndarray, budget: int) -> np.ndarray:
    """Positions of the min(budget, n) largest z; among equal z the lower
    position wins; result ascending (int64)."""
    z = np.asarray(z, np.float64)
    n = z.shape[0]
    if n <= budget:
        return np.arange(n, dtype=np.int64)
    order = np.lexsort((np.arange(n), -z))         # by -z, then by position
    return np.sort(order[:budget]).astype(np.int64)


def evict_slots(z: np.ndarray, budget: int, pos=None) -> np.ndarray:
    """Slot reuse without compaction: the slots NOT among the min(budget, n)
    largest z, ascending.  Equal z: the lower token position pos[slot] is
    kept (the earlier token counts as the original); equal positions: the
    lower slot.  pos defaults to the slot index (then the kept set is
    top_budget's)."""
    z = np.asarray(z, np.float64)
    n = z.shape[0]
    slots = np.arange(n)
    pos = slots if pos is None else np.asarray(pos, np.int64)
    if n <= budget:
        return np.zeros(0, dtype=np.int64)
    order = np.lexsort((slots, pos, -z))          # by -z, then position, then slot
    keep = np.zeros(n, dtype=bool)
    keep[order[:max(budget, 0)]] = True
    return slots[~keep].astype(np.int64)


def head_scores(q_rows, k, lam, form: str = "definition"):
    """(I, R, Z) of one KV head.  form: "definition" or "keysum" for R."""
    i_sc = importance(q_rows, k)
    r_sc = redundancy(k) if form == "definition" else redundancy_keysum(k)
    return i_sc, r_sc, combine(i_sc, r_sc, lam)


def head_budget(budgets, h: int, budget: int) -> int:
    """Budget of KV head h: the scalar budget, or budgets[h] clamped to
    [0, budget] (budget being the row count of the outputs)."""
    if budgets is None:
        return budget
    return min(max(int(budgets[h]), 0), budget)


def score_evict(q, k, v, lengths, lam: float, budget: int, form: str = "definition",
                heads=None, budgets=None):
    """Whole call for b sequences.

    q: [b][Hq][w][d], k, v: [b][Hkv][cap][d] (exact fp32 values of the inputs),
    lengths: [b].  Returns a dict of per-(b, h) results:
      I, R, Z:   lists indexed [b][h] of fp64 arrays of length n_b
      idx:       [b][Hkv][budget] int64, ascending, -1 past min(n_b, B_h)
      k_out, v_out: [b][Hkv][budget][d] rows of k/v at idx (zeros where idx<0)
    ``heads`` optionally restricts the work to a list of (b, h) pairs.
    ``budgets`` optionally gives one budget per KV head (the row of a
    per-head allocation table); B_h = head_budget(budgets, h, budget).
    """
    q = np.asarray(q)
    b, hq, w, d = q.shape
    hkv = k.shape[1]
    g = hq // hkv
    out_i = [[None] * hkv for _ in range(b)]
    out_r = [[None] * hkv for _ in range(b)]
    out_z = [[None] * hkv for _ in range(b)]
    idx = np.full((b, hkv, budget), -1, dtype=np.int64)
    k_out = np.zeros((b, hkv, budget, d), dtype=k.dtype)
    v_out = np.zeros((b, hkv, budget, d), dtype=v.dtype)
    todo = heads if heads is not None else [(bi, h) for bi in range(b) for h in range(hkv)]
    for bi, h in todo:
        n = int(lengths[bi])
        rows = q[bi, h * g:(h + 1) * g].reshape(g * w, d)
        i_sc, r_sc, z = head_scores(rows, k[bi, h, :n], lam, form)
        sel = top_budget(z, head_budget(budgets, h, budget))
        out_i[bi][h], out_r[bi][h], out_z[bi][h] = i_sc, r_sc, z
        idx[bi, h, :len(sel)] = sel
        k_out[bi, h, :len(sel)] = k[bi, h, sel]
        v_out[bi, h, :len(sel)] = v[bi, h, sel]
    return dict(I=out_i, R=out_r, Z=out_z, idx=idx, k_out=k_out, v_out=v_out)
