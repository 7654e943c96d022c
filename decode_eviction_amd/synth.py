"""Seeded synthetic KV caches and queries for the score-and-evict workloads.

This module only draws inputs.  It holds none of the selection method's
arithmetic (no softmax, no cosine, no ranking, no cut), so both the CPU
oracle and the HIP path can be fed from it without sharing any method code.

Shapes follow the workloads the pages describe:

* R-KV article (QbitAI), section "R-KV三步走": decoding-time compression of a
  long chain-of-thought whose output repeats itself ("repeater" content), on an
  8B model (32 layers, 8 KV heads of width 128 behind 32 query heads, a
  32K-token reasoning trace).  Repetition is modelled by near-copies of earlier
  key segments; attention sinks by high-norm keys at positions 0-3.
* ReFreeKV review ("论文综述：ReFreeKV：迈向无阈值的KV缓存压缩"), section 二,
  first step: attention concentrates on the first few tokens (sinks) and on
  recent tokens.  Modelled by a per-head direction u shared by the last query
  and by keys whose alignment with u decays with distance from the end.

Every stream is drawn from ``np.random.default_rng(SeedSequence([...]))`` keyed
by (base seed, workload id, sequence, layer, head), so any single head can be
regenerated on its own.  Values are drawn in fp32; bf16 workloads round them to
bf16 with round-to-nearest-even and keep the bf16 bit patterns (uint16), which
are exact fp32 values when widened.
"""

from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

# workload ids used in the seed keys
WL_TINY = 1
WL_LAYER8B = 2
WL_DECODE = 3
WL_BATCHED = 4
WL_REFREEKV = 5
WL_HEADLINE = 6
WL_REFREEKV_ROWS = 7

_THREADS = 8


# ----------------------------------------------------------------------------
# bf16 helpers (storage format only)
# ----------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round to nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to the fp32 values they denote (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(k) for k in key]))


# ----------------------------------------------------------------------------
# structure generators
# ----------------------------------------------------------------------------

def near_copy_runs(n: int, frac: float, run_lo: int, run_hi: int,
                   rng: np.random.Generator, first: int = 16,
                   history: Optional[int] = None) -> list[tuple[int, int, int]]:
    """Plan repeated segments: a list of (dst, src, length), dst increasing.

    Destination runs are placed at uniformly drawn free positions >= ``first``
    until at least ceil(frac*n) tokens are covered.  Each run copies an earlier
    segment that ends before the run starts; with ``history`` the source start
    is drawn from the last ``history`` tokens before the run (recent loops),
    otherwise from anywhere earlier.
    """
    target = int(math.ceil(frac * n))
    if n <= first or target <= 0:
        return []
    taken = np.zeros(n, dtype=bool)
    runs: list[tuple[int, int]] = []
    covered = 0
    attempts = 0
    while covered < target and attempts < 200 * (target + 1):
        attempts += 1
        r = int(rng.integers(run_lo, run_hi + 1))
        lo = max(first, r)
        if lo > n - r:
            continue
        t = int(rng.integers(lo, n - r + 1))
        if taken[t:t + r].any():
            continue
        taken[t:t + r] = True
        runs.append((t, r))
        covered += r
    runs.sort()
    plan = []
    for t, r in runs:
        s_lo = 0 if history is None else max(0, t - history)
        s = int(rng.integers(s_lo, t - r + 1))
        plan.append((t, s, r))
    return plan


def apply_near_copies(x: np.ndarray, plan, sigma: float, rng: np.random.Generator) -> None:
    """x[dst:dst+r] = x[src:src+r] + sigma*N(0,1), in increasing dst order (in place)."""
    d = x.shape[1]
    for t, s, r in plan:
        x[t:t + r] = x[s:s + r] + sigma * rng.standard_normal((r, d), dtype=np.float32)


# ----------------------------------------------------------------------------
# R-KV workloads
# ----------------------------------------------------------------------------

@dataclass
class RKVCase:
    """One score-and-evict call: q window, K, V for b sequences and Hkv heads."""
    name: str
    dtype: str                 # "bf16" or "f32"
    b: int
    hq: int
    hkv: int
    d: int
    w: int
    cap: int
    budget: int
    lam: float
    lengths: np.ndarray        # int32 [b]
    q: np.ndarray              # [b][hq][w][d]   uint16 bits (bf16) or float32
    k: np.ndarray              # [b][hkv][cap][d]
    v: np.ndarray              # [b][hkv][cap][d]
    meta: dict = field(default_factory=dict)

    def as_f32(self, name: str) -> np.ndarray:
        a = getattr(self, name)
        return bf16_bits_to_f32(a) if self.dtype == "bf16" else np.asarray(a, np.float32)


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(x) if dtype == "bf16" else np.ascontiguousarray(x, np.float32)


def _rkv_head(seed, wl, bi, layer, h, n, cap, d, frac, sigma, run_lo, run_hi,
              sink_scale, history, dtype):
    rng = _rng(seed, wl, bi, layer, h)
    kk = rng.standard_normal((n, d), dtype=np.float32)
    plan = near_copy_runs(n, frac, run_lo, run_hi, rng, history=history)
    apply_near_copies(kk, plan, sigma, rng)
    if sink_scale is not None:
        kk[:min(4, n)] *= np.float32(sink_scale)
    vv = rng.standard_normal((n, d), dtype=np.float32)
    kf = np.zeros((cap, d), np.float32)
    vf = np.zeros((cap, d), np.float32)
    kf[:n] = kk
    vf[:n] = vv
    if cap > n:
        # slots past the valid length hold junk a caller may leave there
        kf[n:] = np.float32(1e30)
        vf[n:] = np.float32(-1e30)
    return _store(kf, dtype), _store(vf, dtype), len(plan)


def rkv_case(name: str, *, seed: int, wl: int, b: int, hq: int, hkv: int, d: int,
             w: int, lengths, cap: int, budget: int, lam: float = 0.1,
             dtype: str = "bf16", frac=0.3, sigma: float = 0.02,
             run_lo: int = 16, run_hi: int = 128, sink_scale: Optional[float] = 8.0,
             history: Optional[int] = None, layer: int = 0) -> RKVCase:
    """Generic R-KV input: K ~ N(0,1) with near-copy runs (+ sinks), V ~ N(0,1),
    window queries ~ N(0,1).  ``frac`` may be a scalar or one value per sequence."""
    lengths = np.asarray(lengths, dtype=np.int32).reshape(b)
    fr = np.broadcast_to(np.asarray(frac, dtype=np.float64), (b,))
    store_dt = np.uint16 if dtype == "bf16" else np.float32
    k = np.empty((b, hkv, cap, d), store_dt)
    v = np.empty((b, hkv, cap, d), store_dt)
    jobs = [(bi, h) for bi in range(b) for h in range(hkv)]

    def one(job):
        bi, h = job
        kb, vb, _ = _rkv_head(seed, wl, bi, layer, h, int(lengths[bi]), cap, d,
                              float(fr[bi]), sigma, run_lo, run_hi, sink_scale,
                              history, dtype)
        k[bi, h] = kb
        v[bi, h] = vb

    with ThreadPoolExecutor(_THREADS) as ex:
        list(ex.map(one, jobs))
    qrng = _rng(seed, wl, 10_000 + layer)
    q = _store(qrng.standard_normal((b, hq, w, d), dtype=np.float32), dtype)
    return RKVCase(name, dtype, b, hq, hkv, d, w, cap, budget, lam, lengths, q, k, v,
                   meta=dict(seed=seed, wl=wl, layer=layer, frac=fr.tolist(), sigma=sigma,
                             runs=(run_lo, run_hi), sink_scale=sink_scale))


def tiny_case(seed: int = 0) -> RKVCase:
    """1 KV head + 1 query head, d=64, fp32, n=512, 20% near-copies (noise 0.01,
    runs of 4-16), w=8, B=128, lambda=0.1."""
    return rkv_case("tiny", seed=seed, wl=WL_TINY, b=1, hq=1, hkv=1, d=64, w=8,
                    lengths=[512], cap=512, budget=128, dtype="f32", frac=0.2,
                    sigma=0.01, run_lo=4, run_hi=16, sink_scale=None)


def layer8b_case(seed: int = 0, n: int = 4096, budget: int = 1024, cap: Optional[int] = None,
                 layer: int = 0, wl: int = WL_LAYER8B) -> RKVCase:
    """8B-shaped layer: 32 q / 8 KV heads, d=128, bf16, b=1, w=8, 30% repeated
    segments (noise 0.02, runs 16-128), keys 0-3 scaled x8 (high-norm sinks)."""
    return rkv_case("layer8b", seed=seed, wl=wl, b=1, hq=32, hkv=8, d=128, w=8,
                    lengths=[n], cap=cap or n, budget=budget, frac=0.3, sigma=0.02,
                    run_lo=16, run_hi=128, sink_scale=8.0, layer=layer)


def headline_case(layer: int, seed: int = 0) -> RKVCase:
    """The n=32768, B=2048 layer of the 8B shape; one distinct cache per layer."""
    return layer8b_case(seed=seed, n=32768, budget=2048, layer=layer, wl=WL_HEADLINE)


def batched_case(seed: int = 0, b: int = 64, n: int = 8192, layer: int = 0) -> RKVCase:
    """b independent sequences of n tokens, per-sequence duplicate fraction
    U[0.1, 0.5], noise 0.02, no sinks; 32 q / 8 KV heads, d=128, B=1024."""
    fr = _rng(seed, WL_BATCHED, 77_777, layer).uniform(0.1, 0.5, size=b)
    return rkv_case("batched", seed=seed, wl=WL_BATCHED, b=b, hq=32, hkv=8, d=128,
                    w=8, lengths=[n] * b, cap=n, budget=1024, frac=fr, sigma=0.02,
                    run_lo=16, run_hi=128, sink_scale=None, layer=layer)


# ----------------------------------------------------------------------------
# decode-loop stream (R-KV decoding-time compression)
# ----------------------------------------------------------------------------

@dataclass
class DecodeStream:
    """Per-layer token stream for the decode loop: keys and values of every
    decoded token (uint16 bf16 bits, [hkv][total][d]).  The query rows of token
    t (one per q head) are drawn on demand from their own seed, so a window of
    the last w tokens' queries can be formed at any step."""
    layer: int
    seed: int
    hq: int
    hkv: int
    d: int
    total: int
    k: np.ndarray
    v: np.ndarray

    def queries(self, t: int) -> np.ndarray:
        """bf16 bits [hq][d]: the query rows token t produced."""
        rng = _rng(self.seed, WL_DECODE, 20_000 + self.layer, t)
        return f32_to_bf16_bits(rng.standard_normal((self.hq, self.d), dtype=np.float32))

    def window(self, t_end: int, w: int) -> np.ndarray:
        """bf16 bits [1][hq][w][d]: queries of tokens t_end-w .. t_end-1."""
        rows = np.stack([self.queries(t) for t in range(t_end - w, t_end)], axis=1)
        return rows[None]


def decode_stream(layer: int, seed: int = 0, total: int = 32768, hq: int = 32,
                  hkv: int = 8, d: int = 128, frac: float = 0.4, sigma: float = 0.02,
                  run_lo: int = 32, run_hi: int = 256, history: int = 1024) -> DecodeStream:
    """Key stream with 40% near-duplicate reasoning-loop segments (lengths 32-256,
    copied from the last ``history`` tokens, noise 0.02) and x8 sinks."""
    k = np.empty((hkv, total, d), np.uint16)
    v = np.empty((hkv, total, d), np.uint16)

    def one(h):
        kb, vb, _ = _rkv_head(seed, WL_DECODE, 0, layer, h, total, total, d, frac, sigma,
                              run_lo, run_hi, 8.0, history, "bf16")
        k[h] = kb
        v[h] = vb

    with ThreadPoolExecutor(_THREADS) as ex:
        list(ex.map(one, range(hkv)))
    return DecodeStream(layer, seed, hq, hkv, d, total, k, v)


# ----------------------------------------------------------------------------
# ReFreeKV workload
# ----------------------------------------------------------------------------

@dataclass
class CutCase:
    """One threshold-cut call: last-row queries and K for b ragged sequences."""
    name: str
    dtype: str
    b: int
    hq: int
    hkv: int
    d: int
    cap: int
    layer: int
    lengths: np.ndarray        # int32 [b]
    q: np.ndarray              # [b][hq][d]
    k: np.ndarray              # [b][hkv][cap][d]
    meta: dict = field(default_factory=dict)

    def as_f32(self, name: str) -> np.ndarray:
        a = getattr(self, name)
        return bf16_bits_to_f32(a) if self.dtype == "bf16" else np.asarray(a, np.float32)


def refreekv_lengths(seed: int = 0, b: int = 16, lo: int = 1024, hi: int = 16384) -> np.ndarray:
    return _rng(seed, WL_REFREEKV, 55_555).integers(lo, hi + 1, size=b).astype(np.int32)


def cut_rows_q(case: "CutCase", k_rows: int) -> np.ndarray:
    """Query rows of the last k_rows tokens for a cut case: [b][hq][k_rows][d]
    in the case's storage type.  The last row is the case's own last-row
    query; earlier rows are drawn like it (N(0,1)^d + sqrt(d)*u with the
    head's direction u) from their own stream (zero for a zero-query case)."""
    b, hq, hkv, d = case.b, case.hq, case.hkv, case.d
    g = hq // hkv
    seed = case.meta["seed"]
    zero = bool(case.meta.get("zero_query", False))
    last = case.as_f32("q")
    out = np.zeros((b, hq, k_rows, d), np.float32)
    for bi in range(b):
        for h in range(hkv):
            u = _rng(seed, WL_REFREEKV, bi, case.layer, h).standard_normal(d)
            u /= np.linalg.norm(u)
            rows = _rng(seed, WL_REFREEKV_ROWS, bi, case.layer, h).standard_normal(
                (g, k_rows - 1, d), dtype=np.float32)
            rows += np.float32(math.sqrt(d)) * u.astype(np.float32)
            out[bi, h * g:(h + 1) * g, :k_rows - 1] = 0.0 if zero else rows
            out[bi, h * g:(h + 1) * g, k_rows - 1] = last[bi, h * g:(h + 1) * g]
    return _store(out, case.dtype)


def cut_case(layer: int, seed: int = 0, b: int = 16, hq: int = 28, hkv: int = 4,
             d: int = 128, lengths=None, cap: Optional[int] = None,
             zero_query: bool = False, dtype: str = "bf16") -> CutCase:
    """Qwen2.5-7B-shaped layer (28 q / 4 KV heads, d=128), ragged lengths.

    Per (sequence, head): a random unit direction u and a decay length
    tau ~ LogUniform[32, 4096]; key j = N(0,1)^d + 4*exp(-(n-1-j)/tau)*u, keys
    0-3 = N(0,1)^d + 8*u, and each of the head's last-row queries is
    N(0,1)^d + sqrt(d)*u.  With ``zero_query`` the queries are all zero.
    """
    if lengths is None:
        lengths = refreekv_lengths(seed, b)
    lengths = np.asarray(lengths, np.int32).reshape(b)
    cap = int(cap or int(lengths.max()))
    g = hq // hkv
    store_dt = np.uint16 if dtype == "bf16" else np.float32
    k = np.empty((b, hkv, cap, d), store_dt)
    q = np.empty((b, hq, d), np.float32)
    taus = np.zeros((b, hkv))

    def one(job):
        bi, h = job
        n = int(lengths[bi])
        rng = _rng(seed, WL_REFREEKV, bi, layer, h)
        u = rng.standard_normal(d)
        u /= np.linalg.norm(u)
        tau = float(np.exp(rng.uniform(np.log(32.0), np.log(4096.0))))
        taus[bi, h] = tau
        kk = rng.standard_normal((cap, d), dtype=np.float32)
        u32 = u.astype(np.float32)
        pull = 4.0 * np.exp(-(n - 1 - np.arange(n)) / tau)     # recency alignment
        pull[:min(4, n)] = 8.0                                   # sinks
        kk[:n] += pull.astype(np.float32)[:, None] * u32
        if cap > n:
            kk[n:] = np.float32(1e30)
        k[bi, h] = _store(kk, dtype)
        qq = rng.standard_normal((g, d), dtype=np.float32) + np.float32(math.sqrt(d)) * u.astype(np.float32)
        q[bi, h * g:(h + 1) * g] = 0.0 if zero_query else qq

    with ThreadPoolExecutor(_THREADS) as ex:
        list(ex.map(one, [(bi, h) for bi in range(b) for h in range(hkv)]))
    return CutCase("refreekv", dtype, b, hq, hkv, d, cap, layer, lengths, _store(q, dtype), k,
                   meta=dict(seed=seed, taus=taus, zero_query=zero_query))
