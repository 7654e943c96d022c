"""Benchmark: KV tokens scored+evicted per second per layer on one MI355X.

Workload: one R-KV score-and-evict call per step at the 8B shape (32 query /
8 KV heads, d = 128, bf16, batch 1, n = 32768 cached tokens, window w = 8,
budget B = 2048, lambda = 0.1).  Steps rotate over --layers distinct seeded
synthetic layer caches (32 x 128 MiB of K+V, beyond the 256 MB last-level
cache) that are resident in HBM before timing starts.

Per step the library launches stats, reduce, pool, gram, gram_fin, thresh,
compact for the Gram form, and for the key-sum form one score kernel (the
statistics, their merge and the pooling in one launch) then thresh, compact
(the compaction kernel also gathers the kept K/V rows).
The timed region (`value`, `ms_per_step`) runs kvsel_score_evict; right
after it the same steps run through kvsel_score_evict_traced, whose kernels
record start/stop HIP events on the benchmark's stream, giving each kernel's
average duration (the roofline figure uses the dominant kernel's).  Both redundancy forms are
measured; --mode picks which one is the headline `value`.

Variants (each with its own value, per-kernel times and roofline):
  decode_<mode>   the decode loop: 32 layers x 240 calls compressing a
                  2176-slot cache to 2048 rows (per-call latency);
  decode_slots_<mode>  the same loop with slot reuse: evicted slots listed and
                  refilled by the next 128 tokens, no compaction;
  batched_<mode>  64 sequences x 8192 tokens, B = 1024 (2 GiB of K and V);
  refreekv        the ReFreeKV threshold cut at the Qwen2.5-7B shape
                  (28 q / 4 KV heads), 16 ragged sequences of 1K-16K tokens;
  heads_<mode>    the headline layer with one budget per KV head (an uneven
                  allocation with the same total as B = 2048 per head).

The CPU baseline times the fp64 oracle (definition form, n x n cosine
matrix) on a bounded sample: whole KV heads of one layer until --cpu-seconds
have passed, scaled to a full layer.

    python bench.py [--gpus 1] [--steps 64] [--warmup 8] [--mode gram|keysum]
                    [--no-variants | --variant decode|batched|refreekv|refreekv_rows|heads ...]
"""

from __future__ import annotations

import argparse
import ctypes
import glob
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KV tokens scored+evicted/s per layer (8B shape, n=32K); % HBM/MFMA peak"
HQ, HKV, D, W, N, BUDGET, LAM = 32, 8, 128, 8, 32768, 2048, 0.1
PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0

KERNELS = {
    "gram": ["stats", "reduce", "pool", "gram", "gram_fin", "thresh", "compact"],
    "keysum": ["stats", "reduce", "pool", "thresh", "compact"],
}


FUSED_MAX_CHUNKS = 16     # kFusedMaxChunks: chunks of 256 tokens per head
FUSED_CAPACITY = 256      # work-groups of the fused step resident at once (one per CU)


def fused_step(mode: str, cap: int, b: int = 1, hkv: int = HKV, m: int = HQ // HKV * W) -> bool:
    """The library runs a key-sum call on a short cache (bf16, d = 128, at
    most 32 window rows per KV head) as one fused launch when its grid of
    ceil(cap / 256) * Hkv * b work-groups fits on the device at once."""
    nch = -(-cap // 256)
    return (mode == "keysum" and m <= 32 and nch <= FUSED_MAX_CHUNKS
            and nch * hkv * b <= FUSED_CAPACITY)


def fused_gram_step(mode: str, cap: int, b: int = 1, hkv: int = HKV, m: int = HQ // HKV * W) -> bool:
    """Short Gram-form caches (bf16, d = 128, at most 32 window rows per KV
    head, the pair-block Gram units), slot reuse: after k_stats and the
    pooling with the Gram units, one launch forms Z from the Gram slots,
    selects and lists the evicted slots, when its grid fits at once."""
    nch = -(-cap // 256)
    return (mode == "gram" and m <= 32 and cap <= GRAM_PAIR_CAP and nch <= FUSED_MAX_CHUNKS
            and nch * hkv * b <= FUSED_CAPACITY)


SCORES_PAIRS_CAPACITY = 768   # work-groups of k_scores_pairs resident at once (three per CU)


def scores_pairs_step(mode: str, cap: int, b: int = 1, hkv: int = HKV, m: int = HQ // HKV * W) -> bool:
    """Short Gram-form caches (bf16, d = 128, at most 32 window rows per KV
    head, the pair-block Gram units): the one-launch score units and the
    pair-block Gram units in one launch, when the score units (their count
    rounded up to a multiple of 8) fit on the device at once; otherwise
    k_stats, then the pooling beside the pair units."""
    nch = -(-cap // 256)
    return (mode == "gram" and m <= 32 and cap <= GRAM_PAIR_CAP and nch <= FUSED_MAX_CHUNKS
            and -(-nch * hkv * b // 8) * 8 <= SCORES_PAIRS_CAPACITY)


SCORES_FUSED_CAPACITY = 1024  # work-groups of the one-launch score pass resident at once (four per CU)


def scores_fused(mode: str, cap: int, b: int = 1, hkv: int = HKV, m: int = HQ // HKV * W) -> bool:
    """The library scores a call on a longer cache (more than 16 chunks of
    256 tokens per head; bf16, d = 128, at most 32 window rows per KV head)
    in one launch when its grid of ceil(cap / 256) * Hkv * b work-groups fits
    on the device at once: the key-sum scores, or the importance and key
    weights of the Gram form."""
    nch = -(-cap // 256)
    return m <= 32 and nch > FUSED_MAX_CHUNKS and nch * hkv * b <= SCORES_FUSED_CAPACITY


SEL_CHUNK = 512               # kSelChunk: positions per selection work-group
SELECT_COMPACT_CAPACITY = 1280  # work-groups of the one-launch selection resident at once (five per CU)
THRESH_HEADS_MANY = 64       # kThreshHeadsMany: from this many heads, one threshold work-group per head


def select_one_launch(cap: int, b: int = 1, hkv: int = HKV, budget: int = BUDGET) -> bool:
    """The library selects and compacts in one launch (k_select_compact) when
    the cache fits the split select (cap <= 32768), the heads are few and the
    grid of ceil(cap / 512) * gsplit * Hkv * b work-groups fits at once
    (gsplit work-groups gather a chunk's kept rows: ceil(kept / 64), at most
    8, with kept = ceil(512 B / cap))."""
    nsc = -(-cap // SEL_CHUNK)
    kept_chunk = -(-SEL_CHUNK * budget // cap)
    gsplit = min(8, max(1, -(-kept_chunk // 64)))
    return (cap <= 32768 and b * hkv < THRESH_HEADS_MANY and nsc <= 64
            and nsc * gsplit * hkv * b <= SELECT_COMPACT_CAPACITY)


def rkv_kernels(mode: str, cap: int, b: int = 1, hkv: int = HKV, budget: int = BUDGET) -> list:
    """Kernels one R-KV call launches, in order: the fused step alone when it
    applies; the one-launch score pass in place of stats, reduce and pool when
    that applies; otherwise with at most 16 chunks of 256 keys per head k_pool
    merges the chunk partials itself and k_reduce is not launched; the
    one-launch selection in place of thresh and compact when it applies."""
    if fused_step(mode, cap, b, hkv):
        return ["fused"]
    ks = unfused_kernels(mode, cap)
    if scores_pairs_step(mode, cap, b, hkv):
        ks = ["scores_pairs"] + [k for k in ks if k not in ("stats", "pool_pairs")]
    if scores_fused(mode, cap, b, hkv):
        ks = ["scores"] + [k for k in ks if k not in ("stats", "reduce", "pool")]
    if select_one_launch(cap, b, hkv, budget):
        ks = [k for k in ks if k not in ("thresh", "compact")] + ["select_compact"]
    return ks


def slot_kernels(mode: str, cap: int, b: int = 1, hkv: int = HKV) -> list:
    """Kernels one slot-reuse call (kvsel_score_evict_slots) launches: the
    fused step's slot-reuse form alone where the fused step applies (scores,
    threshold and the evicted list in one launch); otherwise the scores as a
    compacting call computes them (the one-launch score pass where it
    applies), the threshold, the evicted list."""
    if fused_step(mode, cap, b, hkv):
        return ["fused_slots"]
    if fused_gram_step(mode, cap, b, hkv):
        return (["scores_pairs"] if scores_pairs_step(mode, cap, b, hkv) else ["stats", "pool_pairs"]) \
            + ["fused_fin_slots"]
    ks = [k for k in unfused_kernels(mode, cap) if k not in ("thresh", "compact")]
    if scores_pairs_step(mode, cap, b, hkv):
        ks = ["scores_pairs"] + [k for k in ks if k not in ("stats", "pool_pairs")]
    if scores_fused(mode, cap, b, hkv):
        ks = ["scores"] + [k for k in ks if k not in ("stats", "reduce", "pool")]
    return ks + ["thresh", "evict"]


GRAM_PAIR_CAP = 4096         # kGramPairCap: pair-block Gram units up to this cache size


def unfused_kernels(mode: str, cap: int) -> list:
    """The multi-kernel launch sequence (also the score kernels of the slot
    reuse entry points outside the fused step).  Short Gram-form caches (bf16,
    d = 128, at most 32 window rows) run the pooling and the pair-block Gram
    units in one launch (pool_pairs) after k_stats, which then writes the key
    weights."""
    ks = list(KERNELS[mode])
    if -(-cap // 256) <= 16:
        ks.remove("reduce")
    if mode == "gram" and cap <= GRAM_PAIR_CAP:
        ks = [k for k in ks if k != "gram"]
        ks[ks.index("pool")] = "pool_pairs"
    return ks


def gram_flops(b: int, hkv: int, n: int, d: int = D) -> tuple:
    """(algorithmic, executed) matrix-core flops of the symmetric Gram form.

    Algorithmic: every distinct key pair once, 2 d flops each, the diagonal
    included: n (n + 1) d per head.  Executed: whole block pairs of the
    kernel that runs (pairs of 128-key blocks up to cap 4096, 512-key blocks
    from 8192 (bf16, d = 128), 256-key blocks between), diagonal blocks in
    full; the SQ_VALU_MFMA_BUSY_CYCLES counter agrees with this count."""
    alg = float(b) * hkv * n * (n + 1) * d
    if n <= 4096:
        nbh = -(-n // 128)
        pairs, bs = nbh * (nbh + 1) // 2, 128
    else:
        bs = 512 if n >= 8192 else 256
        nb = -(-n // bs)
        pairs = sum(1 + (nb - 1) // 2 + (1 if nb % 2 == 0 and i < nb // 2 else 0) for i in range(nb))
    return alg, 2.0 * b * hkv * pairs * bs * bs * d


def rkv_cost(mode: str, b: int = 1, n: int = N, budget: int = BUDGET, hkv: int = HKV,
             d: int = D) -> dict:
    """Bytes (and flops) each R-KV kernel must move per call.

    K bytes = b*Hkv*n*d*2; scores are fp32 per token per head; the gather moves
    min(B, n) kept rows of K and V in and out."""
    tok = b * hkv * n
    kb = tok * d * 2
    gath = 2 * 2 * b * hkv * min(budget, n) * d * 2
    cost = {
        "stats": {"bytes": kb},
        "reduce": {"bytes": 0},
        # Gram form: I and the key weights 1/||k||; key-sum form: I and Z
        "pool": {"bytes": kb + 8 * tok},
        "thresh": {"bytes": 4 * tok},
        "compact": {"bytes": 4 * tok + 4 * b * hkv * budget + gath},
    }
    # the one-launch selection: the scores once, the indices and the gather
    cost["select_compact"] = {"bytes": 4 * tok + 4 * b * hkv * budget + gath}
    # slot reuse: scores and position map read, evicted list written
    cost["evict"] = {"bytes": 8 * tok + 4 * b * hkv * max(n - budget, 0)}
    # the fused short-cache step: K once, Z and the indices written, the kept
    # rows of V read and of K and V written (K rows come from registers)
    cost["fused"] = {"bytes": kb + 4 * tok + 4 * b * hkv * budget + 3 * b * hkv * min(budget, n) * d * 2}
    # its slot-reuse form: K once, Z and the evicted list written
    cost["fused_slots"] = {"bytes": kb + 4 * tok + 4 * b * hkv * max(n - budget, 0)}
    # the one-launch score pass: K once, I and Z written
    cost["scores"] = {"bytes": kb + 8 * tok}
    if mode == "gram":
        # symmetric Gram: achieved = algorithmic flops (each key pair once)
        ns = -(-n // 256) // 2
        alg, exe = gram_flops(b, hkv, n, d)
        cost["gram"] = {"bytes": kb + 4 * tok * 2 + 4 * tok * ns // 2, "flops": alg,
                        "flops_executed": exe}
        # short caches: the pooling (K again, I written) and the pair-block
        # Gram units in one launch; counted by its matrix-core work
        cost["pool_pairs"] = {"bytes": 2 * kb + 4 * tok + 4 * tok * -(-n // 128), "flops": alg,
                              "flops_executed": exe}
        # the score units (K once, I and the key weights written) beside the
        # pair units; counted by its matrix-core work
        cost["scores_pairs"] = {"bytes": kb + 8 * tok + 4 * tok * -(-n // 128), "flops": alg,
                                "flops_executed": exe}
        # the one-launch finish of short caches (slot reuse): the Gram slots,
        # weights and importance read, Z and the evicted list written
        cost["fused_fin_slots"] = {"bytes": 4 * tok * -(-n // 128) + 12 * tok
                                   + 4 * b * hkv * max(n - budget, 0)}
        cost["gram_fin"] = {"bytes": 4 * tok * 5 + 4 * tok * ns // 2}
    return cost


def rkv_step_bytes(b: int = 1, n: int = N, budget: int = BUDGET, hkv: int = HKV, d: int = D) -> int:
    """Algorithmic floor of one R-KV call: K once, scores, the gather."""
    tok = b * hkv * n
    return tok * d * 2 + 3 * 4 * tok + 2 * 2 * b * hkv * min(budget, n) * d * 2


def cut_cost(lengths, hq: int, hkv: int, d: int = D) -> dict:
    """Bytes each ReFreeKV kernel moves per scored layer: stats reads K and
    writes the g last-row logits of every token (fp32), cut_energy reads them
    back and writes one 64-bit energy per token, cut_scan reads chunk totals."""
    tok = int(np.sum(lengths)) * hkv
    g = hq // hkv
    return {
        "stats": {"bytes": tok * d * 2 + tok * g * 4},
        "reduce": {"bytes": 0},
        "cut_energy": {"bytes": tok * g * 4 + tok * 8},
        "cut_scan": {"bytes": 0},
    }


class Hip:
    """hipEvent helpers through the HIP runtime torch already loaded."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def events(self, n):
        arr = (ctypes.c_void_p * n)()
        for i in range(n):
            h = ctypes.c_void_p()
            if self.lib.hipEventCreate(ctypes.byref(h)) != 0:
                raise RuntimeError("hipEventCreate failed")
            arr[i] = h
        return arr

    def recorded(self, arr, k) -> bool:
        """Whether kernel k of a traced call recorded its event pair."""
        ms = ctypes.c_float()
        ok = self.lib.hipEventElapsedTime(ctypes.byref(ms), arr[2 * k], arr[2 * k + 1]) == 0
        self.lib.hipGetLastError()  # a failed query of an unrecorded pair is not left behind
        return ok

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        if self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def destroy(self, arr):
        for h in arr:
            self.lib.hipEventDestroy(h)


def make_layers(n_layers: int):
    import torch

    from decode_eviction_amd import synth
    layers = []
    for layer in range(n_layers):
        c = synth.headline_case(layer=layer)
        to = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to("cuda")
        layers.append((to(c.q), to(c.k), to(c.v)))
        if layer == 0:
            first = c
        print(f"# generated layer {layer + 1}/{n_layers}", file=sys.stderr, flush=True)
    return layers, first


def time_calls(call, names, cost, steps, warmup, hip, traced_steps=None):
    """Warm up, time `steps` plain calls (`call(i, None)`), then time the same
    calls with per-kernel HIP events (`call(i, events)`) on the same stream."""
    import torch
    nk = len(names)
    for i in range(warmup):
        call(i, None)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(steps):
        call(i, None)
    t1.record()
    torch.cuda.synchronize()
    ms_plain = t0.elapsed_time(t1) / steps

    ts = traced_steps or steps
    # one event pair more than the predicted launches: it must stay unrecorded
    evs = [hip.events(2 * nk + 2) for _ in range(ts)]
    torch.cuda.synchronize()
    t0.record()
    for i in range(ts):
        call(i, evs[i])
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / ts
    if not hip.recorded(evs[0], nk - 1) or hip.recorded(evs[0], nk):
        raise RuntimeError(f"the call did not launch the {nk} kernels {names}")
    per = {nm: [] for nm in names}
    for e in evs:
        for j, nm in enumerate(names):
            per[nm].append(hip.elapsed_ms(e[2 * j], e[2 * j + 1]))
        hip.destroy(e)
    kern = {}
    for nm in names:
        us = 1000.0 * float(np.mean(per[nm]))
        entry = {"avg_us": round(us, 3), "min_us": round(1000.0 * float(np.min(per[nm])), 3)}
        c = cost[nm]
        if c.get("bytes"):
            entry["alg_GBps"] = round(c["bytes"] / (us * 1e-6) / 1e9, 1)
            entry["hbm_frac"] = round(entry["alg_GBps"] / PEAK_HBM_GBS, 4)
        if c.get("flops"):
            entry["alg_TFLOPs"] = round(c["flops"] / (us * 1e-6) / 1e12, 1)
            entry["mfma_frac"] = round(entry["alg_TFLOPs"] / PEAK_BF16_TFLOPS, 4)
        kern[nm] = entry
    return dict(ms=ms, ms_plain=ms_plain, kernels=kern)


def rkv_caller(mode, layers, b, n, budget, out_bufs=None, budgets=None):
    """call(i, events) running kvsel_score_evict[_traced] on layer i % len(layers).
    layers: list of (q, k, v) device tensors.  With out_bufs the outputs go to
    out_bufs[i % len], else to one shared output.  With budgets (int32 device
    tensor [Hkv]) the per-head entry points run and budget is the row stride."""
    import torch

    from decode_eviction_amd import kvsel as K
    lib = K.lib()
    mcode = K.MODES[mode]
    q0, k0, _ = layers[0]
    nk = len(rkv_kernels(mode, k0.shape[2], b, k0.shape[1]))
    hq, w = q0.shape[1], q0.shape[2]
    hkv, cap = k0.shape[1], k0.shape[2]
    lens = torch.full((b,), n, dtype=torch.int32, device="cuda")
    if out_bufs is None:
        ko = torch.empty((b, hkv, budget, D), dtype=torch.bfloat16, device="cuda")
        out_bufs = [(ko, torch.empty_like(ko))]
    idx = torch.empty((b, hkv, budget), dtype=torch.int32, device="cuda")
    ws_bytes = K.kvsel_score_evict_workspace(b, hq, hkv, D, w, cap, budget)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    P = ctypes.c_void_p

    def call(i, events=None):
        q, k, v = layers[i % len(layers)]
        ko, vo = out_bufs[i % len(out_bufs)]
        head = (K.KVSEL_BF16, mcode, P(q.data_ptr()), P(k.data_ptr()), P(v.data_ptr()),
                P(lens.data_ptr()))
        tail = (b, hq, hkv, D, w, cap, LAM, budget, P(ko.data_ptr()), P(vo.data_ptr()),
                ko.shape[2], P(idx.data_ptr()), None, P(ws.data_ptr()), ws_bytes, sp)
        if budgets is not None:
            args = head + (P(budgets.data_ptr()),) + tail
            st = (lib.kvsel_score_evict_heads(*args) if events is None else
                  lib.kvsel_score_evict_heads_traced(*args, events, len(events)))
        elif events is None:
            st = lib.kvsel_score_evict(*head, *tail)
        else:
            st = lib.kvsel_score_evict_traced(*head, *tail, events, len(events))
        if st != 0:
            raise RuntimeError(f"kvsel_score_evict: {K.status_string(st)}")

    return call, (idx, ws)


def run_mode(mode, layers, steps, warmup, hip):
    call, keep = rkv_caller(mode, layers, 1, N, BUDGET)
    return time_calls(call, rkv_kernels(mode, N), rkv_cost(mode), steps, warmup, hip)


# an uneven per-head allocation with the same total as B=2048 per head
HEAD_BUDGETS = [512, 1024, 1536, 2048, 2048, 2560, 3072, 3584]


def run_heads(mode, layers, steps, warmup, hip):
    """The headline layer with one budget per KV head (HEAD_BUDGETS, output
    stride 3584): same scores, per-head thresholds and compaction."""
    import torch
    budgets = torch.tensor(HEAD_BUDGETS, dtype=torch.int32, device="cuda")
    call, keep = rkv_caller(mode, layers, 1, N, max(HEAD_BUDGETS), budgets=budgets)
    return time_calls(call, rkv_kernels(mode, N), rkv_cost(mode), steps, warmup, hip)


def bf16_dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to("cuda")


def run_decode(mode, n_layers, hip, calls_per_layer=240):
    """Decode-loop workload: per layer a 2176-slot cache compressed to 2048 rows
    every 128 decoded tokens, 240 calls per layer over n_layers layers.  Each
    layer keeps two caches that swap roles every call (the output of one call
    is the next call's input); their last 128 slots hold the next 128 tokens
    of the layer's synthetic stream."""
    import torch

    from decode_eviction_amd import synth
    cap, budget, w = 2176, 2048, W
    layers, outs = [], []
    for layer in range(n_layers):
        ds = synth.decode_stream(layer, total=cap + (cap - budget))
        q = bf16_dev(ds.window(cap, w))
        k = bf16_dev(ds.k[None, :, :cap])
        v = bf16_dev(ds.v[None, :, :cap])
        k2, v2 = k.clone(), v.clone()
        k2[:, :, budget:] = k[:, :, budget:] = bf16_dev(ds.k[None, :, cap:])
        v2[:, :, budget:] = v[:, :, budget:] = bf16_dev(ds.v[None, :, cap:])
        layers.append([(q, k, v), (q, k2, v2)])
    # call i: layer l = i % n_layers, its j-th call with j = i // n_layers;
    # input cache j % 2, output the other one
    seq, obuf = [], []
    for j in range(2):
        for l in range(n_layers):
            seq.append(layers[l][j])
            _, ko, vo = layers[l][1 - j]
            obuf.append((ko, vo))
    call, keep = rkv_caller(mode, seq, 1, cap, budget, out_bufs=obuf)
    total = n_layers * calls_per_layer
    cost = rkv_cost(mode, 1, cap, budget)
    r = time_calls(call, rkv_kernels(mode, cap), cost, total, 2 * n_layers, hip, traced_steps=min(512, total))
    r["calls"] = total
    r["tokens"] = total * cap
    return r


def run_decode_slots(mode, n_layers, hip, calls_per_layer=240):
    """The decode loop with slot reuse: per layer a 2176-slot cache that is
    never compacted.  Call j of a layer scores it, lists the 128 evicted slots
    per head (kvsel_score_evict_slots) and writes the layer's stream tokens
    2176 + 128j .. 2176 + 128j + 127 into them (kvsel_slots_write); both are in
    the timed call.  The per-kernel trace covers the score and select kernels
    (the write is one small kernel after them)."""
    import torch

    from decode_eviction_amd import kvsel as K
    from decode_eviction_amd import synth
    cap, budget, w, nb = 2176, 2048, W, 2176 - 2048
    lib = K.lib()
    mcode = K.MODES[mode]
    names = slot_kernels(mode, cap)
    P = ctypes.c_void_p
    layers = []
    for layer in range(n_layers):
        ds = synth.decode_stream(layer, total=cap + nb * calls_per_layer)
        q = bf16_dev(ds.window(cap, w))
        k = bf16_dev(ds.k[None, :, :cap])
        v = bf16_dev(ds.v[None, :, :cap])
        # new tokens of call j: [calls][1][Hkv][nb][d], each call's block contiguous
        rest = lambda a: np.ascontiguousarray(
            a[:, cap:].reshape(HKV, calls_per_layer, nb, D).transpose(1, 0, 2, 3)[:, None])
        kn, vn = bf16_dev(rest(ds.k)), bf16_dev(rest(ds.v))
        pos = torch.arange(cap, dtype=torch.int32, device="cuda").repeat(HKV, 1)[None].contiguous()
        ev = torch.empty((1, HKV, cap), dtype=torch.int32, device="cuda")
        ne = torch.empty((1, HKV), dtype=torch.int32, device="cuda")
        layers.append((q, k, v, kn, vn, pos, ev, ne))
        del ds
    lens = torch.full((1,), cap, dtype=torch.int32, device="cuda")
    pos_new = torch.arange(cap, cap + nb * calls_per_layer, nb, dtype=torch.int32, device="cuda")
    ws_bytes = K.kvsel_score_evict_workspace(1, HQ, HKV, D, w, cap, budget)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    sp = P(torch.cuda.current_stream().cuda_stream)
    step_new = HKV * nb * D * 2

    done = [0] * n_layers  # calls so far per layer: the stream position keeps advancing

    def call(i, events=None):
        q, k, v, kn, vn, pos, ev, ne = layers[i % n_layers]
        j = done[i % n_layers] % calls_per_layer
        done[i % n_layers] += 1
        args = (K.KVSEL_BF16, mcode, P(q.data_ptr()), P(k.data_ptr()), P(lens.data_ptr()),
                P(pos.data_ptr()), None, 1, HQ, HKV, D, w, cap, LAM, budget, P(ev.data_ptr()),
                cap, P(ne.data_ptr()), None, P(ws.data_ptr()), ws_bytes, sp)
        st = (lib.kvsel_score_evict_slots(*args) if events is None else
              lib.kvsel_score_evict_slots_traced(*args, events, len(events)))
        if st == 0:
            st = lib.kvsel_slots_write(K.KVSEL_BF16, P(k.data_ptr()), P(v.data_ptr()),
                                       P(pos.data_ptr()), P(kn.data_ptr() + j * step_new),
                                       P(vn.data_ptr() + j * step_new),
                                       P(pos_new.data_ptr() + 4 * j), P(ev.data_ptr()), cap,
                                       P(ne.data_ptr()), 1, HKV, D, cap, nb, sp)
        if st != 0:
            raise RuntimeError(f"slot reuse call: {K.status_string(st)}")

    total = n_layers * calls_per_layer
    cost = rkv_cost(mode, 1, cap, budget)
    r = time_calls(call, names, cost, total, 2 * n_layers, hip, traced_steps=min(512, total))
    r["calls"] = total
    r["tokens"] = total * cap
    return r


def run_batched(mode, hip, steps):
    """Batched prefill workload: 64 sequences of 8192 tokens, B = 1024 (1 GiB
    of K and 1 GiB of V, far beyond the 256 MB last-level cache)."""
    from decode_eviction_amd import synth
    c = synth.batched_case(seed=0)
    layer = (bf16_dev(c.q), bf16_dev(c.k), bf16_dev(c.v))
    del c
    b, n, budget = 64, 8192, 1024
    call, keep = rkv_caller(mode, [layer], b, n, budget)
    r = time_calls(call, rkv_kernels(mode, n, b, budget=budget), rkv_cost(mode, b, n, budget), steps, 2, hip)
    r["tokens"] = b * n
    r["step_bytes"] = rkv_step_bytes(b, n, budget)
    return r


CUT_KERNELS = ["stats", "reduce", "cut_energy", "cut_scan"]


def run_refreekv(hip, n_layers, steps):
    """ReFreeKV threshold cut at the Qwen2.5-7B shape (28 q / 4 KV heads,
    d=128, bf16), 16 sequences of 1024-16384 tokens, one scored layer per
    call (layers 0-1 keep everything and cost one tiny kernel); rotates over
    n_layers distinct layers of K."""
    import torch

    from decode_eviction_amd import kvsel as K
    from decode_eviction_amd import synth
    hq, hkv, b = 28, 4, 16
    lengths = synth.refreekv_lengths(0, b)
    cap = int(lengths.max())
    layers = []
    for layer in range(2, 2 + n_layers):
        c = synth.cut_case(layer=layer, seed=0, lengths=lengths, cap=cap)
        layers.append((bf16_dev(c.q), bf16_dev(c.k)))
    lens = torch.from_numpy(lengths).to("cuda")
    kept = torch.empty((b, hkv), dtype=torch.int32, device="cuda")
    ws_bytes = K.kvsel_threshold_cut_workspace(b, hq, hkv, D, cap)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    lib = K.lib()
    sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    P = ctypes.c_void_p

    def call(i, events=None):
        q, k = layers[i % len(layers)]
        args = (K.KVSEL_BF16, P(q.data_ptr()), P(k.data_ptr()), P(lens.data_ptr()), b, hq, hkv,
                D, cap, 2 + i % len(layers), 2, 4, 0.01, P(kept.data_ptr()), P(ws.data_ptr()),
                ws_bytes, sp)
        st = (lib.kvsel_threshold_cut(*args) if events is None else
              lib.kvsel_threshold_cut_traced(*args, events, len(events)))
        if st != 0:
            raise RuntimeError(f"kvsel_threshold_cut: {K.status_string(st)}")

    r = time_calls(call, CUT_KERNELS, cut_cost(lengths, hq, hkv), steps, 4, hip)
    r["tokens"] = int(lengths.sum())
    r["step_bytes"] = int(lengths.sum()) * hkv * D * 2
    r["layer_bytes"] = layers[0][1].numel() * 2
    return r


def run_refreekv_rows(hip, n_layers, steps, k_rows=64):
    """The ReFreeKV cut from the last k_rows attention rows (the k > 1
    ablation; 28 q / 4 KV heads, so 7 * k_rows rows per KV head, scored in
    groups of 128) with the sink + suffix compaction of K and V, at the same
    Qwen2.5-7B shape and lengths as run_refreekv."""
    import torch

    from decode_eviction_amd import kvsel as K
    from decode_eviction_amd import synth
    hq, hkv, b = 28, 4, 16
    g = hq // hkv
    lengths = synth.refreekv_lengths(0, b)
    cap = int(lengths.max())
    layers = []
    for layer in range(2, 2 + n_layers):
        c = synth.cut_case(layer=layer, seed=0, lengths=lengths, cap=cap)
        v = np.random.default_rng(layer).integers(0, 65536, size=c.k.shape, dtype=np.uint16)
        layers.append((bf16_dev(synth.cut_rows_q(c, k_rows)), bf16_dev(c.k), bf16_dev(v)))
    ko = torch.empty_like(layers[0][1])
    vo = torch.empty_like(layers[0][2])
    lens = torch.from_numpy(lengths).to("cuda")
    kept = torch.empty((b, hkv), dtype=torch.int32, device="cuda")
    ws_bytes = K.kvsel_threshold_cut_rows_workspace(b, hq, hkv, D, cap, k_rows)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    lib = K.lib()
    sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    P = ctypes.c_void_p
    rows = g * k_rows
    groups = [min(128, rows - r0) for r0 in range(0, rows, 128)]
    names = [f"{kind}_g{i}" for i in range(len(groups)) for kind in ("stats", "reduce", "cut_energy")]
    names += ["cut_scan", "cut_compact"]
    tok = int(lengths.sum()) * hkv
    cost = {"cut_scan": {"bytes": 0}}
    for i, m in enumerate(groups):
        # groups of more than 32 rows store no logits: the energy kernel
        # recomputes them from Q and K (one more read of K)
        stored = m <= 32
        cost[f"stats_g{i}"] = {"bytes": tok * D * 2 + (tok * m * 4 if stored else 0)}
        cost[f"reduce_g{i}"] = {"bytes": 0}
        cost[f"cut_energy_g{i}"] = {"bytes": (tok * m * 4 if stored else tok * D * 2) +
                                    tok * 8 * (2 if i else 1)}

    def call(i, events=None):
        q, k, v = layers[i % len(layers)]
        args = (K.KVSEL_BF16, P(q.data_ptr()), k_rows, P(k.data_ptr()), P(v.data_ptr()),
                P(lens.data_ptr()), b, hq, hkv, D, cap, 2 + i % len(layers), 2, 4, 0.01,
                P(kept.data_ptr()), P(ko.data_ptr()), P(vo.data_ptr()), cap, P(ws.data_ptr()),
                ws_bytes, sp)
        st = (lib.kvsel_threshold_cut_rows(*args) if events is None else
              lib.kvsel_threshold_cut_rows_traced(*args, events, len(events)))
        if st != 0:
            raise RuntimeError(f"kvsel_threshold_cut_rows: {K.status_string(st)}")

    call(0)
    torch.cuda.synchronize()
    kept_tok = int(kept.sum().item())            # layer 2's kept rows: K and V read and written
    cost["cut_compact"] = {"bytes": kept_tok * D * 2 * 4}
    r = time_calls(call, names, cost, steps, 4, hip)
    r["tokens"] = int(lengths.sum())
    r["k_rows"] = k_rows
    r["kept_fraction"] = kept_tok / tok
    r["cost"] = cost
    return r


KERNEL_SOURCES = {"stats": "scores.hip", "reduce": "scores.hip", "pool": "scores.hip",
                  "gram": "gram.hip", "gram_fin": "gram.hip", "thresh": "select.hip", "select_compact": "select.hip",
                  "compact": "select.hip", "fused": "fused.hip", "fused_slots": "fused.hip", "scores": "fused.hip",
                  "pool_pairs": "scores.hip", "fused_fin_slots": "fused.hip", "scores_pairs": "fused.hip",
                  "evict": "select.hip", "select": "select.hip", "gather": "select.hip",
                  "cut_energy": "cut.hip", "cut_scan": "cut.hip", "cut_compact": "cut.hip"}


def source_digest(kernel: str) -> str:
    """sha1 over the sources a kernel is built from (its file and every
    shared header or included source)."""
    import hashlib
    h = hashlib.sha1()
    csrc = os.path.join(ROOT, "decode_eviction_amd", "csrc")
    shared = sorted(os.path.basename(p) for p in glob.glob(os.path.join(csrc, "*.hpp")) +
                    glob.glob(os.path.join(csrc, "*.inc")))
    for f in [KERNEL_SOURCES[kernel]] + shared:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(profiles: str, mode: str, kernel: str):
    """HBM bytes per launch from profiles/traffic_<mode>_<kernel>.txt (rocprofv3
    FETCH_SIZE + WRITE_SIZE, scaled by a plain copy); None when absent or when
    the kernel's sources changed since the counters were taken."""
    path = os.path.join(profiles, f"traffic_{mode}_{kernel}.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("source_sha1") != source_digest(kernel):
        return None
    return int(float(vals["bytes_per_launch"]))


def rocprof_avg_us(profiles: str, tag: str, kernel: str):
    """(average duration in us, file) of the workload's kernel from a committed
    rocprofv3 kernel-trace summary (profiles/kernel_trace_*.txt, lines
    "bench: <tag> | <kernel> | <rocprof name> | <avg_us> | <source sha1>"),
    or None when absent or when the kernel's sources changed since the trace."""
    for path in sorted(glob.glob(os.path.join(profiles, "kernel_trace_*.txt"))):
        with open(path) as f:
            for line in f:
                if not line.startswith("bench:"):
                    continue
                parts = [x.strip() for x in line[len("bench:"):].split("|")]
                if len(parts) == 5 and parts[0] == tag and parts[1] == kernel and \
                        parts[4] == source_digest(kernel):
                    return float(parts[3]), os.path.basename(path)
    return None


def roofline(res, cost, profiles, tag):
    """Roofline of the call's dominant (longest) kernel: algorithmic flops or
    bytes per launch over its average duration (HIP events on the launch
    stream, this run), with the counter-measured HBM traffic from
    profiles/traffic_<tag>_<kernel>.txt and the same figure over the rocprofv3
    kernel-trace duration committed under profiles/, each when current."""
    kern = res["kernels"]
    dom = max(kern, key=lambda k: kern[k]["avg_us"])
    c = cost[dom]
    traffic = measured_traffic(profiles, tag, dom)
    mfma = "flops" in c
    work, peak = (c["flops"], PEAK_BF16_TFLOPS) if mfma else (c["bytes"], PEAK_HBM_GBS)
    scale = 1e12 if mfma else 1e9
    ach = work / (kern[dom]["avg_us"] * 1e-6) / scale
    out = {"kernel": dom, "bound": "mfma" if mfma else "hbm", "achieved": round(ach, 1), "peak": peak,
           "unit": "TFLOP/s" if mfma else "GB/s", "frac": round(ach / peak, 4), "traffic": traffic,
           "duration_source": "hipEvent average over the traced pass of this run"}
    rp = rocprof_avg_us(profiles, tag, dom) if dom in KERNEL_SOURCES else None
    if rp is not None:
        a2 = work / (rp[0] * 1e-6) / scale
        out["rocprof"] = {"avg_us": rp[0], "achieved": round(a2, 1), "frac": round(a2 / peak, 4),
                          "source": "profiles/" + rp[1]}
    return out


def hbm_frac(nbytes, ms):
    return round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)


def cpu_baseline(case, seconds: float) -> dict:
    """Time the oracle (definition form) on whole heads of one layer."""
    from threadpoolctl import threadpool_info

    from oracle import rkv
    qf, kf, vf = case.as_f32("q"), case.as_f32("k"), case.as_f32("v")
    t0 = time.perf_counter()
    heads = 0
    while heads < HKV:
        rkv.score_evict(qf, kf, vf, case.lengths, LAM, BUDGET, form="definition",
                        heads=[(0, heads)])
        heads += 1
        if time.perf_counter() - t0 >= seconds:
            break
    el = time.perf_counter() - t0
    per_layer = el * HKV / heads
    t1 = time.perf_counter()
    rkv.score_evict(qf, kf, vf, case.lengths, LAM, BUDGET, form="keysum")
    ks = time.perf_counter() - t1
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1):
        t2 = time.perf_counter()
        rkv.score_evict(qf, kf, vf, case.lengths, LAM, BUDGET, form="definition", heads=[(0, 0)])
        one = time.perf_counter() - t2
    return {"value": round(N / per_layer, 1), "unit": "tokens/s/layer", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{heads} of {HKV} KV heads of one n={N} layer through the fp64 oracle "
                      f"(definition form: n x n cosine matrix), {el:.1f} s, scaled x{HKV / heads:g} "
                      f"to a layer; host has {os.cpu_count()} logical CPUs",
            "one_thread_value": round(N / (one * HKV), 1),
            "one_thread_sample": f"1 of {HKV} KV heads with one BLAS thread, {one:.1f} s, scaled x{HKV}",
            "keysum_form_value": round(N / ks, 1)}


def _per_run(fn, min_seconds: float) -> float:
    """Seconds per call of fn, repeated until min_seconds have passed (at least once)."""
    t0 = time.perf_counter()
    k = 0
    while True:
        fn()
        k += 1
        el = time.perf_counter() - t0
        if el >= min_seconds:
            return el / k


def cpu_config_baselines(seconds: float = 1.0) -> dict:
    """The oracle on each workload of the benchmark, with BLAS's default
    threads and with one thread: tokens/s of the key-sum (identity) form of
    the redundancy on every R-KV workload, of the pairwise definition on the
    tiny and n = 4096 configurations, and of the ReFreeKV cut.  Each figure
    times whole calls (or whole heads / sequences, scaled up) for about
    `seconds`; the oracle is a reported baseline, not a target."""
    from threadpoolctl import threadpool_info, threadpool_limits

    from decode_eviction_amd import synth
    from oracle import refreekv, rkv
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    out = {}

    def both(name, unit, tokens, fn, sample):
        mt = _per_run(fn, seconds)
        with threadpool_limits(limits=1):
            st = _per_run(fn, seconds)
        out[name] = {"value": round(tokens / mt, 1), "one_thread_value": round(tokens / st, 1),
                     "unit": unit, "threads": int(threads), "kind": "oracle", "sample": sample}

    c = synth.tiny_case(0)
    q, k, v = c.as_f32("q"), c.as_f32("k"), c.as_f32("v")
    for form in ("definition", "keysum"):
        both(f"tiny_{form}", "tokens/s", 512,
             lambda: rkv.score_evict(q, k, v, c.lengths, c.lam, c.budget, form=form),
             f"the whole tiny call (1 head, n=512, fp32), {form} form")
    c = synth.layer8b_case(0)
    q, k, v = c.as_f32("q"), c.as_f32("k"), c.as_f32("v")
    both("layer_n4096_definition", "tokens/s/layer", 4096 / 8,
         lambda: rkv.score_evict(q, k, v, c.lengths, c.lam, c.budget, form="definition", heads=[(0, 0)]),
         "one of 8 KV heads of the n=4096 layer, definition form (n x n cosine matrix), scaled x8")
    both("layer_n4096_keysum", "tokens/s/layer", 4096,
         lambda: rkv.score_evict(q, k, v, c.lengths, c.lam, c.budget, form="keysum"),
         "the whole n=4096 layer (8 KV heads), key-sum form")
    del c, q, k, v
    c = synth.headline_case(layer=0)
    q, k, v = c.as_f32("q"), c.as_f32("k"), c.as_f32("v")
    both("headline_keysum", "tokens/s/layer", N,
         lambda: rkv.score_evict(q, k, v, c.lengths, c.lam, c.budget, form="keysum"),
         "the whole n=32768 layer (8 KV heads), key-sum form")
    del c, q, k, v
    ds = synth.decode_stream(0, total=2176 + 128)
    qd = synth.bf16_bits_to_f32(ds.window(2176, W))
    kd = synth.bf16_bits_to_f32(ds.k[None, :, :2176])
    vd = synth.bf16_bits_to_f32(ds.v[None, :, :2176])
    both("decode_keysum", "cache tokens scored/s", 2176,
         lambda: rkv.score_evict(qd, kd, vd, [2176], LAM, 2048, form="keysum"),
         "one decode-loop call (2176-slot cache, 8 KV heads, B=2048), key-sum form")
    c = synth.batched_case(seed=0, b=4)
    q, k, v = c.as_f32("q"), c.as_f32("k"), c.as_f32("v")
    both("batched_keysum", "tokens/s/layer", 4 * 8192,
         lambda: rkv.score_evict(q, k, v, c.lengths, c.lam, c.budget, form="keysum"),
         "4 of the 64 sequences of 8192 tokens (8 KV heads each), key-sum form")
    del c, q, k, v
    cc = synth.cut_case(layer=2)
    qc, kc = cc.as_f32("q"), cc.as_f32("k")
    both("refreekv", "tokens/s/layer", int(np.sum(cc.lengths)),
         lambda: refreekv.threshold_cut(qc, kc, cc.lengths, 2),
         "one scored layer (16 ragged sequences of 1K-16K tokens, 4 KV heads) of the threshold cut")
    return out


def copy_calibration(mib: int = 512):
    """A plain device copy of known size, for scaling HBM byte counters."""
    import torch
    a = torch.empty(mib << 20, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": mib << 20, "launches": 5}))


def achievable_copy(mib: int = 1024, reps: int = 10) -> dict:
    """What a plain device-to-device copy reaches on this GPU (torch's copy
    kernel, 1 GiB read + 1 GiB written per launch, timed with events on its
    own stream), reported beside the kernels' fractions of the nameplate
    peak."""
    import torch
    src = torch.empty(mib << 20, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    for _ in range(3):
        dst.copy_(src)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        dst.copy_(src)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / reps
    gbps = 2 * (mib << 20) / (ms * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return {"GBps": round(gbps, 1), "frac_of_peak": round(gbps / PEAK_HBM_GBS, 4),
            "bytes_per_launch": 2 * (mib << 20), "kernel": "torch copy_ (read + write)"}


def run_variants(a, hip) -> dict:
    """The other workloads, each reported with its own value and kernels."""
    import torch
    want = a.variant or ["decode", "batched", "refreekv", "refreekv_rows"]
    out = {}

    def log(name, r):
        print(f"# {name}: {r['ms_plain'] * 1000:.1f} us/call, {r['ms'] * 1000:.1f} us/call traced; "
              + ", ".join(f"{k} {v['avg_us']:.1f}us" for k, v in r["kernels"].items()),
              file=sys.stderr, flush=True)

    if "decode" in want:
        for mode in KERNELS:
            r = run_decode(mode, a.decode_layers, hip, a.decode_calls)
            log(f"decode/{mode}", r)
            out[f"decode_{mode}"] = {
                "workload": "R-KV decode loop: 32 layers x 240 calls, each compressing a "
                            "2176-slot cache to B=2048 (8B shape, batch 1, w=8)",
                "value": round(r["tokens"] / (r["ms_plain"] * 1e-3 * r["calls"]), 1),
                "unit": "cache tokens scored/s", "us_per_call": round(r["ms_plain"] * 1000, 2),
                "us_per_call_traced": round(r["ms"] * 1000, 2), "calls": r["calls"],
                "loop_ms": round(r["ms_plain"] * r["calls"], 3),
                "roofline": roofline(r, rkv_cost(mode, 1, 2176, 2048), a.profiles, f"decode_{mode}"),
                "step_hbm_frac": hbm_frac(rkv_step_bytes(1, 2176, 2048), r["ms_plain"]),
                "kernels": r["kernels"]}
            torch.cuda.empty_cache()
    if "decode" in want:
        for mode in KERNELS:
            r = run_decode_slots(mode, a.decode_layers, hip, a.decode_calls)
            log(f"decode_slots/{mode}", r)
            tok = HKV * 2176
            out[f"decode_slots_{mode}"] = {
                "workload": "R-KV decode loop with slot reuse: 32 layers x 240 calls, each scoring "
                            "a 2176-slot cache, listing the 128 evicted slots per head and "
                            "writing the next 128 tokens into them (no compaction)",
                "value": round(r["tokens"] / (r["ms_plain"] * 1e-3 * r["calls"]), 1),
                "unit": "cache tokens scored/s", "us_per_call": round(r["ms_plain"] * 1000, 2),
                "us_per_call_traced": round(r["ms"] * 1000, 2), "calls": r["calls"],
                "loop_ms": round(r["ms_plain"] * r["calls"], 3),
                "roofline": roofline(r, rkv_cost(mode, 1, 2176, 2048), a.profiles,
                                     f"decode_slots_{mode}"),
                "step_hbm_frac": hbm_frac(tok * D * 2 + 3 * 4 * tok + 4 * HKV * 128 * D * 2,
                                          r["ms_plain"]),
                "kernels": r["kernels"]}
            torch.cuda.empty_cache()
    if "batched" in want:
        for mode in KERNELS:
            r = run_batched(mode, hip, a.batched_steps or (16 if mode == "keysum" else 6))
            log(f"batched/{mode}", r)
            out[f"batched_{mode}"] = {
                "workload": "R-KV batched: 64 sequences x 8192 tokens, B=1024 (8B shape, w=8)",
                "value": round(r["tokens"] / (r["ms_plain"] * 1e-3), 1), "unit": "tokens/s/layer",
                "ms_per_step": round(r["ms_plain"], 5), "ms_per_step_traced": round(r["ms"], 5),
                "roofline": roofline(r, rkv_cost(mode, 64, 8192, 1024), a.profiles, f"batched_{mode}"),
                "step_hbm_frac": hbm_frac(r["step_bytes"], r["ms_plain"]), "kernels": r["kernels"]}
            torch.cuda.empty_cache()
    if "refreekv" in want:
        r = run_refreekv(hip, 4, 32)
        log("refreekv", r)
        out["refreekv"] = {
            "workload": "ReFreeKV threshold cut, one scored layer at the Qwen2.5-7B shape: 28 q / "
                        "4 KV heads, d=128, 16 sequences of 1024-16384 tokens (sum "
                        f"{r['tokens']}), m=4, T=0.01; 4 distinct layers of "
                        f"{r['layer_bytes'] >> 20} MiB K rotated",
            "value": round(r["tokens"] / (r["ms_plain"] * 1e-3), 1), "unit": "tokens/s/layer",
            "ms_per_step": round(r["ms_plain"], 5), "ms_per_step_traced": round(r["ms"], 5),
            "roofline": roofline(r, cut_cost(synth_lengths(), 28, 4), a.profiles, "refreekv"),
            "step_hbm_frac": hbm_frac(r["step_bytes"], r["ms_plain"]), "kernels": r["kernels"]}
    if "refreekv_rows" in want:
        r = run_refreekv_rows(hip, 4, 8)
        log("refreekv_rows", r)
        out["refreekv_rows"] = {
            "workload": f"ReFreeKV cut from the last {r['k_rows']} attention rows per query head "
                        "(the k > 1 ablation: 7*k rows per KV head, causal) with the sink + "
                        "suffix compaction of K and V; same Qwen2.5-7B shape and 16 sequences as "
                        "refreekv",
            "value": round(r["tokens"] / (r["ms_plain"] * 1e-3), 1), "unit": "tokens/s/layer",
            "ms_per_step": round(r["ms_plain"], 5), "ms_per_step_traced": round(r["ms"], 5),
            "kept_fraction": round(r["kept_fraction"], 4),
            "roofline": roofline(r, r["cost"], a.profiles, "refreekv_rows"),
            "kernels": r["kernels"]}
    return out


def synth_lengths():
    from decode_eviction_amd import synth
    return synth.refreekv_lengths(0, 16)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--mode", choices=["gram", "keysum"], default="gram")
    ap.add_argument("--layers", type=int, default=32)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only-mode", action="store_true", help="skip the other redundancy form")
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the decode-loop, batched and ReFreeKV workloads")
    ap.add_argument("--variant", action="append",
                    choices=["decode", "batched", "refreekv", "refreekv_rows", "heads"],
                    help="run only these extra workloads (repeatable)")
    ap.add_argument("--profiles", default=os.path.join(ROOT, "profiles"))
    ap.add_argument("--variants-only", action="store_true",
                    help="skip the headline workload and print only the variants (for profiling)")
    # shorter variant runs for counter collection (which serialises every kernel)
    ap.add_argument("--decode-layers", type=int, default=32)
    ap.add_argument("--decode-calls", type=int, default=240)
    ap.add_argument("--batched-steps", type=int, default=0)
    a = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if a.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the score-and-evict step shards over independent "
              "(sequence, layer, KV head) units with no exchange, so a multi-GPU figure is N "
              "independent copies of this one; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    if a.calibrate_copy:
        copy_calibration()
        return
    torch.cuda.init()
    hip = Hip()
    if a.variants_only:
        print(json.dumps({"variants": run_variants(a, hip)}))
        return
    layers, first = make_layers(a.layers)
    torch.cuda.synchronize()


    res = {}
    order = [a.mode] + ([] if a.only_mode else [m for m in KERNELS if m != a.mode])
    for mode in order:
        res[mode] = run_mode(mode, layers, a.steps, a.warmup, hip)
        print(f"# {mode}: {res[mode]['ms_plain'] * 1000:.1f} us/step, "
              f"{res[mode]['ms'] * 1000:.1f} us/step traced; "
              + ", ".join(f"{k} {v['avg_us']:.1f}us" for k, v in res[mode]["kernels"].items()),
              file=sys.stderr, flush=True)

    main_res = res[a.mode]
    out = {
        "metric": METRIC,
        "value": round(N / (main_res["ms_plain"] * 1e-3), 1),
        "unit": "tokens/s/layer",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(main_res["ms_plain"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; K ~ N(0,1) with 30% near-copy runs and x8 sinks, V ~ N(0,1))",
        "config": {"workload": "R-KV score-and-evict, one layer at the 8B shape: 32 q / 8 KV heads, "
                               "d=128, batch 1, n=32768, w=8, B=2048, lambda=0.1",
                   "redundancy": a.mode, "distinct_layer_caches": a.layers,
                   "kernels_per_step": len(rkv_kernels(a.mode, N))},
        "roofline": roofline(main_res, rkv_cost(a.mode), a.profiles, a.mode),
        "step_hbm_frac": hbm_frac(rkv_step_bytes(), main_res["ms_plain"]),
        "ms_per_step_traced": round(main_res["ms"], 5),
        "kernels": main_res["kernels"],
    }
    out["hbm_copy"] = achievable_copy()
    for mode in order[1:]:
        r = res[mode]
        out.setdefault("variants", {})[mode] = {
            "value": round(N / (r["ms_plain"] * 1e-3), 1), "ms_per_step": round(r["ms_plain"], 5),
            "ms_per_step_traced": round(r["ms"], 5),
            "roofline": roofline(r, rkv_cost(mode), a.profiles, mode),
            "step_hbm_frac": hbm_frac(rkv_step_bytes(), r["ms_plain"]), "kernels": r["kernels"]}
    if not a.no_variants and (a.variant is None or "heads" in a.variant):
        for mode in order:
            r = run_heads(mode, layers, a.steps, a.warmup, hip)
            print(f"# heads/{mode}: {r['ms_plain'] * 1000:.1f} us/step, "
                  f"{r['ms'] * 1000:.1f} us/step traced; "
                  + ", ".join(f"{k} {v['avg_us']:.1f}us" for k, v in r["kernels"].items()),
                  file=sys.stderr, flush=True)
            out.setdefault("variants", {})[f"heads_{mode}"] = {
                "workload": "the headline layer with per-KV-head budgets "
                            f"{HEAD_BUDGETS} (sum {sum(HEAD_BUDGETS)})",
                "value": round(N / (r["ms_plain"] * 1e-3), 1), "unit": "tokens/s/layer",
                "ms_per_step": round(r["ms_plain"], 5), "ms_per_step_traced": round(r["ms"], 5),
                "roofline": roofline(r, rkv_cost(mode), a.profiles, f"heads_{mode}"),
                "step_hbm_frac": hbm_frac(rkv_step_bytes(), r["ms_plain"]),
                "kernels": r["kernels"]}
    del layers
    torch.cuda.empty_cache()
    if not a.no_variants:
        out.setdefault("variants", {}).update(run_variants(a, hip))
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(first, a.cpu_seconds)
        # the oracle on every workload, beside the workload's own figures
        per = cpu_config_baselines()
        out["cpu_baseline"]["configs"] = per
        where = {"decode_keysum": "decode_keysum", "batched_keysum": "batched_keysum",
                 "refreekv": "refreekv", "headline_keysum": "keysum"}
        for key, var in where.items():
            if var in out.get("variants", {}):
                out["variants"][var]["cpu_baseline"] = per[key]
    print(json.dumps(out))


if __name__ == "__main__":
    main()
