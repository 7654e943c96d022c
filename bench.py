"""Benchmark: KV tokens scored+evicted per second per layer on one MI355X.

Workload: one R-KV score-and-evict call per step at the 8B shape (32 query /
8 KV heads, d = 128, bf16, batch 1, n = 32768 cached tokens, window w = 8,
budget B = 2048, lambda = 0.1).  Steps rotate over --layers distinct seeded
synthetic layer caches (32 x 128 MiB of K+V, beyond the 256 MB last-level
cache) that are resident in HBM before timing starts.

Per step the library launches stats, reduce, pool, [gram,] thresh, compact
(the compaction kernel also gathers the kept K/V rows).
The timed region (`value`, `ms_per_step`) runs kvsel_score_evict; right
after it the same steps run through kvsel_score_evict_traced, whose kernels
record start/stop HIP events on the benchmark's stream, giving each kernel's
average duration (the roofline figure uses the dominant kernel's).  Both redundancy forms are
measured; --mode picks which one is the headline `value`.

The CPU baseline times the fp64 oracle (definition form, n x n cosine
matrix) on a bounded sample: whole KV heads of one layer until --cpu-seconds
have passed, scaled to a full layer.

    python bench.py [--gpus 1] [--steps 64] [--warmup 8] [--mode gram|keysum]
"""

from __future__ import annotations

import argparse
import ctypes
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
    "gram": ["stats", "reduce", "pool", "gram", "thresh", "compact"],
    "keysum": ["stats", "reduce", "pool", "thresh", "compact"],
}


def algorithmic_cost(mode: str) -> dict:
    """Bytes (and flops) each kernel must move per call at the headline shape.

    K bytes = Hkv*n*d*2; scores are fp32 per token per head; the gather moves
    B kept rows of K and V in and out."""
    kb = HKV * N * D * 2
    tok = HKV * N
    gath = 2 * 2 * HKV * BUDGET * D * 2
    cost = {
        "stats": {"bytes": kb + (4 * tok if mode == "gram" else 0)},
        "reduce": {"bytes": 0},
        "pool": {"bytes": kb + (4 * tok if mode == "gram" else 8 * tok)},
        "thresh": {"bytes": 4 * tok},
        "compact": {"bytes": 4 * tok + 4 * HKV * BUDGET + gath},
    }
    if mode == "gram":
        cost["gram"] = {"bytes": kb + 4 * tok * 3, "flops": 2.0 * N * N * D * HKV}
    return cost


def step_bytes(mode: str) -> int:
    """Algorithmic floor of one call: K once, scores, the gather."""
    return HKV * N * D * 2 + 3 * 4 * HKV * N + 2 * 2 * HKV * BUDGET * D * 2


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


def run_mode(mode, layers, steps, warmup, hip):
    import torch

    from decode_eviction_amd import kvsel as K
    lib = K.lib()
    mcode = K.MODES[mode]
    names = KERNELS[mode]
    nk = len(names)
    lens = torch.tensor([N], dtype=torch.int32, device="cuda")
    k_out = torch.empty((1, HKV, BUDGET, D), dtype=torch.bfloat16, device="cuda")
    v_out = torch.empty_like(k_out)
    idx = torch.empty((1, HKV, BUDGET), dtype=torch.int32, device="cuda")
    ws_bytes = K.kvsel_score_evict_workspace(1, HQ, HKV, D, W, N, BUDGET)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    P = ctypes.c_void_p

    def call(i, events=None):
        q, k, v = layers[i % len(layers)]
        args = (K.KVSEL_BF16, mcode, P(q.data_ptr()), P(k.data_ptr()), P(v.data_ptr()),
                P(lens.data_ptr()), 1, HQ, HKV, D, W, N, LAM, BUDGET, P(k_out.data_ptr()),
                P(v_out.data_ptr()), BUDGET, P(idx.data_ptr()), None, P(ws.data_ptr()), ws_bytes, sp)
        if events is None:
            st = lib.kvsel_score_evict(*args)
        else:
            st = lib.kvsel_score_evict_traced(*args, events, 2 * nk)
        if st != 0:
            raise RuntimeError(f"kvsel_score_evict: {K.status_string(st)}")

    for i in range(warmup):
        call(i)
    torch.cuda.synchronize()

    # timed region: the plain library call
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(steps):
        call(i)
    t1.record()
    torch.cuda.synchronize()
    ms_plain = t0.elapsed_time(t1) / steps

    # the same steps again with per-kernel events on the same stream
    evs = [hip.events(2 * nk) for _ in range(steps)]
    torch.cuda.synchronize()
    t0.record()
    for i in range(steps):
        call(i, evs[i])
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    per = {nm: [] for nm in names}
    for e in evs:
        for j, nm in enumerate(names):
            per[nm].append(hip.elapsed_ms(e[2 * j], e[2 * j + 1]))
        hip.destroy(e)
    kern = {}
    cost = algorithmic_cost(mode)
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


KERNEL_SOURCES = {"stats": "scores.hip", "reduce": "scores.hip", "pool": "scores.hip",
                  "gram": "gram.hip", "thresh": "select.hip", "compact": "select.hip"}


def source_digest(kernel: str) -> str:
    """sha1 over the sources a kernel is built from (its file + common.hpp)."""
    import hashlib
    h = hashlib.sha1()
    for f in (KERNEL_SOURCES[kernel], "common.hpp", "kernels.hpp"):
        with open(os.path.join(ROOT, "decode_eviction_amd", "csrc", f), "rb") as fh:
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


def roofline(mode, res, profiles):
    kern = res["kernels"]
    dom = max(kern, key=lambda k: kern[k]["avg_us"])
    c = algorithmic_cost(mode)[dom]
    traffic = measured_traffic(profiles, mode, dom)
    if "flops" in c:
        ach = c["flops"] / (kern[dom]["avg_us"] * 1e-6) / 1e12
        return {"kernel": dom, "bound": "mfma", "achieved": round(ach, 1), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4), "traffic": traffic}
    ach = c["bytes"] / (kern[dom]["avg_us"] * 1e-6) / 1e9
    return {"kernel": dom, "bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": traffic}


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
    return {"value": round(N / per_layer, 1), "unit": "tokens/s/layer", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{heads} of {HKV} KV heads of one n={N} layer through the fp64 oracle "
                      f"(definition form: n x n cosine matrix), {el:.1f} s, scaled x{HKV / heads:g} "
                      f"to a layer; host has {os.cpu_count()} logical CPUs",
            "keysum_form_value": round(N / ks, 1)}


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
    ap.add_argument("--profiles", default=os.path.join(ROOT, "profiles"))
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
                   "kernels_per_step": len(KERNELS[a.mode])},
        "roofline": roofline(a.mode, main_res, a.profiles),
        "step_hbm_frac": round(step_bytes(a.mode) / (main_res["ms_plain"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "ms_per_step_traced": round(main_res["ms"], 5),
        "kernels": main_res["kernels"],
    }
    for mode in order[1:]:
        r = res[mode]
        out.setdefault("variants", {})[mode] = {
            "value": round(N / (r["ms_plain"] * 1e-3), 1), "ms_per_step": round(r["ms_plain"], 5),
            "ms_per_step_traced": round(r["ms"], 5), "roofline": roofline(mode, r, a.profiles),
            "step_hbm_frac": round(step_bytes(mode) / (r["ms_plain"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "kernels": r["kernels"]}
    del layers
    torch.cuda.empty_cache()
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(first, a.cpu_seconds)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
