"""The library's launch sequences under HIP graph capture (a decode loop that
replays one captured step per layer): no memory sets are recorded, so each
replay must reproduce the eager outputs exactly.  Replays are separated by
eager work and synchronisations, and every replay is checked."""

import numpy as np
import pytest
import torch

from decode_eviction_amd import kvsel as K
from decode_eviction_amd import synth
from tests.gpu_util import dev, dev_i32, log

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n", [2176, 32768])
@pytest.mark.parametrize("mode", ["keysum", "gram"])
def test_score_evict_graph_replays(mode, n):
    # n = 2176: the one-launch short-cache step (key-sum) and the pooling
    # with the pair-block Gram units (Gram); n = 32768: the one-launch score
    # pass and the one-launch selection, whose tags change every replay
    case = synth.layer8b_case(2, n=n, budget=2048, cap=n)
    q, k, v = dev(case.q, "bf16"), dev(case.k, "bf16"), dev(case.v, "bf16")
    lens = dev_i32(case.lengths)
    b, hq, w, d = case.q.shape
    hkv, cap = case.k.shape[1], case.k.shape[2]
    ws = torch.empty(K.kvsel_score_evict_workspace(b, hq, hkv, d, w, cap, 2048), dtype=torch.uint8,
                     device="cuda")
    ko = torch.empty((b, hkv, 2048, d), dtype=torch.bfloat16, device="cuda")
    vo = torch.empty_like(ko)
    idx = torch.empty((b, hkv, 2048), dtype=torch.int32, device="cuda")
    z = torch.empty((b, hkv, cap), dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()

    def step():
        K.kvsel_score_evict(q, k, v, lens, 2048, 0.1, mode, k_out=ko, v_out=vo, idx_out=idx,
                            scores_out=z, workspace=ws, stream=s)

    with torch.cuda.stream(s):
        step()
    torch.cuda.synchronize()
    want = [t.clone() for t in (ko, vo, idx, z)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        for t in (ko, vo, idx, z):
            t.fill_(-3)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for t, w_ in zip((ko, vo, idx, z), want):
            assert torch.equal(t, w_), (mode, rep)
        with torch.cuda.stream(s):
            step()                                 # eager work between replays
        torch.cuda.synchronize()
    log(f"[graph] {mode} n={n}: 4 replays equal to the eager step")


def test_threshold_cut_graph_replays():
    case = synth.cut_case(8, b=4, lengths=[3000, 777, 9000, 129])
    q, k, lens = dev(case.q, "bf16"), dev(case.k, "bf16"), dev_i32(case.lengths)
    kept = torch.empty((4, case.hkv), dtype=torch.int32, device="cuda")
    ws = torch.empty(K.kvsel_threshold_cut_workspace(4, case.hq, case.hkv, case.d, case.cap),
                     dtype=torch.uint8, device="cuda")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        K.kvsel_threshold_cut(q, k, lens, 8, kept_out=kept, workspace=ws, stream=s)
    torch.cuda.synchronize()
    want = kept.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        K.kvsel_threshold_cut(q, k, lens, 8, kept_out=kept, workspace=ws, stream=s)
    torch.cuda.synchronize()
    for rep in range(4):
        kept.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(kept, want), rep


@pytest.mark.parametrize("mode", ["keysum", "gram"])
def test_score_evict_slots_graph_replays(mode):
    # the slot-reuse entry on the decode cache: the one-launch step's slot
    # form (key-sum) or the Gram finish (Gram), captured once and replayed
    case = synth.layer8b_case(3, n=2176, budget=2048, cap=2176)
    q, k = dev(case.q, "bf16"), dev(case.k, "bf16")
    lens = dev_i32(case.lengths)
    b, hq, w, d = case.q.shape
    hkv, cap = case.k.shape[1], case.k.shape[2]
    rng = np.random.default_rng(5)
    pos = dev_i32(np.stack([rng.permutation(50_000)[:cap] for _ in range(hkv)])[None])
    ws = torch.empty(K.kvsel_score_evict_workspace(b, hq, hkv, d, w, cap, 2048), dtype=torch.uint8,
                     device="cuda")
    ev = torch.empty((b, hkv, cap), dtype=torch.int32, device="cuda")
    ne = torch.empty((b, hkv), dtype=torch.int32, device="cuda")
    z = torch.empty((b, hkv, cap), dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()

    def step():
        K.kvsel_score_evict_slots(q, k, lens, 2048, 0.1, mode, pos=pos, evict_out=ev, n_evict_out=ne,
                                  scores_out=z, workspace=ws, stream=s)

    with torch.cuda.stream(s):
        step()
    torch.cuda.synchronize()
    want = [t.clone() for t in (ev, ne, z)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        for t in (ev, ne, z):
            t.fill_(-3)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for t, w_ in zip((ev, ne, z), want):
            assert torch.equal(t, w_), (mode, rep)
        with torch.cuda.stream(s):
            step()                                 # eager work between replays
        torch.cuda.synchronize()
    log(f"[graph] slots {mode}: 4 replays equal to the eager step")
