"""Decoding-time compression loop (R-KV article, section "R-KV三步走": compress
while decoding so the cache stops growing) at the R1-Llama-8B shape.

Per layer a 32,768-token synthetic key/value stream (40% near-duplicate loop
segments, x8 sinks) is appended to a cache of capacity B + 128 = 2176; each
time the cache is full, kvsel_score_evict keeps B = 2048 tokens into the
other buffer of a ping-pong pair (240 calls per layer).  On sampled steps the
oracle re-runs the step on the GPU's own pre-step cache (an allowed swap
changes later states, so each step is checked on its own input); on every
step the kept rows are checked bit-exact against the stream at the tracked
original positions.  Every one of the 32 layers runs its 240 calls; the
first and the last call of each layer (and every 40th call of two layers)
are checked against the oracle.
"""

import numpy as np
import pytest
import torch

from decode_eviction_amd import kvsel as K
from decode_eviction_amd import synth
from oracle import rkv
from tests.gpu_util import SWAP_WINDOW, check_idx_structure, dev, host_bits, log, score_err, swaps

pytestmark = pytest.mark.gpu

B, BUF, W, LAM = 2048, 128, 8, 0.1


def run_layer(layer, mode, check_calls):
    st = synth.decode_stream(layer)
    cap = B + BUF
    hkv, d = st.hkv, st.d
    ks = dev(st.k, "bf16")                      # [hkv][total][d]
    vs = dev(st.v, "bf16")
    kc = [torch.zeros((1, hkv, cap, d), dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    vc = [torch.zeros((1, hkv, cap, d), dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    pos = np.zeros((hkv, cap), np.int64)        # original token position of each cache row
    lens = torch.tensor([cap], dtype=torch.int32, device="cuda")
    z = torch.empty((1, hkv, cap), dtype=torch.float32, device="cuda")
    ws = torch.empty(K.kvsel_score_evict_workspace(1, st.hq, hkv, d, W, cap, B), dtype=torch.uint8,
                     device="cuda")
    cur, length, t, calls, checked = 0, 0, 0, 0, 0
    worst, nswaps = 0.0, 0
    while t < st.total:
        take = min(cap - length, st.total - t)
        kc[cur][0, :, length:length + take] = ks[:, t:t + take]
        vc[cur][0, :, length:length + take] = vs[:, t:t + take]
        pos[:, length:length + take] = np.arange(t, t + take)
        length += take
        t += take
        if length < cap:
            break
        qw = dev(st.window(t, W), "bf16")
        check = calls in check_calls
        if check:
            k_pre = host_bits(kc[cur])
            v_pre = host_bits(vc[cur])
        _, _, idx = K.kvsel_score_evict(qw, kc[cur], vc[cur], lens, B, LAM, mode,
                                        k_out=kc[1 - cur], v_out=vc[1 - cur], scores_out=z,
                                        workspace=ws)
        idx_h = idx.cpu().numpy()[0]
        for h in range(hkv):
            check_idx_structure(idx_h[h], cap, B)
            pos[h, :B] = pos[h, idx_h[h]]
        kept = host_bits(kc[1 - cur])[0, :, :B]
        for h in range(hkv):
            assert np.array_equal(kept[h], st.k[h, pos[h, :B]]), f"step {calls} head {h}"
        if check:
            zf = z.cpu().numpy()[0]
            qf = synth.bf16_bits_to_f32(host_bits(qw))
            ref = rkv.score_evict(qf, synth.bf16_bits_to_f32(k_pre), synth.bf16_bits_to_f32(v_pre),
                                  [cap], LAM, B)
            for h in range(hkv):
                worst = max(worst, score_err(zf[h], ref["Z"][0][h]))
                ns, gap = swaps(idx_h[h], ref["idx"][0, h], ref["Z"][0][h])
                nswaps += ns
                assert gap < SWAP_WINDOW, (calls, h, gap)
            checked += 1
        cur = 1 - cur
        length = B
        calls += 1
    log(f"[decode] layer={layer} mode={mode}: {calls} calls, {checked} checked against the oracle, "
        f"worst Z err {worst:.2e}, swaps {nswaps}")
    assert calls == 240
    assert worst <= 1e-3


LAYERS = [(layer, "keysum" if layer % 2 == 0 else "gram") for layer in range(32)]


@pytest.mark.parametrize("layer,mode", LAYERS, ids=[f"L{l}-{m}" for l, m in LAYERS])
def test_decode_loop_layer(layer, mode):
    checks = {0, 239}
    if layer in (0, 17):
        checks |= set(range(0, 240, 40))
    run_layer(layer, mode, checks)
