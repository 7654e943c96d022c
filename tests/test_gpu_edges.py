"""Edge cases of both methods on the GPU against the oracle (through the C ABI).

* Zero-norm keys inside bf16 d=128 heads (reading R6: a zero key has cosine 0
  with everything and still counts in n - 1), on each Gram kernel (the
  pair-block kernel below 4097 positions, the 256-key blocks up to 8191,
  the 512-key blocks from 8192) and in the key-sum form.
* lambda = 1 (the score is the attention importance alone) and lambda = 0
  (the score is minus the redundancy) end to end.
* The whole step above 32768 positions (single-kernel select, then gather).
* Negative lengths: treated as empty and flagged.
* The ReFreeKV cut end to end at T = 0.001 and 0.1 and with 0 or 10 sinks,
  and the zero-energy case of the fixed-point walk (tau = 0).
* A call on a stream other than the current one (binding allocations are
  made on the launch stream).
"""

import numpy as np
import pytest
import torch

from decode_eviction_amd import kvsel as K
from decode_eviction_amd import synth
from oracle import refreekv as rf
from oracle import rkv
from tests.gpu_util import dev, dev_i32, host_bits, log
from tests.test_gpu_refreekv import _valid_cut
from tests.test_gpu_rkv import MODES, check_case, gpu_run

pytestmark = pytest.mark.gpu


def _zero_keys(case, positions):
    """Zero the keys at the given positions in every head (bf16 +0 bits)."""
    for b in range(case.b):
        n = int(case.lengths[b])
        for p in positions:
            if p < n:
                case.k[b, :, p] = 0
    return case


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("cap,lengths", [(3000, [3000, 2047]), (6000, [5999, 4500]),
                                         (9216, [9216, 8300])])
def test_zero_norm_keys(mode, cap, lengths):
    case = synth.rkv_case("zerokeys", seed=41, wl=71, b=2, hq=16, hkv=4, d=128, w=8,
                          lengths=lengths, cap=cap, budget=700)
    n0 = min(lengths)
    _zero_keys(case, [1, 5, 127, 128, 255, 511, 512, n0 // 2, n0 - 1, max(lengths) - 1])
    got, ref = check_case(case, mode, form="keysum", sample_rows=8)
    for b in range(case.b):
        n = int(case.lengths[b])
        for p in (5, 127, n0 // 2):
            # a zero key is orthogonal to everything: R = 0 exactly (no NaN)
            assert got["R"][b, 0, p] == 0.0
            assert ref["R"][b][0][p] == 0.0


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("lam", [1.0, 0.0])
def test_lambda_extremes(mode, lam):
    case = synth.rkv_case("lam", seed=42, wl=72, b=1, hq=32, hkv=8, d=128, w=8,
                          lengths=[4000], cap=4096, budget=1024, lam=lam)
    got, ref = check_case(case, mode, form="keysum")
    # lam = 1: Z is I itself; lam = 0: Z is -R
    for h in range(case.hkv):
        want = ref["I"][0][h] if lam == 1.0 else -ref["R"][0][h]
        assert np.array_equal(ref["Z"][0][h], want)


@pytest.mark.parametrize("mode", MODES)
def test_whole_step_cap_above_32768(mode):
    case = synth.rkv_case("bigcap", seed=43, wl=73, b=2, hq=8, hkv=2, d=128, w=8,
                          lengths=[40000, 33001], cap=40001, budget=3000)
    check_case(case, mode, form="keysum", sample_rows=16)


@pytest.mark.parametrize("mode", MODES)
def test_negative_length_is_empty_and_flagged(mode):
    case = synth.rkv_case("neglen", seed=44, wl=74, b=3, hq=8, hkv=2, d=128, w=4,
                          lengths=[700, 0, 512], cap=768, budget=256)
    q, k, v = dev(case.q, "bf16"), dev(case.k, "bf16"), dev(case.v, "bf16")
    ws = torch.empty(K.kvsel_score_evict_workspace(3, 8, 2, 128, 4, 768, 256), dtype=torch.uint8,
                     device="cuda")
    ko0, vo0, idx0 = K.kvsel_score_evict(q, k, v, dev_i32([700, 0, 512]), 256, 0.1, mode,
                                         workspace=ws)
    assert K.kvsel_workspace_error(ws) == 0
    ko1, vo1, idx1 = K.kvsel_score_evict(q, k, v, dev_i32([700, -5, 512]), 256, 0.1, mode,
                                         workspace=ws)
    assert K.kvsel_workspace_error(ws) == 1
    assert np.array_equal(idx0.cpu().numpy(), idx1.cpu().numpy())
    assert (idx1.cpu().numpy()[1] == -1).all()
    assert np.array_equal(host_bits(ko0), host_bits(ko1))


@pytest.mark.parametrize("T,m", [(0.001, 4), (0.1, 4), (0.01, 0), (0.01, 10)])
def test_cut_end_to_end_T_and_sinks(T, m):
    case = synth.cut_case(9)
    log(f"[cut] T={T} m={m} lengths={case.lengths.tolist()[:4]}")
    got = K.kvsel_threshold_cut(dev(case.q, "bf16"), dev(case.k, "bf16"), dev_i32(case.lengths),
                                9, n_sink=m, T=T).cpu().numpy()
    L_ref, es = rf.threshold_cut(case.as_f32("q"), case.as_f32("k"), case.lengths, 9, m=m, T=T)
    exact = 0
    for (bi, h), e in es.items():
        assert _valid_cut(e, int(got[bi, h]), m, T), (bi, h, int(got[bi, h]), int(L_ref[bi, h]))
        exact += int(got[bi, h] == L_ref[bi, h])
    log(f"    exact-match rate {exact / len(es):.3f}")
    assert exact / len(es) >= 0.9


def test_cut_zero_energy_rows():
    # all-zero attention rows: total energy 0, tau = 0, the first queued
    # token reaches it: L = max(min(m, n), 1)
    b, hq, hkv, cap = 3, 4, 2, 600
    lens = np.array([600, 1, 37], np.int32)
    attn = np.zeros((b, hq, cap), np.float32)
    attn[2, 2:] = np.float32(1.0 / 37)                   # one group of sequence 2 uniform
    attn[2, 2:, 37:] = 0.0
    for m in (0, 4):
        got = K.kvsel_threshold_cut_from_attn(dev(attn, "f32"), dev_i32(lens), hkv, m, 0.01)
        want = rf.threshold_cut_from_attn(attn, lens, hkv, m, 0.01)
        assert np.array_equal(got.cpu().numpy(), want), m
        assert int(want[0, 0]) == max(min(m, 600), 1)


@pytest.mark.parametrize("mode", MODES)
def test_call_on_a_side_stream(mode):
    case = synth.layer8b_case(3, n=3000, budget=600, cap=3072)
    ref = gpu_run(case, mode)
    q, k, v = dev(case.q, "bf16"), dev(case.k, "bf16"), dev(case.v, "bf16")
    lens = dev_i32(case.lengths)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    outs = []
    for _ in range(3):                                  # the binding allocates on `side`
        z = torch.full((1, 8, 3072), float("nan"), device="cuda")
        side.wait_stream(torch.cuda.current_stream())
        ko, vo, idx = K.kvsel_score_evict(q, k, v, lens, case.budget, case.lam, mode,
                                          scores_out=z, stream=side)
        outs.append((ko, vo, idx, z))
    side.synchronize()
    for ko, vo, idx, z in outs:
        assert np.array_equal(idx.cpu().numpy(), ref["idx"])
        assert np.array_equal(host_bits(ko), ref["k_out"])
        assert np.array_equal(z.cpu().numpy()[0, :, :3000], ref["Z2"][0, :, :3000])
