"""ReFreeKV threshold cut on the GPU against the oracle (through the C ABI).

* Stage entry (given fp32 attention rows): kept lengths bit-exact with the
  oracle's fixed-point walk, including hand-built rows with closed-form cuts.
* End to end (logits and softmax on the GPU in fp32, oracle in fp64): the GPU
  length must be a valid cut of the oracle's energies for a threshold within
  1e-5 of 1 - T; the exact-match rate is reported and must stay high.
* Closed forms on the GPU path: zero query (uniform attention), spikes;
  layers 0-1 keep everything.
"""

import math

import numpy as np
import pytest
import torch

from decode_eviction_amd import kvsel as K
from decode_eviction_amd import synth
from oracle import refreekv as rf
from tests.gpu_util import dev, dev_i32, host_bits, log

pytestmark = pytest.mark.gpu

DELTA = 1e-5


def _softmax32(logits):
    x = logits - logits.max(axis=-1, keepdims=True)
    e = np.exp(x)
    return (e / e.sum(axis=-1, keepdims=True)).astype(np.float32)


def test_from_attn_bit_exact():
    rng = np.random.default_rng(11)
    b, hq, hkv, cap = 5, 12, 3, 3000
    lens = np.array([3000, 1, 4, 777, 2048], np.int32)
    attn = np.zeros((b, hq, cap), np.float32)
    for bi in range(b):
        n = int(lens[bi])
        lg = rng.standard_normal((hq, n)) * rng.uniform(0.5, 4.0)
        lg[:, :4] += 3.0
        lg[:, max(0, n - 30):] += 2.0
        attn[bi, :, :n] = _softmax32(lg)
    attn[0, 0:4] = np.float32(1.0 / 3000)            # uniform rows for head 0 of sequence 0
    for T in (0.01, 0.001, 0.1):
        for m in (4, 0, 10):
            log(f"[cut-stage] T={T} m={m}")
            got = K.kvsel_threshold_cut_from_attn(dev(attn, "f32"), dev_i32(lens), hkv, m, T)
            want = rf.threshold_cut_from_attn(attn, lens, hkv, m, T)
            assert np.array_equal(got.cpu().numpy(), want), (T, m)


def test_from_attn_closed_forms():
    # uniform rows: L = max(4, ceil(0.99 n)); spike rows: L = m + t
    n_list = [1234, 101, 3, 4999]
    cap = max(n_list)
    attn = np.zeros((len(n_list), 2, cap), np.float32)
    for i, n in enumerate(n_list):
        attn[i, :, :n] = np.float32(1.0 / n)
    got = K.kvsel_threshold_cut_from_attn(dev(attn, "f32"), dev_i32(n_list), 1).cpu().numpy()
    assert got[:, 0].tolist() == [1222, 100, 3, 4950]
    spike = np.zeros((1, 1, 4096), np.float32)
    spike[0, 0, :4] = spike[0, 0, -10:] = np.float32(1.0 / 14)
    got = K.kvsel_threshold_cut_from_attn(dev(spike, "f32"), dev_i32([4096]), 1).cpu().numpy()
    assert got.tolist() == [[14]]


def _valid_cut(e, L, m, T, delta=DELTA):
    n = len(e)
    if n == 0:
        return L == 0
    c = np.cumsum(e[rf.rank_order(n, m)])
    tot = c[-1]
    if L < min(m, n) or L > n:
        return False
    ok_hi = c[L - 1] >= (1 - T - delta) * tot
    ok_lo = L <= min(m, n) or c[L - 2] < (1 - T + delta) * tot
    return bool(ok_hi and ok_lo)


@pytest.mark.parametrize("layer", [2, 13, 27])
def test_cut_end_to_end_qwen_shape(layer):
    case = synth.cut_case(layer)
    log(f"[cut] layer={layer} lengths={case.lengths.tolist()}")
    got = K.kvsel_threshold_cut(dev(case.q, "bf16"), dev(case.k, "bf16"), dev_i32(case.lengths),
                                layer).cpu().numpy()
    L_ref, es = rf.threshold_cut(case.as_f32("q"), case.as_f32("k"), case.lengths, layer)
    exact = 0
    for (bi, h), e in es.items():
        assert _valid_cut(e, int(got[bi, h]), 4, 0.01), (bi, h, int(got[bi, h]), int(L_ref[bi, h]))
        exact += int(got[bi, h] == L_ref[bi, h])
    rate = exact / len(es)
    ratio = got.sum() / case.lengths.repeat(case.hkv).sum()
    log(f"    exact-match rate {rate:.3f}; kept fraction {ratio:.3f}")
    assert rate >= 0.9


def test_first_two_layers_keep_all():
    case = synth.cut_case(0, b=3, lengths=[100, 2000, 5])
    for layer in (0, 1):
        got = K.kvsel_threshold_cut(dev(case.q, "bf16"), dev(case.k, "bf16"),
                                    dev_i32(case.lengths), layer).cpu().numpy()
        assert got.tolist() == [[100] * 4, [2000] * 4, [5] * 4]


def test_zero_query_uniform_closed_form():
    lengths = [1234, 101, 3, 4999, 16384]
    case = synth.cut_case(4, b=5, lengths=lengths, zero_query=True)
    got = K.kvsel_threshold_cut(dev(case.q, "bf16"), dev(case.k, "bf16"), dev_i32(case.lengths),
                                4).cpu().numpy()
    want = [max(4, math.ceil(0.99 * n)) if n > 4 else n for n in lengths]
    assert got[:, 0].tolist() == want
    assert (got == got[:, :1]).all()


def test_spike_keys_closed_form():
    d, n, t = 128, 3000, 10
    k = np.zeros((1, 1, n, d), np.float32)
    spikes = list(range(4)) + list(range(n - t, n))
    k[0, 0, spikes, 0] = 30.0 * math.sqrt(d) / 4.0        # logit 30 with q = 4*e0
    q = np.zeros((1, 1, d), np.float32)
    q[0, 0, 0] = 4.0
    for dtype in ("bf16", "f32"):
        qd = dev(synth.f32_to_bf16_bits(q), "bf16") if dtype == "bf16" else dev(q, "f32")
        kd = dev(synth.f32_to_bf16_bits(k), "bf16") if dtype == "bf16" else dev(k, "f32")
        got = K.kvsel_threshold_cut(qd, kd, dev_i32([n]), 3).cpu().numpy()
        assert got.tolist() == [[4 + t]], dtype


def test_cut_deterministic():
    case = synth.cut_case(5, b=4)
    args = (dev(case.q, "bf16"), dev(case.k, "bf16"), dev_i32(case.lengths), 5)
    a = K.kvsel_threshold_cut(*args).cpu().numpy()
    b = K.kvsel_threshold_cut(*args).cpu().numpy()
    assert np.array_equal(a, b)


# --------------------------------------------- last k rows and the compaction

def _dev_rows(case, k_rows):
    return dev(synth.cut_rows_q(case, k_rows), case.dtype)


def test_cut_rows_k1_is_the_last_row_cut():
    case = synth.cut_case(9, b=6)
    qd, kd, ld = dev(case.q, "bf16"), dev(case.k, "bf16"), dev_i32(case.lengths)
    a = K.kvsel_threshold_cut(qd, kd, ld, 9).cpu().numpy()
    b = K.kvsel_threshold_cut_rows(qd[:, :, None].contiguous(), kd, ld, 9).cpu().numpy()
    assert np.array_equal(a, b)


@pytest.mark.parametrize("k_rows", [3, 18, 40])
def test_cut_rows_end_to_end(k_rows):
    # g*k = 21, 126 (one group of rows) and 280 (three groups)
    case = synth.cut_case(11, b=4, lengths=[3000, 777, 9000, 129])
    log(f"[cut rows] k={k_rows} lengths={case.lengths.tolist()}")
    qr = synth.cut_rows_q(case, k_rows)
    got = K.kvsel_threshold_cut_rows(dev(qr, "bf16"), dev(case.k, "bf16"), dev_i32(case.lengths),
                                     11).cpu().numpy()
    L_ref, es = rf.threshold_cut_rows(synth.bf16_bits_to_f32(qr), case.as_f32("k"), case.lengths, 11)
    exact = 0
    for (bi, h), e in es.items():
        assert _valid_cut(e, int(got[bi, h]), 4, 0.01), (bi, h, int(got[bi, h]), int(L_ref[bi, h]))
        exact += int(got[bi, h] == L_ref[bi, h])
    log(f"    exact-match rate {exact / len(es):.3f}")
    assert exact / len(es) >= 0.75


def test_cut_rows_zero_query_and_short_sequences():
    # zero queries: each row is uniform over the keys it sees; sequences shorter
    # than k have rows that see nothing
    lengths = [2000, 5, 1, 37]
    case = synth.cut_case(6, b=4, lengths=lengths, zero_query=True)
    k_rows = 12
    qr = synth.cut_rows_q(case, k_rows)
    got = K.kvsel_threshold_cut_rows(dev(qr, "bf16"), dev(case.k, "bf16"), dev_i32(lengths),
                                     6).cpu().numpy()
    L_ref, es = rf.threshold_cut_rows(synth.bf16_bits_to_f32(qr), case.as_f32("k"), lengths, 6)
    for (bi, h), e in es.items():
        assert _valid_cut(e, int(got[bi, h]), 4, 0.01), (bi, h, int(got[bi, h]), int(L_ref[bi, h]))
    assert got[1].tolist() == [5] * 4 and got[2].tolist() == [1] * 4


def test_cut_compact_fused_and_stage():
    case = synth.cut_case(7, b=3, lengths=[3000, 4, 1500], dtype="bf16")
    rng = np.random.default_rng(3)
    v = rng.integers(0, 65536, size=case.k.shape, dtype=np.uint16)
    qd, kd, vd, ld = _dev_rows(case, 2), dev(case.k, "bf16"), dev(v, "bf16"), dev_i32(case.lengths)
    ko = torch.zeros_like(kd)
    vo = torch.zeros_like(vd)
    kept = K.kvsel_threshold_cut_rows(qd, kd, ld, 7, v=vd, k_out=ko, v_out=vo).cpu().numpy()
    ko, vo = host_bits(ko), host_bits(vo)
    for bi in range(3):
        n = int(case.lengths[bi])
        for h in range(case.hkv):
            L = int(kept[bi, h])
            rows = rf.kept_positions(n, L, 4)
            assert len(rows) == L
            assert np.array_equal(ko[bi, h, :L], case.k[bi, h, rows]), (bi, h)
            assert np.array_equal(vo[bi, h, :L], v[bi, h, rows]), (bi, h)
            assert (ko[bi, h, L:] == 0).all()
    # the stage entry from given lengths, fp32 and d = 64, into a larger cache
    kf = rng.standard_normal((2, 3, 100, 64)).astype(np.float32)
    vf = rng.standard_normal((2, 3, 100, 64)).astype(np.float32)
    lens = np.array([100, 10], np.int32)
    kl = np.array([[100, 4, 57], [10, 3, 0]], np.int32)
    ko2, vo2 = K.kvsel_cut_compact(dev(kf, "f32"), dev(vf, "f32"), dev_i32(lens), dev_i32(kl),
                                   n_sink=4, k_out=torch.zeros((2, 3, 128, 64), device="cuda"),
                                   v_out=torch.zeros((2, 3, 128, 64), device="cuda"))
    ko2, vo2 = ko2.cpu().numpy(), vo2.cpu().numpy()
    for bi in range(2):
        for h in range(3):
            L = int(kl[bi, h])
            rows = rf.kept_positions(int(lens[bi]), L, 4)
            assert np.array_equal(ko2[bi, h, :L], kf[bi, h, rows])
            assert np.array_equal(vo2[bi, h, :L], vf[bi, h, rows])
            assert (ko2[bi, h, L:] == 0).all()


def test_cut_rows_fp32_d64_two_groups():
    # fp32 inputs, d = 64, 7 * 20 = 140 rows per KV head: two row groups
    case = synth.cut_case(12, b=3, d=64, lengths=[2500, 300, 1024], dtype="f32")
    qr = synth.cut_rows_q(case, 20)
    got = K.kvsel_threshold_cut_rows(dev(qr, "f32"), dev(case.k, "f32"), dev_i32(case.lengths),
                                     12).cpu().numpy()
    L_ref, es = rf.threshold_cut_rows(qr, case.as_f32("k"), case.lengths, 12)
    for (bi, h), e in es.items():
        assert _valid_cut(e, int(got[bi, h]), 4, 0.01), (bi, h, int(got[bi, h]), int(L_ref[bi, h]))
