"""The one-launch key-sum score pass for long caches: more than 16 chunks of
256 tokens per head, bf16 keys of 128 dimensions, at most 32 window rows per
KV head, taken when the whole grid is resident at once (four work-groups per
compute unit, 1024 on the device).

It computes each chunk's partials as k_stats does, merges them in k_reduce's
order and pools as k_pool does, so I, R and Z must equal the multi-kernel
pass's bit for bit.  The reference call repeats the same sequences along the
batch until the grid no longer fits: the library then runs the separate
passes, whose per-sequence arithmetic does not depend on the batch.  Each
case reads from the traced entry point which path ran (a silent fallback
would make the comparison vacuous), checks that no wait timed out (bit 2 of
the error word) and compares sampled heads with the oracle within the score
tolerance.  Repeated calls on one workspace filled with junk exercise the
per-head epochs.  Cases: the n = 32768 layer, a ragged batch, a cache of 256
chunks (the merges loop over blocks of 128 chunks), sequences of fewer than
five chunks (one work-group merges several slices), empty and one-token
sequences, a length above cap and 16 window rows per KV head."""

import ctypes

import numpy as np
import pytest
import torch

from decode_eviction_amd import kvsel as K
from decode_eviction_amd import synth
from oracle import rkv
from tests.gpu_util import SCORE_RTOL, dev, dev_i32, host_bits, log, score_err

pytestmark = pytest.mark.gpu

MAX_KERNELS = 8


class _Hip:
    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]


def launched_kernels(q, k, v, lens, budget, lam):
    """Kernels one kvsel_score_evict call launches: the traced entry point
    records a start/stop event pair per kernel; pairs never recorded have no
    elapsed time."""
    hip = _Hip()
    evs = (ctypes.c_void_p * (2 * MAX_KERNELS))()
    for i in range(2 * MAX_KERNELS):
        h = ctypes.c_void_p()
        assert hip.lib.hipEventCreate(ctypes.byref(h)) == 0
        evs[i] = h
    b, hq, w, d = q.shape
    hkv, cap = k.shape[1], k.shape[2]
    ko = torch.empty((b, hkv, budget, d), dtype=k.dtype, device="cuda")
    vo = torch.empty_like(ko)
    idx = torch.empty((b, hkv, budget), dtype=torch.int32, device="cuda")
    wsb = K.kvsel_score_evict_workspace(b, hq, hkv, d, w, cap, budget)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    P = ctypes.c_void_p
    torch.cuda.synchronize()
    st = K.lib().kvsel_score_evict_traced(
        K.KVSEL_BF16, K.MODES["keysum"], P(q.data_ptr()), P(k.data_ptr()), P(v.data_ptr()),
        P(lens.data_ptr()), b, hq, hkv, d, w, cap, lam, budget, P(ko.data_ptr()), P(vo.data_ptr()),
        budget, P(idx.data_ptr()), None, P(ws.data_ptr()), wsb,
        P(torch.cuda.current_stream().cuda_stream), evs, 2 * MAX_KERNELS)
    assert st == 0, K.status_string(st)
    torch.cuda.synchronize()
    n = 0
    ms = ctypes.c_float()
    while n < MAX_KERNELS and hip.lib.hipEventElapsedTime(ctypes.byref(ms), evs[2 * n], evs[2 * n + 1]) == 0:
        n += 1
    hip.lib.hipGetLastError()  # the failed query of an unrecorded pair is not left behind
    for h in evs:
        hip.lib.hipEventDestroy(h)
    return n


def _scores(q, k, lens, lam, ws=None):
    b, hkv, cap = k.shape[0], k.shape[1], k.shape[2]
    i = torch.full((b, hkv, cap), float("nan"), device="cuda")
    r = torch.full_like(i, float("nan"))
    z = torch.full_like(i, float("nan"))
    K.kvsel_scores(q, k, lens, lam, "keysum", i_out=i, r_out=r, z_out=z, workspace=ws)
    return i, r, z


def _reps_unfused(b, hkv, cap):
    """Copies of the batch whose grid exceeds the capacity of every device
    this library targets (256 compute units, at most 8 work-groups each)."""
    per = -(-cap // 256) * hkv * b
    return -(-2049 // per) + 1


def _check(case, oracle_heads=2, calls=3, lengths=None):
    lengths = case.lengths if lengths is None else np.asarray(lengths, np.int32)
    log(f"[scores_fused] {case.name} b={case.b} hq={case.hq} hkv={case.hkv} cap={case.cap} "
        f"lengths={lengths.tolist()}")
    q, k, v = dev(case.q, "bf16"), dev(case.k, "bf16"), dev(case.v, "bf16")
    lens = dev_i32(lengths)
    B = 64
    assert launched_kernels(q, k, v, lens, B, case.lam) == 3, "the one-launch score pass did not run"
    reps = _reps_unfused(case.b, case.hkv, case.cap)
    qr, kr, vr = (torch.cat([t] * reps, 0).contiguous() for t in (q, k, v))
    lr = dev_i32(np.tile(lengths, reps))
    assert launched_kernels(qr, kr, vr, lr, B, case.lam) == 5, "the reference ran a fused path"
    ref = [x.cpu().numpy()[:case.b] for x in _scores(qr, kr, lr, case.lam)]

    ws = torch.empty(K.kvsel_score_evict_workspace(case.b, case.hq, case.hkv, case.d, case.w,
                                                   case.cap, 1), dtype=torch.uint8, device="cuda")
    ws.fill_(0x5a)
    n_eff = np.clip(lengths, 0, case.cap)
    want_err = 1 if ((lengths < 0) | (lengths > case.cap)).any() else 0
    for call in range(calls):
        got = [x.cpu().numpy() for x in _scores(q, k, lens, case.lam, ws)]
        flags = K.kvsel_workspace_error(ws)
        assert flags & 4 == 0, f"a wait timed out (call {call})"
        assert flags == want_err, flags
        for bi in range(case.b):
            n = int(n_eff[bi])
            for h in range(case.hkv):
                for name, g, rf in zip("IRZ", got, ref):
                    assert np.array_equal(g[bi, h, :n].view(np.uint32), rf[bi, h, :n].view(np.uint32)), \
                        (call, name, bi, h)
                    assert np.isnan(g[bi, h, n:]).all(), (call, name, bi, h, "written past n")
    # sampled heads against the oracle
    heads = [(bi, h) for bi in range(case.b) for h in range(case.hkv) if n_eff[bi] > 0][:oracle_heads]
    if heads:
        orc = rkv.score_evict(case.as_f32("q"), case.as_f32("k"), case.as_f32("v"), n_eff, case.lam, B,
                              form="keysum", heads=heads)
        for bi, h in heads:
            for name, g in zip("IRZ", got):
                err = score_err(g[bi, h, :n_eff[bi]], orc[name][bi][h])
                assert err <= SCORE_RTOL, (name, bi, h, err)


def test_scores_fused_headline():
    _check(synth.headline_case(layer=0))


def test_scores_fused_ragged():
    case = synth.rkv_case("ragged", seed=3, wl=synth.WL_LAYER8B, b=2, hq=32, hkv=8, d=128, w=8,
                          lengths=[12345, 3001], cap=16384, budget=1024)
    _check(case)


def test_scores_fused_256_chunks():
    case = synth.rkv_case("long", seed=4, wl=synth.WL_LAYER8B, b=1, hq=8, hkv=2, d=128, w=8,
                          lengths=[65536 - 77], cap=65536, budget=2048)
    _check(case)


def test_scores_fused_few_chunks_and_empty():
    case = synth.rkv_case("short", seed=5, wl=synth.WL_LAYER8B, b=3, hq=32, hkv=8, d=128, w=8,
                          lengths=[700, 0, 1], cap=8192, budget=1024)
    _check(case, oracle_heads=4)


def test_scores_fused_length_above_cap():
    case = synth.rkv_case("over", seed=6, wl=synth.WL_LAYER8B, b=1, hq=32, hkv=8, d=128, w=8,
                          lengths=[8192], cap=8192, budget=1024)
    _check(case, lengths=[9000])


def test_scores_fused_16_rows():
    case = synth.rkv_case("rows16", seed=7, wl=synth.WL_LAYER8B, b=1, hq=16, hkv=8, d=128, w=8,
                          lengths=[20000], cap=20480, budget=1024)
    _check(case)


def test_score_evict_headline_selection():
    """The whole call on the fused scores: the kept set equals the stage
    select's on the same Z, and the kept rows are bit copies."""
    case = synth.headline_case(layer=1)
    q, k, v = dev(case.q, "bf16"), dev(case.k, "bf16"), dev(case.v, "bf16")
    lens = dev_i32(case.lengths)
    z = torch.empty((1, case.hkv, case.cap), device="cuda")
    ko, vo, idx = K.kvsel_score_evict(q, k, v, lens, case.budget, case.lam, "keysum", scores_out=z)
    want = K.kvsel_select_topb(z, lens, case.budget).cpu().numpy()
    idx = idx.cpu().numpy()
    assert np.array_equal(idx, want)
    kb, vb = host_bits(ko), host_bits(vo)
    for h in range(case.hkv):
        m = int((idx[0, h] >= 0).sum())
        assert m == case.budget
        assert np.array_equal(kb[0, h, :m], case.k[0, h, idx[0, h, :m]])
        assert np.array_equal(vb[0, h, :m], case.v[0, h, idx[0, h, :m]])
