"""The one-launch score pass for longer caches: more than 16 chunks of 256
tokens per head, bf16 keys of 128 dimensions, at most 32 window rows per KV
head, taken when the whole grid is resident at once (four work-groups per
compute unit, 1024 on the device).  It computes the key-sum scores, or the
Gram form's importance and key weights before the Gram kernels.

The score pass computes each chunk's partials as k_stats does, merges them in
k_reduce's order and pools as k_pool does, so I, R and Z must equal the
multi-kernel pass's bit for bit, and so must the indices and compacted K
and V rows that the selection kernels then derive from those scores.  The
reference call runs the separate kernels (KVSEL_SEPARATE_KERNELS=1).  Each
case reads from the traced entry point which path ran (a silent fallback
would make the comparison vacuous), checks that no wait timed out (bit 2 of
the error word) and compares sampled heads with the oracle within the score
tolerance (Gram form: heads of at most 4096 tokens, where the oracle's
similarity matrix stays small).  Repeated calls on one workspace filled with
junk exercise the per-head epochs.  Cases, in both forms: the n = 32768
layer, a ragged batch, sequences of fewer than five chunks (one work-group
merges several slices), empty and
one-token sequences, n <= B, a length above cap, 16 window rows per KV head,
per-head budgets (0, 1, out of range), all-equal keys (the threshold bin
holds every key and is read from memory) and three-valued ties; in the
key-sum form a cache of 256 chunks (the merges loop over blocks of 128
chunks; selection through the large-cache kernels)."""

import ctypes
import os

import numpy as np
import pytest
import torch

import bench
from decode_eviction_amd import kvsel as K
from decode_eviction_amd import synth
from oracle import rkv
from tests.gpu_util import SCORE_RTOL, SWAP_WINDOW, dev, dev_i32, host_bits, log, score_err, swaps

pytestmark = pytest.mark.gpu

FORMS = ["keysum", "gram"]

MAX_KERNELS = 8


class _Hip:
    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]


def launched_kernels(q, k, v, lens, budget, lam, form):
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
        K.KVSEL_BF16, K.MODES[form], P(q.data_ptr()), P(k.data_ptr()), P(v.data_ptr()),
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


def _scores(q, k, lens, lam, form, ws=None):
    b, hkv, cap = k.shape[0], k.shape[1], k.shape[2]
    i = torch.full((b, hkv, cap), float("nan"), device="cuda")
    r = torch.full_like(i, float("nan"))
    z = torch.full_like(i, float("nan"))
    K.kvsel_scores(q, k, lens, lam, form, i_out=i, r_out=r, z_out=z, workspace=ws)
    return i, r, z


class _separate:
    """Calls inside run the separate kernels (KVSEL_SEPARATE_KERNELS=1)."""

    def __enter__(self):
        os.environ["KVSEL_SEPARATE_KERNELS"] = "1"

    def __exit__(self, *a):
        os.environ.pop("KVSEL_SEPARATE_KERNELS", None)


def _host(t):
    """Device tensor -> numpy (bf16 as its raw 16-bit words)."""
    return host_bits(t) if t.dtype == torch.bfloat16 else t.cpu().numpy()


def _evict(q, k, v, lens, budget, lam, form, budgets=None, ws=None):
    b, hkv, cap = k.shape[0], k.shape[1], k.shape[2]
    z = torch.full((b, hkv, cap), float("nan"), device="cuda")
    ko = torch.zeros((b, hkv, budget, k.shape[3]), dtype=k.dtype, device="cuda")
    vo = torch.zeros_like(ko)
    if budgets is None:
        _, _, idx = K.kvsel_score_evict(q, k, v, lens, budget, lam, form, k_out=ko, v_out=vo,
                                        scores_out=z, workspace=ws)
    else:
        _, _, idx = K.kvsel_score_evict_heads(q, k, v, lens, dev_i32(budgets), budget, lam, form,
                                              k_out=ko, v_out=vo, scores_out=z, workspace=ws)
    return z, idx, ko, vo


ORACLE_GRAM_MAX_N = 4096


def _check(case, form="keysum", oracle_heads=2, calls=3, lengths=None, budget=None, budgets=None,
           heads=None):
    lengths = case.lengths if lengths is None else np.asarray(lengths, np.int32)
    budget = case.budget if budget is None else budget
    log(f"[scores_fused] {form} {case.name} b={case.b} hq={case.hq} hkv={case.hkv} cap={case.cap} "
        f"lengths={lengths.tolist()} B={budget} budgets={budgets}")
    q, k, v = dev(case.q, "bf16"), dev(case.k, "bf16"), dev(case.v, "bf16")
    lens = dev_i32(lengths)
    # the score pass, then the Gram kernels (Gram form) and the selection
    fused = bench.rkv_kernels(form, case.cap, case.b, case.hkv, budget)
    assert fused[0] == "scores", fused
    assert launched_kernels(q, k, v, lens, budget, case.lam, form) == len(fused), \
        "the one-launch score pass did not run"
    with _separate():
        assert launched_kernels(q, k, v, lens, budget, case.lam, form) == \
            len(bench.unfused_kernels(form, case.cap)), "the reference ran a fused path"
        ref = [x.cpu().numpy() for x in _scores(q, k, lens, case.lam, form)]
        ref_ev = [_host(x) for x in _evict(q, k, v, lens, budget, case.lam, form, budgets)]

    n_eff = np.clip(lengths, 0, case.cap)
    bad_len = ((lengths < 0) | (lengths > case.cap)).any()
    bad_budget = budgets is not None and any(x < 0 or x > budget for x in budgets)
    wsb = K.kvsel_score_evict_workspace(case.b, case.hq, case.hkv, case.d, case.w, case.cap, budget)
    wss = {e: torch.full((wsb,), 0x5a, dtype=torch.uint8, device="cuda") for e in ("scores", "evict")}
    for call in range(calls):
        for entry in ("scores", "evict"):
            ws = wss[entry]
            if entry == "scores":
                got = [x.cpu().numpy() for x in _scores(q, k, lens, case.lam, form, ws)]
                want_err = 1 if bad_len else 0
            else:
                got = [_host(x) for x in _evict(q, k, v, lens, budget, case.lam, form, budgets, ws)]
                want_err = (1 if bad_len else 0) | (2 if bad_budget else 0)
            flags = K.kvsel_workspace_error(ws)
            assert flags & 4 == 0, f"a wait timed out (call {call}, {entry})"
            assert flags == want_err, (entry, flags)
            for bi in range(case.b):
                n = int(n_eff[bi])
                for h in range(case.hkv):
                    if entry == "scores":
                        for name, g, rf in zip("IRZ", got, ref):
                            assert np.array_equal(g[bi, h, :n].view(np.uint32), rf[bi, h, :n].view(np.uint32)), \
                                (call, name, bi, h)
                            assert np.isnan(g[bi, h, n:]).all(), (call, name, bi, h, "written past n")
                    else:
                        z, idx, ko, vo = got
                        assert np.array_equal(z[bi, h, :n].view(np.uint32), ref_ev[0][bi, h, :n].view(np.uint32)), \
                            (call, "Z", bi, h)
                        assert np.array_equal(idx[bi, h], ref_ev[1][bi, h]), (call, "idx", bi, h)
                        assert np.array_equal(ko[bi, h], ref_ev[2][bi, h]), (call, "k_out", bi, h)
                        assert np.array_equal(vo[bi, h], ref_ev[3][bi, h]), (call, "v_out", bi, h)
    # sampled heads against the oracle
    if heads is None:
        heads = [(bi, h) for bi in range(case.b) for h in range(case.hkv) if n_eff[bi] > 0][:oracle_heads]
    if form == "gram":
        heads = [(bi, h) for bi, h in heads if n_eff[bi] <= ORACLE_GRAM_MAX_N]
    if heads:
        orc = rkv.score_evict(case.as_f32("q"), case.as_f32("k"), case.as_f32("v"), n_eff, case.lam, budget,
                              form=form, heads=heads, budgets=budgets)
        z, idx = got[0], got[1]
        for bi, h in heads:
            err = score_err(z[bi, h, :n_eff[bi]], orc["Z"][bi][h])
            assert err <= SCORE_RTOL, ("Z", bi, h, err)
            ns, gap = swaps(idx[bi, h], orc["idx"][bi, h], orc["Z"][bi][h])
            assert gap < SWAP_WINDOW, (bi, h, ns, gap)


@pytest.mark.parametrize("form", FORMS)
def test_scores_fused_headline(form):
    _check(synth.headline_case(layer=0), form)


@pytest.mark.parametrize("form", FORMS)
def test_scores_fused_ragged(form):
    case = synth.rkv_case("ragged", seed=3, wl=synth.WL_LAYER8B, b=2, hq=32, hkv=8, d=128, w=8,
                          lengths=[12345, 3001], cap=16384, budget=1024)
    _check(case, form, heads=[(1, 0), (1, 6)] if form == "gram" else None)


def test_scores_fused_256_chunks():
    case = synth.rkv_case("long", seed=4, wl=synth.WL_LAYER8B, b=1, hq=8, hkv=2, d=128, w=8,
                          lengths=[65536 - 77], cap=65536, budget=2048)
    _check(case)


@pytest.mark.parametrize("form", FORMS)
def test_scores_fused_few_chunks_and_empty(form):
    # sequence 0 keeps everything (700 <= B), 1 is empty, 2 holds one token
    case = synth.rkv_case("short", seed=5, wl=synth.WL_LAYER8B, b=3, hq=32, hkv=8, d=128, w=8,
                          lengths=[700, 0, 1], cap=8192, budget=1024)
    _check(case, form, heads=[(0, 0), (0, 5), (2, 0), (2, 7)])
    case = synth.rkv_case("short2", seed=12, wl=synth.WL_LAYER8B, b=3, hq=32, hkv=8, d=128, w=8,
                          lengths=[1300, 0, 1], cap=8192, budget=256)
    _check(case, form)


@pytest.mark.parametrize("form", FORMS)
def test_scores_fused_length_above_cap(form):
    case = synth.rkv_case("over", seed=6, wl=synth.WL_LAYER8B, b=1, hq=32, hkv=8, d=128, w=8,
                          lengths=[8192], cap=8192, budget=1024)
    _check(case, form, lengths=[9000])


@pytest.mark.parametrize("form", FORMS)
def test_scores_fused_16_rows(form):
    case = synth.rkv_case("rows16", seed=7, wl=synth.WL_LAYER8B, b=1, hq=16, hkv=8, d=128, w=8,
                          lengths=[20000], cap=20480, budget=1024)
    _check(case, form)


@pytest.mark.parametrize("form", FORMS)
def test_scores_fused_head_budgets(form):
    case = synth.rkv_case("budgets", seed=8, wl=synth.WL_LAYER8B, b=2, hq=32, hkv=8, d=128, w=8,
                          lengths=[16000, 9000], cap=16384, budget=2048)
    _check(case, form, budgets=[0, 1, 2048, 3000, -4, 777, 2047, 1024], calls=2,
           heads=[(0, 1), (0, 5), (1, 7)])


def _tied(case, values):
    """Keys that take only the given rows (all positions share a few keys),
    so that Z takes a few values with thousands of copies each."""
    k = case.k.copy()
    rng = np.random.default_rng(11)
    rows = synth.f32_to_bf16_bits(rng.standard_normal((values, case.d), dtype=np.float32))
    pick = rng.integers(0, values, size=case.cap)
    k[:, :] = rows[pick][None, None]
    case.k = k
    return case


@pytest.mark.parametrize("form", FORMS)
def test_scores_fused_all_equal(form):
    case = _tied(synth.rkv_case("equal", seed=9, wl=synth.WL_LAYER8B, b=1, hq=32, hkv=8, d=128, w=8,
                                lengths=[30000], cap=32768, budget=2048), 1)
    _check(case, form, calls=2, heads=[(0, 0)])


@pytest.mark.parametrize("form", FORMS)
def test_scores_fused_three_values(form):
    case = _tied(synth.rkv_case("three", seed=10, wl=synth.WL_LAYER8B, b=1, hq=32, hkv=8, d=128, w=8,
                                lengths=[32768], cap=32768, budget=2048), 3)
    _check(case, form, calls=2, heads=[(0, 3)])



def _check_select(case, form, budgets=None, calls=2):
    """The one-launch selection where chunks keep most of their rows (several
    work-groups share a chunk's gather) against the two-kernel selection:
    indices, compacted K and V rows and Z bit for bit, over repeated calls on
    one workspace filled with junk; sampled heads against the oracle."""
    budget = case.budget
    log(f"[select_compact split] {form} {case.name} b={case.b} cap={case.cap} "
        f"lengths={case.lengths.tolist()} B={budget} budgets={budgets}")
    q, k, v = dev(case.q, "bf16"), dev(case.k, "bf16"), dev(case.v, "bf16")
    lens = dev_i32(case.lengths)
    names = bench.rkv_kernels(form, case.cap, case.b, case.hkv, budget)
    assert names[-1] == "select_compact", names
    assert launched_kernels(q, k, v, lens, budget, case.lam, form) == len(names), \
        "the one-launch selection did not run"
    with _separate():
        assert launched_kernels(q, k, v, lens, budget, case.lam, form) == \
            len(bench.unfused_kernels(form, case.cap))
        ref = [_host(x) for x in _evict(q, k, v, lens, budget, case.lam, form, budgets)]
    n_eff = np.clip(case.lengths, 0, case.cap)
    bad_budget = budgets is not None and any(x < 0 or x > budget for x in budgets)
    wsb = K.kvsel_score_evict_workspace(case.b, case.hq, case.hkv, case.d, case.w, case.cap, budget)
    ws = torch.full((wsb,), 0x5a, dtype=torch.uint8, device="cuda")
    for call in range(calls):
        got = [_host(x) for x in _evict(q, k, v, lens, budget, case.lam, form, budgets, ws)]
        flags = K.kvsel_workspace_error(ws)
        assert flags == (2 if bad_budget else 0), (call, flags)
        for bi in range(case.b):
            n = int(n_eff[bi])
            for h in range(case.hkv):
                assert np.array_equal(got[0][bi, h, :n].view(np.uint32), ref[0][bi, h, :n].view(np.uint32)), \
                    (call, "Z", bi, h)
                for name, g, r in zip(("idx", "k_out", "v_out"), got[1:], ref[1:]):
                    assert np.array_equal(g[bi, h], r[bi, h]), (call, name, bi, h)
    heads = [(bi, 0) for bi in range(case.b) if 0 < n_eff[bi] <= ORACLE_GRAM_MAX_N][:2]
    if heads:
        orc = rkv.score_evict(case.as_f32("q"), case.as_f32("k"), case.as_f32("v"), n_eff, case.lam, budget,
                              form=form, heads=heads, budgets=budgets)
        for bi, h in heads:
            err = score_err(got[0][bi, h, :n_eff[bi]], orc["Z"][bi][h])
            assert err <= SCORE_RTOL, ("Z", bi, h, err)
            ns, gap = swaps(got[1][bi, h], orc["idx"][bi, h], orc["Z"][bi][h])
            assert gap < SWAP_WINDOW, (bi, h, ns, gap)


@pytest.mark.parametrize("form", FORMS)
def test_select_compact_split_gather(form):
    # the decode loop's cache (about 480 of 512 rows kept per chunk: eight
    # gathering work-groups per chunk); four sequences, so that the key-sum
    # form's fused step does not take the call
    case = synth.rkv_case("decode4", seed=15, wl=synth.WL_LAYER8B, b=4, hq=32, hkv=8, d=128, w=8,
                          lengths=[2176, 2100, 1500, 1], cap=2176, budget=2048)
    _check_select(case, form)
    # half of a 4096-token cache kept (four per chunk), with per-head budgets
    case = synth.rkv_case("half", seed=16, wl=synth.WL_LAYER8B, b=3, hq=32, hkv=8, d=128, w=8,
                          lengths=[4096, 3001, 4000], cap=4096, budget=2048)
    _check_select(case, form)
    _check_select(case, form, budgets=[0, 1, 2048, 3000, -4, 777, 2047, 1024])


def test_select_compact_split_gather_ties():
    # all keys equal: every score ties, the kept copies are the lowest
    # positions
    case = _tied(synth.rkv_case("decode_tied", seed=18, wl=synth.WL_LAYER8B, b=4, hq=32, hkv=8, d=128,
                                w=8, lengths=[2176, 2176, 2000, 2176], cap=2176, budget=2048), 1)
    _check_select(case, "gram")
    case = _tied(synth.rkv_case("decode_three", seed=19, wl=synth.WL_LAYER8B, b=4, hq=32, hkv=8, d=128,
                                w=8, lengths=[2176, 1900, 2176, 2176], cap=2176, budget=2048), 3)
    _check_select(case, "gram")
