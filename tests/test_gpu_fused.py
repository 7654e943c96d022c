"""The one-launch R-KV step for short caches (key-sum form, bf16, d = 128,
at most 32 window rows per KV head, at most 16 chunks of 256 tokens).

Its scores must equal the multi-kernel path's bit for bit (kvsel_scores runs
the separate passes with the same arithmetic and merge order), its kept set
must be exactly the stage select's on those scores, the compacted rows bit
copies, and no barrier may time out (bit 2 of the error word).  Repeated
calls on one workspace exercise the barrier epochs; ragged lengths, lengths
ending inside a chunk, n <= B, B = 0 per head and a length above cap cover
the branches."""

import numpy as np
import pytest
import torch

from decode_eviction_amd import kvsel as K
from decode_eviction_amd import synth
from oracle import rkv
from tests.gpu_util import SCORE_RTOL, dev, dev_i32, host_bits, log, score_err

pytestmark = pytest.mark.gpu


def _run(case, budgets=None, reps=3):
    q, k, v = dev(case.q, "bf16"), dev(case.k, "bf16"), dev(case.v, "bf16")
    lens = dev_i32(case.lengths)
    b, hkv, cap, d = case.b, case.hkv, case.cap, case.d
    ws = torch.empty(K.kvsel_score_evict_workspace(b, case.hq, hkv, d, case.w, cap, case.budget),
                     dtype=torch.uint8, device="cuda")
    ws.fill_(0x5a)                                     # arbitrary contents before the first call
    _, _, z_ref = K.kvsel_scores(q, k, lens, case.lam, "keysum")
    outs = []
    for rep in range(reps):
        z = torch.full((b, hkv, cap), float("nan"), device="cuda")
        if budgets is None:
            ko, vo, idx = K.kvsel_score_evict(q, k, v, lens, case.budget, case.lam, "keysum",
                                              scores_out=z, workspace=ws)
        else:
            ko, vo, idx = K.kvsel_score_evict_heads(q, k, v, lens, dev_i32(budgets), case.budget,
                                                    case.lam, "keysum", scores_out=z, workspace=ws)
        flags = K.kvsel_workspace_error(ws)
        assert flags & 4 == 0, f"a barrier timed out (call {rep})"
        outs.append((z.cpu().numpy(), idx.cpu().numpy(), host_bits(ko), host_bits(vo), flags))
    return outs, z_ref.cpu().numpy()


def _check(case, budgets=None):
    log(f"[fused] {case.name} b={case.b} hkv={case.hkv} cap={case.cap} lengths={case.lengths.tolist()} "
        f"B={case.budget} budgets={None if budgets is None else list(budgets)}")
    outs, z_ref = _run(case, budgets)
    z, idx, ko, vo, flags = outs[0]
    for o in outs[1:]:
        for x, y in zip(o[:4], outs[0][:4]):
            assert np.array_equal(x, y, equal_nan=True)
    # the same selection as the stage entry on the same scores
    lens = np.minimum(case.lengths, case.cap)
    want = K.kvsel_select_topb_heads(dev(z_ref, "f32"), dev_i32(lens), dev_i32(budgets), case.budget) \
        if budgets is not None else K.kvsel_select_topb(dev(z_ref, "f32"), dev_i32(lens), case.budget)
    want = want.cpu().numpy()
    ref = rkv.score_evict(case.as_f32("q"), case.as_f32("k"), case.as_f32("v"), lens, case.lam,
                          case.budget, form="keysum", budgets=budgets)
    for b in range(case.b):
        n = int(lens[b])
        for h in range(case.hkv):
            assert np.array_equal(z[b, h, :n], z_ref[b, h, :n]), (b, h)
            assert score_err(z[b, h, :n], ref["Z"][b][h]) <= SCORE_RTOL
            assert np.array_equal(idx[b, h], want[b, h]), (b, h)
            m = int((idx[b, h] >= 0).sum())
            assert np.array_equal(ko[b, h, :m], case.k[b, h, idx[b, h, :m]])
            assert np.array_equal(vo[b, h, :m], case.v[b, h, idx[b, h, :m]])
    return flags


def test_fused_decode_shape():
    case = synth.layer8b_case(4, n=2176, budget=2048, cap=2176)
    assert _check(case) == 0


def test_fused_full_4096():
    assert _check(synth.layer8b_case(5, n=4096, budget=1024, cap=4096)) == 0


def test_fused_ragged_and_small():
    case = synth.rkv_case("fused_ragged", seed=51, wl=61, b=4, hq=8, hkv=2, d=128, w=4,
                          lengths=[1000, 37, 256, 257], cap=1024, budget=100)
    assert _check(case) == 0
    case = synth.rkv_case("fused_keepall", seed=52, wl=62, b=2, hq=8, hkv=2, d=128, w=4,
                          lengths=[90, 600], cap=640, budget=100)
    assert _check(case) == 0


def test_fused_per_head_budgets():
    case = synth.rkv_case("fused_heads", seed=53, wl=63, b=2, hq=32, hkv=8, d=128, w=4,
                          lengths=[3000, 1700], cap=3072, budget=1024)
    budgets = np.array([1024, 0, 700, 1800, 1, 1023, 5, 2000], np.int32)  # two clamped
    assert _check(case, budgets) == 2


def test_fused_length_above_cap_flagged():
    case = synth.rkv_case("fused_clamp", seed=54, wl=64, b=2, hq=8, hkv=2, d=128, w=4,
                          lengths=[512, 400], cap=512, budget=64)
    case.lengths[0] = 700
    assert _check(case) == 1


def test_fused_tied_scores_take_the_fallback():
    # identical keys: every score is equal, more than the sample select
    # ranks directly, so the histogram rounds decide (lowest positions kept);
    # three groups of exact duplicates: three score values, large tied groups
    case = synth.rkv_case("fused_ties", seed=55, wl=65, b=2, hq=32, hkv=8, d=128, w=8,
                          lengths=[2176, 1800], cap=2176, budget=1000, frac=0.0, sink_scale=None)
    case.k[0] = case.k[0, :, :1]                      # sequence 0: one key repeated
    for g, (a, b_) in enumerate([(0, 700), (700, 1500), (1500, 2176)]):
        case.k[1, :, a:b_] = case.k[1, :, a:a + 1]    # sequence 1: three repeated keys
    assert _check(case) == 0


@pytest.mark.parametrize("n", [2176, 32768])
def test_words_left_in_a_reused_workspace_never_pass(n):
    # A workspace whose memory held an earlier call's data: its per-head
    # epochs back at the values that call started from (zero here, as a
    # zero-filled buffer reused for it leaves them) while the tagged words
    # the call published are still there.  A later call on other keys must
    # not take those words for its own: its results equal those of a call on
    # a clean workspace.  n = 2176 runs the one-launch short-cache step,
    # n = 32768 the one-launch score pass and selection.  Layout used here:
    # the error words (256 bytes), then one 8-byte epoch per (sequence, head).
    first = synth.layer8b_case(5, n=n, budget=2048, cap=n)
    later = synth.layer8b_case(6, n=n, budget=2048, cap=n)
    log(f"[fused] reused workspace n={n}")
    nbytes = K.kvsel_score_evict_workspace(1, first.hq, first.hkv, 128, first.w, n, 2048)
    epochs_end = 256 + 8 * first.b * first.hkv

    def call(case, ws):
        q, k, v = dev(case.q, "bf16"), dev(case.k, "bf16"), dev(case.v, "bf16")
        z = torch.full((case.b, case.hkv, n), float("nan"), device="cuda")
        ko, vo, idx = K.kvsel_score_evict(q, k, v, dev_i32(case.lengths), 2048, case.lam, "keysum",
                                          scores_out=z, workspace=ws)
        flags = K.kvsel_workspace_error(ws)
        return z.cpu().numpy(), idx.cpu().numpy(), host_bits(ko), host_bits(vo), flags

    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    call(first, ws)
    ws[:epochs_end] = 0
    got = call(later, ws)
    want = call(later, torch.zeros(nbytes, dtype=torch.uint8, device="cuda"))
    assert got[4] & 4 == 0 and want[4] & 4 == 0
    for x, y in zip(got[:4], want[:4]):
        assert np.array_equal(x, y, equal_nan=True)


# ---- the slot-reuse form of the one-launch step (kvsel_score_evict_slots)

def _slots_check(case, pos=None, budgets=None, separate=False, monkeypatch=None):
    """The one-launch slot step against the multi-kernel scores and the
    stage selection on them (bit for bit), and the oracle's evicted list on
    the same scores."""
    q, k = dev(case.q, "bf16"), dev(case.k, "bf16")
    lens = dev_i32(case.lengths)
    b, hkv, cap = case.b, case.hkv, case.cap
    log(f"[fused slots] {case.name} b={b} hkv={hkv} cap={cap} lengths={case.lengths.tolist()} "
        f"B={case.budget} budgets={None if budgets is None else list(budgets)} pos={pos is not None}")
    ws = torch.empty(K.kvsel_score_evict_workspace(b, case.hq, hkv, case.d, case.w, cap, case.budget),
                     dtype=torch.uint8, device="cuda")
    ws.fill_(0x5a)
    pos_d = None if pos is None else dev_i32(pos)
    bud_d = None if budgets is None else dev_i32(budgets)
    runs = []
    for rep in range(2):
        z = torch.full((b, hkv, cap), float("nan"), device="cuda")
        ev, ne = K.kvsel_score_evict_slots(q, k, lens, case.budget, case.lam, "keysum", pos=pos_d,
                                           budgets=bud_d, scores_out=z, workspace=ws)
        flags = K.kvsel_workspace_error(ws)
        assert flags & 12 == 0, f"flags {flags}"
        runs.append((z.cpu().numpy(), ev.cpu().numpy(), ne.cpu().numpy(), flags))
    z, ev, ne, flags = runs[0]
    for x, y in zip(runs[1][:3], runs[0][:3]):
        assert np.array_equal(x, y, equal_nan=True)
    lens_c = np.minimum(case.lengths, cap)
    _, _, z_ref = K.kvsel_scores(q, k, lens, case.lam, "keysum")
    want_ev, want_ne = K.kvsel_select_evict_slots(z_ref, dev_i32(lens_c), case.budget, pos=pos_d,
                                                  budgets=bud_d)
    z_ref, want_ev, want_ne = z_ref.cpu().numpy(), want_ev.cpu().numpy(), want_ne.cpu().numpy()
    for bb in range(b):
        n = int(lens_c[bb])
        for h in range(hkv):
            assert np.array_equal(z[bb, h, :n], z_ref[bb, h, :n]), (bb, h)
            assert ne[bb, h] == want_ne[bb, h], (bb, h)
            assert np.array_equal(ev[bb, h], want_ev[bb, h]), (bb, h)
            bh = case.budget if budgets is None else rkv.head_budget(budgets, h, case.budget)
            want = rkv.evict_slots(z[bb, h, :n].astype(np.float64), bh,
                                   None if pos is None else pos[bb, h, :n])
            assert ev[bb, h, :len(want)].tolist() == want.tolist(), (bb, h)
            assert (ev[bb, h, len(want):] == -1).all()
    return flags


def test_fused_slots_decode_shape():
    case = synth.layer8b_case(7, n=2176, budget=2048, cap=2176)
    rng = np.random.default_rng(71)
    pos = np.stack([rng.permutation(40_000)[:2176] for _ in range(case.hkv)])[None].astype(np.int32)
    _slots_check(case, pos=pos)
    _slots_check(case)                                  # no position map: slot order


def test_fused_slots_ties_split_by_position():
    # three groups of exact duplicate keys per head: three score values,
    # the threshold inside a large tied group; positions a permutation (ties
    # go to the lower position) and then with duplicates (equal positions:
    # lower slot)
    case = synth.rkv_case("slots_ties", seed=72, wl=66, b=2, hq=32, hkv=8, d=128, w=8,
                          lengths=[2176, 1800], cap=2176, budget=1000, frac=0.0, sink_scale=None)
    for bb in range(2):
        for a, e in [(0, 700), (700, 1500), (1500, 2176)]:
            case.k[bb, :, a:e] = case.k[bb, :, a:a + 1]
    rng = np.random.default_rng(73)
    perm = np.stack([np.stack([rng.permutation(2176) for _ in range(8)]) for _ in range(2)])
    _slots_check(case, pos=perm.astype(np.int32))
    _slots_check(case, pos=(perm // 3).astype(np.int32))


def test_fused_slots_budgets_and_edges():
    # per-head budgets 0 (every slot evicted), 1, >= n (none evicted) and one
    # clamped; ragged lengths with one inside a chunk and one empty
    case = synth.rkv_case("slots_heads", seed=74, wl=67, b=3, hq=32, hkv=8, d=128, w=4,
                          lengths=[2000, 257, 0], cap=2048, budget=1500)
    budgets = np.array([0, 1, 300, 1500, 2047, 9000, 700, 256], np.int32)
    rng = np.random.default_rng(75)
    pos = np.stack([np.stack([rng.permutation(10_000)[:2048] for _ in range(8)])
                    for _ in range(3)]).astype(np.int32)
    flags = _slots_check(case, pos=pos, budgets=budgets)
    assert flags & 2                                   # 9000 > 1500 was clamped


# ---- the Gram form's finish inside the one-launch step (short caches)

def _gram_outputs(case, slots, pos=None, budgets=None):
    q, k, v = dev(case.q, "bf16"), dev(case.k, "bf16"), dev(case.v, "bf16")
    lens = dev_i32(case.lengths)
    b, hkv, cap = case.b, case.hkv, case.cap
    ws = torch.empty(K.kvsel_score_evict_workspace(b, case.hq, hkv, case.d, case.w, cap, case.budget),
                     dtype=torch.uint8, device="cuda")
    ws.fill_(0x5a)
    z = torch.full((b, hkv, cap), float("nan"), device="cuda")
    bud = None if budgets is None else dev_i32(budgets)
    if slots:
        ev, ne = K.kvsel_score_evict_slots(q, k, lens, case.budget, case.lam, "gram",
                                           pos=None if pos is None else dev_i32(pos), budgets=bud,
                                           scores_out=z, workspace=ws)
        outs = [ev.cpu().numpy(), ne.cpu().numpy()]
    elif budgets is None:
        ko, vo, idx = K.kvsel_score_evict(q, k, v, lens, case.budget, case.lam, "gram", scores_out=z,
                                          workspace=ws)
        outs = [idx.cpu().numpy(), host_bits(ko), host_bits(vo)]
    else:
        ko, vo, idx = K.kvsel_score_evict_heads(q, k, v, lens, bud, case.budget, case.lam, "gram",
                                                scores_out=z, workspace=ws)
        outs = [idx.cpu().numpy(), host_bits(ko), host_bits(vo)]
    flags = K.kvsel_workspace_error(ws)
    assert flags & 12 == 0, f"flags {flags}"
    zh = z.cpu().numpy()
    lens_c = np.minimum(case.lengths, cap)
    zs = [zh[bb, h, :int(lens_c[bb])] for bb in range(b) for h in range(hkv)]
    return zs, outs


@pytest.mark.parametrize("slots", [True, False])
@pytest.mark.parametrize("kind", ["decode", "ties", "heads"])
def test_fused_gram_finish_equals_separate_kernels(kind, slots, monkeypatch):
    # slot reuse: Z formed from the Gram slots inside the one-launch step,
    # then the threshold and the evicted list, bit for bit as the separate
    # finish, threshold and evicted-list kernels give them; compaction (the
    # separate finish and the one-launch selection either way): the same
    # against the two-kernel selection
    pos, budgets = None, None
    if kind == "decode":
        case = synth.layer8b_case(9, n=2176, budget=2048, cap=2176)
    elif kind == "ties":
        case = synth.rkv_case("gram_ties", seed=76, wl=68, b=2, hq=32, hkv=8, d=128, w=8,
                              lengths=[2176, 1800], cap=2176, budget=1000, frac=0.0, sink_scale=None)
        for bb in range(2):
            for a, e in [(0, 700), (700, 1500), (1500, 2176)]:
                case.k[bb, :, a:e] = case.k[bb, :, a:a + 1]
        rng = np.random.default_rng(77)
        pos = np.stack([np.stack([rng.permutation(2176) for _ in range(8)]) for _ in range(2)])
        pos = (pos // 2).astype(np.int32)
    else:
        case = synth.rkv_case("gram_heads", seed=78, wl=69, b=3, hq=32, hkv=8, d=128, w=4,
                              lengths=[4000, 257, 0], cap=4096, budget=1500)
        budgets = np.array([0, 1, 300, 1500, 2047, 9000, 700, 256], np.int32)
    log(f"[fused gram] {kind} slots={slots} lengths={case.lengths.tolist()} B={case.budget}")
    z1, o1 = _gram_outputs(case, slots, pos, budgets)
    monkeypatch.setenv("KVSEL_SEPARATE_KERNELS", "1")
    z2, o2 = _gram_outputs(case, slots, pos, budgets)
    for a, b_ in zip(z1, z2):
        assert np.array_equal(a, b_)
    for a, b_ in zip(o1, o2):
        assert np.array_equal(a, b_)
