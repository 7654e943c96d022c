"""R-KV score-and-evict on the GPU against the fp64 oracle (through the C ABI).

Cases: the tiny fp32 layer (n=512), the 8B-shaped layer (n=4096), ragged and
padded batches covering several tiles and ragged tails, d=64 with 8/64/128
window rows, the n=32768 layer in the launch configuration the benchmark
times, the batched 64 x 8192 workload (all 512 heads), stage entries (top-B
on oracle scores, gather), per-head budgets (stage and whole step),
determinism and the clamped-length flag.
"""

import dataclasses

import numpy as np
import pytest
import torch

from decode_eviction_amd import kvsel as K
from decode_eviction_amd import synth
from oracle import rkv
from tests.gpu_util import (SWAP_WINDOW, SCORE_RTOL, check_idx_structure, dev, dev_i32, host_bits,
                            log, score_err, swaps)

pytestmark = pytest.mark.gpu

MODES = ["gram", "keysum"]


def gpu_run(case, mode):
    """Scores (I, R, Z) and the full step on the device; host copies out."""
    q = dev(case.q, case.dtype)
    k = dev(case.k, case.dtype)
    v = dev(case.v, case.dtype)
    lens = dev_i32(case.lengths)
    shape = (case.b, case.hkv, case.cap)
    i_o = torch.full(shape, float("nan"), device="cuda")
    r_o = torch.full(shape, float("nan"), device="cuda")
    z_o = torch.full(shape, float("nan"), device="cuda")
    K.kvsel_scores(q, k, lens, case.lam, mode, i_o, r_o, z_o)
    z2 = torch.full(shape, float("nan"), device="cuda")
    k_out, v_out, idx = K.kvsel_score_evict(q, k, v, lens, case.budget, case.lam, mode,
                                            scores_out=z2)
    torch.cuda.synchronize()
    return dict(I=i_o.cpu().numpy(), R=r_o.cpu().numpy(), Z=z_o.cpu().numpy(),
                Z2=z2.cpu().numpy(), idx=idx.cpu().numpy(), k_out=host_bits(k_out),
                v_out=host_bits(v_out))


def check_case(case, mode, form="definition", heads=None, sample_rows=0):
    log(f"[rkv] {case.name} mode={mode} b={case.b} hkv={case.hkv} d={case.d} "
        f"lengths={case.lengths.tolist()[:4]} B={case.budget}")
    got = gpu_run(case, mode)
    qf, kf, vf = case.as_f32("q"), case.as_f32("k"), case.as_f32("v")
    ref = rkv.score_evict(qf, kf, vf, case.lengths, case.lam, case.budget, form=form, heads=heads)
    kbits = case.k if case.dtype == "bf16" else case.k.view(np.uint32)
    vbits = case.v if case.dtype == "bf16" else case.v.view(np.uint32)
    todo = heads or [(b, h) for b in range(case.b) for h in range(case.hkv)]
    worst = dict(I=0.0, R=0.0, Z=0.0)
    tot_swaps, max_gap = 0, float("-inf")
    rng = np.random.default_rng(0)
    for b, h in todo:
        n = int(case.lengths[b])
        for name in ("I", "R", "Z"):
            e = score_err(got[name][b, h, :n], ref[name][b][h])
            worst[name] = max(worst[name], e)
        assert np.array_equal(got["Z"][b, h, :n], got["Z2"][b, h, :n]), "Z differs between entry points"
        idx = got["idx"][b, h]
        check_idx_structure(idx, n, case.budget)
        ns, gap = swaps(idx, ref["idx"][b, h], ref["Z"][b][h])
        tot_swaps += ns
        max_gap = max(max_gap, gap)
        assert gap < SWAP_WINDOW, f"head {(b, h)}: swap gap {gap}"
        m = min(n, case.budget)
        assert np.array_equal(got["k_out"][b, h, :m], kbits[b, h, idx[:m]]), "K rows not bit copies"
        assert np.array_equal(got["v_out"][b, h, :m], vbits[b, h, idx[:m]]), "V rows not bit copies"
        if sample_rows and n > 1:
            rows = np.unique(np.concatenate([np.arange(min(4, n)), rng.integers(0, n, sample_rows)]))
            r_def = rkv.redundancy_rows(kf[b, h, :n], rows)
            worst["R_def"] = max(worst.get("R_def", 0.0), score_err(got["R"][b, h, rows], r_def))
            assert score_err(r_def, ref["R"][b][h][rows]) < 1e-9
    log(f"    worst floored-rel err {worst}; swaps={tot_swaps} max_gap={max_gap:.3e}")
    for name, e in worst.items():
        assert e <= SCORE_RTOL, f"{name} error {e}"
    return got, ref


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_tiny_fp32(mode, seed):
    check_case(synth.tiny_case(seed), mode)


@pytest.mark.parametrize("mode", MODES)
def test_layer8b_n4096(mode):
    check_case(synth.layer8b_case(0), mode)


@pytest.mark.parametrize("mode", MODES)
def test_ragged_batch_bf16(mode):
    case = synth.rkv_case("ragged", seed=3, wl=99, b=3, hq=8, hkv=2, d=128, w=4,
                          lengths=[1000, 37, 777], cap=1024, budget=100)
    check_case(case, mode)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("cap,lengths", [(1031, [1031, 500, 1001]), (5003, [5003, 4100, 4099])])
def test_cap_not_multiple_of_4(mode, cap, lengths):
    # rows of the per-key score buffers lose 16-byte alignment: the scalar
    # finishing pass of the Gram form (pair kernel below 4097, 256-key blocks above)
    case = synth.rkv_case("oddcap", seed=11, wl=95, b=3, hq=8, hkv=2, d=128, w=4,
                          lengths=lengths, cap=cap, budget=300)
    check_case(case, mode)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("hq,hkv,w", [(4, 4, 2), (16, 2, 8), (32, 2, 8)])
def test_d64_row_tiles(mode, hq, hkv, w):
    case = synth.rkv_case("d64", seed=4, wl=98, b=2, hq=hq, hkv=hkv, d=64, w=w,
                          lengths=[300, 513], cap=600, budget=64)
    check_case(case, mode)


@pytest.mark.parametrize("mode", MODES)
def test_fp32_d128_single_tile_tail(mode):
    case = synth.rkv_case("f32d128", seed=5, wl=97, b=1, hq=2, hkv=1, d=128, w=3,
                          lengths=[45], cap=64, budget=20, dtype="f32", frac=0.2,
                          run_lo=4, run_hi=8, sink_scale=None)
    check_case(case, mode)


@pytest.mark.parametrize("mode", MODES)
def test_tiny_lengths_edge(mode):
    # n = 0, 1, 2 and n == B
    case = synth.rkv_case("edge", seed=6, wl=96, b=4, hq=4, hkv=2, d=64, w=2,
                          lengths=[0, 1, 2, 16], cap=32, budget=16, frac=0.0, sink_scale=None)
    got = gpu_run(case, mode)
    assert (got["idx"][0] == -1).all()
    assert got["idx"][1, :, 0].tolist() == [0, 0] and (got["idx"][1, :, 1:] == -1).all()
    assert np.allclose(got["R"][1, :, 0], 0.0)
    assert got["idx"][3].tolist() == [list(range(16))] * 2
    check_case(case, mode, heads=[(2, 0), (2, 1), (3, 0), (3, 1)])


def test_duplicate_copy_golden_on_gpu():
    # orthonormal keys e0..e4 plus a copy of e2 (tests/golden/rkv_duplicate_copy.txt), zero query
    d, n = 64, 6
    k = np.zeros((1, 1, n, d), np.float32)
    k[0, 0, np.arange(5), np.arange(5)] = 1.0
    k[0, 0, 5] = k[0, 0, 2]
    case = synth.RKVCase("dup", "f32", 1, 1, 1, d, 1, n, 5, 0.1, np.array([n], np.int32),
                         np.zeros((1, 1, 1, d), np.float32), k, k.copy())
    for mode in MODES:
        got = gpu_run(case, mode)
        assert np.allclose(got["Z"][0, 0], [1 / 60, 1 / 60, 1 / 60 - 0.18, 1 / 60, 1 / 60, 1 / 60 - 0.18],
                           atol=1e-6)
        assert got["idx"][0, 0].tolist() == [0, 1, 2, 3, 4]


@pytest.mark.parametrize("mode", MODES)
def test_headline_n32768_full_size(mode):
    case = synth.headline_case(layer=0)
    check_case(case, mode, form="keysum", sample_rows=48)


@pytest.mark.parametrize("mode", MODES)
def test_large_cap_ragged_lengths(mode):
    # the 512-key-block Gram path (bf16, d=128, cap >= 8192) with lengths that
    # end inside a block: 9001 keys (18 blocks, even) and 8300 (17 blocks, odd)
    case = synth.rkv_case("bigragged", seed=13, wl=93, b=2, hq=8, hkv=2, d=128, w=8,
                          lengths=[9001, 8300], cap=9216, budget=1000)
    check_case(case, mode, form="keysum", sample_rows=24)


def test_pool_merge_matches_reduce_kernel():
    # cap 4096 (16 chunks): k_pool merges the chunk partials itself; the same
    # keys in a 4352-slot cache (17 chunks) go through k_reduce.  Both merge
    # in one order, so the key-sum scores and selections are bitwise equal.
    case = synth.rkv_case("fusedreduce", seed=19, wl=89, b=2, hq=16, hkv=4, d=128, w=8,
                          lengths=[4096, 2500], cap=4096, budget=700)
    pad = 4352 - case.cap
    wide = dataclasses.replace(
        case, cap=4352,
        k=np.concatenate([case.k, np.zeros(case.k.shape[:2] + (pad, case.d), case.k.dtype)], axis=2),
        v=np.concatenate([case.v, np.zeros(case.v.shape[:2] + (pad, case.d), case.v.dtype)], axis=2))
    log("[rkv] fused reduce: cap 4096 vs 4352, keysum")
    a = gpu_run(case, "keysum")
    b = gpu_run(wide, "keysum")
    for bi, n in enumerate(case.lengths.tolist()):
        for name in ("I", "R", "Z"):
            assert np.array_equal(a[name][bi, :, :n], b[name][bi, :, :n]), name
    assert np.array_equal(a["idx"], b["idx"])


@pytest.mark.parametrize("mode", MODES)
def test_many_chunks_ragged(mode):
    # 2048 chunks of 256 keys in the call: the statistics pass gives each
    # work-group two consecutive chunks of a head; lengths end inside a chunk,
    # on a chunk boundary, inside a work-group's first chunk and at 1
    case = synth.rkv_case("manychunks", seed=17, wl=91, b=8, hq=8, hkv=4, d=128, w=4,
                          lengths=[16384, 9000, 300, 16000, 12345, 1, 8192, 4097],
                          cap=16384, budget=500)
    check_case(case, mode, form="keysum", heads=[(0, 0), (1, 3), (2, 1), (4, 2), (5, 0), (6, 3), (7, 1)],
               sample_rows=8)


@pytest.mark.parametrize("mode", ["keysum", "gram"])
def test_batched_64x8192_all_heads(mode):
    # every one of the 512 (sequence, KV head) pairs against the key-sum
    # oracle; a few heads also against the pairwise definition on sampled rows
    case = synth.batched_case(0)
    check_case(case, mode, form="keysum", sample_rows=0)
    check_case(case, mode, form="keysum", heads=[(0, 0), (31, 7), (63, 5)], sample_rows=16)


@pytest.mark.parametrize("separate", [False, True], ids=["one_launch", "two_kernels"])
def test_select_stage_exact(separate, monkeypatch):
    """Top-B on given scores is exact: same set as the oracle on the same fp32 values,
    through the one-launch selection (caps up to 32768) and the two-kernel one."""
    if separate:
        monkeypatch.setenv("KVSEL_SEPARATE_KERNELS", "1")
    rng = np.random.default_rng(7)
    for n, cap, budget, kind in [(5000, 5000, 700, "ties"), (32768, 32768, 2048, "normal"),
                                 (40000, 40001, 3000, "ties"), (2176, 2176, 2048, "normal"),
                                 (100, 128, 100, "normal"), (1000, 1000, 999, "allequal"),
                                 (33000, 33000, 1, "normal"),
                                 # threshold bins larger than the candidate buffer (8192 keys)
                                 (32768, 32768, 2048, "allequal"), (32768, 32768, 5000, "few")]:
        if kind == "ties":
            z = (rng.integers(-40, 40, size=(2, 3, cap)) * 2.0 ** -12).astype(np.float32)
        elif kind == "allequal":
            z = np.full((2, 3, cap), 0.25, np.float32)
        elif kind == "few":
            z = rng.choice(np.array([0.5, 0.25, 0.125], np.float32), size=(2, 3, cap))
        else:
            z = rng.standard_normal((2, 3, cap)).astype(np.float32) * 1e-3
        z[..., 0] = -0.0
        lens = np.array([n, max(1, n // 3)], np.int32)
        log(f"[select] n={n} cap={cap} B={budget} {kind}")
        idx = K.kvsel_select_topb(dev(z, "f32"), dev_i32(lens), budget).cpu().numpy()
        for b in range(2):
            for h in range(3):
                nb = int(lens[b])
                want = rkv.top_budget(z[b, h, :nb].astype(np.float64), budget)
                m = min(nb, budget)
                assert idx[b, h, :m].tolist() == want.tolist(), (n, budget, kind, b, h)
                assert (idx[b, h, m:] == -1).all()


def test_select_stage_exact_many_heads():
    """64 heads or more: the threshold kernel runs one work-group per head; normal
    scores, ties, all-equal scores (the register path for bins larger than its
    candidate buffer) and caps below and at 32768."""
    rng = np.random.default_rng(27)
    for b, hkv, n, budget, kind in [(8, 8, 4000, 700, "normal"), (16, 4, 2176, 2048, "ties"),
                                    (8, 8, 32768, 2048, "allequal"), (2, 32, 32768, 3000, "few"),
                                    (4, 16, 9000, 1, "normal")]:
        cap = n
        if kind == "ties":
            z = (rng.integers(-40, 40, size=(b, hkv, cap)) * 2.0 ** -12).astype(np.float32)
        elif kind == "allequal":
            z = np.full((b, hkv, cap), -0.5, np.float32)
        elif kind == "few":
            z = rng.choice(np.array([0.5, 0.25, 0.125], np.float32), size=(b, hkv, cap))
        else:
            z = rng.standard_normal((b, hkv, cap)).astype(np.float32) * 1e-3
        lens = np.array([n - (i % 3) * (n // 5) for i in range(b)], np.int32)
        log(f"[select many heads] b={b} hkv={hkv} n={n} B={budget} {kind}")
        idx = K.kvsel_select_topb(dev(z, "f32"), dev_i32(lens), budget).cpu().numpy()
        for bi in range(b):
            for h in range(hkv):
                nb = int(lens[bi])
                want = rkv.top_budget(z[bi, h, :nb].astype(np.float64), budget)
                m = min(nb, budget)
                assert idx[bi, h, :m].tolist() == want.tolist(), (kind, bi, h)
                assert (idx[bi, h, m:] == -1).all()


@pytest.mark.parametrize("separate", [False, True], ids=["one_launch", "two_kernels"])
def test_select_heads_stage_exact(separate, monkeypatch):
    """Per-head budgets on given scores: each head's set is the oracle's for its own budget."""
    if separate:
        monkeypatch.setenv("KVSEL_SEPARATE_KERNELS", "1")
    rng = np.random.default_rng(17)
    for n, cap, bmax, kind in [(2176, 2176, 2048, "normal"), (5000, 5000, 900, "ties"),
                               (40000, 40001, 3000, "ties"), (300, 512, 256, "normal")]:
        hkv = 6
        if kind == "ties":
            z = (rng.integers(-40, 40, size=(2, hkv, cap)) * 2.0 ** -12).astype(np.float32)
        else:
            z = rng.standard_normal((2, hkv, cap)).astype(np.float32) * 1e-3
        lens = np.array([n, max(1, n // 3)], np.int32)
        budgets = np.array([0, 1, bmax // 2, bmax, n, bmax + 5], np.int32)
        budgets = budgets[rng.permutation(hkv)]
        log(f"[select heads] n={n} cap={cap} Bmax={bmax} budgets={budgets.tolist()} {kind}")
        ws = torch.empty(K.kvsel_select_workspace(2, hkv, cap), dtype=torch.uint8, device="cuda")
        idx = K.kvsel_select_topb_heads(dev(z, "f32"), dev_i32(lens), dev_i32(budgets), bmax,
                                        workspace=ws).cpu().numpy()
        assert K.kvsel_workspace_error(ws) == 2            # bmax + 5 was clamped
        for b in range(2):
            for h in range(hkv):
                nb = int(lens[b])
                bh = rkv.head_budget(budgets, h, bmax)
                want = rkv.top_budget(z[b, h, :nb].astype(np.float64), bh)
                m = min(nb, bh)
                assert idx[b, h, :m].tolist() == want.tolist(), (n, kind, b, h, bh)
                assert (idx[b, h, m:] == -1).all()
        ok = np.clip(budgets, 0, bmax).astype(np.int32)
        idx2 = K.kvsel_select_topb_heads(dev(z, "f32"), dev_i32(lens), dev_i32(ok), bmax,
                                         workspace=ws).cpu().numpy()
        assert K.kvsel_workspace_error(ws) == 0
        assert np.array_equal(idx, idx2)


@pytest.mark.parametrize("mode", MODES)
def test_score_evict_heads(mode):
    case = synth.rkv_case("heads", seed=12, wl=94, b=2, hq=16, hkv=4, d=128, w=8,
                          lengths=[3000, 1700], cap=3072, budget=1024)
    budgets = np.array([1024, 0, 700, 1800], np.int32)      # 1800 > 1024: clamped
    q, k, v = dev(case.q, "bf16"), dev(case.k, "bf16"), dev(case.v, "bf16")
    ws = torch.empty(K.kvsel_score_evict_workspace(2, 16, 4, 128, 8, 3072, 1024), dtype=torch.uint8,
                     device="cuda")
    z = torch.full((2, 4, 3072), float("nan"), device="cuda")
    k_out, v_out, idx = K.kvsel_score_evict_heads(q, k, v, dev_i32(case.lengths), dev_i32(budgets),
                                                  1024, case.lam, mode, scores_out=z, workspace=ws)
    assert K.kvsel_workspace_error(ws) == 2
    idx, z = idx.cpu().numpy(), z.cpu().numpy()
    k_out, v_out = host_bits(k_out), host_bits(v_out)
    ref = rkv.score_evict(case.as_f32("q"), case.as_f32("k"), case.as_f32("v"), case.lengths,
                          case.lam, 1024, form="keysum", budgets=budgets)
    for b in range(2):
        n = int(case.lengths[b])
        for h in range(4):
            bh = rkv.head_budget(budgets, h, 1024)
            m = min(n, bh)
            assert score_err(z[b, h, :n], ref["Z"][b][h]) <= SCORE_RTOL
            assert (idx[b, h, m:] == -1).all()
            if m:
                check_idx_structure(idx[b, h], n, m)
            ns, gap = swaps(idx[b, h, :m], ref["idx"][b, h, :m], ref["Z"][b][h])
            assert gap < SWAP_WINDOW, (b, h, gap)
            assert np.array_equal(k_out[b, h, :m], case.k[b, h, idx[b, h, :m]])
            assert np.array_equal(v_out[b, h, :m], case.v[b, h, idx[b, h, :m]])
            assert (k_out[b, h, m:] == 0).all()           # rows past the head's budget untouched


def test_gather_stage_bit_exact():
    rng = np.random.default_rng(8)
    for dtype, d in [("bf16", 128), ("bf16", 64), ("f32", 64), ("f32", 128)]:
        b, hkv, cap, budget = 2, 3, 300, 50
        if dtype == "bf16":
            kh = rng.integers(0, 65536, size=(b, hkv, cap, d), dtype=np.uint16)
            vh = rng.integers(0, 65536, size=(b, hkv, cap, d), dtype=np.uint16)
        else:
            kh = rng.standard_normal((b, hkv, cap, d)).astype(np.float32)
            vh = rng.standard_normal((b, hkv, cap, d)).astype(np.float32)
        idx = np.sort(rng.choice(cap, size=(b, hkv, budget)), axis=-1).astype(np.int32)
        idx[1, 2, 40:] = -1
        ko, vo = K.kvsel_gather(dev(kh, dtype), dev(vh, dtype), dev_i32(idx))
        ko, vo = host_bits(ko), host_bits(vo)
        kb = kh if dtype == "bf16" else kh.view(np.uint32)
        vb = vh if dtype == "bf16" else vh.view(np.uint32)
        for bb in range(b):
            for h in range(hkv):
                m = (idx[bb, h] >= 0).sum()
                assert np.array_equal(ko[bb, h, :m], kb[bb, h, idx[bb, h, :m]])
                assert np.array_equal(vo[bb, h, :m], vb[bb, h, idx[bb, h, :m]])
                assert (ko[bb, h, m:] == 0).all()          # untouched rows stay zero


@pytest.mark.parametrize("mode", MODES)
def test_deterministic(mode):
    case = synth.layer8b_case(1, n=3000, budget=500, cap=3072)
    a = gpu_run(case, mode)
    b = gpu_run(case, mode)
    for name in ("I", "R", "Z", "idx", "k_out", "v_out"):
        assert np.array_equal(a[name], b[name], equal_nan=True), name


def test_lengths_above_cap_are_clamped_and_flagged():
    case = synth.rkv_case("clamp", seed=9, wl=95, b=2, hq=4, hkv=2, d=64, w=2,
                          lengths=[200, 150], cap=200, budget=32)
    q, k, v = dev(case.q, "bf16"), dev(case.k, "bf16"), dev(case.v, "bf16")
    ws = torch.empty(K.kvsel_score_evict_workspace(2, 4, 2, 64, 2, 200, 32), dtype=torch.uint8,
                     device="cuda")
    _, _, idx_ok = K.kvsel_score_evict(q, k, v, dev_i32([200, 150]), 32, workspace=ws)
    assert K.kvsel_workspace_error(ws) == 0
    _, _, idx_big = K.kvsel_score_evict(q, k, v, dev_i32([500, 150]), 32, workspace=ws)
    assert K.kvsel_workspace_error(ws) == 1
    assert np.array_equal(idx_ok.cpu().numpy(), idx_big.cpu().numpy())
