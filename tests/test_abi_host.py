"""C-ABI checks that need no GPU: the library loads, exports every function
include/kvsel.h declares, sizes workspaces, and rejects bad arguments on the
host before launching anything."""

import ctypes

import pytest

from decode_eviction_amd import kvsel as K

NULL = None


@pytest.fixture(scope="module")
def lib():
    return K.lib()


def test_exports_every_declared_function(lib):
    names = K.header_functions()
    assert len(names) >= 10
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing
    assert set(names) == set(K._SIGS)


def test_debug_build_exports_the_same_functions():
    """The KVSEL_DEBUG build (every launch waited for, a failing kernel named)
    exports the same C ABI; __graft_entry__.build() builds it beside the
    release library."""
    import os

    from decode_eviction_amd import build as B
    if not os.path.exists(B.LIB_DEBUG):
        pytest.skip("debug library not built (python -m decode_eviction_amd.build --debug)")
    dbg = ctypes.CDLL(B.LIB_DEBUG)
    missing = [n for n in K.header_functions() if not hasattr(dbg, n)]
    assert not missing, missing


def test_status_strings(lib):
    for s in range(5):
        assert K.status_string(s)
    assert K.status_string(99) == "unknown status"


def test_workspace_sizes(lib):
    ws = K.kvsel_score_evict_workspace(1, 32, 8, 128, 8, 32768, 2048)
    # at least the fp32 importance and score buffers, 8 heads x 32768 tokens x 4 B each
    assert ws >= 2 * 8 * 32768 * 4
    assert K.kvsel_score_evict_workspace(0, 32, 8, 128, 8, 32768, 2048) == 0
    assert K.kvsel_score_evict_workspace(1, 32, 8, 96, 8, 32768, 2048) == 0
    cw = K.kvsel_threshold_cut_workspace(16, 28, 4, 128, 16384)
    assert cw >= 16 * 4 * 16384 * (8 + 7 * 4)      # energies + logits
    assert K.kvsel_threshold_cut_workspace(1, 28, 3, 128, 100) == 0


def _fake(addr=0x10000):
    return ctypes.c_void_p(addr)


def _score_evict(lib, **over):
    a = dict(dt=K.KVSEL_BF16, mode=K.KVSEL_R_GRAM, q=_fake(), k=_fake(), v=_fake(), lens=_fake(),
             b=1, hq=32, hkv=8, d=128, w=8, cap=4096, lam=0.1, budget=1024, ko=_fake(), vo=_fake(),
             cap_out=1024, idx=_fake(), z=NULL, ws=_fake(), wsb=1 << 30)
    a.update(over)
    return lib.kvsel_score_evict(a["dt"], a["mode"], a["q"], a["k"], a["v"], a["lens"], a["b"],
                                 a["hq"], a["hkv"], a["d"], a["w"], a["cap"], a["lam"], a["budget"],
                                 a["ko"], a["vo"], a["cap_out"], a["idx"], a["z"], a["ws"], a["wsb"],
                                 NULL)


@pytest.mark.parametrize("over,code", [
    (dict(q=NULL), K.KVSEL_ERR_INVALID_ARG),
    (dict(k=NULL), K.KVSEL_ERR_INVALID_ARG),
    (dict(v=NULL), K.KVSEL_ERR_INVALID_ARG),
    (dict(idx=NULL), K.KVSEL_ERR_INVALID_ARG),
    (dict(k=_fake(0x10008)), K.KVSEL_ERR_INVALID_ARG),          # misaligned
    (dict(hq=30), K.KVSEL_ERR_INVALID_ARG),                      # Hq % Hkv != 0
    (dict(d=96), K.KVSEL_ERR_UNSUPPORTED),
    (dict(w=64), K.KVSEL_ERR_UNSUPPORTED),                       # g*w > 128
    (dict(budget=0), K.KVSEL_ERR_INVALID_ARG),
    (dict(budget=2000), K.KVSEL_ERR_INVALID_ARG),                # > cap_out
    (dict(lam=1.5), K.KVSEL_ERR_INVALID_ARG),
    (dict(lam=float("nan")), K.KVSEL_ERR_INVALID_ARG),
    (dict(mode=7), K.KVSEL_ERR_INVALID_ARG),
    (dict(dt=5), K.KVSEL_ERR_INVALID_ARG),
    (dict(wsb=1024), K.KVSEL_ERR_WORKSPACE),
    (dict(ws=NULL), K.KVSEL_ERR_WORKSPACE),
    (dict(cap=1 << 24), K.KVSEL_ERR_UNSUPPORTED),
])
def test_score_evict_rejects(lib, over, code):
    assert _score_evict(lib, **over) == code


@pytest.mark.parametrize("over,code", [
    (dict(T=1.0), K.KVSEL_ERR_INVALID_ARG),
    (dict(T=-0.1), K.KVSEL_ERR_INVALID_ARG),
    (dict(n_sink=-1), K.KVSEL_ERR_INVALID_ARG),
    (dict(hq=28, hkv=3), K.KVSEL_ERR_INVALID_ARG),
    (dict(hq=66, hkv=2), K.KVSEL_ERR_UNSUPPORTED),               # g > 32
    (dict(d=80), K.KVSEL_ERR_UNSUPPORTED),
    (dict(kept=NULL), K.KVSEL_ERR_INVALID_ARG),
    (dict(wsb=16), K.KVSEL_ERR_WORKSPACE),
])
def test_threshold_cut_rejects(lib, over, code):
    a = dict(dt=K.KVSEL_BF16, q=_fake(), k=_fake(), lens=_fake(), b=16, hq=28, hkv=4, d=128,
             cap=16384, layer=5, nfull=2, n_sink=4, T=0.01, kept=_fake(), ws=_fake(), wsb=1 << 34)
    a.update(over)
    got = lib.kvsel_threshold_cut(a["dt"], a["q"], a["k"], a["lens"], a["b"], a["hq"], a["hkv"],
                                  a["d"], a["cap"], a["layer"], a["nfull"], a["n_sink"], a["T"],
                                  a["kept"], a["ws"], a["wsb"], NULL)
    assert got == code


def test_stage_entries_reject(lib):
    assert lib.kvsel_select_topb(NULL, _fake(), 1, 1, 10, 5, _fake(), NULL, 0, NULL) == K.KVSEL_ERR_INVALID_ARG
    assert lib.kvsel_select_topb(_fake(), _fake(), 1, 1, 10, 0, _fake(), NULL, 0, NULL) == K.KVSEL_ERR_INVALID_ARG
    assert lib.kvsel_gather(K.KVSEL_BF16, _fake(), _fake(), _fake(), 1, 1, 128, 10, 5, _fake(), _fake(),
                            4, NULL) == K.KVSEL_ERR_INVALID_ARG          # cap_out < budget
    assert lib.kvsel_threshold_cut_from_attn(NULL, _fake(), 1, 4, 1, 10, 4, 0.01, _fake(), _fake(),
                                             1 << 20, NULL) == K.KVSEL_ERR_INVALID_ARG
    assert lib.kvsel_workspace_error(NULL, NULL, NULL) == K.KVSEL_ERR_INVALID_ARG


def test_binding_argument_counts_match_header():
    import re
    with open(K.HEADER_PATH) as f:
        text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
    decls = re.findall(r"\b(kvsel_\w+)\s*\(([^;{]*?)\)\s*;", text, flags=re.S)
    assert len(decls) == len(K._SIGS)
    for name, params in decls:
        params = params.strip()
        n = 0 if params in ("", "void") else params.count(",") + 1
        assert n == len(K._SIGS[name][1]), (name, n, len(K._SIGS[name][1]))


def test_next_row_entries_reject(lib):
    f = _fake
    BF = K.KVSEL_BF16
    # per-head budgets: the budget row is required
    assert lib.kvsel_select_topb_heads(f(), f(), NULL, 1, 2, 10, 5, f(), f(), 1 << 20,
                                       NULL) == K.KVSEL_ERR_INVALID_ARG
    assert lib.kvsel_score_evict_heads(BF, 0, f(), f(), f(), f(), NULL, 1, 4, 2, 128, 2, 64, 0.1,
                                       16, f(), f(), 16, f(), NULL, f(), 1 << 30,
                                       NULL) == K.KVSEL_ERR_INVALID_ARG
    # slot reuse: the evicted list must hold cap - budget entries (cap with budgets)
    assert lib.kvsel_select_evict_slots(f(), f(), NULL, NULL, 1, 2, 100, 60, f(), 39, f(), f(),
                                        1 << 20, NULL) == K.KVSEL_ERR_INVALID_ARG
    assert lib.kvsel_select_evict_slots(f(), f(), NULL, f(), 1, 2, 100, 60, f(), 99, f(), f(),
                                        1 << 20, NULL) == K.KVSEL_ERR_INVALID_ARG
    assert lib.kvsel_select_evict_slots(f(), f(), NULL, NULL, 1, 2, 40000, 60, f(), 40000, f(),
                                        f(), 1 << 30, NULL) == K.KVSEL_ERR_UNSUPPORTED
    assert lib.kvsel_select_evict_slots(f(), f(), NULL, NULL, 1, 2, 100, 60, NULL, 100, f(), f(),
                                        1 << 20, NULL) == K.KVSEL_ERR_INVALID_ARG
    assert lib.kvsel_score_evict_slots(BF, 0, f(), f(), f(), NULL, NULL, 1, 4, 2, 128, 2, 64, 0.1,
                                       16, f(), 47, f(), NULL, f(), 1 << 30,
                                       NULL) == K.KVSEL_ERR_INVALID_ARG
    # slot write: positions need the new tokens' first position
    assert lib.kvsel_slots_write(BF, f(), f(), f(), f(), f(), NULL, f(), 10, f(), 1, 2, 128, 10, 4,
                                 NULL) == K.KVSEL_ERR_INVALID_ARG
    assert lib.kvsel_slots_write(BF, f(), f(), NULL, f(), f(), NULL, f(), 10, f(), 1, 2, 80, 10, 4,
                                 NULL) == K.KVSEL_ERR_UNSUPPORTED
    # last-k-rows cut: 1 <= k_rows <= cap, compaction into a cache at least cap long
    for k_rows in (0, 101):
        assert lib.kvsel_threshold_cut_rows(BF, f(), k_rows, f(), NULL, f(), 1, 28, 4, 128, 100, 5,
                                            2, 4, 0.01, f(), NULL, NULL, 0, f(), 1 << 30,
                                            NULL) == K.KVSEL_ERR_INVALID_ARG
    assert lib.kvsel_threshold_cut_rows(BF, f(), 3, f(), f(), f(), 1, 28, 4, 128, 100, 5, 2, 4, 0.01,
                                        f(), f(), f(), 99, f(), 1 << 30,
                                        NULL) == K.KVSEL_ERR_INVALID_ARG
    assert lib.kvsel_threshold_cut_rows(BF, f(), 3, f(), NULL, f(), 1, 28, 4, 128, 100, 5, 2, 4, 0.01,
                                        f(), NULL, NULL, 0, f(), 16, NULL) == K.KVSEL_ERR_WORKSPACE
    assert lib.kvsel_cut_compact(BF, f(), f(), f(), NULL, 1, 2, 128, 10, 4, f(), f(), 10,
                                 NULL) == K.KVSEL_ERR_INVALID_ARG
    # groups of up to 32 rows store their logits (k = 4: 28 rows); larger
    # groups recompute them, so the k = 64 workspace holds no logits buffer
    base = K.kvsel_threshold_cut_workspace(16, 28, 4, 128, 16384)
    assert K.kvsel_threshold_cut_rows_workspace(16, 28, 4, 128, 16384, 4) > base
    assert 0 < K.kvsel_threshold_cut_rows_workspace(16, 28, 4, 128, 16384, 64) < base
    assert K.kvsel_threshold_cut_rows_workspace(16, 28, 4, 128, 16384, 0) == 0


def test_bench_kernel_names_follow_the_reduce_folding():
    # the benchmark names traced kernels by launch order; the library skips
    # k_reduce for R-KV calls with at most kFuseReduceChunks chunks of 256
    # keys per head, and the benchmark's list must drop it at the same caps
    import os
    import re

    import bench
    hdr = os.path.join(os.path.dirname(K.__file__), "csrc", "kernels.hpp")
    src = open(hdr).read()
    fuse = int(re.search(r"constexpr int kFuseReduceChunks = (\d+);", src).group(1))
    chunk = int(re.search(r"constexpr int kChunk = (\d+);", src).group(1))
    fmax = int(re.search(r"constexpr int kFusedMaxChunks = (\d+);", src).group(1))
    pair_cap = int(re.search(r"constexpr int kGramPairCap = (\d+);", src).group(1))
    assert fmax == bench.FUSED_MAX_CHUNKS and pair_cap == bench.GRAM_PAIR_CAP
    for mode in ("gram", "keysum"):
        for cap in (1, 2176, fuse * chunk, fuse * chunk + 1, 32768):
            names = bench.rkv_kernels(mode, cap)
            if bench.fused_step(mode, cap):
                assert names == ["fused"] and mode == "keysum" and -(-cap // chunk) <= fmax
                continue
            sel = ["select_compact"] if bench.select_one_launch(cap) else ["thresh", "compact"]
            assert names[-len(sel):] == sel, (mode, cap)
            names = names[:-len(sel)]
            if bench.scores_fused(mode, cap):
                assert -(-cap // chunk) > fmax
                assert names == ["scores"] + [k for k in bench.KERNELS[mode]
                                              if k not in ("stats", "reduce", "pool", "thresh", "compact")]
                continue
            folded = -(-cap // chunk) <= fuse
            assert ("reduce" not in names) == folded, (mode, cap)
            want = [k for k in bench.KERNELS[mode] if k not in ("reduce", "thresh", "compact")]
            if mode == "gram" and cap <= pair_cap:   # the pair units beside the importance pass
                want = ["scores_pairs", "gram_fin"] if bench.scores_pairs_step(mode, cap) else \
                    ["stats", "pool_pairs", "gram_fin"]
            assert want == [k for k in names if k != "reduce"], (mode, cap)
    # 64 sequences of 2176 tokens: 9 * 8 * 64 work-groups do not fit at once
    assert bench.rkv_kernels("keysum", 2176, b=64) != ["fused"]
    # the n = 32768 layer: 128 * 8 work-groups of the score pass fit at four per
    # compute unit; 64 sequences of 8192 tokens do not
    assert bench.rkv_kernels("keysum", 32768)[0] == "scores"
    assert bench.rkv_kernels("keysum", 8192, b=64)[0] == "stats"
    # the Gram form's score pass on the same caches
    assert bench.rkv_kernels("gram", 2176) == ["scores_pairs", "gram_fin", "select_compact"]
    assert bench.rkv_kernels("gram", 2176, b=64) == ["stats", "pool_pairs", "gram_fin", "thresh", "compact"]
    assert bench.rkv_kernels("gram", 32768)[:3] == ["scores", "gram", "gram_fin"]
    assert bench.rkv_kernels("gram", 8192, b=64)[0] == "stats"
    # slot reuse: the fused step's slot form where the fused step applies,
    # otherwise the scores as a compacting call computes them
    assert bench.slot_kernels("gram", 2176) == ["scores_pairs", "fused_fin_slots"]
    assert bench.slot_kernels("gram", 2176, b=64) == ["stats", "pool_pairs", "gram_fin", "thresh", "evict"]
    assert bench.slot_kernels("keysum", 2176) == ["fused_slots"]
    assert bench.slot_kernels("keysum", 2176, b=64) == ["stats", "pool", "thresh", "evict"]
    assert bench.slot_kernels("gram", 8192)[:2] == ["scores", "gram"]
    # the one-launch selection: the n = 32768 layer (32 of 512 kept per chunk)
    # and the decode cache (about 480 of 512 kept: eight gathering work-groups
    # per chunk), not 64 sequences (many heads)
    assert bench.rkv_kernels("gram", 32768)[-1] == "select_compact"
    assert bench.rkv_kernels("gram", 2176)[-1] == "select_compact"
    assert bench.rkv_kernels("keysum", 8192, b=64, budget=1024)[-2:] == ["thresh", "compact"]
    # 40 heads of the decode cache: 5 chunks * 8 work-groups * 40 do not fit at once
    assert bench.rkv_kernels("gram", 2176, b=5)[-2:] == ["thresh", "compact"]
    src_k = open(hdr).read()
    assert int(re.search(r"constexpr int kMaxGsplit = (\d+);", src_k).group(1)) == 8
    src_sel = open(os.path.join(os.path.dirname(K.__file__), "csrc", "select.hip")).read()
    assert int(re.search(r"constexpr int kThreshHeadsMany = (\d+);", src_sel).group(1)) == bench.THRESH_HEADS_MANY
    assert int(re.search(r"constexpr int kSelChunk = (\d+);", src).group(1)) == bench.SEL_CHUNK
    assert set(bench.KERNEL_SOURCES) >= set(bench.rkv_cost("gram")) - {"evict"}
