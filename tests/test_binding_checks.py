"""Argument checks of the Python binding (CPU only).

The binding raises before it calls into libkvsel when an element type or a
shape is wrong: an int64 lengths tensor would be read as pairs of int32
words, and a short one would be read past its end.  The helpers are called
on host tensors here; the wrappers are exercised with the device check
switched off, so each must reject before reaching the library.
"""

import pytest
import torch

from decode_eviction_amd import kvsel as K


def test_lengths_must_be_int32_and_long_enough():
    with pytest.raises(TypeError):
        K._need_lengths(torch.zeros(3, dtype=torch.int64), 3)
    with pytest.raises(ValueError):
        K._need_lengths(torch.zeros(2, dtype=torch.int32), 3)
    K._need_lengths(torch.zeros(4, dtype=torch.int32), 3)


def test_dtype_must_match_k():
    k = torch.zeros((1, 2, 8, 64), dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        K._need_like(k, "v", torch.zeros((1, 2, 8, 64), dtype=torch.float32))
    K._need_like(k, "v", torch.zeros((1, 2, 8, 64), dtype=torch.bfloat16))
    K._need_like(k, "v", None)


def test_output_shape_and_dtype():
    idx = torch.zeros((1, 8, 100), dtype=torch.int32)
    with pytest.raises(ValueError):
        K._need_out(idx, "idx_out", torch.int32, (1, 8), rows=128)
    with pytest.raises(TypeError):
        K._need_out(idx.float(), "idx_out", torch.int32, (1, 8), rows=100)
    with pytest.raises(ValueError):
        K._need_out(idx, "idx_out", torch.int32, (2, 8), rows=100)
    K._need_out(idx, "idx_out", torch.int32, (1, 8), rows=100)
    ko = torch.zeros((1, 8, 100, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        K._need_out(ko, "k_out", torch.bfloat16, (1, 8), min_rows=101, tail=64)
    with pytest.raises(ValueError):
        K._need_out(ko, "k_out", torch.bfloat16, (1, 8), min_rows=10, tail=128)
    K._need_out(ko, "k_out", torch.bfloat16, (1, 8), min_rows=100, tail=64)


def test_workspace_must_be_bytes():
    with pytest.raises(TypeError):
        K._workspace(100, "cpu", torch.zeros(100, dtype=torch.float32))


@pytest.fixture
def host_tensors(monkeypatch):
    monkeypatch.setattr(K, "_need_cuda", lambda *ts: None)
    b, hq, hkv, w, d, cap = 2, 8, 2, 4, 64, 32
    q = torch.zeros((b, hq, w, d), dtype=torch.bfloat16)
    k = torch.zeros((b, hkv, cap, d), dtype=torch.bfloat16)
    return q, k, k.clone(), torch.full((b,), cap, dtype=torch.int32)


def _no_library(monkeypatch):
    def boom():
        raise AssertionError("the library was reached")
    monkeypatch.setattr(K, "lib", boom)


def test_wrappers_reject_before_the_library(host_tensors, monkeypatch):
    q, k, v, lens = host_tensors
    _no_library(monkeypatch)
    with pytest.raises(TypeError):
        K.kvsel_score_evict(q, k, v, lens.long(), 8)
    with pytest.raises(ValueError):
        K.kvsel_score_evict(q, k, v, lens[:1], 8)
    with pytest.raises(TypeError):
        K.kvsel_score_evict(q, k, v.float(), lens, 8)
    with pytest.raises(TypeError):
        K.kvsel_score_evict(q.float(), k, v, lens, 8)
    with pytest.raises(ValueError):
        K.kvsel_score_evict(q, k, v, lens, 8, idx_out=torch.zeros((2, 2, 7), dtype=torch.int32))
    with pytest.raises(ValueError):
        K.kvsel_score_evict(q, k, v, lens, 8, scores_out=torch.zeros((2, 2, 31)))
    with pytest.raises(TypeError):
        K.kvsel_score_evict_heads(q, k, v, lens, torch.zeros(2, dtype=torch.int64), 8)
    with pytest.raises(ValueError):
        K.kvsel_score_evict_heads(q, k, v, lens, torch.zeros(1, dtype=torch.int32), 8)
    with pytest.raises(TypeError):
        K.kvsel_select_topb(torch.zeros((2, 2, 32)), lens.long(), 8)
    with pytest.raises(TypeError):
        K.kvsel_select_topb(torch.zeros((2, 2, 32), dtype=torch.float64), lens, 8)
    with pytest.raises(TypeError):
        K.kvsel_threshold_cut(q[:, :, 0], k, lens.long(), 3)
    with pytest.raises(ValueError):
        K.kvsel_threshold_cut(q[:, :, 0, :32], k, lens, 3)
    with pytest.raises(TypeError):
        K.kvsel_threshold_cut_from_attn(torch.zeros((2, 8, 32)), lens.long(), 2)
    with pytest.raises(TypeError):
        K.kvsel_gather(k, v, torch.zeros((2, 2, 4), dtype=torch.int64))
    with pytest.raises(ValueError):
        K.kvsel_slots_write(k, v, k[:, :, :4], v[:, :, :4], torch.zeros((2, 2, 4), dtype=torch.int32),
                            torch.zeros((2, 1), dtype=torch.int32))
