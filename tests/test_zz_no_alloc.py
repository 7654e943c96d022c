"""The allocation-free entry point (kvsel_score_evict_static) against
kvsel_score_evict on the same inputs: two calls in a row through the C ABI,
the second on a smaller input (fewer sequences, shorter cache), so that the
scratch array's leftovers from the first call must not leak into the
second.  Both entry points run the same kernels, so Z, the kept indices and
the compacted rows must be bit-identical; Z is also checked against the
oracle.  A layout beyond the array's size is refused."""

import numpy as np
import pytest
import torch

from decode_eviction_amd import kvsel as K
from decode_eviction_amd import synth
from oracle import rkv
from tests.gpu_util import SCORE_RTOL, dev, dev_i32, host_bits, log, score_err

pytestmark = pytest.mark.gpu


def _both(case, mode):
    q, k, v = dev(case.q, case.dtype), dev(case.k, case.dtype), dev(case.v, case.dtype)
    lens = dev_i32(case.lengths)
    shape = (case.b, case.hkv, case.cap)
    z_ref = torch.full(shape, float("nan"), device="cuda")
    ko_ref, vo_ref, idx_ref = K.kvsel_score_evict(q, k, v, lens, case.budget, case.lam, mode,
                                                  scores_out=z_ref)
    z = torch.full(shape, float("nan"), device="cuda")
    ko = torch.zeros_like(ko_ref)
    vo = torch.zeros_like(vo_ref)
    idx = torch.full_like(idx_ref, -7)
    K.kvsel_score_evict_static(q, k, v, lens, case.budget, case.lam, mode, k_out=ko, v_out=vo,
                               idx_out=idx, scores_out=z)
    torch.cuda.synchronize()
    return (z.cpu().numpy(), idx.cpu().numpy(), host_bits(ko), host_bits(vo),
            z_ref.cpu().numpy(), idx_ref.cpu().numpy(), host_bits(ko_ref), host_bits(vo_ref))


@pytest.mark.parametrize("mode", ["keysum", "gram"])
def test_static_matches_workspace_entry(mode):
    big = synth.rkv_case("static_big", seed=31, wl=81, b=3, hq=32, hkv=8, d=128, w=8,
                         lengths=[4096, 3001, 4000], cap=4096, budget=1024)
    small = synth.rkv_case("static_small", seed=32, wl=82, b=2, hq=32, hkv=8, d=128, w=8,
                           lengths=[2176, 1500], cap=2176, budget=700)
    for case in (big, small):
        log(f"[static] {case.name} mode={mode} b={case.b} cap={case.cap} B={case.budget}")
        z, idx, ko, vo, z_r, idx_r, ko_r, vo_r = _both(case, mode)
        assert np.array_equal(idx, idx_r)
        assert np.array_equal(ko, ko_r) and np.array_equal(vo, vo_r)
        ref = rkv.score_evict(case.as_f32("q"), case.as_f32("k"), case.as_f32("v"), case.lengths,
                              case.lam, case.budget, form="keysum")
        for b in range(case.b):
            n = int(case.lengths[b])
            for h in range(case.hkv):
                assert np.array_equal(z[b, h, :n], z_r[b, h, :n])
                assert score_err(z[b, h, :n], ref["Z"][b][h]) <= SCORE_RTOL


def test_static_refuses_layouts_beyond_the_array():
    case = synth.rkv_case("static_huge", seed=33, wl=83, b=1, hq=32, hkv=8, d=128, w=8,
                          lengths=[100], cap=32768, budget=64, frac=0.0, sink_scale=None)
    q, k, v = dev(case.q, "bf16"), dev(case.k, "bf16"), dev(case.v, "bf16")
    with pytest.raises(K.KvselError) as e:
        K.kvsel_score_evict_static(q, k, v, dev_i32(case.lengths), 64, 0.1, "gram")
    assert e.value.status == K.KVSEL_ERR_WORKSPACE
