"""Input generators: storage rounding, structure and determinism (CPU)."""

import numpy as np
import torch

from decode_eviction_amd import synth


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(10000).astype(np.float32) * 10,
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -0.0, 1e30], np.float32)])
    ours = synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(synth.bf16_bits_to_f32(ours),
                          torch.from_numpy(ours.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_near_copy_plan_covers_fraction():
    rng = np.random.default_rng(1)
    plan = synth.near_copy_runs(4096, 0.3, 16, 128, rng)
    covered = sum(r for _, _, r in plan)
    assert covered >= int(np.ceil(0.3 * 4096))
    dst = sorted((t, t + r) for t, _, r in plan)
    assert all(a[1] <= b[0] for a, b in zip(dst, dst[1:]))          # disjoint
    assert all(t >= 16 and s + r <= t for t, s, r in plan)            # source before run


def test_cases_are_deterministic_and_shaped():
    a = synth.tiny_case(3)
    b = synth.tiny_case(3)
    assert np.array_equal(a.k, b.k) and np.array_equal(a.q, b.q)
    assert a.k.shape == (1, 1, 512, 64) and a.q.shape == (1, 1, 8, 64) and a.k.dtype == np.float32
    c = synth.layer8b_case(0, n=1000, budget=100, cap=1024)
    assert c.k.shape == (1, 8, 1024, 128) and c.k.dtype == np.uint16
    kf = c.as_f32("k")
    assert np.all(kf[0, :, 1000:] > 1e29)                                # junk past n
    norms = np.linalg.norm(kf[0, 0, :1000], axis=1)
    assert norms[:4].min() > 4 * np.median(norms[4:])                   # sinks
    cc = synth.cut_case(2, b=2, lengths=[100, 300], hq=8, hkv=2)
    assert cc.k.shape == (2, 2, 300, 128) and cc.q.shape == (2, 8, 128)
