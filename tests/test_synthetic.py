"""Seeded input generators: determinism, bf16 encoding, workload shapes and structure."""
import numpy as np
import pytest

import synthetic as syn

torch = pytest.importorskip("torch")


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.005859375, 3.0e38, -1e-30],
                                 np.float32)])
    ours = syn.f32_to_bf16_bits(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, theirs)
    back = syn.bf16_bits_to_f32(ours)
    np.testing.assert_array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_snapkv_head_is_deterministic_and_independent():
    wl = syn.SNAPKV_WORKLOADS["16k-bf16"].with_(L=2048, H=3)
    a = syn.snapkv_head(wl, 1, 2)
    b = syn.snapkv_head(wl, 1, 2)
    c = syn.snapkv_head(wl, 0, 2)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
    assert not np.array_equal(a[1], c[1])
    q, k, v = syn.snapkv_batch(wl)
    np.testing.assert_array_equal(q[1, 2], a[0])
    np.testing.assert_array_equal(k[1, 2], a[1])
    assert q.shape == (2, 3, 32, 128) and k.shape == (2, 3, 2048, 128) and k.dtype == np.uint16


def test_tiny_workload_shape_and_spans():
    wl = syn.SNAPKV_WORKLOADS["tiny-fp32"]
    q, k, v = syn.snapkv_batch(wl)
    assert q.dtype == np.float32 and k.shape == (1, 4, 512, 64)
    for h in range(4):
        u = q[0, h].astype(np.float64).mean(0)
        u /= np.linalg.norm(u)
        proj = k[0, h] @ u
        starts = syn.workloads.snapkv_spans(wl, 0, h)
        boosted = np.zeros(512, bool)
        for s in starts:
            boosted[s:s + wl.span_len] = True
        # planted keys lean toward the window queries by about the boost magnitude
        assert proj[boosted].mean() > proj[~boosted].mean() + 1.5


def test_needle_depth_range():
    wl = syn.SNAPKV_WORKLOADS["380k-bf16"].with_(L=20000, H=8)
    for h in range(8):
        s = syn.workloads.snapkv_spans(wl, 0, h)
        assert len(s) == 1 and 0.05 * wl.L - 1 <= s[0] <= 0.95 * wl.L


def test_h2o_inputs():
    wl = syn.H2O_WORKLOADS["opt6.7b-decode"].with_(B=2, H=2, prompt_len=200)
    q, k, v, biased = syn.h2o_prompt_head(wl, 1, 1)
    assert q.shape == (200, 128) and len(biased) == 10 and len(set(biased)) == 10
    kf = syn.bf16_bits_to_f32(k)
    assert kf[biased].mean() > kf[np.setdiff1d(np.arange(200), biased)].mean() + 1.2
    s0 = syn.h2o_step_inputs(wl, 0)
    s1 = syn.h2o_step_inputs(wl, 1)
    assert s0[0].shape == (2, 2, 128) and not np.array_equal(s0[0], s1[0])
    np.testing.assert_array_equal(s0[2], syn.h2o_step_inputs(wl, 0)[2])
    full = syn.H2O_WORKLOADS["opt6.7b-decode"]
    assert full.cap == 2 * (4096 // 10) + 1
