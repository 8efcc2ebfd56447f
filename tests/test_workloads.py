"""Checks of the seeded input generators (CPU only)."""
import numpy as np
import pytest
import torch

import workloads as W


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(200_000).astype(np.float32) * 3,
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 65504.0, 1e-40],
                                 dtype=np.float32)])
    ours = W.bf16_bits(x)
    ref = torch.tensor(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    np.testing.assert_array_equal(W.bf16_bits_to_f32(ours),
                                  torch.tensor(x).to(torch.bfloat16).float().numpy())


def test_page_tables():
    rng = np.random.default_rng(1)
    n = np.array([40, 17, 64, 1])
    t, num = W.build_page_table(rng, n, 16, shuffle=True)
    used = np.concatenate([t[b, :(n[b] + 15) // 16] for b in range(4)])
    assert sorted(used) == list(range(num))
    assert (t[1, 2:] == -1).all()
    t2, _ = W.build_page_table(None, np.array([100]), 16, shuffle=False)
    assert list(t2[0]) == list(range(7))


def test_workload_shapes():
    v = W.make_workload_verify("tiny_fp32")
    assert v.q.shape == (1, 4, 2, 64) and v.dtype == "f32"
    assert v.k_cache.shape[1:] == (1, 16, 64) and v.v_cache.shape[1:] == (1, 64, 16)
    assert v.kv_bytes() == (512 + 4) * 64 * 2 * 4 == 264_192
    g = W.make_workload_greedy("tiny_fp32")
    assert g.logits.shape == (1, 4, 1000)


def test_geometric_prefix_law():
    rng = np.random.default_rng(3)
    g = W.make_greedy(rng, B=4000, K=16, V=64, dtype="f32")
    mean = g.planted_len.mean()
    assert 2.6 < mean < 3.4          # truncated Geometric(0.25) on {0, 1, ...}: mean ~ 3
    assert (g.planted_len == 0).mean() == pytest.approx(0.25, abs=0.03)


def test_log_uniform_contexts():
    rng = np.random.default_rng(4)
    c = W.log_uniform_contexts(rng, 20_000)
    assert c.min() >= 4096 and c.max() < 32768
    assert np.mean(np.log(c)) == pytest.approx((np.log(4096) + np.log(32768)) / 2, abs=0.02)


def test_seeded_reproducible():
    a = W.make_workload_greedy("tiny_fp32", cycle=3)
    b = W.make_workload_greedy("tiny_fp32", cycle=3)
    c = W.make_workload_greedy("tiny_fp32", cycle=4)
    np.testing.assert_array_equal(a.logits, b.logits)
    assert not np.array_equal(a.logits, c.logits)
