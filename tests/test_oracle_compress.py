"""Pins of the latent-compressor oracle (CPU only)."""
import numpy as np
import torch

import oracle
import workloads as W


def test_vs_torch_sdpa_scale_one():
    """Library route: torch SDPA (float64, scale 1) with C as queries, F as keys and values."""
    rng = np.random.default_rng(0)
    c = W.make_compress(rng, B=3, C=5, N=17, D=24, q_std=0.3)
    out = oracle.latent_compress_ref(c.queries, c.feats)
    qt = torch.tensor(c.queries.astype(np.float64))[None].expand(3, -1, -1)
    ft = torch.tensor(c.feats.astype(np.float64))
    ref = torch.nn.functional.scaled_dot_product_attention(qt, ft, ft, scale=1.0)
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-12, atol=1e-13)


def test_closed_forms():
    rng = np.random.default_rng(1)
    c = W.make_compress(rng, B=2, C=4, N=9, D=8)
    # zero queries -> uniform weights -> the mean feature row
    out = oracle.latent_compress_ref(np.zeros_like(c.queries), c.feats)
    for b in range(2):
        for i in range(4):
            np.testing.assert_allclose(out[b, i], c.feats[b].astype(np.float64).mean(axis=0),
                                       rtol=1e-12, atol=1e-14)
    # a single feature row -> that row, whatever the queries
    one = c.feats[:, :1, :]
    out = oracle.latent_compress_ref(c.queries, one)
    for i in range(4):
        np.testing.assert_array_equal(out[:, i, :], one[:, 0, :].astype(np.float64))


def test_no_sqrt_d_scale():
    """The printed compressor has no 1/sqrt(D): a query equal to 8x a feature row picks it."""
    rng = np.random.default_rng(2)
    c = W.make_compress(rng, B=1, C=1, N=6, D=64)
    f = c.feats[0].astype(np.float64)
    q = (f[3] / np.linalg.norm(f[3]) * 8).astype(np.float16)[None]
    out = oracle.latent_compress_ref(q, c.feats)
    s = q.astype(np.float64) @ f.T
    w = np.exp(s - s.max())
    w /= w.sum()
    assert w[0, 3] > 0.5
    np.testing.assert_allclose(out[0, 0], w[0] @ f, rtol=1e-12)
