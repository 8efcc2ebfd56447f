"""Reference latent visual compressor in float64 (test infrastructure).

SpecFLASH README, "components", compressor equation: C learnable query vectors
attend over the N visual features F_V of one image and return C latent
features, F_hat = softmax(C . F_V^T) . F_V, with the softmax over the N
features.  The printed formula carries no 1/sqrt(D) factor, so the default
scale is 1.
"""
import numpy as np

from .numerics import decode


def latent_compress_ref(queries, feats, dtype: str = "f16", scale: float = 1.0):
    """queries [C][D], feats [B][N][D] -> float64 [B][C][D]."""
    c = decode(queries, dtype)
    f = decode(feats, dtype)
    B = f.shape[0]
    out = np.zeros((B, c.shape[0], c.shape[1]))
    for b in range(B):
        s = scale * (c @ f[b].T)                 # [C][N]
        s = s - s.max(axis=1, keepdims=True)
        w = np.exp(s)
        w /= w.sum(axis=1, keepdims=True)
        out[b] = w @ f[b]
    return out
