"""Philox4x64-10 counter-based generator and the sampling rule's uniforms (test infrastructure).

Philox4x64 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as
1, 2, 3", SC'11): a 4-word counter and a 2-word key.  One round multiplies
counter words 0 and 2 by the two multipliers into 128-bit products, then
rebuilds the counter as (hi(M1*c2) ^ c1 ^ k0, lo(M1*c2), hi(M0*c0) ^ c3 ^ k1,
lo(M0*c0)); the key is bumped by the two Weyl constants between rounds.  Ten
rounds.  The multipliers and Weyl constants are the ones the paper gives for
the 4x64 variant; they are pinned against numpy's independent Philox
implementation in the tests.

Counter layout for the acceptance rule (the pages fix none; this is the
library's convention):

    key     = (seed, 0)
    counter = (offset, b, (purpose << 32) | row, j >> 2),  output word j & 3
    purpose ACCEPT   = 0: row = draft index k (1 .. K-1), j = 0
    purpose RESAMPLE = 1: row = index of the target row raced over, j = token id
    uniform u = (word >> 11) * 2**-53  in [0, 1)
"""
import numpy as np

M0 = np.uint64(0xD2E7470EE14C6C93)
M1 = np.uint64(0xCA5A826395121157)
W0 = np.uint64(0x9E3779B97F4A7C15)
W1 = np.uint64(0xBB67AE8584CAA73B)
_LO = np.uint64(0xFFFFFFFF)
_S32 = np.uint64(32)

ACCEPT = 0
RESAMPLE = 1


def _mulhilo(a, b):
    """128-bit product of uint64 arrays as (hi, lo), by 32-bit limbs."""
    a0, a1 = a & _LO, a >> _S32
    b0, b1 = b & _LO, b >> _S32
    p00, p01, p10, p11 = a0 * b0, a0 * b1, a1 * b0, a1 * b1
    mid = (p00 >> _S32) + (p01 & _LO) + (p10 & _LO)
    hi = p11 + (p01 >> _S32) + (p10 >> _S32) + (mid >> _S32)
    lo = (mid << _S32) | (p00 & _LO)
    return hi, lo


def philox4x64_10(counter, key):
    """Philox4x64-10 of counters [..., 4] under keys [..., 2] -> words [..., 4] (uint64)."""
    with np.errstate(over="ignore"):
        c = np.array(counter, dtype=np.uint64, copy=True)
        k = np.array(key, dtype=np.uint64, copy=True)
        c0, c1, c2, c3 = c[..., 0], c[..., 1], c[..., 2], c[..., 3]
        k0, k1 = k[..., 0] + np.zeros_like(c0), k[..., 1] + np.zeros_like(c0)
        for r in range(10):
            if r:
                k0 = k0 + W0
                k1 = k1 + W1
            hi0, lo0 = _mulhilo(M0, c0)
            hi1, lo1 = _mulhilo(M1, c2)
            c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
        return np.stack([c0, c1, c2, c3], axis=-1)


def raw_words(seed, offset, b, purpose, row, j):
    """The 64-bit words feeding uniforms for token ids ``j`` (array)."""
    j = np.asarray(j, dtype=np.uint64)
    ctr = np.zeros(j.shape + (4,), dtype=np.uint64)
    ctr[..., 0] = np.uint64(offset)
    ctr[..., 1] = np.uint64(b)
    ctr[..., 2] = (np.uint64(purpose) << _S32) | np.uint64(row)
    ctr[..., 3] = j >> np.uint64(2)
    key = np.array([seed, 0], dtype=np.uint64)
    words = philox4x64_10(ctr, key)
    return np.take_along_axis(words, (j & np.uint64(3)).astype(np.int64)[..., None],
                              axis=-1)[..., 0]


def uniforms(seed, offset, b, purpose, row, j):
    """u = (word >> 11) * 2^-53 for token ids ``j``."""
    w = raw_words(seed, offset, b, purpose, row, j)
    return (w >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)
