"""Pin the oracle's Philox4x64-10 to numpy's independent implementation (CPU only).

numpy's Philox bit generator increments its 256-bit counter before producing a
block, so the block the oracle computes for counter c is what numpy returns
first when its state holds c - 1.
"""
import numpy as np
import pytest

import oracle
from oracle.philox import raw_words


def _numpy_block(counter, key):
    c = sum(int(w) << (64 * i) for i, w in enumerate(counter)) - 1
    c %= 1 << 256
    words = [(c >> (64 * i)) & ((1 << 64) - 1) for i in range(4)]
    bg = np.random.Philox(counter=np.array(words, dtype=np.uint64),
                          key=np.array(key, dtype=np.uint64))
    return [int(bg.random_raw()) for _ in range(4)]


def test_blocks_match_numpy():
    rng = np.random.default_rng(3)
    cases = [([0, 0, 0, 0], [0, 0]), ([1, 0, 0, 0], [0, 0]), ([0, 5, 7, 0], [0x5EED, 0]),
             ([2**64 - 1, 3, 0, 9], [12345, 678])]
    for _ in range(50):
        cases.append((list(rng.integers(0, 2**63, 4, dtype=np.uint64) * 2 + 1),
                      list(rng.integers(0, 2**63, 2, dtype=np.uint64))))
    ctrs = np.array([c for c, _ in cases], dtype=np.uint64)
    keys = np.array([k for _, k in cases], dtype=np.uint64)
    got = oracle.philox4x64_10(ctrs, keys)
    for i, (c, k) in enumerate(cases):
        assert [int(x) for x in got[i]] == _numpy_block(c, k), (c, k)


@pytest.mark.parametrize("purpose,row", [(oracle.ACCEPT, 3), (oracle.RESAMPLE, 31)])
def test_uniforms_match_numpy_generator(purpose, row):
    """u = (word >> 11) * 2^-53, which is numpy Generator.random() on the same words."""
    seed, offset, b = 0x5EED, 17, 2
    j = np.arange(0, 64)
    u = oracle.uniforms(seed, offset, b, purpose, row, j)
    for blk in range(0, 64, 4):
        ctr = [offset, b, (purpose << 32) | row, blk >> 2]
        c = sum(int(w) << (64 * i) for i, w in enumerate(ctr)) - 1
        words = [(c >> (64 * i)) & ((1 << 64) - 1) for i in range(4)]
        g = np.random.Generator(np.random.Philox(counter=np.array(words, dtype=np.uint64),
                                                 key=np.array([seed, 0], dtype=np.uint64)))
        np.testing.assert_array_equal(u[blk:blk + 4], g.random(4))
    w = raw_words(seed, offset, b, purpose, row, j)
    assert (u == (w >> np.uint64(11)).astype(np.float64) * 2.0 ** -53).all()
    assert (u >= 0).all() and (u < 1).all()
