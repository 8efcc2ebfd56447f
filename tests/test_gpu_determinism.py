"""Bitwise reproducibility: 100 identical calls of each acceptance rule and of the
compressor give identical outputs (every reduction runs in a fixed order; the acceptance
rules' integer outputs must not depend on scheduling)."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_helpers import i32, say, to_dev

pytestmark = pytest.mark.gpu
REPEATS = 100


def _same(fn, what):
    say(f"[determinism] {what} x{REPEATS}")
    first = [t.clone() for t in fn()]
    for _ in range(REPEATS - 1):
        got = fn()
        for a, b in zip(first, got):
            assert torch.equal(a, b), what


def test_greedy_repeats(gpu_lib):
    g = W.make_workload_greedy("qwen7b_25k", 0)
    lg, dr = to_dev(g.logits, g.dtype), i32(g.drafts)
    _same(lambda: gpu_lib.accept_greedy(lg, dr), "greedy 7B")


def test_sampling_repeats(gpu_lib):
    s = W.make_sample(np.random.default_rng(1), B=4, K=32, V=20000, dtype="bf16", seed=3,
                      offset=9)
    tl, dl, dr = to_dev(s.target_logits, "bf16"), to_dev(s.draft_logits, "bf16"), i32(s.drafts)
    _same(lambda: gpu_lib.accept_sample(tl, dl, dr, 1.0, 3, 9), "sampling")


def test_tree_sampling_repeats(gpu_lib):
    ts = W.make_tree_sample(np.random.default_rng(2), B=4, V=8000,
                            parents=W.make_tree_topology(np.random.default_rng(4)), dtype="bf16")
    tl, dl, tk = to_dev(ts.target_logits, "bf16"), to_dev(ts.draft_logits, "bf16"), i32(ts.tokens)
    _same(lambda: gpu_lib.accept_sample_tree(tl, dl, ts.parents, tk, 1.0, 5, 2), "tree sampling")


def test_compressor_repeats(gpu_lib):
    c = W.make_compress(np.random.default_rng(3), B=4, C=64, N=576, D=1024)
    qd, fs = to_dev(c.queries, "f16"), to_dev(c.feats, "f16")
    _same(lambda: (gpu_lib.latent_compress(qd, fs),), "compressor")
