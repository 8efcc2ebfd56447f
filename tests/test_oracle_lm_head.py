"""Pins of the LM-head oracle (CPU only): the logits against a dot product written out
element by element, the planted tokens, the margin that makes the argmax independent of
the accumulation precision, and the lowest-index rule on duplicated vocabulary rows."""
import numpy as np
import pytest

import oracle
import workloads as W


def test_logits_are_the_dot_products():
    rng = np.random.default_rng(1)
    li = W.make_lm_head(rng, B=2, K=3, hidden=24, V=37, dtype="bf16", chunk=8)
    got = oracle.lm_head_logits_ref(li.hidden_states, li.weight, "bf16", chunk=5)
    h = W.bf16_bits_to_f32(li.hidden_states)
    w = W.bf16_bits_to_f32(li.weight)
    for b in range(2):
        for i in range(3):
            for v in range(37):
                ref = 0.0
                for k in range(24):
                    ref += float(h[b, i, k]) * float(w[v, k])
                assert abs(got[b, i, v] - ref) <= 1e-12 * max(1.0, abs(ref))


@pytest.mark.parametrize("seed,B,K,hidden,V", [(0, 1, 16, 3584, 4096), (1, 3, 8, 512, 20000),
                                               (2, 2, 1, 256, 1000)])
def test_planted_tokens_with_margin(seed, B, K, hidden, V):
    li = W.make_lm_head(np.random.default_rng(seed), B=B, K=K, hidden=hidden, V=V)
    acc, out, t, logits = oracle.lm_head_greedy_ref(li.hidden_states, li.weight, li.drafts, "bf16")
    assert np.array_equal(t, li.planted_tok)
    assert np.array_equal(acc, li.planted_len)
    # the winner leads the runner-up by far more than any fp32 accumulation error
    # (|err| <= hidden * 2^-24 * sum |h_k w_k|), so every precision takes the same argmax
    top2 = np.sort(logits, axis=-1)[..., -2:]
    gap = top2[..., 1] - top2[..., 0]
    h = np.abs(W.bf16_bits_to_f32(li.hidden_states)).astype(np.float64)
    w = np.abs(W.bf16_bits_to_f32(li.weight[t.reshape(-1)])).astype(np.float64)
    bound = hidden * 2.0 ** -24 * (h.reshape(-1, hidden) * w).sum(axis=1).reshape(B, K)
    assert (gap > 100 * bound).all() and gap.min() > 1.0


def test_duplicated_rows_take_the_lowest_index():
    rng = np.random.default_rng(3)
    li = W.make_lm_head(rng, B=1, K=4, hidden=64, V=300)
    w = li.weight.copy()
    for t in li.planted_tok[0]:
        w[299] = w[t]                     # a later copy of every planted row ties with it
        acc, out, am, _ = oracle.lm_head_greedy_ref(li.hidden_states, w, li.drafts, "bf16")
        assert am[0][list(li.planted_tok[0]).index(t)] == min(t, 299)


def test_full_size_workload():
    """The 7B LM head (16 x 3584 against 152,064 x 3584): every row's planted token wins
    by a gap of several units."""
    li = W.make_workload_lm_head()
    acc, out, t, logits = oracle.lm_head_greedy_ref(li.hidden_states, li.weight, li.drafts, "bf16")
    assert np.array_equal(t, li.planted_tok) and np.array_equal(acc, li.planted_len)
    top2 = np.sort(logits, axis=-1)[..., -2:]
    assert (top2[..., 1] - top2[..., 0]).min() > 4.0
