"""Pins of the greedy acceptance oracle (CPU only)."""
import json
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "vflash_cycle.json")


def test_worked_example_from_the_pages():
    """The VFlash-FM demo cycle: 7 drafts accepted, 'in' supplied, 8 tokens committed."""
    ex = json.load(open(GOLDEN))
    words = [ex["anchor"]] + ex["drafts"] + ex["target_greedy_known"]
    vocab = sorted(set(words))
    tid = {w: i for i, w in enumerate(vocab)}
    K = ex["block"]
    V = len(vocab)
    assert len(ex["drafts"]) == K - 1
    known = [tid[w] for w in ex["target_greedy_known"]]
    # rows past the first disagreement are not shown on the page; make them agree with
    # the later drafts, which the rule must ignore anyway
    later = [tid[w] for w in ex["drafts"][len(known):]] + [tid["in"]]
    greedy = (known + later)[:K]
    rng = np.random.default_rng(0)
    logits = rng.normal(0.0, 1.0, size=(1, K, V)).astype(np.float32)
    for i, t in enumerate(greedy):
        logits[0, i, t] = 10.0
    drafts = np.array([[tid[w] for w in ex["drafts"]]], dtype=np.int32)
    acc, out, am = oracle.accept_greedy_ref(logits, drafts, "f32")
    assert acc[0] == ex["accepted"] == 7
    committed = [vocab[t] for t in out[0, :acc[0] + 1]]
    assert committed == ex["committed"]
    assert committed == ex["autoregressive_tokens"]
    assert committed[-1] == ex["next_anchor"]
    assert (out[0, acc[0] + 1:] == -1).all()
    # closing the cycle: anchor + 7 accepted drafts keep their K/V rows, "in" anchors next
    ctx = 25119
    new_ctx, anchor = oracle.commit_ref(np.array([ctx], np.int32), acc, out)
    assert new_ctx[0] == ctx + ex["accepted"] + 1
    assert vocab[anchor[0]] == ex["next_anchor"]


def test_special_cases():
    rng = np.random.default_rng(1)
    K, V = 6, 40
    logits = rng.normal(0, 3, size=(1, K, V)).astype(np.float32)
    t = logits[0].argmax(axis=1)
    # first draft wrong -> exactly one token, the target's own choice (one AR step)
    d = np.array([[(t[0] + 1) % V] + list(t[1:K - 1])], dtype=np.int32)
    acc, out, _ = oracle.accept_greedy_ref(logits, d, "f32")
    assert acc[0] == 0 and out[0, 0] == t[0] and (out[0, 1:] == -1).all()
    # all drafts right -> K tokens, the last one from the last row
    d = np.array([list(t[:K - 1])], dtype=np.int32)
    acc, out, _ = oracle.accept_greedy_ref(logits, d, "f32")
    assert acc[0] == K - 1 and list(out[0]) == list(t[:K])


def test_lowest_index_ties():
    """Equal maxima: the lowest index is the target's choice, so a draft naming the later
    copy is rejected and the correction is the earlier one."""
    K, V = 3, 10
    logits = np.zeros((1, K, V), dtype=np.float32)
    logits[0, 0, [2, 7]] = 5.0
    logits[0, 1, [1, 4, 9]] = 5.0
    logits[0, 2, 0] = 1.0
    acc, out, am = oracle.accept_greedy_ref(logits, np.array([[7, 1]], np.int32), "f32")
    assert acc[0] == 0 and out[0, 0] == 2 and list(am[0]) == [2, 1, 0]
    acc, out, _ = oracle.accept_greedy_ref(logits, np.array([[2, 1]], np.int32), "f32")
    assert acc[0] == 2 and list(out[0]) == [2, 1, 0]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_planted_generator_agrees(dtype):
    """The generator plants the lowest-index maxima and the accepted length by
    construction; the oracle must recover both."""
    rng = np.random.default_rng(12)
    g = W.make_greedy(rng, B=40, K=8, V=3000, dtype=dtype)
    acc, out, am = oracle.accept_greedy_ref(g.logits, g.drafts, dtype)
    np.testing.assert_array_equal(am, g.planted_tok)
    np.testing.assert_array_equal(acc, g.planted_len)
    for b in range(g.B):
        a = acc[b]
        assert list(out[b, :a]) == list(g.drafts[b, :a])
        assert out[b, a] == g.planted_tok[b, a]


# ------------------------------------------------------------------ greedy == sequential

class ToyTarget:
    """Float64 toy decoder: embedding, one attention layer with a KV cache, LM head."""

    def __init__(self, seed, V=50, D=16):
        r = np.random.default_rng(seed)
        self.V, self.D = V, D
        self.E = r.normal(0, 1, (V, D))
        self.Wq = r.normal(0, 1 / np.sqrt(D), (D, D))
        self.Wk = r.normal(0, 1 / np.sqrt(D), (D, D))
        self.Wv = r.normal(0, 1 / np.sqrt(D), (D, D))
        self.Wo = r.normal(0, 1, (D, V))

    def proj(self, toks):
        x = self.E[np.asarray(toks)]
        return x, x @ self.Wq, x @ self.Wk, x @ self.Wv

    def sequential(self, prompt, n):
        seq = list(prompt)
        for _ in range(n):
            x, q, k, v = self.proj(seq)
            s = (k @ q[-1]) / np.sqrt(self.D)
            w = np.exp(s - s.max())
            o = (w @ v) / w.sum()
            seq.append(int(np.argmax((o + x[-1]) @ self.Wo)))
        return seq[len(prompt):]


def _speculative(model, prompt, n, K, drafter, P=4):
    """Speculative greedy decoding with the oracle's block attention and acceptance."""
    cap = len(prompt) + n + 2 * K + P
    pages = (cap + P - 1) // P
    kc = np.zeros((pages, 1, P, model.D), np.float64)
    vc = np.zeros((pages, 1, model.D, P), np.float64)
    table = np.arange(pages, dtype=np.int32)[None]
    committed = list(prompt)
    # prefill: context K/V of every committed token but the last (the first anchor)
    _, _, k, v = model.proj(committed[:-1])
    for j in range(len(committed) - 1):
        kc[j // P, 0, j % P] = k[j]
        vc[j // P, 0, :, j % P] = v[j]
    cycles = 0
    ctx, anchor = len(committed) - 1, committed[-1]
    while len(committed) - len(prompt) < n:
        # the cycle state comes from commit_ref alone; it must agree with the token list
        assert ctx == len(committed) - 1 and anchor == committed[-1]
        block = [anchor] + list(drafter(committed, K - 1))
        x, q, k, v = model.proj(block)
        for t in range(K):                     # write the block's K/V at [ctx, ctx+K)
            j = ctx + t
            kc[j // P, 0, j % P] = k[t]
            vc[j // P, 0, :, j % P] = v[t]
        inp = W.VerifyInputs(1, K, 1, 1, model.D, P, "f32", q[None, :, None, :], kc, vc,
                             table, np.array([ctx], np.int32), W.causal_mask(K))
        out, _ = oracle.verify_attention_ref(inp)
        logits = (out[0, :, 0, :] + x) @ model.Wo
        acc, toks, _ = oracle.accept_greedy_ref(logits[None], np.array([block[1:]], np.int32),
                                                "f32")
        committed += [int(t) for t in toks[0, :acc[0] + 1]]
        new_ctx, new_anchor = oracle.commit_ref(np.array([ctx], np.int32), acc, toks)
        ctx, anchor = int(new_ctx[0]), int(new_anchor[0])
        cycles += 1
    return committed[len(prompt):len(prompt) + n], cycles


@settings(max_examples=25, deadline=None)
@given(seed=st.integers(0, 10_000), K=st.integers(2, 7),
       kind=st.sampled_from(["perfect", "random", "adversarial", "prefix"]),
       cut=st.integers(0, 6))
def test_greedy_equals_sequential(seed, K, kind, cut):
    """Whatever the drafter proposes, greedy block verification commits exactly the
    tokens sequential argmax decoding produces (VFlash-FM page, "How VFlash-FM works":
    the accepted output is what the target alone would have generated)."""
    model = ToyTarget(seed)
    prompt = list(np.random.default_rng(seed + 1).integers(0, model.V, 5))
    n = 18
    truth = model.sequential(prompt, n + 2 * K)
    rng = np.random.default_rng(seed + 2)

    def drafter(committed, m):
        pos = len(committed) - len(prompt)
        right = truth[pos:pos + m]
        if kind == "perfect":
            return right
        if kind == "random":
            return list(rng.integers(0, model.V, m))
        if kind == "adversarial":        # right except the last draft of every block
            return right[:-1] + [(right[-1] + 1) % model.V]
        c = min(cut, m)                  # right for `cut` drafts, then wrong
        return right[:c] + [(t + 1) % model.V for t in right[c:]]

    got, cycles = _speculative(model, prompt, n, K, drafter)
    assert got == truth[:n]
    if kind == "perfect":
        assert cycles == -(-n // K)       # K tokens per target forward
