"""Pins of the tree sampling oracle (CPU only).

What the pages fix: the drafts are verified with the standard acceptance-rejection rule,
so the committed output follows the target's distribution exactly (SpecFLASH README,
"components"), and a tree-verified variant is reported next to the chain (VFlash-FM
results table, "Tree-60").  The tree rule is pinned by (i) exhaustive enumeration on small
trees: the law of the first committed tokens equals the autoregressive law, for siblings
drafted with and without replacement; (ii) on a chain it is the chain oracle bit for bit;
(iii) its Philox realisation's thresholds and race weights equal the enumerated rule's,
deterministically; (iv) a chi-square of the Philox realisation against the exact law.
"""
from collections import defaultdict
from concurrent.futures import ProcessPoolExecutor
from functools import lru_cache
import itertools
import os

import numpy as np
import pytest
from scipy import stats

import oracle

PROMPT = (2, 0)


def _logits(kind, prefix, v):
    """A fixed float32 logit row per (model, prefix): a toy conditional model."""
    r = np.random.default_rng([77, kind, len(prefix), v] + list(prefix))
    return r.normal(0.0, 1.4 if kind == 0 else 1.0, v).astype(np.float32)


def _softmax(x):
    x = np.asarray(x, dtype=np.float64)
    e = np.exp(x - x.max())
    return e / e.sum()


def p_of(prefix, v):
    return _softmax(_logits(0, tuple(prefix), v))


def q_of(prefix, v):
    return _softmax(_logits(1, tuple(prefix), v))


def ar_law(v, n):
    law = {}
    for ys in itertools.product(range(v), repeat=n):
        pr, pre = 1.0, list(PROMPT)
        for y in ys:
            pr *= p_of(pre, v)[y]
            pre.append(y)
        law[ys] = pr
    return law


def _node_paths(parents):
    """Token-index path (nodes from the first draft to node i) of every node."""
    K = len(parents) + 1
    paths = [[]]
    for i in range(1, K):
        paths.append(paths[int(parents[i - 1])] + [i])
    return paths


def draft_q(parents, toks, pre, v, i, replacement):
    """The distribution node i's token is drafted from: q after the path to its parent;
    without replacement, the tokens of its elder siblings are removed."""
    paths = _node_paths(parents)
    par = int(parents[i - 1])
    q = q_of(list(pre) + [toks[n] for n in paths[par]], v)
    if not replacement:
        q = q.copy()
        for s in range(1, i):
            if int(parents[s - 1]) == par:
                q[toks[s]] = 0.0
        q = q / q.sum()
    return q


def spec_tree_law(v, parents, n, replacement):
    """Exact law of the first n committed tokens under the tree rule, cycle after cycle."""
    K = len(parents) + 1
    paths = _node_paths(parents)
    ch = oracle.children_of(parents, K)

    def commit_law(pre, toks):
        """{committed tokens of one cycle: probability} given the drafted tokens."""
        out = defaultdict(float)

        def visit(u, acc_pr):
            pu = p_of(list(pre) + [toks[nn] for nn in paths[u]], v)
            kids = ch[u]
            qs = [draft_q(parents, toks, pre, v, c, replacement) for c in kids]
            thr, res = oracle.sample_tree_rule(pu, qs, [toks[c] for c in kids])
            reach = acc_pr
            for j, c in enumerate(kids):
                if thr[j] > 0:
                    visit(c, reach * thr[j])
                reach *= 1.0 - thr[j]
            if reach > 0:
                base = tuple(toks[nn] for nn in paths[u])
                for y in range(v):
                    if res[len(kids)][y] > 0:
                        out[base + (y,)] += reach * res[len(kids)][y]

        visit(0, 1.0)
        return out

    @lru_cache(maxsize=None)
    def rest(prefix, need):
        if need <= 0:
            return {(): 1.0}
        pre = list(prefix)
        total = defaultdict(float)
        for assign in itertools.product(range(v), repeat=K - 1):
            toks = [None] + list(assign)
            w = 1.0
            for i in range(1, K):
                w *= draft_q(parents, toks, pre, v, i, replacement)[toks[i]]
                if w == 0:
                    break
            if w == 0:
                continue
            for new, pr in commit_law(pre, toks).items():
                if len(new) >= need:
                    total[new[:need]] += w * pr
                else:
                    for cont, pc in rest(tuple(pre + list(new)), need - len(new)).items():
                        total[new + cont] += w * pr * pc
        return dict(total)

    return rest(PROMPT, n)


TREES = {
    "fork": [0, 0, 1],            # the anchor has two children; the first has one
    "star3": [0, 0, 0],           # three siblings
    "chain": [0, 1, 2],
}


@pytest.mark.parametrize("tree,replacement,v,n", [
    ("fork", True, 3, 3), ("fork", False, 3, 3), ("star3", True, 3, 2),
    ("star3", False, 3, 2), ("chain", True, 2, 4),
])
def test_tree_rule_is_lossless(tree, replacement, v, n):
    """Exact: the first n committed tokens follow the autoregressive law."""
    a = ar_law(v, n)
    s = spec_tree_law(v, TREES[tree], n, replacement)
    assert abs(sum(s.values()) - 1.0) < 1e-12
    for ys in a:
        assert abs(a[ys] - s.get(ys, 0.0)) < 1e-12, (ys, a[ys], s.get(ys))


def test_enumeration_detects_a_wrong_tree_rule():
    """The enumeration is sharp: testing every sibling against p_u (no residual update)
    is not lossless."""
    good = oracle.sample_tree_rule

    def bad(p_u, q_children, tokens):
        thr, res = good(p_u, q_children, tokens)
        pn = np.asarray(p_u) / np.sum(p_u)
        thr = [min(1.0, pn[int(x)] / q[int(x)]) for q, x in zip(q_children, tokens)]
        return thr, res

    oracle.sample_tree_rule = bad
    try:
        s = spec_tree_law(3, TREES["star3"], 2, True)
    finally:
        oracle.sample_tree_rule = good
    a = ar_law(3, 2)
    assert max(abs(a[y] - s.get(y, 0.0)) for y in a) > 1e-3


@pytest.mark.parametrize("seed", range(6))
def test_chain_topology_is_the_chain_rule(seed):
    """On a chain the tree oracle returns exactly the chain oracle's outputs."""
    rng = np.random.default_rng(seed)
    B, K, V = 5, int(rng.integers(2, 9)), int(rng.integers(20, 300))
    T = float(rng.choice([0.6, 1.0, 1.7]))
    tl = rng.normal(0, 3, (B, K, V)).astype(np.float32)
    dl = (tl[:, :K - 1] + rng.normal(0, 1, (B, K - 1, V))).astype(np.float32)
    if seed % 2:
        tl[:, :, : V // 3] = -np.inf           # masked tokens in the target
    drafts = rng.integers(0, V, (B, K - 1)).astype(np.int32)
    drafts[0, 0] = V + 3                         # outside the vocabulary
    parents = np.arange(K - 1, dtype=np.int32)
    for off in range(12):
        a1, o1 = oracle.accept_sample_ref(tl, dl, drafts, "f32", T, 1234, off)
        a2, o2, path = oracle.accept_sample_tree_ref(tl, dl, parents, drafts, "f32", T, 1234, off)
        np.testing.assert_array_equal(a1, a2)
        np.testing.assert_array_equal(o1, o2)
        for b in range(B):
            assert list(path[b, :a2[b] + 1]) == list(range(a2[b] + 1))
            assert (path[b, a2[b] + 1:] == -1).all()


@pytest.mark.parametrize("tree", ["fork", "star3"])
def test_sampler_thresholds_and_weights_equal_the_rule(tree):
    """For every token assignment of a small tree, the Philox realisation's thresholds at
    each test it takes equal the rule's, and the row it races over (normalised) is the
    rule's last residual at the node it stops at; every stop node is reached."""
    v = 3
    parents = TREES[tree]
    K = len(parents) + 1
    paths = _node_paths(parents)
    ch = oracle.children_of(parents, K)
    stops = set()
    for assign in itertools.product(range(v), repeat=K - 1):
        toks = [None] + list(assign)
        pre = list(PROMPT)
        t_rows = np.array([[_logits(0, tuple(pre + [toks[n] for n in paths[u]]), v)
                            for u in range(K)]])
        d_rows = np.array([[_logits(1, tuple(pre + [toks[n] for n in paths[int(parents[i - 1])]]), v)
                            for i in range(1, K)]])
        tk = np.array([assign], dtype=np.int32)
        rule = {}
        for u in range(K):
            pu = _softmax(t_rows[0, u])
            qs = [_softmax(d_rows[0, c - 1]) for c in ch[u]]
            rule[u] = oracle.sample_tree_rule(pu, qs, [toks[c] for c in ch[u]])
        for off in range(40):
            a, out, path, steps = oracle.accept_sample_tree_ref(
                t_rows, d_rows, np.array(parents, np.int32), tk, "f32", 1.0, 7, off,
                return_steps=True)
            st = steps[0]
            for c, thr, _ in st["tests"]:
                par = int(parents[c - 1])
                j = ch[par].index(c)
                assert abs(thr - rule[par][0][j]) <= 1e-12, (assign, c, thr, rule[par][0][j])
            u = st["stop"]
            w = st["weights"] / st["weights"].sum()
            np.testing.assert_allclose(w, rule[u][1][len(ch[u])], rtol=0, atol=1e-12)
            assert path[0, int(a[0])] == u
            stops.add(u)
    leaves = [u for u in range(K) if not ch[u]]
    assert set(leaves) <= stops and 0 in stops


def test_first_child_with_q_equal_p_is_always_accepted():
    rng = np.random.default_rng(3)
    K, V = 4, 40
    parents = np.array([0, 0, 1], np.int32)
    tl = rng.normal(0, 2, (3, K, V)).astype(np.float32)
    dl = rng.normal(0, 2, (3, K - 1, V)).astype(np.float32)
    dl[:, 0] = tl[:, 0]                         # node 1 drafted from p_0 itself
    tk = rng.integers(0, V, (3, K - 1)).astype(np.int32)
    for off in range(25):
        a, out, path = oracle.accept_sample_tree_ref(tl, dl, parents, tk, "f32", 1.0, 5, off)
        assert (path[:, 1] == 1).all() and (a >= 1).all()


def test_zero_probability_children():
    """A child whose token the current residual gives no mass is never accepted; a masked
    stretch of the target vocabulary is never drawn."""
    rng = np.random.default_rng(4)
    K, V = 4, 30
    parents = np.array([0, 0, 0], np.int32)
    tl = rng.normal(0, 2, (1, K, V)).astype(np.float32)
    dl = rng.normal(0, 2, (1, K - 1, V)).astype(np.float32)
    tl[0, 0, 10:20] = -np.inf
    tk = np.array([[12, 15, 19]], np.int32)       # all masked for the anchor's row
    for off in range(30):
        a, out, path, steps = oracle.accept_sample_tree_ref(tl, dl, parents, tk, "f32", 1.0, 2,
                                                            off, return_steps=True)
        assert a[0] == 0 and [t[1] for t in steps[0]["tests"]] == [0.0, 0.0, 0.0]
        assert not 10 <= out[0, 0] < 20


# ------------------------------------------------------------------ Philox Monte-Carlo
def _run_tree(args):
    start, count, v, parents, n = args
    rng = np.random.default_rng([909, start])
    K = len(parents) + 1
    paths = _node_paths(parents)
    counts = defaultdict(int)
    for s in range(start, start + count):
        pre = list(PROMPT)
        gen, cycle = [], 0
        while len(gen) < n:
            toks = [None]
            for i in range(1, K):
                toks.append(None)
                q = draft_q(parents, toks, pre, v, i, True)
                toks[i] = int(rng.choice(v, p=q))
            t_rows = [_logits(0, tuple(pre + [toks[nn] for nn in paths[u]]), v) for u in range(K)]
            d_rows = [_logits(1, tuple(pre + [toks[nn] for nn in paths[int(parents[i - 1])]]), v)
                      for i in range(1, K)]
            a, out, _ = oracle.accept_sample_tree_ref(np.array([t_rows]), np.array([d_rows]),
                                                      np.array(parents, np.int32),
                                                      np.array([toks[1:]], np.int32), "f32",
                                                      1.0, s, cycle)
            new = [int(t) for t in out[0, :a[0] + 1]]
            gen += new
            pre += new
            cycle += 1
        counts[tuple(gen[:n])] += 1
    return dict(counts)


def test_montecarlo_tree_philox_chi2():
    """20,000 Philox-driven decodes over the fork tree: chi-square against the exact law."""
    v, n, runs, parts = 3, 3, 20_000, 20
    parents = TREES["fork"]
    law = ar_law(v, n)
    workers = max(1, min(8, len(os.sched_getaffinity(0))))
    counts = defaultdict(int)
    with ProcessPoolExecutor(max_workers=workers) as ex:
        for part in ex.map(_run_tree, [(i * (runs // parts), runs // parts, v, parents, n)
                                       for i in range(parts)]):
            for k, c in part.items():
                counts[k] += c
    keys = sorted(law)
    obs = np.array([counts[k] for k in keys], dtype=np.float64)
    exp = np.array([law[k] for k in keys]) * runs
    assert obs.sum() == runs
    assert stats.chisquare(obs, exp).pvalue > 1e-3
