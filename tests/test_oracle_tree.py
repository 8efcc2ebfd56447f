"""Pins of the tree-verification oracle (CPU only).

The tree walk is pinned to the chain rule (a chain is a tree), to a worked example
written out by hand, to the paths the input generator plants, and to an independent
"every edge on the root path matches" formulation; tree-masked attention is pinned to
plain causal attention over each node's root path; the tree commit is pinned to the
positions it must fill and to the chain commit.
"""
import numpy as np
import pytest

import oracle
import workloads as W


def _tree_case(rows_greedy, parents, tokens, V):
    """Logits [1][K][V] whose row i has its maximum at rows_greedy[i]."""
    K = len(parents) + 1
    rng = np.random.default_rng(5)
    x = rng.normal(0, 1, size=(1, K, V)).astype(np.float32)
    for i, t in enumerate(rows_greedy):
        x[0, i, t] = 10.0
    return x, np.array([parents], np.int32), np.array([tokens], np.int32)


def test_worked_example():
    # node:      1  2  3  4  5  6
    parents = [0, 0, 1, 1, 2, 4]
    tokens = [3, 5, 2, 4, 1, 0]
    # greedy tokens of rows 0..6: anchor -> 3 (node 1), node 1 -> 4 (node 4),
    # node 4 -> 0 (node 6), node 6 -> 2 (a leaf: the correction)
    x, p, t = _tree_case([3, 4, 1, 1, 0, 1, 2], parents, tokens, 6)
    acc, out, path, am = oracle.accept_greedy_tree_ref(x, p, t, "f32")
    assert acc[0] == 3
    assert list(path[0]) == [0, 1, 4, 6, -1, -1, -1]
    assert list(out[0]) == [3, 4, 0, 2, -1, -1, -1]
    # anchor -> 5 (node 2), node 2 -> 0 but node 5 holds 1: stop with correction 0
    x, p, t = _tree_case([5, 4, 0, 1, 0, 1, 2], parents, tokens, 6)
    acc, out, path, _ = oracle.accept_greedy_tree_ref(x, p, t, "f32")
    assert acc[0] == 1 and list(path[0][:3]) == [0, 2, -1] and list(out[0][:3]) == [5, 0, -1]
    # no child of the anchor matches: one token, the target's own
    x, p, t = _tree_case([4, 4, 0, 1, 0, 1, 2], parents, tokens, 6)
    acc, out, path, _ = oracle.accept_greedy_tree_ref(x, p, t, "f32")
    assert acc[0] == 0 and path[0][0] == 0 and out[0][0] == 4 and (out[0][1:] == -1).all()
    # two siblings with the same token: the lower-numbered one is taken
    x, p, t = _tree_case([3, 1, 1, 1, 1, 1, 1], parents, [3, 3, 2, 4, 1, 0], 6)
    acc, out, path, _ = oracle.accept_greedy_tree_ref(x, p, t, "f32")
    assert list(path[0][:3]) == [0, 1, -1] and list(out[0][:2]) == [3, 1]


@pytest.mark.parametrize("K,V,seed", [(5, 50, 0), (16, 300, 1), (64, 1000, 2)])
def test_chain_is_the_chain_rule(K, V, seed):
    g = W.make_greedy(np.random.default_rng(seed), B=6, K=K, V=V, dtype="f32")
    parents = np.tile(W.chain_topology(K - 1), (6, 1))
    acc, out, path, am = oracle.accept_greedy_tree_ref(g.logits, parents, g.drafts, "f32")
    acc2, out2, am2 = oracle.accept_greedy_ref(g.logits, g.drafts, "f32")
    assert np.array_equal(acc, acc2) and np.array_equal(out, out2) and np.array_equal(am, am2)
    for b in range(6):
        a = int(acc[b])
        assert list(path[b][:a + 1]) == list(range(a + 1)) and (path[b][a + 1:] == -1).all()


@pytest.mark.parametrize("seed", range(6))
def test_planted_paths(seed):
    rng = np.random.default_rng(100 + seed)
    parents = W.make_tree_topology(rng, (4, 6, 5, 3, 2) if seed % 2 else W.TREE60_LEVELS)
    ti = W.make_tree_greedy(rng, B=8, V=500, parents=parents, dtype="bf16")
    acc, out, path, am = oracle.accept_greedy_tree_ref(ti.logits, ti.parents, ti.tokens, "bf16")
    assert np.array_equal(am, ti.planted_tok)
    assert np.array_equal(acc, ti.planted_len)
    assert np.array_equal(path, ti.planted_path)


def _matched_nodes(parents, tokens, t):
    """Nodes whose every edge from the anchor carries the parent's greedy token."""
    K = len(parents) + 1
    ok = [True] + [False] * (K - 1)
    for i in range(1, K):
        u = int(parents[i - 1])
        ok[i] = ok[u] and int(tokens[i - 1]) == int(t[u])
    return [i for i in range(K) if ok[i]]


def _depth(parents, i):
    d = 0
    while i:
        i = int(parents[i - 1])
        d += 1
    return d


@pytest.mark.parametrize("seed", range(4))
def test_matches_the_path_formulation(seed):
    """With distinct sibling tokens the matched nodes form one root path; the walk ends
    at its deepest node."""
    rng = np.random.default_rng(200 + seed)
    parents = W.make_tree_topology(rng, W.TREE60_LEVELS)
    ti = W.make_tree_greedy(rng, B=6, V=64, parents=parents, dtype="f32")
    acc, out, path, am = oracle.accept_greedy_tree_ref(ti.logits, ti.parents, ti.tokens, "f32")
    for b in range(6):
        nodes = _matched_nodes(parents, ti.tokens[b], am[b])
        depths = sorted(_depth(parents, i) for i in nodes)
        assert depths == list(range(len(nodes)))          # one node per depth: a path
        end = max(nodes, key=lambda i: _depth(parents, i))
        assert acc[b] == len(nodes) - 1 and path[b][acc[b]] == end
        assert sorted(path[b][:acc[b] + 1]) == sorted(nodes)
        assert out[b][acc[b]] == am[b][end]
        for j in range(1, acc[b] + 1):
            assert out[b][j - 1] == ti.tokens[b][path[b][j] - 1]


def test_tree_mask_rows():
    rng = np.random.default_rng(7)
    parents = W.make_tree_topology(rng, W.TREE60_LEVELS)
    rows = W.tree_mask(parents)
    for i in range(len(parents) + 1):
        anc, j = {i}, i
        while j:
            j = int(parents[j - 1])
            anc.add(j)
        assert {t for t in range(64) if (int(rows[i]) >> t) & 1} == anc
    assert np.array_equal(W.tree_mask(W.chain_topology(15)), W.causal_mask(16))


def test_tree_attention_is_path_attention():
    """Row i of tree-masked attention equals causal attention over the context followed
    by node i's root path (the tokens an autoregressive decode would have seen)."""
    rng = np.random.default_rng(11)
    parents = W.make_tree_topology(rng, (3, 4, 3, 2))
    K = len(parents) + 1
    ctx = 37
    inp = W.make_verify(rng, B=1, K=K, Hq=4, Hkv=2, D=64, ctx_lens=[ctx], P=16, dtype="f32",
                        shuffle=True, mask=W.tree_mask(parents))
    out, lse = oracle.verify_attention_ref(inp)
    P = inp.P
    for i in range(K):
        chain = [i]
        while chain[-1]:
            chain.append(int(parents[chain[-1] - 1]))
        chain = chain[::-1]                                 # anchor .. i
        n = ctx + len(chain)
        pos = list(range(ctx)) + [ctx + c for c in chain]
        pages = (n + P - 1) // P
        kc = np.zeros((pages, 2, P, 64), np.float32)
        vc = np.zeros((pages, 2, 64, P), np.float32)
        for j, src in enumerate(pos):
            ps = inp.page_table[0][src // P]
            kc[j // P, :, j % P, :] = inp.k_cache[ps, :, src % P, :]
            vc[j // P, :, :, j % P] = inp.v_cache[ps, :, :, src % P]
        sub = W.VerifyInputs(1, len(chain), 4, 2, 64, P, "f32", inp.q[:, chain], kc, vc,
                             np.arange(pages, dtype=np.int32)[None, :],
                             np.array([ctx], np.int32), W.causal_mask(len(chain)))
        o2, l2 = oracle.verify_attention_ref(sub)
        np.testing.assert_allclose(out[0, i], o2[0, -1], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(lse[0, i], l2[0, -1], rtol=1e-12, atol=1e-12)


def test_tree_commit():
    rng = np.random.default_rng(13)
    parents = W.make_tree_topology(rng, (4, 6, 5, 3, 2))
    K = len(parents) + 1
    B = 4
    ctx = np.array([5, 40, 17, 0], np.int32)
    inp = W.make_verify(rng, B=B, K=K, Hq=2, Hkv=2, D=64, ctx_lens=ctx, P=16, dtype="f32",
                        shuffle=True)
    ti = W.make_tree_greedy(rng, B=B, V=50, parents=parents, dtype="f32")
    acc, out, path, _ = oracle.accept_greedy_tree_ref(ti.logits, ti.parents, ti.tokens, "f32")
    kc, vc, new_ctx, anchor = oracle.tree_commit_ref(inp.k_cache, inp.v_cache, inp.page_table,
                                                     ctx, acc, out, path)
    c2, a2 = oracle.commit_ref(ctx, acc, out)
    assert np.array_equal(new_ctx, c2) and np.array_equal(anchor, a2)
    P = inp.P
    touched = set()
    for b in range(B):
        for j in range(int(acc[b]) + 1):
            dst, src = ctx[b] + j, ctx[b] + path[b][j]
            pd, ps = inp.page_table[b][dst // P], inp.page_table[b][src // P]
            assert np.array_equal(kc[pd, :, dst % P, :], inp.k_cache[ps, :, src % P, :])
            assert np.array_equal(vc[pd, :, :, dst % P], inp.v_cache[ps, :, :, src % P])
            touched.add((int(pd), int(dst % P)))
    for pg in range(kc.shape[0]):
        for sl in range(P):
            if (pg, sl) not in touched:
                assert np.array_equal(kc[pg, :, sl, :], inp.k_cache[pg, :, sl, :])
                assert np.array_equal(vc[pg, :, :, sl], inp.v_cache[pg, :, :, sl])
    # a chain path moves nothing
    chain = np.tile(np.arange(K, dtype=np.int32), (B, 1))
    kc, vc, _, _ = oracle.tree_commit_ref(inp.k_cache, inp.v_cache, inp.page_table, ctx,
                                          np.full(B, K - 1, np.int32), chain, chain)
    assert np.array_equal(kc, inp.k_cache) and np.array_equal(vc, inp.v_cache)
