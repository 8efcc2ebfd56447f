"""Reference greedy verification of a draft tree, in float64 (test infrastructure).

The VFlash-FM results table reports a tree-verified variant ("Tree-60") next to chain
verification, and its demo cycle states the greedy rule for a chain: the target keeps
the drafts that match its own greedy choice and supplies the token at the first
disagreement.  On a tree the plainest reading of that rule, and the one that reduces
to it when the tree is a chain, is a walk from the anchor: at the current node the
target's greedy token is compared with the tokens of the node's children; a child
holding it is accepted and becomes the current node, and the walk stops at the first
node none of whose children holds it.  The target's token there is the correction.
Siblings normally carry distinct tokens; if two do, the lower-numbered child is taken.

Tree layout: node 0 is the anchor (block row 0); nodes 1 .. K-1 carry the drafts.
parents[b][i-1] is the parent of node i and tokens[b][i-1] its token; a parent has a
smaller number than its children.  Block row i of the verify pass is the target's
prediction after node i, over node i's ancestors (the mask rows of a tree: row i sees
node i and every ancestor of it).

Committing a tree cycle keeps the K/V rows of the accepted path: the block was appended
at positions ctx .. ctx+K-1 in node order, so the row of the path's j-th node moves from
ctx + path[j] to ctx + j (j = 1 .. a); then the context grows by a + 1 and the
correction anchors the next cycle, as for a chain.
"""
import numpy as np

from .kv import commit_ref
from .numerics import decode


def accept_greedy_tree_ref(logits, parents, tokens, dtype: str):
    """Greedy walk through a draft tree.

    Returns (accept_len int32 [B], out_tokens int32 [B][K], path int32 [B][K],
    argmax int32 [B][K]): the accepted depth a, the accepted nodes' tokens followed by
    the target's token at the last accepted node (padded with -1), the node numbers of
    the path from the anchor (path[0] = 0, padded with -1), and every row's greedy
    token (ties to the lowest index).
    """
    x = decode(logits, dtype)
    B, K, _ = x.shape
    t = np.argmax(x, axis=-1).astype(np.int32)
    acc = np.zeros(B, dtype=np.int32)
    out = np.full((B, K), -1, dtype=np.int32)
    path = np.full((B, K), -1, dtype=np.int32)
    for b in range(B):
        cur = 0
        walk = [0]
        while True:
            nxt = None
            for i in range(1, K):                      # lowest-numbered matching child
                if int(parents[b][i - 1]) == cur and int(tokens[b][i - 1]) == int(t[b, cur]):
                    nxt = i
                    break
            if nxt is None:
                break
            cur = nxt
            walk.append(cur)
        a = len(walk) - 1
        acc[b] = a
        path[b, :a + 1] = walk
        for j in range(1, a + 1):
            out[b, j - 1] = tokens[b][walk[j] - 1]
        out[b, a] = t[b, cur]
    return acc, out, path, t


def tree_commit_ref(k_cache, v_cache, page_table, ctx_lens, accept_len, out_tokens, path):
    """Close a tree cycle: move the accepted path's K/V rows into place, then commit.

    Caches are paged as for the verify pass (K [pages][Hkv][P][d], V [pages][Hkv][d][P]).
    Returns (k_cache, v_cache, new ctx_lens, next anchors) with the caches copied.
    """
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    P = kc.shape[2]
    for b in range(len(ctx_lens)):
        ctx = int(ctx_lens[b])
        for j in range(1, int(accept_len[b]) + 1):
            src = ctx + int(path[b][j])
            dst = ctx + j
            ps, pd = int(page_table[b][src // P]), int(page_table[b][dst // P])
            kc[pd, :, dst % P, :] = k_cache[ps, :, src % P, :]
            vc[pd, :, :, dst % P] = v_cache[ps, :, :, src % P]
    new_ctx, anchor = commit_ref(ctx_lens, accept_len, out_tokens)
    return kc, vc, new_ctx, anchor
