"""Reference sampling verification of a draft tree, in float64 (test infrastructure).

The VFlash-FM results table reports a tree-verified variant ("Tree-60"), and the SpecFLASH
README states that drafts are verified with the standard acceptance-rejection rule, so the
output follows the target's distribution exactly.  On a tree the plainest reading of that
rule, and the one that reduces to it on a chain, is recursive rejection over the children
of the current node: the children are tested in order, each against the residual that
the rejections of its elder siblings left; the first child that passes is accepted and
becomes the current node; if none passes (or the node is a leaf) the target's token is
drawn from the last residual (from the target's own row at a leaf).

With r_0 = p_u (the target's distribution after node u) and children c_1 < c_2 < ... of u,
child c_j carrying token x_j drawn from q_j (the draft distribution stored for c_j):

    test of c_j:  accept iff  u_j < min(1, r_{j-1}(x_j) / q_j(x_j))
                  (never when r_{j-1}(x_j) = 0; always when q_j(x_j) = 0 < r_{j-1}(x_j))
    rejection:    r_j = norm(max(0, r_{j-1} - q_j))   (p_u itself if that is all zero)

Each step is the standard rule with target r_{j-1} and proposal q_j, so the law of what
node u commits is p_u whatever the proposals are (they may differ between siblings, e.g.
siblings drawn without replacement).  The uniforms are the chain rule's: the test of node
c uses the ACCEPT uniform of row c, and the final draw races with the RESAMPLE uniforms of
the row of the node where the walk stopped.  On a chain this is accept_sample_ref exactly.

Tree layout as for the greedy tree walk: node 0 is the anchor (target row 0); nodes
1 .. K-1 carry drafts, parents[i-1] is the parent of node i (smaller than i) and
tokens[b][i-1] its token.  Target row u is the target's prediction after node u; draft
row i-1 is the distribution node i's token was drawn from.  One tree is shared by the
batch (its shape fixes the work plan), the tokens are per sequence.
"""
import numpy as np

from .accept import _log_softmax_rows, race_ref
from .numerics import decode
from .philox import ACCEPT, uniforms


def children_of(parents, K):
    """Children of every node, in increasing node order (parents[i-1] is node i's parent)."""
    ch = [[] for _ in range(K)]
    for i in range(1, K):
        par = int(parents[i - 1])
        if 0 <= par < i:
            ch[par].append(i)
    return ch


def sample_tree_rule(p_u, q_children, tokens):
    """The rule at one node, as probabilities: p_u [V] the target distribution, q_children
    [m][V] the draft distributions of the children in order, tokens [m] their tokens.
    Returns (thresholds [m], residuals [m+1][V] normalised): child j (0-based) is accepted
    with probability thresholds[j] when reached; residuals[j] is r_j (residuals[0] = p_u),
    and the draw after rejecting every child comes from residuals[m]."""
    r = np.asarray(p_u, dtype=np.float64)
    r = r / r.sum()
    res = [r]
    thr = []
    for q, x in zip(q_children, tokens):
        x = int(x)
        if r[x] == 0:
            thr.append(0.0)
        elif q[x] == 0:
            thr.append(1.0)
        else:
            thr.append(min(1.0, r[x] / q[x]))
        nxt = np.maximum(0.0, r - q)
        r = nxt / nxt.sum() if nxt.sum() > 0 else res[0]
        res.append(r)
    return thr, res


def accept_sample_tree_ref(target_logits, draft_logits, parents, tokens, dtype: str,
                           temperature: float, seed: int, offset: int,
                           return_steps: bool = False):
    """Recursive rejection over a draft tree with Philox uniforms.

    target_logits [B][K][V], draft_logits [B][K-1][V], parents [K-1] (shared), tokens
    [B][K-1].  Returns (accept_len [B], out_tokens [B][K], accept_path [B][K]): the accepted
    depth a, the accepted nodes' tokens then the drawn token (padded with -1), and the
    node path from the anchor (padded with -1).  With ``return_steps``, also per sequence
    the tests taken as (node, threshold, uniform), the node the walk stopped at and the
    race weights.
    """
    lp = decode(target_logits, dtype)
    lq = decode(draft_logits, dtype)
    B, K, V = lp.shape
    T = float(temperature)
    ch = children_of(parents, K)
    acc = np.zeros(B, dtype=np.int32)
    out = np.full((B, K), -1, dtype=np.int32)
    path = np.full((B, K), -1, dtype=np.int32)
    steps = []
    for b in range(B):
        logp = _log_softmax_rows(lp[b], T)                          # [K][V]
        logq = _log_softmax_rows(lq[b], T) if K > 1 else np.zeros((0, V))
        cur, walk, tests = 0, [0], []
        while True:
            p = np.exp(logp[cur])
            r = p                                     # r_0 = p_u (a distribution)
            race = p                                  # what the walk draws from if it stops
            nxt = None
            for j, c in enumerate(ch[cur]):
                x = int(tokens[b][c - 1])
                q = np.exp(logq[c - 1])
                u = float(uniforms(seed, offset, b, ACCEPT, c, np.array([0]))[0])
                if not 0 <= x < V or r[x] == 0:       # outside the vocabulary, or r(x) = 0
                    thr = 0.0
                elif j == 0:                          # against p_u: the chain's log form
                    thr = float(np.exp(min(0.0, logp[cur, x] - logq[c - 1, x])))
                elif q[x] == 0:
                    thr = 1.0
                else:
                    thr = min(1.0, r[x] / q[x])
                tests.append((c, thr, u))
                if u < thr:
                    nxt = c
                    break
                race = np.maximum(0.0, r - q)         # drawn from as it is (unnormalised)
                if not (race > 0).any():
                    race = p
                r = race / race.sum()
            if nxt is None:
                break
            cur = nxt
            walk.append(cur)
        r = race
        tok, _, _ = race_ref(race, seed, offset, b, cur)
        a = len(walk) - 1
        acc[b] = a
        path[b, :a + 1] = walk
        for j in range(1, a + 1):
            out[b, j - 1] = tokens[b][walk[j] - 1]
        out[b, a] = tok
        steps.append({"tests": tests, "stop": cur, "weights": r})
    if return_steps:
        return acc, out, path, steps
    return acc, out, path
