"""Reference acceptance rules in float64 (test infrastructure).

Block layout: the block holds K positions, the anchor followed by drafts
d_1 .. d_{K-1} (VFlash-FM cycle figure: "anchor + 15 masks", 16 tokens
verified).  Target row i (0-based) is the target's prediction for the token
after block position i, so draft d_k is checked against target row k-1.

Outputs (both rules): ``accept_len[b]`` = number of drafts accepted, in
[0, K-1]; ``out_tokens[b]`` = the accepted drafts followed by the target's own
token (its correction, or a bonus token when every draft was accepted),
padded with -1 to K entries.  Committed tokens per cycle = accept_len + 1.
"""
import numpy as np

from .numerics import decode
from .philox import ACCEPT, RESAMPLE, uniforms


# ----------------------------------------------------------------------------- greedy

def accept_greedy_ref(logits, drafts, dtype: str):
    """Greedy verification (VFlash-FM page, caption of the cycle figure).

    t_i = argmax_j logits[b, i, j] with ties going to the lowest index (numpy's
    argmax returns the first maximum).  Drafts are accepted while d_k equals
    t_{k-1}; the target supplies t_a at the first disagreement (or after the
    last draft when all are accepted); everything after is discarded.
    Returns (accept_len int32 [B], out_tokens int32 [B][K], argmax int32 [B][K]).
    """
    x = decode(logits, dtype)
    B, K, _ = x.shape
    t = np.argmax(x, axis=-1).astype(np.int32)
    acc = np.zeros(B, dtype=np.int32)
    out = np.full((B, K), -1, dtype=np.int32)
    for b in range(B):
        a = 0
        while a < K - 1 and int(drafts[b][a]) == int(t[b, a]):
            a += 1
        acc[b] = a
        out[b, :a] = drafts[b][:a]
        out[b, a] = t[b, a]
    return acc, out, t


# ----------------------------------------------------------------------------- sampling

def _log_softmax_rows(x, T):
    z = x / T
    m = z.max(axis=-1, keepdims=True)
    return z - (m + np.log(np.exp(z - m).sum(axis=-1, keepdims=True)))


def sample_rule(p_rows, q_rows, drafts):
    """The standard speculative acceptance-rejection rule as probabilities.

    SpecFLASH README, "components" (the K drafts are verified in parallel by the
    target with the standard acceptance-rejection rule, so the output follows
    the target's distribution exactly); the rule itself is the one of the
    speculative-decoding and speculative-sampling papers the SpecFLASH page
    cites.

    p_rows [K][V]: target distributions p_0 .. p_{K-1}; q_rows [K-1][V]: row
    k-1 is the draft distribution q_k of d_k.  Returns, for k = 1 .. K-1, the
    acceptance probabilities a_k = min(1, p_{k-1}(d_k) / q_k(d_k)), the
    residual distribution used on a first rejection at k,
    norm(max(0, p_{k-1} - q_k)) (p_{k-1} itself if that residual is all zero),
    and the bonus distribution p_{K-1} used when every draft is accepted.
    A draft the target gives no probability is never accepted (0/0 counts as 0); one
    the draft distribution gives none but the target does has ratio +inf (accepted).
    """
    K = len(p_rows)
    acc = []
    resid = []
    for k in range(1, K):
        d = int(drafts[k - 1])
        p, q = p_rows[k - 1], q_rows[k - 1]
        if p[d] == 0:
            acc.append(0.0)
        else:
            acc.append(min(1.0, p[d] / q[d]) if q[d] > 0 else 1.0)
        r = np.maximum(0.0, p - q)
        resid.append(r / r.sum() if r.sum() > 0 else p / p.sum())
    return acc, resid, p_rows[K - 1]


def race_ref(r, seed, offset, b, row):
    """Draw from weights r >= 0 (not necessarily normalised) by an exponential race.

    Each j with r_j > 0 gets E_j = -ln(1 - u_j), u_j the RESAMPLE uniform of
    (b, row, j); the winner is argmin_j E_j / r_j, ties to the lowest j.  Since
    E_j / r_j is exponential with rate r_j, independently over j, the winner is
    j with probability r_j / sum(r).  Returns (winner, key of the winner,
    smallest relative gap between the two smallest keys).  With no positive weight
    there is nothing to draw: the winner is -1 (never a token id).
    """
    V = len(r)
    j = np.arange(V)
    u = uniforms(seed, offset, b, RESAMPLE, row, j)
    e = -np.log1p(-u)
    key = np.full(V, np.inf)
    pos = r > 0
    if not pos.any():
        return -1, float("inf"), float("inf")
    key[pos] = e[pos] / r[pos]
    w = int(np.argmin(key))
    srt = np.sort(key[pos])
    gap = (srt[1] - srt[0]) / srt[1] if len(srt) > 1 and srt[1] > 0 else np.inf
    return w, float(key[w]), float(gap)


def accept_sample_ref(target_logits, draft_logits, drafts, dtype: str, temperature: float,
                      seed: int, offset: int, return_diag: bool = False,
                      return_steps: bool = False):
    """Sampling verification with Philox uniforms and an exponential-race resample.

    For each sequence b and k = 1 .. K-1 in order:
      lambda_k = (lp[k-1, d_k] - lq[k-1, d_k]) / T - (Lp_{k-1} - Lq_k)
               = log(p_{k-1}(d_k) / q_k(d_k)), with L the row log-normalisers;
      u_k = uniform(ACCEPT, row k); accept d_k iff u_k < exp(min(0, lambda_k)).
    On the first rejection at k: race over r = max(0, p_{k-1} - q_k) on target
    row k-1 (over p_{k-1} if r is all zero).  With every draft accepted: race over
    p_{K-1} on target row K-1 for the bonus token.
    Returns (accept_len [B], out_tokens [B][K]) and, with ``return_diag``, the
    per-sequence minimum |u_k - exp(min(0, lambda_k))| over the tests taken and
    the race's relative top-2 gap; with ``return_steps``, per sequence the thresholds
    exp(min(0, lambda_k)) of the tests taken, the target row raced over and the race
    weights (unnormalised), in place of the diagnostics.
    """
    lp = decode(target_logits, dtype)
    lq = decode(draft_logits, dtype)
    B, K, V = lp.shape
    T = float(temperature)
    acc = np.zeros(B, dtype=np.int32)
    out = np.full((B, K), -1, dtype=np.int32)
    diag = []
    steps = []
    for b in range(B):
        logp = _log_softmax_rows(lp[b], T)      # [K][V]
        logq = _log_softmax_rows(lq[b], T)      # [K-1][V]
        a = K - 1
        margin = np.inf
        thresholds = []
        for k in range(1, K):
            d = int(drafts[b][k - 1])
            if not 0 <= d < V:                     # a token outside the vocabulary is rejected
                a = k - 1
                break
            u = float(uniforms(seed, offset, b, ACCEPT, k, np.array([0]))[0])
            if logp[k - 1, d] == -np.inf:           # p_{k-1}(d_k) = 0: never accepted
                thr = 0.0
            else:                                    # q_k(d_k) = 0 gives lam = +inf
                lam = logp[k - 1, d] - logq[k - 1, d]
                thr = np.exp(min(0.0, lam))
            margin = min(margin, abs(u - thr))
            thresholds.append(float(thr))
            if not u < thr:
                a = k - 1
                break
        if a < K - 1:
            row = a                                  # target row k-1 with k = a+1
            p = np.exp(logp[row])
            q = np.exp(logq[a])
            r = np.maximum(0.0, p - q)
            if not (r > 0).any():
                r = p
        else:
            row = K - 1
            r = np.exp(logp[row])
        tok, _, gap = race_ref(r, seed, offset, b, row)
        acc[b] = a
        out[b, :a] = drafts[b][:a]
        out[b, a] = tok
        diag.append((margin, gap))
        steps.append({"thresholds": thresholds, "row": row, "weights": r})
    if return_steps:
        return acc, out, steps
    if return_diag:
        return acc, out, diag
    return acc, out
