"""Pins of the sampling acceptance oracle (CPU only).

The pages state the property the rule must have: the verified output follows
the target's distribution exactly (SpecFLASH README, "components" and its
overview).  The rule is pinned by exhaustive enumeration of that property; the
Philox-driven realisation is pinned to the enumerated law by chi-square tests.
"""
from collections import defaultdict
from functools import lru_cache
import itertools

import numpy as np
import pytest
from scipy import stats

import oracle

V, K, L = 3, 3, 3


def _logits(kind, prefix):
    """A fixed float32 logit row per (model, prefix): a toy conditional model."""
    r = np.random.default_rng([99, kind, len(prefix)] + list(prefix))
    return r.normal(0.0, 1.5 if kind == 0 else 1.0, V).astype(np.float32)


def _softmax(x):
    x = np.asarray(x, dtype=np.float64)
    e = np.exp(x - x.max())
    return e / e.sum()


def p_of(prefix):
    return _softmax(_logits(0, tuple(prefix)))


def q_of(prefix):
    return _softmax(_logits(1, tuple(prefix)))


PROMPT = (1, 0)


def ar_law():
    law = {}
    for ys in itertools.product(range(V), repeat=L):
        pr, pre = 1.0, list(PROMPT)
        for y in ys:
            pr *= p_of(pre)[y]
            pre.append(y)
        law[ys] = pr
    return law


def spec_law():
    """Enumerate drafts x accept/reject branches x resampled token, cycle after cycle."""

    @lru_cache(maxsize=None)
    def rest(prefix, need):
        if need <= 0:
            return {(): 1.0}
        out = defaultdict(float)
        pre = list(prefix)
        for drafts in itertools.product(range(V), repeat=K - 1):
            w = 1.0
            q_rows, p_rows = [], [p_of(pre)]
            for k, d in enumerate(drafts):
                q = q_of(pre + list(drafts[:k]))
                q_rows.append(q)
                w *= q[d]
                p_rows.append(p_of(pre + list(drafts[:k + 1])))
            acc, resid, bonus = oracle.sample_rule(p_rows, q_rows, drafts)
            branches = []
            keep = w
            for k in range(K - 1):                  # first rejection at draft k+1
                for y in range(V):
                    branches.append((list(drafts[:k]) + [y], keep * (1 - acc[k]) * resid[k][y]))
                keep *= acc[k]
            for y in range(V):                      # all accepted, bonus token
                branches.append((list(drafts) + [y], keep * bonus[y]))
            for new, pr in branches:
                if pr == 0:
                    continue
                if len(new) >= need:
                    out[tuple(new[:need])] += pr
                else:
                    for cont, pc in rest(tuple(pre + new), need - len(new)).items():
                        out[tuple(new) + cont] += pr * pc
        return dict(out)

    return rest(PROMPT, L)


def test_enumeration_is_lossless():
    """Exact: the law of the first L committed tokens equals the autoregressive law."""
    a, s = ar_law(), spec_law()
    assert set(a) == set(s)
    assert abs(sum(s.values()) - 1) < 1e-12
    for ys in a:
        assert abs(a[ys] - s[ys]) < 1e-12, (ys, a[ys], s[ys])


def test_enumeration_detects_a_wrong_rule():
    """The enumeration is sharp: a rule whose residual is max(0, q - p) is not lossless."""
    good = oracle.sample_rule

    def bad(p_rows, q_rows, drafts):
        acc, _, bonus = good(p_rows, q_rows, drafts)
        res = []
        for k in range(len(drafts)):
            r = np.maximum(0, q_rows[k] - p_rows[k])
            res.append(r / r.sum())
        return acc, res, bonus

    oracle.sample_rule = bad
    try:
        s = spec_law()
    finally:
        oracle.sample_rule = good
    a = ar_law()
    assert max(abs(a[y] - s[y]) for y in a) > 1e-3


def _run_spec(seed, rng):
    """One speculative decode of L tokens with the Philox-driven oracle."""
    pre = list(PROMPT)
    gen = []
    cycle = 0
    while len(gen) < L:
        drafts, q_rows = [], []
        for k in range(K - 1):
            q = q_of(pre + drafts)
            drafts.append(int(rng.choice(V, p=q)))      # the drafter samples d_k ~ q_k
            q_rows.append(_logits(1, tuple(pre + drafts[:-1])))
        t_rows = [_logits(0, tuple(pre + drafts[:k])) for k in range(K)]
        acc, out = oracle.accept_sample_ref(np.array([t_rows]), np.array([q_rows]),
                                            np.array([drafts], np.int32), "f32", 1.0,
                                            seed, cycle)
        new = [int(t) for t in out[0, :acc[0] + 1]]
        gen += new
        pre += new
        cycle += 1
    return tuple(gen[:L])


def test_montecarlo_philox_realisation_chi2():
    """The Philox + exponential-race realisation follows the exact law (chi-square)."""
    n = 6000
    rng = np.random.default_rng(2024)
    counts = defaultdict(int)
    for s in range(n):
        counts[_run_spec(s, rng)] += 1
    law = ar_law()
    keys = sorted(law)
    obs = np.array([counts[k] for k in keys], dtype=np.float64)
    exp = np.array([law[k] for k in keys]) * n
    p = stats.chisquare(obs, exp).pvalue
    assert p > 1e-3, p


def test_race_draws_proportionally():
    r = np.array([0.1, 0.0, 0.5, 0.2, 0.2, 1e-3])
    n = 8000
    wins = np.zeros(len(r))
    for off in range(n):
        w, key, gap = oracle.race_ref(r, 77, off, 0, 5)
        wins[w] += 1
    assert wins[1] == 0
    pos = r > 0
    exp = r[pos] / r.sum() * n
    assert stats.chisquare(wins[pos], exp).pvalue > 1e-3


def test_q_equal_p_accepts_everything():
    rng = np.random.default_rng(5)
    Kb, Vb = 6, 50
    tl = rng.normal(0, 3, (4, Kb, Vb)).astype(np.float32)
    dl = tl[:, :Kb - 1, :].copy()
    drafts = rng.integers(0, Vb, (4, Kb - 1)).astype(np.int32)
    for off in range(20):
        acc, out = oracle.accept_sample_ref(tl, dl, drafts, "f32", 1.0, 1, off)
        assert (acc == Kb - 1).all()
        np.testing.assert_array_equal(out[:, :Kb - 1], drafts)
        assert ((out[:, Kb - 1] >= 0) & (out[:, Kb - 1] < Vb)).all()


def test_temperature_scales_logits():
    """T enters only through logits / T: scaling logits and T together changes nothing."""
    rng = np.random.default_rng(8)
    tl = rng.normal(0, 3, (3, 5, 40)).astype(np.float32)
    dl = (tl[:, :4] + rng.normal(0, 1, (3, 4, 40))).astype(np.float32)
    d = rng.integers(0, 40, (3, 4)).astype(np.int32)
    for off in range(10):
        a1, o1 = oracle.accept_sample_ref(tl, dl, d, "f32", 0.5, 9, off)
        a2, o2 = oracle.accept_sample_ref(tl * 2, dl * 2, d, "f32", 1.0, 9, off)
        np.testing.assert_array_equal(a1, a2)
        np.testing.assert_array_equal(o1, o2)


def test_out_of_vocabulary_draft_is_rejected():
    rng = np.random.default_rng(6)
    tl = rng.normal(0, 3, (1, 5, 30)).astype(np.float32)
    dl = tl[:, :4].copy()                       # q == p: in-vocabulary drafts always pass
    for bad in (-1, 30, 10**6):
        d = np.array([[3, 4, bad, 5]], dtype=np.int32)
        acc, out = oracle.accept_sample_ref(tl, dl, d, "f32", 1.0, 2, 0)
        assert acc[0] == 2 and list(out[0, :2]) == [3, 4] and 0 <= out[0, 2] < 30
