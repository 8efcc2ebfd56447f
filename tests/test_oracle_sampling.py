"""Pins of the sampling acceptance oracle (CPU only).

The pages state the property the rule must have: the verified output follows
the target's distribution exactly (SpecFLASH README, "components" and its
overview).  The rule is pinned by exhaustive enumeration of that property; the
Philox-driven realisation is pinned to the enumerated law by chi-square tests,
and its per-draft thresholds and race weights are tied to the enumerated rule
deterministically.
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

V, K, L = 3, 3, 3


def _logits(kind, prefix, v=V):
    """A fixed float32 logit row per (model, prefix): a toy conditional model."""
    r = np.random.default_rng([99, kind, len(prefix), v] + list(prefix))
    return r.normal(0.0, 1.5 if kind == 0 else 1.0, v).astype(np.float32)


def _softmax(x):
    x = np.asarray(x, dtype=np.float64)
    e = np.exp(x - x.max())
    return e / e.sum()


def p_of(prefix, v=V):
    return _softmax(_logits(0, tuple(prefix), v))


def q_of(prefix, v=V):
    return _softmax(_logits(1, tuple(prefix), v))


PROMPT = (1, 0)


def ar_law(v=V, n=L):
    law = {}
    for ys in itertools.product(range(v), repeat=n):
        pr, pre = 1.0, list(PROMPT)
        for y in ys:
            pr *= p_of(pre, v)[y]
            pre.append(y)
        law[ys] = pr
    return law


def spec_law(v=V, kb=K, n=L):
    """Enumerate drafts x accept/reject branches x resampled token, cycle after cycle."""

    @lru_cache(maxsize=None)
    def rest(prefix, need):
        if need <= 0:
            return {(): 1.0}
        out = defaultdict(float)
        pre = list(prefix)
        for drafts in itertools.product(range(v), repeat=kb - 1):
            w = 1.0
            q_rows, p_rows = [], [p_of(pre, v)]
            for k, d in enumerate(drafts):
                q = q_of(pre + list(drafts[:k]), v)
                q_rows.append(q)
                w *= q[d]
                p_rows.append(p_of(pre + list(drafts[:k + 1]), v))
            acc, resid, bonus = oracle.sample_rule(p_rows, q_rows, drafts)
            branches = []
            keep = w
            for k in range(kb - 1):                 # first rejection at draft k+1
                for y in range(v):
                    branches.append((list(drafts[:k]) + [y], keep * (1 - acc[k]) * resid[k][y]))
                keep *= acc[k]
            for y in range(v):                      # all accepted, bonus token
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

    return rest(PROMPT, n)


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


def _run_spec(seed, rng, v=V, kb=K, n=L):
    """One speculative decode of n tokens with the Philox-driven oracle."""
    pre = list(PROMPT)
    gen = []
    cycle = 0
    while len(gen) < n:
        drafts, q_rows = [], []
        for k in range(kb - 1):
            q = q_of(pre + drafts, v)
            drafts.append(int(rng.choice(v, p=q)))      # the drafter samples d_k ~ q_k
            q_rows.append(_logits(1, tuple(pre + drafts[:-1]), v))
        t_rows = [_logits(0, tuple(pre + drafts[:k]), v) for k in range(kb)]
        acc, out = oracle.accept_sample_ref(np.array([t_rows]), np.array([q_rows]),
                                            np.array([drafts], np.int32), "f32", 1.0,
                                            seed, cycle)
        new = [int(t) for t in out[0, :acc[0] + 1]]
        gen += new
        pre += new
        cycle += 1
    return tuple(gen[:n])


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


# ------------------------------------------------------------------ deterministic ties
@pytest.mark.parametrize("v,kb", [(3, 3), (4, 3), (3, 4)])
def test_thresholds_and_race_weights_equal_the_rule(v, kb):
    """For every draft sequence of a small toy model, the Philox realisation's ratio
    thresholds exp(min(0, lambda_k)) equal the rule's min(1, p/q), and the row it races
    over (normalised) equals the rule's residual on a rejection, or p_{K-1} when every
    draft passes -- on each branch that some Philox offset takes.  Every branch (a
    rejection at each k, and all accepted) is reached."""
    seen = set()
    for drafts in itertools.product(range(v), repeat=kb - 1):
        pre = list(PROMPT)
        p_rows = [p_of(pre + list(drafts[:k]), v) for k in range(kb)]
        q_rows = [q_of(pre + list(drafts[:k]), v) for k in range(kb - 1)]
        acc, resid, bonus = oracle.sample_rule(p_rows, q_rows, drafts)
        t_rows = np.array([[_logits(0, tuple(pre + list(drafts[:k])), v) for k in range(kb)]])
        d_rows = np.array([[_logits(1, tuple(pre + list(drafts[:k])), v)
                            for k in range(kb - 1)]])
        for off in range(48):
            a, out, steps = oracle.accept_sample_ref(t_rows, d_rows, np.array([drafts], np.int32),
                                                     "f32", 1.0, 3, off, return_steps=True)
            st = steps[0]
            a = int(a[0])
            assert len(st["thresholds"]) == min(a + 1, kb - 1)
            for k, thr in enumerate(st["thresholds"]):
                assert abs(thr - acc[k]) <= 1e-12, (drafts, k, thr, acc[k])
            w = st["weights"] / st["weights"].sum()
            if a < kb - 1:
                assert st["row"] == a
                np.testing.assert_allclose(w, resid[a], rtol=0, atol=1e-12)
            else:
                assert st["row"] == kb - 1
                np.testing.assert_allclose(w, bonus, rtol=0, atol=1e-12)
            assert list(out[0, :a]) == list(drafts[:a])
            seen.add(a)
    assert seen == set(range(kb))


def test_zero_probability_drafts():
    """A draft the target gives probability 0 (a -inf logit) is never accepted, one the
    draft distribution gives 0 is always accepted, a whole masked stretch of the
    vocabulary is never drawn, and a race with no positive weight draws nothing (-1)."""
    rng = np.random.default_rng(31)
    Kb, Vb = 4, 40
    tl = rng.normal(0, 2, (1, Kb, Vb)).astype(np.float32)
    dl = (tl[:, :Kb - 1] + rng.normal(0, 1, (1, Kb - 1, Vb))).astype(np.float32)
    tl[0, :, 20:] = -np.inf                    # the target masks tokens 20..39
    dl[0, 1, 5] = -np.inf                      # the draft of d_2 gives token 5 no mass
    d = np.array([[25, 5, 7]], dtype=np.int32)
    for off in range(30):
        a, out, steps = oracle.accept_sample_ref(tl, dl, d, "f32", 1.0, 4, off,
                                                 return_steps=True)
        assert a[0] == 0 and steps[0]["thresholds"] == [0.0]
        assert 0 <= out[0, 0] < 20                    # the resample avoids the masked tokens
    d = np.array([[3, 5, 7]], dtype=np.int32)
    tl2 = tl.copy()
    dl2 = dl.copy()
    dl2[0, 0] = tl2[0, 0]                       # q_1 = p_0: d_1 always passes
    for off in range(30):
        a, out, steps = oracle.accept_sample_ref(tl2, dl2, d, "f32", 1.0, 4, off,
                                                 return_steps=True)
        assert a[0] >= 1
        assert steps[0]["thresholds"][1] == 1.0      # q_2(5) = 0 < p_1(5): ratio +inf
        assert a[0] >= 2
    assert oracle.race_ref(np.zeros(5), 1, 0, 0, 0)[0] == -1


# ------------------------------------------------------------------ large Monte-Carlo
def _mc_chunk(args):
    start, count, v, kb, n = args
    rng = np.random.default_rng([555, start])
    out = defaultdict(int)
    for s in range(start, start + count):
        out[_run_spec(s, rng, v, kb, n)] += 1
    return dict(out)


@pytest.mark.slow
def test_montecarlo_v4_hundred_thousand_runs():
    """10^5 Philox-driven decodes at V = 4 (K = 3, 3 tokens): chi-square against the
    enumerated law."""
    v, kb, n, runs = 4, 3, 3, 100_000
    law = ar_law(v, n)
    spec = spec_law(v, kb, n)
    assert max(abs(law[y] - spec[y]) for y in law) < 1e-12
    workers = max(1, min(8, len(os.sched_getaffinity(0))))
    per = runs // 40
    counts = defaultdict(int)
    with ProcessPoolExecutor(max_workers=workers) as ex:
        for part in ex.map(_mc_chunk, [(i * per, per, v, kb, n) for i in range(40)]):
            for key, c in part.items():
                counts[key] += c
    keys = sorted(law)
    obs = np.array([counts[k] for k in keys], dtype=np.float64)
    exp = np.array([law[k] for k in keys]) * runs
    assert obs.sum() == runs
    p = stats.chisquare(obs, exp).pvalue
    assert p > 1e-3, p


def test_stored_72b_verdicts_are_the_oracles():
    """The stored 72B sampling verdicts (tests/golden/sample_72b_1024.json, written by
    tests/golden/make_sample_72b.py from the oracle alone) still describe these inputs and
    this oracle: the input digest matches and two offsets re-run give the same verdicts."""
    import json
    import sys
    here = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
    sys.path.insert(0, here)
    import make_sample_72b as G
    with open(os.path.join(here, "sample_72b_1024.json")) as fh:
        gold = json.load(fh)
    s = G.inputs()
    assert G.digest(s) == gold["input_digest"]
    assert len(gold["offsets"]) == G.OFFSETS == 128
    for off in (0, 77):
        acc, out = oracle.accept_sample_ref(s.target_logits, s.draft_logits, s.drafts, s.dtype,
                                            s.temperature, s.seed, off)
        g = gold["offsets"][str(off)]
        assert list(acc) == g["accept_len"]
        assert [int(out[b, acc[b]]) for b in range(s.B)] == g["token"]
