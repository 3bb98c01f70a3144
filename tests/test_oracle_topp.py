"""Pins of the oracle's top-p cut ("KV Cache + Speculative Decoding" 7.5 and
its answer on top-p: the target row is cut to its own top-p set and
renormalised; whatever the draft sampled from is q; the rule stays exact).

Reading: tokens are ranked by logit; a token is kept iff the mass ranked
strictly above it is below top_p, and the top logit's tokens are always kept.
What fixes it without trusting the oracle:
  * the usual nucleus recipe written independently here (sort ascending,
    cumulative sum, drop what lies at or below 1 - top_p), on rows without
    ties, away from the boundary;
  * the threshold form on rows with ties: the cut is the largest logit v with
    mass(l >= v) >= top_p, everything at or above it kept, by brute force;
  * top_p >= 1 and NaN change nothing, bit for bit;
  * top_p -> 0 is the greedy limit (one-hot at the argmax);
  * every emitted position follows the cut, renormalised target
    (chi-square over 10^6 rounds), with and without a temperature, for a
    draft that samples its own cut distribution;
  * the boundary flag: a cut decided within 1e-6 of top_p sets near_pos.
"""
import numpy as np
import pytest
from scipy.special import softmax

import oracle
import workloads as W
from .test_oracle_sampler import U_MAX, _rows, chi2_pvalue


def _nucleus_ascending(p, top_p):
    """Kept mask by the common recipe: ascending sort, cumulative sum, drop
    entries whose cumulative mass is <= 1 - top_p, keep at least the top one."""
    order = np.argsort(p, kind="stable")
    csum = np.cumsum(p[order])
    drop_sorted = csum <= 1.0 - top_p
    drop_sorted[-1] = False
    keep = np.ones(p.size, dtype=bool)
    keep[order[drop_sorted]] = False
    return keep


def test_cut_matches_the_ascending_cumsum_recipe():
    rng = np.random.default_rng(51)
    checked = 0
    for trial in range(300):
        V = int(rng.integers(2, 400))
        row = (rng.standard_normal(V) * rng.uniform(0.5, 4)).astype(np.float32)
        if np.unique(row).size != V:
            continue
        T = float(rng.choice([1.0, 0.6, 1.7]))
        top_p = float(np.float32(rng.uniform(0.05, 0.99)))
        p = softmax(row.astype(np.float64) / T)
        got, amb = oracle.target_row(row, T, top_p, return_ambiguous=True)
        if amb:
            continue
        keep = _nucleus_ascending(p, top_p)
        assert np.array_equal(got > 0, keep), (trial, top_p)
        want = np.where(keep, p, 0.0)
        want /= want.sum()
        assert np.max(np.abs(got - want)) < 1e-12
        checked += 1
    assert checked > 250


def test_cut_matches_the_threshold_form_with_ties():
    rng = np.random.default_rng(52)
    for trial in range(300):
        V = int(rng.integers(1, 12))
        row = rng.integers(-3, 3, size=V).astype(np.float32)   # many ties
        top_p = float(np.float32(rng.choice([0.0, 0.1, 0.3, 0.5, 0.7, 0.9, 0.999])))
        p = softmax(row.astype(np.float64))
        got, amb = oracle.target_row(row, 1.0, top_p, return_ambiguous=True)
        if amb:
            continue
        values = sorted(set(row.tolist()), reverse=True)
        cut = values[0]
        for v in values:           # the largest v whose upper set reaches top_p
            if p[row >= v].sum() >= top_p:
                cut = v
                break
        keep = row >= cut
        assert np.array_equal(got > 0, keep), (trial, row, top_p)
        assert abs(got.sum() - 1.0) < 1e-12


def test_full_or_nan_top_p_changes_nothing():
    s = W.make_sample_from_params(53, 16, 4, 3000, 3.0, 1.0)
    a = oracle.sample(s.target_logits, s.draft_probs, s.draft_tokens, s.uniforms,
                      temperature=np.full(s.B, 0.8, np.float32))
    for tp in (1.0, 1.5, np.nan):
        b = oracle.sample(s.target_logits, s.draft_probs, s.draft_tokens, s.uniforms,
                          temperature=np.full(s.B, 0.8, np.float32), top_p=np.full(s.B, tp, np.float32))
        for key in a:
            assert np.array_equal(a[key], b[key], equal_nan=True), (tp, key)


def test_vanishing_top_p_is_the_greedy_limit():
    s = W.make_sample_from_params(54, 48, 5, 700, 2.0, 0.3)
    arg = np.argmax(s.target_logits, axis=-1)
    rng = np.random.default_rng(55)
    tokens = np.where(rng.random((s.B, s.K)) < 0.7, arg[:, :s.K], s.draft_tokens).astype(np.int32)
    g = oracle.sample(s.target_logits, s.draft_probs, tokens, s.uniforms, temperature=np.zeros(s.B, np.float32))
    for tp in (0.0, 1e-9):
        c = oracle.sample(s.target_logits, s.draft_probs, tokens, s.uniforms, top_p=np.full(s.B, tp, np.float32))
        assert np.array_equal(g["num_accepted"], c["num_accepted"])
        assert np.array_equal(g["out_tokens"], c["out_tokens"])
    assert g["num_accepted"].sum() > 0


@pytest.mark.parametrize("T,top_p", [(1.0, 0.8), (0.7, 0.9), (1.5, 0.6)])
def test_every_emitted_position_follows_the_cut_target(T, top_p):
    K, V, N = 3, 12, 1_000_000
    logits, _ = _rows(301, K, V, sigma=1.5)
    rng = np.random.default_rng(302)
    dl = logits[:K].astype(np.float64) + 0.7 * rng.standard_normal((K, V))
    # the draft samples its own tempered, cut distribution
    q = np.stack([oracle.target_row(dl[i].astype(np.float32), T, top_p) for i in range(K)]).astype(np.float32)
    q /= q.sum(axis=1, keepdims=True)
    tokens = np.empty((N, K), dtype=np.int32)
    for i in range(K):
        tokens[:, i] = rng.choice(V, size=N, p=q[i].astype(np.float64) / q[i].astype(np.float64).sum())
    u = np.minimum(rng.random((N, K + 1)).astype(np.float32), U_MAX)
    tl = np.ascontiguousarray(np.broadcast_to(logits, (N, K + 1, V)))
    dp = np.ascontiguousarray(np.broadcast_to(q, (N, K, V)))
    res = oracle.sample(tl, dp, tokens, u, temperature=np.full(N, T, np.float32),
                        top_p=np.full(N, top_p, np.float32))
    n, toks = res["num_accepted"], res["out_tokens"]
    checked = 0
    for i in range(K + 1):
        p = softmax(logits[i].astype(np.float64) / T)
        keep = _nucleus_ascending(p, top_p)
        want = np.where(keep, p, 0.0)
        want /= want.sum()
        present = n >= i
        if present.sum() < 20_000:
            continue
        pv = chi2_pvalue(np.bincount(toks[present, i], minlength=V), want)
        assert pv > 1e-3, (T, top_p, i, pv)
        checked += 1
    assert checked >= 2


def test_ambiguous_cut_sets_near_pos():
    # two tokens of mass ~0.5 each; top_p at that mass (within 1e-6) is ambiguous
    row = np.array([0.0, -1e-7, -30.0], dtype=np.float32)
    p = softmax(row.astype(np.float64))
    _, amb = oracle.target_row(row, 1.0, float(np.float32(p[0])), return_ambiguous=True)
    assert amb
    _, amb = oracle.target_row(row, 1.0, 0.3, return_ambiguous=True)
    assert not amb
    lg = np.tile(row, (1, 3, 1)).astype(np.float32)
    q = np.full((1, 2, 3), 1.0 / 3, np.float32)
    res = oracle.sample(lg, q, np.zeros((1, 2), np.int32), np.full((1, 3), 0.1, np.float32),
                        top_p=np.array([p[0]], np.float32))
    assert res["near_pos"][0] == 0
