"""Pins for the oracle's verify sampler (CPU only).

What fixes the sampler without trusting the oracle:
  * exactness ("50 | Speculative Decoding" 3.2; "KV Cache + Speculative
    Decoding" 7.3): every emitted position is distributed as the target p_i,
    whatever the draft q is -- chi-square over 10^6 trials, p-value > 1e-3;
  * the residual normaliser identity sum max(0,p-q) = 1 - sum min(p,q)
    ("50 | Speculative Decoding" 3.2) against a library softmax;
  * expected tokens per round (1 - a^(K+1)) / (1 - a) under i.i.d. acceptance
    ("KV Cache + Speculative Decoding" 7.4; "50 | Speculative Decoding" 4.1);
  * the pages' own sanity checks ("KV Cache + Speculative Decoding" A.2):
    acceptance rate from 100k samples within 1% of theory, TV < 0.01;
  * the exact law of a round for V in {2,3}, K in {1,2} in rational arithmetic;
  * the two-token worked example ("Lecture 10 - Inference" section 8, whose
    notation swaps the names p and q);
  * boundary uniforms, q = p, one-hot targets, the strict "<" of the test.
"""
from fractions import Fraction

import numpy as np
import pytest
from scipy import stats
from scipy.special import softmax

import oracle
import workloads as W

U_MAX = np.float32(np.nextafter(np.float32(1.0), np.float32(0.0)))  # 1 - 2^-24


def run_trials(logits, q, N, seed):
    """N independent rounds with fixed target rows (logits [K+1,V]) and draft
    rows (q [K,V]): fresh draft tokens x_i ~ q_i and fresh uniforms per round."""
    logits = np.asarray(logits, dtype=np.float32)
    q = np.asarray(q, dtype=np.float32)
    K1, V = logits.shape
    K = K1 - 1
    rng = np.random.default_rng(seed)
    tokens = np.empty((N, K), dtype=np.int32)
    for i in range(K):
        qi = q[i].astype(np.float64)
        tokens[:, i] = rng.choice(V, size=N, p=qi / qi.sum())
    u = np.minimum(rng.random((N, K + 1)).astype(np.float32), U_MAX)
    tl = np.ascontiguousarray(np.broadcast_to(logits, (N, K + 1, V)))
    dp = np.ascontiguousarray(np.broadcast_to(q, (N, K, V)))
    return oracle.sample(tl, dp, tokens, u)


def chi2_pvalue(obs, p):
    obs = np.asarray(obs, dtype=np.float64)
    exp = obs.sum() * np.asarray(p, dtype=np.float64)
    small = exp < 5
    if small.any():
        obs = np.append(obs[~small], obs[small].sum())
        exp = np.append(exp[~small], exp[small].sum())
    keep = exp > 0
    assert obs[~keep].sum() == 0, "token of zero target probability emitted"
    return stats.chisquare(obs[keep], exp[keep]).pvalue


def _rows(seed, K, V, sigma=2.0, noise=0.8):
    rng = np.random.default_rng(seed)
    logits = (rng.standard_normal((K + 1, V)) * sigma).astype(np.float32)
    dl = logits[:K].astype(np.float64) + noise * rng.standard_normal((K, V))
    q = softmax(dl, axis=-1).astype(np.float32)
    return logits, q


def _qvariants(seed, K, V):
    logits, q_noisy = _rows(seed, K, V)
    q_onehot = np.full((K, V), 0.0, dtype=np.float32)
    q_onehot[np.arange(K), np.argmax(logits[:K], axis=1)] = 1.0   # a point-mass draft
    q_uniform = np.full((K, V), 1.0 / V, dtype=np.float32)
    return logits, {"noisy": q_noisy, "onehot": q_onehot, "uniform": q_uniform}


@pytest.mark.parametrize("variant", ["noisy", "onehot", "uniform"])
def test_every_emitted_position_follows_target(variant):
    K, V, N = 3, 12, 1_000_000
    logits, qs = _qvariants(101, K, V)
    res = run_trials(logits, qs[variant], N, seed=7)
    n = res["num_accepted"]
    toks = res["out_tokens"]
    p = softmax(logits.astype(np.float64), axis=-1)
    checked = 0
    for i in range(K + 1):
        present = n >= i
        if present.sum() < 20_000:
            continue
        obs = np.bincount(toks[present, i], minlength=V)
        pv = chi2_pvalue(obs, p[i])
        assert pv > 1e-3, (variant, i, pv)
        checked += 1
    assert checked >= 2
    # positions past the drawn token are padding
    pad = np.arange(K + 1)[None, :] > n[:, None]
    assert np.all(toks[pad] == -1)


def test_residual_mass_identity_on_config_rows():
    for name in ("c1", "c3"):
        s = W.make_sample(name, seed=3)
        res = oracle.sample(s.target_logits, s.draft_probs, s.draft_tokens, s.uniforms)
        for b in range(s.B):
            n = int(res["num_accepted"][b])
            if n == s.K:
                continue
            p = softmax(s.target_logits[b, n].astype(np.float64))
            q = s.draft_probs[b, n].astype(np.float64)
            assert abs(res["resid_mass"][b] - (1.0 - np.minimum(p, q).sum())) < 1e-12


def test_accept_ratio_matches_library_softmax():
    s = W.make_sample("c1", seed=5)
    s2 = W.make_sample_from_params(9, 16, 4, 777, 3.0, 1.0)
    for smp in (s, s2):
        res = oracle.sample(smp.target_logits, smp.draft_probs, smp.draft_tokens, smp.uniforms)
        for b in range(smp.B):
            for i in range(int(res["num_accepted"][b]) + (1 if res["num_accepted"][b] < smp.K else 0)):
                p = softmax(smp.target_logits[b, i].astype(np.float64))
                x = smp.draft_tokens[b, i]
                want = min(1.0, p[x] / float(smp.draft_probs[b, i, x]))
                assert abs(res["accept_ratio"][b, i] - want) <= 1e-13 * max(1.0, want)


def _tau_law(alpha, K):
    """Law of tokens per round n+1 under i.i.d. acceptance alpha."""
    probs = [alpha ** j * (1 - alpha) for j in range(K)] + [alpha ** K]
    vals = np.arange(1, K + 2, dtype=np.float64)
    return vals, np.array(probs)


@pytest.mark.parametrize("K,noise", [(4, 0.6), (7, 1.5), (2, 0.2)])
def test_mean_tokens_per_round_closed_form(K, noise):
    V, N = 20, 1_000_000
    logits1, q1 = _rows(202 + K, 1, V, noise=noise)
    logits = np.repeat(logits1[:1], K + 1, axis=0)
    q = np.repeat(q1[:1], K, axis=0)
    p = softmax(logits1[0].astype(np.float64))
    alpha = float(np.minimum(p, q1[0].astype(np.float64)).sum())
    res = run_trials(logits, q, N, seed=K)
    tau = res["num_accepted"].astype(np.float64) + 1
    closed = (1 - alpha ** (K + 1)) / (1 - alpha)
    vals, probs = _tau_law(alpha, K)
    assert abs((vals * probs).sum() - closed) < 1e-12     # the series sums to the closed form
    var = (vals ** 2 * probs).sum() - closed ** 2
    se = np.sqrt(var / N)
    assert abs(tau.mean() - closed) < 4 * se, (tau.mean(), closed, se)


def test_pages_sanity_alpha_and_tv():
    """100k rounds: empirical acceptance rate within 1% of sum min(p,q), and the
    first emitted token within total variation 0.01 of p."""
    K, V, N = 1, 10, 100_000
    logits, q = _rows(303, K, V, noise=0.7)
    res = run_trials(logits, q, N, seed=11)
    p0 = softmax(logits[0].astype(np.float64))
    alpha = float(np.minimum(p0, q[0].astype(np.float64)).sum())
    acc = (res["num_accepted"] >= 1).mean()
    assert abs(acc - alpha) / alpha < 0.01
    freq = np.bincount(res["out_tokens"][:, 0], minlength=V) / N
    assert 0.5 * np.abs(freq - p0).sum() < 0.01


def _exact_law(p, q, K):
    """Exact law of one round as {(n, tokens...): probability} in rationals.
    p: K+1 target rows, q: K draft rows (lists of Fractions)."""
    V = len(p[0])
    law = {}

    def resid(i):
        w = [max(Fraction(0), p[i][y] - q[i][y]) for y in range(V)]
        s = sum(w)
        return [wy / s for wy in w]

    def rec(i, prefix, prob):
        if i == K:
            for y in range(V):
                if p[K][y]:
                    law[(K,) + prefix + (y,)] = law.get((K,) + prefix + (y,), 0) + prob * p[K][y]
            return
        reject = Fraction(0)
        for x in range(V):
            if q[i][x] == 0:
                continue
            acc = min(Fraction(1), p[i][x] / q[i][x])
            rec(i + 1, prefix + (x,), prob * q[i][x] * acc)
            reject += q[i][x] * (1 - acc)
        if reject:
            r = resid(i)
            for y in range(V):
                if r[y]:
                    key = (i,) + prefix + (y,)
                    law[key] = law.get(key, 0) + prob * reject * r[y]

    rec(0, (), Fraction(1))
    return law


EXACT_CASES = [
    (2, 1, [[Fraction(1, 4), Fraction(3, 4)], [Fraction(1, 2), Fraction(1, 2)]],
     [[Fraction(1, 2), Fraction(1, 2)]]),
    (3, 2, [[Fraction(1, 2), Fraction(1, 4), Fraction(1, 4)],
            [Fraction(1, 8), Fraction(3, 8), Fraction(1, 2)],
            [Fraction(1, 4), Fraction(1, 2), Fraction(1, 4)]],
     [[Fraction(1, 4), Fraction(1, 4), Fraction(1, 2)],
      [Fraction(1, 2), Fraction(1, 4), Fraction(1, 4)]]),
]


@pytest.mark.parametrize("V,K,p,q", EXACT_CASES)
def test_exact_small_vocab_law(V, K, p, q):
    law = _exact_law(p, q, K)
    assert sum(law.values()) == 1
    # token marginal at every position, given the position exists, is p_i exactly
    for i in range(K + 1):
        mass = Fraction(0)
        marg = [Fraction(0)] * V
        for key, pr in law.items():
            n = key[0]
            if n >= i:
                mass += pr
                marg[key[1 + i]] += pr
        assert all(marg[y] / mass == p[i][y] for y in range(V))
    # the oracle's empirical law matches the exact one (dyadic values are exact in fp32)
    logits = np.log(np.array([[float(x) for x in row] for row in p]))
    qa = np.array([[float(x) for x in row] for row in q], dtype=np.float32)
    N = 400_000
    res = run_trials(logits, qa, N, seed=V * 10 + K)
    keys = list(law.keys())
    index = {k: j for j, k in enumerate(keys)}
    obs = np.zeros(len(keys))
    for b in range(N):
        n = int(res["num_accepted"][b])
        key = (n,) + tuple(int(t) for t in res["out_tokens"][b, :n + 1])
        obs[index[key]] += 1
    pv = chi2_pvalue(obs, [float(law[k]) for k in keys])
    assert pv > 1e-3


def test_two_token_worked_example():
    """Vocabulary {A, B}; the draft over-estimates A.  Draft q = (3/4, 1/4),
    target p = (1/2, 1/2).  Drafting A is accepted for u < 2/3 and otherwise
    replaced by B (all residual mass is on B); drafting B is always accepted.
    Over an even grid of uniforms the output law is exactly p."""
    M = 3000
    u0 = ((np.arange(M) + 0.5) / M).astype(np.float32)
    tl = np.zeros((M, 2, 2), dtype=np.float32)               # p = (1/2, 1/2)
    dp = np.tile(np.array([0.75, 0.25], dtype=np.float32), (M, 1, 1))
    u = np.stack([u0, np.full(M, 0.5, np.float32)], axis=1)
    outA = oracle.sample(tl, dp, np.zeros((M, 1), np.int32), u)
    outB = oracle.sample(tl, dp, np.ones((M, 1), np.int32), u)
    acceptedA = int((outA["num_accepted"] == 1).sum())
    assert acceptedA == 2000                                  # #{u < 2/3}
    assert np.all(outA["out_tokens"][outA["num_accepted"] == 0, 0] == 1)
    assert np.all(outB["num_accepted"] == 1)
    pA = Fraction(3, 4) * Fraction(acceptedA, M)
    assert pA == Fraction(1, 2)


def _one(logits, q, tokens, u):
    res = oracle.sample(np.asarray(logits, np.float32)[None], np.asarray(q, np.float32)[None],
                        np.asarray(tokens, np.int32)[None], np.asarray(u, np.float32)[None])
    return int(res["num_accepted"][0]), res["out_tokens"][0].tolist()


def test_boundary_uniforms():
    V = 4
    lg = np.array([[0.0, 1.0, -np.inf, 2.0], [0.5, 0.0, 0.0, 0.0]], dtype=np.float32)
    q = np.array([[0.25, 0.25, 0.25, 0.25]], dtype=np.float32)
    # u = 0 accepts whenever p(x) > 0 and rejects p(x) = 0
    assert _one(lg, q, [1], [0.0, 0.5])[0] == 1
    assert _one(lg, q, [2], [0.0, 0.5])[0] == 0
    # u = 1 - 2^-24 rejects p(x) < q(x) and accepts p(x) >= q(x)
    p = softmax(lg[0].astype(np.float64))
    lo = int(np.argmin(np.where(p > 0, p, np.inf)))
    assert p[lo] < 0.25 and p[3] > 0.25
    assert _one(lg, q, [lo], [U_MAX, 0.5])[0] == 0
    assert _one(lg, q, [3], [U_MAX, 0.5])[0] == 1
    # strict "<": u*q(x) == p(x) rejects (p = 1/4 exactly, q = 1/2, u = 1/2)
    flat = np.zeros((2, V), np.float32)
    qh = np.array([[0.5, 0.5 / 3, 0.5 / 3, 0.5 / 3]], np.float32)
    assert _one(flat, qh, [0], [0.5, 0.5])[0] == 0
    assert _one(flat, qh, [0], [np.nextafter(np.float32(0.5), np.float32(0)), 0.5])[0] == 1
    # final draw: u_K = 0 -> first positive weight; u_K -> 1 -> last positive weight
    lg2 = np.array([[0.0, 0.0, 0.0, 0.0], [-np.inf, 0.0, 0.0, -np.inf]], np.float32)
    q2 = np.array([[0.25, 0.25, 0.25, 0.25]], np.float32)
    n, toks = _one(lg2, q2, [0], [0.0, 0.0])
    assert n == 1 and toks == [0, 1]
    n, toks = _one(lg2, q2, [0], [0.0, U_MAX])
    assert n == 1 and toks == [0, 2]
    # residual draw skips zero-weight tokens: p = (.1,.2,.3,.4)-ish vs q concentrated
    lg3 = np.log(np.array([[0.1, 0.2, 0.3, 0.4], [0.25] * 4], np.float64)).astype(np.float32)
    q3 = np.array([[0.7, 0.1, 0.1, 0.1]], np.float32)
    n, toks = _one(lg3, q3, [0], [U_MAX, 0.0])
    assert n == 0 and toks[0] == 1          # first token with p > q
    n, toks = _one(lg3, q3, [0], [U_MAX, U_MAX])
    assert n == 0 and toks[0] == 3


def test_draft_equal_to_target_accepts_all_and_draws_bonus():
    V, K = 8, 3
    lg = np.zeros((K + 1, V), np.float32)
    lg[K] = np.log(np.arange(1, V + 1) / 36.0)
    q = np.full((K, V), 1.0 / V, np.float32)
    N = 200_000
    res = run_trials(lg, q, N, seed=1)
    assert np.all(res["num_accepted"] == K)
    counts = np.bincount(res["out_tokens"][:, K], minlength=V)
    assert chi2_pvalue(counts, np.arange(1, V + 1) / 36.0) > 1e-3


def test_one_hot_target_always_emits_its_token():
    V, K = 6, 2
    lg = np.full((K + 1, V), -np.inf, np.float32)
    lg[0, 4] = 0.0
    lg[1, 1] = 0.0
    lg[2, 5] = 0.0
    q = softmax(np.random.default_rng(3).standard_normal((K, V)), axis=-1).astype(np.float32)
    res = run_trials(lg, q, 20_000, seed=2)
    toks = res["out_tokens"]
    n = res["num_accepted"]
    assert np.all(toks[:, 0] == 4)
    assert np.all(toks[n >= 1, 1] == 1)
    assert np.all(toks[n >= 2, 2] == 5)


def test_near_threshold_flags():
    """A uniform within 1e-6 of min(1, p/q) is flagged at its position."""
    V = 4
    lg = np.zeros((2, V), np.float32)               # p = 1/4
    q = np.array([[0.5, 0.5 / 3, 0.5 / 3, 0.5 / 3]], np.float32)   # ratio for token 0 = 1/2
    res = oracle.sample(lg[None], q[None], np.array([[0]], np.int32),
                        np.array([[0.5 + 4e-7, 0.3]], np.float32))
    assert res["near_pos"][0] == 0
    res = oracle.sample(lg[None], q[None], np.array([[0]], np.int32),
                        np.array([[0.6, 0.3]], np.float32))
    assert res["near_pos"][0] == -1


def test_padding_and_shapes_on_config():
    s = W.make_sample("c1", seed=0)
    res = oracle.sample(s.target_logits, s.draft_probs, s.draft_tokens, s.uniforms)
    n = int(res["num_accepted"][0])
    toks = res["out_tokens"][0]
    assert list(toks[:n]) == list(s.draft_tokens[0, :n])
    assert 0 <= toks[n] < s.V
    assert all(t == -1 for t in toks[n + 1:])
