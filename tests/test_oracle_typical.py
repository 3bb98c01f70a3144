"""Pins of the oracle's typical acceptance ("50 | Speculative Decoding" 9.1;
"KV Cache + Speculative Decoding" 8.2 and Q18: a draft is accepted iff the
target's own probability of it exceeds min(eps, delta * exp(-H(p)));
not exact; eps and delta are not given on the pages, so they are
parameters here).

  * the entropy against scipy's (a library routine), and its closed forms
    (log V for a uniform row, 0 for a one-hot row);
  * the closed forms of the rule: a uniform target accepts every draft when
    delta < 1 <= eps*V and none when delta > 1, a one-hot target accepts
    exactly its argmax, eps = 0 accepts every draft of positive probability;
  * a two-token worked example computed by hand on both sides of the
    threshold;
  * monotonicity: raising eps or delta never lengthens an accepted prefix;
  * temperature is a rescaling of the logits;
  * the token after the accepted prefix follows the target row at that
    position (chi-square, conditioned on the prefix length).
"""
import numpy as np
import pytest
from scipy import stats
from scipy.special import softmax

import oracle
import workloads as W
from .test_oracle_sampler import U_MAX, chi2_pvalue


def test_entropy_matches_library_and_closed_forms():
    rng = np.random.default_rng(91)
    for V in (2, 17, 1000, 50000):
        p = softmax(rng.standard_normal(V) * rng.uniform(0.5, 4))
        assert abs(oracle.entropy(p) - stats.entropy(p)) < 1e-10
    assert abs(oracle.entropy(np.full(1000, 1e-3)) - np.log(1000)) < 1e-12
    assert oracle.entropy(np.eye(7)[3]) == 0.0


def _run(logits, tokens, eps, delta, u=None, temperature=None):
    logits = np.asarray(logits, np.float32)
    B, T, V = logits.shape
    if u is None:
        u = np.full((B, T), 0.5, np.float32)
    return oracle.sample_typical(logits, np.asarray(tokens, np.int32), u, eps, delta, temperature=temperature)


def test_uniform_target_closed_form():
    V, K = 64, 4
    lg = np.zeros((3, K + 1, V), np.float32)
    tok = np.random.default_rng(92).integers(0, V, size=(3, K))
    # tau = min(eps, delta / V): 1/V > tau iff delta < 1 (with eps > delta / V)
    assert list(_run(lg, tok, eps=0.5, delta=0.9)["num_accepted"]) == [K] * 3
    assert list(_run(lg, tok, eps=0.5, delta=1.1)["num_accepted"]) == [0] * 3
    r = _run(lg, tok, eps=0.5, delta=0.9)
    assert np.allclose(r["threshold"], 0.9 / V, rtol=1e-12)


def test_one_hot_target_accepts_exactly_its_argmax():
    V, K = 50, 5
    lg = np.full((4, K + 1, V), -np.inf, np.float32)
    lg[:, :, 7] = 0.0
    tok = np.full((4, K), 7, np.int32)
    tok[1, 2] = 8          # sequence 1 rejects at 2
    r = _run(lg, tok, eps=0.2, delta=0.5)
    assert list(r["num_accepted"]) == [K, 2, K, K]
    assert np.all(r["out_tokens"][1, :3] == [7, 7, 7]) and np.all(r["out_tokens"][1, 3:] == -1)
    assert np.allclose(r["threshold"][0], 0.2)   # H = 0: min(eps, delta)


def test_zero_eps_accepts_every_positive_draft():
    s = W.make_sample_from_params(93, 16, 5, 500, 3.0, 1.0)
    r = oracle.sample_typical(s.target_logits, s.draft_tokens, s.uniforms, 0.0, 1.0)
    assert np.all(r["num_accepted"] == s.K)
    # ... and none of probability 0: the comparison is strict
    lg = s.target_logits.copy()
    for b in range(s.B):
        lg[b, 2, s.draft_tokens[b, 2]] = -np.inf
    r = oracle.sample_typical(lg, s.draft_tokens, s.uniforms, 0.0, 1.0)
    assert np.all(r["num_accepted"] == 2)


def test_two_token_worked_example():
    # p = (0.8, 0.2): H = -(0.8 ln 0.8 + 0.2 ln 0.2) = 0.500402..., exp(-H) = 0.606287...
    # eps = 0.25, delta = 0.3: tau = 0.181886 < 0.2 -> token 1 accepted;
    # delta = 0.4: tau = 0.242515 > 0.2 -> rejected.
    lg = np.log(np.array([[[0.8, 0.2], [0.5, 0.5]]], np.float64)).astype(np.float32)
    r = _run(lg, [[1]], eps=0.25, delta=0.3)
    assert r["num_accepted"][0] == 1 and abs(r["threshold"][0, 0] - 0.181886) < 1e-6
    r = _run(lg, [[1]], eps=0.25, delta=0.4)
    assert r["num_accepted"][0] == 0 and abs(r["threshold"][0, 0] - 0.242515) < 1e-6
    # the drawn token at position 0 comes from p_0 = (0.8, 0.2) itself
    for uu, want in ((0.79, 0), (0.81, 1)):
        r = _run(lg, [[1]], eps=0.25, delta=0.4, u=np.array([[0.5, uu]], np.float32))
        assert r["out_tokens"][0, 0] == want


def test_raising_eps_or_delta_never_lengthens_the_prefix():
    s = W.make_sample_from_params(94, 64, 6, 2000, 2.0, 0.8)
    prev = None
    for eps, delta in ((0.01, 0.05), (0.05, 0.1), (0.1, 0.3), (0.3, 0.6), (0.6, 2.0)):
        n = oracle.sample_typical(s.target_logits, s.draft_tokens, s.uniforms, eps, delta)["num_accepted"]
        if prev is not None:
            assert np.all(n <= prev)
        prev = n
    assert prev.sum() < n.size * s.K


def test_temperature_rescales_the_logits():
    s = W.make_sample_from_params(95, 32, 4, 3000, 3.0, 1.0)
    for T in (0.6, 1.8):
        a = oracle.sample_typical(s.target_logits, s.draft_tokens, s.uniforms, 0.1, 0.3,
                                  temperature=np.full(s.B, T, np.float32))
        b = oracle.sample_typical((s.target_logits / np.float32(T)).astype(np.float32), s.draft_tokens,
                                  s.uniforms, 0.1, 0.3)
        for i in range(s.B):
            k = max(a["near_pos"][i], b["near_pos"][i])
            if k < 0:
                assert a["num_accepted"][i] == b["num_accepted"][i]
                assert np.array_equal(a["out_tokens"][i], b["out_tokens"][i])


def test_token_after_the_prefix_follows_its_row():
    K, V, N = 3, 12, 600_000
    rng = np.random.default_rng(96)
    logits = (rng.standard_normal((K + 1, V)) * 1.5).astype(np.float32)
    p = softmax(logits.astype(np.float64), axis=-1)
    q = softmax(logits[:K].astype(np.float64) + 0.8 * rng.standard_normal((K, V)), axis=-1)
    tok = np.stack([rng.choice(V, size=N, p=q[i]) for i in range(K)], axis=1).astype(np.int32)
    u = np.minimum(rng.random((N, K + 1)).astype(np.float32), U_MAX)
    r = oracle.sample_typical(np.ascontiguousarray(np.broadcast_to(logits, (N, K + 1, V))), tok, u, 0.1, 0.3)
    n, ot = r["num_accepted"], r["out_tokens"]
    for i in range(K + 1):
        sel = n == i
        if sel.sum() < 20_000:
            continue
        pv = chi2_pvalue(np.bincount(ot[sel, i], minlength=V), p[i])
        assert pv > 1e-3, (i, pv)
