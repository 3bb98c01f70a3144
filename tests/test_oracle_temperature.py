"""Pins of the oracle's sampler under a target temperature ("KV Cache +
Speculative Decoding" 7.5 and its answer on temperature / top-p: exactness
holds once p is replaced by the sampler-transformed p~, with p~ proportional
to p^(1/T), while q is whatever distribution the draft actually sampled from).

  * T = 1 is the plain sampler, bit for bit;
  * every emitted position follows softmax(logits / T) (chi-square over 10^6
    rounds), for T below and above 1 and for a draft that ignores T;
  * the greedy limit (T = 0): n = number of leading drafts equal to the
    target's first argmax, the drawn token is the argmax of row n -- written
    out from that definition here;
  * temperature is a rescaling of the logits: running at T equals running at
    T = 1 on logits / T, except where rounding puts a decision within 1e-6 of
    its threshold;
  * p~ itself against a library softmax of logits / T.
"""
import numpy as np
import pytest
from scipy.special import softmax

import oracle
import workloads as W
from .test_oracle_sampler import U_MAX, _rows, chi2_pvalue


def _trials(logits, q, N, seed, T):
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
    return oracle.sample(tl, dp, tokens, u, temperature=np.full(N, T, dtype=np.float32))


def test_unit_temperature_is_the_plain_sampler():
    s = W.make_sample("c1", seed=21)
    s2 = W.make_sample_from_params(22, 16, 4, 3000, 3.0, 1.0)
    for smp in (s, s2):
        a = oracle.sample(smp.target_logits, smp.draft_probs, smp.draft_tokens, smp.uniforms)
        b = oracle.sample(smp.target_logits, smp.draft_probs, smp.draft_tokens, smp.uniforms,
                          temperature=np.ones(smp.B, dtype=np.float32))
        for key in a:
            assert np.array_equal(a[key], b[key], equal_nan=True), key


def test_target_row_matches_library_softmax():
    rng = np.random.default_rng(23)
    row = (rng.standard_normal(5000) * 4).astype(np.float32)
    for T in (0.3, 0.7, 1.0, 1.6, 4.0):
        want = softmax(row.astype(np.float64) / T)
        got = oracle.target_row(row, T)
        assert np.max(np.abs(got - want)) < 1e-13
    g = oracle.target_row(np.array([1.0, 3.0, 2.0, 3.0], dtype=np.float32), 0.0)
    assert list(g) == [0.0, 1.0, 0.0, 0.0]   # first maximum


@pytest.mark.parametrize("T,draft_T", [(0.5, 0.5), (2.0, 2.0), (0.6, 1.0)])
def test_every_emitted_position_follows_tempered_target(T, draft_T):
    K, V, N = 3, 10, 1_000_000
    logits, _ = _rows(201, K, V, sigma=1.5)
    rng = np.random.default_rng(202)
    dl = logits[:K].astype(np.float64) + 0.7 * rng.standard_normal((K, V))
    q = softmax(dl / draft_T, axis=-1).astype(np.float32)   # the draft's own tempered proposal
    res = _trials(logits, q, N, seed=203, T=T)
    n, toks = res["num_accepted"], res["out_tokens"]
    p = softmax(logits.astype(np.float64) / T, axis=-1)
    checked = 0
    for i in range(K + 1):
        present = n >= i
        if present.sum() < 20_000:
            continue
        pv = chi2_pvalue(np.bincount(toks[present, i], minlength=V), p[i])
        assert pv > 1e-3, (T, draft_T, i, pv)
        checked += 1
    assert checked >= 2


def test_greedy_limit_is_greedy_decoding():
    s = W.make_sample_from_params(24, 64, 5, 500, 2.0, 0.3)
    # make some drafts equal to the target argmax so acceptance happens
    arg = np.argmax(s.target_logits, axis=-1)
    rng = np.random.default_rng(25)
    take = rng.random((s.B, s.K)) < 0.7
    tokens = np.where(take, arg[:, :s.K], s.draft_tokens).astype(np.int32)
    res = oracle.sample(s.target_logits, s.draft_probs, tokens, s.uniforms,
                        temperature=np.zeros(s.B, dtype=np.float32))
    for b in range(s.B):
        n = 0
        while n < s.K and tokens[b, n] == arg[b, n]:
            n += 1
        assert res["num_accepted"][b] == n
        assert res["out_tokens"][b, n] == arg[b, n]
        assert list(res["out_tokens"][b, :n]) == list(tokens[b, :n])
        assert np.all(res["out_tokens"][b, n + 1:] == -1)


def test_temperature_rescales_the_logits():
    s = W.make_sample_from_params(26, 32, 4, 2000, 3.0, 1.0)
    for T in (0.5, 1.7):
        a = oracle.sample(s.target_logits, s.draft_probs, s.draft_tokens, s.uniforms,
                          temperature=np.full(s.B, T, dtype=np.float32))
        b = oracle.sample((s.target_logits / np.float32(T)).astype(np.float32), s.draft_probs, s.draft_tokens,
                          s.uniforms)
        for i in range(s.B):
            k = max(a["near_pos"][i], b["near_pos"][i])
            if k < 0:
                assert a["num_accepted"][i] == b["num_accepted"][i]
                assert np.array_equal(a["out_tokens"][i], b["out_tokens"][i])
            else:
                assert np.array_equal(a["out_tokens"][i, :k], b["out_tokens"][i, :k])
