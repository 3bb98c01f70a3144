"""GPU parity of the verify sampler under a target temperature per sequence
(spec_verify_sample_ex; "KV Cache + Speculative Decoding" 7.5: the exactness
argument holds with the tempered target p~ = softmax(logits / T) in place of
p, while the draft probabilities are used as given).

Same bar as the plain sampler: accepted counts and emitted tokens bit for bit
against the oracle, except from the first position the oracle decided within
1e-6 of its threshold.  Covered: T below and above 1 on the chunked and
scalar paths, a mix of temperatures in one batch (greedy rows included), the
greedy limit against its definition, T = 1 against the plain entry point, and
the law of the emitted tokens from the GPU path itself.
"""
import numpy as np
import pytest
import torch
from scipy.special import softmax

import speculative_decoding_verify_attn_amd as sv
import workloads as W
from .gpu_helpers import compare_sampler, dev, run_sample, upload_sample
from .test_gpu_sampler import _chi2

pytestmark = pytest.mark.gpu

CASES = [
    # (seed, B, K, V, sigma, noise, temperature)
    (31, 48, 4, 32000, 3.0, 1.0, 0.5),
    (32, 48, 4, 32000, 3.0, 1.0, 1.8),
    (33, 20, 6, 777, 2.0, 1.0, 0.7),      # scalar path (V % 4 != 0)
    (34, 16, 3, 8193, 2.0, 0.5, 3.0),     # two chunks and a 1-entry tail
    (35, 8, 5, 128256, 3.0, 1.0, 0.25),   # Llama-3 vocabulary, sharp target
]


@pytest.mark.parametrize("case", CASES, ids=[str(c[0]) for c in CASES])
def test_uniform_temperature_parity(case):
    seed, B, K, V, sigma, noise, T = case
    s = W.make_sample_from_params(seed, B, K, V, sigma, noise)
    temp = np.full(B, T, np.float32)
    n, toks, ap = run_sample(s, temperature=temp)
    mism, flagged, ref = compare_sampler(s, n, toks, temperature=temp)
    print("case %d T=%.2f mismatches=%d near-threshold=%d mean accepted=%.3f"
          % (seed, T, mism, flagged, float(n.mean())))
    assert mism == 0
    for b in range(s.B):
        for i in range(int(ref["num_accepted"][b]) + (1 if ref["num_accepted"][b] < s.K else 0)):
            assert abs(ap[b, i] - ref["accept_ratio"][b, i]) <= 1e-6


def test_mixed_temperatures_with_greedy_rows():
    s = W.make_sample_from_params(36, 64, 5, 50000, 3.0, 1.0)
    rng = np.random.default_rng(37)
    temp = rng.choice(np.array([0.0, 0.3, 0.8, 1.0, 1.5, -1.0, 4.0], np.float32), size=s.B)
    temp[5] = np.nan                                       # NaN is greedy too
    # greedy rows need drafts equal to the argmax to accept anything
    arg = np.argmax(s.target_logits, axis=-1)
    take = rng.random((s.B, s.K)) < 0.6
    s = W.SampleInputs(s.target_logits, s.draft_probs,
                       np.where(take, arg[:, :s.K], s.draft_tokens).astype(np.int32), s.uniforms)
    n, toks, _ = run_sample(s, temperature=temp)
    mism, flagged, _ = compare_sampler(s, n, toks, temperature=temp)
    print("mixed: mismatches=%d near-threshold=%d" % (mism, flagged))
    assert mism == 0
    greedy = ~(temp > 0)
    for b in np.nonzero(greedy)[0]:
        m = 0
        while m < s.K and s.draft_tokens[b, m] == arg[b, m]:
            m += 1
        assert n[b] == m and toks[b, m] == arg[b, m]


def test_greedy_ties_take_the_first_maximum():
    B, K, V = 4, 2, 4099
    lg = np.zeros((B, K + 1, V), np.float32)
    lg[:, :, 1000] = 5.0
    lg[:, :, 3000] = 5.0                                   # tie: the first index wins
    lg[1, :, 4098] = 6.0                                   # maximum in the tail entry
    q = np.full((B, K, V), 1.0 / V, np.float32)
    tok = np.full((B, K), 1000, np.int32)
    tok[1] = 4098
    tok[2, 1] = 3000                                       # second draft is the later tie: rejected
    u = np.full((B, K + 1), 0.5, np.float32)
    s = W.SampleInputs(lg, q, tok, u)
    n, toks, _ = run_sample(s, temperature=np.zeros(B, np.float32))
    assert list(n) == [2, 2, 1, 2]
    assert list(toks[0]) == [1000, 1000, 1000]
    assert list(toks[1]) == [4098, 4098, 4098]
    assert list(toks[2]) == [1000, 1000, -1]


def test_unit_temperature_equals_plain_entry():
    s = W.make_sample_from_params(38, 40, 5, 32000, 3.0, 1.0)
    t = upload_sample(s)
    a = run_sample(s, t)
    b = run_sample(s, t, temperature=np.ones(s.B, np.float32))
    for x, y in zip(a, b):
        assert np.array_equal(x, y, equal_nan=True)


@pytest.mark.parametrize("T", [0.5, 2.0])
def test_gpu_output_law_matches_tempered_target(T):
    K, V, N, calls = 3, 48, 65536, 12
    rng = np.random.default_rng(40)
    logits = (rng.standard_normal((K + 1, V)) * 2).astype(np.float32)
    q = softmax((logits[:K].astype(np.float64) + 0.8 * rng.standard_normal((K, V))) / T,
                axis=-1).astype(np.float32)
    d = dev()
    tl = torch.from_numpy(np.ascontiguousarray(np.broadcast_to(logits, (N, K + 1, V)))).to(d)
    dp = torch.from_numpy(np.ascontiguousarray(np.broadcast_to(q, (N, K, V)))).to(d)
    temp = torch.full((N,), T, dtype=torch.float32, device=d)
    ws = sv.alloc_workspace(sv.sample_workspace_size(N, K, V), d)
    n_t = torch.empty(N, dtype=torch.int32, device=d)
    o_t = torch.empty((N, K + 1), dtype=torch.int32, device=d)
    ns, toks = [], []
    for _ in range(calls):
        tok = np.stack([rng.choice(V, size=N, p=q[i].astype(np.float64) / q[i].astype(np.float64).sum())
                        for i in range(K)], axis=1).astype(np.int32)
        u = np.minimum(rng.random((N, K + 1)).astype(np.float32), np.float32(1 - 2 ** -24))
        sv.spec_verify_sample(tl, dp, torch.from_numpy(tok).to(d), torch.from_numpy(u).to(d), n_t, o_t, ws,
                              temperature=temp)
        torch.cuda.synchronize()
        ns.append(n_t.cpu().numpy())
        toks.append(o_t.cpu().numpy())
    n, toks = np.concatenate(ns), np.concatenate(toks)
    p = softmax(logits.astype(np.float64) / T, axis=-1)
    for i in range(K + 1):
        present = n >= i
        pv = _chi2(np.bincount(toks[present, i], minlength=V).astype(np.float64), p[i])
        print("T=%.1f position %d: %d samples, chi2 p=%.3g" % (T, i, present.sum(), pv))
        assert pv > 1e-3


@pytest.mark.parametrize("T", [1.0, 1.8, 0.6, 0.0])
def test_masked_chunks_and_minus_inf_entries(T):
    """Logits that are -inf over a whole 8192-entry chunk and at scattered
    entries (a masked vocabulary), at T = 1, above and below 1, and greedy."""
    s = W.make_sample_from_params(41, 12, 3, 30000, 3.0, 1.0)
    lg = s.target_logits.copy()
    lg[:, :, 8192:16384] = -np.inf
    rng = np.random.default_rng(42)
    lg[rng.random(lg.shape) < 0.2] = -np.inf
    lg[:, :, 29999] = np.maximum(lg[:, :, 29999], 0.0)  # every row keeps a finite entry
    s = W.SampleInputs(lg, s.draft_probs, s.draft_tokens, s.uniforms)
    temp = np.full(s.B, T, np.float32)
    n, toks, _ = run_sample(s, temperature=temp)
    mism, flagged, _ = compare_sampler(s, n, toks, temperature=temp)
    print("T=%.1f mismatches=%d near-threshold=%d" % (T, mism, flagged))
    assert mism == 0
    assert np.all(toks >= -1) and np.all(toks < s.V)
    emitted = toks[toks >= 0]
    assert not np.any((emitted >= 8192) & (emitted < 16384))
