"""GPU parity of the verify sampler with a top-p cut of the target rows
(spec_verify_sample_ex; "KV Cache + Speculative Decoding" 7.5: the target row
is cut to its own top-p set and renormalised, the draft probabilities are
used as given, and the rejection rule stays exact).

Same bar as the plain sampler: accepted counts and emitted tokens bit for bit
against the oracle, except from the first position the oracle decided within
1e-6 of a threshold (a top-p boundary included).  Covered: several cuts with
and without a temperature on the chunked and scalar paths, a batch mixing
cuts, no-ops (1, NaN, > 1), zero and greedy rows, ties and signed zeros at
the boundary, masked vocabularies, determinism, and the law of the emitted
tokens from the GPU path itself.
"""
import numpy as np
import pytest
import torch
from scipy.special import softmax

import oracle
import speculative_decoding_verify_attn_amd as sv
import workloads as W
from .gpu_helpers import compare_sampler, dev, run_sample, upload_sample
from .test_gpu_sampler import _chi2

pytestmark = pytest.mark.gpu

CASES = [
    # (seed, B, K, V, sigma, noise, temperature, top_p)
    (61, 32, 4, 32000, 3.0, 1.0, 1.0, 0.9),
    (62, 32, 4, 32000, 3.0, 1.0, 0.7, 0.5),
    (63, 20, 6, 777, 2.0, 1.0, 1.0, 0.95),     # scalar path
    (64, 16, 3, 8193, 2.0, 0.5, 1.3, 0.8),     # two chunks and a 1-entry tail
    (65, 8, 5, 128256, 3.0, 1.0, 1.0, 0.9),    # Llama-3 vocabulary
    (66, 8, 5, 128256, 1.0, 1.0, 2.0, 0.99),   # flat rows: the cut keeps ~10^5 tokens
]


def _check(s, temp, cut, label):
    n, toks, ap = run_sample(s, temperature=temp, top_p=cut)
    mism, flagged, ref = compare_sampler(s, n, toks, temperature=temp, top_p=cut)
    print("%s: mismatches=%d near-threshold=%d mean accepted=%.3f" % (label, mism, flagged, float(n.mean())))
    assert mism == 0
    for b in range(s.B):
        k = int(ref["near_pos"][b])
        last = int(ref["num_accepted"][b]) + (1 if ref["num_accepted"][b] < s.K else 0)
        for i in range(last if k < 0 else min(last, k)):
            assert abs(ap[b, i] - ref["accept_ratio"][b, i]) <= 1e-6, (label, b, i)
    return n, toks


@pytest.mark.parametrize("case", CASES, ids=[str(c[0]) for c in CASES])
def test_uniform_cut_parity(case):
    seed, B, K, V, sigma, noise, T, tp = case
    s = W.make_sample_from_params(seed, B, K, V, sigma, noise)
    _check(s, np.full(B, T, np.float32), np.full(B, tp, np.float32), "case %d T=%.1f top_p=%.2f" % (seed, T, tp))


def test_mixed_cuts_no_ops_and_greedy_rows():
    s = W.make_sample_from_params(67, 64, 5, 50000, 3.0, 1.0)
    rng = np.random.default_rng(68)
    cut = rng.choice(np.array([0.0, 0.2, 0.5, 0.9, 0.999, 1.0, 1.5, -0.5], np.float32), size=s.B)
    cut[3] = np.nan
    temp = rng.choice(np.array([1.0, 0.6, 1.4, 0.0], np.float32), size=s.B)
    arg = np.argmax(s.target_logits, axis=-1)
    tok = np.where(rng.random((s.B, s.K)) < 0.5, arg[:, :s.K], s.draft_tokens).astype(np.int32)
    s = W.SampleInputs(s.target_logits, s.draft_probs, tok, s.uniforms)
    _check(s, temp, cut, "mixed")


def test_no_op_cut_equals_plain_call():
    s = W.make_sample_from_params(69, 24, 4, 32000, 3.0, 1.0)
    t = upload_sample(s)
    a = run_sample(s, t)
    for tp in (1.0, np.nan, 2.0):
        b = run_sample(s, t, top_p=np.full(s.B, tp, np.float32))
        for x, y in zip(a, b):
            assert np.array_equal(x, y, equal_nan=True)


def test_ties_and_signed_zeros_at_the_boundary():
    B, K, V = 24, 3, 4096
    rng = np.random.default_rng(70)
    lg = rng.integers(-4, 3, size=(B, K + 1, V)).astype(np.float32)   # heavy ties
    lg[lg == 0] = np.where(rng.random(int((lg == 0).sum())) < 0.5, -0.0, 0.0).astype(np.float32)
    q = softmax(lg[:, :K].astype(np.float64) + rng.standard_normal((B, K, V)), axis=-1).astype(np.float32)
    tok = rng.integers(0, V, size=(B, K)).astype(np.int32)
    u = rng.random((B, K + 1)).astype(np.float32)
    s = W.SampleInputs(lg, q, tok, u)
    for tp in (0.05, 0.3, 0.6, 0.9):
        _check(s, None, np.full(B, tp, np.float32), "ties top_p=%.2f" % tp)


def test_masked_vocabulary_with_cut():
    s = W.make_sample_from_params(71, 12, 3, 30000, 3.0, 1.0)
    lg = s.target_logits.copy()
    lg[:, :, 8192:16384] = -np.inf
    rng = np.random.default_rng(72)
    lg[rng.random(lg.shape) < 0.2] = -np.inf
    lg[:, :, 29999] = np.maximum(lg[:, :, 29999], 0.0)
    s = W.SampleInputs(lg, s.draft_probs, s.draft_tokens, s.uniforms)
    _, toks = _check(s, np.full(s.B, 1.2, np.float32), np.full(s.B, 0.9, np.float32), "masked")
    emitted = toks[toks >= 0]
    assert not np.any((emitted >= 8192) & (emitted < 16384))


def test_cut_is_deterministic():
    s = W.make_sample_from_params(73, 16, 5, 128256, 1.0, 1.0)
    t = upload_sample(s)
    cut = np.full(s.B, 0.95, np.float32)
    first = run_sample(s, t, top_p=cut)
    for _ in range(4):
        again = run_sample(s, t, top_p=cut)
        for x, y in zip(first, again):
            assert np.array_equal(x, y, equal_nan=True)


@pytest.mark.parametrize("T,tp", [(1.0, 0.8), (0.7, 0.6)])
def test_gpu_output_law_matches_cut_target(T, tp):
    K, V, N, calls = 3, 40, 65536, 12
    rng = np.random.default_rng(74)
    logits = (rng.standard_normal((K + 1, V)) * 2).astype(np.float32)
    dl = (logits[:K].astype(np.float64) + 0.8 * rng.standard_normal((K, V))).astype(np.float32)
    q = np.stack([oracle.target_row(dl[i], T, tp) for i in range(K)]).astype(np.float32)
    d = dev()
    tl = torch.from_numpy(np.ascontiguousarray(np.broadcast_to(logits, (N, K + 1, V)))).to(d)
    dp = torch.from_numpy(np.ascontiguousarray(np.broadcast_to(q, (N, K, V)))).to(d)
    temp = torch.full((N,), T, dtype=torch.float32, device=d)
    cut = torch.full((N,), tp, dtype=torch.float32, device=d)
    ws = sv.alloc_workspace(sv.sample_workspace_size(N, K, V), d)
    n_t = torch.empty(N, dtype=torch.int32, device=d)
    o_t = torch.empty((N, K + 1), dtype=torch.int32, device=d)
    ns, toks = [], []
    for _ in range(calls):
        tok = np.stack([rng.choice(V, size=N, p=q[i].astype(np.float64) / q[i].astype(np.float64).sum())
                        for i in range(K)], axis=1).astype(np.int32)
        u = np.minimum(rng.random((N, K + 1)).astype(np.float32), np.float32(1 - 2 ** -24))
        sv.spec_verify_sample(tl, dp, torch.from_numpy(tok).to(d), torch.from_numpy(u).to(d), n_t, o_t, ws,
                              temperature=temp, top_p=cut)
        torch.cuda.synchronize()
        ns.append(n_t.cpu().numpy())
        toks.append(o_t.cpu().numpy())
    n, toks = np.concatenate(ns), np.concatenate(toks)
    for i in range(K + 1):
        want = oracle.target_row(logits[i], T, tp)
        present = n >= i
        obs = np.bincount(toks[present, i], minlength=V).astype(np.float64)
        assert obs[want == 0].sum() == 0, "token outside the top-p set emitted"
        keep = want > 0
        if keep.sum() == 1:   # a one-token set: the check above is the whole law
            print("T=%.1f top_p=%.1f position %d: one-token set" % (T, tp, i))
            continue
        pv = _chi2(obs[keep], want[keep])
        print("T=%.1f top_p=%.1f position %d: %d samples, chi2 p=%.3g" % (T, tp, i, present.sum(), pv))
        assert pv > 1e-3
