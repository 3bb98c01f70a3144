"""GPU parity of spec_verify_sample against the CPU oracle.

Accepted counts and emitted tokens must match bit for bit, except from the
first position the oracle decided within 1e-6 of its threshold (such
sequences are counted and printed).  Statistical checks run the GPU path
itself: emitted tokens follow the target rows, and the mean tokens per round
matches (1 - a^(K+1)) / (1 - a).
"""
import numpy as np
import pytest
import torch
from scipy import stats
from scipy.special import softmax

import speculative_decoding_verify_attn_amd as sv
import workloads as W
from .gpu_helpers import compare_sampler, dev, run_sample, upload_sample

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4", "c5a"])
def test_config_parity(name):
    s = W.make_sample(name, seed=0)
    n, toks, ap = run_sample(s)
    mism, flagged, ref = compare_sampler(s, n, toks)
    print("%s: B=%d mismatches=%d near-threshold=%d mean accepted=%.3f"
          % (name, s.B, mism, flagged, float(n.mean())))
    assert mism == 0
    # acceptance ratios agree with the oracle wherever the oracle evaluated them
    for b in range(s.B):
        for i in range(int(ref["num_accepted"][b]) + (1 if ref["num_accepted"][b] < s.K else 0)):
            assert abs(ap[b, i] - ref["accept_ratio"][b, i]) <= 1e-6


SHAPES = [
    # (seed, B, K, V, sigma, noise)
    (1, 64, 4, 1024, 2.0, 0.5),
    (2, 33, 1, 8193, 3.0, 1.0),     # two chunks, 1-entry tail, K = 1
    (3, 17, 15, 777, 2.0, 1.0),     # K = 15, V not a multiple of 4 (scalar path)
    (4, 9, 3, 1, 1.0, 1.0),         # V = 1
    (5, 12, 6, 30001, 3.0, 2.0),    # scalar path, several chunks
    (6, 256, 2, 64, 0.5, 0.1),      # high acceptance
    (7, 40, 5, 16384, 3.0, 3.0),    # low acceptance, exact chunk multiple
    (8, 64, 3, 99001, 2.0, 1.5),    # decide workgroups of 4 sub-chunks, the last one with 1; scalar path
    (9, 100, 2, 50000, 3.0, 1.0),   # decide workgroups of 3 sub-chunks, the last one with 1
]


@pytest.mark.parametrize("case", SHAPES, ids=[str(c[0]) for c in SHAPES])
def test_shapes_parity(case):
    seed, B, K, V, sigma, noise = case
    s = W.make_sample_from_params(seed, B, K, V, sigma, noise)
    n, toks, _ = run_sample(s)
    mism, flagged, _ = compare_sampler(s, n, toks)
    print("case %d mismatches=%d flagged=%d" % (seed, mism, flagged))
    assert mism == 0


def test_edge_uniforms_and_degenerate_rows():
    V, K, B = 64, 3, 6
    rng = np.random.default_rng(0)
    lg = (rng.standard_normal((B, K + 1, V)) * 2).astype(np.float32)
    q = softmax(lg[:, :K].astype(np.float64) + rng.standard_normal((B, K, V)), axis=-1).astype(np.float32)
    tok = rng.integers(0, V, size=(B, K)).astype(np.int32)
    u = np.zeros((B, K + 1), np.float32)
    u[1] = np.float32(np.nextafter(np.float32(1), np.float32(0)))     # reject unless p >= q
    u[2, K] = np.float32(np.nextafter(np.float32(1), np.float32(0)))  # last positive weight
    lg[3] = -np.inf                                                   # one-hot targets
    lg[3, :, 5] = 0.0
    q[4] = softmax(lg[4, :K].astype(np.float64), axis=-1).astype(np.float32)  # q ~= p
    s = W.SampleInputs(lg, q, tok, u)
    n, toks, _ = run_sample(s)
    mism, flagged, ref = compare_sampler(s, n, toks)
    assert mism == 0
    assert np.all(toks[3, :n[3] + 1] == 5)


def test_deterministic_and_workspace_reusable():
    s = W.make_sample_from_params(11, 24, 5, 50000, 3.0, 1.0)
    t = upload_sample(s)
    ws = sv.alloc_workspace(sv.sample_workspace_size(s.B, s.K, s.V), dev())
    ws.fill_(0xAB)  # contents before the call must not matter
    n1, t1, a1 = run_sample(s, t, ws)
    for _ in range(5):
        n2, t2, a2 = run_sample(s, t, ws)
        assert np.array_equal(n1, n2) and np.array_equal(t1, t2) and np.array_equal(a1, a2, equal_nan=True)


def _gpu_trials(logits, q, N, seed, calls):
    """calls x N rounds through the GPU path with fixed rows, fresh draft tokens
    and uniforms per round."""
    K1, V = logits.shape
    K = K1 - 1
    d = dev()
    tl = torch.from_numpy(np.ascontiguousarray(np.broadcast_to(logits, (N, K1, V)))).to(d)
    dp = torch.from_numpy(np.ascontiguousarray(np.broadcast_to(q, (N, K, V)))).to(d)
    ws = sv.alloc_workspace(sv.sample_workspace_size(N, K, V), d)
    rng = np.random.default_rng(seed)
    ns, toks = [], []
    n_t = torch.empty(N, dtype=torch.int32, device=d)
    o_t = torch.empty((N, K1), dtype=torch.int32, device=d)
    for _ in range(calls):
        tok = np.stack([rng.choice(V, size=N, p=q[i].astype(np.float64) / q[i].astype(np.float64).sum())
                        for i in range(K)], axis=1).astype(np.int32)
        u = np.minimum(rng.random((N, K1)).astype(np.float32), np.float32(1 - 2 ** -24))
        sv.spec_verify_sample(tl, dp, torch.from_numpy(tok).to(d), torch.from_numpy(u).to(d), n_t, o_t, ws)
        torch.cuda.synchronize()
        ns.append(n_t.cpu().numpy())
        toks.append(o_t.cpu().numpy())
    return np.concatenate(ns), np.concatenate(toks)


def _chi2(obs, p):
    exp = obs.sum() * p
    small = exp < 5
    if small.any():
        obs = np.append(obs[~small], obs[small].sum())
        exp = np.append(exp[~small], exp[small].sum())
    return stats.chisquare(obs, exp).pvalue


def test_gpu_output_law_matches_target():
    K, V = 4, 64
    rng = np.random.default_rng(5)
    logits = (rng.standard_normal((K + 1, V)) * 2).astype(np.float32)
    q = softmax(logits[:K].astype(np.float64) + 0.8 * rng.standard_normal((K, V)), axis=-1).astype(np.float32)
    n, toks = _gpu_trials(logits, q, 65536, seed=1, calls=16)
    p = softmax(logits.astype(np.float64), axis=-1)
    for i in range(K + 1):
        present = n >= i
        obs = np.bincount(toks[present, i], minlength=V).astype(np.float64)
        pv = _chi2(obs, p[i])
        print("position %d: %d samples, chi2 p=%.3g" % (i, present.sum(), pv))
        assert pv > 1e-3


def test_gpu_mean_tokens_per_round():
    K, V = 5, 32
    rng = np.random.default_rng(6)
    l1 = (rng.standard_normal(V) * 2).astype(np.float32)
    q1 = softmax(l1.astype(np.float64) + 0.7 * rng.standard_normal(V)).astype(np.float32)
    logits = np.repeat(l1[None], K + 1, axis=0)
    q = np.repeat(q1[None], K, axis=0)
    p = softmax(l1.astype(np.float64))
    alpha = float(np.minimum(p, q1.astype(np.float64)).sum())
    n, _ = _gpu_trials(logits, q, 65536, seed=2, calls=16)
    tau = n.astype(np.float64) + 1
    closed = (1 - alpha ** (K + 1)) / (1 - alpha)
    probs = np.array([alpha ** j * (1 - alpha) for j in range(K)] + [alpha ** K])
    vals = np.arange(1, K + 2, dtype=np.float64)
    se = np.sqrt(((vals ** 2 * probs).sum() - closed ** 2) / tau.size)
    print("mean tau %.5f closed form %.5f (se %.2e)" % (tau.mean(), closed, se))
    assert abs(tau.mean() - closed) < 4 * se


# Early exit (large batches, no acceptance-ratio output): the row statistics
# run as two launches and the second skips the sequences that rejected a
# draft among the first half of the positions, so rows after a sequence's
# first rejection are not summarised.  The result must be that of the full
# pass: bit for bit against the same call with acceptance ratios requested
# (which reads every row), and against the oracle.  The workspace starts
# filled with garbage, and a second call on other inputs runs over the
# statistics the first call left, so a skipped row's stale statistics can
# never leak into the output.
EARLY = [
    # (seed, B, K, V, sigma, noise): B * (K+1) * V * 4 >= 64 MiB
    (21, 64, 7, 32768, 3.0, 1.0),
    (22, 64, 7, 32768, 0.5, 0.1),    # high acceptance: most sequences need the later rows
    (23, 64, 7, 32768, 3.0, 4.0),    # low acceptance: most skip them
    (24, 32, 5, 99001, 2.0, 1.5),    # scalar path (V not a multiple of 4)
    (25, 16, 15, 65536, 1.0, 0.5),   # K = 15
    (26, 128, 3, 40000, 2.0, 1.0),   # K = 3: rows 0-1, then 2-3
]


def _sample_no_ratios(s, t, ws):
    d = dev()
    n = torch.full((s.B,), -7, dtype=torch.int32, device=d)
    toks = torch.full((s.B, s.K + 1), -7, dtype=torch.int32, device=d)
    sv.spec_verify_sample(t["logits"], t["probs"], t["tokens"], t["u"], n, toks, ws)
    torch.cuda.synchronize()
    return n.cpu().numpy(), toks.cpu().numpy()


@pytest.mark.parametrize("case", EARLY, ids=[str(c[0]) for c in EARLY])
def test_early_exit_parity(case):
    seed, B, K, V, sigma, noise = case
    assert B * (K + 1) * V * 4 >= 64 * 1024 * 1024
    s = W.make_sample_from_params(seed, B, K, V, sigma, noise)
    t = upload_sample(s)
    ws = sv.alloc_workspace(sv.sample_workspace_size(B, K, V), dev())
    ws.fill_(0xFF)  # NaN statistics wherever a row is not summarised
    n_e, toks_e = _sample_no_ratios(s, t, ws)
    n_f, toks_f, _ = run_sample(s, t=t, ws=ws)  # acceptance ratios requested: every row summarised
    assert np.array_equal(n_e, n_f) and np.array_equal(toks_e, toks_f)
    mism, flagged, _ = compare_sampler(s, n_e, toks_e)
    print("case %d: mean accepted %.2f of %d, mismatches=%d flagged=%d" % (seed, float(n_e.mean()), K, mism, flagged))
    assert mism == 0
    # another batch over the statistics this one left behind
    s2 = W.make_sample_from_params(seed + 100, B, K, V, sigma, noise)
    t2 = upload_sample(s2)
    n2, toks2 = _sample_no_ratios(s2, t2, ws)
    mism2, _, _ = compare_sampler(s2, n2, toks2)
    assert mism2 == 0


def test_early_exit_with_temperatures():
    """Temperature alone keeps the early exit: a mix of temperatures, greedy
    rows (T = 0) among them, on the two-stage path against the full pass and
    the oracle."""
    B, K, V = 64, 7, 32768
    s = W.make_sample_from_params(27, B, K, V, 3.0, 1.0)
    rng = np.random.default_rng(28)
    temp = rng.choice(np.array([0.0, 0.4, 0.8, 1.0, 1.6], np.float32), size=B)
    arg = np.argmax(s.target_logits, axis=-1)  # greedy rows accept only the argmax
    take = rng.random((B, K)) < 0.7
    s = W.SampleInputs(s.target_logits, s.draft_probs,
                       np.where(take, arg[:, :K], s.draft_tokens).astype(np.int32), s.uniforms)
    t = upload_sample(s)
    d = dev()
    ws = sv.alloc_workspace(sv.sample_workspace_size(B, K, V), d)
    ws.fill_(0xFF)
    tt = torch.from_numpy(temp).to(d)
    n = torch.full((B,), -7, dtype=torch.int32, device=d)
    toks = torch.full((B, K + 1), -7, dtype=torch.int32, device=d)
    sv.spec_verify_sample(t["logits"], t["probs"], t["tokens"], t["u"], n, toks, ws, temperature=tt)
    torch.cuda.synchronize()
    n_e, toks_e = n.cpu().numpy(), toks.cpu().numpy()
    n_f, toks_f, _ = run_sample(s, t=t, ws=ws, temperature=temp)
    assert np.array_equal(n_e, n_f) and np.array_equal(toks_e, toks_f)
    mism, flagged, _ = compare_sampler(s, n_e, toks_e, temperature=temp)
    print("mean accepted %.2f of %d, mismatches=%d flagged=%d" % (float(n_e.mean()), K, mism, flagged))
    assert mism == 0
    assert 0 < (n_e >= K // 2 + K % 2).sum() < B  # both sides of the gate are exercised
