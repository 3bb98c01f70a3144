"""GPU parity of spec_verify_sample_typical (typical acceptance, "50 |
Speculative Decoding" 9.1; not exact) against the CPU oracle.

Accepted counts and emitted tokens bit for bit, except from the first
position the oracle decided within 1e-6 of its threshold or of a CDF edge;
p~(x_i) and the thresholds within 1e-6 (relative to 1) where tested.
Covered: several (eps, delta) on the chunked and scalar paths, mixed
temperatures with greedy rows, masked vocabularies, the closed form on a
uniform target, determinism.
"""
import numpy as np
import pytest
import torch

import oracle
import speculative_decoding_verify_attn_amd as sv
import workloads as W
from .gpu_helpers import dev, upload_sample

pytestmark = pytest.mark.gpu


def _run(s, eps, delta, temperature=None, t=None, ws=None):
    d = dev()
    if t is None:
        t = upload_sample(s)
    n = torch.full((s.B,), -7, dtype=torch.int32, device=d)
    ot = torch.full((s.B, s.K + 1), -7, dtype=torch.int32, device=d)
    pd = torch.full((s.B, s.K), -7.0, dtype=torch.float32, device=d)
    th = torch.full((s.B, s.K), -7.0, dtype=torch.float32, device=d)
    if ws is None:
        ws = sv.alloc_workspace(sv.sample_workspace_size(s.B, s.K, s.V), d)
    temp = None if temperature is None else torch.from_numpy(np.asarray(temperature, np.float32)).to(d)
    sv.spec_verify_sample_typical(t["logits"], t["tokens"], t["u"], n, ot, ws, eps, delta, temperature=temp,
                                  p_draft=pd, threshold=th)
    torch.cuda.synchronize()
    return n.cpu().numpy(), ot.cpu().numpy(), pd.cpu().numpy(), th.cpu().numpy()


def _check(s, eps, delta, temperature=None, label=""):
    n, ot, pd, th = _run(s, eps, delta, temperature)
    ref = oracle.sample_typical(s.target_logits, s.draft_tokens, s.uniforms, eps, delta,
                                temperature=None if temperature is None else np.asarray(temperature, np.float32))
    mism = flagged = 0
    for b in range(s.B):
        k = int(ref["near_pos"][b])
        last = int(ref["num_accepted"][b]) + (1 if ref["num_accepted"][b] < s.K else 0)
        upto = last if k < 0 else min(last, k)
        assert np.all(np.abs(pd[b, :upto] - ref["p_draft"][b, :upto]) <= 1e-6), (label, b)
        assert np.all(np.abs(th[b, :upto] - ref["threshold"][b, :upto]) <= 1e-6), (label, b)
        if k < 0:
            ok = n[b] == ref["num_accepted"][b] and np.array_equal(ot[b], ref["out_tokens"][b])
        else:
            flagged += 1
            ok = np.array_equal(ot[b, :k], ref["out_tokens"][b, :k])
        mism += 0 if ok else 1
    print("%s: mismatches=%d near-threshold=%d mean accepted=%.3f" % (label, mism, flagged, n.mean()))
    return mism


CASES = [
    # (seed, B, K, V, sigma, noise, eps, delta)
    (1, 32, 5, 32000, 2.0, 0.5, 0.09, 0.3),
    (2, 32, 5, 32000, 1.0, 0.5, 0.3, 0.6),
    (3, 16, 4, 777, 2.0, 0.5, 0.05, 0.2),        # scalar path
    (4, 8, 5, 128256, 3.0, 1.0, 0.09, 0.3),      # Llama-3 vocabulary
    (5, 12, 3, 8193, 0.5, 0.3, 0.01, 0.5),       # flat rows, two chunks and a tail
]


@pytest.mark.parametrize("case", CASES, ids=[str(c[0]) for c in CASES])
def test_typical_parity(case):
    seed, B, K, V, sigma, noise, eps, delta = case
    s = W.make_sample_from_params(seed, B, K, V, sigma, noise)
    assert _check(s, eps, delta, label="case %d" % seed) == 0


def test_typical_with_temperatures_and_greedy_rows():
    s = W.make_sample_from_params(6, 48, 5, 50000, 2.0, 0.5)
    rng = np.random.default_rng(7)
    temp = rng.choice(np.array([0.0, 0.5, 1.0, 1.5, 3.0], np.float32), size=s.B)
    arg = np.argmax(s.target_logits, axis=-1)
    tok = np.where(rng.random((s.B, s.K)) < 0.5, arg[:, :s.K], s.draft_tokens).astype(np.int32)
    s = W.SampleInputs(s.target_logits, s.draft_probs, tok, s.uniforms)
    assert _check(s, 0.09, 0.3, temp, "temperatures") == 0


def test_typical_masked_vocabulary():
    s = W.make_sample_from_params(8, 12, 3, 30000, 2.0, 0.5)
    lg = s.target_logits.copy()
    lg[:, :, 8192:16384] = -np.inf
    lg[np.random.default_rng(9).random(lg.shape) < 0.2] = -np.inf
    lg[:, :, 29999] = np.maximum(lg[:, :, 29999], 0.0)
    s = W.SampleInputs(lg, s.draft_probs, s.draft_tokens, s.uniforms)
    assert _check(s, 0.09, 0.3, label="masked") == 0


def test_uniform_target_accepts_everything_below_delta_one():
    B, K, V = 8, 4, 4096
    lg = np.zeros((B, K + 1, V), np.float32)
    tok = np.random.default_rng(10).integers(0, V, size=(B, K)).astype(np.int32)
    s = W.SampleInputs(lg, np.full((B, K, V), 1.0 / V, np.float32), tok,
                       np.random.default_rng(11).random((B, K + 1)).astype(np.float32))
    n, _, _, th = _run(s, 0.5, 0.9)
    assert np.all(n == K)
    assert np.allclose(th, 0.9 / V, rtol=1e-5)
    n, _, _, _ = _run(s, 0.5, 1.1)
    assert np.all(n == 0)


def test_typical_deterministic():
    s = W.make_sample_from_params(12, 16, 5, 50000, 2.0, 0.5)
    t = upload_sample(s)
    ws = sv.alloc_workspace(sv.sample_workspace_size(s.B, s.K, s.V), dev())
    first = _run(s, 0.09, 0.3, t=t, ws=ws)
    for _ in range(3):
        again = _run(s, 0.09, 0.3, t=t, ws=ws)
        for x, y in zip(first, again):
            assert np.array_equal(x, y, equal_nan=True)
