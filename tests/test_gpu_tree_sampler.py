"""GPU parity of spec_verify_sample_tree (tree verification, "KV Cache +
Speculative Decoding" 8.2, with the rejection rule applied per rejected
sibling) against the CPU oracle.

Same bar as the chain: accepted counts, emitted tokens and accepted paths bit
for bit, except from the first position the oracle decided within 1e-6 of a
threshold; acceptance ratios within 1e-6 where tested.  Covered: the tree
shapes of the workload module on the chunked and scalar paths, a random tree
per sequence, a chain tree against the chain sampler, determinism, and the
law of the emitted tokens from the GPU path itself.
"""
import numpy as np
import pytest
import torch
from scipy.special import softmax

import oracle
import speculative_decoding_verify_attn_amd as sv
import workloads as W
from .gpu_helpers import dev, run_sample
from .test_gpu_sampler import _chi2

pytestmark = pytest.mark.gpu


def max_children(parents):
    par = np.asarray(parents)
    return int(max([0] + [np.bincount(row[1:], minlength=par.shape[1]).max() for row in par if row.size > 1]))


def _upload(t):
    d = dev()
    return {k: torch.from_numpy(np.ascontiguousarray(v)).to(d) for k, v in dict(
        logits=t.target_logits, probs=t.draft_probs, tokens=t.tokens, parents=t.parents, u=t.uniforms).items()}


def _run(t, g=None, ws=None):
    d = dev()
    if g is None:
        g = _upload(t)
    n = torch.full((t.B,), -7, dtype=torch.int32, device=d)
    ot = torch.full((t.B, t.N), -7, dtype=torch.int32, device=d)
    path = torch.full((t.B, t.N), -7, dtype=torch.int32, device=d)
    ap = torch.full((t.B, t.N), -7.0, dtype=torch.float32, device=d)
    if ws is None:
        ws = sv.alloc_workspace(sv.sample_tree_workspace_size(t.B, t.N, t.V), d)
    sv.spec_verify_sample_tree(g["logits"], g["probs"], g["tokens"], g["parents"], g["u"], n, ot, path, ws,
                               max_children(t.parents), accept_prob=ap)
    torch.cuda.synchronize()
    return n.cpu().numpy(), ot.cpu().numpy(), path.cpu().numpy(), ap.cpu().numpy()


def _compare(t, got, label):
    n, ot, path, ap = got
    ref = oracle.sample_tree(t.target_logits, t.draft_probs, t.tokens, t.parents, t.uniforms)
    mism = flagged = 0
    for b in range(t.B):
        k = int(ref["near_pos"][b])
        if k < 0:
            ok = (n[b] == ref["num_accepted"][b] and np.array_equal(ot[b], ref["out_tokens"][b])
                  and np.array_equal(path[b], ref["path"][b]))
            tested = ~np.isnan(ref["accept_ratio"][b])
            ok = ok and np.array_equal(np.isnan(ap[b]), ~tested)
            ok = ok and np.all(np.abs(ap[b, tested] - ref["accept_ratio"][b, tested]) <= 1e-6)
        else:
            flagged += 1
            ok = np.array_equal(ot[b, :k], ref["out_tokens"][b, :k]) and np.array_equal(path[b, :k], ref["path"][b, :k])
        mism += 0 if ok else 1
    print("%s: B=%d mismatches=%d near-threshold=%d mean accepted=%.3f" % (label, t.B, mism, flagged, n.mean()))
    return mism


CASES = [
    # (seed, shape, B, V, sigma, noise)
    (1, "binary3", 16, 32000, 3.0, 1.0),
    (2, "wide5x2", 16, 32000, 2.0, 0.5),
    (3, "top3-2-1", 8, 128256, 3.0, 1.0),
    (4, "binary3", 12, 777, 2.0, 0.7),      # scalar path
    (5, "wide5x2", 8, 8193, 1.0, 0.3),      # two chunks and a 1-entry tail, high acceptance
    (6, "chain5", 16, 32000, 3.0, 1.0),
    (7, "wide5x2", 24, 99001, 2.0, 1.0),    # decide workgroups of 2 sub-chunks, the last one with 1; scalar path
    (8, "binary3", 48, 50000, 3.0, 1.0),    # decide workgroups of 2 sub-chunks, the last one with 1
]


@pytest.mark.parametrize("case", CASES, ids=[str(c[0]) for c in CASES])
def test_tree_shapes_parity(case):
    seed, shape, B, V, sigma, noise = case
    t = W.make_tree(seed, B, W.tree_parents(W.TREE_SHAPES[shape]), V, sigma, noise)
    assert _compare(t, _run(t), "case %d %s V=%d" % (seed, shape, V)) == 0


def test_random_tree_per_sequence():
    rng = np.random.default_rng(7)
    B, N, V = 32, 16, 5000
    par = np.empty((B, N), np.int32)
    par[:, 0] = -1
    for c in range(1, N):
        par[:, c] = rng.integers(0, c, size=B)
    t = W.make_tree(8, B, par, V, 2.0, 0.5)
    assert _compare(t, _run(t), "random trees") == 0


def test_single_node_tree_is_a_bonus_draw():
    t = W.make_tree(9, 8, np.array([-1], np.int32), 3000, 2.0, 1.0)
    got = _run(t)
    assert np.all(got[0] == 0)
    assert _compare(t, got, "root only") == 0


def test_chain_tree_equals_the_chain_sampler():
    s = W.make_sample_from_params(10, 24, 5, 32000, 3.0, 1.0)
    B, K, V = s.B, s.K, s.V
    N = K + 1
    tokens = np.zeros((B, N), np.int32)
    tokens[:, 1:] = s.draft_tokens
    probs = np.zeros((B, N, V), np.float32)
    probs[:, :K] = s.draft_probs
    u = np.zeros((B, N), np.float32)
    u[:, 1:] = s.uniforms[:, :K]
    u[:, 0] = s.uniforms[:, K]
    t = W.TreeInputs(s.target_logits, probs, tokens, np.ascontiguousarray(
        np.broadcast_to(W.tree_parents((1,) * K), (B, N))), u)
    n1, ot1, _ = run_sample(s)
    n2, ot2, path, _ = _run(t)
    assert np.array_equal(n1, n2) and np.array_equal(ot1, ot2)


def test_children_beyond_max_children_are_skipped():
    """A star of 6 children with max_children = 3: the GPU must match the
    oracle run on the tree with children 4..6 removed (their columns left
    untested)."""
    par = np.array([-1, 0, 0, 0, 0, 0, 0], np.int32)
    t = W.make_tree(13, 32, par, 4000, 2.0, 1.5)
    g = _upload(t)
    d = dev()
    n = torch.empty(t.B, dtype=torch.int32, device=d)
    ot = torch.empty((t.B, t.N), dtype=torch.int32, device=d)
    path = torch.empty((t.B, t.N), dtype=torch.int32, device=d)
    ws = sv.alloc_workspace(sv.sample_tree_workspace_size(t.B, t.N, t.V), d)
    sv.spec_verify_sample_tree(g["logits"], g["probs"], g["tokens"], g["parents"], g["u"], n, ot, path, ws, 3)
    torch.cuda.synchronize()
    keep = 4
    sub = W.TreeInputs(np.ascontiguousarray(t.target_logits[:, :keep]), np.ascontiguousarray(t.draft_probs[:, :keep]),
                       np.ascontiguousarray(t.tokens[:, :keep]), np.ascontiguousarray(t.parents[:, :keep]),
                       np.ascontiguousarray(t.uniforms[:, :keep]))
    ref = oracle.sample_tree(sub.target_logits, sub.draft_probs, sub.tokens, sub.parents, sub.uniforms)
    n, ot = n.cpu().numpy(), ot.cpu().numpy()
    for b in range(t.B):
        k = int(ref["near_pos"][b])
        if k < 0:
            assert n[b] == ref["num_accepted"][b]
            assert np.array_equal(ot[b, :keep], ref["out_tokens"][b]) and np.all(ot[b, keep:] == -1)


def test_deterministic_and_workspace_reusable():
    t = W.make_tree(11, 16, W.tree_parents(W.TREE_SHAPES["wide5x2"]), 50000, 2.0, 0.5)
    g = _upload(t)
    ws = sv.alloc_workspace(sv.sample_tree_workspace_size(t.B, t.N, t.V), dev())
    ws.fill_(0xAB)
    first = _run(t, g, ws)
    for _ in range(4):
        again = _run(t, g, ws)
        for x, y in zip(first, again):
            assert np.array_equal(x, y, equal_nan=True)


def test_gpu_output_law_follows_the_rows():
    """Binary tree of depth 3 whose target and draft rows depend only on the
    depth: every emitted position i must follow the depth-i target row."""
    par = W.tree_parents((2, 2, 2))
    N, V, R, calls = par.shape[0], 24, 65536, 8
    rng = np.random.default_rng(12)
    depth = np.zeros(N, int)
    for c in range(1, N):
        depth[c] = depth[par[c]] + 1
    lrows = (rng.standard_normal((4, V)) * 1.5).astype(np.float32)
    qrows = softmax(lrows.astype(np.float64) + 0.8 * rng.standard_normal((4, V)), axis=-1)
    d = dev()
    logits = torch.from_numpy(np.ascontiguousarray(np.broadcast_to(lrows[depth], (R, N, V)))).to(d)
    probs = torch.from_numpy(np.ascontiguousarray(np.broadcast_to(qrows[depth].astype(np.float32), (R, N, V)))).to(d)
    parents = torch.from_numpy(np.ascontiguousarray(np.broadcast_to(par, (R, N)))).to(d)
    ws = sv.alloc_workspace(sv.sample_tree_workspace_size(R, N, V), d)
    n_t = torch.empty(R, dtype=torch.int32, device=d)
    o_t = torch.empty((R, N), dtype=torch.int32, device=d)
    p_t = torch.empty((R, N), dtype=torch.int32, device=d)
    ns, toks = [], []
    for _ in range(calls):
        tk = np.zeros((R, N), np.int32)
        for c in range(1, N):
            tk[:, c] = rng.choice(V, size=R, p=qrows[depth[par[c]]])
        u = np.minimum(rng.random((R, N)).astype(np.float32), np.float32(1 - 2 ** -24))
        sv.spec_verify_sample_tree(logits, probs, torch.from_numpy(tk).to(d), parents, torch.from_numpy(u).to(d),
                                   n_t, o_t, p_t, ws, 2)
        torch.cuda.synchronize()
        ns.append(n_t.cpu().numpy())
        toks.append(o_t.cpu().numpy())
    n, toks = np.concatenate(ns), np.concatenate(toks)
    pt = softmax(lrows.astype(np.float64), axis=-1)
    for i in range(4):
        present = n >= i
        pv = _chi2(np.bincount(toks[present, i], minlength=V).astype(np.float64), pt[i])
        print("position %d: %d samples, chi2 p=%.3g" % (i, present.sum(), pv))
        assert pv > 1e-3


def test_star_tree_fifteen_sibling_ranks():
    """A root with fifteen children: fifteen sibling tests in a row, each
    normaliser's coefficient carried through fourteen rank launches."""
    par = np.array([-1] + [0] * 15, np.int32)
    for seed, noise in ((14, 0.3), (15, 2.0)):   # high and low acceptance
        t = W.make_tree(seed, 8, par, 5000, 1.5, noise)
        assert _compare(t, _run(t), "star tree noise %.1f" % noise) == 0
