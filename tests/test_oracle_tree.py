"""Pins of the oracle's tree verification ("KV Cache + Speculative Decoding"
8.2 and Q14: the draft tree's nodes are flattened in BFS order and scored in
one target forward, node i attending to its ancestors and itself; exact
verification keeps the rejection rule of "50 | Speculative Decoding" 3.1).

Attention:
  * chain ancestor sets reproduce the causal oracle bit for bit;
  * every node's output equals plain causal attention over a rebuilt
    sequence holding the prefix and the node's root path, nothing else.
Sampler (reading: siblings tried in BFS order, each against the residual
left by the rejected ones):
  * a chain tree is the chain sampler, bit for bit;
  * exact law in rational arithmetic for a root with 2 or 3 i.i.d. drafted
    children: the first emitted token is distributed exactly as p (the
    property that makes the rule exact), and the oracle's empirical law of
    (first, second) matches that law by chi-square;
  * a worked third-sibling ratio in fractions;
  * every emitted position of a depth-3 binary tree follows its target row
    (chi-square over 10^6 rounds);
  * structural invariants of path and out_tokens.
"""
from fractions import Fraction
from itertools import product

import numpy as np
import pytest
from scipy.special import softmax

import oracle
import workloads as W
from .test_oracle_sampler import U_MAX, chi2_pvalue


# ------------------------------------------------------------------ attention

def test_chain_masks_are_the_causal_mask():
    a = W.make_attn_from_lens(81, 3, 6, 8, 2, 64, [6, 40, 77], kv="bf16")
    chain = oracle.tree_masks(np.broadcast_to(W.tree_parents((1,) * 5), (3, 6)))
    assert list(chain[0]) == [(2 << t) - 1 for t in range(6)]
    o1 = oracle.attn(a.q, a.k_cache, a.v_cache, a.block_table, a.context_lens, kv_dtype=a.kv_dtype)
    o2 = oracle.attn(a.q, a.k_cache, a.v_cache, a.block_table, a.context_lens, kv_dtype=a.kv_dtype,
                     tree_mask=chain)
    assert np.array_equal(o1, o2)


@pytest.mark.parametrize("shape", ["binary3", "wide5x2", "top3-2-1"])
def test_node_sees_exactly_prefix_and_root_path(shape):
    par = W.tree_parents(W.TREE_SHAPES[shape])
    N = par.shape[0]
    B, Hq, Hkv, d = 2, 8, 2, 64
    lens = [N + 3, N + 37]
    a = W.make_attn_from_lens(82, B, N, Hq, Hkv, d, lens, kv="f32")
    masks = oracle.tree_masks(np.broadcast_to(par, (B, N)))
    got = oracle.attn(a.q, a.k_cache, a.v_cache, a.block_table, a.context_lens, kv_dtype=a.kv_dtype,
                      tree_mask=masks)
    for b in range(B):
        L = lens[b]
        P = L - N
        pos = np.arange(L)
        kseq = a.k_cache[a.block_table[b, pos // 16], pos % 16]   # [L, Hkv, d]
        vseq = a.v_cache[a.block_table[b, pos // 16], pos % 16]
        for t in range(N):
            path, c = [], t            # the root path, walked up the parents
            while c >= 0:
                path.append(c)
                c = int(par[c])
            path = path[::-1]
            assert [j for j in range(N) if (masks[b, t] >> j) & 1] == path
            keep = np.concatenate([np.arange(P), P + np.array(path)])
            Lp = keep.size
            nb = (Lp + 15) // 16
            kc = np.full((nb + 1, 16, Hkv, d), np.nan, np.float32)
            vc = np.full((nb + 1, 16, Hkv, d), np.nan, np.float32)
            kc.reshape(-1, Hkv, d)[:Lp] = kseq[keep]
            vc.reshape(-1, Hkv, d)[:Lp] = vseq[keep]
            ref = oracle.attn(a.q[b:b + 1, t:t + 1], kc, vc, np.arange(nb, dtype=np.int32)[None],
                              np.array([Lp], np.int32), kv_dtype=W.KV_F32)
            assert np.allclose(got[b, t], ref[0, 0], rtol=0, atol=1e-12), (shape, b, t)


def test_bad_ancestor_sets_are_rejected():
    a = W.make_attn_from_lens(83, 1, 3, 4, 1, 64, [10], kv="f32")
    with pytest.raises(ValueError):   # node 1 without itself
        oracle.attn(a.q, a.k_cache, a.v_cache, a.block_table, a.context_lens, kv_dtype=a.kv_dtype,
                    tree_mask=np.array([[1, 1, 5]], np.uint32))
    with pytest.raises(ValueError):   # node 0 seeing a later node
        oracle.attn(a.q, a.k_cache, a.v_cache, a.block_table, a.context_lens, kv_dtype=a.kv_dtype,
                    tree_mask=np.array([[3, 3, 5]], np.uint32))


# -------------------------------------------------------------------- sampler

def test_chain_tree_is_the_chain_sampler():
    s = W.make_sample_from_params(84, 32, 5, 3000, 3.0, 1.0)
    B, K, V = s.B, s.K, s.V
    N = K + 1
    par = np.broadcast_to(W.tree_parents((1,) * K), (B, N))
    tokens = np.zeros((B, N), np.int32)
    tokens[:, 1:] = s.draft_tokens
    probs = np.zeros((B, N, V), np.float32)
    probs[:, :K] = s.draft_probs
    u = np.zeros((B, N), np.float32)
    u[:, 1:] = s.uniforms[:, :K]
    u[:, 0] = s.uniforms[:, K]
    a = oracle.sample(s.target_logits, s.draft_probs, s.draft_tokens, s.uniforms)
    t = oracle.sample_tree(s.target_logits, probs, tokens, par, u)
    assert np.array_equal(a["num_accepted"], t["num_accepted"])
    assert np.array_equal(a["out_tokens"], t["out_tokens"])
    assert np.array_equal(a["near_pos"], t["near_pos"])
    for b in range(B):
        n = a["num_accepted"][b]
        assert list(t["path"][b, :n]) == list(range(1, n + 1))
        for i in range(min(n + 1, K)):
            assert t["accept_ratio"][b, i + 1] == a["accept_ratio"][b, i]


def _rrs_law(p, q, child_rows, m):
    """Exact law of one verify step of a root with m leaf children drafted
    i.i.d. from q, by recursive rejection: outcomes (x, y) = child token x
    accepted then bonus y from child_rows[x]; (z,) = all rejected, z drawn from
    the final residual."""
    V = len(p)
    law = {}
    for xs in product(range(V), repeat=m):
        pr = Fraction(1)
        for x in xs:
            pr *= q[x]
        if pr == 0:
            continue
        C = Fraction(0)
        for x in xs:
            R = [max(Fraction(0), p[j] - C * q[j]) for j in range(V)]
            Z = sum(R)
            pk = R[x] / Z if Z > 0 else Fraction(0)
            acc = min(Fraction(1), pk / q[x])
            for y in range(V):
                law[(x, y)] = law.get((x, y), Fraction(0)) + pr * acc * child_rows[x][y]
            pr *= 1 - acc
            C += Z
            if pr == 0:
                break
        if pr:
            R = [max(Fraction(0), p[j] - C * q[j]) for j in range(V)]
            Z = sum(R)
            fin = [r / Z for r in R] if Z > 0 else list(p)
            for z in range(V):
                law[(z,)] = law.get((z,), Fraction(0)) + pr * fin[z]
    return law


P3 = [Fraction(1, 2), Fraction(1, 3), Fraction(1, 6)]
Q3 = [Fraction(1, 4), Fraction(1, 4), Fraction(1, 2)]
ROWS3 = [[Fraction(1, 3)] * 3, [Fraction(1, 2), Fraction(1, 4), Fraction(1, 4)],
         [Fraction(1, 6), Fraction(1, 6), Fraction(2, 3)]]


@pytest.mark.parametrize("m", [2, 3])
def test_exact_law_of_recursive_rejection(m):
    law = _rrs_law(P3, Q3, ROWS3, m)
    assert sum(law.values()) == 1
    first = [sum(v for k, v in law.items() if k[0] == x) for x in range(3)]
    assert first == P3          # the emitted token is distributed exactly as p
    # the oracle's empirical law of the same step
    N, V, R = 1 + m, 3, 400_000
    par = np.broadcast_to(np.array([-1] + [0] * m, np.int32), (R, N))
    logits = np.zeros((R, N, V), np.float32)
    logits[:, 0] = np.log(np.array([float(x) for x in P3], np.float64)).astype(np.float32)
    q = np.zeros((R, N, V), np.float32)
    q[:, 0] = np.array([float(x) for x in Q3], np.float32)
    rng = np.random.default_rng(85 + m)
    toks = np.zeros((R, N), np.int32)
    toks[:, 1:] = rng.choice(V, size=(R, m), p=np.array([float(x) for x in Q3]))
    rows = np.log(np.array([[float(y) for y in r] for r in ROWS3])).astype(np.float32)
    logits[:, 1:] = rows[toks[:, 1:]]
    u = np.minimum(rng.random((R, N)).astype(np.float32), U_MAX)
    res = oracle.sample_tree(logits, q, toks, par, u)
    keys = sorted(law)
    idx = {k: i for i, k in enumerate(keys)}
    obs = np.zeros(len(keys))
    for n, ot in zip(res["num_accepted"], res["out_tokens"]):
        obs[idx[(int(ot[0]), int(ot[1])) if n == 1 else (int(ot[0]),)]] += 1
    pv = chi2_pvalue(obs, np.array([float(law[k]) for k in keys]))
    assert pv > 1e-3, pv


def test_third_sibling_ratio_worked_example():
    # p = (9,7,9,4)/29, q = (5,5,8,9)/27, children tokens (3, 2, 1): the three
    # tests run against p, then max(0, p - q)/Z_2, then max(0, p - (1 + Z_2) q)/Z_3;
    # by hand in fractions the ratios are 12/29, 33/136 and 1269/1280, all
    # below 1, so uniforms just under 1 reject all three
    p = [Fraction(x, 29) for x in (9, 7, 9, 4)]
    q = [Fraction(x, 27) for x in (5, 5, 8, 9)]
    want = [Fraction(12, 29), Fraction(33, 136), Fraction(1269, 1280)]
    logits = np.zeros((1, 4, 4), np.float32)
    logits[0, 0] = np.log([float(x) for x in p])
    probs = np.zeros((1, 4, 4), np.float32)
    probs[0, 0] = [float(x) for x in q]
    toks = np.array([[0, 3, 2, 1]], np.int32)
    par = np.array([[-1, 0, 0, 0]], np.int32)
    u = np.array([[0.5, U_MAX, U_MAX, U_MAX]], np.float32)
    res = oracle.sample_tree(logits, probs, toks, par, u)
    for c in range(3):
        assert abs(res["accept_ratio"][0, c + 1] - float(want[c])) < 1e-6, c
    assert res["num_accepted"][0] == 0
    # the final draw comes from max(0, p - (1 + Z_2 + Z_3) q): only token 0 survives
    assert res["out_tokens"][0, 0] == 0


def test_every_emitted_position_follows_its_row_in_a_binary_tree():
    par = W.tree_parents((2, 2, 2))
    N, V, R = par.shape[0], 10, 1_000_000
    rng = np.random.default_rng(86)
    depth = np.zeros(N, int)
    for c in range(1, N):
        depth[c] = depth[par[c]] + 1
    lrows = (rng.standard_normal((4, V)) * 1.5).astype(np.float32)   # target row by depth
    qrows = softmax(lrows.astype(np.float64) + 0.8 * rng.standard_normal((4, V)), axis=-1)
    logits = np.ascontiguousarray(np.broadcast_to(lrows[depth], (R, N, V)))
    q = np.ascontiguousarray(np.broadcast_to(qrows[depth].astype(np.float32), (R, N, V)))
    toks = np.zeros((R, N), np.int32)
    for c in range(1, N):
        d0 = depth[par[c]]
        toks[:, c] = rng.choice(V, size=R, p=qrows[d0])
    u = np.minimum(rng.random((R, N)).astype(np.float32), U_MAX)
    res = oracle.sample_tree(logits, q, toks, np.broadcast_to(par, (R, N)), u)
    n, ot = res["num_accepted"], res["out_tokens"]
    pt = softmax(lrows.astype(np.float64), axis=-1)
    for i in range(4):
        present = n >= i
        if present.sum() < 20_000:
            continue
        pv = chi2_pvalue(np.bincount(ot[present, i], minlength=V), pt[i])
        assert pv > 1e-3, (i, pv)


def test_path_and_tokens_are_consistent():
    for shape in W.TREE_SHAPES.values():
        par = W.tree_parents(shape)
        t = W.make_tree(87, 64, par, 500, 2.0, 0.4)
        res = oracle.sample_tree(t.target_logits, t.draft_probs, t.tokens, t.parents, t.uniforms)
        for b in range(t.B):
            n = res["num_accepted"][b]
            node = 0
            for i in range(n):
                c = res["path"][b, i]
                assert t.parents[b, c] == node
                assert res["out_tokens"][b, i] == t.tokens[b, c]
                node = c
            assert 0 <= res["out_tokens"][b, n] < t.V
            assert np.all(res["out_tokens"][b, n + 1:] == -1) and np.all(res["path"][b, n:] == -1)
            # a node is tested only if its parent is on the path and its earlier siblings were rejected
            tested = np.nonzero(~np.isnan(res["accept_ratio"][b]))[0]
            on_path = [0] + list(res["path"][b, :n])
            assert all(t.parents[b, c] in on_path for c in tested)
