"""Pins of the oracle's tree commit: after tree verification the cache keeps
the root and the accepted path at consecutive positions ("KV Cache +
Speculative Decoding" 8.2, with 7.6's note that a paged cache rolls back by
editing its bookkeeping).

  * a chain path moves nothing and equals the chain's rollback (K = N-1);
  * the committed cache, read back through the block table, is the prefix,
    the root and the path's nodes in order -- gathered here independently
    (bit for bit for fp32 and bf16; E4M3 values that change page are
    re-encoded for the destination page, checked against torch's cast);
  * attention at the new last position over the committed cache equals
    attention over a cache holding exactly that linear sequence;
  * nothing outside the moved positions changes.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W


def _random_paths(rng, B, N):
    par = np.empty((B, N), np.int32)
    par[:, 0] = -1
    for c in range(1, N):
        par[:, c] = rng.integers(0, c, size=B)
    paths = np.full((B, N), -1, np.int32)
    n = np.zeros(B, np.int32)
    for b in range(B):
        end = int(rng.integers(0, N))
        walk = []
        while end > 0:
            walk.append(end)
            end = int(par[b, end])
        walk = walk[::-1]
        n[b] = len(walk)
        paths[b, :len(walk)] = walk
    return paths, n


def _gather(cache, table, b, pos):
    return cache[table[b, pos // 16], pos % 16]


def test_chain_path_moves_nothing_and_is_the_rollback():
    B, N = 4, 6
    a = W.make_attn_from_lens(101, B, N, 8, 2, 64, [6, 40, 77, 160], kv="bf16")
    n = np.array([0, 5, 2, 3], np.int32)
    path = np.tile(np.arange(1, N + 1, dtype=np.int32), (B, 1))
    kc, vc, lens, pages = oracle.tree_commit(path, n, a.k_cache, a.v_cache, a.block_table, a.context_lens,
                                             a.kv_dtype)
    assert np.array_equal(kc, a.k_cache) and np.array_equal(vc, a.v_cache)
    l2, p2 = oracle.rollback(n, a.context_lens, N - 1)
    assert np.array_equal(lens, l2) and np.array_equal(pages, p2)


@pytest.mark.parametrize("kv", ["f32", "bf16", "fp8"])
def test_committed_cache_is_prefix_root_and_path(kv):
    rng = np.random.default_rng(102)
    B, N = 12, 16
    # roots late in a page, so that moved nodes often change page
    lens = [16, 17, 31, 100, 250, 511, 30, 45, 61, 78, 95, 126]
    a = W.make_attn_from_lens(103, B, N, 8, 2, 64, lens, kv=kv, extra_blocks=2)
    path, n = _random_paths(rng, B, N)
    crossing = sum(int(a.block_table[b, (lens[b] - N + path[b, i]) // 16] != a.block_table[b, (lens[b] - N + 1 + i) // 16])
                   for b in range(B) for i in range(n[b]))
    assert crossing > 0
    kc, vc, new_lens, pages = oracle.tree_commit(path, n, a.k_cache, a.v_cache, a.block_table, a.context_lens,
                                                 a.kv_dtype, a.k_scale, a.v_scale)
    touched = np.zeros(a.k_cache.shape[:2], bool)
    for b in range(B):
        L, base = lens[b], lens[b] - N
        assert new_lens[b] == base + 1 + n[b] and pages[b] == (new_lens[b] + 15) // 16
        for p in range(base + 1):   # prefix and root unchanged
            assert np.array_equal(_gather(kc, a.block_table, b, p).view(np.uint8),
                                  _gather(a.k_cache, a.block_table, b, p).view(np.uint8))
        for i in range(n[b]):
            ps, pd = base + path[b, i], base + 1 + i
            touched[a.block_table[b, pd // 16], pd % 16] = True
            for old, new, scale in ((a.k_cache, kc, a.k_scale), (a.v_cache, vc, a.v_scale)):
                src = _gather(old, a.block_table, b, ps)
                got = _gather(new, a.block_table, b, pd)
                pgs, pgd = a.block_table[b, ps // 16], a.block_table[b, pd // 16]
                if a.kv_dtype != W.KV_FP8_E4M3 or pgs == pgd:
                    assert np.array_equal(got.view(np.uint8), src.view(np.uint8)), (kv, b, i)
                else:
                    vals = torch.from_numpy(src.copy()).view(torch.float8_e4m3fn).float().numpy()
                    x = (vals * np.float32(scale[pgs])).astype(np.float32)
                    q = (x / np.float32(scale[pgd])).astype(np.float32)
                    want = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
                    big = np.abs(q) > 464
                    want[big] = np.where(q[big] > 0, 0x7E, 0xFE)
                    assert np.array_equal(got, want), (kv, b, i)
    for old, new in ((a.k_cache, kc), (a.v_cache, vc)):
        ob = old.view(np.uint8).reshape(old.shape[0], 16, -1)
        nb = new.view(np.uint8).reshape(new.shape[0], 16, -1)
        assert np.array_equal(ob[~touched], nb[~touched])


def test_attention_after_commit_sees_the_linear_sequence():
    rng = np.random.default_rng(104)
    B, N, Hq, Hkv, d = 3, 15, 8, 2, 64
    lens = [15, 90, 333]
    a = W.make_attn_from_lens(105, B, N, Hq, Hkv, d, lens, kv="f32")
    path, n = _random_paths(rng, B, N)
    kc, vc, new_lens, _ = oracle.tree_commit(path, n, a.k_cache, a.v_cache, a.block_table, a.context_lens,
                                             a.kv_dtype)
    q1 = np.ascontiguousarray(a.q[:, :1])
    got = oracle.attn(q1, kc, vc, a.block_table, new_lens, kv_dtype=a.kv_dtype)
    for b in range(B):
        base = lens[b] - N
        order = list(range(base + 1)) + [base + int(c) for c in path[b, :n[b]]]
        Lp = len(order)
        nb = (Lp + 15) // 16
        kl = np.full((nb + 1, 16, Hkv, d), np.nan, np.float32)
        vl = np.full((nb + 1, 16, Hkv, d), np.nan, np.float32)
        pos = np.array(order)
        kl.reshape(-1, Hkv, d)[:Lp] = a.k_cache[a.block_table[b, pos // 16], pos % 16]
        vl.reshape(-1, Hkv, d)[:Lp] = a.v_cache[a.block_table[b, pos // 16], pos % 16]
        ref = oracle.attn(q1[b:b + 1], kl, vl, np.arange(nb, dtype=np.int32)[None], np.array([Lp], np.int32),
                          kv_dtype=W.KV_F32)
        assert np.allclose(got[b], ref[0], rtol=0, atol=1e-12)


def test_bad_paths_are_rejected():
    a = W.make_attn_from_lens(106, 1, 6, 4, 1, 64, [20], kv="f32")
    for path, n in (([3, 2, -1, -1, -1, -1], 2), ([0, -1, -1, -1, -1, -1], 1), ([1, 2, 3, 4, 5, 6], 6)):
        with pytest.raises(ValueError):
            oracle.tree_commit(np.array([path], np.int32), np.array([n], np.int32), a.k_cache, a.v_cache,
                               a.block_table, a.context_lens, a.kv_dtype)
