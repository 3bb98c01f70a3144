"""Pins for the oracle's verify attention (CPU only).

The oracle is checked against things other than itself:
  * torch's own scaled_dot_product_attention (a library routine) on the cache
    gathered into dense [L, Hkv, d] form, decoded with torch's dtype casts,
    broadcast over the group with repeat_interleave and masked with
    tril(diagonal = L_total - L_new) -- the dense formulation of "KV Cache +
    Speculative Decoding" 6.1 and 6.3;
  * closed forms: constant values, zero queries, a single visible key, two
    visible keys, per-head constants that expose the GQA head map;
  * invariance under a consistent relabelling of physical blocks;
  * NaN-poisoned slots, spare blocks and table entries that must never be read.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import workloads as W


def _decode_cache(a: W.AttnInputs, which: str) -> torch.Tensor:
    """Stored cache -> float64 via torch's casts (independent of the oracle's decoders)."""
    c = a.k_cache if which == "k" else a.v_cache
    if a.kv_dtype == W.KV_F32:
        return torch.from_numpy(c).to(torch.float64)
    if a.kv_dtype == W.KV_BF16:
        return torch.from_numpy(c.view(np.int16)).view(torch.bfloat16).to(torch.float64)
    s = a.k_scale if which == "k" else a.v_scale
    x = torch.from_numpy(c).view(torch.float8_e4m3fn).to(torch.float64)
    return x * torch.from_numpy(s).to(torch.float64)[:, None, None, None]


def dense_reference(a: W.AttnInputs, sm_scale=None) -> np.ndarray:
    B, T, Hq, d, Hkv = a.B, a.T, a.Hq, a.d, a.Hkv
    G = Hq // Hkv
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    kd, vd = _decode_cache(a, "k"), _decode_cache(a, "v")
    out = np.empty((B, T, Hq, d))
    for b in range(B):
        L = int(a.context_lens[b])
        pos = torch.arange(L)
        blk = torch.from_numpy(a.block_table[b].astype(np.int64))[pos // W.BLOCK]
        k = kd[blk, pos % W.BLOCK]                           # [L, Hkv, d]
        v = vd[blk, pos % W.BLOCK]
        k = k.permute(1, 0, 2).repeat_interleave(G, dim=0)  # [Hq, L, d]
        v = v.permute(1, 0, 2).repeat_interleave(G, dim=0)
        q = torch.from_numpy(a.q[b]).to(torch.float64).permute(1, 0, 2)  # [Hq, T, d]
        mask = torch.ones(T, L, dtype=torch.bool).tril(diagonal=L - T)
        o = F.scaled_dot_product_attention(q[None], k[None], v[None], attn_mask=mask, scale=sm_scale)
        out[b] = o[0].permute(1, 0, 2).numpy()
    return out


def _oracle(a: W.AttnInputs, **kw):
    return oracle.attn(a.q, a.k_cache, a.v_cache, a.block_table, a.context_lens,
                       kv_dtype=a.kv_dtype, k_scale=a.k_scale, v_scale=a.v_scale, **kw)


def _rel_rows(o, r):
    o = o.reshape(-1, o.shape[-1])
    r = r.reshape(-1, r.shape[-1])
    return np.max(np.abs(o - r), axis=1) / np.max(np.abs(r), axis=1)


CASES = [
    # (seed, B, T, Hq, Hkv, d, lens, kv)
    (1, 1, 5, 4, 1, 64, [256], "f32"),             # the tiny fp32 MQA shape
    (2, 2, 3, 8, 2, 64, [37, 16], "f32"),          # partial and exactly-full last block
    (3, 3, 6, 8, 8, 32, [6, 17, 70], "bf16"),      # MHA (G=1), L_b = T case
    (4, 2, 2, 16, 2, 64, [33, 100], "bf16"),       # K=1
    (5, 2, 8, 8, 1, 128, [129, 40], "fp8"),        # e4m3 with per-block scales
    (6, 1, 1, 4, 2, 16, [1], "f32"),               # single query, single key
    (7, 4, 4, 12, 3, 64, [4, 5, 47, 48], "bf16"),  # G=4 over three kv heads
]


@pytest.mark.parametrize("seed,B,T,Hq,Hkv,d,lens,kv", CASES)
def test_oracle_matches_library_attention(seed, B, T, Hq, Hkv, d, lens, kv):
    a = W.make_attn_from_lens(seed, B, T, Hq, Hkv, d, lens, kv=kv, extra_blocks=2)
    o = _oracle(a, nthreads=2)
    r = dense_reference(a)
    assert np.all(np.isfinite(o))
    assert np.max(_rel_rows(o, r)) < 1e-12


def test_oracle_rows_subset_matches_full():
    a = W.make_attn_from_lens(11, 3, 4, 8, 2, 64, [40, 64, 9], kv="bf16")
    full = _oracle(a)
    rows = np.array([0, 5, 17, 31, a.B * a.T * a.Hq - 1], dtype=np.int64)
    sub = _oracle(a, rows=rows)
    np.testing.assert_array_equal(sub, full.reshape(-1, a.d)[rows])


def test_constant_values_give_constant_output():
    a = W.make_attn_from_lens(12, 2, 3, 4, 2, 32, [20, 50], kv="f32")
    c = np.linspace(-2, 3, 32).astype(np.float32)
    a.v_cache[:a.meta["n_real_blocks"]] = c
    o = _oracle(a)
    assert np.max(np.abs(o - c)) < 1e-12


def test_zero_query_gives_mean_of_visible_values():
    a = W.make_attn_from_lens(13, 1, 3, 2, 1, 16, [35], kv="f32")
    a.q[:] = 0
    o = _oracle(a)
    L = int(a.context_lens[0])
    vals = np.stack([a.v_cache[a.block_table[0, p // 16], p % 16, 0] for p in range(L)]).astype(np.float64)
    for t in range(a.T):
        nvis = L - a.T + 1 + t
        np.testing.assert_allclose(o[0, t, 0], vals[:nvis].mean(axis=0), rtol=0, atol=1e-13)


def test_single_visible_key_returns_that_value():
    # L_b = T: row 0 sees exactly position 0.
    a = W.make_attn_from_lens(14, 1, 4, 2, 1, 16, [4], kv="bf16")
    o = _oracle(a)
    v0 = torch.from_numpy(a.v_cache[a.block_table[0, 0], 0, 0].view(np.int16)).view(torch.bfloat16)
    np.testing.assert_array_equal(o[0, 0, 0], v0.to(torch.float64).numpy())
    np.testing.assert_array_equal(o[0, 0, 1], v0.to(torch.float64).numpy())


def test_two_visible_keys_closed_form():
    a = W.make_attn_from_lens(15, 1, 2, 1, 1, 8, [3], kv="f32")
    o = _oracle(a, sm_scale=0.5)
    k = [a.k_cache[a.block_table[0, 0], p, 0].astype(np.float64) for p in range(2)]
    v = [a.v_cache[a.block_table[0, 0], p, 0].astype(np.float64) for p in range(2)]
    q = a.q[0, 0, 0].astype(np.float64)
    s0, s1 = 0.5 * float(q @ k[0]), 0.5 * float(q @ k[1])
    want = (math.exp(s0) * v[0] + math.exp(s1) * v[1]) / (math.exp(s0) + math.exp(s1))
    np.testing.assert_allclose(o[0, 0, 0], want, rtol=1e-13, atol=1e-14)


def test_gqa_head_map_uses_floor_h_over_G():
    Hq, Hkv = 12, 3
    a = W.make_attn_from_lens(16, 2, 3, Hq, Hkv, 16, [30, 18], kv="f32")
    for g in range(Hkv):
        a.v_cache[:a.meta["n_real_blocks"], :, g, :] = float(g)
    o = _oracle(a)
    G = Hq // Hkv
    for h in range(Hq):
        assert np.max(np.abs(o[:, :, h, :] - float(h // G))) < 1e-12


def test_block_relabelling_is_invisible():
    a = W.make_attn_from_lens(17, 3, 5, 8, 2, 32, [70, 23, 5], kv="bf16", identity_table=True)
    o1 = _oracle(a)
    rng = np.random.default_rng(0)
    perm = rng.permutation(a.num_blocks)          # new physical id of old block i
    k2 = np.empty_like(a.k_cache)
    v2 = np.empty_like(a.v_cache)
    k2[perm] = a.k_cache
    v2[perm] = a.v_cache
    a.k_cache, a.v_cache = k2, v2
    a.block_table = perm[a.block_table].astype(np.int32)
    o2 = _oracle(a)
    np.testing.assert_array_equal(o1, o2)


def test_poisoned_slots_are_never_read():
    a = W.make_attn_from_lens(18, 2, 3, 4, 2, 32, [19, 33], kv="fp8", extra_blocks=3)
    # every unused table entry already points at the all-NaN spare block
    assert np.isnan(a.k_scale[a.spare_block])
    assert (a.block_table == a.spare_block).sum() > 0
    o = _oracle(a)
    assert np.all(np.isfinite(o))


def test_causal_mask_offset():
    """Row t must not see position L - T + t + 1: making that key's score huge
    changes only rows that may see it."""
    a = W.make_attn_from_lens(19, 1, 4, 1, 1, 16, [40], kv="f32")
    base = _oracle(a)
    L, T = 40, 4
    p = L - T + 2          # visible to rows t >= 2 only
    blk, slot = a.block_table[0, p // 16], p % 16
    a.k_cache[blk, slot, 0] = 100.0 * a.q[0, 3, 0] / np.linalg.norm(a.q[0, 3, 0])
    o = _oracle(a)
    np.testing.assert_array_equal(o[0, :2], base[0, :2])
    assert not np.allclose(o[0, 3], base[0, 3])


def test_bf16_decoder_exhaustive():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([oracle.decode_bf16(int(c)) for c in codes])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(got[~nan], ref[~nan])


def test_e4m3_decoder_exhaustive():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle.decode_e4m3(int(c)) for c in codes])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.nanmax(got) == 448.0 and oracle.decode_e4m3(0x01) == 2.0 ** -9
