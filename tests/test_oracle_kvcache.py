"""Pins of the oracle's paged append, rollback and value encoders ("KV Cache +
Speculative Decoding" 6.1 append, 6.2 paged data structure, 7.6 the loop and
its rollback note; "Lecture 10 - Inference" 9.2).

The encoders are checked against torch's CPU casts (a library routine) and
against the format's own values; the append against gathering the written
positions back through the block table and against every other byte being
untouched; the rollback against the loop invariant of the pages (at the start
of a round the cache holds the whole sequence except its last token), run as
a small simulation."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W


def _bf16_torch(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_bf16_encoder_matches_library_cast():
    rng = np.random.default_rng(5)
    x = np.concatenate([
        rng.standard_normal(4000).astype(np.float32) * np.float32(10.0) ** rng.integers(-40, 38, 4000).astype(np.float32),
        # exact ties: bf16 value plus half an ulp, both parities
        (np.arange(1, 300, dtype=np.uint32) << 16 | 0x8000).view(np.float32),
        (np.arange(1, 300, dtype=np.uint32) << 16 | 0x8001).view(np.float32),
        np.array([0.0, -0.0, np.inf, -np.inf, 3.4e38, -1e-45, 1e-40], dtype=np.float32),
    ]).astype(np.float32)
    got = oracle.encode_bf16(x)
    want = _bf16_torch(x)
    assert np.array_equal(got, want)
    nan = oracle.encode_bf16(np.array([np.nan, -np.nan], dtype=np.float32))
    assert np.all((nan & 0x7F80) == 0x7F80) and np.all(nan & 0x007F)


def test_e4m3_encoder_matches_library_cast_within_range():
    rng = np.random.default_rng(6)
    x = np.concatenate([
        rng.uniform(-464, 464, 3000).astype(np.float32),
        (rng.standard_normal(3000) * 2.0 ** rng.integers(-12, 6, 3000)).astype(np.float32),
        # every midpoint between neighbouring positive codes (ties to even)
        np.array([(oracle_val(c) + oracle_val(c + 1)) / 2 for c in range(0, 0x7E)], dtype=np.float32),
        np.array([464.0, -464.0, 448.0, 0.0, -0.0, 2.0 ** -10, 1.5 * 2.0 ** -9], dtype=np.float32),
    ])
    got = oracle.encode_e4m3(x, np.float32(1.0))
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # +-0 agree up to the sign of zero only where torch keeps it; compare values
    same = (got == want) | ((got & 0x7F) == 0) & ((want & 0x7F) == 0)
    assert same.all(), x[~same][:10]


def oracle_val(c):
    return oracle._load().oracle_decode_e4m3(c)


def test_e4m3_encoder_round_trips_every_finite_code_and_saturates():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = np.array([oracle_val(int(c)) for c in codes], dtype=np.float32)
    back = oracle.encode_e4m3(vals, np.float32(1.0))
    # +0 and -0 both encode to a zero code
    assert np.array_equal(back[vals != 0], codes[vals != 0])
    sat = oracle.encode_e4m3(np.array([449.0, 465.0, 1e6, np.inf, -500.0, -np.inf], dtype=np.float32), np.float32(1.0))
    assert list(sat) == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE]
    assert oracle.encode_e4m3(np.array([np.nan], dtype=np.float32), np.float32(1.0))[0] & 0x7F == 0x7F


def test_e4m3_encoder_divides_by_the_scale_in_float():
    # x / scale rounded to float first, then to E4M3
    x = np.array([3.0, 1.0, 1.0, -7.5, 0.37], dtype=np.float32)
    s = np.array([0.5, 3.0, 0.01, 2.5, 0.0123], dtype=np.float32)
    q = (x / s).astype(np.float32)
    want = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.encode_e4m3(x, s), want)


def _gather(a, cache, b, pos):
    return cache[a.block_table[b, pos // 16], pos % 16]


@pytest.mark.parametrize("kv", ["f32", "bf16", "fp8"])
def test_append_writes_exactly_the_new_positions(kv):
    ap = W.make_append(11, 4, 6, 2, 64, [6, 21, 40, 300], kv=kv, extra_blocks=2)
    a = ap.cache
    kc, vc = oracle.kv_append(ap.k_new, ap.v_new, a.k_cache, a.v_cache, a.block_table, a.context_lens,
                              a.kv_dtype, a.k_scale, a.v_scale)
    written = np.zeros(a.k_cache.shape[:2], dtype=bool)
    for b in range(a.B):
        L = int(a.context_lens[b])
        for t in range(6):
            pos = L - 6 + t
            page = a.block_table[b, pos // 16]
            written[page, pos % 16] = True
            for new, cache, scale in ((ap.k_new, kc, a.k_scale), (ap.v_new, vc, a.v_scale)):
                got = cache[page, pos % 16]
                x = new[b, t]
                if a.kv_dtype == W.KV_F32:
                    assert np.array_equal(got.view(np.uint32), x.view(np.uint32))
                elif a.kv_dtype == W.KV_BF16:
                    assert np.array_equal(got, _bf16_torch(x))
                else:
                    q = (x / scale[page]).astype(np.float32)
                    want = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
                    big = np.abs(q) > 464
                    want[big] = np.where(q[big] > 0, 0x7E, 0xFE)
                    assert np.array_equal(got, want)
    # nothing else moved (compare bit patterns: NaN poison included)
    for old, new in ((a.k_cache, kc), (a.v_cache, vc)):
        ob = old.view(np.uint8).reshape(old.shape[0], 16, -1)
        nb = new.view(np.uint8).reshape(new.shape[0], 16, -1)
        assert np.array_equal(ob[~written], nb[~written])


def test_append_then_attention_equals_attention_on_the_full_cache():
    # a cache generated with the verify positions already inside, versus the
    # same cache with those positions poisoned and then appended
    full = W.make_attn_from_lens(12, 2, 5, 8, 2, 64, [37, 100], kv="bf16")
    ap = W.make_append(12, 2, 5, 2, 64, [37, 100], kv="bf16")
    # take the verify positions' values from the full cache
    for b in range(2):
        L = int(full.context_lens[b])
        for t in range(5):
            pos = L - 5 + t
            ap.k_new[b, t] = (_gather(full, full.k_cache, b, pos).astype(np.uint32) << 16).view(np.float32)
            ap.v_new[b, t] = (_gather(full, full.v_cache, b, pos).astype(np.uint32) << 16).view(np.float32)
    a = ap.cache
    assert np.array_equal(a.block_table, full.block_table)
    kc, vc = oracle.kv_append(ap.k_new, ap.v_new, a.k_cache, a.v_cache, a.block_table, a.context_lens, a.kv_dtype)
    o1 = oracle.attn(full.q, full.k_cache, full.v_cache, full.block_table, full.context_lens, kv_dtype=full.kv_dtype)
    o2 = oracle.attn(full.q, kc, vc, a.block_table, a.context_lens, kv_dtype=a.kv_dtype)
    assert np.array_equal(o1, o2)


def test_append_rejects_out_of_range_positions():
    ap = W.make_append(13, 2, 4, 1, 64, [10, 20], kv="f32")
    a = ap.cache
    bad = a.context_lens.copy()
    bad[0] = 3  # shorter than T
    with pytest.raises(ValueError):
        oracle.kv_append(ap.k_new, ap.v_new, a.k_cache, a.v_cache, a.block_table, bad, a.kv_dtype)


def test_rollback_keeps_the_loop_invariant():
    """Simulates rounds of the pages' loop: at a round's start the cache holds
    len(seq) - 1 tokens; the verify step appends last token + K drafts; after n
    acceptances the sequence grows by n + 1 and the cache must again hold
    len(seq) - 1 tokens."""
    rng = np.random.default_rng(14)
    B, K = 6, 5
    seq_len = rng.integers(1, 50, size=B)
    cache_len = seq_len - 1
    for _ in range(20):
        lens = (cache_len + K + 1).astype(np.int32)      # after appending the verify positions
        n = rng.integers(0, K + 1, size=B).astype(np.int32)
        new_lens, pages = oracle.rollback(n, lens, K)
        seq_len = seq_len + n + 1
        cache_len = new_lens.astype(np.int64)
        assert np.array_equal(cache_len, seq_len - 1)
        assert np.array_equal(pages, (cache_len + 15) // 16)


def test_rollback_extremes():
    lens = np.array([6, 6, 17, 32, 33], dtype=np.int32)
    n = np.array([0, 5, 0, 5, 1], dtype=np.int32)
    new, pages = oracle.rollback(n, lens, 5)
    assert list(new) == [1, 6, 12, 32, 29]
    assert list(pages) == [1, 1, 1, 2, 2]
