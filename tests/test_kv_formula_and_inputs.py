"""KV-cache size formula against the numbers printed on the pages, and the
seeded input generator (shapes, pool sizes, poisoning, determinism)."""
import json
import os

import numpy as np
import pytest

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "kv_cache_sizes.json")
UNITS = {"B": 1, "GB": 1e9, "GiB": 2.0 ** 30}


def _cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c["cite"][:60])
def test_kv_formula_reproduces_page_values(case):
    got = oracle.kv_cache_bytes(case["ctx"], case["layers"], case["kv_heads"], case["d"],
                                case["bytes"], case["batch"])
    assert abs(got / UNITS[case["unit"]] - case["value"]) <= case["tol"] + 1e-12


def test_kv_formula_never_counts_query_heads():
    # Only KV heads enter: the 70B-style layer with 64 query and 8 KV heads.
    assert oracle.kv_cache_bytes(8192, 1, 8, 128, 2, batch=32) == 1_073_741_824


@pytest.mark.parametrize("name", ["c1", "c2"])
def test_generated_pool_matches_formula(name):
    a = W.make_attn(name, seed=0)
    cfg = W.CONFIGS[name]
    lens = a.context_lens.astype(np.int64)
    nblk = (lens + 15) // 16
    # logical bytes follow the formula; the pool rounds each sequence up to whole pages
    logical = sum(oracle.kv_cache_bytes(int(L), 1, cfg["Hkv"], cfg["d"], W.KV_BYTES[a.kv_dtype]) for L in lens)
    per_tensor_pool = int(nblk.sum()) * 16 * cfg["Hkv"] * cfg["d"] * W.KV_BYTES[a.kv_dtype]
    assert a.k_cache[:a.meta["n_real_blocks"]].nbytes == per_tensor_pool
    assert 2 * per_tensor_pool >= logical
    assert 2 * per_tensor_pool - logical < 2 * cfg["B"] * 16 * cfg["Hkv"] * cfg["d"] * W.KV_BYTES[a.kv_dtype]


def test_generator_is_deterministic_and_seed_sensitive():
    a1 = W.make_attn_from_lens(5, 2, 3, 4, 2, 32, [40, 17], kv="fp8")
    a2 = W.make_attn_from_lens(5, 2, 3, 4, 2, 32, [40, 17], kv="fp8")
    a3 = W.make_attn_from_lens(6, 2, 3, 4, 2, 32, [40, 17], kv="fp8")
    for f in ("q", "k_cache", "v_cache", "block_table", "k_scale", "v_scale"):
        np.testing.assert_array_equal(getattr(a1, f), getattr(a2, f))
    assert not np.array_equal(a1.q, a3.q)
    s1 = W.make_sample("c1", seed=4)
    s2 = W.make_sample("c1", seed=4)
    for f in ("target_logits", "draft_probs", "draft_tokens", "uniforms"):
        np.testing.assert_array_equal(getattr(s1, f), getattr(s2, f))


def test_block_table_is_a_permutation_with_poisoned_spare():
    a = W.make_attn_from_lens(8, 3, 4, 8, 2, 32, [33, 16, 70], kv="bf16", max_blocks=8)
    nblk = (a.context_lens + 15) // 16
    used = np.concatenate([a.block_table[b, :nblk[b]] for b in range(a.B)])
    assert sorted(used.tolist()) == list(range(a.meta["n_real_blocks"]))
    for b in range(a.B):
        assert np.all(a.block_table[b, nblk[b]:] == a.spare_block)
    def isnan_bf16(x):
        return ((x & 0x7F80) == 0x7F80) & ((x & 0x7F) != 0)

    assert np.all(isnan_bf16(a.k_cache[a.spare_block]))
    # the slots past L_b in a partial last block are NaN
    last = a.block_table[0, nblk[0] - 1]
    assert np.all(isnan_bf16(a.k_cache[last, 33 % 16:]))
    assert not np.any(isnan_bf16(a.k_cache[last, :33 % 16]))


def test_e4m3_quantisation_scale_is_block_max_over_448():
    a = W.make_attn_from_lens(9, 1, 2, 2, 2, 16, [40], kv="fp8", poison=False)
    import torch
    for blk in range(a.meta["n_real_blocks"]):
        x = torch.from_numpy(a.k_cache[blk]).view(torch.float8_e4m3fn).to(torch.float64).numpy()
        assert np.max(np.abs(x)) == 448.0                 # the block maximum hits the top code
        assert np.isfinite(a.k_scale[blk]) and a.k_scale[blk] > 0


@pytest.mark.parametrize("name", list(W.CONFIGS))
def test_config_shapes(name):
    cfg = W.CONFIGS[name]
    lens, max_blocks = W.config_lens(name, seed=0)
    assert lens.shape == (cfg["B"],)
    assert np.all(lens >= cfg["K"] + 1) and np.all((lens + 15) // 16 <= max_blocks)
    if isinstance(cfg["ctx"], tuple):
        assert lens.min() >= cfg["ctx"][1] and lens.max() <= cfg["ctx"][2]


def test_uniforms_are_below_one():
    s = W.make_sample_from_params(1, 4096, 3, 8, 1.0, 1.0)
    assert s.uniforms.max() < 1.0 and s.uniforms.min() >= 0.0
