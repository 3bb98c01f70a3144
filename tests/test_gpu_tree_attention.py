"""GPU parity of spec_verify_attn_tree (tree verification attention, "KV
Cache + Speculative Decoding" 8.2 and Q14) against the CPU oracle.

Same gate as the chain: per output row max_c |o - o_ref| / max_c |o_ref| <=
1e-3 (fp32 KV), 2e-2 (bf16, E4M3).  Covered: the tree shapes of the
workload module on both kernels and all three storage types, a different
random tree per sequence, contexts that end mid-page and contexts holding
only the tree, several context splits, and the chain's ancestor sets
reproducing spec_verify_attn bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import speculative_decoding_verify_attn_amd as sv
import workloads as W
from .gpu_helpers import TOL, dev, row_rel_err, run_attn, upload_attn

pytestmark = pytest.mark.gpu


def _run_tree(a, masks, algo=sv.SV_ATTN_AUTO, bps=0):
    t = upload_attn(a)
    d = dev()
    out = torch.full((a.B, a.T, a.Hq, a.d), float("nan"), dtype=torch.float32, device=d)
    ws = sv.alloc_workspace(sv.attn_workspace_size(a.B, a.T, a.Hq, a.Hkv, a.d, a.max_blocks, bps), d)
    tm = torch.from_numpy(np.ascontiguousarray(masks, dtype=np.uint32).view(np.int32)).to(d)
    sv.spec_verify_attn_tree(t["q"], t["k"], t["v"], t["table"], t["lens"], tm, out, ws,
                             k_scale=t.get("ks"), v_scale=t.get("vs"), kv_dtype=a.kv_dtype, algo=algo,
                             blocks_per_split=bps)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _random_parents(rng, B, N):
    par = np.empty((B, N), np.int32)
    par[:, 0] = -1
    for c in range(1, N):
        par[:, c] = rng.integers(0, c, size=B)
    return par


def _err(a, got, masks):
    ref = oracle.attn(a.q, a.k_cache, a.v_cache, a.block_table, a.context_lens, kv_dtype=a.kv_dtype,
                      k_scale=a.k_scale, v_scale=a.v_scale, tree_mask=masks)
    assert np.all(np.isfinite(got)), "non-finite output"
    return float(row_rel_err(got.reshape(-1, a.d), ref.reshape(-1, a.d)).max())


CASES = [
    # (seed, shape, B, Hq, Hkv, d, lens, kv)
    (1, "binary3", 3, 32, 8, 128, [15, 200, 1000], "bf16"),
    (2, "wide5x2", 2, 32, 8, 128, [16, 517], "bf16"),
    (3, "top3-2-1", 2, 32, 8, 128, [300, 2049], "fp8"),
    (4, "binary3", 2, 16, 4, 64, [45, 130], "f32"),
    (5, "chain5", 2, 32, 8, 128, [6, 333], "bf16"),
    (6, "wide5x2", 2, 8, 2, 64, [100, 31], "fp8"),
]


@pytest.mark.parametrize("case", CASES, ids=[str(c[0]) for c in CASES])
def test_tree_shapes(case):
    seed, shape, B, Hq, Hkv, d, lens, kv = case
    par = W.tree_parents(W.TREE_SHAPES[shape])
    N = par.shape[0]
    a = W.make_attn_from_lens(seed, B, N, Hq, Hkv, d, lens, kv=kv, extra_blocks=2)
    masks = oracle.tree_masks(np.broadcast_to(par, (B, N)))
    for algo in ((sv.SV_ATTN_AUTO,) if kv == "f32" else (sv.SV_ATTN_AUTO, sv.SV_ATTN_VALU)):
        err = _err(a, _run_tree(a, masks, algo), masks)
        print("case %d %s algo %d: max row rel err %.3e" % (seed, shape, algo, err))
        assert err <= TOL[a.kv_dtype]


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_random_tree_per_sequence_and_splits(kv):
    rng = np.random.default_rng(7)
    B, N, Hq, Hkv, d = 4, 16, 32, 8, 128
    lens = [16, 700, 1601, 4000]
    a = W.make_attn_from_lens(8, B, N, Hq, Hkv, d, lens, kv=kv, extra_blocks=1)
    masks = oracle.tree_masks(_random_parents(rng, B, N))
    for bps in (0, 8, 64):
        err = _err(a, _run_tree(a, masks, bps=bps), masks)
        print("%s bps %d: max row rel err %.3e" % (kv, bps, err))
        assert err <= TOL[a.kv_dtype]


@pytest.mark.parametrize("shape,kv", [("wide5x2", "bf16"), ("binary3", "bf16"), ("top3-2-1", "fp8")])
def test_tree_at_70b_geometry(shape, kv):
    """Sixteen-node trees at the 70B layer's GQA ratio (Hq=64, Hkv=8: up to
    128 rows per KV head), ragged contexts, the planner's split and balanced
    shares."""
    par = W.tree_parents(W.TREE_SHAPES[shape])
    N = par.shape[0]
    B = 3
    a = W.make_attn_from_lens(11, B, N, 64, 8, 128, [N, 900, 5000], kv=kv, extra_blocks=2)
    masks = oracle.tree_masks(np.broadcast_to(par, (B, N)))
    for bps in (0, -1):
        err = _err(a, _run_tree(a, masks, bps=bps), masks)
        print("%s %s bps %d: max row rel err %.3e" % (shape, kv, bps, err))
        assert err <= TOL[a.kv_dtype]


@pytest.mark.parametrize("shape,kv", [("wide5x2", "bf16"), ("binary3", "fp8")])
def test_tree_head_pairs(shape, kv):
    """Trees at a GQA ratio of 2 (at most 32 rows per KV head): balanced
    shares then run two KV heads per workgroup (head pairs), each head's
    rows with its own ancestor sets; ragged contexts so shares start and
    end inside a pair's pages."""
    par = W.tree_parents(W.TREE_SHAPES[shape])
    N = par.shape[0]
    B = 5
    a = W.make_attn_from_lens(13, B, N, 16, 8, 128, [N, 900, 5000, 40, 2000], kv=kv, extra_blocks=2)
    masks = oracle.tree_masks(np.broadcast_to(par, (B, N)))
    for bps in (0, -1):
        err = _err(a, _run_tree(a, masks, bps=bps), masks)
        print("%s %s bps %d: max row rel err %.3e" % (shape, kv, bps, err))
        assert err <= TOL[a.kv_dtype]


def test_chain_sets_equal_the_chain_call():
    B, T = 3, 6
    a = W.make_attn_from_lens(9, B, T, 32, 8, 128, [6, 250, 1200], kv="bf16")
    masks = oracle.tree_masks(np.broadcast_to(W.tree_parents((1,) * (T - 1)), (B, T)))
    chain = run_attn(a).cpu().numpy()
    tree = _run_tree(a, masks)
    assert np.array_equal(chain, tree)
