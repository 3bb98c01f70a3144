"""GPU parity of spec_verify_tree_commit (the accepted path of a verified
tree moved next to its root, "KV Cache + Speculative Decoding" 8.2 and 7.6)
against the CPU oracle, bit for bit: caches (every byte), lengths and pages,
for the three storage types with page-crossing moves, a chain path, the
lengths at their extremes, and paths written by the GPU tree sampler."""
import numpy as np
import pytest
import torch

import oracle
import speculative_decoding_verify_attn_amd as sv
import workloads as W
from .gpu_helpers import dev, upload_attn
from .test_oracle_tree_commit import _random_paths

pytestmark = pytest.mark.gpu


def _bytes(t):
    return t.contiguous().view(torch.uint8).cpu().numpy()


def _commit_and_compare(a, path, n):
    t = upload_attn(a)
    d = dev()
    pt = torch.from_numpy(np.ascontiguousarray(path, np.int32)).to(d)
    nt = torch.from_numpy(np.ascontiguousarray(n, np.int32)).to(d)
    pages = torch.full((a.B,), -1, dtype=torch.int32, device=d)
    sv.spec_verify_tree_commit(pt, nt, t["k"], t["v"], t["table"], t["lens"], pages_in_use=pages,
                               k_scale=t.get("ks"), v_scale=t.get("vs"), kv_dtype=a.kv_dtype)
    torch.cuda.synchronize()
    kc, vc, lens, pg = oracle.tree_commit(path, n, a.k_cache, a.v_cache, a.block_table, a.context_lens,
                                          a.kv_dtype, a.k_scale, a.v_scale)
    assert np.array_equal(t["lens"].cpu().numpy(), lens)
    assert np.array_equal(pages.cpu().numpy(), pg)
    for got, want in ((t["k"], kc), (t["v"], vc)):
        gb = _bytes(got).reshape(-1)
        wb = np.ascontiguousarray(want).view(np.uint8).reshape(-1)
        bad = np.count_nonzero(gb != wb)
        assert bad == 0, "%d bytes differ" % bad


@pytest.mark.parametrize("kv", ["f32", "bf16", "fp8"])
def test_random_paths(kv):
    rng = np.random.default_rng(111)
    B, N = 24, 16
    lens = list(rng.integers(16, 700, size=B))
    lens[:4] = [16, 30, 31, 47]           # tree starts at 0; roots late in a page
    a = W.make_attn_from_lens(112, B, N, 8, 8, 128, lens, kv=kv, extra_blocks=3)
    path, n = _random_paths(rng, B, N)
    _commit_and_compare(a, path, n)


def test_chain_path_is_the_rollback():
    B, N = 8, 6
    a = W.make_attn_from_lens(113, B, N, 32, 8, 128, list(range(6, 6 + 8 * 37, 37)), kv="bf16")
    n = (np.arange(B) % N).astype(np.int32)
    path = np.tile(np.arange(1, N + 1, dtype=np.int32), (B, 1))
    _commit_and_compare(a, path, n)


def test_paths_from_the_gpu_tree_sampler():
    par = W.tree_parents(W.TREE_SHAPES["binary3"])
    N = par.shape[0]
    B, V = 16, 3000
    t = W.make_tree(114, B, par, V, 1.0, 0.3)
    d = dev()
    up = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(d)
    n = torch.empty(B, dtype=torch.int32, device=d)
    ot = torch.empty((B, N), dtype=torch.int32, device=d)
    path = torch.empty((B, N), dtype=torch.int32, device=d)
    ws = sv.alloc_workspace(sv.sample_tree_workspace_size(B, N, V), d)
    sv.spec_verify_sample_tree(up(t.target_logits), up(t.draft_probs), up(t.tokens), up(t.parents),
                               up(t.uniforms), n, ot, path, ws, 2)
    torch.cuda.synchronize()
    assert n.cpu().numpy().sum() > 0
    a = W.make_attn_from_lens(115, B, N, 16, 4, 64, list(range(N, N + 40 * B, 40)), kv="fp8")
    _commit_and_compare(a, path.cpu().numpy(), n.cpu().numpy())
