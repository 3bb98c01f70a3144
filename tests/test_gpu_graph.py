"""The verify step captured in a HIP graph: every replay must reproduce the
eager result bit for bit, also with other eager work (on other inputs, into
the same workspaces) run between the replays."""
import pytest
import torch

import speculative_decoding_verify_attn_amd as sv
import workloads as W
from .gpu_helpers import upload_attn, upload_sample

pytestmark = pytest.mark.gpu


def _setup(seed):
    a = W.make_attn_from_lens(seed, 3, 6, 32, 8, 128, [1500, 80, 999], kv="bf16")
    s = W.make_sample_from_params(seed, 3, 5, 40000, 3.0, 1.0)
    return a, s, upload_attn(a), upload_sample(s)


def test_graph_replay_matches_eager():
    dev = torch.device("cuda", 0)
    a, s, ta, ts = _setup(31)
    a2, s2, ta2, ts2 = _setup(32)
    ws_a = sv.alloc_workspace(sv.attn_workspace_size(a.B, a.T, a.Hq, a.Hkv, a.d, a.max_blocks, 16), dev)
    ws_s = sv.alloc_workspace(sv.sample_workspace_size(s.B, s.K, s.V), dev)

    def outputs():
        return (torch.empty((a.B, a.T, a.Hq, a.d), dtype=torch.float32, device=dev),
                torch.empty(s.B, dtype=torch.int32, device=dev),
                torch.empty((s.B, s.K + 1), dtype=torch.int32, device=dev))

    def step(t_a, t_s, o, stream=None):
        sv.spec_verify_attn(t_a["q"], t_a["k"], t_a["v"], t_a["table"], t_a["lens"], o[0], ws_a,
                            kv_dtype=a.kv_dtype, blocks_per_split=16, stream=stream)
        sv.spec_verify_sample(t_s["logits"], t_s["probs"], t_s["tokens"], t_s["u"], o[1], o[2], ws_s,
                              stream=stream)

    ref = outputs()
    step(ta, ts, ref)
    ref2 = outputs()
    step(ta2, ts2, ref2)
    torch.cuda.synchronize()

    got = outputs()
    for x in got:
        x.fill_(-7)
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            step(ta, ts, got, stream=side)
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()

    other = outputs()
    for rep in range(4):
        for x in got:
            x.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        for r, x in zip(ref, got):
            assert torch.equal(r, x), "replay %d differs from eager" % rep
        # eager work on other inputs through the same workspaces in between
        step(ta2, ts2, other)
        torch.cuda.synchronize()
        for r, x in zip(ref2, other):
            assert torch.equal(r, x)


def _same_bits(a, b):
    """Bitwise equality (NaN-poisoned cache slots compare equal to themselves)."""
    if a.is_floating_point():
        a = a.view({2: torch.int16, 4: torch.int32, 8: torch.int64}[a.element_size()])
        b = b.view(a.dtype)
    return torch.equal(a, b)


def _replays_match(make_call, outputs, dev, reps=4):
    """Captures make_call(out, stream) on a side stream; each replay must equal
    the eager result, with an eager call on other inputs in between."""
    ref = outputs()
    make_call(ref, None, 0)
    ref2 = outputs()
    make_call(ref2, None, 1)
    torch.cuda.synchronize()
    got = outputs()
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            make_call(got, side, 0)
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    other = outputs()
    for rep in range(reps):
        for x in got:
            x.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        for r, x in zip(ref, got):
            assert _same_bits(r, x), "replay %d differs from eager" % rep
        make_call(other, None, 1)
        torch.cuda.synchronize()
        for r, x in zip(ref2, other):
            assert _same_bits(r, x)


def test_graph_replay_sampler_variants():
    """Temperature + top-p, and typical acceptance, captured and replayed."""
    dev = torch.device("cuda", 0)
    ss = [W.make_sample_from_params(33 + i, 4, 5, 40000, 2.0, 0.7) for i in range(2)]
    ts = [upload_sample(s) for s in ss]
    s = ss[0]
    ws = sv.alloc_workspace(sv.sample_workspace_size(s.B, s.K, s.V), dev)
    temp = torch.tensor([0.7, 1.0, 1.3, 0.0], dtype=torch.float32, device=dev)
    cut = torch.tensor([0.9, 0.5, 1.0, 0.8], dtype=torch.float32, device=dev)

    def outputs():
        return (torch.empty(s.B, dtype=torch.int32, device=dev),
                torch.empty((s.B, s.K + 1), dtype=torch.int32, device=dev))

    def topp(o, stream, which):
        t = ts[which]
        sv.spec_verify_sample(t["logits"], t["probs"], t["tokens"], t["u"], o[0], o[1], ws, stream=stream,
                              temperature=temp, top_p=cut)

    def typical(o, stream, which):
        t = ts[which]
        sv.spec_verify_sample_typical(t["logits"], t["tokens"], t["u"], o[0], o[1], ws, 0.09, 0.3,
                                      temperature=temp, stream=stream)

    _replays_match(topp, outputs, dev)
    _replays_match(typical, outputs, dev)


def test_graph_replay_sampler_early_exit():
    """A batch large enough for the two-stage row statistics (64 sequences x
    8 rows x 32768 entries = 64 MiB): the per-sequence gate flags and the
    statistics of skipped rows are left in the shared workspace by the eager
    call on the other inputs between replays."""
    dev = torch.device("cuda", 0)
    ss = [W.make_sample_from_params(41 + i, 64, 7, 32768, 3.0, 0.5 + 1.5 * i) for i in range(2)]
    assert ss[0].B * (ss[0].K + 1) * ss[0].V * 4 >= 64 * 1024 * 1024
    ts = [upload_sample(s) for s in ss]
    s = ss[0]
    ws = sv.alloc_workspace(sv.sample_workspace_size(s.B, s.K, s.V), dev)

    def outputs():
        return (torch.empty(s.B, dtype=torch.int32, device=dev),
                torch.empty((s.B, s.K + 1), dtype=torch.int32, device=dev))

    def chain(o, stream, which):
        t = ts[which]
        sv.spec_verify_sample(t["logits"], t["probs"], t["tokens"], t["u"], o[0], o[1], ws, stream=stream)

    _replays_match(chain, outputs, dev)


def test_graph_replay_tree_sampler_and_commit():
    dev = torch.device("cuda", 0)
    par = W.tree_parents(W.TREE_SHAPES["wide5x2"])
    N = par.shape[0]
    trees = [W.make_tree(35 + i, 4, par, 20000, 2.0, 0.5) for i in range(2)]
    up = lambda x: torch.from_numpy(x).to(dev)
    tt = [{k: up(getattr(t, k)) for k in ("target_logits", "draft_probs", "tokens", "parents", "uniforms")}
          for t in trees]
    ws = sv.alloc_workspace(sv.sample_tree_workspace_size(4, N, 20000), dev)

    def outputs():
        return (torch.empty(4, dtype=torch.int32, device=dev), torch.empty((4, N), dtype=torch.int32, device=dev),
                torch.empty((4, N), dtype=torch.int32, device=dev))

    def tree(o, stream, which):
        t = tt[which]
        sv.spec_verify_sample_tree(t["target_logits"], t["draft_probs"], t["tokens"], t["parents"], t["uniforms"],
                                   o[0], o[1], o[2], ws, 5, stream=stream)

    _replays_match(tree, outputs, dev)

    # the commit: each call starts from a fresh copy of the cache and lengths
    a = W.make_attn_from_lens(37, 4, N, 16, 4, 64, [40, 77, 100, 300], kv="bf16")
    base = upload_attn(a)
    res = outputs()
    tree(res, None, 0)
    torch.cuda.synchronize()

    def commit(o, stream, which):
        k, v, lens = o
        k.copy_(base["k"])
        v.copy_(base["v"])
        lens.copy_(base["lens"])
        sv.spec_verify_tree_commit(res[2], res[0], k, v, base["table"], lens, kv_dtype=a.kv_dtype, stream=stream)

    def commit_outputs():
        return (torch.empty_like(base["k"]), torch.empty_like(base["v"]), torch.empty_like(base["lens"]))

    _replays_match(commit, commit_outputs, dev)


def test_graph_replay_attention_balanced_and_check():
    """Attention with balanced shares (prefix sums in the workspace, cut units
    merged), fp8 and bf16 (fp8 also with four row tiles: two waves per page),
    and the input check, captured and replayed."""
    dev = torch.device("cuda", 0)
    cases = []
    for kv, T, Hq in (("bf16", 5, 32), ("fp8", 5, 32), ("fp8", 7, 64)):
        aa = [W.make_attn_from_lens(40 + i, 5, T, Hq, 8, 128, [700, 33, 2100, 7, 1290], kv=kv) for i in range(2)]
        cases.append((aa, [upload_attn(a) for a in aa]))
    for aa, tt in cases:
        a = aa[0]
        ws = sv.alloc_workspace(sv.attn_workspace_size(a.B, a.T, a.Hq, a.Hkv, a.d, a.max_blocks, -1), dev)

        def outputs():
            return (torch.empty((a.B, a.T, a.Hq, a.d), dtype=torch.float32, device=dev),
                    torch.empty(sv.SV_CHECK_COUNTS, dtype=torch.int32, device=dev))

        def call(o, stream, which):
            t = tt[which]
            sv.spec_verify_attn(t["q"], t["k"], t["v"], t["table"], t["lens"], o[0], ws,
                                k_scale=t.get("ks"), v_scale=t.get("vs"), kv_dtype=a.kv_dtype, blocks_per_split=-1,
                                stream=stream)
            sv.spec_verify_check_inputs(a.B, block_table=t["table"], context_lens=t["lens"], T=a.T,
                                        num_blocks=a.num_blocks, counts=o[1], stream=stream)

        _replays_match(call, outputs, dev)
