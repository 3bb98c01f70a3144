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
