"""spec_verify_attn_noalloc (static device scratch, no workspace argument)
against spec_verify_attn with a caller workspace: the same kernels and split
plan, so the outputs must agree bit for bit.  Two calls in a row on the same
GPU, the second on a smaller input, so the second call runs over scratch the
first one left behind."""
import numpy as np
import pytest
import torch

import speculative_decoding_verify_attn_amd as sv
import workloads as W
from .gpu_helpers import run_attn, upload_attn

pytestmark = pytest.mark.gpu

# (seed, B, T, Hq, Hkv, d, lens, kv): each pair is a larger call, then a
# smaller one.  The first pair splits contexts with the fixed split (merge
# kernel reads the scratch), the second takes balanced shares (prefix sums
# and partials in the scratch), the third is E4M3 with one long sequence,
# the fourth balanced shares over head groups (two KV heads per workgroup)
# twice, the second on a smaller batch.
PAIRS = [
    ((31, 4, 6, 32, 8, 128, [2000, 1500, 37, 900], "bf16"), (32, 2, 6, 32, 8, 128, [700, 100], "bf16")),
    ((33, 16, 5, 64, 8, 128, [int(x) for x in np.linspace(300, 8192, 16)], "bf16"),
     (34, 3, 4, 32, 8, 128, [1200, 16, 555], "bf16")),
    ((35, 1, 7, 64, 8, 128, [20000], "fp8"), (36, 1, 3, 16, 2, 64, [900], "fp8")),
    ((38, 24, 8, 32, 8, 128, [int(x) for x in np.linspace(8192, 40, 24)], "bf16"),
     (39, 16, 4, 16, 8, 64, [int(x) for x in np.linspace(100, 8192, 16)], "bf16")),
]


def _noalloc(a, t):
    out = torch.full((a.B, a.T, a.Hq, a.d), float("nan"), dtype=torch.float32, device=t["q"].device)
    sv.spec_verify_attn_noalloc(t["q"], t["k"], t["v"], t["table"], t["lens"], out,
                                k_scale=t.get("ks"), v_scale=t.get("vs"), kv_dtype=a.kv_dtype)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("pair", PAIRS, ids=["fixed-split", "balanced", "e4m3", "head-groups"])
def test_noalloc_matches_workspace_entry(pair):
    for case in pair:
        seed, B, T, Hq, Hkv, d, lens, kv = case
        a = W.make_attn_from_lens(seed, B, T, Hq, Hkv, d, lens, kv=kv, extra_blocks=2)
        need = sv.attn_workspace_size(a.B, a.T, a.Hq, a.Hkv, a.d, a.max_blocks)
        assert need <= sv.attn_noalloc_max_bytes()
        t = upload_attn(a)
        ref = run_attn(a, t).clone()
        got = _noalloc(a, t)
        assert torch.isfinite(got).all()
        assert torch.equal(got, ref), "case %d: max |diff| %.3e" % (
            seed, float((got - ref).abs().max()))


def test_noalloc_rejects_oversize():
    # a split plan larger than the static scratch: refused before any launch
    a = W.make_attn_from_lens(37, 1, 8, 32, 8, 128, [64], kv="bf16")
    t = upload_attn(a)
    B, T, Hq, Hkv, d = 1024, 8, 32, 8, 128
    assert sv.attn_workspace_size(B, T, Hq, Hkv, d, 8192) > sv.attn_noalloc_max_bytes()
    big_q = torch.zeros((B, T, Hq, d), dtype=torch.float32, device=t["q"].device)
    table = torch.zeros((B, 8192), dtype=torch.int32, device=t["q"].device)
    lens = torch.full((B,), 64, dtype=torch.int32, device=t["q"].device)
    with pytest.raises(sv.SpecVerifyError) as ei:
        sv.spec_verify_attn_noalloc(big_q, t["k"], t["v"], table, lens, big_q.clone(), kv_dtype=a.kv_dtype)
    assert ei.value.status == 3
