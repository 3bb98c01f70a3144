"""GPU parity of spec_verify_kv_append and spec_verify_rollback against the
CPU oracle: bit-exact cache bytes (every byte, so untouched positions are
checked too) and bit-exact lengths."""
import numpy as np
import pytest
import torch

import oracle
import speculative_decoding_verify_attn_amd as sv
import workloads as W
from .gpu_helpers import dev, run_attn, upload_attn

pytestmark = pytest.mark.gpu

CASES = [
    # (seed, B, T, Hkv, d, lens, kv, extremes)
    (31, 3, 6, 8, 128, [37, 400, 16], "bf16", True),
    (32, 3, 6, 8, 128, [37, 400, 16], "fp8", True),
    (33, 3, 6, 8, 128, [37, 400, 16], "f32", True),
    (34, 4, 16, 1, 64, [16, 17, 33, 300], "fp8", False),   # T = 16 crosses a page boundary
    (35, 2, 5, 2, 64, [5, 1000], "bf16", False),
    (36, 1, 1, 4, 128, [1], "fp8", True),                   # one position, one slot
]


def _upload_cache(a):
    d = dev()
    t = {}
    if a.kv_dtype == W.KV_BF16:
        t["k"] = torch.from_numpy(a.k_cache.view(np.int16).copy()).to(d).view(torch.bfloat16)
        t["v"] = torch.from_numpy(a.v_cache.view(np.int16).copy()).to(d).view(torch.bfloat16)
    else:
        t["k"] = torch.from_numpy(a.k_cache.copy()).to(d)
        t["v"] = torch.from_numpy(a.v_cache.copy()).to(d)
    if a.kv_dtype == W.KV_FP8_E4M3:
        t["ks"] = torch.from_numpy(a.k_scale).to(d)
        t["vs"] = torch.from_numpy(a.v_scale).to(d)
    t["table"] = torch.from_numpy(a.block_table).to(d)
    t["lens"] = torch.from_numpy(a.context_lens.copy()).to(d)
    return t


def _bytes(x):
    return x.contiguous().view(torch.uint8).cpu().numpy().reshape(-1)


def _same_bytes(gpu, ref):
    got, want = _bytes(gpu), ref.view(np.uint8).reshape(-1)
    assert got.shape == want.shape
    bad = int((got != want).sum())
    assert bad == 0, "%d of %d bytes differ (first at %d)" % (bad, got.size, int(np.argmax(got != want)))


@pytest.mark.parametrize("case", CASES, ids=[str(c[0]) for c in CASES])
def test_append_parity(case):
    seed, B, T, Hkv, d, lens, kv, extremes = case
    ap = W.make_append(seed, B, T, Hkv, d, lens, kv=kv, extremes=extremes, extra_blocks=2)
    a = ap.cache
    t = _upload_cache(a)
    kn = torch.from_numpy(ap.k_new).to(dev())
    vn = torch.from_numpy(ap.v_new).to(dev())
    sv.spec_verify_kv_append(kn, vn, t["k"], t["v"], t["table"], t["lens"], k_scale=t.get("ks"),
                             v_scale=t.get("vs"), kv_dtype=a.kv_dtype)
    torch.cuda.synchronize()
    kc, vc = oracle.kv_append(ap.k_new, ap.v_new, a.k_cache, a.v_cache, a.block_table, a.context_lens,
                              a.kv_dtype, a.k_scale, a.v_scale)
    _same_bytes(t["k"], kc)
    _same_bytes(t["v"], vc)


def test_append_full_size_c2_layer():
    cfg = W.CONFIGS["c2"]
    lens = [cfg["ctx"]] * cfg["B"]
    ap = W.make_append(37, cfg["B"], cfg["K"] + 1, cfg["Hkv"], cfg["d"], lens, kv=cfg["kv"])
    a = ap.cache
    t = _upload_cache(a)
    kn = torch.from_numpy(ap.k_new).to(dev())
    vn = torch.from_numpy(ap.v_new).to(dev())
    sv.spec_verify_kv_append(kn, vn, t["k"], t["v"], t["table"], t["lens"], kv_dtype=a.kv_dtype)
    torch.cuda.synchronize()
    kc, vc = oracle.kv_append(ap.k_new, ap.v_new, a.k_cache, a.v_cache, a.block_table, a.context_lens, a.kv_dtype)
    _same_bytes(t["k"], kc)
    _same_bytes(t["v"], vc)


def test_append_then_attention_matches_attention_on_full_cache():
    full = W.make_attn_from_lens(38, 3, 6, 32, 8, 128, [37, 400, 700], kv="bf16")
    ap = W.make_append(38, 3, 6, 8, 128, [37, 400, 700], kv="bf16")
    for b in range(3):
        L = int(full.context_lens[b])
        for tt in range(6):
            pos = L - 6 + tt
            pg = full.block_table[b, pos // 16]
            ap.k_new[b, tt] = (full.k_cache[pg, pos % 16].astype(np.uint32) << 16).view(np.float32)
            ap.v_new[b, tt] = (full.v_cache[pg, pos % 16].astype(np.uint32) << 16).view(np.float32)
    a = ap.cache
    t = _upload_cache(a)
    sv.spec_verify_kv_append(torch.from_numpy(ap.k_new).to(dev()), torch.from_numpy(ap.v_new).to(dev()),
                             t["k"], t["v"], t["table"], t["lens"], kv_dtype=a.kv_dtype)
    torch.cuda.synchronize()
    ref = run_attn(full)
    tf = upload_attn(full)
    tf["k"], tf["v"] = t["k"], t["v"]
    got = run_attn(full, tf)
    assert torch.equal(ref, got)


def test_rollback_parity():
    rng = np.random.default_rng(39)
    for B, K in ((1, 1), (8, 5), (300, 15), (64, 7)):
        lens = rng.integers(K + 1, 20000, size=B).astype(np.int32)
        n = rng.integers(0, K + 1, size=B).astype(np.int32)
        want_lens, want_pages = oracle.rollback(n, lens, K)
        tl = torch.from_numpy(lens).to(dev())
        tn = torch.from_numpy(n).to(dev())
        tp = torch.full((B,), -7, dtype=torch.int32, device=dev())
        sv.spec_verify_rollback(tn, tl, K, pages_in_use=tp)
        torch.cuda.synchronize()
        assert np.array_equal(tl.cpu().numpy(), want_lens)
        assert np.array_equal(tp.cpu().numpy(), want_pages)
        # without the optional output
        tl2 = torch.from_numpy(lens).to(dev())
        sv.spec_verify_rollback(tn, tl2, K)
        torch.cuda.synchronize()
        assert np.array_equal(tl2.cpu().numpy(), want_lens)
