"""Shared helpers for the GPU parity tests: upload seeded inputs, run the HIP
path through the C ABI binding, and compare with the CPU oracle."""
import numpy as np
import torch

import oracle
import speculative_decoding_verify_attn_amd as sv
import workloads as W

TOL = {W.KV_F32: 1e-3, W.KV_BF16: 2e-2, W.KV_FP8_E4M3: 2e-2}


def dev():
    return torch.device("cuda", 0)


def upload_attn(a: W.AttnInputs):
    d = dev()
    t = {}
    t["q"] = torch.from_numpy(a.q).to(d)
    if a.kv_dtype == W.KV_F32:
        t["k"] = torch.from_numpy(a.k_cache).to(d)
        t["v"] = torch.from_numpy(a.v_cache).to(d)
    elif a.kv_dtype == W.KV_BF16:
        t["k"] = torch.from_numpy(a.k_cache.view(np.int16)).to(d).view(torch.bfloat16)
        t["v"] = torch.from_numpy(a.v_cache.view(np.int16)).to(d).view(torch.bfloat16)
    else:
        t["k"] = torch.from_numpy(a.k_cache).to(d)
        t["v"] = torch.from_numpy(a.v_cache).to(d)
        t["ks"] = torch.from_numpy(a.k_scale).to(d)
        t["vs"] = torch.from_numpy(a.v_scale).to(d)
    t["table"] = torch.from_numpy(a.block_table).to(d)
    t["lens"] = torch.from_numpy(a.context_lens).to(d)
    return t


def run_attn(a: W.AttnInputs, t=None, algo=sv.SV_ATTN_AUTO, blocks_per_split=0, ws=None, out=None):
    if t is None:
        t = upload_attn(a)
    d = dev()
    if out is None:
        out = torch.full((a.B, a.T, a.Hq, a.d), float("nan"), dtype=torch.float32, device=d)
    if ws is None:
        ws = sv.alloc_workspace(sv.attn_workspace_size(a.B, a.T, a.Hq, a.Hkv, a.d, a.max_blocks,
                                                       blocks_per_split), d)
    sv.spec_verify_attn(t["q"], t["k"], t["v"], t["table"], t["lens"], out, ws,
                        k_scale=t.get("ks"), v_scale=t.get("vs"), kv_dtype=a.kv_dtype,
                        algo=algo, blocks_per_split=blocks_per_split)
    torch.cuda.synchronize()
    return out


def oracle_attn(a: W.AttnInputs, rows=None):
    return oracle.attn(a.q, a.k_cache, a.v_cache, a.block_table, a.context_lens,
                       kv_dtype=a.kv_dtype, k_scale=a.k_scale, v_scale=a.v_scale, rows=rows)


def row_rel_err(got, ref):
    got = np.asarray(got, dtype=np.float64).reshape(-1, got.shape[-1])
    ref = np.asarray(ref, dtype=np.float64).reshape(-1, ref.shape[-1])
    return np.max(np.abs(got - ref), axis=1) / np.max(np.abs(ref), axis=1)


def sample_rows(a: W.AttnInputs, n, seed=0):
    """Flat row indices covering first/last sequences, every verify row t and
    every head group, plus random rows."""
    rng = np.random.default_rng(seed)
    total = a.B * a.T * a.Hq
    fixed = []
    for b in sorted({0, a.B - 1}):
        for t in range(a.T):
            for h in sorted({0, a.Hq - 1, (a.Hq // a.Hkv) - 1}):
                fixed.append((b * a.T + t) * a.Hq + h)
    extra = rng.choice(total, size=min(total, max(0, n - len(fixed))), replace=False)
    return np.unique(np.concatenate([np.array(fixed, dtype=np.int64), extra.astype(np.int64)]))


def unit_rows(a: W.AttnInputs, seed=0):
    """Flat row indices with at least one row of every (sequence, KV head)
    unit: a random (verify row, head of the group) per unit, plus the last
    verify row of the group's first and last head.  Returns (rows, units
    covered)."""
    rng = np.random.default_rng(seed)
    G = a.Hq // a.Hkv
    rows = []
    for b in range(a.B):
        for g in range(a.Hkv):
            t = int(rng.integers(0, a.T))
            rows.append((b * a.T + t) * a.Hq + g * G + int(rng.integers(0, G)))
            rows.append((b * a.T + a.T - 1) * a.Hq + g * G)
            rows.append((b * a.T + a.T - 1) * a.Hq + g * G + G - 1)
    rows = np.unique(np.array(rows, dtype=np.int64))
    units = {(int(r) // (a.T * a.Hq), (int(r) % a.Hq) // G) for r in rows}
    return rows, units


def upload_sample(s: W.SampleInputs):
    d = dev()
    return {
        "logits": torch.from_numpy(s.target_logits).to(d),
        "probs": torch.from_numpy(s.draft_probs).to(d),
        "tokens": torch.from_numpy(s.draft_tokens).to(d),
        "u": torch.from_numpy(s.uniforms).to(d),
    }


def run_sample(s: W.SampleInputs, t=None, ws=None, temperature=None, top_p=None):
    if t is None:
        t = upload_sample(s)
    d = dev()
    n = torch.full((s.B,), -7, dtype=torch.int32, device=d)
    toks = torch.full((s.B, s.K + 1), -7, dtype=torch.int32, device=d)
    ap = torch.full((s.B, s.K), float("nan"), dtype=torch.float32, device=d)
    if ws is None:
        ws = sv.alloc_workspace(sv.sample_workspace_size(s.B, s.K, s.V), d)
    temp = None if temperature is None else torch.from_numpy(np.asarray(temperature, np.float32)).to(d)
    cut = None if top_p is None else torch.from_numpy(np.asarray(top_p, np.float32)).to(d)
    sv.spec_verify_sample(t["logits"], t["probs"], t["tokens"], t["u"], n, toks, ws, accept_prob=ap,
                          temperature=temp, top_p=cut)
    torch.cuda.synchronize()
    return n.cpu().numpy(), toks.cpu().numpy(), ap.cpu().numpy()


def compare_sampler(s: W.SampleInputs, n_gpu, toks_gpu, ref=None, temperature=None, top_p=None):
    """Bit-exact comparison except from the first position the oracle decided
    within 1e-6 of its threshold.  Returns (mismatches, flagged)."""
    if ref is None:
        ref = oracle.sample(s.target_logits, s.draft_probs, s.draft_tokens, s.uniforms,
                            temperature=None if temperature is None else np.asarray(temperature, np.float32),
                            top_p=None if top_p is None else np.asarray(top_p, np.float32))
    mism, flagged = 0, 0
    for b in range(s.B):
        k = int(ref["near_pos"][b])
        if k < 0:
            if n_gpu[b] != ref["num_accepted"][b] or not np.array_equal(toks_gpu[b], ref["out_tokens"][b]):
                mism += 1
        else:
            flagged += 1
            if not np.array_equal(toks_gpu[b, :k], ref["out_tokens"][b, :k]):
                mism += 1
    return mism, flagged, ref
