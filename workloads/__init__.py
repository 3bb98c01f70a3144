"""Seeded synthetic inputs for the speculative-decoding verify step.

This module only draws inputs.  It holds none of the verify step's own
arithmetic (no attention, no acceptance test, no residual, no sampling of the
output), so both the CPU oracle and the HIP path can consume what it makes.

Workloads follow the shapes the pages use as examples: LLaMA-3-8B and 70B-style
GQA layers ("KV Cache + Speculative Decoding" 2.2; "Speculative decoding and KV
cache optimisation" 3.1), 16-token KV pages read through a per-sequence block
table whose physical ids are scattered ("KV Cache + Speculative Decoding"
5.2-5.3), K draft tokens verified by K+1 target rows ("50 | Speculative
Decoding" section 2), and 8-bit (E4M3) KV storage with a wider compute type
("Speculative decoding and KV cache optimisation" 3.5).

Random streams: numpy ``SeedSequence(seed).spawn`` gives fixed, independent
streams in this order: perm, ctx, q, k, v, logits, noise, noise_scale,
draft_draw, uniforms.  Unused slots (past L_b in a sequence's last block), a
spare block and every unused block-table entry (pointing at the spare) are
NaN-poisoned, so a reader that touches them shows it.
"""
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

BLOCK = 16
KV_F32, KV_BF16, KV_FP8_E4M3 = 0, 1, 2
KV_NAMES = {"f32": KV_F32, "bf16": KV_BF16, "fp8": KV_FP8_E4M3}
KV_BYTES = {KV_F32: 4, KV_BF16: 2, KV_FP8_E4M3: 1}
E4M3_MAX = 448.0
E4M3_NAN = 0x7F
BF16_NAN = 0x7FC0

# name -> parameters.  ctx is either an int or ("uniform", lo, hi);
# noise is either a float or ("uniform", lo, hi) drawn per sequence.
CONFIGS = {
    "c1": dict(desc="tiny fp32 MQA", B=1, Hq=4, Hkv=1, d=64, ctx=256, K=4, kv="f32",
               V=1024, target_sigma=2.0, noise=0.5),
    "c2": dict(desc="LLaMA-3-8B-style layer", B=8, Hq=32, Hkv=8, d=128, ctx=4096, K=5, kv="bf16",
               V=128256, target_sigma=3.0, noise=1.0),
    "c3": dict(desc="70B-style layer", B=32, Hq=64, Hkv=8, d=128, ctx=8192, K=4, kv="bf16",
               V=32000, target_sigma=3.0, noise=0.7),
    "c4": dict(desc="ragged batch", B=64, Hq=32, Hkv=8, d=128, ctx=("uniform", 512, 16384), K=7,
               kv="bf16", V=128256, target_sigma=3.0, noise=("uniform", 0.2, 2.0)),
    "c5a": dict(desc="long context bf16", B=1, Hq=64, Hkv=8, d=128, ctx=131072, K=6, kv="bf16",
                V=128256, target_sigma=3.0, noise=1.0),
    "c5b": dict(desc="long context fp8 e4m3", B=1, Hq=64, Hkv=8, d=128, ctx=131072, K=6, kv="fp8",
                V=128256, target_sigma=3.0, noise=1.0),
}

_STREAMS = ("perm", "ctx", "q", "k", "v", "logits", "noise", "noise_scale", "draft_draw", "uniforms",
            "append", "accepted", "tree")


def streams(seed: int):
    ss = np.random.SeedSequence(seed)
    return {name: np.random.default_rng(s) for name, s in zip(_STREAMS, ss.spawn(len(_STREAMS)))}


@dataclass
class AttnInputs:
    q: np.ndarray              # [B,T,Hq,d] float32
    k_cache: np.ndarray        # [num_blocks,16,Hkv,d] float32 | uint16 (bf16 bits) | uint8 (e4m3)
    v_cache: np.ndarray
    block_table: np.ndarray    # [B,max_blocks] int32
    context_lens: np.ndarray   # [B] int32
    kv_dtype: int
    k_scale: Optional[np.ndarray] = None   # [num_blocks] float32 (e4m3 only)
    v_scale: Optional[np.ndarray] = None
    spare_block: int = -1
    meta: dict = field(default_factory=dict)

    @property
    def B(self):
        return self.q.shape[0]

    @property
    def T(self):
        return self.q.shape[1]

    @property
    def Hq(self):
        return self.q.shape[2]

    @property
    def d(self):
        return self.q.shape[3]

    @property
    def Hkv(self):
        return self.k_cache.shape[2]

    @property
    def num_blocks(self):
        return self.k_cache.shape[0]

    @property
    def max_blocks(self):
        return self.block_table.shape[1]


@dataclass
class SampleInputs:
    target_logits: np.ndarray  # [B,K+1,V] float32
    draft_probs: np.ndarray    # [B,K,V] float32
    draft_tokens: np.ndarray   # [B,K] int32
    uniforms: np.ndarray       # [B,K+1] float32 in [0,1)
    meta: dict = field(default_factory=dict)

    @property
    def B(self):
        return self.target_logits.shape[0]

    @property
    def K(self):
        return self.target_logits.shape[1] - 1

    @property
    def V(self):
        return self.target_logits.shape[2]


# ------------------------------------------------------------------ encodings

def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bfloat16 bit patterns, round to nearest even (torch's CPU cast)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def to_e4m3_codes(x: np.ndarray) -> np.ndarray:
    """fp32 (already within +-448) -> OCP E4M3 (fn) codes, round to nearest even
    (torch's CPU cast), saturated to +-448."""
    import torch
    y = np.clip(np.ascontiguousarray(x, dtype=np.float32), -E4M3_MAX, E4M3_MAX)
    t = torch.from_numpy(y)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _uniform01(rng, shape):
    """float32 uniforms in [0, 1): values that round up to 1.0 are pulled back."""
    u = rng.random(shape, dtype=np.float64).astype(np.float32)
    return np.minimum(u, np.float32(np.nextafter(np.float32(1.0), np.float32(0.0))))


# ------------------------------------------------------------------ attention

def make_attn_from_lens(seed, B, T, Hq, Hkv, d, lens, kv="bf16", max_blocks=None,
                        extra_blocks=0, poison=True, identity_table=False, q_scale=1.0):
    """Paged attention inputs for explicit per-sequence lengths.

    lens: [B] context lengths (each >= T; they count the T new positions).
    The pool holds sum(ceil(L_b/16)) + extra_blocks blocks in a random
    permutation, plus one spare block (the last) that is NaN-poisoned and is
    the target of every unused block-table entry.
    """
    kv_dtype = KV_NAMES[kv] if isinstance(kv, str) else int(kv)
    st = streams(seed)
    lens = np.asarray(lens, dtype=np.int64)
    assert lens.shape == (B,)
    nblk = (lens + BLOCK - 1) // BLOCK
    if max_blocks is None:
        max_blocks = int(max(1, nblk.max()))
    assert nblk.max() <= max_blocks
    n_real = int(nblk.sum()) + int(extra_blocks)
    num_blocks = n_real + 1
    spare = num_blocks - 1
    perm = np.arange(n_real) if identity_table else st["perm"].permutation(n_real)
    table = np.full((B, max_blocks), spare, dtype=np.int32)
    off = 0
    for b in range(B):
        table[b, :nblk[b]] = perm[off:off + nblk[b]]
        off += nblk[b]

    q = (st["q"].standard_normal((B, T, Hq, d), dtype=np.float32) * np.float32(q_scale))
    shape = (num_blocks, BLOCK, Hkv, d)

    def draw(rng):
        x = np.empty(shape, dtype=np.float32)
        x[:n_real] = rng.standard_normal((n_real, BLOCK, Hkv, d), dtype=np.float32)
        x[spare] = np.nan
        return x

    def poison_tails(x):
        for b in range(B):
            tail = int(lens[b] % BLOCK)
            if tail:
                x[table[b, nblk[b] - 1], tail:] = np.nan

    kx = draw(st["k"])
    vx = draw(st["v"])
    if poison:
        poison_tails(kx)
        poison_tails(vx)

    k_scale = v_scale = None
    if kv_dtype == KV_F32:
        kc, vc = kx, vx
    elif kv_dtype == KV_BF16:
        kc, vc = to_bf16_bits(kx), to_bf16_bits(vx)
        del kx, vx
    else:
        kc, k_scale = _quant_e4m3_blocks(kx)
        vc, v_scale = _quant_e4m3_blocks(vx)
        del kx, vx
    return AttnInputs(q=q, k_cache=kc, v_cache=vc, block_table=table,
                      context_lens=lens.astype(np.int32), kv_dtype=kv_dtype,
                      k_scale=k_scale, v_scale=v_scale, spare_block=spare,
                      meta=dict(seed=seed, n_real_blocks=n_real))


def _quant_e4m3_blocks(x):
    """Per physical block: scale = max|x| over the block's finite values / 448
    (1 for an all-zero block), code = RNE(x/scale) saturated to +-448.
    NaN-poisoned slots get the E4M3 NaN code; an all-NaN block gets scale NaN."""
    nb = x.shape[0]
    flat = x.reshape(nb, -1)
    finite = np.isfinite(flat)
    amax = np.where(finite, np.abs(flat), 0.0).max(axis=1).astype(np.float32)
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    scale[~finite.any(axis=1)] = np.nan
    codes = np.empty(flat.shape, dtype=np.uint8)
    chunk = 4096
    for s in range(0, nb, chunk):
        e = min(nb, s + chunk)
        sc = np.where(np.isfinite(scale[s:e]), scale[s:e], 1.0).astype(np.float32)
        y = flat[s:e] / sc[:, None]
        c = to_e4m3_codes(np.where(np.isfinite(y), y, 0.0))
        c[~np.isfinite(flat[s:e])] = E4M3_NAN
        codes[s:e] = c
    return codes.reshape(x.shape), scale


def config_lens(name, seed):
    cfg = CONFIGS[name]
    ctx = cfg["ctx"]
    if isinstance(ctx, tuple):
        _, lo, hi = ctx
        lens = streams(seed)["ctx"].integers(lo, hi + 1, size=cfg["B"])
        max_blocks = (hi + BLOCK - 1) // BLOCK
    else:
        lens = np.full(cfg["B"], ctx, dtype=np.int64)
        max_blocks = (ctx + BLOCK - 1) // BLOCK
    return lens, max_blocks


def make_attn(name, seed=0, poison=True):
    """Attention inputs of a named configuration (see CONFIGS)."""
    cfg = CONFIGS[name]
    lens, max_blocks = config_lens(name, seed)
    return make_attn_from_lens(seed, cfg["B"], cfg["K"] + 1, cfg["Hq"], cfg["Hkv"], cfg["d"], lens,
                               kv=cfg["kv"], max_blocks=max_blocks, poison=poison)


# -------------------------------------------------------------------- sampler

def _softmax64(x):
    m = x.max(axis=-1, keepdims=True)
    e = np.exp(x - m)
    return e / e.sum(axis=-1, keepdims=True)


def make_sample_from_params(seed, B, K, V, target_sigma, noise, chunk_rows=64):
    """Sampler inputs: target logits ~ N(0, target_sigma^2); draft logits =
    target + N(0, noise_b^2) with noise_b fixed or U[lo,hi] per sequence;
    draft probabilities = softmax of the draft logits (fp64, stored fp32);
    draft tokens drawn from those probabilities; uniforms U[0,1)."""
    st = streams(seed)
    target = st["logits"].standard_normal((B, K + 1, V), dtype=np.float32)
    target *= np.float32(target_sigma)
    if isinstance(noise, tuple):
        _, lo, hi = noise
        sig = st["noise_scale"].uniform(lo, hi, size=B)
    else:
        sig = np.full(B, float(noise))
    draft = np.empty((B, K, V), dtype=np.float32)
    tokens = np.empty((B, K), dtype=np.int32)
    rows_per = max(1, chunk_rows // max(1, K))
    for s in range(0, B, rows_per):
        e = min(B, s + rows_per)
        z = st["noise"].standard_normal((e - s, K, V), dtype=np.float32).astype(np.float64)
        dl = target[s:e, :K].astype(np.float64) + sig[s:e, None, None] * z
        qd = _softmax64(dl)
        draft[s:e] = qd.astype(np.float32)
        u = st["draft_draw"].random((e - s, K))
        cdf = np.cumsum(qd, axis=-1)
        for i in range(e - s):
            for k in range(K):
                j = int(np.searchsorted(cdf[i, k], u[i, k] * cdf[i, k, -1], side="right"))
                tokens[s + i, k] = min(j, V - 1)
    uniforms = _uniform01(st["uniforms"], (B, K + 1))
    return SampleInputs(target_logits=target, draft_probs=draft, draft_tokens=tokens,
                        uniforms=uniforms, meta=dict(seed=seed, noise=sig))


def make_sample(name, seed=0):
    cfg = CONFIGS[name]
    return make_sample_from_params(seed, cfg["B"], cfg["K"], cfg["V"], cfg["target_sigma"], cfg["noise"])


# ------------------------------------------------------------------- trees

# Tree shapes for tree verification: children per node at each depth, in
# BFS order (N = 1 + b1 + b1*b2 + ... <= 16 nodes).
TREE_SHAPES = {
    "chain5": (1, 1, 1, 1, 1),   # the chain of K = 5 drafts
    "binary3": (2, 2, 2),        # 15 nodes
    "wide5x2": (5, 2),           # 16 nodes: 5 first-token candidates, 2 continuations each
    "top3-2-1": (3, 2, 1),       # 16 nodes: a static top-k tree
}


def tree_parents(branching):
    """BFS parent array of the tree with branching[d] children per node at
    depth d; parents[0] = -1 (the root: the last committed token)."""
    parents = [-1]
    level = [0]
    for bf in branching:
        nxt = []
        for u in level:
            for _ in range(bf):
                parents.append(u)
                nxt.append(len(parents) - 1)
        level = nxt
    return np.array(parents, dtype=np.int32)


@dataclass
class TreeInputs:
    target_logits: np.ndarray  # [B,N,V] float32: row c = target after node c's path
    draft_probs: np.ndarray    # [B,N,V] float32: row c = the draft distribution of c's children
    tokens: np.ndarray         # [B,N] int32 (column 0 unused)
    parents: np.ndarray        # [B,N] int32, BFS order, parents[:,0] = -1
    uniforms: np.ndarray       # [B,N] float32 in [0,1): column c tests node c, column 0 the final draw

    @property
    def B(self):
        return self.target_logits.shape[0]

    @property
    def N(self):
        return self.target_logits.shape[1]

    @property
    def V(self):
        return self.target_logits.shape[2]


def make_tree(seed, B, parents, V, target_sigma=3.0, noise=1.0):
    """Tree verification inputs: target logits ~ N(0, sigma^2) per node; each
    node's draft row q_c = softmax(target_c + noise * N(0,1)) (fp64, stored
    fp32); every child's token drawn independently from its parent's draft
    row; uniforms U[0,1).  parents: [N] (one shape for the batch) or [B,N]."""
    st = streams(seed)
    par = np.asarray(parents, dtype=np.int32)
    if par.ndim == 1:
        par = np.broadcast_to(par, (B, par.shape[0]))
    par = np.ascontiguousarray(par)
    N = par.shape[1]
    target = st["logits"].standard_normal((B, N, V), dtype=np.float32) * np.float32(target_sigma)
    z = st["noise"].standard_normal((B, N, V), dtype=np.float32).astype(np.float64)
    qd = _softmax64(target.astype(np.float64) + float(noise) * z)
    draft = qd.astype(np.float32)
    tokens = np.zeros((B, N), dtype=np.int32)
    cdf = np.cumsum(qd, axis=-1)
    u = st["tree"].random((B, N))
    for b in range(B):
        for c in range(1, N):
            row = cdf[b, par[b, c]]
            tokens[b, c] = min(int(np.searchsorted(row, u[b, c] * row[-1], side="right")), V - 1)
    uniforms = _uniform01(st["uniforms"], (B, N))
    return TreeInputs(target_logits=target, draft_probs=draft, tokens=tokens, parents=par, uniforms=uniforms)


# --------------------------------------------------------------- byte models

def attn_algorithmic_bytes(a: AttnInputs) -> int:
    """Bytes the attention must move: every visible K/V element once, Q in,
    out written, the used block-table entries, and the per-block scales of
    the used blocks for E4M3."""
    lens = a.context_lens.astype(np.int64)
    kvb = KV_BYTES[a.kv_dtype]
    nblk = (lens + BLOCK - 1) // BLOCK
    total = int(2 * lens.sum() * a.Hkv * a.d * kvb)
    total += 2 * a.B * a.T * a.Hq * a.d * 4
    total += 4 * int(nblk.sum()) + 4 * a.B
    if a.kv_dtype == KV_FP8_E4M3:
        total += 8 * int(nblk.sum())
    return total


def attn_flops(a: AttnInputs) -> int:
    lens = a.context_lens.astype(np.int64)
    vis = sum(int(L - a.T + 1 + t) for L in lens for t in range(a.T))
    return 4 * a.d * a.Hq * vis


def sample_algorithmic_bytes(s: SampleInputs, n_rejected: int) -> int:
    """Every target row once, plus the draft row at the first rejection of each
    rejected sequence, plus tokens, uniforms and outputs."""
    B, K, V = s.B, s.K, s.V
    return 4 * V * B * (K + 1) + 4 * V * int(n_rejected) + 4 * B * K * 2 + 4 * B * (K + 1) * 2 + 4 * B


# ------------------------------------------------------------------ paged append

@dataclass
class AppendInputs:
    cache: AttnInputs          # caches, table and lengths (lengths include the T new positions)
    k_new: np.ndarray          # [B,T,Hkv,d] float32
    v_new: np.ndarray
    num_accepted: np.ndarray   # [B] int32 in [0, T-1], for the rollback that follows


def make_append(seed, B, T, Hkv, d, lens, kv="bf16", extremes=False, extra_blocks=0):
    """Inputs for appending the T verify positions of every sequence: a paged
    cache whose last T positions per sequence are NaN-poisoned (the old
    contents the append must overwrite), fresh float32 K/V for those
    positions, and accepted counts for the rollback.  E4M3 values are drawn at
    the scale of their destination page (about 1% of them beyond +-448 times
    the scale, so saturation is exercised); `extremes` plants +-inf, NaN,
    zero, denormals and huge values."""
    a = make_attn_from_lens(seed, B, T, Hkv, Hkv, d, lens, kv=kv, poison=True, extra_blocks=extra_blocks)
    st = streams(seed)
    lens = a.context_lens.astype(np.int64)
    # poison the positions about to be written
    for b in range(B):
        for t in range(T):
            pos = int(lens[b]) - T + t
            page, slot = a.block_table[b, pos // BLOCK], pos % BLOCK
            for c in (a.k_cache, a.v_cache):
                if a.kv_dtype == KV_F32:
                    c[page, slot] = np.nan
                elif a.kv_dtype == KV_BF16:
                    c[page, slot] = BF16_NAN
                else:
                    c[page, slot] = E4M3_NAN
    rng = st["append"]
    k_new = rng.standard_normal((B, T, Hkv, d), dtype=np.float32)
    v_new = rng.standard_normal((B, T, Hkv, d), dtype=np.float32)
    if a.kv_dtype == KV_FP8_E4M3:
        for b in range(B):
            for t in range(T):
                pos = int(lens[b]) - T + t
                page = a.block_table[b, pos // BLOCK]
                k_new[b, t] *= np.float32(a.k_scale[page] * 130.0)
                v_new[b, t] *= np.float32(a.v_scale[page] * 130.0)
    if extremes:
        flat_k, flat_v = k_new.reshape(-1), v_new.reshape(-1)
        specials = np.array([np.inf, -np.inf, np.nan, 0.0, -0.0, 1e-40, -3e-39, 3e38, -1e30, 65504.0],
                            dtype=np.float32)
        idx = rng.choice(flat_k.size, size=min(flat_k.size, 4 * len(specials)), replace=False)
        flat_k[idx] = np.resize(specials, len(idx))
        flat_v[idx[::-1]] = np.resize(specials, len(idx))
    n = st["accepted"].integers(0, T, size=B).astype(np.int32)
    return AppendInputs(cache=a, k_new=k_new, v_new=v_new, num_accepted=n)


def append_algorithmic_bytes(ap: AppendInputs) -> int:
    """fp32 K/V in, stored K/V out, the table entries and lengths read (+ page
    scales for E4M3)."""
    a = ap.cache
    elems = ap.k_new.size
    out_b = {KV_F32: 4, KV_BF16: 2, KV_FP8_E4M3: 1}[a.kv_dtype]
    extra = 8 * a.B * ap.k_new.shape[1] if a.kv_dtype == KV_FP8_E4M3 else 0
    return 2 * elems * (4 + out_b) + 4 * a.B * ap.k_new.shape[1] + 4 * a.B + extra
