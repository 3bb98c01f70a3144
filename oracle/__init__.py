"""CPU oracle for the speculative-decoding verify step (test infrastructure).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path never does: it shares
no code with the HIP library, and the HIP path never falls back to it.

The arithmetic lives in ``oracle.c`` (IEEE double, plain loops, one function
per definition on the pages); this module only marshals numpy arrays.

Sources (page title, section):
  "KV Cache + Speculative Decoding": 2.1 (KV-cache size), 5.2-5.3 (paging),
      6.1/6.3 (cached causal GQA attention), 7.1-7.6 (rejection sampler)
  "50 | Speculative Decoding": 3.1 (decision rule), 3.2 (exactness proof)
  "Lecture 10 - Inference": 3.3 (KV-cache bytes)
  "Speculative decoding and KV cache optimisation": 3.1 (KV-cache bytes)
"""
import contextlib
import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")

KV_F32, KV_BF16, KV_FP8_E4M3 = 0, 1, 2

_lib = None


def _bind(lib):
    c = ctypes
    lib.oracle_decode_bf16.restype = c.c_double
    lib.oracle_decode_bf16.argtypes = [c.c_uint16]
    lib.oracle_decode_e4m3.restype = c.c_double
    lib.oracle_decode_e4m3.argtypes = [c.c_uint8]
    lib.oracle_softmax_row.restype = None
    lib.oracle_softmax_row.argtypes = [c.c_void_p, c.c_int64, c.c_void_p]
    lib.oracle_attn_rows.restype = c.c_int
    lib.oracle_attn_rows.argtypes = (
        [c.c_void_p] * 7 + [c.c_int] * 8 + [c.c_double, c.c_void_p, c.c_int64, c.c_void_p, c.c_int])
    lib.oracle_sample.restype = c.c_int
    lib.oracle_sample.argtypes = (
        [c.c_void_p] * 4 + [c.c_int, c.c_int, c.c_int64, c.c_double] + [c.c_void_p] * 5 + [c.c_int])
    lib.oracle_sample_t.restype = c.c_int
    lib.oracle_sample_t.argtypes = (
        [c.c_void_p] * 5 + [c.c_int, c.c_int, c.c_int64, c.c_double] + [c.c_void_p] * 5 + [c.c_int])
    lib.oracle_sample_tp.restype = c.c_int
    lib.oracle_sample_tp.argtypes = (
        [c.c_void_p] * 6 + [c.c_int, c.c_int, c.c_int64, c.c_double] + [c.c_void_p] * 5 + [c.c_int])
    lib.oracle_top_p.restype = c.c_int
    lib.oracle_top_p.argtypes = [c.c_void_p, c.c_int64, c.c_double, c.c_double, c.c_void_p]
    lib.oracle_attn_rows_tree.restype = c.c_int
    lib.oracle_attn_rows_tree.argtypes = (
        [c.c_void_p] * 8 + [c.c_int] * 8 + [c.c_double, c.c_void_p, c.c_int64, c.c_void_p, c.c_int])
    lib.oracle_sample_tree.restype = c.c_int
    lib.oracle_sample_tree.argtypes = (
        [c.c_void_p] * 5 + [c.c_int, c.c_int, c.c_int64, c.c_double] + [c.c_void_p] * 5 + [c.c_int])
    lib.oracle_tree_masks.restype = c.c_int
    lib.oracle_tree_masks.argtypes = [c.c_void_p, c.c_int, c.c_int, c.c_void_p]
    lib.oracle_entropy.restype = c.c_double
    lib.oracle_entropy.argtypes = [c.c_void_p, c.c_int64]
    lib.oracle_sample_typical.restype = c.c_int
    lib.oracle_sample_typical.argtypes = (
        [c.c_void_p] * 4 + [c.c_double, c.c_double, c.c_int, c.c_int, c.c_int64, c.c_double] + [c.c_void_p] * 5
        + [c.c_int])
    lib.oracle_target_row.restype = None
    lib.oracle_target_row.argtypes = [c.c_void_p, c.c_int64, c.c_double, c.c_void_p]
    lib.oracle_encode_bf16.restype = c.c_uint16
    lib.oracle_encode_bf16.argtypes = [c.c_float]
    lib.oracle_encode_e4m3.restype = c.c_uint8
    lib.oracle_encode_e4m3.argtypes = [c.c_float, c.c_float]
    lib.oracle_kv_append.restype = c.c_int
    lib.oracle_kv_append.argtypes = [c.c_void_p] * 8 + [c.c_int] * 7
    lib.oracle_tree_commit.restype = c.c_int
    lib.oracle_tree_commit.argtypes = [c.c_void_p] * 9 + [c.c_int] * 7
    lib.oracle_rollback.restype = None
    lib.oracle_rollback.argtypes = [c.c_void_p] * 3 + [c.c_int] * 2
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from . import build as _build
            _build.build()
        _lib = _bind(ctypes.CDLL(LIB_PATH))
    return _lib


@contextlib.contextmanager
def use_library(path):
    """Routes every oracle call through another build of oracle.c while the
    context is open (the test that plants mistakes in copies of the oracle
    uses this to show that the pins catch them)."""
    global _lib
    saved = _load()
    _lib = _bind(ctypes.CDLL(path))
    try:
        yield
    finally:
        _lib = saved


def _ptr(a):
    return None if a is None else a.ctypes.data


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:
        return max(1, os.cpu_count() or 1)


def decode_bf16(bits: int) -> float:
    """bfloat16 bit pattern -> value, from the format definition."""
    return _load().oracle_decode_bf16(int(bits) & 0xFFFF)


def decode_e4m3(bits: int) -> float:
    """OCP E4M3 (fn) bit pattern -> value, from the format definition."""
    return _load().oracle_decode_e4m3(int(bits) & 0xFF)


def softmax_row(logits: np.ndarray) -> np.ndarray:
    """fp64 softmax of one fp32 logit row (max subtracted)."""
    x = np.ascontiguousarray(logits, dtype=np.float32)
    p = np.empty(x.shape[0], dtype=np.float64)
    _load().oracle_softmax_row(_ptr(x), x.shape[0], _ptr(p))
    return p


def attn(q, k_cache, v_cache, block_table, context_lens, *, kv_dtype, k_scale=None,
         v_scale=None, sm_scale=None, rows=None, block_size=16, nthreads=None, tree_mask=None):
    """Verify attention by the plain definition, in fp64.

    q [B,T,Hq,d] fp32; k_cache/v_cache [num_blocks,16,Hkv,d] as stored
    (fp32, bf16 bits as uint16, or E4M3 codes as uint8); k_scale/v_scale
    [num_blocks] fp32 for E4M3; block_table [B,max_blocks] int32;
    context_lens [B] int32 (the T new positions included).
    rows: optional flat row indices (b*T + t)*Hq + h.
    tree_mask: optional [B,T] uint32 ancestor sets of a BFS-ordered draft
    tree (bit j of row t: node j is visible to node t); None is the chain.
    Returns [B,T,Hq,d] fp64, or [len(rows), d] when rows is given.
    """
    q = np.ascontiguousarray(q, dtype=np.float32)
    B, T, Hq, d = q.shape
    k_cache = np.ascontiguousarray(k_cache)
    v_cache = np.ascontiguousarray(v_cache)
    Hkv = k_cache.shape[2]
    block_table = np.ascontiguousarray(block_table, dtype=np.int32)
    context_lens = np.ascontiguousarray(context_lens, dtype=np.int32)
    max_blocks = block_table.shape[1]
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(d)
    if kv_dtype == KV_FP8_E4M3:
        k_scale = np.ascontiguousarray(k_scale, dtype=np.float32)
        v_scale = np.ascontiguousarray(v_scale, dtype=np.float32)
    if rows is None:
        nrows = B * T * Hq
        rows_arr = None
        out = np.empty((B, T, Hq, d), dtype=np.float64)
    else:
        rows_arr = np.ascontiguousarray(rows, dtype=np.int64)
        nrows = rows_arr.shape[0]
        out = np.empty((nrows, d), dtype=np.float64)
    tm = None if tree_mask is None else np.ascontiguousarray(tree_mask, dtype=np.uint32)
    assert tm is None or tm.shape == (B, T)
    rc = _load().oracle_attn_rows_tree(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
        _ptr(block_table), _ptr(context_lens), _ptr(tm), B, T, Hq, Hkv, d, block_size, max_blocks,
        int(kv_dtype), float(sm_scale), _ptr(rows_arr), nrows, _ptr(out),
        nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle_attn_rows rejected its arguments")
    return out


def sample(target_logits, draft_probs, draft_tokens, uniforms, *, near_eps=1e-6, nthreads=None, temperature=None,
           top_p=None):
    """The verify sampler by the pages' rule, in fp64.  temperature: [B]
    per-sequence temperatures (None: 1; <= 0: greedy), applied to the target
    rows only (the draft probabilities are the draft's actual distribution).
    top_p: [B] per-sequence top-p cuts of the (tempered) target rows (None,
    >= 1 or NaN: no cut); an ambiguous cut also sets near_pos.

    Returns a dict: num_accepted [B] int32, out_tokens [B,K+1] int32,
    accept_ratio [B,K] fp64 (NaN after the first rejection), near_pos [B]
    int32 (first position decided within near_eps of its threshold, or -1),
    resid_mass [B] fp64.
    """
    tl = np.ascontiguousarray(target_logits, dtype=np.float32)
    dp = np.ascontiguousarray(draft_probs, dtype=np.float32)
    dt = np.ascontiguousarray(draft_tokens, dtype=np.int32)
    u = np.ascontiguousarray(uniforms, dtype=np.float32)
    B, T, V = tl.shape
    K = T - 1
    assert dp.shape == (B, K, V) and dt.shape == (B, K) and u.shape == (B, K + 1)
    res = {
        "num_accepted": np.empty(B, dtype=np.int32),
        "out_tokens": np.empty((B, K + 1), dtype=np.int32),
        "accept_ratio": np.empty((B, K), dtype=np.float64),
        "near_pos": np.empty(B, dtype=np.int32),
        "resid_mass": np.empty(B, dtype=np.float64),
    }
    temp = None if temperature is None else np.ascontiguousarray(temperature, dtype=np.float32)
    assert temp is None or temp.shape == (B,)
    tpp = None if top_p is None else np.ascontiguousarray(top_p, dtype=np.float32)
    assert tpp is None or tpp.shape == (B,)
    rc = _load().oracle_sample_tp(
        _ptr(tl), _ptr(dp), _ptr(dt), _ptr(u), _ptr(temp), _ptr(tpp), B, K, V, float(near_eps),
        _ptr(res["num_accepted"]), _ptr(res["out_tokens"]), _ptr(res["accept_ratio"]),
        _ptr(res["near_pos"]), _ptr(res["resid_mass"]), nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle_sample rejected its arguments")
    return res


def entropy(p):
    """-sum p log p of a probability row, nats (fp64)."""
    row = np.ascontiguousarray(p, dtype=np.float64)
    return float(_load().oracle_entropy(row.ctypes.data, row.shape[0]))


def sample_typical(target_logits, draft_tokens, uniforms, eps, delta, *, temperature=None, near_eps=1e-6,
                   nthreads=None):
    """Typical acceptance (not exact): draft x_i kept iff
    p~_i(x_i) > min(eps, delta * exp(-H(p~_i))); the next token drawn from
    p~_n.  Returns a dict: num_accepted [B], out_tokens [B,K+1], p_draft and
    threshold [B,K] (NaN after the first rejection), near_pos [B]."""
    tl = np.ascontiguousarray(target_logits, dtype=np.float32)
    dt = np.ascontiguousarray(draft_tokens, dtype=np.int32)
    u = np.ascontiguousarray(uniforms, dtype=np.float32)
    B, T, V = tl.shape
    K = T - 1
    assert dt.shape == (B, K) and u.shape == (B, K + 1)
    temp = None if temperature is None else np.ascontiguousarray(temperature, dtype=np.float32)
    res = {
        "num_accepted": np.empty(B, dtype=np.int32),
        "out_tokens": np.empty((B, K + 1), dtype=np.int32),
        "p_draft": np.empty((B, K), dtype=np.float64),
        "threshold": np.empty((B, K), dtype=np.float64),
        "near_pos": np.empty(B, dtype=np.int32),
    }
    rc = _load().oracle_sample_typical(
        _ptr(tl), _ptr(dt), _ptr(u), _ptr(temp), float(eps), float(delta), B, K, V, float(near_eps),
        _ptr(res["num_accepted"]), _ptr(res["out_tokens"]), _ptr(res["p_draft"]), _ptr(res["threshold"]),
        _ptr(res["near_pos"]), nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle_sample_typical rejected its arguments")
    return res


def tree_masks(parents):
    """Ancestor sets [B,N] uint32 of BFS-ordered trees given by parents [B,N]
    (parents[:,0] < 0; 0 <= parents[:,c] < c): bit j of masks[b,c] is set iff
    node j is on the path from the root to node c, c included."""
    par = np.ascontiguousarray(parents, dtype=np.int32)
    B, N = par.shape
    out = np.empty((B, N), dtype=np.uint32)
    if _load().oracle_tree_masks(_ptr(par), B, N, _ptr(out)) != 0:
        raise ValueError("oracle_tree_masks rejected the parents")
    return out


def sample_tree(target_logits, draft_probs, tokens, parents, uniforms, *, near_eps=1e-6, nthreads=None):
    """Tree verification sampler (recursive rejection over siblings), fp64.

    target_logits, draft_probs [B,N,V] f32 (row c: the target after node c's
    path; the draft distribution c's children were drawn from); tokens,
    parents [B,N] int32 (BFS order, parents[:,0] = -1); uniforms [B,N] f32
    (column c >= 1 tests node c, column 0 drives the final draw).
    Returns a dict: num_accepted [B], out_tokens [B,N], path [B,N] (accepted
    node ids), accept_ratio [B,N] (NaN where untested), near_pos [B].
    """
    tl = np.ascontiguousarray(target_logits, dtype=np.float32)
    dp = np.ascontiguousarray(draft_probs, dtype=np.float32)
    tk = np.ascontiguousarray(tokens, dtype=np.int32)
    par = np.ascontiguousarray(parents, dtype=np.int32)
    u = np.ascontiguousarray(uniforms, dtype=np.float32)
    B, N, V = tl.shape
    assert dp.shape == (B, N, V) and tk.shape == (B, N) and par.shape == (B, N) and u.shape == (B, N)
    res = {
        "num_accepted": np.empty(B, dtype=np.int32),
        "out_tokens": np.empty((B, N), dtype=np.int32),
        "path": np.empty((B, N), dtype=np.int32),
        "accept_ratio": np.empty((B, N), dtype=np.float64),
        "near_pos": np.empty(B, dtype=np.int32),
    }
    rc = _load().oracle_sample_tree(
        _ptr(tl), _ptr(dp), _ptr(tk), _ptr(par), _ptr(u), B, N, V, float(near_eps),
        _ptr(res["num_accepted"]), _ptr(res["out_tokens"]), _ptr(res["path"]), _ptr(res["accept_ratio"]),
        _ptr(res["near_pos"]), nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle_sample_tree rejected its arguments")
    return res


def target_row(logits, temperature=1.0, top_p=None, near_eps=1e-6, return_ambiguous=False):
    """p~ of one target row at a temperature (<= 0: greedy one-hot), cut to
    its top-p set and renormalised if top_p is given (not for greedy rows),
    fp64.  With return_ambiguous, also whether the cut lies within near_eps."""
    row = np.ascontiguousarray(logits, dtype=np.float32)
    out = np.empty(row.shape[0], dtype=np.float64)
    lib = _load()
    lib.oracle_target_row(row.ctypes.data, row.shape[0], float(temperature), out.ctypes.data)
    amb = 0
    if top_p is not None and float(temperature) > 0:
        amb = lib.oracle_top_p(row.ctypes.data, row.shape[0], float(np.float32(top_p)), float(near_eps),
                               out.ctypes.data)
        if amb < 0:
            raise MemoryError("oracle_top_p")
    return (out, bool(amb)) if return_ambiguous else out


def tree_commit(path, num_accepted, k_cache, v_cache, block_table, context_lens, kv_dtype, k_scale=None,
                v_scale=None):
    """Keeps the root and the accepted path of each sequence's tree at
    consecutive positions (see oracle_tree_commit).  path [B,N] (accepted
    node ids, then anything), num_accepted [B]; the caches as stored.
    Returns (k_cache, v_cache, context_lens, pages_in_use), all new arrays."""
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    lens = np.array(context_lens, dtype=np.int32, copy=True)
    pages = np.empty_like(lens)
    pa = np.ascontiguousarray(path, dtype=np.int32)
    n = np.ascontiguousarray(num_accepted, dtype=np.int32)
    table = np.ascontiguousarray(block_table, dtype=np.int32)
    B, N = pa.shape
    Hkv, d = kc.shape[2], kc.shape[3]
    ks = None if k_scale is None else np.ascontiguousarray(k_scale, dtype=np.float32)
    vs = None if v_scale is None else np.ascontiguousarray(v_scale, dtype=np.float32)
    rc = _load().oracle_tree_commit(_ptr(pa), _ptr(n), _ptr(kc), _ptr(vc), _ptr(ks), _ptr(vs), _ptr(table),
                                    _ptr(lens), _ptr(pages), B, N, Hkv, d, table.shape[1], kc.shape[0], int(kv_dtype))
    if rc != 0:
        raise ValueError("oracle_tree_commit rejected its arguments")
    return kc, vc, lens, pages


def kv_cache_bytes(ctx_len, n_layers, n_kv_heads, head_dim, bytes_per_elem, batch=1):
    """KV-cache size: 2 (K and V) * L_ctx * N_layers * N_kv_heads * d_head * bytes,
    times the batch ("KV Cache + Speculative Decoding" 2.1; "Lecture 10 -
    Inference" 3.3; "Speculative decoding and KV cache optimisation" 3.1).
    The query-head count never enters."""
    return 2 * ctx_len * n_layers * n_kv_heads * head_dim * bytes_per_elem * batch


def encode_bf16(x):
    """float32 array -> bfloat16 bit patterns (uint16), element by element."""
    L = _load()
    x = np.ascontiguousarray(x, dtype=np.float32).ravel()
    return np.array([L.oracle_encode_bf16(float(v)) for v in x], dtype=np.uint16)


def encode_e4m3(x, scale):
    """float32 arrays x, scale (broadcast) -> E4M3 codes of x / scale (uint8)."""
    L = _load()
    x, scale = np.broadcast_arrays(np.asarray(x, dtype=np.float32), np.asarray(scale, dtype=np.float32))
    return np.array([L.oracle_encode_e4m3(float(a), float(s)) for a, s in zip(x.ravel(), scale.ravel())],
                    dtype=np.uint8).reshape(x.shape)


def kv_append(k_new, v_new, k_cache, v_cache, block_table, context_lens, kv_dtype, k_scale=None, v_scale=None):
    """Writes the T new positions into copies of the caches and returns them
    (k_cache, v_cache).  k_new/v_new [B,T,Hkv,d] float32; caches as stored
    (float32, uint16 bf16 bits or uint8 E4M3 codes) [num_blocks,16,Hkv,d]."""
    L = _load()
    k_new = np.ascontiguousarray(k_new, dtype=np.float32)
    v_new = np.ascontiguousarray(v_new, dtype=np.float32)
    kc = np.array(k_cache, copy=True, order="C")
    vc = np.array(v_cache, copy=True, order="C")
    table = np.ascontiguousarray(block_table, dtype=np.int32)
    lens = np.ascontiguousarray(context_lens, dtype=np.int32)
    B, T, Hkv, d = k_new.shape
    ks = None if k_scale is None else np.ascontiguousarray(k_scale, dtype=np.float32)
    vs = None if v_scale is None else np.ascontiguousarray(v_scale, dtype=np.float32)
    p = lambda a: None if a is None else a.ctypes.data
    rc = L.oracle_kv_append(p(k_new), p(v_new), p(kc), p(vc), p(ks), p(vs), p(table), p(lens),
                            B, T, Hkv, d, table.shape[1], kc.shape[0], kv_dtype)
    if rc != 0:
        raise ValueError("oracle_kv_append: position or page id out of range")
    return kc, vc


def rollback(num_accepted, context_lens, K):
    """Returns (new context_lens, pages_in_use) after keeping the accepted drafts."""
    L = _load()
    n = np.ascontiguousarray(num_accepted, dtype=np.int32)
    lens = np.array(context_lens, dtype=np.int32, copy=True)
    pages = np.zeros_like(lens)
    L.oracle_rollback(n.ctypes.data, lens.ctypes.data, pages.ctypes.data, len(lens), K)
    return lens, pages
