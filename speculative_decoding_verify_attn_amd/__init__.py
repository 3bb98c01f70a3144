"""Python binding of libspecverify (the speculative-decoding verify step on MI355X).

Argument marshalling only: every step of the verify path runs in the HIP
kernels of ``libspecverify.so``; torch supplies device memory and the stream.
There is no fallback: if the library is missing or a call fails, this module
raises.

Calls (same names as the C ABI in include/spec_verify.h):
    spec_verify_kv_append(...)  write the K+1 verify positions' K/V into the paged cache
    spec_verify_attn(...)       paged GQA attention for the K+1 verify rows
    spec_verify_sample(...)     the accept / residual / bonus rejection sampler
    spec_verify_rollback(...)   drop the rejected drafts' positions (context_lens in place)
"""
import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libspecverify.so")

SV_OK = 0
SV_KV_F32, SV_KV_BF16, SV_KV_FP8_E4M3 = 0, 1, 2
SV_ATTN_AUTO, SV_ATTN_VALU, SV_ATTN_MFMA = 0, 1, 2
BLOCK_SIZE = 16

_lib = None


class SpecVerifyError(RuntimeError):
    def __init__(self, fn, status, detail):
        super().__init__("%s failed with status %d: %s" % (fn, status, detail))
        self.status = status


def lib():
    """The loaded library (ctypes.CDLL); raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libspecverify.so is not built (run __graft_entry__.build() or "
                              "python speculative_decoding_verify_attn_amd/build.py)")
        L = ctypes.CDLL(LIB_PATH)
        c = ctypes
        P, I, S, F = c.c_void_p, c.c_int, c.c_size_t, c.c_float
        L.sv_abi_version.restype = I
        L.sv_abi_version.argtypes = []
        L.sv_status_string.restype = c.c_char_p
        L.sv_status_string.argtypes = [I]
        L.sv_last_error.restype = c.c_char_p
        L.sv_last_error.argtypes = []
        L.spec_verify_workspace_clear.restype = I
        L.spec_verify_workspace_clear.argtypes = [P, S, P]
        L.spec_verify_attn_workspace_size.restype = S
        L.spec_verify_attn_workspace_size.argtypes = [I] * 6
        L.spec_verify_attn_workspace_size_ex.restype = S
        L.spec_verify_attn_workspace_size_ex.argtypes = [I] * 7
        attn_args = [P] * 8 + [I] * 9 + [F, P, S, P]
        L.spec_verify_attn.restype = I
        L.spec_verify_attn.argtypes = attn_args
        L.spec_verify_attn_ex.restype = I
        L.spec_verify_attn_ex.argtypes = attn_args + [I, I, P]
        L.spec_verify_attn_timing_main_only.restype = I
        L.spec_verify_attn_timing_main_only.argtypes = attn_args + [I, I]
        L.spec_verify_attn_noalloc_max_bytes.restype = S
        L.spec_verify_attn_noalloc_max_bytes.argtypes = []
        L.spec_verify_attn_noalloc.restype = I
        L.spec_verify_attn_noalloc.argtypes = [P] * 8 + [I] * 9 + [F, P]
        L.spec_verify_probe_read_sink_floats.restype = S
        L.spec_verify_probe_read_sink_floats.argtypes = []
        L.spec_verify_probe_read.restype = I
        L.spec_verify_probe_read.argtypes = [P, S, P, S, P]
        L.spec_verify_attn_tree.restype = I
        L.spec_verify_attn_tree.argtypes = [P] * 9 + [I] * 9 + [F, P, S, P, I, I]
        L.spec_verify_sample_workspace_size.restype = S
        L.spec_verify_sample_workspace_size.argtypes = [I] * 3
        L.spec_verify_sample.restype = I
        L.spec_verify_sample.argtypes = [P] * 7 + [I] * 3 + [P, S, P]
        L.spec_verify_sample_ex.restype = I
        L.spec_verify_sample_ex.argtypes = [P] * 9 + [I] * 3 + [P, S, P]
        L.spec_verify_sample_typical.restype = I
        L.spec_verify_sample_typical.argtypes = [P] * 4 + [c.c_double, c.c_double] + [P] * 4 + [I] * 3 + [P, S, P]
        L.spec_verify_sample_tree_workspace_size.restype = S
        L.spec_verify_sample_tree_workspace_size.argtypes = [I] * 3
        L.spec_verify_sample_tree.restype = I
        L.spec_verify_sample_tree.argtypes = [P] * 9 + [I] * 4 + [P, S, P]
        L.spec_verify_kv_append.restype = I
        L.spec_verify_kv_append.argtypes = [P] * 8 + [I] * 8 + [P]
        L.spec_verify_tree_commit.restype = I
        L.spec_verify_tree_commit.argtypes = [P] * 9 + [I] * 8 + [P]
        L.spec_verify_rollback.restype = I
        L.spec_verify_rollback.argtypes = [P] * 3 + [I] * 2 + [P]
        L.spec_verify_check_inputs.restype = I
        L.spec_verify_check_inputs.argtypes = [P, P] + [I] * 3 + [P, I, I, P, I, I, P, P]
        if L.sv_abi_version() != 1:
            raise ImportError("libspecverify ABI version mismatch")
        _lib = L
    return _lib


def _check(fn, status):
    if status != SV_OK:
        L = lib()
        raise SpecVerifyError(fn, status, "%s (%s)" % (L.sv_status_string(status).decode(),
                                                       L.sv_last_error().decode()))


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream_handle(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream


def kv_dtype_of(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return SV_KV_F32
    if t.dtype == torch.bfloat16:
        return SV_KV_BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return SV_KV_FP8_E4M3
    raise TypeError("unsupported KV cache dtype %s" % t.dtype)


def attn_workspace_size(B, T, Hq, Hkv, d, max_blocks_per_seq, blocks_per_split=0) -> int:
    n = lib().spec_verify_attn_workspace_size_ex(B, T, Hq, Hkv, d, max_blocks_per_seq, blocks_per_split)
    if n == 0:
        raise ValueError("unsupported attention shape")
    return n


def attn_shape_supported(B, T, Hq, Hkv, d, max_blocks_per_seq, blocks_per_split=0) -> bool:
    """Whether spec_verify_attn accepts this shape (its workspace query is non-zero)."""
    return lib().spec_verify_attn_workspace_size_ex(B, T, Hq, Hkv, d, max_blocks_per_seq, blocks_per_split) != 0


def sample_workspace_size(B, K, V) -> int:
    n = lib().spec_verify_sample_workspace_size(B, K, V)
    if n == 0:
        raise ValueError("unsupported sampler shape")
    return n


def alloc_workspace(nbytes: int, device) -> torch.Tensor:
    """A zero-filled device workspace (the caching allocator aligns to >= 256 B)."""
    return torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def workspace_clear(ws: torch.Tensor, stream=None):
    _check("spec_verify_workspace_clear",
           lib().spec_verify_workspace_clear(_ptr(ws), ws.numel() * ws.element_size(),
                                             _stream_handle(stream, ws.device)))


def spec_verify_attn(q, k_cache, v_cache, block_table, context_lens, out, workspace, *,
                     k_scale=None, v_scale=None, sm_scale=None, kv_dtype=None, stream=None,
                     algo=SV_ATTN_AUTO, blocks_per_split=0, main_done_event=None):
    """Paged GQA verify attention (see include/spec_verify.h).

    q [B,T,Hq,d] f32; k_cache/v_cache [num_blocks,16,Hkv,d] (f32, bf16, or E4M3
    codes as uint8 / float8_e4m3fn); block_table [B,max_blocks] i32;
    context_lens [B] i32; out [B,T,Hq,d] f32; workspace: uint8 device tensor of
    at least attn_workspace_size(...) bytes.  main_done_event: optional raw
    hipEvent_t handle recorded between the main kernel and the split merge.
    """
    B, T, Hq, d = q.shape
    num_blocks, bs, Hkv, d2 = k_cache.shape
    if kv_dtype is None:
        kv_dtype = kv_dtype_of(k_cache)
    if sm_scale is None:
        sm_scale = 1.0 / (d ** 0.5)
    _check("spec_verify_attn", lib().spec_verify_attn_ex(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale), _ptr(block_table),
        _ptr(context_lens), _ptr(out), B, T, Hq, Hkv, d, bs, block_table.shape[1], num_blocks,
        kv_dtype, float(sm_scale), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream_handle(stream, q.device), int(algo), int(blocks_per_split), main_done_event))
    return out


def spec_verify_attn_timing_main_only(q, k_cache, v_cache, block_table, context_lens, out, workspace, *,
                                      k_scale=None, v_scale=None, sm_scale=None, kv_dtype=None, stream=None,
                                      algo=SV_ATTN_AUTO, blocks_per_split=0):
    """MEASUREMENT ONLY: enqueues the main attention kernel alone (no split
    merge), so back-to-back calls time that kernel; `out` is not a result
    (it is not written when the context is split)."""
    B, T, Hq, d = q.shape
    num_blocks, bs, Hkv, d2 = k_cache.shape
    if kv_dtype is None:
        kv_dtype = kv_dtype_of(k_cache)
    if sm_scale is None:
        sm_scale = 1.0 / (d ** 0.5)
    _check("spec_verify_attn_timing_main_only", lib().spec_verify_attn_timing_main_only(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale), _ptr(block_table),
        _ptr(context_lens), _ptr(out), B, T, Hq, Hkv, d, bs, block_table.shape[1], num_blocks,
        kv_dtype, float(sm_scale), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream_handle(stream, q.device), int(algo), int(blocks_per_split)))


def probe_read_sink(device) -> torch.Tensor:
    """A sink tensor for spec_verify_probe_read."""
    return torch.empty(int(lib().spec_verify_probe_read_sink_floats()), dtype=torch.float32, device=device)


def spec_verify_probe_read(src: torch.Tensor, nbytes: int, sink: torch.Tensor, stream=None):
    """MEASUREMENT ONLY: one streaming read of the first nbytes of src (the
    practical HBM read ceiling)."""
    if nbytes > src.numel() * src.element_size():
        raise ValueError("nbytes exceeds the source tensor")
    _check("spec_verify_probe_read", lib().spec_verify_probe_read(
        _ptr(src), int(nbytes), _ptr(sink), sink.numel(), _stream_handle(stream, src.device)))


def attn_noalloc_max_bytes() -> int:
    """Size of the static scratch behind spec_verify_attn_noalloc."""
    return int(lib().spec_verify_attn_noalloc_max_bytes())


def spec_verify_attn_noalloc(q, k_cache, v_cache, block_table, context_lens, out, *,
                             k_scale=None, v_scale=None, sm_scale=None, kv_dtype=None, stream=None):
    """spec_verify_attn without a workspace: the library's static device
    scratch stands in for it (see include/spec_verify.h; calls that overlap
    in time on one GPU race)."""
    B, T, Hq, d = q.shape
    num_blocks, bs, Hkv, d2 = k_cache.shape
    if kv_dtype is None:
        kv_dtype = kv_dtype_of(k_cache)
    if sm_scale is None:
        sm_scale = 1.0 / (d ** 0.5)
    _check("spec_verify_attn_noalloc", lib().spec_verify_attn_noalloc(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale), _ptr(block_table),
        _ptr(context_lens), _ptr(out), B, T, Hq, Hkv, d, bs, block_table.shape[1], num_blocks,
        kv_dtype, float(sm_scale), _stream_handle(stream, q.device)))
    return out


def spec_verify_attn_tree(q, k_cache, v_cache, block_table, context_lens, tree_mask, out, workspace, *,
                          k_scale=None, v_scale=None, sm_scale=None, kv_dtype=None, stream=None,
                          algo=SV_ATTN_AUTO, blocks_per_split=0):
    """Tree verification attention (see include/spec_verify.h): as
    spec_verify_attn with T = the tree's BFS-ordered nodes and tree_mask
    [B,T] int32/uint32 ancestor sets (bit j of row t: node j visible to t)."""
    B, T, Hq, d = q.shape
    num_blocks, bs, Hkv, d2 = k_cache.shape
    if kv_dtype is None:
        kv_dtype = kv_dtype_of(k_cache)
    if sm_scale is None:
        sm_scale = 1.0 / (d ** 0.5)
    _check("spec_verify_attn_tree", lib().spec_verify_attn_tree(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale), _ptr(block_table),
        _ptr(context_lens), _ptr(tree_mask), _ptr(out), B, T, Hq, Hkv, d, bs, block_table.shape[1], num_blocks,
        kv_dtype, float(sm_scale), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream_handle(stream, q.device), int(algo), int(blocks_per_split)))
    return out


def spec_verify_sample(target_logits, draft_probs, draft_tokens, uniforms, num_accepted, out_tokens,
                       workspace, *, accept_prob=None, stream=None, temperature=None, top_p=None):
    """Verify sampler (see include/spec_verify.h).

    target_logits [B,K+1,V] f32, draft_probs [B,K,V] f32, draft_tokens [B,K] i32,
    uniforms [B,K+1] f32 in [0,1); outputs num_accepted [B] i32, out_tokens
    [B,K+1] i32, optional accept_prob [B,K] f32.  temperature: optional [B]
    f32 target temperatures (<= 0 is greedy); top_p: optional [B] f32 top-p
    cuts of the target rows (>= 1 or NaN: none).  Either routes the call to
    spec_verify_sample_ex.
    """
    B, K1, V = target_logits.shape
    _check("spec_verify_sample", lib().spec_verify_sample_ex(
        _ptr(target_logits), _ptr(draft_probs), _ptr(draft_tokens), _ptr(uniforms), _ptr(temperature),
        _ptr(top_p), _ptr(num_accepted), _ptr(out_tokens), _ptr(accept_prob), B, K1 - 1, V,
        _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream_handle(stream, target_logits.device)))
    return num_accepted, out_tokens


def spec_verify_sample_typical(target_logits, draft_tokens, uniforms, num_accepted, out_tokens, workspace,
                               eps, delta, *, temperature=None, p_draft=None, threshold=None, stream=None):
    """Typical acceptance (see include/spec_verify.h; not exact).

    target_logits [B,K+1,V] f32, draft_tokens [B,K] i32, uniforms [B,K+1] f32;
    eps, delta: the threshold min(eps, delta * exp(-H)); optional
    temperature [B] f32; optional outputs p_draft and threshold [B,K] f32.
    Workspace: sample_workspace_size(B, K, V).
    """
    B, K1, V = target_logits.shape
    _check("spec_verify_sample_typical", lib().spec_verify_sample_typical(
        _ptr(target_logits), _ptr(draft_tokens), _ptr(uniforms), _ptr(temperature), float(eps), float(delta),
        _ptr(num_accepted), _ptr(out_tokens), _ptr(p_draft), _ptr(threshold), B, K1 - 1, V,
        _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream_handle(stream, target_logits.device)))
    return num_accepted, out_tokens


def sample_tree_workspace_size(B, N, V):
    n = lib().spec_verify_sample_tree_workspace_size(B, N, V)
    if n == 0:
        raise ValueError("unsupported tree sampler shape B=%d N=%d V=%d" % (B, N, V))
    return n


def spec_verify_sample_tree(target_logits, draft_probs, tokens, parents, uniforms, num_accepted, out_tokens,
                            path, workspace, max_children, *, accept_prob=None, stream=None):
    """Tree verification sampler (see include/spec_verify.h).

    target_logits, draft_probs [B,N,V] f32; tokens, parents [B,N] i32 (BFS
    order, parents[:,0] = -1); uniforms [B,N] f32; max_children: the largest
    number of children of any node; outputs num_accepted [B], out_tokens
    [B,N], path [B,N] i32, optional accept_prob [B,N] f32.
    """
    B, N, V = target_logits.shape
    _check("spec_verify_sample_tree", lib().spec_verify_sample_tree(
        _ptr(target_logits), _ptr(draft_probs), _ptr(tokens), _ptr(parents), _ptr(uniforms),
        _ptr(num_accepted), _ptr(out_tokens), _ptr(path), _ptr(accept_prob), B, N, V, int(max_children),
        _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream_handle(stream, target_logits.device)))
    return num_accepted, out_tokens, path


def spec_verify_kv_append(k_new, v_new, k_cache, v_cache, block_table, context_lens, *,
                          k_scale=None, v_scale=None, kv_dtype=None, stream=None):
    """Writes k_new/v_new [B,T,Hkv,d] float32 into the paged caches at
    positions context_lens[b] - T + t (see include/spec_verify.h)."""
    B, T, Hkv, d = k_new.shape
    num_blocks, bs = k_cache.shape[0], k_cache.shape[1]
    if kv_dtype is None:
        kv_dtype = kv_dtype_of(k_cache)
    _check("spec_verify_kv_append", lib().spec_verify_kv_append(
        _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
        _ptr(block_table), _ptr(context_lens), B, T, Hkv, d, bs, block_table.shape[1], num_blocks, kv_dtype,
        _stream_handle(stream, k_new.device)))
    return k_cache, v_cache


def spec_verify_rollback(num_accepted, context_lens, K, pages_in_use=None, stream=None):
    """context_lens[b] <- context_lens[b] - K + num_accepted[b], in place;
    pages_in_use[b] = ceil(context_lens[b] / 16) if given."""
    _check("spec_verify_rollback", lib().spec_verify_rollback(
        _ptr(num_accepted), _ptr(context_lens), _ptr(pages_in_use), context_lens.shape[0], int(K),
        _stream_handle(stream, context_lens.device)))
    return context_lens, pages_in_use


SV_CHECK_COUNTS = 4


def spec_verify_check_inputs(B, *, block_table=None, context_lens=None, T=1, max_blocks_per_seq=None, num_blocks=0,
                             tokens=None, V=0, uniforms=None, counts=None, stream=None):
    """Counts violations of the documented device-data preconditions (see
    include/spec_verify.h): [0] context lengths outside [T, 16*max_blocks],
    [1] out-of-range table entries of visible pages, [2] tokens outside
    [0, V), [3] uniforms outside [0, 1).  Returns the int32[4] device tensor
    (allocated here unless `counts` is given); read it after synchronising."""
    ref = next(x for x in (block_table, context_lens, tokens, uniforms, counts) if x is not None)
    if counts is None:
        counts = torch.empty(SV_CHECK_COUNTS, dtype=torch.int32, device=ref.device)
    max_blocks = max_blocks_per_seq
    if max_blocks is None:
        if block_table is None and context_lens is not None:
            raise ValueError("checking context_lens without block_table needs max_blocks_per_seq")
        max_blocks = block_table.shape[1] if block_table is not None else 1
    n_tokens = tokens.shape[1] if tokens is not None else 0
    n_uniforms = uniforms.shape[1] if uniforms is not None else 0
    _check("spec_verify_check_inputs", lib().spec_verify_check_inputs(
        _ptr(block_table), _ptr(context_lens), int(T), int(max_blocks), int(num_blocks), _ptr(tokens), int(n_tokens),
        int(V), _ptr(uniforms), int(n_uniforms), int(B), _ptr(counts), _stream_handle(stream, ref.device)))
    return counts


def spec_verify_tree_commit(path, num_accepted, k_cache, v_cache, block_table, context_lens, *, pages_in_use=None,
                            k_scale=None, v_scale=None, kv_dtype=None, stream=None):
    """Keeps the root and the accepted path of each tree at consecutive
    positions and updates context_lens (see include/spec_verify.h)."""
    B, N = path.shape
    num_blocks, bs, Hkv, d = k_cache.shape
    if kv_dtype is None:
        kv_dtype = kv_dtype_of(k_cache)
    _check("spec_verify_tree_commit", lib().spec_verify_tree_commit(
        _ptr(path), _ptr(num_accepted), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
        _ptr(block_table), _ptr(context_lens), _ptr(pages_in_use), B, N, Hkv, d, bs, block_table.shape[1],
        num_blocks, int(kv_dtype), _stream_handle(stream, k_cache.device)))
    return context_lens

