/*
 * spec_verify.h -- C ABI of libspecverify: the verify step of speculative
 * decoding on AMD Instinct MI355X (gfx950).
 *
 * One verify step is one spec_verify_attn call per layer (the target model
 * scoring K+1 positions against its paged KV cache) followed by one
 * spec_verify_sample call on the target logits (the rejection sampler that
 * decides how many of the K draft tokens survive and draws one more token).
 * Around it, spec_verify_kv_append writes the K+1 positions' K/V into the
 * cache (per layer, before the attention) and spec_verify_rollback drops the
 * rejected drafts' positions afterwards.
 *
 * Conventions shared by every call:
 *   - Tensor pointers are DEVICE pointers, row-major, dense, owned by the
 *     caller.  The library never allocates, frees or retains them.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *     default stream).  Outputs are valid once the stream has been
 *     synchronised.  No call synchronises or reads device data on the host.
 *   - Every call returns an sv_status.  Host-checkable preconditions are
 *     validated before anything is enqueued; sv_last_error() then holds a
 *     thread-local description.  Nothing aborts and no exception crosses
 *     the ABI.
 *   - Device-data preconditions (block ids, context lengths, token ids,
 *     uniforms) are documented, not checked: results for violating data are
 *     unspecified, but every index is clamped, so kernels stay in bounds.
 *   - Workspaces: size them with the *_workspace_size queries.  Their
 *     contents on entry do not matter (every byte read is written earlier in
 *     the same call); calls that share a workspace must not overlap in time.
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SV_ABI_VERSION 1

typedef enum {
    SV_OK = 0,
    SV_ERR_NULL = 1,        /* a required pointer is NULL                          */
    SV_ERR_SHAPE = 2,       /* a size is out of range or inconsistent              */
    SV_ERR_UNSUPPORTED = 3, /* a valid request the library does not implement      */
    SV_ERR_WORKSPACE = 4,   /* workspace NULL or smaller than the query returned   */
    SV_ERR_ALIGN = 5,       /* a pointer lacks the alignment stated for it         */
    SV_ERR_HIP = 6          /* the HIP runtime reported an error while enqueueing  */
} sv_status;

/* Storage type of the KV cache. */
typedef enum {
    SV_KV_F32 = 0,       /* float32                                                */
    SV_KV_BF16 = 1,      /* bfloat16                                               */
    SV_KV_FP8_E4M3 = 2   /* OCP 8-bit float E4M3 ("fn": bias 7, no inf, max 448),
                            value = decode(code) * scale[physical block]           */
} sv_kv_dtype;

/* Attention implementation (spec_verify_attn_ex only). */
typedef enum {
    SV_ATTN_AUTO = 0,  /* matrix cores for bf16/fp8 storage, vector ALU for fp32  */
    SV_ATTN_VALU = 1,  /* vector-ALU kernel, any storage type                      */
    SV_ATTN_MFMA = 2   /* matrix-core kernel (bf16 and fp8 storage only)           */
} sv_attn_algo;

int sv_abi_version(void);
const char *sv_status_string(int status);
/* Thread-local text of the last non-OK return on this thread ("" if none). */
const char *sv_last_error(void);

/* Zero-fills `bytes` bytes at the device pointer `workspace` on `stream` with a
 * fill kernel (safe to capture in a HIP graph).  Optional: no call requires a
 * zeroed workspace. */
int spec_verify_workspace_clear(void *workspace, size_t bytes, void *stream);

/* ------------------------------------------------------------------------
 * spec_verify_attn: paged GQA attention for the K+1 verify rows.
 *
 * Defines ("KV Cache + Speculative Decoding" 5.2-5.3 paging, 6.1 cached
 * causal attention, 6.3 GQA; "Lecture 10 - Inference" 9.2):
 * for sequence b, verify row t in [0,T) and query head h in [0,Hq),
 *   g     = h / (Hq/Hkv)                      (query head -> KV head)
 *   n_vis = L_b - T + 1 + t                   (L_b counts the T new tokens,
 *                                              whose K/V are already cached)
 *   key/value of position p < n_vis: block_table[b][p/16], slot p%16, head g
 *   s_p   = sm_scale * <q[b,t,h,:], k_p>,  w = softmax(s),  out = sum_p w_p v_p
 *
 * q            [B,T,Hq,d] float32, 16-byte aligned.
 * k_cache      [num_blocks,16,Hkv,d] in kv_dtype, 16-byte aligned (8 for fp8).
 * v_cache      same shape and type as k_cache.
 * k_scale      [num_blocks] float32 per-block scales, positive and finite;
 * v_scale        required for SV_KV_FP8_E4M3, must be NULL otherwise.
 * block_table  [B,max_blocks_per_seq] int32 physical block ids in
 *              [0,num_blocks); entries at and past ceil(L_b/16) are never read.
 * context_lens [B] int32, T <= L_b <= 16*max_blocks_per_seq.
 * out          [B,T,Hq,d] float32, 16-byte aligned; fully overwritten.
 * T            = K+1 verify rows per sequence, 1..16.
 * Hq % Hkv == 0; T*(Hq/Hkv) <= 128; d in {64,128}; block_size == 16;
 * max_blocks_per_seq <= 65536 (contexts up to 1M tokens).
 * sm_scale     softmax scale, normally 1/sqrt(d).
 * workspace    >= spec_verify_attn_workspace_size(...) bytes, 256-byte
 *              aligned.
 * Work: one attention kernel, plus a small merge kernel when a sequence's
 * context is split across workgroups.
 * Slots past L_b in a sequence's last block may hold anything (NaN
 * included): they never reach the result.
 * ------------------------------------------------------------------------ */
size_t spec_verify_attn_workspace_size(int B, int T, int Hq, int Hkv, int d,
                                       int max_blocks_per_seq);

int spec_verify_attn(const float *q, const void *k_cache, const void *v_cache,
                     const float *k_scale, const float *v_scale,
                     const int32_t *block_table, const int32_t *context_lens,
                     float *out,
                     int B, int T, int Hq, int Hkv, int d, int block_size,
                     int max_blocks_per_seq, int num_blocks, int kv_dtype,
                     float sm_scale, void *workspace, size_t workspace_bytes,
                     void *stream);

/* As spec_verify_attn, with the implementation and the context split chosen
 * by the caller (for measurement).  blocks_per_split = 0 lets the planner
 * choose; -1 asks for balanced shares (below); otherwise it must be a
 * positive multiple of 4, at most 512, with
 * ceil(max_blocks_per_seq / blocks_per_split) <= 128, and every sequence's
 * context is cut into splits of that many pages.  The workspace must then
 * hold spec_verify_attn_workspace_size_ex(..., blocks_per_split) bytes.
 *
 * Balanced shares (matrix-core kernel only; B <= 1024 and
 * B*Hkv*max_blocks_per_seq <= 2^30, else SV_ERR_UNSUPPORTED): the
 * (sequence, KV head, page) triples of the whole batch, in that order, are
 * cut on the device, from context_lens, into equal runs of S pages, one per
 * workgroup, so a ragged batch leaves no long workgroup behind.  With 8-wave
 * workgroups -- at most two or exactly four 16-row tiles of verify rows per
 * KV head, E4M3 with d = 128 and three or more tiles, or more than four
 * tiles -- S = min(2048, max(4, ceil(total / 256))), one run per compute
 * unit; otherwise (4 waves) S = max(4, ceil(total / 256)) while that is at
 * most 512, else S = min(1024, ceil(total / 512)).  With at most two tiles
 * and an even Hkv a workgroup runs KV heads 2j and 2j+1 side by side: the
 * runs then cut the (sequence, head pair, page) triples, total being half
 * the pages of the batch's (sequence, KV head) units.  The planner uses them for
 * batches of two or more sequences with B*Hkv*max_blocks_per_seq >= 65536
 * when the matrix-core kernel runs.  Results agree with the fixed split up
 * to the order of floating-point additions.
 *
 * main_done_event: optional hipEvent_t (NULL to skip), recorded on `stream`
 * after the main attention kernel and before the split merge, so a caller
 * can time the main kernel on its own. */
size_t spec_verify_attn_workspace_size_ex(int B, int T, int Hq, int Hkv, int d,
                                          int max_blocks_per_seq, int blocks_per_split);

int spec_verify_attn_ex(const float *q, const void *k_cache, const void *v_cache,
                        const float *k_scale, const float *v_scale,
                        const int32_t *block_table, const int32_t *context_lens,
                        float *out,
                        int B, int T, int Hq, int Hkv, int d, int block_size,
                        int max_blocks_per_seq, int num_blocks, int kv_dtype,
                        float sm_scale, void *workspace, size_t workspace_bytes,
                        void *stream, int algo, int blocks_per_split,
                        void *main_done_event);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the
 * attention of spec_verify_attn, with the planner's split, using a static
 * device scratch array of the library instead of a caller workspace.  The
 * results are those of spec_verify_attn bit for bit.  Nothing is allocated:
 * the array (spec_verify_attn_noalloc_max_bytes() bytes, 32 MiB) lives in the
 * library's code object, one copy per GPU, held until the process ends; the
 * first call on a device looks up its address there (hipGetSymbolAddress)
 * with that device current.  A shape whose split needs more scratch than the
 * array holds (spec_verify_attn_workspace_size > the maximum) returns
 * SV_ERR_UNSUPPORTED before anything is enqueued.  Every call on one GPU
 * shares that GPU's array: calls that overlap in time on one GPU (two
 * streams, two threads) race and give undefined results; calls in one
 * stream order are safe.  Nothing in the array needs clearing between calls.
 * Arguments, errors and the device the work runs on (that of `stream`) as
 * spec_verify_attn. */
size_t spec_verify_attn_noalloc_max_bytes(void);
int spec_verify_attn_noalloc(const float *q, const void *k_cache, const void *v_cache,
                             const float *k_scale, const float *v_scale,
                             const int32_t *block_table, const int32_t *context_lens,
                             float *out, int B, int T, int Hq, int Hkv, int d,
                             int block_size, int max_blocks_per_seq, int num_blocks,
                             int kv_dtype, float sm_scale, void *stream);

/* MEASUREMENT ONLY -- not part of the verify step.  Validates exactly as
 * spec_verify_attn_ex, then enqueues the main attention kernel alone, so
 * that back-to-back calls between two events time that kernel by itself.
 * When the planner (or blocks_per_split) splits a sequence's context, `out`
 * is NOT written: the unnormalised partials stay in the workspace and the
 * split merge that spec_verify_attn_ex would run next is skipped.  Never use
 * its `out` as a result. */
int spec_verify_attn_timing_main_only(const float *q, const void *k_cache, const void *v_cache,
                                      const float *k_scale, const float *v_scale,
                                      const int32_t *block_table, const int32_t *context_lens,
                                      float *out, int B, int T, int Hq, int Hkv, int d,
                                      int block_size, int max_blocks_per_seq, int num_blocks,
                                      int kv_dtype, float sm_scale, void *workspace,
                                      size_t workspace_bytes, void *stream, int algo,
                                      int blocks_per_split);

/* MEASUREMENT ONLY -- not part of the verify step.  The practical HBM read
 * ceiling the attention kernel is compared with: one plain streaming read
 * of `bytes` bytes (a positive multiple of 16) at the 16-byte aligned device
 * pointer `src`, contiguous chunks per workgroup.  Each thread leaves a
 * float in `sink` (device memory of at least
 * spec_verify_probe_read_sink_floats() floats), so the reads cannot be
 * dropped; its values mean nothing. */
size_t spec_verify_probe_read_sink_floats(void);
int spec_verify_probe_read(const void *src, size_t bytes, float *sink, size_t sink_floats,
                           void *stream);

/* ------------------------------------------------------------------------
 * spec_verify_sample: the rejection sampler of the verify step.
 *
 * Defines ("50 | Speculative Decoding" 3.1; "KV Cache + Speculative
 * Decoding" 7.1-7.3, 7.6): with p_i = softmax(target_logits[b,i,:]),
 *   for i = 0..K-1, draft x_i = draft_tokens[b,i] is accepted iff
 *     u[b,i] * q_i(x_i) < p_i(x_i)        (acceptance with min(1, p/q));
 *   n = index of the first rejection, or K if none;
 *   weights w = max(0, p_n - q_n) if n < K, else w = p_K (bonus);
 *   if sum(w) == 0 (reachable only by rounding) w = p_n;
 *   the drawn token is the smallest j with sum_{j'<=j} w_j' > u[b,K]*sum(w)
 *   in ascending token order (the largest j with w_j > 0 if rounding leaves
 *   none).
 * Outputs: num_accepted[b] = n; out_tokens[b,0:n] = the accepted drafts,
 * out_tokens[b,n] = the drawn token, out_tokens[b,n+1:] = -1.
 *
 * target_logits [B,K+1,V] float32 (finite), draft_probs [B,K,V] float32
 * (>= 0, used as given), draft_tokens [B,K] int32 in [0,V), uniforms [B,K+1]
 * float32 in [0,1): [:, :K] drive acceptance, [:, K] the final draw.
 * num_accepted [B] int32; out_tokens [B,K+1] int32; accept_prob [B,K] float32
 * (optional, NULL to skip) receives min(1, p_i(x_i)/q_i(x_i)) for every i.
 * 1 <= K <= 15; V >= 1.  workspace as for attention.
 * Rows after a sequence's first rejection cannot change any output; when the
 * batch holds at least 64 MiB of target rows and accept_prob is NULL (and no
 * top-p cut is asked for), the rows after a rejection among the first
 * max(2, 3(K+1)/8) drafts are not read at all.
 * ------------------------------------------------------------------------ */
/* Typical acceptance ("50 | Speculative Decoding" 9.1; "KV Cache +
 * Speculative Decoding" 8.2 and Q18): NOT exact.  Draft x_i is accepted iff
 * the target's own probability of it exceeds an entropy-based threshold,
 *   p~_i(x_i) > min(eps, delta * exp(-H(p~_i))),
 * with p~_i = softmax(target_logits row i / T_b) and H its entropy in nats;
 * no draft probabilities are needed.  n = the first rejected position (or
 * K); the next token is drawn from p~_n itself with uniforms[b][K] (inverse
 * CDF in token order, as spec_verify_sample).  T_b <= 0 is greedy (H = 0).
 *   temperature: [B] or NULL (1); eps, delta: finite, >= 0 (the pages give no
 *   values: the caller's choice).
 *   p_draft, threshold: optional [B][K] float outputs (NULL ok): p~_i(x_i)
 *   and the threshold of every position up to the first rejection.
 * Outputs and workspace as spec_verify_sample. */
int spec_verify_sample_typical(const float *target_logits, const int32_t *draft_tokens,
                               const float *uniforms, const float *temperature,
                               double eps, double delta,
                               int32_t *num_accepted, int32_t *out_tokens,
                               float *p_draft, float *threshold,
                               int B, int K, int V,
                               void *workspace, size_t workspace_bytes, void *stream);

/* Tree verification attention ("KV Cache + Speculative Decoding" 8.2 and
 * Q14): the T nodes of a draft tree, flattened in BFS order, are the T verify
 * rows; their K/V occupy the last T cache positions (L_b - T .. L_b - 1, in
 * node order).  Node t attends to the prefix (positions < L_b - T) and to the
 * nodes of its ancestor set: bit j of tree_mask[b*T + t] set iff node j lies
 * on the path from the root (node 0) to t, t itself included.
 *   tree_mask: [B][T] uint32, device memory, 4-byte aligned.  Every set must
 *   hold its own node and no later node (ancestors precede in BFS order);
 *   other sets give undefined (but memory-safe) results.  The chain's sets
 *   {0..t} make this spec_verify_attn_ex exactly.
 * Every other argument, the workspace and the errors as spec_verify_attn_ex
 * (T <= 16, T*Hq/Hkv <= 128). */
int spec_verify_attn_tree(const float *q, const void *k_cache, const void *v_cache,
                          const float *k_scale, const float *v_scale,
                          const int32_t *block_table, const int32_t *context_lens,
                          const uint32_t *tree_mask, float *out,
                          int B, int T, int Hq, int Hkv, int d, int block_size,
                          int max_blocks_per_seq, int num_blocks, int kv_dtype,
                          float sm_scale, void *workspace, size_t workspace_bytes,
                          void *stream, int algo, int blocks_per_split);

size_t spec_verify_sample_workspace_size(int B, int K, int V);

int spec_verify_sample(const float *target_logits, const float *draft_probs,
                       const int32_t *draft_tokens, const float *uniforms,
                       int32_t *num_accepted, int32_t *out_tokens, float *accept_prob,
                       int B, int K, int V,
                       void *workspace, size_t workspace_bytes, void *stream);

/* As spec_verify_sample with the target rows transformed per sequence by a
 * temperature and a top-p cut ("KV Cache + Speculative Decoding" 7.5 and its
 * answer on temperature / top-p: exactness holds with the sampler-
 * transformed target p~ in place of p, whatever distribution the draft
 * sampled from).  Every target row of sequence b becomes
 *   p~ = softmax(target_logits / T_b), then cut to its top-p set and
 *   renormalised,
 * in the acceptance tests, the residual and the bonus draw.  draft_probs are
 * the draft's actual (already transformed) distribution and are used as
 * given.
 *   temperature: [B] float32, or NULL for T = 1.  T_b <= 0 (or NaN) is the
 *     greedy limit: all mass on the first maximal logit of the row, so a
 *     draft is accepted iff it is that token and the drawn token is the
 *     argmax of row n (top_p does not apply).
 *   top_p: [B] float32, or NULL for no cut.  Tokens are ranked by logit; a
 *     token is kept iff the p~-mass ranked strictly above it is below top_p_b;
 *     the tokens of the maximal logit are always kept (so top_p_b <= 0 keeps
 *     only them) and equal logits are kept or dropped together.
 *     top_p_b >= 1 or NaN: no cut.  Masses are summed in 2^-43 fixed point
 *     (deterministic), which needs V < 2^20 when top_p is given
 *     (SV_ERR_UNSUPPORTED otherwise).  Adds one launch.
 * With both NULL this is spec_verify_sample.  Same workspace. */
int spec_verify_sample_ex(const float *target_logits, const float *draft_probs,
                          const int32_t *draft_tokens, const float *uniforms,
                          const float *temperature, const float *top_p,
                          int32_t *num_accepted, int32_t *out_tokens, float *accept_prob,
                          int B, int K, int V,
                          void *workspace, size_t workspace_bytes, void *stream);

/* Tree verification sampler ("KV Cache + Speculative Decoding" 8.2: the draft
 * tree's N nodes, flattened in BFS order, are scored by one target forward;
 * exact verification keeps the rejection rule of "50 | Speculative
 * Decoding" 3.1 and "KV Cache + Speculative Decoding" 7.1-7.3).
 *   target_logits [B][N][V] f32: row c = target logits after node c's path
 *     (node 0, the root, is the last committed token);
 *   draft_probs   [B][N][V] f32: row c = the draft distribution the children
 *     of node c were drawn from (rows of leaves are not read);
 *   tokens  [B][N] i32: token of node c (column 0 unused), in [0, V);
 *   parents [B][N] i32: BFS parents, parents[b][0] = -1, 0 <= parents[b][c] < c;
 *   uniforms [B][N] f32 in [0,1): column c >= 1 tests node c, column 0 drives
 *     the final draw.
 * Rule: from the root, the children of the current node are tried in BFS
 * order, each against the target as left by the siblings rejected before it
 * (after k rejections p_{k+1} = norm(max(0, p_k - q)), the chain's residual
 * step applied per rejected sibling; for the first child this is the chain's
 * test u * q(x) < p(x)).  An accepted child becomes the current node; when
 * no child is accepted, or the node is a leaf, the final token is drawn from
 * the current residual (p itself if nothing was rejected) by the chain's
 * inverse CDF.  With siblings drawn independently from their parent's draft
 * row every emitted token follows the target.  A chain tree is
 * spec_verify_sample exactly (uniforms remapped: column i+1 tests draft i,
 * column 0 is the chain's last uniform).
 * Outputs: num_accepted [B] (accepted nodes, the root not counted);
 *   out_tokens [B][N] (the accepted nodes' tokens, the drawn token, then -1);
 *   path [B][N] (the accepted node ids in order, then -1) -- the K/V of
 *   these nodes are the ones the cache keeps; accept_prob [B][N] optional
 *   (NULL ok): min(1, p_k(x)/q(x)) of every tested node, NaN elsewhere.
 * max_children: the largest number of children of any node (0 .. N-1,
 *   known to the caller from its tree shape).  One extra launch per sibling
 *   rank 2 .. max_children prepares the normalisers; a node's children of
 *   higher rank are skipped (never tested), so pass at least the true
 *   maximum.
 * Parents that break the BFS order are clamped into [0, c-1] (results
 * undefined, memory-safe).  N <= 16.  Workspace:
 * spec_verify_sample_tree_workspace_size(B, N, V) bytes, 256-byte aligned. */
size_t spec_verify_sample_tree_workspace_size(int B, int N, int V);
int spec_verify_sample_tree(const float *target_logits, const float *draft_probs,
                            const int32_t *tokens, const int32_t *parents, const float *uniforms,
                            int32_t *num_accepted, int32_t *out_tokens, int32_t *path,
                            float *accept_prob, int B, int N, int V, int max_children,
                            void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * spec_verify_kv_append: write the K/V of the T verify positions into the
 * paged cache, before spec_verify_attn.
 *
 * Defines ("KV Cache + Speculative Decoding" 6.1 append, 6.2 paged data
 * structure; "Lecture 10 - Inference" 9.2): for sequence b, verify position
 * t in [0,T) and KV head g, with L_b = context_lens[b] (which, as for
 * spec_verify_attn, already counts the T new positions):
 *   p = L_b - T + t,  page = block_table[b][p/16],  slot = p % 16
 *   k_cache[page][slot][g][:] = enc(k_new[b][t][g][:]);  v likewise.
 * enc: SV_KV_F32 stores the float; SV_KV_BF16 rounds to nearest, ties to
 * even (NaN stays NaN); SV_KV_FP8_E4M3 stores the OCP E4M3 code of
 * x / scale[page] (the quotient rounded to float, then to nearest E4M3 with
 * ties to even; magnitudes above 448, infinities included, saturate to
 * +-448; NaN gives the NaN code 0x7F).  The page scales belong to the
 * caller: they are read, never written.  No other byte of the caches is
 * touched.
 *
 * k_new, v_new [B,T,Hkv,d] float32, 16-byte aligned; k_cache/v_cache as for
 * spec_verify_attn, aligned to 16 (fp32), 8 (bf16) or 4 (E4M3) bytes.
 * k_scale, v_scale: [num_blocks] float32, positive and finite, required for
 * SV_KV_FP8_E4M3, NULL otherwise.  1 <= T <= 16; d % 4 == 0; block_size ==
 * 16.  The pages the new positions fall in must already be in the table
 * (allocation is the caller's).  Device-data preconditions: T <= L_b <=
 * 16*max_blocks_per_seq, page ids in [0,num_blocks).
 * ------------------------------------------------------------------------ */
int spec_verify_kv_append(const float *k_new, const float *v_new, void *k_cache, void *v_cache,
                          const float *k_scale, const float *v_scale, const int32_t *block_table,
                          const int32_t *context_lens, int B, int T, int Hkv, int d, int block_size,
                          int max_blocks_per_seq, int num_blocks, int kv_dtype, void *stream);

/* ------------------------------------------------------------------------
 * spec_verify_rollback: truncate the cache after the sampler, in O(1) per
 * sequence ("KV Cache + Speculative Decoding" 7.6: keep the last committed
 * token and the accepted drafts; the drawn token enters the cache in the
 * next round; a paged cache rolls back by changing its table, not its data).
 *
 *   context_lens[b] <- context_lens[b] - K + num_accepted[b]
 *   pages_in_use[b]  = ceil(context_lens[b] / 16)      (optional, NULL to skip)
 * Table entries from pages_in_use[b] on no longer hold live positions; the
 * caller may return them to its page pool.  num_accepted[b] is clamped to
 * [0,K]; context_lens must count the T = K+1 verify positions on entry.
 * num_accepted [B] int32 (as written by spec_verify_sample); context_lens [B]
 * int32, updated in place; pages_in_use [B] int32.  1 <= K <= 15.
 * ------------------------------------------------------------------------ */
int spec_verify_rollback(const int32_t *num_accepted, int32_t *context_lens, int32_t *pages_in_use, int B, int K,
                         void *stream);

/* Tree commit ("KV Cache + Speculative Decoding" 8.2, with 7.6's note that a
 * paged cache rolls back by editing its bookkeeping): after
 * spec_verify_sample_tree, each sequence keeps the root (the last committed
 * token, at base = L_b - N) and the n_b accepted nodes of the path, in path
 * order, at the consecutive positions base+1 .. base+n_b: node path[b][i]
 * moves from base + path[b][i] to base + 1 + i (all K and V heads), then
 * context_lens[b] = base + 1 + n_b and, if pages_in_use is non-NULL,
 * pages_in_use[b] = ceil(that / 16).  The drawn token is appended next
 * round, as after spec_verify_rollback; a chain path (path[i] = i + 1) moves
 * nothing and equals spec_verify_rollback with K = N - 1.
 * E4M3: a value that changes page is re-encoded for the destination page
 * (decode * scale_src in float, then x / scale_dst encoded as
 * spec_verify_kv_append encodes); scales are never rewritten.
 *   path [B][N], num_accepted [B]: as written by spec_verify_sample_tree
 *   (entries past n_b are not read).  Out-of-contract data is clamped
 *   (results undefined, memory-safe).  Two launches; no workspace.
 *   N <= 16, d a multiple of 4 up to 256, block_size 16. */
int spec_verify_tree_commit(const int32_t *path, const int32_t *num_accepted,
                            void *k_cache, void *v_cache,
                            const float *k_scale, const float *v_scale,
                            const int32_t *block_table, int32_t *context_lens,
                            int32_t *pages_in_use, int B, int N, int Hkv, int d,
                            int block_size, int max_blocks_per_seq, int num_blocks,
                            int kv_dtype, void *stream);

/* ------------------------------------------------------------------------
 * spec_verify_check_inputs: a debug aid that counts the device-data
 * preconditions the calls above document but do not check (they stay
 * memory-safe on such data by clamping; their results are then undefined).
 *
 * Checks ("KV Cache + Speculative Decoding" 5.2-5.3 paged cache and 6.1
 * cached attention; "50 | Speculative Decoding" 3.1 acceptance test), per
 * sequence b < B, each into one counter of counts[SV_CHECK_COUNTS]:
 *   [0] context_lens[b] outside [T, 16 * max_blocks_per_seq];
 *   [1] block_table[b][i] outside [0, num_blocks) for the pages holding
 *       visible positions, i < ceil(min(max(L_b, 0), 16*max_blocks)/16);
 *   [2] tokens[b][i], i < n_tokens, outside [0, V);
 *   [3] uniforms[b][i], i < n_uniforms, outside [0, 1) or not finite.
 * context_lens NULL skips [0] and [1]; block_table NULL skips [1]; tokens
 * NULL skips [2]; uniforms NULL skips [3] (the sizes of a skipped check
 * are ignored).  counts: int32[SV_CHECK_COUNTS] device memory, cleared and
 * then written on `stream` (read it after synchronising).  Allocates
 * nothing; two launches.
 * ------------------------------------------------------------------------ */
#define SV_CHECK_COUNTS 4
int spec_verify_check_inputs(const int32_t *block_table, const int32_t *context_lens, int T,
                             int max_blocks_per_seq, int num_blocks,
                             const int32_t *tokens, int n_tokens, int V,
                             const float *uniforms, int n_uniforms,
                             int B, int32_t *counts, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
