// sv_internal.hpp -- host-side argument blocks shared by the C ABI layer and
// the kernel launchers.  Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sv {

constexpr int kBlock = 16;          // tokens per KV page
constexpr int kMaxRows = 128;       // T * (Hq/Hkv) per (sequence, kv head) unit
constexpr int kMaxSplits = 128;     // context splits per unit
constexpr int kMaxBps = 512;        // context pages per split
constexpr int kAttnThreads = 256;   // 4 waves per workgroup (vector-ALU kernel)

// Workgroup shape of the matrix-core attention kernel for head size d, rg
// 16-row tiles per KV head, E4M3 storage (fp8) and balanced shares (bal).
// Shared pages (two waves per page stream, each holding half of the row
// tiles) for E4M3 with d = 128 and three or more tiles, for more than four
// tiles, and for four tiles under balanced shares (ragged 64-sequence batch
// with 16 verify rows: 504 -> 488 us; with three tiles, the 70B-layer shape,
// they measured slower: 196 -> 216 us; with fixed splits slower too).
// Otherwise every wave holds every row tile and streams pages of its own: 4
// waves, one per SIMD, except that balanced shares with at most two tiles run
// 8 (two per SIMD, one workgroup per compute unit): two 4-wave workgroups on
// one compute unit do not progress alike (the one dispatched first finished a
// 528-page share ~25% sooner), so the unit idled at the end; one 8-wave
// workgroup per unit finishes its waves together.  (Fixed splits measured
// faster with 4 waves: 64-page splits of an 8B-layer shape 28.3 against
// 29.1 us.)
constexpr bool attn_share_pages(int d, int rg, bool fp8, bool bal)
{
    return (fp8 && d == 128 && rg >= 3) || rg > 4 || (bal && rg == 4);
}
constexpr int attn_page_streams(int d, int rg, bool fp8, bool bal)
{
    return (bal && !attn_share_pages(d, rg, fp8, bal) && rg <= 2) ? 8 : 4;
}
constexpr int attn_waves(int d, int rg, bool fp8, bool bal)
{
    return attn_share_pages(d, rg, fp8, bal) ? 8 : attn_page_streams(d, rg, fp8, bal);
}

// Everything one attention launch needs.  Sizes are validated by the caller.
struct AttnParams {
    const float *q;
    const void *k_cache;
    const void *v_cache;
    const float *k_scale;
    const float *v_scale;
    const int32_t *block_table;
    const int32_t *context_lens;
    float *out;
    float *part_o;         // [slot][TG][d]  unnormalised partial outputs
    float *part_ml;        // [slot][TG][2]  (running max in log2 units, sum)
                           // fixed splits: slot = unit * max_splits + split;
                           // balanced shares: slot = unit + workgroup
    int *bal_prefix;       // balanced shares: [B+1] pages of the sequences before b (written by workgroup 0)
    int balanced;          // 1: every workgroup takes an equal share of all (unit, page) pairs
    int bal_one;           // balanced shares: 1 = one share per compute unit (8-wave workgroups)
    int bal_hg;            // balanced shares: KV heads a workgroup runs side by side (see bal_heads), else 1
    int B, T, Hq, Hkv, G, TG, d;
    int max_blocks, num_blocks;
    int bps;               // context blocks per split (multiple of 8)
    int max_splits;        // ceil(max_blocks / bps)
    int grid;              // workgroups launched (multiple of 8)
    float qscale;          // sm_scale * log2(e): scores are kept in base-2 units
    const uint32_t *tree_mask;  // [B][T] ancestor sets of the verify rows, or null (the chain)
};

struct AttnPlan {
    int bps;
    int max_splits;
    size_t off_part_o, off_part_ml;
    // balanced shares (usable by the matrix-core kernel only): grid and
    // workspace layout; the fixed-split fields above stay valid for the
    // vector-ALU kernel
    int balanced;
    int grid_bal;
    size_t off_prefix, off_bal_o, off_bal_ml;
    size_t total;  // bytes covering whichever layout the call uses
};

// Balanced shares.  The (unit, page) pairs of the whole batch, units in
// order b * Hkv + g and pages in order within a unit, are cut into equal
// shares of S pages, one per workgroup, so ragged context lengths leave no
// long workgroup behind.  8-wave workgroups (one fills a compute unit):
// S = min(kBalMaxShareOne, max(4, ceil(total / kBalTargetWgs))), one share
// per compute unit.  4-wave workgroups: the same while S is at most
// kBalOneShare pages, else S = min(kBalMaxShare, ceil(total / (2 *
// kBalTargetWgs))) (two per compute unit, all resident at once, rather than a
// second round of a few).
// Chosen by the planner for large batches of several sequences (at least
// kBalMinPages pairs at the longest context, at most kBalMaxB sequences).
// Head groups.  With 8-wave workgroups in which every wave streams pages of
// its own (at most two row tiles), the workgroup runs bal_heads(Hkv) KV heads
// side by side: wave w takes head w % hg of the group and every (8 / hg)-th
// page of the run, so both heads' slices of a page are read at about the same
// time, and each head's pages go to two older and two younger waves.  Shares
// then cut the list of (group, page) pairs, groups in order
// b * (Hkv / hg) + head group.  Ragged 64-sequence batch of 8 KV heads, main
// kernel: one head per workgroup 419.5 us, 2 heads 412, 4 heads 412, 8 heads
// 414.5; every sequence at the mean length: 383, 376, 401, 412 (the larger
// groups cut every group of that batch, and with 8 heads the heads of the
// younger waves set the pace).  (A read-only probe of the same bytes: one
// head's slices at a time 351 us, whole pages 328 us.)
constexpr int bal_heads(int hkv)
{
    return hkv % 2 == 0 ? 2 : 1;
}
constexpr int kSplitBalanced = -1;      // blocks_per_split value that asks for balanced shares
constexpr int kBalMaxB = 1024;          // sequences (prefix sums held in LDS)
constexpr int kBalTargetWgs = 256;      // shares aimed for: one per compute unit
constexpr int kBalOneShare = 512;      // longest share at one workgroup per compute unit
constexpr int kBalMaxShare = 1024;     // pages per share, two per compute unit (page ids held in LDS)
constexpr int kBalMaxShareOne = 2048;  // pages per share, one per compute unit
constexpr long long kBalMinPages = 65536;
constexpr long long kBalMaxPages = 1LL << 30;  // (unit, page) pairs: positions stay in int

AttnPlan plan_attention(int B, int T, int Hq, int Hkv, int d, int max_blocks, int bps_request);

// The main attention kernel of each implementation, and the split merge
// (a no-op launch-wise when max_splits == 1).
hipError_t launch_attn_mfma(const AttnParams &p, int kv_dtype, hipStream_t stream);
hipError_t launch_attn_valu(const AttnParams &p, int kv_dtype, hipStream_t stream);
hipError_t launch_attn_merge(const AttnParams &p, hipStream_t stream);

constexpr int kSampleChunk = 8192;  // vocabulary entries per sampler workgroup
constexpr int kSampleSub = 1024;    // entries per sub-chunk (unit of the draw's rescan)
constexpr int kSampleThreads = 256;
constexpr int kDecideMaxSpw = 16;    // sub-chunks one decide workgroup covers at most
constexpr int kMaxSampleChunks = 2048;  // V <= 2048 * 8192
// Chain sampler, early exit: at least this many bytes of target rows (and
// no output that needs every row) split the row statistics in two launches,
// the second reading only the sequences that accepted every draft the first
// half of the rows tests (see launch_sample).
constexpr double kGateMinBytes = 64.0 * 1024 * 1024;

struct SampleParams {
    const float *logits;     // [B][K+1][V]
    const float *probs;      // [B][K][V]
    const int32_t *tokens;   // [B][K]
    const float *uniforms;   // [B][K+1]
    const float *temperature;  // [B] or null (1)
    const float *top_p;        // [B] or null (no cut)
    int32_t *num_accepted;   // [B]
    int32_t *out_tokens;     // [B][K+1]
    float *accept_prob;      // [B][K] or null
    void *seq_state;         // [B] {accepted count, row max, 1/row sum, 1/T, greedy, argmax, cut}
    void *row_cut;           // [B*(K+1)] {cut logit, 1/kept mass}, or null without top_p
    unsigned long long *cut_part;  // [B*(K+1)][nchunk][kCutCoarse] partial coarse histograms
    int qrows;               // draft rows per sequence: K (chain) or N (tree)
    int tree;                // tree verification: K + 1 = N nodes, see launch_sample_tree
    const int32_t *parents;  // tree: [B][N] BFS parents (parents[b][0] < 0)
    int32_t *path;           // tree: [B][N] accepted node ids, then -1
    double *coefs;           // tree: [B][N][nchunk] chunk partials of each node's test normaliser
    double *tree_c;          // tree: [B][N] coefficient C of each node's test (ranks >= 2)
    int tree_max_children;   // tree: children tested per node (ranks beyond are skipped)
    int typical;             // typical acceptance instead of the rejection rule
    double ty_eps, ty_delta; // its threshold min(eps, delta exp(-H))
    double *row_ent;         // typical: [B*(K+1)][nchunk] sum over the chunk of e^{a - a_max}(a - a_max)
    float *threshold_out;    // typical: [B][K] thresholds, or null
    void *row_stats;         // [B*(K+1)][nchunk] {float max, double sum}
    void *row_x;             // [B*K] {target logit, draft probability} of draft token x_i
    double *sub_mass;        // [B][ceil(V/1024)][2] {residual weight, target mass}
    int B, K, V, nchunk;
    int vec4;                // rows start 16-byte aligned and V % 4 == 0
    int spw;                 // chain decide: consecutive sub-chunks per workgroup (1..kDecideMaxSpw; set by launch_sample)
    int row_lo, row_cnt;     // rowstats: rows row_lo .. row_lo + row_cnt - 1 of every sequence (set by the launchers)
    int gate_r;              // rowstats: > 0 reads only the sequences whose gate flag is set
    int32_t *gate;           // [B] 1 iff drafts 0 .. R-1 are all accepted (early exit, see launch_sample)
};

struct SamplePlan {
    int nchunk;
    size_t off_state, off_stats, off_rowx, off_mass, off_cut, off_part, off_ent, off_gate, total;
};

constexpr size_t kSeqStateBytes = 64;  // workspace bytes per sequence of the decide -> pick state
constexpr size_t kRowCutBytes = 16;    // workspace bytes per target row of the top-p cut
constexpr int kCutMaxV = 1 << 20;      // the cut's fixed-point masses need V < 2^20
constexpr int kCutCoarse = 512;        // coarse buckets of the top-p cut

SamplePlan plan_sample(int B, int K, int V);
hipError_t launch_sample(const SampleParams &p, hipStream_t stream);

// Tree verification: B sequences of N <= 16 BFS-ordered nodes.
struct TreePlan {
    int nchunk;
    size_t off_state, off_stats, off_mass, off_coefs, off_tree_c, total;
};
TreePlan plan_sample_tree(int B, int N, int V);
hipError_t launch_sample_tree(const SampleParams &p, hipStream_t stream);
hipError_t launch_clear(void *ptr, size_t bytes, hipStream_t stream);

// Appending the T verify positions to the paged cache.
struct AppendParams {
    const float *k_new;            // [B][T][Hkv][d]
    const float *v_new;
    void *k_cache;                 // [num_blocks][16][Hkv][d] of the storage type
    void *v_cache;
    const float *k_scale;          // [num_blocks] (E4M3 only)
    const float *v_scale;
    const int32_t *block_table;    // [B][max_blocks]
    const int32_t *context_lens;   // [B], including the T new positions
    int B, T, Hkv, d, max_blocks, num_blocks;
};

// Moving the accepted path of a tree next to its root.
struct TreeCommitParams {
    const int32_t *path;          // [B][N] accepted node ids
    const int32_t *num_accepted;  // [B]
    void *k_cache;
    void *v_cache;
    const float *k_scale;
    const float *v_scale;
    const int32_t *block_table;
    int32_t *context_lens;
    int32_t *pages_in_use;
    int B, N, Hkv, d, max_blocks, num_blocks;
};
hipError_t launch_tree_commit(const TreeCommitParams &p, int kv_dtype, hipStream_t stream);

hipError_t launch_kv_append(const AppendParams &p, int kv_dtype, hipStream_t stream);

// Counting violations of the device-data preconditions (a debug aid).
constexpr int kCheckCounts = 4;
struct CheckParams {
    const int32_t *block_table;   // [B][max_blocks] or null
    const int32_t *context_lens;  // [B] or null
    const int32_t *tokens;        // [B][n_tokens] or null
    const float *uniforms;        // [B][n_uniforms] or null
    int32_t *counts;              // [kCheckCounts]
    int B, T, max_blocks, num_blocks, n_tokens, V, n_uniforms;
};
hipError_t launch_check_inputs(const CheckParams &p, hipStream_t stream);
// Measurement only: a plain streaming read of a device buffer (the practical
// HBM read ceiling); the sink holds kProbeWgs * kProbeThreads floats.
constexpr int kProbeWgs = 1024;
constexpr int kProbeThreads = 256;
hipError_t launch_probe_read(const void *src, size_t bytes, float *sink, hipStream_t stream);

hipError_t launch_rollback(const int32_t *num_accepted, int32_t *context_lens, int32_t *pages_in_use, int B, int K,
                           hipStream_t stream);

}  // namespace sv
