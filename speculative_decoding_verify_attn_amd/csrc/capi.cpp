// capi.cpp -- the C ABI of libspecverify: argument validation, the split
// planner, workspace layout and kernel dispatch on the caller's stream.
// Nothing here reads device memory, synchronises, or allocates.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/spec_verify.h"
#include "sv_internal.hpp"

namespace {

thread_local char g_err[512];

int fail(int status, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return status;
}

int ok()
{
    g_err[0] = '\0';
    return SV_OK;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int ceil_div(long long a, long long b) { return (int)((a + b - 1) / b); }

}  // namespace

// Scratch memory of spec_verify_attn_noalloc: the split partials and prefix
// sums that spec_verify_attn keeps in the caller's workspace, held instead in
// a static device array.  Every GPU the library runs on holds its own copy
// until the process ends.  In host code `scratch` names a host-side stand-in,
// not device memory: host code only ever uses the device address that
// hipGetSymbolAddress returns for the current device (noalloc_scratch).
static constexpr size_t kNoAllocScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

constexpr int kNoAllocMaxDevices = 256;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kNoAllocMaxDevices];  // device address of `scratch`, per device (null: not looked up yet)

// The device address of `scratch` on the device that `stream` belongs to (the
// current device for the NULL stream), looked up once per device with that
// device current.
int noalloc_scratch(hipStream_t stream, void **ptr)
{
    int dev = -1;
    hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess)
        return fail(SV_ERR_HIP, "finding the stream's device: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kNoAllocMaxDevices)
        return fail(SV_ERR_UNSUPPORTED, "device %d is beyond the %d devices the static scratch supports", dev,
                    kNoAllocMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        int cur = -1;
        e = hipGetDevice(&cur);
        if (e != hipSuccess)
            return fail(SV_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess)
            return fail(SV_ERR_HIP, "hipSetDevice(%d): %s", dev, hipGetErrorString(e));
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess && e2 != hipSuccess)
                e = e2;
        }
        if (e != hipSuccess || !p)
            return fail(SV_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                        e != hipSuccess ? hipGetErrorString(e) : "null address");
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return SV_OK;
}

}  // namespace

namespace sv {

// KV heads that one balanced-share workgroup runs side by side (head groups,
// see bal_heads): 8-wave workgroups whose waves each stream pages of their
// own, i.e. at most two row tiles per KV head (with balanced shares that
// shape does not depend on the KV storage type).
int bal_group_heads(int T, int Hq, int Hkv, int d)
{
    const int rg = (T * (Hq / Hkv) + 15) / 16;
    return attn_page_streams(d, rg, false, true) == 8 ? bal_heads(Hkv) : 1;
}

// Context split.  A workgroup streams its pages through a deep LDS pipeline,
// so it wants long splits; the grid wants at least one workgroup per compute
// unit (256).  Splits are multiples of 4 pages (one per wave) and at most
// kMaxBps pages, which also bounds ragged batches' longest workgroups.
AttnPlan plan_attention(int B, int T, int Hq, int Hkv, int d, int max_blocks, int bps_request)
{
    AttnPlan pl{};
    const long long units = (long long)B * Hkv;
    const long long pairs = units * max_blocks;  // (unit, page) pairs at the longest context
    const bool bal_ok = B <= kBalMaxB && pairs <= kBalMaxPages;
    // (one sequence cannot be ragged: the fixed split is as balanced and
    // needs no merge when it is not split)
    pl.balanced = bal_ok && (bps_request == kSplitBalanced || (bps_request == 0 && B > 1 && pairs >= kBalMinPages));
    int bps;
    if (bps_request > 0) {
        bps = bps_request;
    } else {  // the planner's fixed split (also the vector-ALU kernel's under balanced shares)
        const long long target_wgs = 256;
        long long splits = (target_wgs + units - 1) / units;
        if (splits < 1)
            splits = 1;
        bps = ceil_div(max_blocks, splits);
        bps = ((bps + 3) / 4) * 4;
        if (bps > kMaxBps)
            bps = kMaxBps;
        if (bps < 4)
            bps = 4;
    }
    pl.bps = bps;
    pl.max_splits = ceil_div(max_blocks, bps);
    const int TG = T * (Hq / Hkv);
    size_t off = 0;
    pl.off_part_o = off;
    if (pl.max_splits > 1) {
        off = align256(off + (size_t)units * pl.max_splits * TG * d * 4);
        pl.off_part_ml = off;
        off = align256(off + (size_t)units * pl.max_splits * TG * 2 * 4);
    } else {
        pl.off_part_ml = off;
    }
    size_t total = off;
    if (pl.balanced) {
        // ceil(total / S) shares never exceed this many workgroups (4-wave
        // shares: S is kBalMaxShare, or at least ceil(total / (2 *
        // kBalTargetWgs)); 8-wave shares, one per compute unit, are fewer:
        // at most max(kBalTargetWgs, ceil(total / kBalMaxShareOne)), the grid
        // such a call launches, see attn_impl).  Partials: slot unit + share;
        // with head groups of hg heads, (group + share) * hg + head in group,
        // below units + grid * hg.
        const long long g = std::max<long long>(2 * kBalTargetWgs, (pairs + kBalMaxShare - 1) / kBalMaxShare);
        pl.grid_bal = (int)g;
        const int hg = bal_group_heads(T, Hq, Hkv, d);
        const long long g1 = std::max<long long>(kBalTargetWgs, (pairs / hg + kBalMaxShareOne - 1) / kBalMaxShareOne);
        const long long slots = units + std::max(g, g1 * hg);
        size_t o = 0;
        pl.off_prefix = o;
        o = align256(o + (size_t)(B + 1) * 4);
        pl.off_bal_o = o;
        o = align256(o + (size_t)slots * TG * d * 4);
        pl.off_bal_ml = o;
        o = align256(o + (size_t)slots * TG * 2 * 4);
        total = std::max(total, o);
    }
    pl.total = total > 256 ? total : 256;
    return pl;
}

TreePlan plan_sample_tree(int B, int N, int V)
{
    TreePlan pl{};
    pl.nchunk = ceil_div(V, kSampleChunk);
    size_t off = 0;
    pl.off_state = off;
    off = align256(off + (size_t)B * kSeqStateBytes);
    pl.off_stats = off;
    off = align256(off + (size_t)B * N * pl.nchunk * 16);
    pl.off_mass = off;
    off = align256(off + (size_t)B * ceil_div(V, kSampleSub) * 2 * 8);
    pl.off_coefs = off;  // chunk partials of every node's test normaliser
    off = align256(off + (size_t)B * N * pl.nchunk * 8);
    pl.off_tree_c = off;  // coefficient of every node's test
    off = align256(off + (size_t)B * N * 8);
    pl.total = off;
    return pl;
}

SamplePlan plan_sample(int B, int K, int V)
{
    SamplePlan pl{};
    pl.nchunk = ceil_div(V, kSampleChunk);
    size_t off = 0;
    pl.off_state = off;
    off = align256(off + (size_t)B * kSeqStateBytes);
    pl.off_stats = off;
    off = align256(off + (size_t)B * (K + 1) * pl.nchunk * 16);
    pl.off_rowx = off;
    off = align256(off + (size_t)B * K * 8);
    pl.off_mass = off;
    off = align256(off + (size_t)B * ceil_div(V, kSampleSub) * 2 * 8);
    pl.off_cut = off;
    off = align256(off + (size_t)B * (K + 1) * kRowCutBytes);
    pl.off_part = off;  // top-p: partial coarse histograms per chunk
    off = align256(off + (size_t)B * (K + 1) * pl.nchunk * kCutCoarse * 8);
    pl.off_ent = off;  // typical acceptance: entropy sums per chunk
    off = align256(off + (size_t)B * (K + 1) * pl.nchunk * 8);
    pl.off_gate = off;  // early exit: one flag per sequence
    off = align256(off + (size_t)B * 4);
    pl.total = off;
    return pl;
}

}  // namespace sv

namespace {

int check_attn_shape(int B, int T, int Hq, int Hkv, int d, int max_blocks)
{
    if (B < 1 || T < 1 || Hq < 1 || Hkv < 1 || max_blocks < 1)
        return fail(SV_ERR_SHAPE, "B, T, Hq, Hkv and max_blocks_per_seq must be >= 1 (got %d, %d, %d, %d, %d)",
                    B, T, Hq, Hkv, max_blocks);
    if (T > 16)
        return fail(SV_ERR_SHAPE, "T = K+1 must be <= 16 (got %d)", T);
    if (Hq % Hkv)
        return fail(SV_ERR_SHAPE, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
    if (T * (Hq / Hkv) > sv::kMaxRows)
        return fail(SV_ERR_UNSUPPORTED, "T*(Hq/Hkv) = %d exceeds %d", T * (Hq / Hkv), sv::kMaxRows);
    if (d != 64 && d != 128)
        return fail(SV_ERR_UNSUPPORTED, "head dim d must be 64 or 128 (got %d)", d);
    if ((long long)max_blocks * sv::kBlock > 0x7FFFFFFFLL)
        return fail(SV_ERR_SHAPE, "max_blocks_per_seq too large");
    return SV_OK;
}

}  // namespace

extern "C" {

int sv_abi_version(void) { return SV_ABI_VERSION; }

const char *sv_status_string(int status)
{
    switch (status) {
    case SV_OK: return "ok";
    case SV_ERR_NULL: return "null pointer";
    case SV_ERR_SHAPE: return "bad shape";
    case SV_ERR_UNSUPPORTED: return "unsupported";
    case SV_ERR_WORKSPACE: return "workspace too small";
    case SV_ERR_ALIGN: return "misaligned pointer";
    case SV_ERR_HIP: return "HIP error";
    default: return "unknown status";
    }
}

const char *sv_last_error(void) { return g_err; }

int spec_verify_workspace_clear(void *workspace, size_t bytes, void *stream)
{
    if (bytes == 0)
        return ok();
    if (!workspace)
        return fail(SV_ERR_NULL, "workspace is NULL");
    const hipError_t e = sv::launch_clear(workspace, bytes, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return fail(SV_ERR_HIP, "workspace clear: %s", hipGetErrorString(e));
    return ok();
}

size_t spec_verify_attn_workspace_size_ex(int B, int T, int Hq, int Hkv, int d, int max_blocks_per_seq,
                                          int blocks_per_split)
{
    if (check_attn_shape(B, T, Hq, Hkv, d, max_blocks_per_seq) != SV_OK)
        return 0;
    if (ceil_div(max_blocks_per_seq, sv::kMaxBps) > sv::kMaxSplits)
        return 0;
    if (blocks_per_split == sv::kSplitBalanced) {
        const sv::AttnPlan pl = sv::plan_attention(B, T, Hq, Hkv, d, max_blocks_per_seq, blocks_per_split);
        return pl.balanced ? pl.total : 0;
    }
    if (blocks_per_split < 0 || (blocks_per_split > 0 && blocks_per_split % 4) || blocks_per_split > sv::kMaxBps)
        return 0;
    if (blocks_per_split > 0 && ceil_div(max_blocks_per_seq, blocks_per_split) > sv::kMaxSplits)
        return 0;
    if (ceil_div(max_blocks_per_seq, sv::kMaxBps) > sv::kMaxSplits)
        return 0;
    return sv::plan_attention(B, T, Hq, Hkv, d, max_blocks_per_seq, blocks_per_split).total;
}

size_t spec_verify_attn_workspace_size(int B, int T, int Hq, int Hkv, int d, int max_blocks_per_seq)
{
    return spec_verify_attn_workspace_size_ex(B, T, Hq, Hkv, d, max_blocks_per_seq, 0);
}

namespace {

int attn_impl(const float *q, const void *k_cache, const void *v_cache, const float *k_scale, const float *v_scale,
              const int32_t *block_table, const int32_t *context_lens, const uint32_t *tree_mask, float *out, int B,
              int T, int Hq, int Hkv, int d, int block_size, int max_blocks_per_seq, int num_blocks, int kv_dtype,
              float sm_scale, void *workspace, size_t workspace_bytes, void *stream, int algo, int blocks_per_split,
              void *main_done_event, bool main_only)
{
    if (!q || !k_cache || !v_cache || !block_table || !context_lens || !out)
        return fail(SV_ERR_NULL, "q, k_cache, v_cache, block_table, context_lens and out must be non-NULL");
    int st = check_attn_shape(B, T, Hq, Hkv, d, max_blocks_per_seq);
    if (st != SV_OK)
        return st;
    if (block_size != sv::kBlock)
        return fail(SV_ERR_UNSUPPORTED, "block_size must be 16 (got %d)", block_size);
    if (num_blocks < 1)
        return fail(SV_ERR_SHAPE, "num_blocks must be >= 1 (got %d)", num_blocks);
    if (kv_dtype != SV_KV_F32 && kv_dtype != SV_KV_BF16 && kv_dtype != SV_KV_FP8_E4M3)
        return fail(SV_ERR_UNSUPPORTED, "unknown kv_dtype %d", kv_dtype);
    const bool fp8 = kv_dtype == SV_KV_FP8_E4M3;
    if (fp8 && (!k_scale || !v_scale))
        return fail(SV_ERR_NULL, "k_scale and v_scale are required for E4M3 storage");
    if (!fp8 && (k_scale || v_scale))
        return fail(SV_ERR_SHAPE, "k_scale / v_scale must be NULL unless kv_dtype is E4M3");
    if (!(std::isfinite(sm_scale)) || sm_scale <= 0.0f)
        return fail(SV_ERR_SHAPE, "sm_scale must be finite and positive");
    if (algo != SV_ATTN_AUTO && algo != SV_ATTN_VALU && algo != SV_ATTN_MFMA)
        return fail(SV_ERR_UNSUPPORTED, "unknown algo %d", algo);
    if (algo == SV_ATTN_MFMA && kv_dtype == SV_KV_F32)
        return fail(SV_ERR_UNSUPPORTED, "the matrix-core kernel needs bf16 or E4M3 storage");
    const bool use_mfma = (algo == SV_ATTN_MFMA) || (algo == SV_ATTN_AUTO && kv_dtype != SV_KV_F32);
    if (blocks_per_split == sv::kSplitBalanced) {
        if (!use_mfma)
            return fail(SV_ERR_UNSUPPORTED, "balanced shares (blocks_per_split = -1) need the matrix-core kernel");
        if (B > sv::kBalMaxB || (long long)B * Hkv * max_blocks_per_seq > sv::kBalMaxPages)
            return fail(SV_ERR_UNSUPPORTED, "balanced shares need B <= %d and B*Hkv*max_blocks_per_seq <= 2^30",
                        sv::kBalMaxB);
    } else if (blocks_per_split < 0 || (blocks_per_split > 0 && blocks_per_split % 4)) {
        return fail(SV_ERR_SHAPE, "blocks_per_split must be -1, 0 or a positive multiple of 4 (got %d)",
                    blocks_per_split);
    }
    if (blocks_per_split > sv::kMaxBps)
        return fail(SV_ERR_SHAPE, "blocks_per_split must be <= %d (got %d)", sv::kMaxBps, blocks_per_split);
    if (blocks_per_split > 0 && ceil_div(max_blocks_per_seq, blocks_per_split) > sv::kMaxSplits)
        return fail(SV_ERR_SHAPE, "blocks_per_split %d gives more than %d splits", blocks_per_split, sv::kMaxSplits);
    if (ceil_div(max_blocks_per_seq, sv::kMaxBps) > sv::kMaxSplits)
        return fail(SV_ERR_UNSUPPORTED, "max_blocks_per_seq %d exceeds %d pages", max_blocks_per_seq,
                    sv::kMaxBps * sv::kMaxSplits);
    if (!aligned(q, 16) || !aligned(out, 16))
        return fail(SV_ERR_ALIGN, "q and out must be 16-byte aligned");
    if (!aligned(k_cache, fp8 ? 8 : 16) || !aligned(v_cache, fp8 ? 8 : 16))
        return fail(SV_ERR_ALIGN, "k_cache and v_cache must be %d-byte aligned", fp8 ? 8 : 16);
    if (!aligned(block_table, 4) || !aligned(context_lens, 4) || (tree_mask && !aligned(tree_mask, 4)))
        return fail(SV_ERR_ALIGN, "block_table, context_lens and tree_mask must be 4-byte aligned");

    const sv::AttnPlan pl = sv::plan_attention(B, T, Hq, Hkv, d, max_blocks_per_seq, blocks_per_split);
    if (!workspace)
        return fail(SV_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", pl.total);
    if (!aligned(workspace, 256))
        return fail(SV_ERR_ALIGN, "workspace must be 256-byte aligned");
    if (workspace_bytes < pl.total)
        return fail(SV_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, pl.total);

    sv::AttnParams p{};
    unsigned char *ws = static_cast<unsigned char *>(workspace);
    p.q = q;
    p.k_cache = k_cache;
    p.v_cache = v_cache;
    p.k_scale = k_scale;
    p.v_scale = v_scale;
    p.block_table = block_table;
    p.context_lens = context_lens;
    p.tree_mask = tree_mask;
    p.out = out;
    p.balanced = (pl.balanced && use_mfma) ? 1 : 0;
    // the share rule follows the kernel's workgroup shape (8 waves: one share per compute unit)
    p.bal_one = (p.balanced && sv::attn_waves(d, (T * (Hq / Hkv) + 15) / 16, fp8, true) == 8) ? 1 : 0;
    p.bal_hg = p.bal_one ? sv::bal_group_heads(T, Hq, Hkv, d) : 1;
    p.part_o = reinterpret_cast<float *>(ws + (p.balanced ? pl.off_bal_o : pl.off_part_o));
    p.part_ml = reinterpret_cast<float *>(ws + (p.balanced ? pl.off_bal_ml : pl.off_part_ml));
    p.bal_prefix = p.balanced ? reinterpret_cast<int *>(ws + pl.off_prefix) : nullptr;
    p.B = B;
    p.T = T;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.G = Hq / Hkv;
    p.TG = T * p.G;
    p.d = d;
    p.max_blocks = max_blocks_per_seq;
    p.num_blocks = num_blocks;
    p.bps = pl.bps;
    p.max_splits = pl.max_splits;
    // fixed splits: 8 * ceil(units / 8) * max_splits workgroups (see
    // work_item in attn.hip); balanced shares: the most shares the rule can
    // make from at most (B * Hkv / bal_hg) * max_blocks pairs (one per
    // compute unit: shares of up to kBalMaxShareOne pages; else the plan's
    // grid, which also sizes the workspace)
    const long long pairs = (long long)B * (Hkv / p.bal_hg) * max_blocks_per_seq;
    const long long wgs = !p.balanced  ? ((long long)B * Hkv + 7) / 8 * 8 * pl.max_splits
                          : p.bal_one ? std::max<long long>(sv::kBalTargetWgs,
                                                             (pairs + sv::kBalMaxShareOne - 1) / sv::kBalMaxShareOne)
                                      : (long long)pl.grid_bal;
    if (wgs > 0x7FFFFFF0LL)
        return fail(SV_ERR_SHAPE, "too many workgroups");
    p.grid = (int)wgs;
    p.qscale = (float)((double)sm_scale * 1.4426950408889634);

    const hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = use_mfma ? sv::launch_attn_mfma(p, kv_dtype, s) : sv::launch_attn_valu(p, kv_dtype, s);
    if (e != hipSuccess)
        return fail(SV_ERR_HIP, "attention launch: %s", hipGetErrorString(e));
    if (main_done_event) {
        e = hipEventRecord(static_cast<hipEvent_t>(main_done_event), s);
        if (e != hipSuccess)
            return fail(SV_ERR_HIP, "recording main_done_event: %s", hipGetErrorString(e));
    }
    if (main_only)
        return ok();
    e = sv::launch_attn_merge(p, s);
    if (e != hipSuccess)
        return fail(SV_ERR_HIP, "split-merge launch: %s", hipGetErrorString(e));
    return ok();
}

}  // namespace

int spec_verify_attn_ex(const float *q, const void *k_cache, const void *v_cache, const float *k_scale,
                        const float *v_scale, const int32_t *block_table, const int32_t *context_lens,
                        float *out, int B, int T, int Hq, int Hkv, int d, int block_size,
                        int max_blocks_per_seq, int num_blocks, int kv_dtype, float sm_scale, void *workspace,
                        size_t workspace_bytes, void *stream, int algo, int blocks_per_split,
                        void *main_done_event)
{
    return attn_impl(q, k_cache, v_cache, k_scale, v_scale, block_table, context_lens, nullptr, out, B, T, Hq, Hkv,
                     d, block_size, max_blocks_per_seq, num_blocks, kv_dtype, sm_scale, workspace, workspace_bytes,
                     stream, algo, blocks_per_split, main_done_event, false);
}

size_t spec_verify_attn_noalloc_max_bytes(void) { return kNoAllocScratchBytes; }

int spec_verify_attn_noalloc(const float *q, const void *k_cache, const void *v_cache, const float *k_scale,
                             const float *v_scale, const int32_t *block_table, const int32_t *context_lens,
                             float *out, int B, int T, int Hq, int Hkv, int d, int block_size,
                             int max_blocks_per_seq, int num_blocks, int kv_dtype, float sm_scale, void *stream)
{
    // the plan of spec_verify_attn (the planner's split), so results agree bit for bit
    const size_t need = spec_verify_attn_workspace_size(B, T, Hq, Hkv, d, max_blocks_per_seq);
    if (need > kNoAllocScratchBytes)
        return fail(SV_ERR_UNSUPPORTED, "this shape needs %zu bytes of scratch; the static scratch holds %zu "
                                        "(use spec_verify_attn with a workspace)", need, kNoAllocScratchBytes);
    void *ws = nullptr;
    const int st = noalloc_scratch(static_cast<hipStream_t>(stream), &ws);
    if (st != SV_OK)
        return st;
    // need == 0 (a shape the planner rejects) falls through to attn_impl's own
    // validation, which names the problem
    return attn_impl(q, k_cache, v_cache, k_scale, v_scale, block_table, context_lens, nullptr, out, B, T, Hq, Hkv,
                     d, block_size, max_blocks_per_seq, num_blocks, kv_dtype, sm_scale, ws, kNoAllocScratchBytes,
                     stream, SV_ATTN_AUTO, 0, nullptr, false);
}

size_t spec_verify_probe_read_sink_floats(void) { return (size_t)sv::kProbeWgs * sv::kProbeThreads; }

int spec_verify_probe_read(const void *src, size_t bytes, float *sink, size_t sink_floats, void *stream)
{
    if (!src || !sink)
        return fail(SV_ERR_NULL, "src and sink must be non-NULL");
    if (bytes == 0 || bytes % 16)
        return fail(SV_ERR_SHAPE, "bytes must be a positive multiple of 16 (got %zu)", bytes);
    if (sink_floats < spec_verify_probe_read_sink_floats())
        return fail(SV_ERR_SHAPE, "sink holds %zu floats, needs %zu", sink_floats,
                    spec_verify_probe_read_sink_floats());
    if (!aligned(src, 16) || !aligned(sink, 4))
        return fail(SV_ERR_ALIGN, "src must be 16-byte and sink 4-byte aligned");
    const hipError_t e = sv::launch_probe_read(src, bytes, sink, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return fail(SV_ERR_HIP, "read probe launch: %s", hipGetErrorString(e));
    return ok();
}

int spec_verify_attn_timing_main_only(const float *q, const void *k_cache, const void *v_cache,
                                      const float *k_scale, const float *v_scale, const int32_t *block_table,
                                      const int32_t *context_lens, float *out, int B, int T, int Hq, int Hkv,
                                      int d, int block_size, int max_blocks_per_seq, int num_blocks, int kv_dtype,
                                      float sm_scale, void *workspace, size_t workspace_bytes, void *stream,
                                      int algo, int blocks_per_split)
{
    return attn_impl(q, k_cache, v_cache, k_scale, v_scale, block_table, context_lens, nullptr, out, B, T, Hq, Hkv,
                     d, block_size, max_blocks_per_seq, num_blocks, kv_dtype, sm_scale, workspace, workspace_bytes,
                     stream, algo, blocks_per_split, nullptr, true);
}

int spec_verify_attn_tree(const float *q, const void *k_cache, const void *v_cache, const float *k_scale,
                          const float *v_scale, const int32_t *block_table, const int32_t *context_lens,
                          const uint32_t *tree_mask, float *out, int B, int T, int Hq, int Hkv, int d,
                          int block_size, int max_blocks_per_seq, int num_blocks, int kv_dtype, float sm_scale,
                          void *workspace, size_t workspace_bytes, void *stream, int algo, int blocks_per_split)
{
    if (!tree_mask)
        return fail(SV_ERR_NULL, "tree_mask must be non-NULL (spec_verify_attn is the chain)");
    return attn_impl(q, k_cache, v_cache, k_scale, v_scale, block_table, context_lens, tree_mask, out, B, T, Hq,
                     Hkv, d, block_size, max_blocks_per_seq, num_blocks, kv_dtype, sm_scale, workspace,
                     workspace_bytes, stream, algo, blocks_per_split, nullptr, false);
}

int spec_verify_attn(const float *q, const void *k_cache, const void *v_cache, const float *k_scale,
                     const float *v_scale, const int32_t *block_table, const int32_t *context_lens, float *out,
                     int B, int T, int Hq, int Hkv, int d, int block_size, int max_blocks_per_seq, int num_blocks,
                     int kv_dtype, float sm_scale, void *workspace, size_t workspace_bytes, void *stream)
{
    return spec_verify_attn_ex(q, k_cache, v_cache, k_scale, v_scale, block_table, context_lens, out, B, T, Hq,
                               Hkv, d, block_size, max_blocks_per_seq, num_blocks, kv_dtype, sm_scale, workspace,
                               workspace_bytes, stream, SV_ATTN_AUTO, 0, nullptr);
}

size_t spec_verify_sample_workspace_size(int B, int K, int V)
{
    if (B < 1 || K < 1 || K > 15 || V < 1 || V > sv::kMaxSampleChunks * sv::kSampleChunk)
        return 0;
    return sv::plan_sample(B, K, V).total;
}

int spec_verify_sample(const float *target_logits, const float *draft_probs, const int32_t *draft_tokens,
                       const float *uniforms, int32_t *num_accepted, int32_t *out_tokens, float *accept_prob, int B,
                       int K, int V, void *workspace, size_t workspace_bytes, void *stream)
{
    return spec_verify_sample_ex(target_logits, draft_probs, draft_tokens, uniforms, nullptr, nullptr,
                                 num_accepted, out_tokens, accept_prob, B, K, V, workspace, workspace_bytes, stream);
}

namespace {

// The chain sampler behind spec_verify_sample_ex and spec_verify_sample_typical.
int sample_impl(const float *target_logits, const float *draft_probs, const int32_t *draft_tokens,
                const float *uniforms, const float *temperature, const float *top_p, bool typical, double eps,
                double delta, int32_t *num_accepted, int32_t *out_tokens, float *accept_prob, float *threshold,
                int B, int K, int V, void *workspace, size_t workspace_bytes, void *stream)
{
    if (B < 1 || K < 1 || V < 1)
        return fail(SV_ERR_SHAPE, "B, K and V must be >= 1 (got %d, %d, %d)", B, K, V);
    if (K > 15)
        return fail(SV_ERR_SHAPE, "K must be <= 15 (got %d)", K);
    if (V > sv::kMaxSampleChunks * sv::kSampleChunk)
        return fail(SV_ERR_UNSUPPORTED, "V must be <= %d (got %d)", sv::kMaxSampleChunks * sv::kSampleChunk, V);
    if (top_p && V >= sv::kCutMaxV)
        return fail(SV_ERR_UNSUPPORTED, "top_p needs V < %d (got %d)", sv::kCutMaxV, V);
    if ((long long)B * (K + 1) * ((V + sv::kSampleChunk - 1) / sv::kSampleChunk) > 0x7FFFFFFFLL ||
        (long long)B * ((V + sv::kSampleSub - 1) / sv::kSampleSub) > 0x7FFFFFFFLL)
        return fail(SV_ERR_SHAPE, "B*(K+1)*ceil(V/%d) or B*ceil(V/%d) exceeds the grid limit", sv::kSampleChunk,
                    sv::kSampleSub);
    if (!aligned(target_logits, 4) || (draft_probs && !aligned(draft_probs, 4)) || !aligned(draft_tokens, 4) ||
        !aligned(uniforms, 4) || !aligned(num_accepted, 4) || !aligned(out_tokens, 4) ||
        (accept_prob && !aligned(accept_prob, 4)) || (threshold && !aligned(threshold, 4)) ||
        (temperature && !aligned(temperature, 4)) || (top_p && !aligned(top_p, 4)))
        return fail(SV_ERR_ALIGN, "sampler arrays must be 4-byte aligned");
    const sv::SamplePlan pl = sv::plan_sample(B, K, V);
    if (!workspace)
        return fail(SV_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", pl.total);
    if (!aligned(workspace, 256))
        return fail(SV_ERR_ALIGN, "workspace must be 256-byte aligned");
    if (workspace_bytes < pl.total)
        return fail(SV_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, pl.total);
    sv::SampleParams p{};
    unsigned char *ws = static_cast<unsigned char *>(workspace);
    p.logits = target_logits;
    p.probs = draft_probs;
    p.tokens = draft_tokens;
    p.uniforms = uniforms;
    p.temperature = temperature;
    p.top_p = top_p;
    p.qrows = K;
    p.tree = 0;
    p.typical = typical ? 1 : 0;
    p.ty_eps = eps;
    p.ty_delta = delta;
    p.row_ent = reinterpret_cast<double *>(ws + pl.off_ent);
    p.threshold_out = threshold;
    p.num_accepted = num_accepted;
    p.out_tokens = out_tokens;
    p.accept_prob = accept_prob;
    p.seq_state = ws + pl.off_state;
    p.row_stats = ws + pl.off_stats;
    p.row_x = ws + pl.off_rowx;
    p.sub_mass = reinterpret_cast<double *>(ws + pl.off_mass);
    p.row_cut = top_p ? ws + pl.off_cut : nullptr;
    p.cut_part = reinterpret_cast<unsigned long long *>(ws + pl.off_part);
    p.gate = reinterpret_cast<int32_t *>(ws + pl.off_gate);
    p.B = B;
    p.K = K;
    p.V = V;
    p.nchunk = pl.nchunk;
    p.vec4 = (V % 4 == 0) && aligned(target_logits, 16) && (!draft_probs || aligned(draft_probs, 16));
    const hipError_t e = sv::launch_sample(p, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return fail(SV_ERR_HIP, "sampler launch: %s", hipGetErrorString(e));
    return ok();
}

}  // namespace

int spec_verify_sample_ex(const float *target_logits, const float *draft_probs, const int32_t *draft_tokens,
                          const float *uniforms, const float *temperature, const float *top_p,
                          int32_t *num_accepted, int32_t *out_tokens, float *accept_prob, int B, int K, int V,
                          void *workspace, size_t workspace_bytes, void *stream)
{
    if (!target_logits || !draft_probs || !draft_tokens || !uniforms || !num_accepted || !out_tokens)
        return fail(SV_ERR_NULL, "target_logits, draft_probs, draft_tokens, uniforms, num_accepted and "
                                 "out_tokens must be non-NULL");
    return sample_impl(target_logits, draft_probs, draft_tokens, uniforms, temperature, top_p, false, 0.0, 0.0,
                       num_accepted, out_tokens, accept_prob, nullptr, B, K, V, workspace, workspace_bytes,
                       stream);
}

int spec_verify_sample_typical(const float *target_logits, const int32_t *draft_tokens, const float *uniforms,
                               const float *temperature, double eps, double delta, int32_t *num_accepted,
                               int32_t *out_tokens, float *p_draft, float *threshold, int B, int K, int V,
                               void *workspace, size_t workspace_bytes, void *stream)
{
    if (!target_logits || !draft_tokens || !uniforms || !num_accepted || !out_tokens)
        return fail(SV_ERR_NULL, "target_logits, draft_tokens, uniforms, num_accepted and out_tokens must be "
                                 "non-NULL");
    if (!std::isfinite(eps) || !std::isfinite(delta) || eps < 0.0 || delta < 0.0)
        return fail(SV_ERR_SHAPE, "eps and delta must be finite and >= 0");
    return sample_impl(target_logits, nullptr, draft_tokens, uniforms, temperature, nullptr, true, eps, delta,
                       num_accepted, out_tokens, p_draft, threshold, B, K, V, workspace, workspace_bytes, stream);
}

int spec_verify_kv_append(const float *k_new, const float *v_new, void *k_cache, void *v_cache,
                          const float *k_scale, const float *v_scale, const int32_t *block_table,
                          const int32_t *context_lens, int B, int T, int Hkv, int d, int block_size,
                          int max_blocks_per_seq, int num_blocks, int kv_dtype, void *stream)
{
    if (!k_new || !v_new || !k_cache || !v_cache || !block_table || !context_lens)
        return fail(SV_ERR_NULL, "k_new, v_new, k_cache, v_cache, block_table and context_lens must be non-NULL");
    if (B < 1 || T < 1 || T > 16 || Hkv < 1 || d < 4 || d % 4 != 0 || max_blocks_per_seq < 1 || num_blocks < 1)
        return fail(SV_ERR_SHAPE, "need B >= 1, 1 <= T <= 16, Hkv >= 1, d a positive multiple of 4, "
                                  "max_blocks_per_seq >= 1, num_blocks >= 1 (got %d, %d, %d, %d, %d, %d)",
                    B, T, Hkv, d, max_blocks_per_seq, num_blocks);
    if (block_size != sv::kBlock)
        return fail(SV_ERR_UNSUPPORTED, "block_size must be %d (got %d)", sv::kBlock, block_size);
    if (kv_dtype != SV_KV_F32 && kv_dtype != SV_KV_BF16 && kv_dtype != SV_KV_FP8_E4M3)
        return fail(SV_ERR_UNSUPPORTED, "unknown kv_dtype %d", kv_dtype);
    const bool fp8 = kv_dtype == SV_KV_FP8_E4M3;
    if (fp8 && (!k_scale || !v_scale))
        return fail(SV_ERR_NULL, "k_scale and v_scale are required for SV_KV_FP8_E4M3");
    if (!fp8 && (k_scale || v_scale))
        return fail(SV_ERR_SHAPE, "k_scale and v_scale must be NULL unless kv_dtype is SV_KV_FP8_E4M3");
    if ((long long)max_blocks_per_seq * sv::kBlock > 0x7FFFFFFFLL ||
        (long long)B * max_blocks_per_seq > 0x7FFFFFFFFFFFLL)
        return fail(SV_ERR_SHAPE, "max_blocks_per_seq too large");
    const size_t cache_align = kv_dtype == SV_KV_F32 ? 16 : (kv_dtype == SV_KV_BF16 ? 8 : 4);
    if (!aligned(k_new, 16) || !aligned(v_new, 16))
        return fail(SV_ERR_ALIGN, "k_new and v_new must be 16-byte aligned");
    if (!aligned(k_cache, cache_align) || !aligned(v_cache, cache_align))
        return fail(SV_ERR_ALIGN, "k_cache and v_cache must be %zu-byte aligned", cache_align);
    if (!aligned(block_table, 4) || !aligned(context_lens, 4) || (fp8 && (!aligned(k_scale, 4) || !aligned(v_scale, 4))))
        return fail(SV_ERR_ALIGN, "block_table, context_lens and the scales must be 4-byte aligned");
    const long long threads = (long long)B * T * Hkv * (d / 4);
    if ((threads + 255) / 256 > 0x7FFFFFFFLL)
        return fail(SV_ERR_SHAPE, "B*T*Hkv*d too large");
    sv::AppendParams p{};
    p.k_new = k_new;
    p.v_new = v_new;
    p.k_cache = k_cache;
    p.v_cache = v_cache;
    p.k_scale = k_scale;
    p.v_scale = v_scale;
    p.block_table = block_table;
    p.context_lens = context_lens;
    p.B = B;
    p.T = T;
    p.Hkv = Hkv;
    p.d = d;
    p.max_blocks = max_blocks_per_seq;
    p.num_blocks = num_blocks;
    const hipError_t e = sv::launch_kv_append(p, kv_dtype, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return fail(SV_ERR_HIP, "append launch: %s", hipGetErrorString(e));
    return ok();
}

int spec_verify_check_inputs(const int32_t *block_table, const int32_t *context_lens, int T, int max_blocks_per_seq,
                             int num_blocks, const int32_t *tokens, int n_tokens, int V, const float *uniforms,
                             int n_uniforms, int B, int32_t *counts, void *stream)
{
    static_assert(SV_CHECK_COUNTS == sv::kCheckCounts, "counter count of the header");
    if (!counts)
        return fail(SV_ERR_NULL, "counts must be non-NULL");
    if (B < 1)
        return fail(SV_ERR_SHAPE, "B must be >= 1 (got %d)", B);
    if (block_table && !context_lens)
        return fail(SV_ERR_NULL, "checking block_table needs context_lens (the visible pages)");
    if (context_lens && (T < 1 || max_blocks_per_seq < 1))
        return fail(SV_ERR_SHAPE, "need T >= 1 and max_blocks_per_seq >= 1 (got %d, %d)", T, max_blocks_per_seq);
    if (block_table && num_blocks < 1)
        return fail(SV_ERR_SHAPE, "num_blocks must be >= 1 (got %d)", num_blocks);
    if (tokens && (n_tokens < 0 || V < 1))
        return fail(SV_ERR_SHAPE, "need n_tokens >= 0 and V >= 1 (got %d, %d)", n_tokens, V);
    if (uniforms && n_uniforms < 0)
        return fail(SV_ERR_SHAPE, "n_uniforms must be >= 0 (got %d)", n_uniforms);
    if (!aligned(counts, 4) || (block_table && !aligned(block_table, 4)) || (context_lens && !aligned(context_lens, 4)) ||
        (tokens && !aligned(tokens, 4)) || (uniforms && !aligned(uniforms, 4)))
        return fail(SV_ERR_ALIGN, "arrays must be 4-byte aligned");
    sv::CheckParams p{};
    p.block_table = block_table;
    p.context_lens = context_lens;
    p.tokens = tokens;
    p.uniforms = uniforms;
    p.counts = counts;
    p.B = B;
    p.T = T;
    p.max_blocks = max_blocks_per_seq;
    p.num_blocks = num_blocks;
    p.n_tokens = tokens ? n_tokens : 0;
    p.V = V;
    p.n_uniforms = uniforms ? n_uniforms : 0;
    const hipError_t e = sv::launch_check_inputs(p, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return fail(SV_ERR_HIP, "input check launch: %s", hipGetErrorString(e));
    return ok();
}

int spec_verify_rollback(const int32_t *num_accepted, int32_t *context_lens, int32_t *pages_in_use, int B, int K,
                         void *stream)
{
    if (!num_accepted || !context_lens)
        return fail(SV_ERR_NULL, "num_accepted and context_lens must be non-NULL");
    if (B < 1 || K < 1 || K > 15)
        return fail(SV_ERR_SHAPE, "need B >= 1 and 1 <= K <= 15 (got %d, %d)", B, K);
    if (!aligned(num_accepted, 4) || !aligned(context_lens, 4) || (pages_in_use && !aligned(pages_in_use, 4)))
        return fail(SV_ERR_ALIGN, "rollback arrays must be 4-byte aligned");
    const hipError_t e = sv::launch_rollback(num_accepted, context_lens, pages_in_use, B, K,
                                             static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return fail(SV_ERR_HIP, "rollback launch: %s", hipGetErrorString(e));
    return ok();
}


size_t spec_verify_sample_tree_workspace_size(int B, int N, int V)
{
    if (B < 1 || N < 1 || N > 16 || V < 1 || V > sv::kMaxSampleChunks * sv::kSampleChunk)
        return 0;
    return sv::plan_sample_tree(B, N, V).total;
}

int spec_verify_sample_tree(const float *target_logits, const float *draft_probs, const int32_t *tokens,
                            const int32_t *parents, const float *uniforms, int32_t *num_accepted,
                            int32_t *out_tokens, int32_t *path, float *accept_prob, int B, int N, int V,
                            int max_children, void *workspace, size_t workspace_bytes, void *stream)
{
    if (!target_logits || !draft_probs || !tokens || !parents || !uniforms || !num_accepted || !out_tokens || !path)
        return fail(SV_ERR_NULL, "target_logits, draft_probs, tokens, parents, uniforms, num_accepted, out_tokens "
                                 "and path must be non-NULL");
    if (B < 1 || N < 1 || V < 1)
        return fail(SV_ERR_SHAPE, "B, N and V must be >= 1 (got %d, %d, %d)", B, N, V);
    if (N > 16)
        return fail(SV_ERR_SHAPE, "N must be <= 16 (got %d)", N);
    if (max_children < 0 || max_children > N - 1)
        return fail(SV_ERR_SHAPE, "max_children must be in [0, N-1] (got %d, N = %d)", max_children, N);
    if (V > sv::kMaxSampleChunks * sv::kSampleChunk)
        return fail(SV_ERR_UNSUPPORTED, "V must be <= %d (got %d)", sv::kMaxSampleChunks * sv::kSampleChunk, V);
    if ((long long)B * N * ((V + sv::kSampleChunk - 1) / sv::kSampleChunk) > 0x7FFFFFFFLL ||
        (long long)B * ((V + sv::kSampleSub - 1) / sv::kSampleSub) > 0x7FFFFFFFLL)
        return fail(SV_ERR_SHAPE, "B*N*ceil(V/%d) or B*ceil(V/%d) exceeds the grid limit", sv::kSampleChunk,
                    sv::kSampleSub);
    if (!aligned(target_logits, 4) || !aligned(draft_probs, 4) || !aligned(tokens, 4) || !aligned(parents, 4) ||
        !aligned(uniforms, 4) || !aligned(num_accepted, 4) || !aligned(out_tokens, 4) || !aligned(path, 4) ||
        (accept_prob && !aligned(accept_prob, 4)))
        return fail(SV_ERR_ALIGN, "tree sampler arrays must be 4-byte aligned");
    const sv::TreePlan pl = sv::plan_sample_tree(B, N, V);
    if (!workspace)
        return fail(SV_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", pl.total);
    if (!aligned(workspace, 256))
        return fail(SV_ERR_ALIGN, "workspace must be 256-byte aligned");
    if (workspace_bytes < pl.total)
        return fail(SV_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, pl.total);
    unsigned char *ws = static_cast<unsigned char *>(workspace);
    sv::SampleParams p{};
    p.logits = target_logits;
    p.probs = draft_probs;
    p.tokens = tokens;
    p.uniforms = uniforms;
    p.num_accepted = num_accepted;
    p.out_tokens = out_tokens;
    p.accept_prob = accept_prob;
    p.seq_state = ws + pl.off_state;
    p.row_stats = ws + pl.off_stats;
    p.sub_mass = reinterpret_cast<double *>(ws + pl.off_mass);
    p.coefs = reinterpret_cast<double *>(ws + pl.off_coefs);
    p.tree_c = reinterpret_cast<double *>(ws + pl.off_tree_c);
    p.parents = parents;
    p.path = path;
    p.B = B;
    p.K = N - 1;
    p.V = V;
    p.nchunk = pl.nchunk;
    p.qrows = N;
    p.tree = 1;
    p.tree_max_children = max_children;
    p.vec4 = (V % 4 == 0) && aligned(target_logits, 16) && aligned(draft_probs, 16);
    const hipError_t e = sv::launch_sample_tree(p, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return fail(SV_ERR_HIP, "tree sampler launch: %s", hipGetErrorString(e));
    return ok();
}

int spec_verify_tree_commit(const int32_t *path, const int32_t *num_accepted, void *k_cache, void *v_cache,
                            const float *k_scale, const float *v_scale, const int32_t *block_table,
                            int32_t *context_lens, int32_t *pages_in_use, int B, int N, int Hkv, int d,
                            int block_size, int max_blocks_per_seq, int num_blocks, int kv_dtype, void *stream)
{
    if (!path || !num_accepted || !k_cache || !v_cache || !block_table || !context_lens)
        return fail(SV_ERR_NULL, "path, num_accepted, k_cache, v_cache, block_table and context_lens must be "
                                 "non-NULL");
    if (B < 1 || N < 1 || N > 16 || Hkv < 1 || d < 4 || d % 4 != 0 || d > 256 || max_blocks_per_seq < 1 ||
        num_blocks < 1)
        return fail(SV_ERR_SHAPE, "need B >= 1, 1 <= N <= 16, Hkv >= 1, d a multiple of 4 in [4, 256], "
                                  "max_blocks_per_seq >= 1, num_blocks >= 1 (got %d, %d, %d, %d, %d, %d)",
                    B, N, Hkv, d, max_blocks_per_seq, num_blocks);
    if ((long long)B * Hkv > 0x7FFFFFFFLL || (long long)max_blocks_per_seq * sv::kBlock > 0x7FFFFFFFLL)
        return fail(SV_ERR_SHAPE, "B*Hkv or max_blocks_per_seq too large");
    if (block_size != sv::kBlock)
        return fail(SV_ERR_UNSUPPORTED, "block_size must be %d (got %d)", sv::kBlock, block_size);
    if (kv_dtype != SV_KV_F32 && kv_dtype != SV_KV_BF16 && kv_dtype != SV_KV_FP8_E4M3)
        return fail(SV_ERR_UNSUPPORTED, "unknown kv_dtype %d", kv_dtype);
    const bool fp8 = kv_dtype == SV_KV_FP8_E4M3;
    if (fp8 && (!k_scale || !v_scale))
        return fail(SV_ERR_NULL, "k_scale and v_scale are required for E4M3 storage");
    if (!fp8 && (k_scale || v_scale))
        return fail(SV_ERR_SHAPE, "k_scale / v_scale must be NULL unless kv_dtype is E4M3");
    const int align = kv_dtype == SV_KV_F32 ? 16 : (kv_dtype == SV_KV_BF16 ? 8 : 4);
    if (!aligned(k_cache, align) || !aligned(v_cache, align) || !aligned(path, 4) || !aligned(num_accepted, 4) ||
        !aligned(block_table, 4) || !aligned(context_lens, 4) || (pages_in_use && !aligned(pages_in_use, 4)) ||
        (k_scale && !aligned(k_scale, 4)) || (v_scale && !aligned(v_scale, 4)))
        return fail(SV_ERR_ALIGN, "k_cache / v_cache must be %d-byte aligned, the int and scale arrays 4-byte",
                    align);
    sv::TreeCommitParams p{};
    p.path = path;
    p.num_accepted = num_accepted;
    p.k_cache = k_cache;
    p.v_cache = v_cache;
    p.k_scale = k_scale;
    p.v_scale = v_scale;
    p.block_table = block_table;
    p.context_lens = context_lens;
    p.pages_in_use = pages_in_use;
    p.B = B;
    p.N = N;
    p.Hkv = Hkv;
    p.d = d;
    p.max_blocks = max_blocks_per_seq;
    p.num_blocks = num_blocks;
    const hipError_t e = sv::launch_tree_commit(p, kv_dtype, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return fail(SV_ERR_HIP, "tree commit launch: %s", hipGetErrorString(e));
    return ok();
}

}  // extern "C"
