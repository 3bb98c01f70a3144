// attn.hip -- paged GQA verify attention for gfx950.
//
// What is computed ("KV Cache + Speculative Decoding" 5.2-5.3, 6.1, 6.3;
// "Lecture 10 - Inference" 9.2): for sequence b, verify row t and query head
// h, softmax(sm_scale * q . k_p) over the positions p <= L_b - T + t, applied
// to v_p, where K/V of position p live in block block_table[b][p/16], slot
// p%16, KV head h / (Hq/Hkv).
//
// Work decomposition (one design for the whole family of shapes):
//   * a workgroup owns one (sequence b, KV head g) unit and one contiguous
//     split of its context pages; all T*G query rows of the unit share every
//     K/V byte it loads, so each cached byte is fetched once per step;
//   * the four waves of a workgroup take interleaved 16-token pages of the
//     split and keep independent online-softmax states, merged through LDS
//     at the end of the split;
//   * when a unit has several splits, each workgroup writes an unnormalised
//     partial (o, running max, running sum) and a second, small kernel
//     merges them (flash-decoding style).  Kernel order on the stream makes
//     the partials visible; no device-wide fence is used (on this multi-die
//     part such a fence writes back the L2 and costs far more than a launch).
//
// Matrix-core kernel (bf16 / E4M3 storage), per wave and page:
//   * the page's K and V slices (16 slots x d) stream HBM -> LDS with direct
//     buffer-to-LDS copies into a small ring (about 8 KB in flight behind
//     the page being computed), so no registers hold data in flight;
//   * S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (keys on M, query rows on N);
//     K moves as whole slot rows and each lane reads its operand from an
//     XOR-swizzled position (conflict-free), Q sits in registers as bf16;
//   * each lane reads four keys' worth of V head dims and builds the PV A
//     operand with byte permutes (no transpose through LDS);
//   * S^T leaves each lane holding one query row's P for four keys, which is
//     exactly the B operand of v_mfma_f32_16x16x16_bf16 for O^T += V^T P^T,
//     so P needs no cross-lane shuffle; bf16 row sums come from the same
//     instruction with an all-ones A operand.
// Scores are kept in base-2 units (q pre-scaled by sm_scale*log2 e) and
// exponentiated with v_exp_f32; the running maximum only moves (with a
// rescale of the accumulators) when a score exceeds it by more than 8.
//
// Vector-ALU kernel: the same decomposition one page at a time through LDS,
// with fp32 arithmetic throughout.  It serves fp32 storage and is the
// baseline the matrix-core kernel is measured against.
#include "sv_device.hpp"
#include "sv_internal.hpp"

namespace sv {
namespace {

constexpr float kSlack = 8.0f;  // base-2 headroom before the running max is moved

// Clamped context length and its page count (the same everywhere a unit's pages
// are counted).
__device__ __forceinline__ int clamp_len(const AttnParams &p, int Lraw)
{
    return Lraw < 0 ? 0 : (Lraw > p.max_blocks * kBlock ? p.max_blocks * kBlock : Lraw);
}

// Pages per balanced share for `total` (unit, page) pairs.  Share j (the
// block index) is pairs [j*S, (j+1)*S) of the batch's list (units in order
// b * Hkv + g, pages in order within a unit); a unit cut by several shares
// leaves partials in slots unit + j, consecutive in j.  With head groups
// (bal_heads) the list holds (group, page) pairs, groups in order
// b * (Hkv / hg) + g / hg, and head g's partials go to slots
// (group + j) * hg + g % hg.  Shares go to the dies round robin with the
// block index.  (Giving each die the units of its
// own KV heads measured 9% slower on a ragged batch, 3% faster on one long
// sequence.)
// one_per_cu: the kernel's 8-wave workgroups fill a compute unit each.
__device__ __forceinline__ int bal_share(int total, bool one_per_cu)
{
    const int s1 = (total + kBalTargetWgs - 1) / kBalTargetWgs;
    if (one_per_cu)
        return s1 < 4 ? 4 : (s1 > kBalMaxShareOne ? kBalMaxShareOne : s1);
    if (s1 <= kBalOneShare)
        return s1 < 4 ? 4 : s1;
    const int s2 = (total + 2 * kBalTargetWgs - 1) / (2 * kBalTargetWgs);
    return s2 > kBalMaxShare ? kBalMaxShare : s2;
}

struct UnitWork {
    int b, g, unit, split;
    int L;          // clamped context length
    int blk_begin;  // first logical block of the split
    int blk_end;    // one past the last
    int nsplit;     // splits of this sequence
};

// Workgroup -> (unit, split).  Workgroups are handed to the eight dies
// (XCDs) round robin, block id mod 8.  Die x takes units x, x+8, x+16, ...
// with all their splits: with 8 KV heads that is head x of every sequence, so
// each die gets the same share of work however ragged the context lengths
// are (a die cannot take over another die's work).  The grid holds
// 8 * ceil(units / 8) * max_splits workgroups.
__device__ __forceinline__ void work_item(const AttnParams &p, int &unit, int &split)
{
    const int x = blockIdx.x & 7, j = blockIdx.x >> 3;
    unit = (j / p.max_splits) * 8 + x;
    split = j - (j / p.max_splits) * p.max_splits;
}

__device__ __forceinline__ bool decode_work(const AttnParams &p, UnitWork &w)
{
    int unit, split;
    work_item(p, unit, split);
    if (unit >= p.B * p.Hkv)
        return false;
    w.unit = unit;
    w.split = split;
    w.b = unit / p.Hkv;
    w.g = unit - w.b * p.Hkv;
    int L = p.context_lens[w.b];
    L = L < 0 ? 0 : (L > p.max_blocks * kBlock ? p.max_blocks * kBlock : L);
    w.L = L;
    const int nblk = (L + kBlock - 1) / kBlock;
    w.blk_begin = w.split * p.bps;
    if (w.blk_begin >= nblk)
        return false;
    w.blk_end = min(w.blk_begin + p.bps, nblk);
    w.nsplit = (nblk + p.bps - 1) / p.bps;
    return true;
}

__device__ __forceinline__ int clamp_block(int v, int n) { return v < 0 ? 0 : (v >= n ? n - 1 : v); }

// Normalises and stores the workgroup's result when its unit has a single
// split, or publishes it as an unnormalised partial (o, running max, running
// sum) for the merge kernel.  obuf: [TG][D+4] unnormalised output in LDS;
// mrow/lrow: per-row max (base-2 units) and sum in LDS.  Called by all
// threads.  No fence or atomic is needed: the merge runs as the next kernel
// on the same stream.
template <int D>
__device__ void finish_unit(const AttnParams &p, const UnitWork &w, const float *obuf, const float *mrow,
                            const float *lrow)
{
    constexpr int OP = D + 4;
    constexpr int C4 = D / 4;
    const int tid = threadIdx.x;
    const int TG = p.TG, G = p.G;
    if (w.nsplit == 1) {
        for (int idx = tid; idx < TG * C4; idx += kAttnThreads) {
            const int row = idx / C4, c4 = idx - row * C4;
            const float inv = 1.0f / lrow[row];
            float4 o = *reinterpret_cast<const float4 *>(obuf + row * OP + c4 * 4);
            o.x *= inv; o.y *= inv; o.z *= inv; o.w *= inv;
            const int t = row / G, hh = row - t * G;
            float *dst = p.out + (((size_t)w.b * p.T + t) * p.Hq + (size_t)w.g * G + hh) * D + c4 * 4;
            *reinterpret_cast<float4 *>(dst) = o;
        }
        return;
    }
    const size_t base = ((size_t)w.unit * p.max_splits + w.split) * TG;
    for (int idx = tid; idx < TG * C4; idx += kAttnThreads) {
        const int row = idx / C4, c4 = idx - row * C4;
        *reinterpret_cast<float4 *>(p.part_o + (base + row) * D + c4 * 4) =
            *reinterpret_cast<const float4 *>(obuf + row * OP + c4 * 4);
    }
    for (int row = tid; row < TG; row += kAttnThreads)
        reinterpret_cast<float2 *>(p.part_ml)[base + row] = make_float2(mrow[row], lrow[row]);
}

// Split merge (flash-decoding second pass): one wave per R consecutive rows
// of one unit (R = 1 unless the grid would exceed one resident round).
//   M = max_s m_s,  L = sum_s l_s 2^(m_s - M),  out = sum_s o_s 2^(m_s - M) / L.
// Lanes hold one split's statistics each (reduced with DPP) and slices of
// the head dim.  Fixed splits: the context length, the statistics and the
// partial rows of the first NB splits are requested together (all lie
// inside the workspace), so the common case costs one round trip to memory;
// entries of splits past the context are discarded.  Balanced shares: the
// unit's first slot and its number of partials come from the prefix sums the
// attention kernel left in the workspace, then the same loads follow (for
// all R rows at once).
// NB: splits whose partial rows are requested at once (16 or 32 for many
// fixed splits, where the grid has few waves: c5b's 32 splits 10.1 us with
// 8, 9.0 with 16; 4 under balanced shares, 8 otherwise: the fewer
// registers keep more waves resident, balanced shares at B = 64 12.0 us
// with 8 against 15.6 with 16).
template <int D, int NB, int R>
__global__ __launch_bounds__(256) void sv_attn_merge_kernel(AttnParams p)
{
    constexpr int PER = D / 64;  // floats per lane
    const int gw = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int units = p.B * p.Hkv;
    const int TG = p.TG;
    const int ngrp = (TG + R - 1) / R;  // groups of R consecutive rows per unit, one wave each
    if (gw >= units * ngrp)
        return;
    const int unit = gw / ngrp, row0 = (gw - unit * ngrp) * R;
    const int b = unit / p.Hkv, g = unit - b * p.Hkv;
    const float ninf = -__builtin_inff();
    size_t slot0, sst = 1;  // first slot, slots between consecutive partials
    int cnt, ns = 0;  // partials that may be read; partials of the unit
    int Lraw = 0;
    if (p.balanced) {
        // head groups: group b * (Hkv / hg) + g / hg, partials in slots
        // (group + share) * hg + g % hg
        const int hg = p.bal_hg, ngr = p.Hkv / hg, gi = g / hg;
        const int nblk = (clamp_len(p, p.context_lens[b]) + kBlock - 1) / kBlock;
        const int S = bal_share(ngr * p.bal_prefix[p.B], p.bal_one != 0);
        const int start = ngr * p.bal_prefix[b] + gi * nblk;
        ns = nblk > 0 ? (start + nblk - 1) / S - start / S + 1 : 0;
        if (ns <= 1)
            return;  // written directly by the attention kernel (or no context)
        slot0 = ((size_t)b * ngr + gi + start / S) * hg + (g - gi * hg);
        sst = (size_t)hg;
        cnt = ns;
    } else {
        slot0 = (size_t)unit * p.max_splits;
        cnt = p.max_splits;
        Lraw = p.context_lens[b];
    }
    const size_t sstride = sst * TG * D;  // floats between consecutive partials' rows
    const size_t mstride = sst * TG;      // (max, sum) pairs between them
    // every row's statistics and first NB partial rows, requested together
    float2 st0[R];
    float o[R][NB][PER];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int row = row0 + r;
        const bool valid = row < TG;
        const float2 *ml = reinterpret_cast<const float2 *>(p.part_ml) + slot0 * TG + row;
        const float *po = p.part_o + (slot0 * TG + row) * D + lane * PER;
        st0[r] = (valid && lane < cnt) ? ml[(size_t)lane * mstride] : make_float2(ninf, 0.0f);
#pragma unroll
        for (int j = 0; j < NB; ++j) {
#pragma unroll
            for (int k = 0; k < PER; ++k)
                o[r][j][k] = 0.0f;
            if (valid && j < cnt) {
                if constexpr (PER == 2) {
                    const float2 v = *reinterpret_cast<const float2 *>(po + j * sstride);
                    o[r][j][0] = v.x;
                    o[r][j][1] = v.y;
                } else {
                    o[r][j][0] = po[j * sstride];
                }
            }
        }
    }
    if (!p.balanced) {
        const int nblk = (clamp_len(p, Lraw) + kBlock - 1) / kBlock;
        ns = (nblk + p.bps - 1) / p.bps;
        if (ns <= 1)
            return;  // written directly by the attention kernel
    }

#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int row = row0 + r;
        if (row >= TG)
            break;  // uniform
        const float2 *ml = reinterpret_cast<const float2 *>(p.part_ml) + slot0 * TG + row;
        const float *po = p.part_o + (slot0 * TG + row) * D + lane * PER;
        float mloc = lane < ns ? st0[r].x : ninf;
        for (int s = lane + kWave; s < ns; s += kWave)
            mloc = fmaxf(mloc, ml[(size_t)s * mstride].x);
        const float M = wave_max_f32(mloc);
        double Lsum = 0.0;
        if (lane < ns && st0[r].x != ninf)
            Lsum = (double)(st0[r].y * __builtin_amdgcn_exp2f(st0[r].x - M));
        for (int s = lane + kWave; s < ns; s += kWave) {
            const float2 v = ml[(size_t)s * mstride];
            if (v.x != ninf)
                Lsum += (double)(v.y * __builtin_amdgcn_exp2f(v.x - M));
        }
        const float inv = (float)(1.0 / wave_sum_f64(Lsum));

        float acc[PER];
#pragma unroll
        for (int k = 0; k < PER; ++k)
            acc[k] = 0.0f;
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            if (j < ns) {  // uniform
                const float mj = readlane_f32(st0[r].x, j);
                const float f = (mj == ninf) ? 0.0f : __builtin_amdgcn_exp2f(mj - M);
#pragma unroll
                for (int k = 0; k < PER; ++k)
                    acc[k] += f * o[r][j][k];
            }
        }
        for (int s0 = NB; s0 < ns; s0 += NB) {
            float f[NB], ov[NB][PER];
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const int s = s0 + j;
                f[j] = 0.0f;
#pragma unroll
                for (int k = 0; k < PER; ++k)
                    ov[j][k] = 0.0f;
                if (s < ns) {
                    const float ms = ml[(size_t)s * mstride].x;
                    f[j] = (ms == ninf) ? 0.0f : __builtin_amdgcn_exp2f(ms - M);
                    if constexpr (PER == 2) {
                        const float2 v = *reinterpret_cast<const float2 *>(po + s * sstride);
                        ov[j][0] = v.x;
                        ov[j][1] = v.y;
                    } else {
                        ov[j][0] = po[s * sstride];
                    }
                }
            }
#pragma unroll
            for (int j = 0; j < NB; ++j)
#pragma unroll
                for (int k = 0; k < PER; ++k)
                    acc[k] += f[j] * ov[j][k];
        }
        const int t = row / p.G, hh = row - t * p.G;
        float *dst = p.out + (((size_t)b * p.T + t) * p.Hq + (size_t)g * p.G + hh) * D + lane * PER;
#pragma unroll
        for (int k = 0; k < PER; ++k)
            dst[k] = acc[k] * inv;
    }
}

// ---------------------------------------------------------------- MFMA kernel

typedef short short4v __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef int int4v __attribute__((ext_vector_type(4)));

// Buffer descriptor (V#) of one physical page of one tensor, as four SGPRs:
// base, stride 0, num_records = page bytes, raw 32-bit data format (gfx9
// family word 3).  Reads outside the page return zero.
__device__ __forceinline__ int4v page_desc(const unsigned char *base, int page, uint32_t page_bytes)
{
    const uint64_t a = reinterpret_cast<uint64_t>(base) + (uint64_t)page * page_bytes;
    int4v r;
    r.x = (int)(uint32_t)a;
    r.y = (int)((uint32_t)(a >> 32) & 0xFFFFu);
    r.z = (int)page_bytes;
    r.w = 0x00020000;
    return r;
}

// Direct HBM -> LDS copy (gfx950 buffer_load ... lds): every lane moves BYTES
// bytes from desc + voff + soff to LDS address lds + lane * BYTES (the LDS
// base travels in m0, which the "{m0}" operand hands to the compiler).
// Issued from inline assembly so that the kernel, not the compiler, decides
// how many copies stay in flight; completion is awaited with wait_dma<N>().
// lgkmcnt(0) first: the copy may overwrite LDS that this wave has only just
// finished reading.  s_nop 4: a vector-memory instruction that reads an SGPR
// written by a VALU instruction (v_readlane of a spilled SGPR, readfirstlane)
// needs five wait states in between, and the compiler's hazard check does not
// look inside inline assembly; without them the copy can take the SGPR's
// previous value as its offset or descriptor (seen: a spilled soffset reloaded
// one instruction before the copy, which then fetched the wrong key).
template <int BYTES>
__device__ __forceinline__ void dma_to_lds(uint32_t lds, int4v desc, int voff, int soff)
{
    if constexpr (BYTES == 16)
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_nop 4\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
                     :: "v"(voff), "s"(desc), "s"(soff), "{m0}"(lds) : "memory");
    else
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_nop 4\n\tbuffer_load_dword %0, %1, %2 offen lds"
                     :: "v"(voff), "s"(desc), "s"(soff), "{m0}"(lds) : "memory");
}

// Waits until at most N of this wave's memory loads are outstanding (they
// complete in issue order).
template <int N>
__device__ __forceinline__ void wait_dma() { asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory"); }

// All-ones if V slot `key` (absolute position) is part of the context,
// else zero: slots past the context may hold anything, NaN included, and
// are cleared with a mask (no branch) before they reach the PV product.
// Visibility of cache position pos to a verify row whose ancestor set is
// `anc`: the prefix (pos < L - T) always; verify position L - T + j (tree
// node j in BFS order) iff bit j of the set is set.  The chain's row t has
// the set {0 .. t}, i.e. the causal mask.
__device__ __forceinline__ bool key_visible(int pos, int L, int T, uint32_t anc)
{
    const int rel = pos - (L - T);
    return rel < 0 || (rel < T && ((anc >> rel) & 1u));
}

__device__ __forceinline__ uint32_t row_ancestors(const AttnParams &p, int b, int t)
{
    return p.tree_mask ? p.tree_mask[(size_t)b * p.T + t] : ((2u << t) - 1u);
}

__device__ __forceinline__ uint32_t slot_keep(bool tail, int key, int L)
{
    return (tail && key >= L) ? 0u : 0xFFFFFFFFu;
}

// Eight stored values -> four packed bf16 pairs.
__device__ __forceinline__ uint4 to_bf16x8(uint2 v)
{
    const uint2 lo = e4m3x4_to_bf16x4(v.x);
    const uint2 hi = e4m3x4_to_bf16x4(v.y);
    return make_uint4(lo.x, lo.y, hi.x, hi.y);
}

// Geometry of one 16-token page of one KV head as it travels HBM -> LDS.
// A wave reads back only bytes that its own copies wrote, once its vmcnt
// wait has passed (shared pages add a barrier: see MfmaShape).
//   K: each copy instruction moves whole 256-byte (bf16, d = 128) slot rows
//      of the slice, several slots per copy; whole rows stream faster from
//      HBM than the same bytes cut into 64-byte pieces of 16 rows.  Lane
//      l = (slot l%16, lane group q4 = l/16) then reads from LDS the A
//      operand of S^T = K Q^T for every 32-wide head-dim chunk dc (eight
//      dims): bf16: piece 4*dc + q4 of its slot; E4M3: one 16-byte piece
//      carries two chunks (sixteen dims), so the chunk -> dim map is permuted
//      the same way on the Q side.
//   V: lane l = (dim group m = l%16, key group q4 = l/16) carries, for each
//      of the keys 4*q4 .. 4*q4+3, the NDT = D/16 consecutive head dims
//      NDT*m .. NDT*m+NDT-1.  Row m of PV dim tile t is head dim NDT*m + t,
//      so the A operand of tile t (four keys of one dim) is gathered from the
//      lane's own registers with byte permutes: no transpose through LDS.
//      16 bytes per key and lane (bf16, d=128) travel in one 16-byte copy;
//      otherwise in 4-byte copies (the LDS copy has no 8-byte form).
//   E4M3 scales: the page's K and V scales follow as two 4-byte copies in
//      which every lane fetches the same word, so each lane reads its own
//      copy back.  (A plain load would make the compiler wait for every
//      copy in flight before the scale could be used.)
template <int D, bool FP8>
struct PageGeom {
    static constexpr int EB = FP8 ? 1 : 2;
    static constexpr int PT = 16 * D * EB;             // bytes of one tensor's page slice
    static constexpr int SCB = FP8 ? 2 * 256 : 0;      // scale copies (E4M3)
    static constexpr int STAGE = 2 * PT + SCB;          // K slice, V slice, scales
    static constexpr int NDC = D / 32;                 // MFMA chunks of the head dim (S)
    static constexpr int NKI = FP8 ? D / 64 : D / 32;  // 16-byte K copies per page
    static constexpr int NDT = D / 16;                 // PV dim tiles = dims per lane and key
    static constexpr int VKB = NDT * EB;               // V bytes per lane and key: 16, 8 or 4
    static constexpr int VBYTES = VKB >= 16 ? 16 : 4;  // V copy width
    static constexpr int VPK = VKB / VBYTES;           // V copies per key
    static constexpr int NVI = 4 * VPK;                // V copies per page
    static constexpr int NI = NKI + NVI + (FP8 ? 2 : 0);  // copies per page
    static_assert(NVI * 64 * VBYTES == PT, "V copies cover the page slice");
    // K copies move whole slot rows: a row of the head's slice is KPS
    // 16-byte pieces, a copy carries KSPC consecutive slots, and within a row
    // the pieces are stored XOR-swizzled by kswz(slot), so that the 16 lanes
    // reading one piece of 16 different slots hit distinct LDS banks.
    static constexpr int KPS = D * EB / 16;   // pieces per slot row
    static constexpr int KSPC = 64 / KPS;     // slots per copy
    static constexpr int KRPB = 16 / KPS;     // slots per 256-byte LDS row
    static_assert(NKI * KSPC == 16, "K copies cover the page's 16 slots");
    static __device__ __forceinline__ int kswz(int slot) { return (slot / KRPB) % KPS; }
    // byte offset, within the K slice in LDS, of piece pc (head dims
    // 16*pc/EB .. +16/EB) of slot `slot`
    static __device__ __forceinline__ int kread(int slot, int pc)
    {
        return (slot / KSPC) * 1024 + ((slot % KSPC) * KPS + (pc ^ kswz(slot))) * 16;
    }
    // first head dim of lane group q4 in MFMA chunk dc
    static __device__ __forceinline__ int qdim(int dc, int q4)
    {
        return FP8 ? (dc >> 1) * 64 + q4 * 16 + (dc & 1) * 8 : dc * 32 + q4 * 8;
    }
};

// Stores row tiles rt0 .. rt0+TPH-1 of a wave's unnormalised O tile (lane:
// rows rt*16 + l16, head dims NDT*(4*q4 + i) + t) into an LDS tile
// [TPH*16][D+4].
template <int D, int RG, int TPH>
__device__ __forceinline__ void tile_store(float *tile, const floatx4 (&acc)[D / 16][RG], int l16, int q4, int rt0)
{
    constexpr int OP = D + 4;
    constexpr int NDT = D / 16;
#pragma unroll
    for (int rt = 0; rt < RG; ++rt) {
        if (rt < rt0 || rt >= rt0 + TPH)
            continue;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int t0 = 0; t0 < NDT; t0 += 4)
                *reinterpret_cast<float4 *>(tile + ((rt - rt0) * 16 + l16) * OP + NDT * (4 * q4 + i) + t0) =
                    make_float4(acc[t0][rt][i], acc[t0 + 1][rt][i], acc[t0 + 2][rt][i], acc[t0 + 3][rt][i]);
    }
}

// Stores row pair pp (row tiles 2pp, 2pp+1) of a wave's unnormalised O kept
// in the 32x32 result layout (d = 128): lane l, register v holds head dims
// 4i .. 4i+3 (one per dim tile u) of row 32pp + l%32, i = 8(v/4) + 4(l/32) +
// v%4, into an LDS tile [32][D+4] (its rows 0..31).
template <int NP>
__device__ __forceinline__ void tile_store32(float *tile, const floatx16 (&acc)[4][NP], int lane, int pp)
{
    constexpr int OP = 128 + 4;
    const int r = lane & 31, i0 = 4 * (lane >> 5);
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const int i = 8 * (v >> 2) + i0 + (v & 3);
        *reinterpret_cast<float4 *>(tile + r * OP + 4 * i) =
            make_float4(acc[0][pp][v], acc[1][pp][v], acc[2][pp][v], acc[3][pp][v]);
    }
}

// Merges the wave tiles of rows r0 .. r1-1 of one workgroup and stores the
// result, for nh KV heads side by side (g .. g+nh-1): head hh's NT / nh waves
// are hh, hh + nh, ...  Normalised output when slot < 0 (the workgroup saw
// the unit's whole context), else the unnormalised partial (o, max, sum) in
// workspace slot slot + hh for the merge kernel.  tiles: NT tiles holding
// rows r0.. as [rows][D+4] floats, `pitch` floats apart; sm/sl: per-wave row
// max (base-2 units) and row sum.
template <int D, int RG, int NT>
__device__ __forceinline__ void merge_waves_and_store(const AttnParams &p, const float *tiles, int pitch,
                                                      const float (*sm)[kMaxRows], const float (*sl)[kMaxRows],
                                                      int slot, int b, int g, int r0, int r1, int nh = 1)
{
    constexpr int OP = D + 4;
    constexpr int C4 = D / 4;
    const float ninf = -__builtin_inff();
    const int G = p.G;
    const int nv = NT / nh;           // waves per head
    const int per = (r1 - r0) * C4;   // items per head
    for (int idx = threadIdx.x; idx < nh * per; idx += blockDim.x) {
        const int hh = nh == 1 ? 0 : idx / per;
        const int r = idx - hh * per;
        const int lr = r / C4, c4 = r - lr * C4;
        const int row = r0 + lr;
        float M = sm[hh][row];
#pragma unroll
        for (int v = 1; v < NT; ++v) {
            if (v >= nv)
                break;
            M = fmaxf(M, sm[hh + v * nh][row]);
        }
        float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
        float Ls = 0.0f;
#pragma unroll
        for (int v = 0; v < NT; ++v) {
            if (v >= nv)
                break;
            const int w = hh + v * nh;
            const float mv = sm[w][row];
            const float f = (mv == ninf) ? 0.0f : __builtin_amdgcn_exp2f(mv - M);
            const float4 x = *reinterpret_cast<const float4 *>(tiles + w * pitch + lr * OP + c4 * 4);
            o.x += f * x.x; o.y += f * x.y; o.z += f * x.z; o.w += f * x.w;
            Ls += f * sl[w][row];
        }
        if (slot < 0) {
            const float inv = 1.0f / Ls;
            o.x *= inv; o.y *= inv; o.z *= inv; o.w *= inv;
            const int t = row / G, q = row - t * G;
            *reinterpret_cast<float4 *>(p.out + (((size_t)b * p.T + t) * p.Hq + (size_t)(g + hh) * G + q) * D +
                                        c4 * 4) = o;
        } else {
            const size_t pbase = (size_t)(slot + hh) * p.TG;
            *reinterpret_cast<float4 *>(p.part_o + (pbase + row) * D + c4 * 4) = o;
            if (c4 == 0)
                reinterpret_cast<float2 *>(p.part_ml)[pbase + row] = make_float2(M, Ls);
        }
    }
}

// Shared pages (E4M3, d = 128, three or four row tiles): the workgroup runs
// 8 waves, two per SIMD.  Waves w and w+4 take the same pages (every 4th of
// the run) and each owns two of the row tiles; wave w copies each page into
// their common ring and a workgroup barrier per page hands it to wave w+4.
// One wave per SIMD leaves about half of such a page's time in stalls (the
// matrix instructions alone issue at near their peak rate from one wave);
// the second wave fills them.  bf16 storage uses them for more than four
// row tiles (T*G > 64, e.g. 16-node trees at G = 8), where one wave cannot
// hold every row tile's accumulators, and for four under balanced shares
// (see attn_share_pages); otherwise with up to four row tiles it streams at
// the memory's rate with 4 waves (shared pages measured slower there:
// 70B-layer shape 196 -> 231 us, 131k context 106 -> 125 us).  Also measured: 8 waves
// each with every row tile and every 8th page streamed no faster for bf16
// with fixed splits (8B-layer shape: 29.1 vs 28.3 us) and slower for E4M3
// (registers spill); they are used for balanced shares with at most two row
// tiles (ragged 64-sequence batch 430 -> 419 us: see attn_page_streams);
// handing pages out from an LDS counter instead of every 8th page measured
// the same there (and gives up run-to-run bit equality); 8 waves in which w
// and w+4 each copy the same pages into their own rings doubled the memory
// traffic.
constexpr int kTilesPerPhase = 2;  // row tiles merged per epilogue phase

template <int D, int RG, bool FP8, bool BAL>
struct MfmaShape {
    typedef PageGeom<D, FP8> PG;
    static constexpr bool SHARE = attn_share_pages(D, RG, FP8, BAL);
    static constexpr int HV = SHARE ? 2 : 1;                      // waves per page stream
    static constexpr int NWP = attn_page_streams(D, RG, FP8, BAL);  // page streams
    static constexpr int NW = NWP * HV;               // waves per workgroup
    static_assert(NW == attn_waves(D, RG, FP8, BAL), "workgroup shape");
    // page ids a balanced share holds (one share per compute unit for 8 waves)
    static constexpr int PCAP_BAL = NW == 8 ? kBalMaxShareOne : kBalMaxShare;
    static constexpr int RGW = (RG + HV - 1) / HV;    // row tiles per wave
    // d = 128 and an even number of row tiles per wave, for E4M3 and for
    // bf16 from four tiles per wave on: PV runs on the 32x32x16 matrix
    // instruction (see mfma_segment).
    static constexpr bool PV32 = D == 128 && RGW % 2 == 0 && (FP8 || RGW >= 4);
    // PV32: the V slice moves in key-major rows of D * EB bytes (16-byte
    // copies: two per page for E4M3, four for bf16), and each lane reads its
    // keys' dims from other lanes' bytes once the copying wave's wait (and,
    // with shared pages, the barrier) has passed; otherwise each lane reads
    // back only its own copies.
    static constexpr int VLPR = D * PG::EB / 16;                // PV32: lanes per key row of a copy
    static constexpr int NVI = PV32 ? PG::PT / 1024 : PG::NVI;  // V copies per page
    static constexpr int VB = PV32 ? 16 : PG::VBYTES;           // V copy width
    static constexpr int NI = PG::NKI + NVI + (FP8 ? 2 : 0);  // copies per page
    // Ring stages per page stream: about 8 KB of copies in flight behind the
    // page being computed (shared pages: one page behind the page being
    // waited for, which one barrier later is computed; 3 stages measured
    // 67.8 us on c5b against 70-72 with 4 and 72.6 with 5).  (Deeper rings
    // measured slower: more requests queue at the memory controllers without
    // raising the stream rate.)
    static constexpr int NS0 = 1 + (8192 + PG::STAGE - 1) / PG::STAGE;
    static constexpr int NS = NS0 > 4 ? 4 : NS0;
    static constexpr int OP = D + 4;
    static constexpr int TPH = RGW < kTilesPerPhase ? RGW : kTilesPerPhase;  // row tiles per epilogue phase
    static constexpr int WT = TPH * 16 * OP;  // floats of one wave's parked O rows
    // LDS: the page rings (one per page stream, RSTRIDE bytes apart) and, at
    // the end, each wave's parked O rows (PSTRIDE bytes apart).  Without
    // shared pages (one wave per stream) a wave's ring and parked rows share
    // one region.
    static constexpr int RING = (NS * PG::STAGE + 15) & ~15;
    static constexpr int PARK = (WT * 4 + 15) & ~15;
    static constexpr int RW = RING > PARK ? RING : PARK;
    static constexpr int RSTRIDE = SHARE ? RING : RW;
    static constexpr int PSTRIDE = SHARE ? PARK : RW;
    // Four row tiles per wave with shared pages (seven or eight row tiles in
    // all): the bf16 Q operands of the workgroup's rows wait in LDS, behind
    // the rings, instead of in registers (those would not fit beside four
    // tiles' accumulators).  Tile t, chunk dc: 64 lanes x 16 bytes at
    // QOFF + (t * NDC + dc) * 1024.
    static constexpr bool QLDS = SHARE && RGW >= 4;
    static constexpr int QOFF = NWP * RSTRIDE;
    static constexpr int QBYTES = QLDS ? HV * RGW * PG::NDC * 1024 : 0;
    static constexpr int LOOP_LDS = QOFF + QBYTES;
    static constexpr int SMEM = LOOP_LDS > NW * PSTRIDE ? LOOP_LDS : NW * PSTRIDE;
};

// One run of pages of one (sequence b, KV head g0) unit: pages blk_begin ..
// blk_begin + cap - 1, clipped to the context.  slot >= 0: the result is an
// unnormalised partial in that workspace slot; slot < 0: the run is the
// unit's whole context and the result is normalised into `out`.  With fixed
// splits (fixed = true) the slot given is that of (unit, split), replaced by
// -1 when the sequence has a single split.  Head groups (balanced shares,
// p.bal_hg > 1, see bal_heads): the run covers heads g0 .. g0 + bal_hg - 1,
// whose partials go to slots slot .. slot + bal_hg - 1.  Called by every
// thread of the workgroup.
template <int D, int RG, bool FP8, bool BAL>
__device__ __forceinline__ void mfma_segment(const AttnParams &p, unsigned char *smem, float (*s_m)[kMaxRows],
                                             float (*s_l)[kMaxRows], int *s_pages, const int b, const int g0,
                                             const int blk_begin, const int cap, const int slot, const bool fixed)
{
    typedef MfmaShape<D, RG, FP8, BAL> SH;
    typedef typename SH::PG PG;
    constexpr int NW = SH::NW;
    constexpr int NT = 64 * NW;          // threads
    constexpr int NDC = PG::NDC;
    constexpr int NDT = PG::NDT;
    constexpr int NS = SH::NS;
    constexpr int EB = PG::EB;
    constexpr int TPH = SH::TPH;
    constexpr bool PV32 = SH::PV32;
    constexpr bool SHARE = SH::SHARE;
    constexpr int NWP = SH::NWP;           // page streams
    constexpr int RGW = SH::RGW;           // row tiles of this wave
    constexpr int NP = PV32 ? RGW / 2 : 1;  // row-tile pairs (PV32)

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
    // Head groups: with 8 waves that each stream pages of their own, wave w
    // runs head g0 + w % hg and every (8 / hg)-th page of the run.
    constexpr bool HGRP = BAL && NWP == 8 && SH::HV == 1;
    const int hg = HGRP ? p.bal_hg : 1;
    const int g = g0 + (HGRP ? wave % hg : 0);       // this wave's KV head
    const int nstr = HGRP ? NWP / hg : NWP;          // page streams of the head
    const int pw = HGRP ? wave / hg : wave % NWP;    // page stream: pages pw, pw + nstr, ... of the run
    const int ring_id = HGRP ? wave : pw;            // the stream's copy ring
    const bool copier = wave < NWP;           // the wave that copies its stream's pages
    const int rt_base = (wave / NWP) * RGW;   // first row tile of this wave
    const int lane = tid & 63;
    const int l16 = lane & 15, q4 = lane >> 4;
    const int T = p.T, G = p.G, TG = p.TG, Hkv = p.Hkv;
    const float ninf = -__builtin_inff();

    // ---- prologue: one round trip to memory.  The context length, the
    // split's page ids (into LDS, and this wave's first NS-1 directly) and Q
    // are all requested before any of them is used.  Table entries past the
    // context are read (they are in bounds) but never used.
    const int32_t *trow = p.block_table + (size_t)b * p.max_blocks + blk_begin;
    const int avail = min(cap, p.max_blocks - blk_begin);
    const int Lraw = p.context_lens[b];
    int first[NS - 1];
#pragma unroll
    for (int k = 0; k < NS - 1; ++k) {
        const int i = pw + k * nstr;
        first[k] = i < avail ? trow[i] : 0;
    }
    // (all of the run's table entries are requested before any is stored:
    // a load-store loop would wait one round trip per NT entries, which
    // under full streaming load took ~10 us per run of 528 pages)
    constexpr int kPer = ((BAL ? SH::PCAP_BAL : kMaxBps) + NT - 1) / NT;
    int tv[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int i = tid + j * NT;
        tv[j] = i < avail ? trow[i] : 0;
    }
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int i = tid + j * NT;
        if (i < avail)
            s_pages[i] = clamp_block(tv[j], p.num_blocks);
    }
    float4 qraw[RGW][NDC][2];
    uint32_t anc[RGW];  // ancestor set of the lane's verify row (padding rows see everything)
#pragma unroll
    for (int rt = 0; rt < RGW; ++rt) {
        const int row = (rt_base + rt) * 16 + l16;
        const bool valid = row < TG;
        const int t = valid ? row / G : 0;
        anc[rt] = valid ? row_ancestors(p, b, t) : 0xFFFFFFFFu;
        const int hh = valid ? row - t * G : 0;
        const float *src = p.q + (((size_t)b * T + t) * p.Hq + (size_t)g * G + hh) * D;
#pragma unroll
        for (int dc = 0; dc < NDC; ++dc) {
            qraw[rt][dc][0] = make_float4(0.f, 0.f, 0.f, 0.f);
            qraw[rt][dc][1] = qraw[rt][dc][0];
            if (valid) {
                qraw[rt][dc][0] = *reinterpret_cast<const float4 *>(src + PG::qdim(dc, q4));
                qraw[rt][dc][1] = *reinterpret_cast<const float4 *>(src + PG::qdim(dc, q4) + 4);
            }
        }
    }
    const int L = Lraw < 0 ? 0 : (Lraw > p.max_blocks * kBlock ? p.max_blocks * kBlock : Lraw);
    const int nblk = (L + kBlock - 1) / kBlock;
    if (blk_begin >= nblk)
        return;  // uniform over the workgroup: nothing of this split is visible
    const int npg = min(blk_begin + cap, nblk) - blk_begin;
    const int oslot = (fixed && (nblk + p.bps - 1) / p.bps == 1) ? -1 : slot;

    // Q tile as the B operand of S^T = K Q^T (row = l16, eight dims), bf16,
    // pre-scaled into base-2 units.
    // (QLDS: the first page stream's waves store their row tiles' operands
    // in LDS, which the prologue's barrier publishes to the other streams.)
    constexpr bool QLDS = SH::QLDS;
    bf16x8 qf[QLDS ? 1 : RGW][NDC];
    unsigned char *const qlds = smem + SH::QOFF;
#pragma unroll
    for (int rt = 0; rt < RGW; ++rt) {
#pragma unroll
        for (int dc = 0; dc < NDC; ++dc) {
            const float sc = p.qscale;
            const float4 a = qraw[rt][dc][0], c = qraw[rt][dc][1];
            uint4 u;
            u.x = f32x2_to_bf16x2(a.x * sc, a.y * sc);
            u.y = f32x2_to_bf16x2(a.z * sc, a.w * sc);
            u.z = f32x2_to_bf16x2(c.x * sc, c.y * sc);
            u.w = f32x2_to_bf16x2(c.z * sc, c.w * sc);
            if constexpr (QLDS) {
                if (pw == 0)
                    *reinterpret_cast<uint4 *>(qlds + (((rt_base + rt) * NDC + dc) * 64 + lane) * 16) = u;
            } else {
                qf[rt][dc] = __builtin_bit_cast(bf16x8, u);
            }
        }
    }
    // Q operand of row tile rt (of this wave) and chunk dc
    auto qop = [&](int rt, int dc) -> bf16x8 {
        if constexpr (QLDS)
            return *reinterpret_cast<const bf16x8 *>(qlds + (((rt_base + rt) * NDC + dc) * 64 + lane) * 16);
        else
            return qf[rt][dc];
    };

    // Running state per row tile: reference maximum m (base-2 units), the
    // row sums and the unnormalised outputs O^T (lane: dims NDT*(4*q4+i)+t of
    // tile t, row l16).  bf16 storage gets its row sums from one extra MFMA
    // with an all-ones A operand; E4M3 storage scales P per page, so it sums
    // P on the VALU.
    // mth = m + kSlack and nms = -(m, or 0 while m is -inf) change only with
    // m (in the rare rescale branch), so they are kept rather than recomputed
    // for every page.
    float m[RGW], mth[RGW], nms[RGW], lpart[RGW];
    floatx4 lsum[RGW];
    floatx4 acc[PV32 ? 1 : NDT][PV32 ? 1 : RGW];
    floatx16 acc32[PV32 ? 4 : 1][NP];  // PV32: O^T of dim tile u, row pair pp
#pragma unroll
    for (int rt = 0; rt < RGW; ++rt) {
        m[rt] = ninf;
        mth[rt] = ninf + kSlack;
        nms[rt] = -0.0f;
        lpart[rt] = 0.0f;
        lsum[rt] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
    if constexpr (PV32) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int pp = 0; pp < NP; ++pp)
                acc32[u][pp] = floatx16{};
    } else {
#pragma unroll
        for (int rt = 0; rt < RGW; ++rt)
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
                acc[dt][rt] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
    const short4v ones4 = __builtin_bit_cast(short4v, make_uint2(0x3F803F80u, 0x3F803F80u));

    const unsigned char *kbase = static_cast<const unsigned char *>(p.k_cache);
    const unsigned char *vbase = static_cast<const unsigned char *>(p.v_cache);
    const int slot_stride = Hkv * D * EB;                          // bytes between slots of a page
    const uint32_t page_bytes = (uint32_t)slot_stride * kBlock;    // bytes of one page (all heads)
    const int head_off = g * D * EB;
    // K copy i: lane -> slot i*KSPC + lane/KPS, piece (lane%KPS) ^ kswz(slot)
    int k_voff[PG::NKI];
#pragma unroll
    for (int i = 0; i < PG::NKI; ++i) {
        const int r = lane / PG::KPS;
        k_voff[i] = head_off + r * slot_stride + ((lane % PG::KPS) ^ PG::kswz(i * PG::KSPC + r)) * 16;
    }
    // V copy: lane -> (dims NDT*l16.., key 4*q4 + copy / VPK); PV32: lane ->
    // (bytes 16*(l%VLPR) .. +15 of key l/VLPR + (64/VLPR)*copy)
    constexpr int VLPR = SH::VLPR;
    const int v_voff = PV32 ? head_off + (lane / VLPR) * slot_stride + 16 * (lane % VLPR)
                            : head_off + 4 * q4 * slot_stride + l16 * PG::VKB;
    const uint32_t ring_lds =
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char *)(smem) + ring_id * SH::RSTRIDE;
    const unsigned char *ring = smem + ring_id * SH::RSTRIDE;
    int4v dks{}, dvs{};
    if constexpr (FP8) {
        dks = page_desc(reinterpret_cast<const unsigned char *>(p.k_scale), 0, (uint32_t)p.num_blocks * 4u);
        dvs = page_desc(reinterpret_cast<const unsigned char *>(p.v_scale), 0, (uint32_t)p.num_blocks * 4u);
    }

    // This wave's pages are blk_begin + pw + k*nstr, k = 0, 1, ...  With
    // shared pages every wave runs the same number of steps (one barrier
    // each); a stream with one page fewer skips its last step's work.
    const int nk = npg > pw ? (npg - pw + nstr - 1) / nstr : 0;
    const int nsteps = SHARE ? (npg + NWP - 1) / NWP : nk;
    auto issue = [&](int k, int ph) {
        const int stage = k % NS;
        const uint32_t lds = ring_lds + stage * PG::STAGE;
        const int4v dk = page_desc(kbase, __builtin_amdgcn_readfirstlane(ph), page_bytes);
        const int4v dv = page_desc(vbase, __builtin_amdgcn_readfirstlane(ph), page_bytes);
#pragma unroll
        for (int i = 0; i < PG::NKI; ++i)
            dma_to_lds<16>(lds + i * 1024, dk, k_voff[i], i * PG::KSPC * slot_stride);
#pragma unroll
        for (int n = 0; n < SH::NVI; ++n)
            dma_to_lds<SH::VB>(lds + PG::PT + n * 64 * SH::VB, dv, v_voff,
                               PV32 ? n * (64 / VLPR) * slot_stride
                                    : (n / PG::VPK) * slot_stride + (n % PG::VPK) * PG::VBYTES);
        if constexpr (FP8) {
            const int soff = __builtin_amdgcn_readfirstlane(ph) * 4;
            dma_to_lds<4>(lds + 2 * PG::PT, dks, 0, soff);
            dma_to_lds<4>(lds + 2 * PG::PT + 256, dvs, 0, soff);
        }
    };
    // Waits until at most `younger` pages' copies are outstanding (they
    // complete in issue order).
    auto wait_pages = [&](int younger) {
        if (younger >= 3)
            wait_dma<3 * SH::NI>();
        else if (younger == 2)
            wait_dma<2 * SH::NI>();
        else if (younger == 1)
            wait_dma<SH::NI>();
        else
            wait_dma<0>();
    };
#pragma unroll
    for (int k = 0; k < NS - 1; ++k)
        if (copier && k < nk)
            issue(k, clamp_block(first[k], p.num_blocks));
    __syncthreads();  // s_pages ready

    // soff: byte offset of page k's ring stage, (k % NS) * STAGE, carried from
    // step to step (a wave-uniform scalar) instead of divided out per page
    for (int k = 0, soff = 0; k < nsteps; ++k, soff = (soff == (NS - 1) * PG::STAGE) ? 0 : soff + PG::STAGE) {
        if constexpr (SHARE) {
            // Page k has landed (pages k+1 .. k+NS-2 may stay in flight);
            // after the barrier the partner may read it, and both waves are
            // done with page k-1, whose stage the next copy reuses.
            if (copier)
                wait_pages(min(NS - 2, nk - 1 - k));
            __syncthreads();
            if (copier && k + NS - 1 < nk)
                issue(k + NS - 1, s_pages[pw + (k + NS - 1) * nstr]);
            if (k >= nk)
                continue;  // wave-uniform: this stream has one page fewer
        } else {
            if (k + NS - 1 < nk)
                issue(k + NS - 1, s_pages[pw + (k + NS - 1) * nstr]);
            // wait for page k: the copies of up to NS-1 younger pages may stay in flight
            wait_pages(min(NS - 1, nk - 1 - k));
        }
        const int pg = pw + k * nstr;
        const int key0 = (blk_begin + pg) * kBlock;
        const unsigned char *st = ring + soff;

        // 1. Read back this lane's K operands and V bytes of the page.
        uint4 kraw[PG::NKI];
#pragma unroll
        for (int i = 0; i < PG::NKI; ++i)
            kraw[i] = *reinterpret_cast<const uint4 *>(st + PG::kread(l16, 4 * i + q4));
        uint32_t vr[4][NDT / 2];  // [key j][dims 2w, 2w+1 as bf16]
        // PV32: dims 4i..4i+3 (i = l%32) of key 8*(l/32) + j, as E4M3 codes
        // (vc) or as two bf16 pairs (vb)
        uint32_t vc[8];
        uint2 vb[8];
        if constexpr (PV32) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const unsigned char *vrow = st + PG::PT + (8 * (lane >> 5) + j) * (D * EB);
                if constexpr (FP8)
                    vc[j] = *reinterpret_cast<const uint32_t *>(vrow + 4 * (lane & 31));
                else
                    vb[j] = *reinterpret_cast<const uint2 *>(vrow + 8 * (lane & 31));
            }
        } else if constexpr (PG::VBYTES == 16) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint4 x = *reinterpret_cast<const uint4 *>(st + PG::PT + j * 1024 + lane * 16);
                vr[j][0] = x.x; vr[j][1] = x.y; vr[j][2] = x.z; vr[j][3] = x.w;
            }
        } else {
#pragma unroll
            for (int n = 0; n < PG::NVI; ++n) {
                const uint32_t x = *reinterpret_cast<const uint32_t *>(st + PG::PT + n * 256 + lane * 4);
                const int j = n / PG::VPK, h = n % PG::VPK;
                if constexpr (FP8) {
                    const uint2 y = e4m3x4_to_bf16x4(x);
                    vr[j][2 * h] = y.x;
                    vr[j][2 * h + 1] = y.y;
                } else {
                    vr[j][h] = x;
                }
            }
        }

        // 2. S^T = K Q^T (keys on M, rows on N).
        floatx4 s[RGW];
#pragma unroll
        for (int rt = 0; rt < RGW; ++rt)
            s[rt] = floatx4{0.f, 0.f, 0.f, 0.f};
        if constexpr (FP8) {
#pragma unroll
            for (int i = 0; i < PG::NKI; ++i) {
                const bf16x8 k0 = __builtin_bit_cast(bf16x8, to_bf16x8(make_uint2(kraw[i].x, kraw[i].y)));
                const bf16x8 k1 = __builtin_bit_cast(bf16x8, to_bf16x8(make_uint2(kraw[i].z, kraw[i].w)));
#pragma unroll
                for (int rt = 0; rt < RGW; ++rt) {
                    s[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qop(rt, 2 * i), s[rt], 0, 0, 0);
                    s[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qop(rt, 2 * i + 1), s[rt], 0, 0, 0);
                }
            }
        } else {
#pragma unroll
            for (int dc = 0; dc < NDC; ++dc) {
                const bf16x8 kf = __builtin_bit_cast(bf16x8, kraw[dc]);
#pragma unroll
                for (int rt = 0; rt < RGW; ++rt)
                    s[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qop(rt, dc), s[rt], 0, 0, 0);
            }
        }

        // 3. V operands: slots past the context are cleared, then tile t's
        //    A operand (dim NDT*l16 + t of keys 4*q4 .. 4*q4+3) is gathered.
        //    PV32: dim tile u's A operand is dim 4*(l%32) + u of keys
        //    8*(l/32) .. +7 (codes are cleared before conversion; converting
        //    them later measured faster).
        if (key0 + kBlock > L) {  // wave-uniform: only a sequence's last page
            if constexpr (PV32) {
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const uint32_t keep = slot_keep(true, key0 + 8 * (lane >> 5) + j, L);
                    if constexpr (FP8) {
                        vc[j] &= keep;
                    } else {
                        vb[j].x &= keep;
                        vb[j].y &= keep;
                    }
                }
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t keep = slot_keep(true, key0 + 4 * q4 + j, L);
#pragma unroll
                    for (int w2 = 0; w2 < NDT / 2; ++w2)
                        vr[j][w2] &= keep;
                }
            }
        }
        short4v va4[PV32 ? 1 : NDT];
        bf16x8 va32[PV32 ? 4 : 1];
        if constexpr (PV32 && FP8) {
            // E4M3: one byte permute puts dims (4i, 4i+1) -- or (4i+2, 4i+3)
            // -- of keys 2w and 2w+1 side by side, so the two conversions of
            // its halves are already A-operand pairs (key 2w low, 2w+1 high)
            // of dim tiles u and u+1: 8 permutes per page instead of 16 after
            // converting.
            uint32_t w[4][4];  // [dim tile u][key pair w2]
#pragma unroll
            for (int w2 = 0; w2 < 4; ++w2) {
                const uint32_t zl = perm_b32(vc[2 * w2 + 1], vc[2 * w2], 0x05010400u);
                const uint32_t zh = perm_b32(vc[2 * w2 + 1], vc[2 * w2], 0x07030602u);
                w[0][w2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(zl, 1.0f, false));
                w[1][w2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(zl, 1.0f, true));
                w[2][w2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(zh, 1.0f, false));
                w[3][w2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(zh, 1.0f, true));
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
                va32[u] = __builtin_bit_cast(bf16x8, make_uint4(w[u][0], w[u][1], w[u][2], w[u][3]));
        } else if constexpr (PV32) {
            uint2 y[8];  // per key: dims (4i, 4i+1), (4i+2, 4i+3) as bf16 pairs
#pragma unroll
            for (int j = 0; j < 8; ++j)
                y[j] = vb[j];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                uint32_t w[4];
#pragma unroll
                for (int w2 = 0; w2 < 4; ++w2) {
                    const uint32_t a = u < 2 ? y[2 * w2].x : y[2 * w2].y;
                    const uint32_t c = u < 2 ? y[2 * w2 + 1].x : y[2 * w2 + 1].y;
                    w[w2] = (u & 1) ? pack_hi16(a, c) : pack_lo16(a, c);
                }
                va32[u] = __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
            }
        } else {
#pragma unroll
            for (int t = 0; t < NDT; ++t) {
                const int w2 = t >> 1;
                const uint32_t lo = (t & 1) ? pack_hi16(vr[0][w2], vr[1][w2]) : pack_lo16(vr[0][w2], vr[1][w2]);
                const uint32_t hi = (t & 1) ? pack_hi16(vr[2][w2], vr[3][w2]) : pack_lo16(vr[2][w2], vr[3][w2]);
                va4[t] = __builtin_bit_cast(short4v, make_uint2(lo, hi));
            }
        }

        // E4M3 page scales: K's multiplies the scores (folded into the
        // exponent below; scales are positive, so the maximum of the scaled
        // scores is the scaled maximum), V's multiplies P.
        float ksc = 1.0f, vsc = 1.0f;
        if constexpr (FP8) {
            ksc = *reinterpret_cast<const float *>(st + 2 * PG::PT + lane * 4);
            vsc = *reinterpret_cast<const float *>(st + 2 * PG::PT + 256 + lane * 4);
        }
        // 4. Causal (or tree) / length mask (only the last pages of a
        //    sequence need it).
        if (key0 + kBlock - 1 > L - T) {
#pragma unroll
            for (int rt = 0; rt < RGW; ++rt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (!key_visible(key0 + q4 * 4 + i, L, T, anc[rt]))
                        s[rt][i] = ninf;
        }
        // 5. Online softmax.  The common path only checks that no score of
        //    this lane exceeds its row's reference maximum by more than
        //    kSlack; only then (a wave-uniform, rarely taken branch) are the
        //    row maxima reduced across lanes and the accumulators rescaled.
        //    So P = 2^(s - m) <= 2^kSlack always.
        float mloc[RGW];
        bool need = false;
#pragma unroll
        for (int rt = 0; rt < RGW; ++rt) {
            mloc[rt] = ksc * fmaxf(fmaxf(s[rt][0], s[rt][1]), fmaxf(s[rt][2], s[rt][3]));
            need = need || (mloc[rt] > mth[rt]);
        }
        if (__builtin_expect(__ballot(need) != 0, 0)) {
            __asm__ volatile("" ::: "memory");  // keep this block a real branch
#pragma unroll
            for (int rt = 0; rt < RGW; ++rt) {
                float mx = mloc[rt];
                mx = fmaxf(mx, xor_lane_f32(mx, 16));
                mx = fmaxf(mx, xor_lane_f32(mx, 32));
                const float mnew = fmaxf(m[rt], mx);
                const float alpha = (mnew == ninf) ? 1.0f : __builtin_amdgcn_exp2f(m[rt] - mnew);
                m[rt] = mnew;
                mth[rt] = mnew + kSlack;
                nms[rt] = -((mnew == ninf) ? 0.0f : mnew);
                lpart[rt] *= alpha;
                lsum[rt] *= alpha;
                if constexpr (PV32) {
                    // the 32x32 result: lane l holds row l%16 of tile 2pp + (l%32)/16
                    const float a2 = (((lane >> 4) & 1) == (rt & 1)) ? alpha : 1.0f;
#pragma unroll
                    for (int u = 0; u < 4; ++u)
                        acc32[u][rt >> 1] *= a2;
                } else {
#pragma unroll
                    for (int dt = 0; dt < NDT; ++dt)
                        acc[dt][rt] *= alpha;
                }
            }
        }
        short4v pb[RGW];
#pragma unroll
        for (int rt = 0; rt < RGW; ++rt) {
            float pr[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                pr[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[rt][i], ksc, nms[rt]));
            if constexpr (FP8)
                lpart[rt] += (pr[0] + pr[1]) + (pr[2] + pr[3]);
            pb[rt] = __builtin_bit_cast(short4v, make_uint2(f32x2_to_bf16x2(pr[0] * vsc, pr[1] * vsc),
                                                             f32x2_to_bf16x2(pr[2] * vsc, pr[3] * vsc)));
        }
        // 6. O^T += V^T P^T over the page's 16 keys: A = V^T (dim row l16 of
        //    tile t, keys 4*q4..+3), B = P^T (keys 4*q4..+3, row l16), exactly
        //    the S^T output layout.
        //    PV32: O^T (32 dims x 32 rows) += V^T (32 dims x 16 keys) P^T per
        //    dim tile and row pair.  P^T's B operand (keys 8*(l/32) .. +7 of
        //    row l%32 of the pair) is the two tiles' S^T-layout P with the
        //    16-lane rows exchanged.
        if constexpr (PV32) {
#pragma unroll
            for (int pp = 0; pp < NP; ++pp) {
                const uint2 a = __builtin_bit_cast(uint2, pb[2 * pp]), c = __builtin_bit_cast(uint2, pb[2 * pp + 1]);
                const auto x0 = __builtin_amdgcn_permlane16_swap(a.x, c.x, false, false);
                const auto x1 = __builtin_amdgcn_permlane16_swap(a.y, c.y, false, false);
                const bf16x8 pbb = __builtin_bit_cast(bf16x8, make_uint4(x0[0], x1[0], x0[1], x1[1]));
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    acc32[u][pp] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va32[u], pbb, acc32[u][pp], 0, 0, 0);
            }
        } else {
#pragma unroll
            for (int t = 0; t < NDT; ++t)
#pragma unroll
                for (int rt = 0; rt < RGW; ++rt)
                    acc[t][rt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va4[t], pb[rt], acc[t][rt], 0, 0, 0);
        }
        if constexpr (!FP8) {
#pragma unroll
            for (int rt = 0; rt < RGW; ++rt)
                lsum[rt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ones4, pb[rt], lsum[rt], 0, 0, 0);
        }
    }

    // ---- epilogue: each wave parks its (max, sum) rows and unnormalised
    // tile in its own LDS region (without shared pages its ring, idle once
    // its copies have landed; with shared pages after a barrier, once both
    // waves of every stream are done with the rings), and after one barrier a
    // single pass merges the waves of each row half and writes the result.
    wait_dma<0>();
#pragma unroll
    for (int rt = 0; rt < RGW; ++rt) {
        float ls;
        if constexpr (FP8) {
            ls = lpart[rt];
            ls += xor_lane_f32(ls, 16);
            ls += xor_lane_f32(ls, 32);
        } else {
            ls = lsum[rt][0];
        }
        if (q4 == 0) {
            s_m[wave][(rt_base + rt) * 16 + l16] = m[rt];
            s_l[wave][(rt_base + rt) * 16 + l16] = ls;
        }
    }
    if constexpr (SHARE)
        __syncthreads();  // the parked rows overwrite the rings
    float *park = reinterpret_cast<float *>(smem + wave * SH::PSTRIDE);
#pragma unroll
    for (int rt0 = 0; rt0 < RGW; rt0 += TPH) {
        if (rt0 > 0)
            __syncthreads();  // the previous phase's tiles are consumed
        if constexpr (PV32)
            tile_store32<NP>(park, acc32, lane, rt0 / 2);
        else
            tile_store<D, RGW, TPH>(park, acc, l16, q4, rt0);
        __syncthreads();
        // row half h: the tiles of waves h*NWP .. h*NWP + NWP-1 (a phase
        // never reaches past the half's own RGW tiles into the next half's)
#pragma unroll
        for (int h = 0; h < SH::HV; ++h) {
            const int r0 = (h * RGW + rt0) * 16;
            const int r1 = min(p.TG, (h * RGW + min(rt0 + TPH, RGW)) * 16);
            if (r0 < r1)
                merge_waves_and_store<D, RGW, NWP>(p, reinterpret_cast<const float *>(smem + h * NWP * SH::PSTRIDE),
                                                   SH::PSTRIDE / 4, s_m + h * NWP, s_l + h * NWP, oslot, b, g0, r0,
                                                   r1, hg);
        }
    }
}

// Fixed splits: the workgroup's (unit, split) comes from its block index
// alone (see work_item), so every load of the segment's prologue can be in
// flight at once.  Balanced shares (see bal_share): the workgroup first sums
// the page counts of all sequences (one round trip for the context lengths,
// a workgroup prefix sum into LDS), then runs one segment per unit its share
// meets.  The merge kernel finds a cut unit's partials from the same prefix
// sums, which workgroup 0 leaves in the workspace.
template <int D, int RG, bool FP8, bool BAL>
__global__ __launch_bounds__((64 * MfmaShape<D, RG, FP8, BAL>::NW), 1) void sv_attn_mfma_kernel(AttnParams p)
{
    typedef MfmaShape<D, RG, FP8, BAL> SH;
    constexpr int NW = SH::NW;
    constexpr int NT = 64 * NW;
    __shared__ __attribute__((aligned(16))) unsigned char smem[SH::SMEM];
    __shared__ float s_m[NW][kMaxRows], s_l[NW][kMaxRows];
    __shared__ int s_pages[BAL ? SH::PCAP_BAL : kMaxBps];  // the segment's page ids

    if constexpr (!BAL) {
        int unit, split;
        work_item(p, unit, split);
        if (unit >= p.B * p.Hkv)
            return;
        const int b = unit / p.Hkv;
        mfma_segment<D, RG, FP8, BAL>(p, smem, s_m, s_l, s_pages, b, unit - b * p.Hkv, split * p.bps, p.bps,
                                 unit * p.max_splits + split, true);
        return;
    }
    __shared__ int s_P[kBalMaxB + 1];  // pages of the sequences before b
    __shared__ int s_wsum[NW];
    // head groups (see bal_heads): the share cuts (group, page) pairs, ngr
    // groups of hg heads per sequence
    constexpr bool HGRP = SH::NWP == 8 && SH::HV == 1;
    const int hg = HGRP ? p.bal_hg : 1;
    const int ngr = p.Hkv / hg;
    int pos = 0, end = 0, sb = 0, total = 0;
    {
        const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
        constexpr int PER = (kBalMaxB + NT - 1) / NT;  // sequences per thread
        int nbk[PER];
        int sum = 0;
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int bb = tid * PER + k;
            nbk[k] = bb < p.B ? (clamp_len(p, p.context_lens[bb]) + kBlock - 1) / kBlock : 0;
            sum += nbk[k];
        }
        int incl = sum;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
            const int t = __shfl_up(incl, o, kWave);
            if (lane >= o)
                incl += t;
        }
        if (lane == kWave - 1)
            s_wsum[wave] = incl;
        __syncthreads();
        int run = incl - sum;
        for (int w = 0; w < wave; ++w)
            run += s_wsum[w];
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int bb = tid * PER + k;
            if (bb < p.B)
                s_P[bb] = run;
            run += nbk[k];
        }
        if (tid == NT - 1)
            s_P[p.B] = run;  // every sequence's pages
        __syncthreads();
        if (blockIdx.x == 0)
            for (int i = tid; i <= p.B; i += NT)
                p.bal_prefix[i] = s_P[i];
        total = ngr * s_P[p.B];
        const int S = bal_share(total, SH::NW == 8);
        pos = (int)blockIdx.x * S;
        if (pos >= total)
            return;
        end = min(total, pos + S);
        // the sequence holding pair pos: the largest sb with ngr * P[sb] <= pos
        // (sequences without pages are skipped: their successor has the same P)
        int lo = 0, hi = p.B - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (ngr * s_P[mid] <= pos)
                lo = mid;
            else
                hi = mid - 1;
        }
        sb = lo;
    }
    for (;;) {
        int b, g, blk_begin, cap, slot;
        {
            const int Pb = s_P[sb], nb = s_P[sb + 1] - Pb;
            if (nb <= 0)
                return;  // unreachable: pair pos lies inside sequence sb
            const int base = ngr * Pb, rel = pos - base;
            const int gg = rel / nb;                // head group
            const int uend = base + (gg + 1) * nb;  // one past the group's last pair
            const int send = min(end, uend);
            const int off = rel - gg * nb;
            b = __builtin_amdgcn_readfirstlane(sb);
            g = __builtin_amdgcn_readfirstlane(gg * hg);
            blk_begin = __builtin_amdgcn_readfirstlane(off);
            cap = __builtin_amdgcn_readfirstlane(send - pos);
            slot = __builtin_amdgcn_readfirstlane((off == 0 && send == uend) ? -1
                                                                              : (sb * ngr + gg + (int)blockIdx.x) * hg);
        }
        mfma_segment<D, RG, FP8, BAL>(p, smem, s_m, s_l, s_pages, b, g, blk_begin, cap, slot, false);
        pos += cap;
        if (pos >= end)
            return;
        __syncthreads();  // the next segment reuses the LDS this one's epilogue read
        while (sb < p.B - 1 && ngr * s_P[sb + 1] <= pos)
            ++sb;
    }
}

// ---------------------------------------------------------------- VALU kernel

template <int KVT>
__device__ __forceinline__ float load_kv(const void *base, size_t idx)
{
    if constexpr (KVT == 0) {
        return static_cast<const float *>(base)[idx];
    } else if constexpr (KVT == 1) {
        return bf16_bits_to_f32(static_cast<const uint16_t *>(base)[idx]);
    } else {
        const uint32_t code = static_cast<const uint8_t *>(base)[idx];
        return __builtin_amdgcn_cvt_f32_fp8((int)code, 0);
    }
}

// MAXR: the most query rows per unit (T*G) this instantiation serves (64 or
// kMaxRows; the smaller one keeps its outputs in half the registers).
template <int D, int KVT, int MAXR>
__global__ __launch_bounds__(kAttnThreads) void sv_attn_valu_kernel(AttnParams p)
{
    constexpr int OP = D + 4;
    constexpr int KP = D + 1;
    constexpr int PER = (MAXR * D + kAttnThreads - 1) / kAttnThreads;
    __shared__ __attribute__((aligned(16))) float s_q[MAXR * OP];  // later: obuf
    __shared__ float s_k[kBlock * KP], s_v[kBlock * D], s_p[MAXR * (kBlock + 1)];
    __shared__ float s_alpha[MAXR], s_mrow[MAXR], s_lrow[MAXR];
    __shared__ uint32_t s_anc[MAXR];

    UnitWork w;
    if (!decode_work(p, w))
        return;
    const int tid = threadIdx.x;
    const int T = p.T, G = p.G, TG = p.TG, Hkv = p.Hkv;
    const int L = w.L;
    const float ninf = -__builtin_inff();

    for (int idx = tid; idx < TG * D; idx += kAttnThreads) {
        const int row = idx / D, col = idx - row * D;
        const int t = row / G, hh = row - t * G;
        s_q[row * OP + col] = p.q[(((size_t)w.b * T + t) * p.Hq + (size_t)w.g * G + hh) * D + col] * p.qscale;
    }
    for (int row = tid; row < TG; row += kAttnThreads)
        s_anc[row] = row_ancestors(p, w.b, row / G);
    float o[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k)
        o[k] = 0.0f;
    float m_row = ninf, l_row = 0.0f;  // owned by thread `row` < TG
    const int32_t *table = p.block_table + (size_t)w.b * p.max_blocks;

    for (int lb = w.blk_begin; lb < w.blk_end; ++lb) {
        const int ph = clamp_block(table[lb], p.num_blocks);
        float ks = 1.0f, vs = 1.0f;
        if constexpr (KVT == 2) {
            ks = p.k_scale[ph];
            vs = p.v_scale[ph];
        }
        __syncthreads();  // previous page fully consumed
        for (int idx = tid; idx < kBlock * D; idx += kAttnThreads) {
            const int s = idx / D, col = idx - s * D;
            const size_t e = (((size_t)ph * kBlock + s) * Hkv + w.g) * D + col;
            const bool ok = lb * kBlock + s < L;
            s_k[s * KP + col] = ok ? load_kv<KVT>(p.k_cache, e) * ks : 0.0f;
            s_v[s * D + col] = ok ? load_kv<KVT>(p.v_cache, e) * vs : 0.0f;
        }
        __syncthreads();
        for (int idx = tid; idx < TG * kBlock; idx += kAttnThreads) {
            const int row = idx >> 4, key = idx & 15;
            float dot = 0.0f;
#pragma unroll 8
            for (int col = 0; col < D; ++col)
                dot += s_q[row * OP + col] * s_k[key * KP + col];
            const int pos = lb * kBlock + key;
            s_p[row * (kBlock + 1) + key] = key_visible(pos, L, T, s_anc[row]) ? dot : ninf;
        }
        __syncthreads();
        if (tid < TG) {
            float mx = ninf;
            for (int key = 0; key < kBlock; ++key)
                mx = fmaxf(mx, s_p[tid * (kBlock + 1) + key]);
            const float mnew = fmaxf(m_row, mx);
            const float msafe = (mnew == ninf) ? 0.0f : mnew;
            const float alpha = __builtin_amdgcn_exp2f(m_row - msafe);
            float ps = 0.0f;
            for (int key = 0; key < kBlock; ++key) {
                const float pv = __builtin_amdgcn_exp2f(s_p[tid * (kBlock + 1) + key] - msafe);
                s_p[tid * (kBlock + 1) + key] = pv;
                ps += pv;
            }
            l_row = l_row * alpha + ps;
            m_row = mnew;
            s_alpha[tid] = alpha;
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int idx = tid + k * kAttnThreads;
            if (idx < TG * D) {
                const int row = idx / D, col = idx - row * D;
                float a = o[k] * s_alpha[row];
#pragma unroll
                for (int key = 0; key < kBlock; ++key)
                    a += s_p[row * (kBlock + 1) + key] * s_v[key * D + col];
                o[k] = a;
            }
        }
    }
    __syncthreads();
    float *obuf = s_q;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const int idx = tid + k * kAttnThreads;
        if (idx < TG * D) {
            const int row = idx / D, col = idx - row * D;
            obuf[row * OP + col] = o[k];
        }
    }
    if (tid < TG) {
        s_mrow[tid] = m_row;
        s_lrow[tid] = l_row;
    }
    __syncthreads();
    finish_unit<D>(p, w, obuf, s_mrow, s_lrow);
}

template <typename Kernel>
hipError_t launch(Kernel k, const AttnParams &p, hipStream_t stream)
{
    hipLaunchKernelGGL(k, dim3(p.grid), dim3(kAttnThreads), 0, stream, p);
    return hipGetLastError();
}

template <int D, int RG, bool FP8>
hipError_t launch_mfma_rg(const AttnParams &p, hipStream_t s)
{
    if (p.balanced)
        hipLaunchKernelGGL((sv_attn_mfma_kernel<D, RG, FP8, true>), dim3(p.grid),
                           dim3(64 * MfmaShape<D, RG, FP8, true>::NW), 0, s, p);
    else
        hipLaunchKernelGGL((sv_attn_mfma_kernel<D, RG, FP8, false>), dim3(p.grid),
                           dim3(64 * MfmaShape<D, RG, FP8, false>::NW), 0, s, p);
    return hipGetLastError();
}

template <int D, bool FP8>
hipError_t launch_mfma_d(const AttnParams &p, hipStream_t s)
{
    const int rg = (p.TG + 15) / 16;
    switch (rg) {
    case 1: return launch_mfma_rg<D, 1, FP8>(p, s);
    case 2: return launch_mfma_rg<D, 2, FP8>(p, s);
    case 3: return launch_mfma_rg<D, 3, FP8>(p, s);
    case 4: return launch_mfma_rg<D, 4, FP8>(p, s);
    case 5: return launch_mfma_rg<D, 5, FP8>(p, s);
    case 6: return launch_mfma_rg<D, 6, FP8>(p, s);
    case 7: return launch_mfma_rg<D, 7, FP8>(p, s);
    default: return launch_mfma_rg<D, 8, FP8>(p, s);
    }
}

template <int D, int MAXR>
hipError_t launch_valu_dr(const AttnParams &p, int kv, hipStream_t s)
{
    switch (kv) {
    case 0: return launch(sv_attn_valu_kernel<D, 0, MAXR>, p, s);
    case 1: return launch(sv_attn_valu_kernel<D, 1, MAXR>, p, s);
    default: return launch(sv_attn_valu_kernel<D, 2, MAXR>, p, s);
    }
}

template <int D>
hipError_t launch_valu_d(const AttnParams &p, int kv, hipStream_t s)
{
    return p.TG <= 64 ? launch_valu_dr<D, 64>(p, kv, s) : launch_valu_dr<D, kMaxRows>(p, kv, s);
}

}  // namespace

template <int D, int NB>
void launch_merge_r(const AttnParams &p, int R, dim3 grid, hipStream_t stream)
{
    if (R == 1)
        hipLaunchKernelGGL((sv_attn_merge_kernel<D, NB, 1>), grid, dim3(256), 0, stream, p);
    else if (R == 2)
        hipLaunchKernelGGL((sv_attn_merge_kernel<D, NB, 2>), grid, dim3(256), 0, stream, p);
    else
        hipLaunchKernelGGL((sv_attn_merge_kernel<D, NB, 4>), grid, dim3(256), 0, stream, p);
}

hipError_t launch_attn_merge(const AttnParams &p, hipStream_t stream)
{
    if (!p.balanced && p.max_splits <= 1)
        return hipSuccess;
    // One wave per group of R rows of a unit: R = 1 while one wave per row
    // fits in one resident round (about 8192 waves), else 2 or 4 (a unit's
    // rows then share one wave, whose loads for all of them are in flight
    // together)
    const long long rows = (long long)p.B * p.Hkv * p.TG;
    const int R = rows <= 8192 ? 1 : (rows <= 16384 ? 2 : 4);
    const long long waves = (long long)p.B * p.Hkv * ((p.TG + R - 1) / R);
    const dim3 grid((unsigned)((waves + 3) / 4));
    // Partial rows requested at once: 4 under balanced shares (which cut a
    // unit into two or three), whose smaller waves keep more of the grid
    // resident (ragged 64-sequence batch: 12.0-12.2 -> 10.6-11.3 us in two
    // traces), else 8.
    const bool few = p.balanced != 0;
    if (p.d == 64) {
        if (few)
            launch_merge_r<64, 4>(p, R, grid, stream);
        else
            launch_merge_r<64, 8>(p, R, grid, stream);
    } else if (!p.balanced && p.max_splits > 16) {
        const dim3 g1((unsigned)((rows + 3) / 4));
        hipLaunchKernelGGL((sv_attn_merge_kernel<128, 32, 1>), g1, dim3(256), 0, stream, p);
    } else if (!p.balanced && p.max_splits > 8) {
        const dim3 g1((unsigned)((rows + 3) / 4));
        hipLaunchKernelGGL((sv_attn_merge_kernel<128, 16, 1>), g1, dim3(256), 0, stream, p);
    } else if (few) {
        launch_merge_r<128, 4>(p, R, grid, stream);
    } else {
        launch_merge_r<128, 8>(p, R, grid, stream);
    }
    return hipGetLastError();
}

hipError_t launch_attn_mfma(const AttnParams &p, int kv_dtype, hipStream_t stream)
{
    const bool fp8 = kv_dtype == 2;
    if (p.d == 64)
        return fp8 ? launch_mfma_d<64, true>(p, stream) : launch_mfma_d<64, false>(p, stream);
    return fp8 ? launch_mfma_d<128, true>(p, stream) : launch_mfma_d<128, false>(p, stream);
}

hipError_t launch_attn_valu(const AttnParams &p, int kv_dtype, hipStream_t stream)
{
    return p.d == 64 ? launch_valu_d<64>(p, kv_dtype, stream) : launch_valu_d<128>(p, kv_dtype, stream);
}

}  // namespace sv
