// sample.hip -- the rejection sampler of the verify step, for gfx950.
//
// What is computed ("50 | Speculative Decoding" 3.1; "KV Cache + Speculative
// Decoding" 7.1-7.3 and 7.6): p_i = softmax(target row i); draft x_i is kept
// iff u_i * q_i(x_i) < p_i(x_i) (acceptance with probability
// min(1, p/q)); at the first rejection n the replacement is drawn from
// max(0, p_n - q_n) normalised, and with no rejection the bonus token is
// drawn from p_K.  Draws use the caller's uniform u_K and the inverse CDF in
// ascending token order.
//
// Three launches on the caller's stream (kernel boundaries order them, so no
// fences or counters are needed):
//   rowstats  grid (vocab chunk x row): one streaming pass over every target
//             row; per chunk the maximum and sum_j exp(l_j - max) (hardware
//             exp2, fp64 accumulation), reduced across the wave with DPP.
//             The first chunk's workgroup of draft row i also records the
//             target logit and draft probability of x_i;
//   decide    grid (1024-entry sub-chunk x sequence): every workgroup merges
//             the row statistics of its sequence, runs the (at most 15)
//             acceptance tests in fp64, and sums the weights of the chosen
//             row over its sub-chunk in fp64;
//   pick      grid (sequence): one wave prefix-scans the sub-chunk masses and
//             locates the sub-chunk holding u_K * S; the workgroup rescans
//             that sub-chunk (four entries per thread) with a prefix scan and
//             writes the outputs.
// The acceptance tests run in fp64; the weights take fp32 exp of an argument
// formed in fp64 and split exactly (about 1e-7 relative) and every sum runs
// in fp64, so the decisions agree with an exact evaluation except within
// ~1e-7 of a threshold.
//
// Temperature ("KV Cache + Speculative Decoding" 7.5): with a per-sequence T,
// every target row is p~ = softmax(logits / T) (the draft probabilities are
// taken as the draft's actual distribution); T <= 0 is the greedy limit,
// all mass on the first maximal logit of the row.
//
// Top-p (same section): with a per-sequence top_p < 1 the cut runs between
// rowstats and decide.  Tokens are ranked by logit; a token is kept iff the mass ranked
// strictly above it is below top_p (the top logit always kept), and p~ is
// renormalised over the kept set.  The masses exp((l - M) / T) are summed in
// 2^-43 fixed point with LDS integer atomics, so nothing depends on the order
// of the additions: a coarse histogram over (M - l) / T finds the bucket
// holding the cut, its entries are gathered into LDS, and a radix select on
// an order-preserving 32-bit key of the logit finds the cut exactly.  The
// output per row is the cut logit tau (every l >= tau is kept) and
// 1 / kept mass.
#include <atomic>

#include "sv_device.hpp"
#include "sv_internal.hpp"

namespace sv {
namespace {

constexpr int kPer = kSampleChunk / kSampleThreads;  // 32 entries per thread
constexpr int kNWs = kSampleThreads / kWave;
static_assert(kSampleSub == 4 * kSampleThreads, "a sub-chunk is four entries per thread");

struct RowStat {
    float m;
    int arg;     // first index of the chunk's maximum (greedy rows only)
    double z;    // sum over the chunk of exp((l - m) / T)
};

// Target logit and draft probability of draft token x_i.
struct RowX {
    float lx;
    float qx;
};

// What the draw of one sequence needs from the decide pass: the final
// token is drawn from max(0, p~ - coef * q) over target row `row` and draft
// row `qrow` (coef = 0: p~ itself).
struct SeqState {
    double inv_z;  // 1 / (kept) sum_j exp((l_j - m) / T) of the target row
    double inv_t;  // 1 / T
    double coef;   // residual coefficient: 1 after a chain rejection, C_k in a tree, 0 for a bonus
    int n;         // accepted drafts (tree: accepted nodes)
    int greedy;    // T <= 0: all mass on the first maximal logit ...
    int arg;       // ... which is this index
    int row;       // target row of the draw within the sequence
    int qrow;      // draft row of the draw within the sequence
    int tree;      // 1: the decide pass already wrote every output but the drawn token
    int ucol;      // column of the sequence's uniforms that drives the draw
    float m;       // max logit of the target row
    float tau;     // top-p cut of the row: entries with l < tau have p~ = 0
};
static_assert(sizeof(SeqState) <= kSeqStateBytes, "workspace slot of SeqState");

// Top-p cut of one target row: entries with l >= tau are kept; inv_p is
// 1 / sum of exp((l - M) / T) over them, or negative when the row is not cut.
struct RowCut {
    float tau;
    int pad;
    double inv_p;
};
static_assert(sizeof(RowCut) == kRowCutBytes, "workspace slot of RowCut");

// Temperature of sequence b: 1 without a temperature array; T <= 0 (or NaN)
// is the greedy limit.
struct Temp {
    bool greedy;
    double inv;    // 1 / T in fp64
    double l2inv;  // log2(e) / T in fp64
    float c_hi;    // log2(e) / T split into two floats for the exponent
    float c_lo;
};

// The temperature's constants from 1 / T (greedy: T <= 0 or NaN).
__device__ __forceinline__ Temp temp_from_inv(bool greedy, double inv)
{
    Temp t;
    t.greedy = greedy;
    t.inv = inv;
    t.l2inv = 1.4426950408889634074 * inv;
    t.c_hi = (float)t.l2inv;
    t.c_lo = (float)(t.l2inv - (double)t.c_hi);
    return t;
}

__device__ __forceinline__ Temp temp_of(const SampleParams &p, int b)
{
    const float T = p.temperature ? p.temperature[b] : 1.0f;
    const bool greedy = !(T > 0.0f);
    return temp_from_inv(greedy, greedy ? 1.0 : 1.0 / (double)T);
}

// Loads this thread's 32 entries of a chunk: entries tid*4 + k*1024 .. +3
// (float4 path) or tid + k*256 (scalar path); missing entries read `fill`.
template <bool VEC>
__device__ __forceinline__ void load_chunk(const float *row, int n, float fill, float (&v)[kPer])
{
    const int tid = threadIdx.x;
    if constexpr (VEC) {
#pragma unroll
        for (int k = 0; k < kPer / 4; ++k) {
            const int e = (k * kSampleThreads + tid) * 4;
            float4 x = make_float4(fill, fill, fill, fill);
            if (e < n)  // n is a multiple of 4 on this path
                x = *reinterpret_cast<const float4 *>(row + e);
            v[4 * k + 0] = x.x; v[4 * k + 1] = x.y; v[4 * k + 2] = x.z; v[4 * k + 3] = x.w;
        }
    } else {
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
            const int e = k * kSampleThreads + tid;
            v[k] = e < n ? row[e] : fill;
        }
    }
}

__device__ __forceinline__ float block_max(float v, float *s_red)
{
    v = wave_max_f32(v);
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0)
        s_red[wave] = v;
    __syncthreads();
    float r = s_red[0];
#pragma unroll
    for (int i = 1; i < kNWs; ++i)
        r = fmaxf(r, s_red[i]);
    __syncthreads();
    return r;
}

__device__ __forceinline__ double block_sum(double v, double *s_red)
{
    v = wave_sum_f64(v);
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0)
        s_red[wave] = v;
    __syncthreads();
    double r = s_red[0];
#pragma unroll
    for (int i = 1; i < kNWs; ++i)
        r += s_red[i];
    __syncthreads();
    return r;
}

__device__ __forceinline__ int clamp_token(int x, int V) { return x < 0 ? 0 : (x >= V ? V - 1 : x); }

// ptr[i] if ok, else fill.  The index is clamped to 0 instead of branching
// around the load (ptr[0] must be readable), so that a run of such loads
// stays in flight together.
template <typename T>
__device__ __forceinline__ T load_or(const T *ptr, size_t i, bool ok, T fill)
{
    const T v = ptr[ok ? i : 0];
    return ok ? v : fill;
}

// Target probability p~_j of entry j from its logit, the row maximum M, 1/Z
// and the temperature, to about one fp32 ulp: the base-2 argument
// t = (l - M) log2(e) / T is formed in fp64 (l - M is exact there) and split
// into a float hi and the remainder lo; 2^hi comes from the hardware exp2
// (v_exp_f32, about 1 ulp) and 2^lo = 1 + lo ln 2 to second order
// (|lo| <= ulp(hi)/2); products in fp64.  (The hardware exp2 replaced the
// library expf of the natural-base split: the same accuracy, a third of the
// vector instructions per entry, which the decide pass is bound by at large
// batches.)  Greedy rows are one-hot at `arg`.
__device__ __forceinline__ double target_prob_fast(float l, int j, float M, double invZ, const Temp &tp, int arg,
                                                   float tau)
{
    if (tp.greedy)
        return j == arg ? 1.0 : 0.0;
    if (!(l >= tau))
        return 0.0;  // outside the top-p set
    const double t = ((double)l - (double)M) * tp.l2inv;
    if (!(t > -150.0))
        return 0.0;  // underflows in fp32 (and catches l = -inf)
    const float hi = (float)t;
    const double lo = t - (double)hi;
    return (double)__builtin_amdgcn_exp2f(hi) * __builtin_fma(lo, 0.69314718055994530942, 1.0) * invZ;
}

// Same quantity in fp64 throughout (used for the K acceptance tests).
__device__ __forceinline__ double target_prob(float l, int j, float M, double invZ, const Temp &tp, int arg,
                                              float tau)
{
    if (tp.greedy)
        return j == arg ? 1.0 : 0.0;
    if (!(l >= tau))
        return 0.0;
    return exp(((double)l - (double)M) * tp.inv) * invZ;
}

// Weight of entry j of the chosen row: the residual max(0, p~ - coef * q)
// after a rejection (coef = 1 in the chain), p~ itself (coef = 0) for the
// bonus row or the zero-mass fallback.
__device__ __forceinline__ double weight(float l, float q, int j, float M, double invZ, double coef, const Temp &tp,
                                         int arg, float tau)
{
    const double pj = target_prob_fast(l, j, M, invZ, tp, arg, tau);
    if (coef == 0.0)
        return pj;
    const double r = pj - coef * (double)q;
    return r > 0.0 ? r : 0.0;
}

// ---------------------------------------------------------------- top-p cut

constexpr int kCutThreads = 1024;      // cut (select) kernel: one workgroup per row
constexpr int kCutWaves = kCutThreads / kWave;
constexpr int kCutDigit = 4096;        // 12-bit key digits (the last pass uses 8)
constexpr int kCutCap = 8192;          // entries of the crossing bucket held in LDS
constexpr int kCutBatch = 8;           // row loads in flight per thread
constexpr float kCutSpan = 45.0f;      // 2^t * 2^43 rounds to 0 below t = -44.5
constexpr float kCutPerUnit = kCutCoarse / kCutSpan;
constexpr double kCutScale = 8796093022208.0;  // 2^43

// Order-preserving key of a float: larger logit, larger key; -0 takes the
// key of +0, as the two compare equal.
__device__ __forceinline__ uint32_t logit_key(float l)
{
    uint32_t u = __builtin_bit_cast(uint32_t, l);
    if (u == 0x80000000u)
        u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_logit(uint32_t k)
{
    return __builtin_bit_cast(float, (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Tempered log2-mass of an entry relative to the row maximum,
// t = (l - M) log2(e) / T <= 0, with the constant split in two floats.
__device__ __forceinline__ float cut_t(float l, float M, const Temp &tp)
{
    const float dv = l - M;
    return __builtin_fmaf(dv, tp.c_hi, dv * tp.c_lo);
}

// Coarse bucket of t: kCutCoarse equal steps over (-45, 0], bucket 0 holding
// the largest logits; -1 below the span (and for -inf / NaN).  Never
// decreases as the logit decreases.
__device__ __forceinline__ int cut_bucket(float t)
{
    if (!(t > -kCutSpan))
        return -1;
    const int bk = (int)(-t * kCutPerUnit);
    return bk > kCutCoarse - 1 ? kCutCoarse - 1 : bk;
}

// 2^t in 2^-43 fixed point, rounded half up, from the hardware exp2: the
// float's 24-bit significand shifted into place (exact integer steps).
__device__ __forceinline__ uint64_t cut_mass(float t)
{
    const uint32_t bits = __builtin_bit_cast(uint32_t, __builtin_amdgcn_exp2f(t));
    const int E = (int)((bits >> 23) & 0xFFu);
    if (E == 0)
        return 0;  // zero or subnormal: far below 2^-43
    const uint64_t m = (bits & 0x7FFFFFu) | 0x800000u;
    const int sh = E - 107;  // value = m * 2^(E - 150), times 2^43
    if (sh >= 0)
        return m << sh;
    if (sh < -24)
        return 0;
    return (m + (1ull << (-sh - 1))) >> (-sh);
}

__device__ __forceinline__ uint64_t wave_incl_scan_u64(uint64_t v)
{
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint64_t t = __shfl_up(v, o, 64);
        if (lane >= o)
            v += t;
    }
    return v;
}

// Streams entries [begin, end) of a row through f, NT threads, kCutBatch
// loads in flight per thread; on the float4 path begin and end are multiples
// of 4.  Entries past the end read -inf.
template <bool VEC, int NT, typename F>
__device__ __forceinline__ void cut_stream(const float *row, int begin, int end, F &&f)
{
    const int tid = threadIdx.x;
    const float ninf = -__builtin_inff();
    if constexpr (VEC) {
        for (int base = begin; base < end; base += NT * 4 * kCutBatch) {
            float4 x[kCutBatch];
#pragma unroll
            for (int k = 0; k < kCutBatch; ++k) {
                const int e = base + (k * NT + tid) * 4;
                x[k] = e < end ? *reinterpret_cast<const float4 *>(row + e) : make_float4(ninf, ninf, ninf, ninf);
            }
#pragma unroll
            for (int k = 0; k < kCutBatch; ++k) {
                f(x[k].x);
                f(x[k].y);
                f(x[k].z);
                f(x[k].w);
            }
        }
    } else {
        for (int base = begin; base < end; base += NT * kCutBatch) {
            float x[kCutBatch];
#pragma unroll
            for (int k = 0; k < kCutBatch; ++k) {
                const int e = base + k * NT + tid;
                x[k] = e < end ? row[e] : ninf;
            }
#pragma unroll
            for (int k = 0; k < kCutBatch; ++k)
                f(x[k]);
        }
    }
}

// Whether row `row` is cut, and its maximum (from the chunk statistics;
// wave 0 of the calling workgroup reduces them into *s_M).
__device__ __forceinline__ bool cut_active(const SampleParams &p, int b, const Temp &tp)
{
    return !tp.greedy && p.top_p[b] < 1.0f;  // NaN or >= 1: no cut
}

__device__ __forceinline__ void cut_row_max(const SampleParams &p, int row, float *s_M)
{
    if (threadIdx.x < kWave) {
        const RowStat *st = static_cast<const RowStat *>(p.row_stats) + (size_t)row * p.nchunk;
        float m = -__builtin_inff();
        for (int c = threadIdx.x; c < p.nchunk; c += kWave)
            m = fmaxf(m, st[c].m);
        m = wave_max_f32(m);
        if (threadIdx.x == 0)
            *s_M = m;
    }
}

// Coarse histogram, part 1: grid (vocabulary chunk x row), shaped as the
// rowstats pass (its chunk loads are issued before the row maximum is
// read); each workgroup histograms the masses of its chunk over the coarse
// buckets in LDS and stores that partial histogram.
template <bool VEC>
__global__ __launch_bounds__(kSampleThreads) void sv_sample_cut_hist_kernel(SampleParams p)
{
    __shared__ unsigned long long s_hist[kCutCoarse];
    __shared__ float s_M;
    const int row = blockIdx.x / p.nchunk;
    const int chunk = blockIdx.x - row * p.nchunk;
    const int b = row / (p.K + 1);
    const Temp tp = temp_of(p, b);
    if (!cut_active(p, b, tp))
        return;  // uniform across the workgroup
    const int base = chunk * kSampleChunk;
    float v[kPer];
    load_chunk<VEC>(p.logits + (size_t)row * p.V + base, min(kSampleChunk, p.V - base), -__builtin_inff(), v);
    cut_row_max(p, row, &s_M);
    for (int i = threadIdx.x; i < kCutCoarse; i += kSampleThreads)
        s_hist[i] = 0;
    __syncthreads();
    const float M = s_M;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const float t = cut_t(v[k], M, tp);
        const int bk = cut_bucket(t);
        if (bk >= 0) {
            const uint64_t w = cut_mass(t);
            if (w)
                atomicAdd(&s_hist[bk], (unsigned long long)w);
        }
    }
    __syncthreads();
    unsigned long long *part = p.cut_part + ((size_t)row * p.nchunk + chunk) * kCutCoarse;
    for (int i = threadIdx.x; i < kCutCoarse; i += kSampleThreads)
        part[i] = s_hist[i];
}

struct CutShared {
    unsigned long long wsum[kCutWaves];
    unsigned long long carry, found;
    int digit, cnt;
    float M;
};

// The crossing bucket of a mass histogram: visiting the buckets in rank
// order (rank r is bucket r, or bucket nb-1-r when `descending`), the one
// at which the mass ranked before it, plus `carry`, is below tgt and with it
// reaches tgt.  Thread t owns ranks 4t .. 4t+3; one block scan.  Leaves the
// bucket in cs.digit (-1 if none), the mass ranked before it (carry
// included) in cs.carry and its own mass in cs.found.  With tgt = 0 the
// target is first set to max(1, ceil(top_p * total)).  Returns the target.
// Every thread of the workgroup calls it.
__device__ __forceinline__ unsigned long long cut_cross(const unsigned long long *hist, int nb, bool descending,
                                                        unsigned long long carry, unsigned long long tgt,
                                                        float top_p, CutShared &cs)
{
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    unsigned long long h[4] = {0, 0, 0, 0}, own = 0;
    int bk[4] = {0, 0, 0, 0};
    if (4 * tid < nb) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            bk[k] = descending ? nb - 1 - 4 * tid - k : 4 * tid + k;
            h[k] = hist[bk[k]];
            own += h[k];
        }
    }
    const unsigned long long incl = wave_incl_scan_u64(own);
    if (lane == 63)
        cs.wsum[wave] = incl;
    if (tid == 0)
        cs.digit = -1;
    __syncthreads();
    unsigned long long above = incl - own, total = 0;
#pragma unroll
    for (int w = 0; w < kCutWaves; ++w) {
        const unsigned long long t = cs.wsum[w];
        if (w < wave)
            above += t;
        total += t;
    }
    if (tgt == 0) {
        // a token is kept iff the mass ranked above it is < top_p * total
        tgt = (unsigned long long)__builtin_ceil((double)top_p * (double)total);
        if (tgt < 1)
            tgt = 1;
    }
    unsigned long long run = carry + above;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        if (run < tgt && run + h[k] >= tgt) {
            cs.digit = bk[k];
            cs.carry = run;
            cs.found = h[k];
        }
        run += h[k];
    }
    __syncthreads();
    return tgt;
}

// Streams one vocabulary chunk of a row through f with the 64 lanes of one
// wave, kCutBatch loads in flight per lane; entries past the end read -inf.
template <bool VEC, typename F>
__device__ __forceinline__ void cut_stream_chunk(const float *row, int base, int n, F &&f)
{
    const int lane = threadIdx.x & 63;
    const float ninf = -__builtin_inff();
    if constexpr (VEC) {
        for (int off = 0; off < n; off += kWave * 4 * kCutBatch) {
            float4 x[kCutBatch];
#pragma unroll
            for (int k = 0; k < kCutBatch; ++k) {
                const int e = off + (k * kWave + lane) * 4;
                x[k] = e < n ? *reinterpret_cast<const float4 *>(row + base + e) : make_float4(ninf, ninf, ninf, ninf);
            }
#pragma unroll
            for (int k = 0; k < kCutBatch; ++k) {
                f(x[k].x);
                f(x[k].y);
                f(x[k].z);
                f(x[k].w);
            }
        }
    } else {
        for (int off = 0; off < n; off += kWave * kCutBatch) {
            float x[kCutBatch];
#pragma unroll
            for (int k = 0; k < kCutBatch; ++k) {
                const int e = off + k * kWave + lane;
                x[k] = e < n ? row[base + e] : ninf;
            }
#pragma unroll
            for (int k = 0; k < kCutBatch; ++k)
                f(x[k]);
        }
    }
}

constexpr int kCutDirect = 512;  // up to this many candidates: rank them directly
static_assert(2 * kCutDirect + 2 * (kCutThreads / kWave) <= kCutDigit, "direct ranking scratch fits in s_hist");

// Part 2, one workgroup per row: sums the partial histograms (exact integer
// sums), finds the coarse bucket d0 holding the cut, and gathers the entries
// of d0 into LDS (each wave takes whole chunks; a chunk whose partial
// histogram has no mass in d0 holds no entry that matters and is skipped).
// The exact cut among the candidates: with at most kCutDirect of them each
// is ranked directly (the mass of the candidates with a larger key); with
// more, a radix select on their keys (12 + 12 + 8 bits).  Should d0 hold
// more than kCutCap entries, the digit passes stream the row instead,
// filtered to d0.  All masses are the fixed-point ones of part 1.
template <bool VEC>
__global__ __launch_bounds__(kCutThreads) void sv_sample_cut_kernel(SampleParams p)
{
    __shared__ unsigned long long s_hist[kCutDigit];
    __shared__ float s_cand[kCutCap];
    __shared__ CutShared cs;

    const int row = blockIdx.x;
    const int b = row / (p.K + 1);
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    RowCut *out = static_cast<RowCut *>(p.row_cut) + row;
    const Temp tp = temp_of(p, b);
    if (!cut_active(p, b, tp)) {  // uniform across the workgroup
        if (tid == 0)
            *out = RowCut{-__builtin_inff(), 0, -1.0};
        return;
    }
    const float top_p = p.top_p[b];
    const int nchunk = p.nchunk;
    const unsigned long long *part = p.cut_part + (size_t)row * nchunk * kCutCoarse;
    cut_row_max(p, row, &cs.M);
    for (int i = tid; i < kCutCoarse; i += kCutThreads)
        s_hist[i] = 0;
    if (tid == 0)
        cs.cnt = 0;
    __syncthreads();
    {
        // two threads per bucket, each summing every other chunk, eight
        // loads in flight
        constexpr int kLanesPerBucket = kCutThreads / kCutCoarse;
        const int bk = tid % kCutCoarse, c0 = tid / kCutCoarse;
        unsigned long long h = 0;
        for (int c = c0; c < nchunk; c += 8 * kLanesPerBucket) {
            unsigned long long x[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int cc = c + j * kLanesPerBucket;
                x[j] = cc < nchunk ? part[(size_t)cc * kCutCoarse + bk] : 0ull;
            }
#pragma unroll
            for (int j = 0; j < 8; ++j)
                h += x[j];
        }
        if (h)
            atomicAdd(&s_hist[bk], h);
    }
    __syncthreads();
    const float M = cs.M;
    const float *lrow = p.logits + (size_t)row * p.V;
    const int V = p.V;

    const unsigned long long tgt = cut_cross(s_hist, kCutCoarse, false, 0, 0, top_p, cs);
    const int d0 = cs.digit;
    const unsigned long long carry0 = cs.carry;
    if (d0 < 0) {  // unreachable for rows with a finite maximum: leave the row uncut
        if (tid == 0)
            *out = RowCut{-__builtin_inff(), 0, -1.0};
        return;
    }

    // Gather the entries of d0 (those of zero mass included: they add nothing).
    for (int c = wave; c < nchunk; c += kCutWaves) {
        if (part[(size_t)c * kCutCoarse + d0] == 0)
            continue;  // uniform across the wave
        const int base = c * kSampleChunk;
        cut_stream_chunk<VEC>(lrow, base, min(kSampleChunk, V - base), [&](float l) {
            if (cut_bucket(cut_t(l, M, tp)) == d0) {
                const int slot = atomicAdd(&cs.cnt, 1);
                if (slot < kCutCap)
                    s_cand[slot] = l;
            }
        });
    }
    __syncthreads();
    const int cnt = cs.cnt;

    if (cnt <= kCutDirect) {
        // Candidate i is kept iff carry0 + (mass of candidates with a larger
        // key) < tgt; the cut is the smallest kept key.
        uint32_t ki = 0xFFFFFFFFu;
        unsigned long long wi = 0;
        bool kept = false;
        if (tid < cnt) {
            const float l = s_cand[tid];
            ki = logit_key(l);
            wi = cut_mass(cut_t(l, M, tp));
        }
        // keys and masses side by side in s_hist: [2i] key, [2i+1] mass
        if (tid < cnt) {
            s_hist[2 * tid] = ki;
            s_hist[2 * tid + 1] = wi;
        }
        __syncthreads();
        if (tid < cnt) {
            unsigned long long above = 0;
            for (int j = 0; j < cnt; ++j) {
                const uint32_t kj = (uint32_t)s_hist[2 * j];
                if (kj > ki)
                    above += s_hist[2 * j + 1];
            }
            kept = carry0 + above < tgt;
        }
        const uint32_t kmin = kept ? ki : 0xFFFFFFFFu;
        const unsigned long long wk = kept ? wi : 0ull;
        // block reductions: smallest kept key, kept mass
        uint32_t m = kmin;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1)
            m = min(m, (uint32_t)__shfl_xor((int)m, o, 64));
        const unsigned long long ws = wave_incl_scan_u64(wk);
        __syncthreads();  // s_hist reads above are done
        if (lane == 63) {
            s_hist[2 * kCutDirect + wave] = ws;  // scratch past the candidates' slots
            s_hist[2 * kCutDirect + kCutWaves + wave] = m;
        }
        __syncthreads();
        if (tid == 0) {
            unsigned long long kept_mass = carry0;
            uint32_t kcut = 0xFFFFFFFFu;
            for (int w = 0; w < kCutWaves; ++w) {
                kept_mass += s_hist[2 * kCutDirect + w];
                kcut = min(kcut, (uint32_t)s_hist[2 * kCutDirect + kCutWaves + w]);
            }
            if (kcut == 0xFFFFFFFFu || kept_mass == 0)
                *out = RowCut{-__builtin_inff(), 0, -1.0};  // unreachable: the top candidate is kept
            else
                *out = RowCut{key_logit(kcut), 0, kCutScale / (double)kept_mass};
        }
        return;
    }

    const bool in_lds = cnt <= kCutCap;
    unsigned long long carry = carry0;
    uint32_t prefix = 0;
    for (int pass = 0; pass < 3; ++pass) {
        const int shift = pass == 0 ? 20 : (pass == 1 ? 8 : 0);
        const int nb = pass == 2 ? 256 : kCutDigit;
        const int pshift = pass == 0 ? 32 : (pass == 1 ? 20 : 8);  // bits above the digit
        for (int i = tid; i < nb; i += kCutThreads)
            s_hist[i] = 0;
        __syncthreads();
        auto visit = [&](float l, float t) {
            const uint32_t k = logit_key(l);
            if (pshift < 32 && (k >> pshift) != prefix)
                return;
            const uint64_t w = cut_mass(t);
            if (w)
                atomicAdd(&s_hist[(k >> shift) & (uint32_t)(nb - 1)], (unsigned long long)w);
        };
        if (in_lds) {
            for (int i = tid; i < cnt; i += kCutThreads) {
                const float l = s_cand[i];
                visit(l, cut_t(l, M, tp));
            }
        } else {
            cut_stream<VEC, kCutThreads>(lrow, 0, V, [&](float l) {
                const float t = cut_t(l, M, tp);
                if (cut_bucket(t) == d0)
                    visit(l, t);
            });
        }
        __syncthreads();
        cut_cross(s_hist, nb, true, carry, tgt, top_p, cs);
        const int d = cs.digit;
        if (d < 0) {  // unreachable: the entries of d0 sum to its coarse mass
            if (tid == 0)
                *out = RowCut{-__builtin_inff(), 0, -1.0};
            return;
        }
        prefix = (prefix << (pass == 2 ? 8 : 12)) | (uint32_t)d;
        carry = cs.carry;
    }
    if (tid == 0)
        *out = RowCut{key_logit(prefix), 0, kCutScale / (double)(cs.carry + cs.found)};
}

// Loads this thread's four consecutive entries tid*4 .. tid*4+3 of a
// sub-chunk of n entries; missing entries read `fill`.
template <bool VEC>
__device__ __forceinline__ void load_sub(const float *row, int n, float fill, float (&v)[4])
{
    const int e0 = threadIdx.x * 4;
    if constexpr (VEC) {
        float4 x = make_float4(fill, fill, fill, fill);
        if (e0 < n)  // n is a multiple of 4 on this path
            x = *reinterpret_cast<const float4 *>(row + e0);
        v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
    } else {
#pragma unroll
        for (int k = 0; k < 4; ++k)
            v[k] = e0 + k < n ? row[e0 + k] : fill;
    }
}

// Chosen-row weights and plain target mass of sub-chunks sub0 .. sub0+nsh-1
// of one sequence, into s_part[j][wave][0 / 1] (each sub-chunk summed in its
// own fixed order).  The weight of entry j is max(0, p~_j - coef * q_j)
// (the draft row is read only when coef > 0), else p~_j.  The loads run one
// sub-chunk ahead of the sums, so a workgroup that covers several sub-chunks
// keeps two in flight while holding registers for two.
template <bool VEC>
__device__ __forceinline__ void sub_chunk_masses(const float *lrow, const float *qrow, double coef, int sub0,
                                                 int nsh, int V, float M, double invZ, const Temp &tp, int arg,
                                                 float tau, double (*s_part)[kNWs][2])
{
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    auto load = [&](int j, float (&lv)[4], float (&qv)[4]) {
        const int base = (sub0 + j) * kSampleSub;
        const int cnt = min(kSampleSub, V - base);
        load_sub<VEC>(lrow + base, cnt, -__builtin_inff(), lv);
        if (coef > 0.0) {
            load_sub<VEC>(qrow + base, cnt, 0.0f, qv);
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k)
                qv[k] = 0.0f;
        }
    };
    auto mass = [&](int j, const float (&lv)[4], const float (&qv)[4]) {
        const int base = (sub0 + j) * kSampleSub;
        double sw = 0.0, sp = 0.0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const double pj = target_prob_fast(lv[k], base + tid * 4 + k, M, invZ, tp, arg, tau);
            sp += pj;
            if (coef > 0.0) {
                const double r = pj - coef * (double)qv[k];
                sw += r > 0.0 ? r : 0.0;
            } else {
                sw += pj;
            }
        }
        sw = wave_sum_f64(sw);
        sp = wave_sum_f64(sp);
        if (lane == 0) {
            s_part[j][wave][0] = sw;
            s_part[j][wave][1] = sp;
        }
    };
    float la[4], qa[4], lb[4], qb[4];
    load(0, la, qa);
    for (int j = 0; j < nsh; j += 2) {  // nsh >= 1, uniform
        if (j + 1 < nsh)
            load(j + 1, lb, qb);
        mass(j, la, qa);
        if (j + 1 >= nsh)
            break;
        if (j + 2 < nsh)
            load(j + 2, la, qa);
        mass(j + 1, lb, qb);
    }
}

// Per-sequence statistics and tests shared by the decide kernel and the
// gated second rowstats launch (see launch_sample).
struct SeqTests {
    float M[16];
    double Z[16];  // 1 / (kept) row mass
    int A[16];
    float tau[16];
    double ratio[16];
    double th[16];
    int acc[16];
    int n;
};

// Merges the chunk statistics of rows 0 .. nrows-1 of sequence b into each
// row's maximum, 1/Z (or the top-p cut's 1/kept mass), first argmax and cut,
// and runs the tests of positions 0 .. ntests-1 (ntests <= nrows, rows past
// nrows are not read), leaving the first rejection (or ntests) in sh.n.  The
// arithmetic of a row or a test does not depend on nrows or ntests, so two
// callers with different counts agree on every position both test.  Called
// by every thread of the workgroup.
__device__ __forceinline__ void seq_tests(const SampleParams &p, int b, const Temp &tp, int nrows, int ntests,
                                          SeqTests &sh)
{
    float *s_M = sh.M;
    double *s_Z = sh.Z;
    int *s_A = sh.A;
    float *s_tau = sh.tau;
    double *s_ratio = sh.ratio;
    double *s_th = sh.th;
    int *s_acc = sh.acc;
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int K = p.K, K1 = K + 1, V = p.V;
    // 1. Row statistics of the first nrows rows of this sequence (one wave
    //    per row, lanes over vocabulary chunks) and the draft tokens'
    //    entries, all requested together.
    RowX rx{0.0f, 0.0f};
    float u = 0.0f;
    int x = 0;
    if (tid < ntests) {
        rx = static_cast<const RowX *>(p.row_x)[(size_t)b * K + tid];
        u = p.uniforms[(size_t)b * K1 + tid];
        x = clamp_token(p.tokens[(size_t)b * K + tid], V);
    }
    // Per row: maximum, 1/Z (or the top-p cut's 1/kept mass), first argmax
    // (greedy rows) and the typical-acceptance threshold, from the chunk
    // statistics of lane c = chunk c (and further chunks c + 64k).
    auto finish_row = [&](int i, float M, double Z, int A, double S) {
        if (lane == 0) {
            if (p.typical) {
                const double H = tp.greedy ? 0.0 : log(Z) - S / Z;  // entropy in nats
                s_th[i] = fmin(p.ty_eps, p.ty_delta * exp(-H));
            }
            float tau = -__builtin_inff();
            double invZ = 1.0 / Z;
            if (p.row_cut) {
                const RowCut rc = static_cast<const RowCut *>(p.row_cut)[(size_t)b * K1 + i];
                if (rc.inv_p > 0.0) {
                    tau = rc.tau;
                    invZ = rc.inv_p;
                }
            }
            s_M[i] = M;
            s_Z[i] = invZ;
            s_A[i] = A;
            s_tau[i] = tau;
        }
    };
    if (p.nchunk <= kWave) {
        // every row of this wave (rows wave, wave + 4, ..) requested at once
        constexpr int kRowsPerWave = 16 / kNWs;
        RowStat rs[kRowsPerWave];
        double re[kRowsPerWave];
#pragma unroll
        for (int j = 0; j < kRowsPerWave; ++j) {
            const int i = wave + j * kNWs;
            rs[j] = RowStat{-__builtin_inff(), 0x7FFFFFFF, 0.0};
            re[j] = 0.0;
            if (i < nrows && lane < p.nchunk) {
                rs[j] = static_cast<const RowStat *>(p.row_stats)[(size_t)(b * K1 + i) * p.nchunk + lane];
                if (p.typical)
                    re[j] = p.row_ent[(size_t)(b * K1 + i) * p.nchunk + lane];
            }
        }
#pragma unroll
        for (int j = 0; j < kRowsPerWave; ++j) {
            const int i = wave + j * kNWs;
            if (i >= nrows)
                break;  // uniform
            const float M = wave_max_f32(rs[j].m);
            double z = 0.0, sl = 0.0;
            int al = 0x7FFFFFFF;
            if (lane < p.nchunk) {
                if (tp.greedy) {
                    if (rs[j].m == M)
                        al = rs[j].arg;
                } else if (rs[j].z > 0.0) {
                    const double d = ((double)rs[j].m - (double)M) * tp.inv;
                    const double e = exp(d);
                    z = rs[j].z * e;
                    if (p.typical)
                        sl = e * (re[j] + d * rs[j].z);  // e^{d}(s_c + d z_c), d = (m_c - M) / T
                }
            }
            const double Z = wave_sum_f64(z);
            const int A = wave_min_i32(al);
            const double S = p.typical ? wave_sum_f64(sl) : 0.0;
            finish_row(i, M, Z, A, S);
        }
    } else {
        for (int i = wave; i < nrows; i += kNWs) {
            const RowStat *st = static_cast<const RowStat *>(p.row_stats) + (size_t)(b * K1 + i) * p.nchunk;
            float mloc = -__builtin_inff();
            for (int c = lane; c < p.nchunk; c += kWave)
                mloc = fmaxf(mloc, st[c].m);
            const float M = wave_max_f32(mloc);
            double zloc = 0.0, sloc = 0.0;
            int aloc = 0x7FFFFFFF;
            const double *ent = p.row_ent + (size_t)(b * K1 + i) * p.nchunk;
            for (int c = lane; c < p.nchunk; c += kWave) {
                const RowStat r = st[c];
                if (tp.greedy) {
                    if (r.m == M && r.arg < aloc)
                        aloc = r.arg;  // chunks are in index order: the first maximal chunk
                } else if (r.z > 0.0) {  // a chunk that is -inf throughout adds nothing
                    const double d = ((double)r.m - (double)M) * tp.inv;
                    const double e = exp(d);
                    zloc += r.z * e;
                    if (p.typical)
                        sloc += e * (ent[c] + d * r.z);
                }
            }
            const double Z = wave_sum_f64(zloc);
            const int A = wave_min_i32(aloc);
            const double S = p.typical ? wave_sum_f64(sloc) : 0.0;
            finish_row(i, M, Z, A, S);
        }
    }
    __syncthreads();
    // 2. Acceptance tests u_i * q_i(x_i) < p~_i(x_i), or for typical
    //    acceptance p~_i(x_i) > min(eps, delta exp(-H_i)).
    if (tid < ntests) {
        const double a = target_prob(rx.lx, x, s_M[tid], s_Z[tid], tp, s_A[tid], s_tau[tid]);
        if (p.typical) {
            s_acc[tid] = (a > s_th[tid]) ? 1 : 0;
            s_ratio[tid] = a;
        } else {
            const double c = (double)rx.qx;
            s_acc[tid] = ((double)u * c < a) ? 1 : 0;
            s_ratio[tid] = c > 0.0 ? fmin(1.0, a / c) : (a > 0.0 ? 1.0 : 0.0);
        }
    }
    __syncthreads();
    if (tid == 0) {
        int n = ntests;
        for (int i = 0; i < ntests; ++i)
            if (!s_acc[i]) {
                n = i;
                break;
            }
        sh.n = n;
    }
    __syncthreads();
}

// GATED: the launch covers rows row_lo .. row_lo + row_cnt - 1 of every
// sequence and skips the sequences whose gate flag is 0; otherwise it covers
// every row (and reads neither the range nor the flags).
template <bool VEC, bool GATED>
__global__ __launch_bounds__(kSampleThreads) void sv_sample_rowstats_kernel(SampleParams p)
{
    __shared__ float s_f[kNWs];
    __shared__ double s_d[kNWs];
    const int rloc = blockIdx.x / p.nchunk;
    const int chunk = blockIdx.x - rloc * p.nchunk;
    const int K = p.K, K1 = K + 1;
    const int rc = GATED ? p.row_cnt : K1;
    const int b = rloc / rc, i = (GATED ? p.row_lo : 0) + (rloc - b * rc);
    const int row = b * K1 + i;
    if (GATED && p.gate_r > 0 && p.gate[b] == 0)
        return;  // uniform: a draft before this row was rejected, so the row never reaches the output
    const int base = chunk * kSampleChunk;
    const int n = min(kSampleChunk, p.V - base);
    float v[kPer];
    load_chunk<VEC>(p.logits + (size_t)row * p.V + base, n, -__builtin_inff(), v);
    // x_i's own entries, fetched while the chunk streams in.
    const bool rec = !p.tree && chunk == 0 && i < K;
    RowX rx{0.0f, 0.0f};
    if (rec) {
        const int x = clamp_token(p.tokens[(size_t)b * K + i], p.V);
        rx.lx = p.logits[(size_t)row * p.V + x];
        rx.qx = p.probs ? p.probs[((size_t)b * K + i) * p.V + x] : 0.0f;
    }
    float mx = v[0];
#pragma unroll
    for (int k = 1; k < kPer; ++k)
        mx = fmaxf(mx, v[k]);
    const float M = block_max(mx, s_f);
    const Temp tp = temp_of(p, b);
    RowStat st;
    st.m = M;
    st.arg = 0;
    st.z = 0.0;
    if (tp.greedy) {
        // first index of the maximum within the chunk
        int first = 0x7FFFFFFF;
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
            const int e = VEC ? ((k >> 2) * kSampleThreads + (int)threadIdx.x) * 4 + (k & 3)
                              : k * kSampleThreads + (int)threadIdx.x;
            if (v[k] == M && e < first)
                first = e;
        }
        first = wave_min_i32(first);
        __shared__ int s_i[kNWs];
        if ((threadIdx.x & 63) == 0)
            s_i[threadIdx.x >> 6] = first;
        __syncthreads();
#pragma unroll
        for (int w = 0; w < kNWs; ++w)
            first = min(first, s_i[w]);
        st.arg = base + first;
        if (p.typical && threadIdx.x == 0)
            p.row_ent[(size_t)row * p.nchunk + chunk] = 0.0;
    } else {
        // exp((v - M) / T) = 2^((v - M) log2(e) / T) with the hardware exp2;
        // the constant log2(e) / T enters as two floats, so the scaled
        // argument carries one rounding; terms are summed in fp64.  The clamp
        // sends -inf entries (and a chunk that is -inf throughout, where
        // v - M is NaN) to a finite difference whose term is 0, whatever the
        // sign of the low part of the constant.
        double z = 0.0, ze = 0.0;
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
            const float dv = fmaxf(v[k] - M, -3.0e38f);
            const double w = (double)__builtin_amdgcn_exp2f(__builtin_fmaf(dv, tp.c_hi, dv * tp.c_lo));
            z += w;
            if (p.typical)  // entropy: sum of w * (l - m) / T, in nats
                ze += w * ((double)dv * tp.inv);
        }
        st.z = block_sum(z, s_d);
        if (p.typical) {
            ze = block_sum(ze, s_d);
            if (threadIdx.x == 0)
                p.row_ent[(size_t)row * p.nchunk + chunk] = ze;
        }
    }
    if (threadIdx.x == 0) {
        static_cast<RowStat *>(p.row_stats)[(size_t)row * p.nchunk + chunk] = st;
        if (rec)
            static_cast<RowX *>(p.row_x)[(size_t)b * K + i] = rx;
    }
}

// Early exit, between the two row-statistics launches: one workgroup per
// sequence runs the tests of positions 0 .. gate_r-1 from the first gate_r
// rows (as the decide pass will, with the same arithmetic) and flags the
// sequences that accepted all of them, whose later rows are still needed.
__global__ __launch_bounds__(kSampleThreads) void sv_sample_gate_kernel(SampleParams p)
{
    __shared__ SeqTests sh;
    const int b = blockIdx.x;
    seq_tests(p, b, temp_of(p, b), p.gate_r, p.gate_r, sh);
    if (threadIdx.x == 0)
        p.gate[b] = sh.n >= p.gate_r ? 1 : 0;
}

template <bool VEC>
__global__ __launch_bounds__(kSampleThreads) void sv_sample_decide_kernel(SampleParams p)
{
    __shared__ SeqTests sh;
    __shared__ double s_part[kDecideMaxSpw][kNWs][2];

    // This workgroup covers sub-chunks sub0 .. sub0 + nsh - 1 of sequence b
    // (the statistics and the tests are done once for all of them).
    const int nsub = (p.V + kSampleSub - 1) / kSampleSub;
    const int spw = p.spw;
    const int ngrp = (nsub + spw - 1) / spw;
    const int b = blockIdx.x / ngrp;
    const int sub0 = (blockIdx.x - b * ngrp) * spw;
    const int nsh = min(spw, nsub - sub0);
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int K = p.K, K1 = K + 1, V = p.V;

    const Temp tp = temp_of(p, b);
    seq_tests(p, b, tp, K1, K, sh);
    const int n = sh.n;
    const float *s_M = sh.M;
    const double *s_Z = sh.Z;
    const int *s_A = sh.A;
    const float *s_tau = sh.tau;
    const double *s_ratio = sh.ratio;
    const double *s_th = sh.th;
    const bool residual = n < K && !p.typical;  // typical: the draw is from p~_n itself
    const float M = s_M[n];
    const double invZ = s_Z[n];
    const int arg = s_A[n];
    const float tau = s_tau[n];

    // 3. Mass of each sub-chunk: residual (or bonus) weights and plain
    //    target mass.
    sub_chunk_masses<VEC>(p.logits + ((size_t)b * K1 + n) * V, p.probs + ((size_t)b * K + n) * V,
                          residual ? 1.0 : 0.0, sub0, nsh, V, M, invZ, tp, arg, tau, s_part);
    __syncthreads();
    if (tid < 2 * nsh) {
        const int j = tid >> 1, c = tid & 1;
        double t = s_part[j][0][c];
#pragma unroll
        for (int w = 1; w < kNWs; ++w)
            t += s_part[j][w][c];
        p.sub_mass[((size_t)b * nsub + sub0 + j) * 2 + c] = t;
    }

    // The first workgroup of the sequence records what the draw needs.
    const int sub = sub0;
    if (sub == 0 && tid == 0) {
        SeqState ss;
        ss.n = n;
        ss.m = M;
        ss.inv_z = invZ;
        ss.inv_t = tp.inv;
        ss.coef = residual ? 1.0 : 0.0;
        ss.greedy = tp.greedy ? 1 : 0;
        ss.arg = arg;
        ss.row = n;
        ss.qrow = residual ? n : 0;
        ss.tree = 0;
        ss.ucol = K;
        ss.tau = tau;
        static_cast<SeqState *>(p.seq_state)[b] = ss;
    }
    if (sub == 0 && p.accept_prob && tid < K)
        p.accept_prob[(size_t)b * K + tid] = (float)s_ratio[tid];
    if (sub == 0 && p.threshold_out && tid < K)
        p.threshold_out[(size_t)b * K + tid] = (float)s_th[tid];
}

// The draw: one workgroup per sequence.  Wave 0 prefix-scans the sub-chunk
// masses in order (DPP scan, 64 sub-chunks at a time) and locates the one
// holding u_K * S; the workgroup then rescans it, each thread owning four
// consecutive entries, with a workgroup prefix scan, and the first entry
// whose cumulative weight exceeds u_K * S is the token.
template <bool VEC>
__global__ __launch_bounds__(kSampleThreads) void sv_sample_pick_kernel(SampleParams p)
{
    __shared__ double s_d[kNWs];
    __shared__ int s_i[kNWs];
    __shared__ int s_cstar, s_mode;
    __shared__ double s_cum, s_target;

    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int K = p.K, K1 = K + 1, V = p.V;
    const int nsub = (V + kSampleSub - 1) / kSampleSub;
    const SeqState ss = static_cast<const SeqState *>(p.seq_state)[b];
    const int n = ss.n;
    const bool residual = ss.coef > 0.0;
    const float M = ss.m;
    const double invZ = ss.inv_z;
    const Temp tp = temp_from_inv(ss.greedy != 0, ss.inv_t);
    const float *lrow = p.logits + ((size_t)b * K1 + ss.row) * V;
    const float *qrow = p.probs ? p.probs + ((size_t)b * p.qrows + ss.qrow) * V : nullptr;

    // The draw's uniform is column K (chain) or 0 (tree): both are requested
    // with the state, before the column is known.
    const float u_chain = p.uniforms[(size_t)b * K1 + K], u_tree = p.uniforms[(size_t)b * K1];
    if (tid < kWave) {
        const double *gmass = p.sub_mass + (size_t)b * nsub * 2;
        constexpr int kRegSub = 4;  // sub-chunk masses held per lane (nsub <= 256)
        double wr[kRegSub], pr[kRegSub];
        const bool in_regs = nsub <= kRegSub * kWave;
        double sw = 0.0, sp = 0.0;
        if (in_regs) {
#pragma unroll
            for (int k = 0; k < kRegSub; ++k) {
                const int c = lane + k * kWave;
                wr[k] = c < nsub ? gmass[2 * c] : 0.0;
                pr[k] = c < nsub ? gmass[2 * c + 1] : 0.0;
            }
#pragma unroll
            for (int k = 0; k < kRegSub; ++k) {
                sw += wr[k];
                sp += pr[k];
            }
        } else {
            for (int c = lane; c < nsub; c += kWave) {
                sw += gmass[2 * c];
                sp += gmass[2 * c + 1];
            }
        }
        double S = wave_sum_f64(sw);
        int mode = 0;  // 0: residual/bonus weights, 1: fallback to p_n
        if (!(S > 0.0)) {
            mode = 1;
            S = wave_sum_f64(sp);
        }
        const float uf = ss.ucol == K ? u_chain : (ss.ucol == 0 ? u_tree : p.uniforms[(size_t)b * K1 + ss.ucol]);
        const double tgt = (double)uf * S;
        double carry = 0.0, cum = 0.0;
        int cstar = -1, lastpos = -1;
        double cum_last = 0.0;
        for (int c0 = 0, k = 0; c0 < nsub; c0 += kWave, ++k) {
            const int c = c0 + lane;
            double mc = 0.0;
            if (in_regs) {
#pragma unroll
                for (int kk = 0; kk < kRegSub; ++kk)
                    if (kk == k)
                        mc = mode ? pr[kk] : wr[kk];
            } else {
                mc = c < nsub ? gmass[2 * c + mode] : 0.0;
            }
            const double incl = wave_inclusive_scan_f64(mc) + carry;
            const uint64_t hit = __ballot(c < nsub && incl > tgt);
            const uint64_t pos = __ballot(c < nsub && mc > 0.0);
            if (pos) {
                const int ll = 63 - __builtin_clzll(pos);
                lastpos = c0 + ll;
                cum_last = readlane_f64(incl - mc, ll);
            }
            if (hit) {
                const int fl = __builtin_ctzll(hit);
                cstar = c0 + fl;
                cum = readlane_f64(incl - mc, fl);
                break;
            }
            carry = readlane_f64(incl, 63);
        }
        int take_last = 0;
        if (cstar < 0) {  // rounding left u*S at or past the total: last positive weight
            take_last = 1;
            cstar = lastpos < 0 ? 0 : lastpos;
            cum = cum_last;
        }
        if (lane == 0) {
            s_cstar = cstar;
            s_cum = cum;
            s_target = tgt;
            s_mode = mode | (take_last << 1);
        }
    }
    __syncthreads();
    const bool use_resid = residual && !(s_mode & 1);
    const bool take_last = (s_mode & 2) != 0;
    const int base = s_cstar * kSampleSub;
    const int cnt = min(kSampleSub, V - base);
    const int e0 = tid * 4;
    float lv[4], qv[4];
    if constexpr (VEC) {
        float4 x = make_float4(-__builtin_inff(), -__builtin_inff(), -__builtin_inff(), -__builtin_inff());
        float4 y = make_float4(0.f, 0.f, 0.f, 0.f);
        if (e0 < cnt) {  // cnt is a multiple of 4 on this path
            x = *reinterpret_cast<const float4 *>(lrow + base + e0);
            if (use_resid)
                y = *reinterpret_cast<const float4 *>(qrow + base + e0);
        }
        lv[0] = x.x; lv[1] = x.y; lv[2] = x.z; lv[3] = x.w;
        qv[0] = y.x; qv[1] = y.y; qv[2] = y.z; qv[3] = y.w;
    } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const bool ok = e0 + k < cnt;
            lv[k] = ok ? lrow[base + e0 + k] : -__builtin_inff();
            qv[k] = (ok && use_resid) ? qrow[base + e0 + k] : 0.0f;
        }
    }
    double wv[4];
    double seg = 0.0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        wv[k] = weight(lv[k], qv[k], base + e0 + k, M, invZ, use_resid ? ss.coef : 0.0, tp, ss.arg, ss.tau);
        seg += wv[k];
    }
    // Exclusive prefix of the run sums across the workgroup.
    const double incl = wave_inclusive_scan_f64(seg);
    if (lane == 63)
        s_d[wave] = incl;
    __syncthreads();
    double before = 0.0;
    for (int i = 0; i < wave; ++i)
        before += s_d[i];
    double run = s_cum + before + (incl - seg);
    int cand = 0x7FFFFFFF, lastpos = -1;
    const double tgt = s_target;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        if (wv[k] > 0.0)
            lastpos = base + e0 + k;
        run += wv[k];
        if (cand == 0x7FFFFFFF && run > tgt && wv[k] > 0.0)
            cand = base + e0 + k;
    }
    const int wmin = wave_min_i32(cand), wmax = wave_max_i32(lastpos);
    if (lane == 0)
        s_i[wave] = wmin;
    __syncthreads();
    int best = s_i[0];
    for (int i = 1; i < kNWs; ++i)
        best = min(best, s_i[i]);
    __syncthreads();
    if (lane == 0)
        s_i[wave] = wmax;
    __syncthreads();
    int last = s_i[0];
    for (int i = 1; i < kNWs; ++i)
        last = max(last, s_i[i]);
    const int token = (!take_last && best != 0x7FFFFFFF) ? best : last;

    if (ss.tree) {
        if (tid == 0) {
            p.out_tokens[(size_t)b * K1 + n] = token;
            p.num_accepted[b] = n;
        }
        return;
    }
    if (tid < K1) {
        int32_t v;
        if (tid < n)
            v = clamp_token(p.tokens[(size_t)b * K + tid], V);
        else
            v = (tid == n) ? token : -1;
        p.out_tokens[(size_t)b * K1 + tid] = v;
    }
    if (tid == 0)
        p.num_accepted[b] = n;
}

// ------------------------------------------------------------ tree verify
//
// A draft tree of N BFS-ordered nodes per sequence ("KV Cache + Speculative
// Decoding" 8.2): target row c holds the logits after node c's path, draft
// row c the distribution q_c that c's children were drawn from.  The walk
// starts at the root; the children of the current node u are tried in
// order, the k-th (k = 1, 2, ..) accepted iff
//     u_c * q_u(x) < max(0, p_u(x) - C_{k-1} q_u(x)) / Z_k,
// C_0 = 0, Z_1 = 1, Z_k = sum_j max(0, p_u(j) - C_{k-1} q_u(j)),
// C_k = C_{k-1} + Z_k: the rejection step of the chain applied once per
// rejected sibling (for k = 1 this is the chain's test).  The walk moves to
// an accepted child; when none is accepted the final token is drawn from
// max(0, p_u - C q_u) with C the coefficient reached (0 at a leaf: p_u).
// C_k and Z_k depend only on node u's two rows, never on the drafts or
// uniforms, so they are computed for every node before the walk:
//   tree_level  one launch per sibling rank k = 2 .. max_children, grid
//               (vocabulary chunk x node): the chunk partials of
//               Z = sum_j max(0, p_u(j) - C q_u(j)) for every child of rank k
//               (C from the complete sums of its earlier siblings);
//   tree_decide grid (1024-entry sub-chunk x sequence): every workgroup
//               loads the gathered (logit, q) of each node's token, the row
//               statistics and the normalisers in one round trip, walks the
//               tree (one thread), and sums the final weights over its
//               sub-chunk; the first one writes the path and the tokens;
//   pick        the chain's draw, from the row and coefficient the walk left.

// Row maximum and 1 / sum_j exp(l_j - M) of target row `row` (T = 1), merged
// from the chunk statistics by one wave.
__device__ __forceinline__ void tree_row_mz(const SampleParams &p, int row, float &M, double &invZ)
{
    const int lane = threadIdx.x & 63;
    const RowStat *st = static_cast<const RowStat *>(p.row_stats) + (size_t)row * p.nchunk;
    float mloc = -__builtin_inff();
    for (int c = lane; c < p.nchunk; c += kWave)
        mloc = fmaxf(mloc, st[c].m);
    M = wave_max_f32(mloc);
    double zloc = 0.0;
    for (int c = lane; c < p.nchunk; c += kWave) {
        const RowStat r = st[c];
        if (r.z > 0.0)
            zloc += r.z * exp((double)r.m - (double)M);
    }
    invZ = 1.0 / wave_sum_f64(zloc);
}

__device__ __forceinline__ int tree_parent(const SampleParams &p, int b, int c)
{
    const int pc = p.parents[(size_t)b * (p.K + 1) + c];
    return pc < 0 ? 0 : (pc >= c ? c - 1 : pc);  // out-of-contract parents stay in bounds
}

constexpr int kTreeMaxN = 16;

// Parents of sequence b into LDS, clamped into [0, c-1] (the root: -1); one
// load per thread.
__device__ __forceinline__ void tree_load_parents(const SampleParams &p, int b, int *s_par)
{
    const int N = p.K + 1, c = threadIdx.x;
    if (c < N)
        s_par[c] = c == 0 ? -1 : tree_parent(p, b, c);
}

// Rank of node c >= 1 among its siblings (1 for the first child).
__device__ __forceinline__ int tree_rank(const int *s_par, int c)
{
    const int u = s_par[c];
    int r = 1;
    for (int c2 = u + 1; c2 < c; ++c2)
        r += s_par[c2] == u ? 1 : 0;
    return r;
}

// This lane's share of the normaliser of node c's test: chunks lane,
// lane + 64, ... of its partials.  The normaliser is the wave sum of the
// shares (fixed order), the same wherever it is needed.
__device__ __forceinline__ double tree_z_share(const SampleParams &p, int b, int c)
{
    const double *part = p.coefs + ((size_t)b * (p.K + 1) + c) * p.nchunk;
    double z = 0.0;
    for (int i = threadIdx.x & 63; i < p.nchunk; i += kWave)
        z += part[i];
    return z;
}

constexpr int kLevelWaves = 16;                             // waves of a rank's workgroup
constexpr int kLevelSlice = kSampleChunk / kLevelWaves;      // entries per wave: 512
static_assert(kLevelSlice == 8 * kWave, "a slice is eight entries per lane");

// This lane's eight entries of a 512-entry slice starting at entry `base` of
// a row (n of them exist; n may be <= 0): float4 path entries base + lane*4
// + k*256 + i, scalar path base + lane + k*64.  Loads never branch: a
// missing entry reads the row's first and is replaced by `fill`.
template <bool VEC>
__device__ __forceinline__ void load_slice(const float *row, int base, int n, float fill, float (&v)[8])
{
    const int lane = threadIdx.x & 63;
    if constexpr (VEC) {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int e = lane * 4 + k * 256;
            const bool ok = e < n;  // n is a multiple of 4 on this path
            const float4 x = *reinterpret_cast<const float4 *>(row + (ok ? base + e : 0));
            v[4 * k + 0] = ok ? x.x : fill; v[4 * k + 1] = ok ? x.y : fill;
            v[4 * k + 2] = ok ? x.z : fill; v[4 * k + 3] = ok ? x.w : fill;
        }
    } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int e = lane + k * kWave;
            const bool ok = e < n;
            const float x = row[ok ? base + e : 0];
            v[k] = ok ? x : fill;
        }
    }
}

// One sibling rank: grid (vocabulary chunk x sequence), sixteen waves per
// workgroup, wave w on entries [512w, 512w + 512) of the chunk.  For every
// child c of rank `rank` (>= 2) of the sequence, in node order, each wave
// sums over its slice max(0, p_u(j) - C q_u(j)) (u the parent) with
// C = 1 + the normalisers of c's earlier siblings of rank >= 2, i.e. the C
// of c's previous sibling (kept in tree_c by the launch that tested it)
// plus that sibling's normaliser (its chunk partials are complete: they
// belong to an earlier launch).  The waves work independently, each
// requesting a child's row statistics, C terms and slice together; one
// barrier at the end sums the sixteen slices of each child into its chunk
// partial.  The sum of a node's chunk partials is the normaliser Z of its
// test.
template <bool VEC>
__global__ __launch_bounds__(kSampleThreads * 4) void sv_tree_level_kernel(SampleParams p, int rank)
{
    __shared__ int s_par[kTreeMaxN], s_pv[kTreeMaxN], s_kid[kTreeMaxN], s_prev[kTreeMaxN];
    __shared__ int s_nk;
    __shared__ double s_part[kLevelWaves][kTreeMaxN];
    __shared__ float s_M[kTreeMaxN];                 // per child of the rank: parent row maximum,
    __shared__ double s_iZ[kTreeMaxN], s_C[kTreeMaxN];  // its 1/Z, and the child's C
    const int N = p.K + 1;
    const int chunk = blockIdx.x % p.nchunk;
    const int b = blockIdx.x / p.nchunk;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    tree_load_parents(p, b, s_par);
    __syncthreads();
    // thread c: node c's sibling rank and its previous sibling (the child of
    // the same parent just before it; rank - 1)
    bool mine = false;
    if (tid >= 1 && tid < N) {
        const int u = s_par[tid];
        int r = 1, prev = -1;
        for (int c2 = u + 1; c2 < tid; ++c2)
            if (s_par[c2] == u) {
                ++r;
                prev = c2;
            }
        s_pv[tid] = prev;
        mine = r == rank;
    }
    if (wave == 0) {  // the children of this rank in node order (N <= 16 < 64)
        const uint64_t m = __ballot(mine);
        if (mine) {
            const int pos = __builtin_popcountll(m & ((1ull << lane) - 1ull));
            s_kid[pos] = lane;
            s_prev[pos] = s_pv[lane];
        }
        if (lane == 0)
            s_nk = __builtin_popcountll(m);
    }
    __syncthreads();
    const int nk = __builtin_amdgcn_readfirstlane(s_nk);
    if (nk == 0)
        return;  // uniform over the workgroup
    const int base = chunk * kSampleChunk + wave * kLevelSlice;
    const int n = min(kLevelSlice, p.V - base);
    const Temp t1 = temp_from_inv(false, 1.0);
    const bool fast = p.nchunk <= kWave;  // one chunk statistic per lane
    const bool hp = rank > 2;             // the previous sibling has its own test (rank >= 2)
    // Child j's slices, all requested together; the next child's are in
    // flight while this one is summed.
    struct Fetch {
        float v[8], w[8];
    };
    auto fetch = [&](int j, Fetch &f) {
        const int c = __builtin_amdgcn_readfirstlane(s_kid[j]);
        const int row = b * N + __builtin_amdgcn_readfirstlane(s_par[c]);
        load_slice<VEC>(p.logits + (size_t)row * p.V, base, n, -__builtin_inff(), f.v);
        load_slice<VEC>(p.probs + (size_t)row * p.V, base, n, 0.0f, f.w);
    };
    auto finish = [&](int j, const Fetch &f) {
        const float M = s_M[j];
        const double invZ = s_iZ[j], C = s_C[j];
        double acc = 0.0;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int e = VEC ? lane * 4 + (k >> 2) * 256 + (k & 3) : lane + k * kWave;
            const double r = target_prob_fast(f.v[k], base + e, M, invZ, t1, 0, -__builtin_inff()) - C * (double)f.w[k];
            acc += r > 0.0 ? r : 0.0;
        }
        acc = wave_sum_f64(acc);
        if (lane == 0)
            s_part[wave][j] = acc;
    };
    Fetch fa, fb;
    fetch(0, fa);  // in flight during the per-child pass
    // Per child j of this rank (wave j; nk <= 15 < kLevelWaves): its parent
    // row's maximum and 1/Z and the child's C, once for the workgroup rather
    // than in every wave (the same reductions on the same values).
    if (wave < nk) {
        const int c = __builtin_amdgcn_readfirstlane(s_kid[wave]);
        const int prev = __builtin_amdgcn_readfirstlane(s_prev[wave]);
        const int row = b * N + __builtin_amdgcn_readfirstlane(s_par[c]);
        const int pn = hp ? prev : c;  // (c: a valid address when unused)
        const RowStat st = load_or(static_cast<const RowStat *>(p.row_stats), (size_t)row * p.nchunk + lane,
                                   fast && lane < p.nchunk, RowStat{-__builtin_inff(), 0, 0.0});
        const double zp = load_or(p.coefs, ((size_t)b * N + pn) * p.nchunk + lane, fast && hp && lane < p.nchunk, 0.0);
        const double cp = load_or(p.tree_c, (size_t)b * N + pn, hp, 1.0);
        float M;
        double invZ;
        if (fast) {
            M = wave_max_f32(st.m);
            const double z = st.z > 0.0 ? st.z * exp((double)st.m - (double)M) : 0.0;
            invZ = 1.0 / wave_sum_f64(z);
        } else {
            tree_row_mz(p, row, M, invZ);
        }
        const double C = hp ? cp + wave_sum_f64(fast ? zp : tree_z_share(p, b, prev)) : 1.0;
        if (lane == 0) {
            s_M[wave] = M;
            s_iZ[wave] = invZ;
            s_C[wave] = C;
            if (chunk == 0)
                p.tree_c[(size_t)b * N + c] = C;  // for c's next sibling
        }
    }
    __syncthreads();
    for (int j = 0; j < nk; j += 2) {
        if (j + 1 < nk)
            fetch(j + 1, fb);
        finish(j, fa);
        if (j + 1 < nk) {
            if (j + 2 < nk)
                fetch(j + 2, fa);
            finish(j + 1, fb);
        }
    }
    __syncthreads();
    if (tid < nk) {
        double z = 0.0;
#pragma unroll
        for (int w2 = 0; w2 < kLevelWaves; ++w2)
            z += s_part[w2][tid];
        p.coefs[((size_t)b * N + s_kid[tid]) * p.nchunk + chunk] = z;
    }
}

template <bool VEC>
__global__ __launch_bounds__(kSampleThreads) void sv_tree_decide_kernel(SampleParams p)
{
    constexpr int kMaxN = kTreeMaxN;
    __shared__ float s_M[kMaxN], s_l[kMaxN], s_q[kMaxN], s_u[kMaxN];
    __shared__ double s_iZ[kMaxN];
    __shared__ int s_par[kMaxN], s_tok[kMaxN];
    __shared__ double s_z[kMaxN];     // normaliser of node c's test (rank >= 2)
    __shared__ int s_rank[kMaxN];
    __shared__ double s_ratio[kMaxN];
    __shared__ int s_path[kMaxN];
    __shared__ int s_n, s_t;
    __shared__ double s_coef;
    __shared__ double s_part[kDecideMaxSpw][kNWs][2];

    const int N = p.K + 1, V = p.V;
    // This workgroup covers sub-chunks sub0 .. sub0 + nsh - 1 of sequence b
    // (the walk is done once for all of them).
    const int nsub = (V + kSampleSub - 1) / kSampleSub;
    const int spw = p.spw;
    const int ngrp = (nsub + spw - 1) / spw;
    const int b = blockIdx.x / ngrp;
    const int sub0 = (blockIdx.x - b * ngrp) * spw;
    const int nsh = min(spw, nsub - sub0);
    const int sub = sub0;
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const Temp t1 = temp_from_inv(false, 1.0);
    const float ninf = -__builtin_inff();

    // 1. Everything the walk reads, requested together: each node's token,
    //    uniform and gathered (logit, q); the row statistics; the
    //    normalisers of the tests of rank >= 2.
    if (tid < N) {
        const int c = tid;
        s_u[c] = p.uniforms[(size_t)b * N + c];
        s_ratio[c] = __builtin_nan("");
        if (c > 0) {
            const int pc = tree_parent(p, b, c);
            const int x = clamp_token(p.tokens[(size_t)b * N + c], V);
            s_par[c] = pc;
            s_tok[c] = x;
            s_l[c] = p.logits[((size_t)b * N + pc) * V + x];
            s_q[c] = p.probs[((size_t)b * N + pc) * V + x];
        } else {
            s_par[0] = -1;
            s_tok[0] = 0;
        }
    }
    {
        // wave w: the partial shares of nodes w, w + 4, w + 8, w + 12
        double share[kTreeMaxN / kNWs];
#pragma unroll
        for (int i = 0; i < kTreeMaxN / kNWs; ++i) {
            const int c = wave + i * kNWs;
            share[i] = (c > 0 && c < N) ? tree_z_share(p, b, c) : 0.0;  // read only where the rank is >= 2
        }
#pragma unroll
        for (int i = 0; i < kTreeMaxN / kNWs; ++i) {
            const int c = wave + i * kNWs;
            const double z = wave_sum_f64(share[i]);
            if (lane == 0 && c < N)
                s_z[c] = z;
        }
    }
    if (p.nchunk <= kWave) {
        // wave w: rows w, w + 4, w + 8, w + 12, their chunk statistics
        // requested together (lane = chunk, as in tree_row_mz)
        RowStat st[kTreeMaxN / kNWs];
#pragma unroll
        for (int i = 0; i < kTreeMaxN / kNWs; ++i) {
            const int r = wave + i * kNWs;
            st[i] = RowStat{-__builtin_inff(), 0, 0.0};
            if (r < N && lane < p.nchunk)
                st[i] = static_cast<const RowStat *>(p.row_stats)[((size_t)b * N + r) * p.nchunk + lane];
        }
#pragma unroll
        for (int i = 0; i < kTreeMaxN / kNWs; ++i) {
            const int r = wave + i * kNWs;
            const float M = wave_max_f32(st[i].m);
            const double z = (lane < p.nchunk && st[i].z > 0.0) ? st[i].z * exp((double)st[i].m - (double)M) : 0.0;
            const double iZ = 1.0 / wave_sum_f64(z);
            if (lane == 0 && r < N) {
                s_M[r] = M;
                s_iZ[r] = iZ;
            }
        }
    } else {
        for (int r = wave; r < N; r += kNWs) {
            float M;
            double iZ;
            tree_row_mz(p, b * N + r, M, iZ);
            if (lane == 0) {
                s_M[r] = M;
                s_iZ[r] = iZ;
            }
        }
    }
    __syncthreads();
    if (tid < N)
        s_rank[tid] = tid > 0 ? tree_rank(s_par, tid) : 0;
    __syncthreads();

    // 2. The walk.
    if (tid == 0) {
        int node = 0, depth = 0;
        double C = 0.0;
        for (;;) {
            int next = -1;
            C = 0.0;
            for (int c = node + 1; c < N; ++c) {
                if (s_par[c] != node || s_rank[c] > p.tree_max_children)
                    continue;  // not a child, or beyond the ranks prepared
                const double qx = (double)s_q[c];
                const double px = target_prob(s_l[c], 0, s_M[node], s_iZ[node], t1, 0, ninf);
                double a;
                if (s_rank[c] == 1) {
                    a = px;
                } else {
                    const double Zk = s_z[c];  // written by tree_level for ranks 2 .. max_children
                    const double rx = px - C * qx;
                    a = (Zk > 0.0 && rx > 0.0) ? rx / Zk : 0.0;
                }
                s_ratio[c] = qx > 0.0 ? fmin(1.0, a / qx) : (a > 0.0 ? 1.0 : 0.0);
                if ((double)s_u[c] * qx < a) {
                    next = c;
                    break;
                }
                C = (s_rank[c] == 1) ? 1.0 : C + s_z[c];
            }
            if (next < 0)
                break;
            s_path[depth++] = next;
            node = next;
        }
        s_n = depth;
        s_t = node;
        s_coef = C;
    }
    __syncthreads();
    const int n = s_n, t = s_t;
    const double coef = s_coef;
    const float M = s_M[t];
    const double invZ = s_iZ[t];

    // 3. Mass of each sub-chunk: final weights and plain target mass.
    sub_chunk_masses<VEC>(p.logits + ((size_t)b * N + t) * V, p.probs + ((size_t)b * N + t) * V, coef, sub0, nsh,
                          V, M, invZ, t1, 0, ninf, s_part);
    __syncthreads();
    if (tid < 2 * nsh) {
        const int j = tid >> 1, c = tid & 1;
        double acc = s_part[j][0][c];
#pragma unroll
        for (int w = 1; w < kNWs; ++w)
            acc += s_part[j][w][c];
        p.sub_mass[((size_t)b * nsub + sub0 + j) * 2 + c] = acc;
    }

    // 4. The first workgroup of the sequence writes the state of the draw and
    //    every output but the drawn token.
    if (sub == 0) {
        if (tid == 0) {
            SeqState ss;
            ss.n = n;
            ss.m = M;
            ss.inv_z = invZ;
            ss.inv_t = 1.0;
            ss.coef = coef;
            ss.greedy = 0;
            ss.arg = 0;
            ss.row = t;
            ss.qrow = t;
            ss.tree = 1;
            ss.ucol = 0;
            ss.tau = ninf;
            static_cast<SeqState *>(p.seq_state)[b] = ss;
        }
        if (tid < N) {
            const size_t o = (size_t)b * N + tid;
            if (tid < n) {
                p.out_tokens[o] = s_tok[s_path[tid]];
                p.path[o] = s_path[tid];
            } else {
                if (tid > n)
                    p.out_tokens[o] = -1;  // position n: the drawn token, written by pick
                p.path[o] = -1;
            }
            if (p.accept_prob)
                p.accept_prob[o] = (float)s_ratio[tid];
        }
    }
}

__global__ void sv_fill_zero_kernel(uint4 *p, size_t n16, unsigned char *tail, size_t ntail)
{
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
        p[i] = make_uint4(0u, 0u, 0u, 0u);
    if (blockIdx.x == 0)
        for (size_t i = threadIdx.x; i < ntail; i += blockDim.x)
            tail[i] = 0;
}

// Workgroups of one decide kernel that the device holds at once: compute
// units times the kernel's resident workgroups per unit, queried on first use
// per device and kernel (slot `which`) and kept.  0 if the query fails.
constexpr int kSpwMaxDevices = 64;
std::atomic<int> g_resident[kSpwMaxDevices][4];

long long resident_workgroups(const void *kernel, int which, hipStream_t stream)
{
    int dev = 0;
    if ((stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev)) != hipSuccess || dev < 0 ||
        dev >= kSpwMaxDevices)
        return 0;
    int r = g_resident[dev][which].load(std::memory_order_relaxed);
    if (r == 0) {
        int cus = 0, per = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kernel, kSampleThreads, 0) != hipSuccess ||
            cus <= 0 || per <= 0)
            return 0;
        r = cus * per;
        g_resident[dev][which].store(r, std::memory_order_relaxed);
    }
    return r;
}

// Sub-chunks per decide workgroup for `total` (sequence, sub-chunk) pairs:
// the fewest that keep the grid within one resident round (2048 workgroups
// assumed if the occupancy query fails), at most kDecideMaxSpw.
int decide_spw(long long total, const void *kernel, int which, hipStream_t stream)
{
    long long slots = resident_workgroups(kernel, which, stream);
    if (slots <= 0)
        slots = 2048;
    const long long want = (total + slots - 1) / slots;
    return (int)(want < 1 ? 1 : (want > kDecideMaxSpw ? kDecideMaxSpw : want));
}

}  // namespace

hipError_t launch_sample(const SampleParams &p0, hipStream_t stream)
{
    // Decide: one workgroup per sub-chunk while the grid fits in one round of
    // resident workgroups; larger batches give each workgroup consecutive
    // sub-chunks (up to kDecideMaxSpw), so that the statistics merge and the
    // tests (two dependent round trips) run once per workgroup and the whole
    // grid stays resident.
    SampleParams p = p0;
    const long long nsub = (p.V + kSampleSub - 1) / kSampleSub;
    p.spw = decide_spw(nsub * p.B, p.vec4 ? (const void *)sv_sample_decide_kernel<true>
                                          : (const void *)sv_sample_decide_kernel<false>,
                       p.vec4 ? 0 : 1, stream);
    const int K1 = p.K + 1;
    p.row_lo = 0;
    p.row_cnt = K1;
    p.gate_r = 0;
    // Early exit ("50 | Speculative Decoding" 3.1: verification stops at the
    // first rejected draft, so the target rows after it never reach the
    // output): for large batches the row statistics run as two launches,
    // rows 0 .. R-1 of every sequence, then (after a one-workgroup-per-
    // sequence launch that flags the sequences whose drafts 0 .. R-1 were all
    // accepted) rows R .. K of the flagged sequences, when no output needs
    // every row (acceptance ratios, typical acceptance, top-p cuts).  The
    // decide pass uses the statistics only of rows up to the first rejection
    // (those of a skipped row may be stale and never reach the output).
    const bool gate = !p.tree && !p.typical && !p.row_cut && !p.accept_prob && !p.threshold_out && K1 >= 4 &&
                      (double)p.B * K1 * p.V * 4.0 >= kGateMinBytes;
    // R = max(2, 3(K+1)/8): with a per-draft acceptance rate a the rows read
    // per sequence are R + (K+1-R) a^R, which this R keeps within a few per
    // cent of the best for a in 0.5 .. 0.9 (ragged 64-sequence batch, K = 7:
    // sampler 63.3-64.3 us with R = 4, 60.5-61.1 with R = 3, 59.0-60.0 with R = 2)
    const int R = max(2, (3 * K1) / 8);
    SampleParams pa = p, pb = p;
    pa.row_cnt = R;
    pb.row_lo = R;
    pb.row_cnt = K1 - R;
    pb.gate_r = R;
    const dim3 gg((unsigned)p.B);
    const dim3 block(kSampleThreads);
    const dim3 g1((unsigned)(p.nchunk * p.B * K1));
    const dim3 ga((unsigned)(p.nchunk * p.B * R));
    const dim3 gb((unsigned)(p.nchunk * p.B * (K1 - R)));
    const dim3 g2((unsigned)(((nsub + p.spw - 1) / p.spw) * p.B));
    const dim3 g3((unsigned)p.B);
    const dim3 gc((unsigned)(p.B * K1));
    const dim3 gh = g1;
    if (p.vec4) {
        if (gate) {
            hipLaunchKernelGGL((sv_sample_rowstats_kernel<true, true>), ga, block, 0, stream, pa);
            hipLaunchKernelGGL(sv_sample_gate_kernel, gg, block, 0, stream, pb);
            hipLaunchKernelGGL((sv_sample_rowstats_kernel<true, true>), gb, block, 0, stream, pb);
        } else {
            hipLaunchKernelGGL((sv_sample_rowstats_kernel<true, false>), g1, block, 0, stream, p);
        }
        if (p.row_cut) {
            hipLaunchKernelGGL(sv_sample_cut_hist_kernel<true>, gh, block, 0, stream, p);
            hipLaunchKernelGGL(sv_sample_cut_kernel<true>, gc, dim3(kCutThreads), 0, stream, p);
        }
        hipLaunchKernelGGL(sv_sample_decide_kernel<true>, g2, block, 0, stream, p);
        hipLaunchKernelGGL(sv_sample_pick_kernel<true>, g3, block, 0, stream, p);
    } else {
        if (gate) {
            hipLaunchKernelGGL((sv_sample_rowstats_kernel<false, true>), ga, block, 0, stream, pa);
            hipLaunchKernelGGL(sv_sample_gate_kernel, gg, block, 0, stream, pb);
            hipLaunchKernelGGL((sv_sample_rowstats_kernel<false, true>), gb, block, 0, stream, pb);
        } else {
            hipLaunchKernelGGL((sv_sample_rowstats_kernel<false, false>), g1, block, 0, stream, p);
        }
        if (p.row_cut) {
            hipLaunchKernelGGL(sv_sample_cut_hist_kernel<false>, gh, block, 0, stream, p);
            hipLaunchKernelGGL(sv_sample_cut_kernel<false>, gc, dim3(kCutThreads), 0, stream, p);
        }
        hipLaunchKernelGGL(sv_sample_decide_kernel<false>, g2, block, 0, stream, p);
        hipLaunchKernelGGL(sv_sample_pick_kernel<false>, g3, block, 0, stream, p);
    }
    return hipGetLastError();
}

hipError_t launch_sample_tree(const SampleParams &p0, hipStream_t stream)
{
    SampleParams p = p0;  // decide workgroups per sequence: as in launch_sample
    const long long nsub = (p.V + kSampleSub - 1) / kSampleSub;
    p.spw = decide_spw(nsub * p.B, p.vec4 ? (const void *)sv_tree_decide_kernel<true>
                                          : (const void *)sv_tree_decide_kernel<false>,
                       p.vec4 ? 2 : 3, stream);
    const dim3 block(kSampleThreads);
    const int N = p.K + 1;
    p.row_lo = 0;  // every row of every sequence
    p.row_cnt = N;
    p.gate_r = 0;
    const dim3 g1((unsigned)(p.nchunk * p.B * N));
    const dim3 gl((unsigned)(p.nchunk * p.B));
    const dim3 g2((unsigned)(((nsub + p.spw - 1) / p.spw) * p.B));
    const dim3 g3((unsigned)p.B);
    if (p.vec4) {
        hipLaunchKernelGGL((sv_sample_rowstats_kernel<true, false>), g1, block, 0, stream, p);
        for (int r = 2; r <= p.tree_max_children; ++r)
            hipLaunchKernelGGL(sv_tree_level_kernel<true>, gl, dim3(kSampleThreads * 4), 0, stream, p, r);
        hipLaunchKernelGGL(sv_tree_decide_kernel<true>, g2, block, 0, stream, p);
        hipLaunchKernelGGL(sv_sample_pick_kernel<true>, g3, block, 0, stream, p);
    } else {
        hipLaunchKernelGGL((sv_sample_rowstats_kernel<false, false>), g1, block, 0, stream, p);
        for (int r = 2; r <= p.tree_max_children; ++r)
            hipLaunchKernelGGL(sv_tree_level_kernel<false>, gl, dim3(kSampleThreads * 4), 0, stream, p, r);
        hipLaunchKernelGGL(sv_tree_decide_kernel<false>, g2, block, 0, stream, p);
        hipLaunchKernelGGL(sv_sample_pick_kernel<false>, g3, block, 0, stream, p);
    }
    return hipGetLastError();
}

hipError_t launch_clear(void *ptr, size_t bytes, hipStream_t stream)
{
    if (bytes == 0)
        return hipSuccess;
    const size_t n16 = bytes / 16;
    const size_t ntail = bytes - n16 * 16;
    size_t blocks = (n16 + 255) / 256;
    if (blocks < 1)
        blocks = 1;
    if (blocks > 4096)
        blocks = 4096;
    hipLaunchKernelGGL(sv_fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<uint4 *>(ptr), n16, static_cast<unsigned char *>(ptr) + n16 * 16, ntail);
    return hipGetLastError();
}

}  // namespace sv
