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
// The acceptance tests run in fp64; the weights take fp32 exp of an exactly
// split argument (about 1e-7 relative) and every sum runs in fp64, so the
// decisions agree with an exact evaluation except within ~1e-7 of a
// threshold.
#include "sv_device.hpp"
#include "sv_internal.hpp"

namespace sv {
namespace {

constexpr int kPer = kSampleChunk / kSampleThreads;  // 32 entries per thread
constexpr int kNWs = kSampleThreads / kWave;
static_assert(kSampleSub == 4 * kSampleThreads, "a sub-chunk is four entries per thread");

struct RowStat {
    float m;
    float pad;
    double z;
};

// Target logit and draft probability of draft token x_i.
struct RowX {
    float lx;
    float qx;
};

// What the draw of one sequence needs from the decide pass.
struct SeqState {
    int n;       // accepted drafts
    float m;     // max logit of row n
    double inv_z;  // 1 / sum_j exp(l_j - m) of row n
};

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

template <bool VEC>
__global__ __launch_bounds__(kSampleThreads) void sv_sample_rowstats_kernel(SampleParams p)
{
    __shared__ float s_f[kNWs];
    __shared__ double s_d[kNWs];
    const int row = blockIdx.x / p.nchunk;
    const int chunk = blockIdx.x - row * p.nchunk;
    const int K = p.K, K1 = K + 1;
    const int b = row / K1, i = row - b * K1;
    const int base = chunk * kSampleChunk;
    const int n = min(kSampleChunk, p.V - base);
    float v[kPer];
    load_chunk<VEC>(p.logits + (size_t)row * p.V + base, n, -__builtin_inff(), v);
    // x_i's own entries, fetched while the chunk streams in.
    const bool rec = chunk == 0 && i < K;
    RowX rx{0.0f, 0.0f};
    if (rec) {
        const int x = clamp_token(p.tokens[(size_t)b * K + i], p.V);
        rx.lx = p.logits[(size_t)row * p.V + x];
        rx.qx = p.probs[((size_t)b * K + i) * p.V + x];
    }
    float mx = v[0];
#pragma unroll
    for (int k = 1; k < kPer; ++k)
        mx = fmaxf(mx, v[k]);
    const float M = block_max(mx, s_f);
    // exp(v - M) = 2^((v - M) log2 e) with the hardware exp2; terms summed in
    // fp64 (the rounding of the scaled argument, |v - M| * 2^-24 relative,
    // is largest for the terms that matter least).
    double z = 0.0;
#pragma unroll
    for (int k = 0; k < kPer; ++k)
        z += (double)__builtin_amdgcn_exp2f((v[k] - M) * kLog2e);
    z = block_sum(z, s_d);
    if (threadIdx.x == 0) {
        RowStat st;
        st.m = M;
        st.pad = 0.0f;
        st.z = z;
        static_cast<RowStat *>(p.row_stats)[(size_t)row * p.nchunk + chunk] = st;
        if (rec)
            static_cast<RowX *>(p.row_x)[(size_t)b * K + i] = rx;
    }
}

// Target probability of entry j from its logit, the row maximum M and 1/Z,
// to about one fp32 ulp: the difference l - M is split exactly into hi + lo
// (TwoSum), exp(hi) comes from the accurate fp32 exp, exp(lo) = 1 + lo to
// second order (|lo| <= ulp(hi)/2), and the products are taken in fp64.
__device__ __forceinline__ double target_prob_fast(float l, float M, double invZ)
{
    const float hi = l - M;
    if (!(hi > -104.0f))
        return 0.0;  // underflows in fp32 (and catches l = -inf)
    const float bb = hi - l;
    const float lo = (l - (hi - bb)) + (-M - bb);
    return (double)expf(hi) * (1.0 + (double)lo) * invZ;
}

// Same quantity in fp64 throughout (used for the K acceptance tests).
__device__ __forceinline__ double target_prob(float l, float M, double invZ)
{
    return exp((double)l - (double)M) * invZ;
}

// Weight of entry j of the chosen row: the residual max(0, p - q) after a
// rejection, p itself for the bonus row or the zero-mass fallback.
__device__ __forceinline__ double weight(float l, float q, float M, double invZ, bool residual)
{
    const double pj = target_prob_fast(l, M, invZ);
    if (!residual)
        return pj;
    const double r = pj - (double)q;
    return r > 0.0 ? r : 0.0;
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

template <bool VEC>
__global__ __launch_bounds__(kSampleThreads) void sv_sample_decide_kernel(SampleParams p)
{
    __shared__ float s_M[16];
    __shared__ double s_Z[16];
    __shared__ double s_ratio[16];
    __shared__ int s_acc[16];
    __shared__ int s_n;
    __shared__ double s_part[kNWs][2];

    const int nsub = (p.V + kSampleSub - 1) / kSampleSub;
    const int b = blockIdx.x / nsub;
    const int sub = blockIdx.x - b * nsub;
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int K = p.K, K1 = K + 1, V = p.V;

    // 1. Row statistics of the K+1 rows of this sequence (one wave per row,
    //    lanes over vocabulary chunks) and the draft tokens' entries, all
    //    requested together.
    RowX rx{0.0f, 0.0f};
    float u = 0.0f;
    if (tid < K) {
        rx = static_cast<const RowX *>(p.row_x)[(size_t)b * K + tid];
        u = p.uniforms[(size_t)b * K1 + tid];
    }
    for (int i = wave; i < K1; i += kNWs) {
        const RowStat *st = static_cast<const RowStat *>(p.row_stats) + (size_t)(b * K1 + i) * p.nchunk;
        float mloc = -__builtin_inff();
        for (int c = lane; c < p.nchunk; c += kWave)
            mloc = fmaxf(mloc, st[c].m);
        const float M = wave_max_f32(mloc);
        double zloc = 0.0;
        for (int c = lane; c < p.nchunk; c += kWave) {
            const RowStat r = st[c];
            zloc += r.z * exp((double)r.m - (double)M);
        }
        const double Z = wave_sum_f64(zloc);
        if (lane == 0) {
            s_M[i] = M;
            s_Z[i] = Z;
        }
    }
    __syncthreads();
    // 2. Acceptance tests u_i * q_i(x_i) < p_i(x_i).
    if (tid < K) {
        const double a = target_prob(rx.lx, s_M[tid], 1.0 / s_Z[tid]);
        const double c = (double)rx.qx;
        s_acc[tid] = ((double)u * c < a) ? 1 : 0;
        s_ratio[tid] = c > 0.0 ? fmin(1.0, a / c) : (a > 0.0 ? 1.0 : 0.0);
    }
    __syncthreads();
    if (tid == 0) {
        int n = K;
        for (int i = 0; i < K; ++i)
            if (!s_acc[i]) {
                n = i;
                break;
            }
        s_n = n;
    }
    __syncthreads();
    const int n = s_n;
    const bool residual = n < K;
    const float M = s_M[n];
    const double invZ = 1.0 / s_Z[n];

    // 3. Mass of this sub-chunk: residual (or bonus) weights and plain
    //    target mass.
    const int base = sub * kSampleSub;
    const int cnt = min(kSampleSub, V - base);
    float lv[4], qv[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    load_sub<VEC>(p.logits + ((size_t)b * K1 + n) * V + base, cnt, -__builtin_inff(), lv);
    if (residual)
        load_sub<VEC>(p.probs + ((size_t)b * K + n) * V + base, cnt, 0.0f, qv);
    double sw = 0.0, sp = 0.0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const double pj = target_prob_fast(lv[k], M, invZ);
        sp += pj;
        if (residual) {
            const double r = pj - (double)qv[k];
            sw += r > 0.0 ? r : 0.0;
        } else {
            sw += pj;
        }
    }
    sw = wave_sum_f64(sw);
    sp = wave_sum_f64(sp);
    if (lane == 0) {
        s_part[wave][0] = sw;
        s_part[wave][1] = sp;
    }
    __syncthreads();
    if (tid < 2) {
        double t = s_part[0][tid];
#pragma unroll
        for (int w = 1; w < kNWs; ++w)
            t += s_part[w][tid];
        p.sub_mass[((size_t)b * nsub + sub) * 2 + tid] = t;
    }

    // The first workgroup of the sequence records what the draw needs.
    if (sub == 0 && tid == 0) {
        SeqState ss;
        ss.n = n;
        ss.m = M;
        ss.inv_z = invZ;
        static_cast<SeqState *>(p.seq_state)[b] = ss;
    }
    if (sub == 0 && p.accept_prob && tid < K)
        p.accept_prob[(size_t)b * K + tid] = (float)s_ratio[tid];
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
    const bool residual = n < K;
    const float M = ss.m;
    const double invZ = ss.inv_z;
    const float *lrow = p.logits + ((size_t)b * K1 + n) * V;
    const float *qrow = p.probs + ((size_t)b * K + (residual ? n : 0)) * V;

    if (tid < kWave) {
        const double *gmass = p.sub_mass + (size_t)b * nsub * 2;
        double sw = 0.0, sp = 0.0;
        for (int c = lane; c < nsub; c += kWave) {
            sw += gmass[2 * c];
            sp += gmass[2 * c + 1];
        }
        double S = wave_sum_f64(sw);
        int mode = 0;  // 0: residual/bonus weights, 1: fallback to p_n
        if (!(S > 0.0)) {
            mode = 1;
            S = wave_sum_f64(sp);
        }
        const double tgt = (double)p.uniforms[(size_t)b * K1 + K] * S;
        double carry = 0.0, cum = 0.0;
        int cstar = -1, lastpos = -1;
        double cum_last = 0.0;
        for (int c0 = 0; c0 < nsub; c0 += kWave) {
            const int c = c0 + lane;
            const double mc = c < nsub ? gmass[2 * c + mode] : 0.0;
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
        wv[k] = weight(lv[k], qv[k], M, invZ, use_resid);
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

__global__ void sv_fill_zero_kernel(uint4 *p, size_t n16, unsigned char *tail, size_t ntail)
{
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
        p[i] = make_uint4(0u, 0u, 0u, 0u);
    if (blockIdx.x == 0)
        for (size_t i = threadIdx.x; i < ntail; i += blockDim.x)
            tail[i] = 0;
}

}  // namespace

hipError_t launch_sample(const SampleParams &p, hipStream_t stream)
{
    const dim3 block(kSampleThreads);
    const dim3 g1((unsigned)(p.nchunk * p.B * (p.K + 1)));
    const dim3 g2((unsigned)(((p.V + kSampleSub - 1) / kSampleSub) * p.B));
    const dim3 g3((unsigned)p.B);
    if (p.vec4) {
        hipLaunchKernelGGL(sv_sample_rowstats_kernel<true>, g1, block, 0, stream, p);
        hipLaunchKernelGGL(sv_sample_decide_kernel<true>, g2, block, 0, stream, p);
        hipLaunchKernelGGL(sv_sample_pick_kernel<true>, g3, block, 0, stream, p);
    } else {
        hipLaunchKernelGGL(sv_sample_rowstats_kernel<false>, g1, block, 0, stream, p);
        hipLaunchKernelGGL(sv_sample_decide_kernel<false>, g2, block, 0, stream, p);
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
