// kvcache.hip -- the paged-cache steps on either side of the verify step, for
// gfx950: appending the K/V of the T verify positions, and the O(1) rollback
// after the sampler ("KV Cache + Speculative Decoding" 6.1 append, 6.2 paged
// data structure, 7.6 the loop and its note that a paged cache rolls back by
// changing table entries; "Lecture 10 - Inference" 9.2).
//
// Append: one thread per four consecutive head dims of one (sequence, verify
// position, KV head) row; position p = L_b - T + t lands in page
// block_table[b][p / 16], slot p % 16.  The stored value is the float itself,
// its bf16 rounding (nearest, ties to even, on the bit pattern) or the E4M3
// code of x / scale[page] (the quotient is an IEEE float division; nearest,
// ties to even; saturating at +-448; NaN -> the NaN code).
// Rollback: one thread per sequence, L_b <- L_b - K + n_b.
// Tree commit: the accepted path's K/V moved next to the root (below).
#include "sv_device.hpp"
#include "sv_internal.hpp"

namespace sv {
namespace {

// float -> bf16 bits, round to nearest even on the bit pattern; NaN stays a
// (quiet) NaN.
__device__ __forceinline__ uint32_t bf16_bits_rne(float x)
{
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u)
        return (u >> 16) | 0x0040u;
    const uint32_t lsb = (u >> 16) & 1u;
    return (u + 0x7FFFu + lsb) >> 16;
}

// float (already divided by the page scale) -> OCP E4M3 code.
__device__ __forceinline__ uint32_t e4m3_code(float q)
{
    const uint32_t u = __builtin_bit_cast(uint32_t, q);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7FFFFFFFu;
    if (a > 0x7F800000u)
        return 0x7Fu;                      // NaN
    if (a >= 0x43E00000u)
        return sign | 0x7Eu;               // |q| >= 448, infinity included: saturate
    if (a < 0x3C800000u) {                 // |q| < 2^-6: multiples of 2^-9 (code = m)
        const float m = __builtin_rintf(__builtin_bit_cast(float, a) * 512.0f);
        return sign | (uint32_t)m;         // m = 8 is the smallest normal, code 0x08
    }
    // normal: keep 3 of the 23 fraction bits, ties to even; a carry moves the
    // exponent, which the field extraction below picks up
    const uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);
    const uint32_t e = (r >> 23) - 120u;   // E4M3 biased exponent (bias 7 vs 127)
    uint32_t code = (e << 3) | ((r >> 20) & 7u);
    if (code > 0x7Eu)
        code = 0x7Eu;
    return sign | code;
}

template <int KVT>
__global__ __launch_bounds__(256) void sv_kv_append_kernel(AppendParams p)
{
    const int quads = p.d >> 2;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t total = (int64_t)p.B * p.T * p.Hkv * quads;
    if (i >= total)
        return;
    const int64_t row = i / quads;
    const int c4 = (int)(i - row * quads);
    const int g = (int)(row % p.Hkv);
    const int64_t bt = row / p.Hkv;
    const int t = (int)(bt % p.T);
    const int b = (int)(bt / p.T);
    int L = p.context_lens[b];
    const int Lmax = p.max_blocks * kBlock;
    L = L < p.T ? p.T : (L > Lmax ? Lmax : L);  // out-of-contract lengths stay in bounds
    const int pos = L - p.T + t;
    int page = p.block_table[(size_t)b * p.max_blocks + pos / kBlock];
    page = page < 0 ? 0 : (page >= p.num_blocks ? p.num_blocks - 1 : page);
    const size_t dst = (((size_t)page * kBlock + pos % kBlock) * p.Hkv + g) * p.d + (size_t)c4 * 4;
    const size_t src = (size_t)row * p.d + (size_t)c4 * 4;
    const float4 kx = *reinterpret_cast<const float4 *>(p.k_new + src);
    const float4 vx = *reinterpret_cast<const float4 *>(p.v_new + src);
    if constexpr (KVT == 0) {
        *reinterpret_cast<float4 *>(static_cast<float *>(p.k_cache) + dst) = kx;
        *reinterpret_cast<float4 *>(static_cast<float *>(p.v_cache) + dst) = vx;
    } else if constexpr (KVT == 1) {
        const uint2 kb = make_uint2(bf16_bits_rne(kx.x) | (bf16_bits_rne(kx.y) << 16),
                                    bf16_bits_rne(kx.z) | (bf16_bits_rne(kx.w) << 16));
        const uint2 vb = make_uint2(bf16_bits_rne(vx.x) | (bf16_bits_rne(vx.y) << 16),
                                    bf16_bits_rne(vx.z) | (bf16_bits_rne(vx.w) << 16));
        *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(p.k_cache) + dst) = kb;
        *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(p.v_cache) + dst) = vb;
    } else {
        const float ks = p.k_scale[page], vs = p.v_scale[page];
        const uint32_t kc = e4m3_code(kx.x / ks) | (e4m3_code(kx.y / ks) << 8) | (e4m3_code(kx.z / ks) << 16) |
                            (e4m3_code(kx.w / ks) << 24);
        const uint32_t vc = e4m3_code(vx.x / vs) | (e4m3_code(vx.y / vs) << 8) | (e4m3_code(vx.z / vs) << 16) |
                            (e4m3_code(vx.w / vs) << 24);
        *reinterpret_cast<uint32_t *>(static_cast<uint8_t *>(p.k_cache) + dst) = kc;
        *reinterpret_cast<uint32_t *>(static_cast<uint8_t *>(p.v_cache) + dst) = vc;
    }
}

__global__ __launch_bounds__(256) void sv_rollback_kernel(const int32_t *num_accepted, int32_t *context_lens,
                                                          int32_t *pages_in_use, int B, int K)
{
    const int b = blockIdx.x * 256 + threadIdx.x;
    if (b >= B)
        return;
    int n = num_accepted[b];
    n = n < 0 ? 0 : (n > K ? K : n);
    int L = context_lens[b] - K + n;
    L = L < 0 ? 0 : L;
    context_lens[b] = L;
    if (pages_in_use)
        pages_in_use[b] = (L + kBlock - 1) / kBlock;
}

// ------------------------------------------------------------- tree commit
//
// After tree verification the root (position base = L - N) stays and the
// accepted path's nodes move from base + path[i] to base + 1 + i.  One
// workgroup per (sequence, KV head) reads every moved row (K and V, d
// elements) into registers, then writes them after a barrier, since a
// destination can be another move's source.  E4M3 values that change page
// are re-encoded for the destination page: decode * scale_src in float, then
// the append's encoder of x / scale_dst.  The lengths are updated by a second
// launch, after every workgroup has read them.
constexpr int kCommitThreads = 256;
constexpr int kCommitPer = 4;  // (node, quad) pairs per thread: N-1 <= 15 nodes x d/4 <= 64 quads

__device__ __forceinline__ float e4m3_value(uint32_t code)
{
    return __builtin_amdgcn_cvt_f32_fp8((int)code, 0);
}

template <int KVT>
__global__ __launch_bounds__(kCommitThreads) void sv_tree_commit_kernel(TreeCommitParams p)
{
    const int b = blockIdx.x / p.Hkv, g = blockIdx.x - (blockIdx.x / p.Hkv) * p.Hkv;
    const int N = p.N, quads = p.d >> 2;
    const int Lmax = p.max_blocks * kBlock;
    int L = p.context_lens[b];
    L = L < N ? N : (L > Lmax ? Lmax : L);
    int n = p.num_accepted[b];
    n = n < 0 ? 0 : (n > N - 1 ? N - 1 : n);
    const int base = L - N;
    auto page_of = [&](int pos) {
        const int pg = p.block_table[(size_t)b * p.max_blocks + pos / kBlock];
        return pg < 0 ? 0 : (pg >= p.num_blocks ? p.num_blocks - 1 : pg);
    };
    auto row_off = [&](int page, int pos) {
        return (((size_t)page * kBlock + pos % kBlock) * p.Hkv + g) * p.d;
    };
    uint4 kx[kCommitPer], vx[kCommitPer];
    int src_page[kCommitPer];
#pragma unroll
    for (int j = 0; j < kCommitPer; ++j) {
        const int idx = threadIdx.x + j * kCommitThreads;
        src_page[j] = 0;
        kx[j] = vx[j] = make_uint4(0u, 0u, 0u, 0u);
        if (idx < n * quads) {
            const int i = idx / quads, c4 = idx - i * quads;
            int c = p.path[(size_t)b * N + i];
            c = c < 1 ? 1 : (c > N - 1 ? N - 1 : c);
            const int ps = base + c;
            const int pg = page_of(ps);
            src_page[j] = pg;
            const size_t e = row_off(pg, ps) + (size_t)c4 * 4;
            if constexpr (KVT == 0) {
                kx[j] = *reinterpret_cast<const uint4 *>(static_cast<const float *>(p.k_cache) + e);
                vx[j] = *reinterpret_cast<const uint4 *>(static_cast<const float *>(p.v_cache) + e);
            } else if constexpr (KVT == 1) {
                const uint2 a = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(p.k_cache) + e);
                const uint2 c2 = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(p.v_cache) + e);
                kx[j].x = a.x; kx[j].y = a.y;
                vx[j].x = c2.x; vx[j].y = c2.y;
            } else {
                kx[j].x = *reinterpret_cast<const uint32_t *>(static_cast<const uint8_t *>(p.k_cache) + e);
                vx[j].x = *reinterpret_cast<const uint32_t *>(static_cast<const uint8_t *>(p.v_cache) + e);
            }
        }
    }
    __syncthreads();  // every source row is read before any destination is written
#pragma unroll
    for (int j = 0; j < kCommitPer; ++j) {
        const int idx = threadIdx.x + j * kCommitThreads;
        if (idx >= n * quads)
            continue;
        const int i = idx / quads, c4 = idx - i * quads;
        const int pd = base + 1 + i;
        const int pg = page_of(pd);
        const size_t e = row_off(pg, pd) + (size_t)c4 * 4;
        if constexpr (KVT == 0) {
            *reinterpret_cast<uint4 *>(static_cast<float *>(p.k_cache) + e) = kx[j];
            *reinterpret_cast<uint4 *>(static_cast<float *>(p.v_cache) + e) = vx[j];
        } else if constexpr (KVT == 1) {
            *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(p.k_cache) + e) = make_uint2(kx[j].x, kx[j].y);
            *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(p.v_cache) + e) = make_uint2(vx[j].x, vx[j].y);
        } else {
            uint32_t kc = kx[j].x, vc = vx[j].x;
            if (pg != src_page[j]) {
                const float kss = p.k_scale[src_page[j]], ksd = p.k_scale[pg];
                const float vss = p.v_scale[src_page[j]], vsd = p.v_scale[pg];
                uint32_t k2 = 0, v2 = 0;
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const float xk = e4m3_value((kc >> (8 * t)) & 0xFFu) * kss;
                    const float xv = e4m3_value((vc >> (8 * t)) & 0xFFu) * vss;
                    k2 |= e4m3_code(xk / ksd) << (8 * t);
                    v2 |= e4m3_code(xv / vsd) << (8 * t);
                }
                kc = k2;
                vc = v2;
            }
            *reinterpret_cast<uint32_t *>(static_cast<uint8_t *>(p.k_cache) + e) = kc;
            *reinterpret_cast<uint32_t *>(static_cast<uint8_t *>(p.v_cache) + e) = vc;
        }
    }
}

__global__ __launch_bounds__(256) void sv_tree_length_kernel(const int32_t *num_accepted, int32_t *context_lens,
                                                             int32_t *pages_in_use, int B, int N, int Lmax)
{
    const int b = blockIdx.x * 256 + threadIdx.x;
    if (b >= B)
        return;
    int L = context_lens[b];
    L = L < N ? N : (L > Lmax ? Lmax : L);
    int n = num_accepted[b];
    n = n < 0 ? 0 : (n > N - 1 ? N - 1 : n);
    L = L - N + 1 + n;
    context_lens[b] = L;
    if (pages_in_use)
        pages_in_use[b] = (L + kBlock - 1) / kBlock;
}

}  // namespace

hipError_t launch_tree_commit(const TreeCommitParams &p, int kv_dtype, hipStream_t stream)
{
    const dim3 grid((unsigned)(p.B * p.Hkv)), block(kCommitThreads);
    if (kv_dtype == 0)
        hipLaunchKernelGGL(sv_tree_commit_kernel<0>, grid, block, 0, stream, p);
    else if (kv_dtype == 1)
        hipLaunchKernelGGL(sv_tree_commit_kernel<1>, grid, block, 0, stream, p);
    else
        hipLaunchKernelGGL(sv_tree_commit_kernel<2>, grid, block, 0, stream, p);
    hipLaunchKernelGGL(sv_tree_length_kernel, dim3((unsigned)((p.B + 255) / 256)), dim3(256), 0, stream,
                       p.num_accepted, p.context_lens, p.pages_in_use, p.B, p.N, p.max_blocks * kBlock);
    return hipGetLastError();
}

hipError_t launch_kv_append(const AppendParams &p, int kv_dtype, hipStream_t stream)
{
    const int64_t total = (int64_t)p.B * p.T * p.Hkv * (p.d / 4);
    const dim3 grid((unsigned)((total + 255) / 256));
    if (kv_dtype == 0)
        hipLaunchKernelGGL(sv_kv_append_kernel<0>, grid, dim3(256), 0, stream, p);
    else if (kv_dtype == 1)
        hipLaunchKernelGGL(sv_kv_append_kernel<1>, grid, dim3(256), 0, stream, p);
    else
        hipLaunchKernelGGL(sv_kv_append_kernel<2>, grid, dim3(256), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_rollback(const int32_t *num_accepted, int32_t *context_lens, int32_t *pages_in_use, int B, int K,
                           hipStream_t stream)
{
    hipLaunchKernelGGL(sv_rollback_kernel, dim3((unsigned)((B + 255) / 256)), dim3(256), 0, stream, num_accepted,
                       context_lens, pages_in_use, B, K);
    return hipGetLastError();
}

}  // namespace sv
