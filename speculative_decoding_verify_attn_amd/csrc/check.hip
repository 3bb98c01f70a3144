// check.hip -- counts violations of the device-data preconditions that the
// verify calls document but do not check (a debug aid; the calls themselves
// stay memory-safe on such inputs by clamping indices):
//   [0] context lengths outside [T, 16 * max_blocks]  (each cached position
//       needs a page, and the T verify positions must be cached:
//       "KV Cache + Speculative Decoding" 5.2-5.3, 6.1);
//   [1] block-table entries of visible pages outside [0, num_blocks)  (the
//       page table maps logical pages to physical ones, same sections);
//   [2] draft tokens outside [0, V);
//   [3] uniforms outside [0, 1) or not finite  (the acceptance test and the
//       draw take u ~ U[0, 1): "50 | Speculative Decoding" 3.1).
// One workgroup per sequence; counts are summed in LDS, then added to the
// caller's counters with one atomic per category and workgroup.
#include "sv_device.hpp"
#include "sv_internal.hpp"

namespace sv {
namespace {

constexpr int kCheckThreads = 256;

__global__ __launch_bounds__(kCheckThreads) void sv_check_inputs_kernel(CheckParams p)
{
    __shared__ int s_cnt[kCheckCounts];
    const int b = blockIdx.x, tid = threadIdx.x;
    if (tid < kCheckCounts)
        s_cnt[tid] = 0;
    __syncthreads();
    if (p.context_lens) {
        const int L = p.context_lens[b];
        const long long cap = (long long)p.max_blocks * kBlock;
        if (tid == 0 && (L < p.T || (long long)L > cap))
            atomicAdd(&s_cnt[0], 1);
        if (p.block_table) {
            // the pages that hold visible positions (length clamped as the
            // attention kernels clamp it)
            const int Lc = L < 0 ? 0 : ((long long)L > cap ? (int)cap : L);
            const int np = (Lc + kBlock - 1) / kBlock;
            int bad = 0;
            for (int i = tid; i < np; i += kCheckThreads) {
                const int e = p.block_table[(size_t)b * p.max_blocks + i];
                bad += (e < 0 || e >= p.num_blocks) ? 1 : 0;
            }
            if (bad)
                atomicAdd(&s_cnt[1], bad);
        }
    }
    if (p.tokens)
        for (int i = tid; i < p.n_tokens; i += kCheckThreads) {
            const int x = p.tokens[(size_t)b * p.n_tokens + i];
            if (x < 0 || x >= p.V)
                atomicAdd(&s_cnt[2], 1);
        }
    if (p.uniforms)
        for (int i = tid; i < p.n_uniforms; i += kCheckThreads) {
            const float u = p.uniforms[(size_t)b * p.n_uniforms + i];
            if (!(u >= 0.0f && u < 1.0f))  // NaN fails both comparisons
                atomicAdd(&s_cnt[3], 1);
        }
    __syncthreads();
    if (tid < kCheckCounts && s_cnt[tid] != 0)
        atomicAdd(&p.counts[tid], s_cnt[tid]);
}

}  // namespace

hipError_t launch_check_inputs(const CheckParams &p, hipStream_t stream)
{
    // counters cleared with a fill kernel (no memset node under capture)
    hipError_t e = launch_clear(p.counts, sizeof(int32_t) * kCheckCounts, stream);
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(sv_check_inputs_kernel, dim3((unsigned)p.B), dim3(kCheckThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace sv
