// probe.hip -- measurement only: the practical HBM read ceiling that the
// attention kernel is compared with.  Not part of the verify step.
//
// A plain streaming read of `bytes` bytes: workgroup w reads one contiguous
// chunk of the buffer with 16-byte loads, eight per thread in flight, and
// each thread leaves one float (a sum of what it read, so the loads cannot be
// dropped) in the sink.  1024 workgroups of 256 threads measured fastest of
// the chunked and grid-strided shapes tried (about 6.2 TB/s on MI355X from
// 0.5 GB up).
#include "sv_internal.hpp"

namespace sv {
namespace {

constexpr int kProbeUnroll = 8;

__global__ __launch_bounds__(kProbeThreads) void sv_probe_read_kernel(const float4 *__restrict__ src, size_t n4,
                                                                      size_t chunk4, float *sink)
{
    const size_t base = (size_t)blockIdx.x * chunk4;
    size_t end = base + chunk4;
    if (end > n4)
        end = n4;
    float acc = 0.0f;
    size_t i = base + threadIdx.x;
    for (; i + (kProbeUnroll - 1) * (size_t)kProbeThreads < end; i += kProbeUnroll * (size_t)kProbeThreads) {
        float4 v[kProbeUnroll];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u)
            v[u] = src[i + u * (size_t)kProbeThreads];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u)
            acc += (v[u].x + v[u].y) + (v[u].z + v[u].w);
    }
    for (; i < end; i += kProbeThreads) {
        const float4 v = src[i];
        acc += (v.x + v.y) + (v.z + v.w);
    }
    sink[(size_t)blockIdx.x * kProbeThreads + threadIdx.x] = acc;
}

}  // namespace

hipError_t launch_probe_read(const void *src, size_t bytes, float *sink, hipStream_t stream)
{
    const size_t n4 = bytes / 16;
    const size_t chunk4 = (n4 + kProbeWgs - 1) / kProbeWgs;
    hipLaunchKernelGGL(sv_probe_read_kernel, dim3(kProbeWgs), dim3(kProbeThreads), 0, stream,
                       static_cast<const float4 *>(src), n4, chunk4, sink);
    return hipGetLastError();
}

}  // namespace sv
