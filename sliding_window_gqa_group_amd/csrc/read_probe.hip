// The achievable HBM read rate on this GPU, measured the way the attention kernels read: a
// plain streaming read of a buffer in which every 16-byte element is loaded exactly once.
// Each thread issues kReadUnroll coalesced 16-byte loads back to back (a wave covers 1 KiB per
// load instruction) and folds them into a running sum, which reaches memory only when it is
// not a number: the loads cannot be dropped, and the launch writes nothing for finite data.
// One workgroup per 256 * kReadUnroll elements, so a 32 MiB buffer gives 1024 workgroups,
// four per CU, each with 32 KiB in flight.
#include "launch.h"

namespace winattn {

constexpr int kReadUnroll = 8;

__global__ __launch_bounds__(kThreads) void read_probe_kernel(const vf4* src, long long n4,
                                                              float* sink) {
    const long long base = (long long)blockIdx.x * kThreads * kReadUnroll + threadIdx.x;
    vf4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) {
        const long long j = base + (long long)u * kThreads;
        v[u] = src[j < n4 ? j : n4 - 1];   // clamped address; the extra element is dropped below
    }
    float s = 0.0f;
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) {
        const bool in = base + (long long)u * kThreads < n4;
        s += in ? (v[u].x + v[u].y) + (v[u].z + v[u].w) : 0.0f;
    }
    if (s != s) sink[blockIdx.x & 255] = s;
}

hipError_t launch_read_probe(const void* src, size_t bytes, float* sink, hipStream_t stream) {
    const long long n4 = (long long)(bytes / 16);
    const long long per_block = (long long)kThreads * kReadUnroll;
    const long long blocks = (n4 + per_block - 1) / per_block;
    if (n4 < 1 || blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(read_probe_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                       static_cast<const vf4*>(src), n4, sink);
    return hipGetLastError();
}

}  // namespace winattn
