// Ring commit and meta advance after a chunk: the state a decode loop carries from one call to
// the next (o1c page: `o1c_ring_commit` writes the chunk's K/V rows into the ring at the slots
// their pushes land in, `o1c_meta` advances length, head and far count; `o1c_tok_commit` is
// the one-row form).
//
// Row j of the chunk lands in slot (head0 + len0 + j) mod wg of its group's ring. If
// len0 + rows exceeds wg, the ring is full afterwards, its head has moved on by the number of
// evicted entries and the far count (meta field 2) grows by the same number; the pages leave
// head and far count untouched otherwise. Reading for chunks longer than the window: pushes
// are sequential, so only the chunk's last wg rows are written (the earlier ones would be
// overwritten within the same chunk).
//
// One workgroup per KV group: every thread reads the group's metadata, a barrier, then the
// rows are copied with 16-byte loads and stores and thread 0 writes the new metadata.
#include "launch.h"

namespace winattn {

__global__ __launch_bounds__(kThreads) void ring_commit_kernel(const CommitParams p) {
    const int g = blockIdx.x;
    const uint32_t* m = p.meta + 4 * g;
    // Out-of-range metadata is clamped the way the attention kernels clamp it, so no store
    // leaves the group's ring.
    const uint32_t w = (uint32_t)p.w;
    const uint32_t ov = m[3];
    const uint32_t wg = (ov != 0u && ov < w) ? ov : w;
    const uint32_t len0 = m[0] < wg ? m[0] : wg;
    uint32_t head0 = m[1];
    if (head0 >= wg) head0 %= wg;
    const uint32_t far0 = m[2];
    __syncthreads();   // every thread has read the old metadata before thread 0 rewrites it

    const int first = p.rows > (int)wg ? p.rows - (int)wg : 0;
    const int d4 = p.d / 4;
    const long long n = (long long)(p.rows - first) * d4;
    for (long long idx = threadIdx.x; idx < n; idx += kThreads) {
        const int j = first + (int)(idx / d4), c = (int)(idx % d4);
        const uint32_t slot = (uint32_t)(((unsigned long long)head0 + len0 + (unsigned)j) % wg);
        const size_t src = ((size_t)j * p.ng + g) * p.d + 4 * (size_t)c;
        const size_t dst = ((size_t)g * p.w + slot) * p.d + 4 * (size_t)c;
        *reinterpret_cast<float4*>(p.ring_k + dst) = *reinterpret_cast<const float4*>(p.chunk_k + src);
        *reinterpret_cast<float4*>(p.ring_v + dst) = *reinterpret_cast<const float4*>(p.chunk_v + src);
    }
    if (threadIdx.x == 0) {
        const unsigned long long tot = (unsigned long long)len0 + (unsigned)p.rows;
        uint32_t* mo = p.meta + 4 * g;
        if (tot <= wg) {
            mo[0] = (uint32_t)tot;
        } else {
            const unsigned long long ev = tot - wg;
            mo[0] = wg;
            mo[1] = (uint32_t)(((unsigned long long)head0 + ev) % wg);
            mo[2] = far0 + (uint32_t)ev;
        }
    }
}

hipError_t launch_ring_commit(const CommitParams& p, hipStream_t stream) {
    hipLaunchKernelGGL(ring_commit_kernel, dim3(p.ng), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace winattn
