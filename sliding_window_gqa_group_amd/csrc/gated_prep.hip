// Rotation, unit heads and the ring write of the gated call (dory page, "Dory's token path",
// `dory_prep`): one wave per (head, row); lane e handles element pairs (e, e + hd/2), and
// (e + 64, e + 64 + hd/2) when hd/2 > 64.
//   u = x*c - y*s, v = y*c + x*s over the halves x, y of the raw head and c, s of the table row
//   inv = 1 / sqrt(sum u^2 + sum v^2 + eps)
//   query head a:  qout[row][a] = (u, v) * inv * q_scale[a]
//   KV head kh:    ring_k[(pos0+row) % cap][kh] = (u, v) * inv; ring_v[...] = raw yv
#include "launch.h"

namespace winattn {

__global__ __launch_bounds__(64) void gated_prep_kernel(const PrepParams p) {
    const int a = blockIdx.x, row = blockIdx.y, lane = threadIdx.x;
    const int half = p.hd / 2;
    const bool is_q = a < p.nh;
    const float* raw = is_q ? p.yq + ((size_t)row * p.nh + a) * p.hd
                            : p.yk + ((size_t)row * p.nk + (a - p.nh)) * p.hd;
    const float* cs = p.rope + (size_t)row * p.hd;
    float u[2], v[2];
    float ss = 0.0f;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int e = lane + 64 * k;
        u[k] = 0.0f;
        v[k] = 0.0f;
        if (e < half) {
            const float x = raw[e], y = raw[half + e], c = cs[e], s = cs[half + e];
            u[k] = x * c - y * s;
            v[k] = y * c + x * s;
            ss += u[k] * u[k] + v[k] * v[k];
        }
    }
    ss = wave_sum(ss);
    const float inv = 1.0f / sqrtf(ss + p.eps);
    if (is_q) {
        float* qo = p.qout + ((size_t)row * p.nh + a) * p.hd;
        const float* sc = p.q_scale + (size_t)a * p.hd;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int e = lane + 64 * k;
            if (e < half) {
                qo[e] = u[k] * inv * sc[e];
                qo[half + e] = v[k] * inv * sc[half + e];
            }
        }
    } else {
        const int kh = a - p.nh;
        const size_t slot = (size_t)(((long long)p.pos0 + row) % p.cap);
        const size_t at = (slot * p.nk + kh) * p.hd;
        const float* yv = p.yv + ((size_t)row * p.nk + kh) * p.hd;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int e = lane + 64 * k;
            if (e < half) {
                p.ring_k[at + e] = u[k] * inv;
                p.ring_k[at + half + e] = v[k] * inv;
                p.ring_v[at + e] = yv[e];
                p.ring_v[at + half + e] = yv[half + e];
            }
        }
    }
}

hipError_t launch_gated_prep(const PrepParams& p, hipStream_t stream) {
    hipLaunchKernelGGL(gated_prep_kernel, dim3(p.nh + p.nk, p.rows), dim3(64), 0, stream, p);
    return hipGetLastError();
}

__global__ void fill_zero_kernel(unsigned int* p, size_t n) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (size_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

__global__ void fill_zero_bytes_kernel(unsigned char* p, size_t n) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (size_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

hipError_t launch_fill_zero(void* ptr, size_t bytes, hipStream_t stream) {
    const size_t words = bytes / 4;
    if (words > 0) {
        size_t blocks = (words + 255) / 256;
        if (blocks > 4096) blocks = 4096;
        hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                           (unsigned int*)ptr, words);
    }
    const size_t tail = bytes - words * 4;
    if (tail > 0)
        hipLaunchKernelGGL(fill_zero_bytes_kernel, dim3(1), dim3(64), 0, stream,
                           (unsigned char*)ptr + words * 4, tail);
    return hipGetLastError();
}

}  // namespace winattn
