// The far field: landmark summaries of keys that have left a group's window (o1c page, "A
// sealed layer's attention for a chunk of rows, on Metal": `o1c_far_e`, `o1c_land`, `o1c_far`,
// `o1c_add`, `o1c_far_commit`; token path `o1c_tok_far`, `o1c_tok_merge`, `o1c_tok_commit`).
//
// Per query head gh and landmark b the state is a far max mx_b and far mass z_b (mz [gh][2m])
// and a far numerator t_hat_b [d]: sums of exp(s - mx_b) and exp(s - mx_b) V over evicted keys,
// s = scale <q_tilde_b, K>. A row reads them through landmark keys k_tilde [g][m][d] and the
// mixing matrix mu [gh][m][m]: landmark b weighs sum_a exp(fl_a) mu[a][b], fl_a = scale <q,
// k_tilde_a>. Chunk row j >= j0 = wg - len0 evicts the group's oldest entry x = j - j0 (ring
// slot (head0 + x) mod wg while x < len0, else chunk row x - len0).
//
// On the GPU the far part of a (row, head) is one more partial (max, mass, numerator) in the
// split-K partial buffer, so the merge launch folds it with the near splits exactly as it
// folds the splits with each other. Three kernels:
//   far_evict_kernel   one wave per (head, landmark), lane = chunk row: eviction scores, far
//                      max, rescale of the old state and the prefix far mass, into workspace
//                      (f64);
//   far_part_kernel    one workgroup per (row, head): landmark scores, weights through mu,
//                      gains, far mass and numerator -> the far partial (a one-row call
//                      scores its own eviction here instead of in far_evict_kernel);
//   far_commit_kernel  one wave per (head, landmark), lane = chunk row: the far state after
//                      the chunk (before the ring commit overwrites the evicted rows).
// A chunk with a far field has at most 64 rows and at most 64 landmarks (one wave's lanes; the
// page's far path keeps 64-entry row buffers).
#include "far_part.h"
#include "launch.h"

namespace winattn {

namespace {

__global__ __launch_bounds__(64) void far_evict_kernel(const FarParams p) {
    const int gh = blockIdx.x / p.m, b = blockIdx.x % p.m;
    const int g = gh / p.hpg, lane = threadIdx.x;
    const GroupState s = group_state(p, g);
    const Eviction ev = evict_landmark(p, s, g, gh, b, lane);
    const size_t at = (size_t)gh * p.m + b;
    if (lane < p.rows) {
        p.ev_e[at * p.rows + lane] = ev.e;
        p.ev_z[at * p.rows + lane] = ev.z;
    }
    if (lane == 0) {
        p.ev_mx[at] = ev.mx;
        p.ev_r[at] = ev.r;
    }
}

template <int DP, int MODE>
__global__ __launch_bounds__(256) void far_part_kernel(const FarParams p) {
    far_part_block<DP, MODE>(p, blockIdx.x);
}

// The far state after the chunk, before the ring commit overwrites the evicted rows: for every
// landmark with evictions, t_hat <- t_hat r + sum_j e_j V_ev(j), max <- mx, mass <- the mass
// after the chunk's last row.
__global__ __launch_bounds__(64) void far_commit_kernel(const FarParams p) {
    __shared__ double s_e[64];
    const int gh = blockIdx.x / p.m, b = blockIdx.x % p.m;
    const int g = gh / p.hpg, lane = threadIdx.x;
    const GroupState s = group_state(p, g);
    if (s.j0 >= p.rows) return;   // the chunk evicts nothing: the state is unchanged
    const Eviction ev = evict_landmark(p, s, g, gh, b, lane);
    s_e[lane] = ev.e;
    const double z_last = __shfl(ev.z, p.rows - 1);
    __syncthreads();
    float* th = p.t_hat + ((size_t)gh * p.m + b) * p.d;
    for (int c = lane; c < p.d / 4; c += 64) {
        const float4 t = reinterpret_cast<const float4*>(th)[c];
        Acc4 a{(double)t.x * ev.r, (double)t.y * ev.r, (double)t.z * ev.r, (double)t.w * ev.r};
        for (int jj = s.j0; jj < p.rows; ++jj)
            acc4_fma(a, s_e[jj], reinterpret_cast<const float4*>(evicted_row(p, s, g, jj, true))[c]);
        reinterpret_cast<float4*>(th)[c] = make_float4((float)a.x, (float)a.y, (float)a.z, (float)a.w);
    }
    if (lane == 0) {
        p.mz[(size_t)gh * 2 * p.m + b] = (float)ev.mx;
        p.mz[(size_t)gh * 2 * p.m + p.m + b] = (float)z_last;
    }
}

}  // namespace

hipError_t launch_far_evict(const FarParams& p, hipStream_t stream) {
    hipLaunchKernelGGL(far_evict_kernel, dim3(p.nh * p.m), dim3(64), 0, stream, p);
    return hipGetLastError();
}

template <int DP>
static void launch_far_part_dp(const FarParams& p, int mode, hipStream_t stream) {
    const dim3 grid(p.rows * p.nh), block(256);
    if (mode == kFarFromWorkspace)
        hipLaunchKernelGGL((far_part_kernel<DP, kFarFromWorkspace>), grid, block, 0, stream, p);
    else if (mode == kFarFusedOneRow)
        hipLaunchKernelGGL((far_part_kernel<DP, kFarFusedOneRow>), grid, block, 0, stream, p);
    else
        hipLaunchKernelGGL((far_part_kernel<DP, kFarCurrent>), grid, block, 0, stream, p);
}

hipError_t launch_far_part(const FarParams& p, int mode, hipStream_t stream) {
    if (p.dpad == 64)
        launch_far_part_dp<64>(p, mode, stream);
    else if (p.dpad == 128)
        launch_far_part_dp<128>(p, mode, stream);
    else
        launch_far_part_dp<256>(p, mode, stream);
    return hipGetLastError();
}

hipError_t launch_far_commit(const FarParams& p, hipStream_t stream) {
    hipLaunchKernelGGL(far_commit_kernel, dim3(p.nh * p.m), dim3(64), 0, stream, p);
    return hipGetLastError();
}

}  // namespace winattn
