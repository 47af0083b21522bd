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
//   far_part_kernel    one wave per (row, head), lane = landmark: landmark scores, weights
//                      through mu, gains, far mass and numerator -> the far partial;
//   far_commit_kernel  one wave per (head, landmark), lane = chunk row: the far state after
//                      the chunk (before the ring commit overwrites the evicted rows).
// A chunk with a far field has at most 64 rows and at most 64 landmarks (one wave's lanes; the
// page's far path keeps 64-entry row buffers).
#include "launch.h"

namespace winattn {

namespace {

// The far sums run in f64: with signed mixing weights the landmark gains, the far mass and the
// far numerator are sums of terms of both signs that can cancel by orders of magnitude, and in
// f32 the rounding of every term (scores, exponentials, products) would be amplified by that
// cancellation. The near partials and the far partial itself stay f32.
__device__ inline double far_wave_max(double v) {
#pragma unroll
    for (int k = 32; k >= 1; k >>= 1) v = fmax(v, __shfl_xor(v, k));
    return v;
}
__device__ inline double far_wave_sum(double v) {
#pragma unroll
    for (int k = 32; k >= 1; k >>= 1) v += __shfl_xor(v, k);
    return v;
}
// Inclusive prefix sum over the wave's lanes.
__device__ inline double far_wave_scan(double v, int lane) {
#pragma unroll
    for (int k = 1; k < 64; k <<= 1) {
        const double u = __shfl_up(v, k);
        if (lane >= k) v += u;
    }
    return v;
}

constexpr double kLog2eD = 1.4426950408889634074;

// f64 dot product of two f32 rows of d floats (d a multiple of 4, 16-byte aligned).
__device__ inline double dot_f64(const float* a, const float* b, int d) {
    const float4* x = reinterpret_cast<const float4*>(a);
    const float4* y = reinterpret_cast<const float4*>(b);
    double acc = 0.0;
    for (int c = 0; c < d / 4; ++c) {
        const float4 u = x[c], v = y[c];
        acc = fma((double)u.x, (double)v.x, acc);
        acc = fma((double)u.y, (double)v.y, acc);
        acc = fma((double)u.z, (double)v.z, acc);
        acc = fma((double)u.w, (double)v.w, acc);
    }
    return acc;
}

struct Acc4 {
    double x, y, z, w;
};
__device__ inline void acc4_fma(Acc4& a, double s, float4 v) {
    a.x = fma(s, (double)v.x, a.x);
    a.y = fma(s, (double)v.y, a.y);
    a.z = fma(s, (double)v.z, a.z);
    a.w = fma(s, (double)v.w, a.w);
}

struct GroupState {
    uint32_t wg, len0, head0, far0;
    int j0;   // first evicting chunk row
};

// The group's window, clamped as the attention kernels clamp it.
__device__ inline GroupState group_state(const FarParams& p, int g) {
    const uint32_t* m = p.meta + 4 * g;
    GroupState s;
    const uint32_t w = (uint32_t)p.w, ov = m[3];
    s.wg = (ov != 0u && ov < w) ? ov : w;
    s.len0 = m[0] < s.wg ? m[0] : s.wg;
    s.head0 = m[1] >= s.wg ? m[1] % s.wg : m[1];
    s.far0 = m[2];
    s.j0 = (int)s.wg - (int)s.len0;
    return s;
}

// K or V row of the entry chunk row j (>= j0) evicts.
__device__ inline const float* evicted_row(const FarParams& p, const GroupState& s, int g, int j,
                                           bool value) {
    const uint32_t x = (uint32_t)(j - s.j0);
    if (x < s.len0) {
        const uint32_t slot = (uint32_t)(((unsigned long long)s.head0 + x) % s.wg);
        return (value ? p.ring_v : p.ring_k) + ((size_t)g * p.w + slot) * p.d;
    }
    const size_t row = (size_t)(x - s.len0);
    return (value ? p.chunk_v : p.chunk_k) + (row * p.ng + g) * p.d;
}

struct Eviction {
    double e;    // this lane's (chunk row's) eviction weight exp(fe - mx), 0 if it evicts nothing
    double z;    // far mass as of this lane's row: old mass * r + sum of e up to the row
    double mx;   // far max after the chunk
    double r;    // rescale of the old mass and numerator: exp(old max - mx), 1 if unchanged
};

// One wave, lane = chunk row: the chunk's evictions scored against landmark (gh, b).
__device__ inline Eviction evict_landmark(const FarParams& p, const GroupState& s, int g, int gh,
                                          int b, int lane) {
    const double m_old = p.mz[(size_t)gh * 2 * p.m + b];
    const double mass = p.mz[(size_t)gh * 2 * p.m + p.m + b];
    const bool evicts = lane < p.rows && lane >= s.j0;
    double fe = -INFINITY;
    if (evicts)
        fe = (double)p.scale *
             dot_f64(p.q_tilde + ((size_t)gh * p.m + b) * p.d, evicted_row(p, s, g, lane, false), p.d);
    Eviction ev;
    ev.mx = fmax(m_old, far_wave_max(fe));
    // An empty far field starts at -inf: without evictions its max stays and r = 1; the first
    // eviction rescales the zero mass by exp(-inf) = 0.
    ev.r = ev.mx == m_old ? 1.0 : exp(m_old - ev.mx);
    ev.e = evicts ? exp(fe - ev.mx) : 0.0;
    ev.z = mass * ev.r + far_wave_scan(ev.e, lane);
    return ev;
}

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

// One wave per (row i, head gh); lane a is landmark a for the scores and weights, lane j is
// chunk row j for the evicted rows' weights, then lane c owns float4 column c of the numerator.
__global__ __launch_bounds__(64) void far_part_kernel(const FarParams p) {
    __shared__ double s_ea[64], s_gain[64], s_gn[64], s_cf[64];
    const int i = blockIdx.x / p.nh, gh = blockIdx.x % p.nh;
    const int g = gh / p.hpg, lane = threadIdx.x;
    const GroupState s = group_state(p, g);
    const int m = p.m, d4 = p.d / 4;

    // This (row, head)'s slot in the partial buffer.
    const int qi = i * p.hpg + gh % p.hpg;   // query index within the group, row-major
    const int blk = g * p.nqblocks + qi / p.qb, j = qi % p.qb;
    const size_t at = ((size_t)blk * p.slot_stride + p.far_slot) * p.qb + j;
    float* acc_out = p.pacc + at * p.dpad;

    const long long farl = (long long)s.far0 + (i >= s.j0 ? i - s.j0 + 1 : 0);
    float pm = -INFINITY;
    double far_den = 0.0;
    bool have = false;
    if (farl > 0) {
        const size_t lb = (size_t)gh * m + lane;
        // landmark scores of the row's query
        double fl = -INFINITY;
        if (lane < m)
            fl = (double)p.scale * dot_f64(p.q + ((size_t)i * p.nh + gh) * p.d,
                                           p.k_tilde + ((size_t)g * m + lane) * p.d, p.d);
        const double f = far_wave_max(fl);
        s_ea[lane] = lane < m ? exp(fl - f) : 0.0;
        // The far partial's max, rounded to f32 as the merge reads it; the gains are taken
        // against that rounded value, so the merge's rescale of this partial is exact.
        const double Mb = lane < m ? f + p.ev_mx[lb] : -INFINITY;
        pm = (float)(far_wave_max(Mb) * kLog2eD);
        const double M = (double)pm / kLog2eD;
        __syncthreads();
        // weight of landmark b (lane b): sum_a exp(fl_a - f) mu[a][b]
        double wb = 0.0;
        if (lane < m)
            for (int a = 0; a < m; ++a)
                wb = fma(s_ea[a], (double)p.mu[((size_t)gh * m + a) * m + lane], wb);
        const double gain = lane < m ? wb * exp(Mb - M) : 0.0;
        far_den = far_wave_sum(lane < m ? gain * p.ev_z[lb * p.rows + i] : 0.0);
        have = far_den >= 0.0 && pm > -INFINITY;
        s_gain[lane] = gain;
        s_gn[lane] = lane < m ? gain * p.ev_r[lb] : 0.0;
        __syncthreads();
        // weight of each evicted row j0 <= jj <= i: sum_b gain_b e_b(jj) (lane jj)
        double cf = 0.0;
        if (lane <= i && lane >= s.j0)
            for (int bb = 0; bb < m; ++bb)
                cf = fma(s_gain[bb], p.ev_e[((size_t)gh * m + bb) * p.rows + lane], cf);
        s_cf[lane] = cf;
        __syncthreads();
    }
    if (!have) {   // empty field, or a negative far mass: the far part is dropped
        for (int c = lane; c < p.dpad / 4; c += 64)
            reinterpret_cast<float4*>(acc_out)[c] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (lane == 0) {
            p.pm[at] = -INFINITY;
            p.pl[at] = 0.0f;
        }
        return;
    }
    for (int c = lane; c < p.dpad / 4; c += 64) {
        Acc4 a{0.0, 0.0, 0.0, 0.0};
        if (c < d4) {
            for (int bb = 0; bb < m; ++bb)
                acc4_fma(a, s_gn[bb],
                         reinterpret_cast<const float4*>(p.t_hat + ((size_t)gh * m + bb) * p.d)[c]);
            for (int jj = s.j0; jj <= i; ++jj)
                acc4_fma(a, s_cf[jj], reinterpret_cast<const float4*>(evicted_row(p, s, g, jj, true))[c]);
        }
        reinterpret_cast<float4*>(acc_out)[c] =
            make_float4((float)a.x, (float)a.y, (float)a.z, (float)a.w);
    }
    if (lane == 0) {
        p.pm[at] = pm;   // the merge works in the log2 domain
        p.pl[at] = (float)far_den;
    }
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

hipError_t launch_far_part(const FarParams& p, hipStream_t stream) {
    hipLaunchKernelGGL(far_part_kernel, dim3(p.rows * p.nh), dim3(64), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_far_commit(const FarParams& p, hipStream_t stream) {
    hipLaunchKernelGGL(far_commit_kernel, dim3(p.nh * p.m), dim3(64), 0, stream, p);
    return hipGetLastError();
}

}  // namespace winattn
