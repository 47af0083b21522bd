// Device code of the far field shared by its launches: f64 cross-lane helpers, the group's far
// state, eviction scoring, and far_part_block (one workgroup per (row, head) of a chunk, which
// writes that row's far partial). The far field itself is described in far_field.hip.
#pragma once
#include "launch.h"
#include "winattn_dev.h"

namespace winattn {
namespace {


// The far sums run in f64: with signed mixing weights the landmark gains, the far mass and the
// far numerator are sums of terms of both signs that can cancel by orders of magnitude, and in
// f32 the rounding of every term (scores, exponentials, products) would be amplified by that
// cancellation. The near partials and the far partial itself stay f32.
// f64 cross-lane steps on DPP: both 32-bit halves move with the same control (lanes whose
// source is outside the row, or rows outside ROW_MASK, take `fill`).
template <int CTRL, int ROW_MASK = 0xF>
__device__ inline double dpp64(double v, double fill) {
    const unsigned long long b = (unsigned long long)__double_as_longlong(v);
    const unsigned long long f = (unsigned long long)__double_as_longlong(fill);
    const int lo = __builtin_amdgcn_update_dpp((int)(unsigned)f, (int)(unsigned)b, CTRL, ROW_MASK,
                                               0xF, false);
    const int hi = __builtin_amdgcn_update_dpp((int)(unsigned)(f >> 32), (int)(unsigned)(b >> 32),
                                               CTRL, ROW_MASK, 0xF, false);
    return __longlong_as_double((long long)(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo));
}
__device__ inline double readlane64(double v, int lane) {
    const unsigned long long b = (unsigned long long)__double_as_longlong(v);
    const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)b, lane);
    const unsigned hi = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)(b >> 32), lane);
    return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}

// Max / sum over the whole wave, returned in every lane.
__device__ inline double far_wave_max(double v) {
    v = fmax(v, dpp64<kDppXor1>(v, -INFINITY));
    v = fmax(v, dpp64<kDppXor2>(v, -INFINITY));
    v = fmax(v, dpp64<kDppHalfMirror>(v, -INFINITY));
    v = fmax(v, dpp64<kDppMirror>(v, -INFINITY));
    v = fmax(v, dpp64<kDppBcast15, 0xA>(v, -INFINITY));
    v = fmax(v, dpp64<kDppBcast31, 0xC>(v, -INFINITY));
    return readlane64(v, 63);
}
__device__ inline double far_wave_sum(double v) {
    v += dpp64<kDppXor1>(v, 0.0);
    v += dpp64<kDppXor2>(v, 0.0);
    v += dpp64<kDppHalfMirror>(v, 0.0);
    v += dpp64<kDppMirror>(v, 0.0);
    v += dpp64<kDppBcast15, 0xA>(v, 0.0);
    v += dpp64<kDppBcast31, 0xC>(v, 0.0);
    return readlane64(v, 63);
}
// Sum over each aligned group of N lanes (N = 4, 8 or 16), in every lane of the group.
template <int N>
__device__ inline double far_group_sum(double v) {
    v += dpp64<kDppXor1>(v, 0.0);
    v += dpp64<kDppXor2>(v, 0.0);
    if constexpr (N >= 8) v += dpp64<kDppHalfMirror>(v, 0.0);
    if constexpr (N >= 16) v += dpp64<kDppMirror>(v, 0.0);
    return v;
}
// Inclusive prefix sum over the wave's lanes: shifts of 1, 2, 4, 8 within each row of 16,
// then each row adds the totals of the rows before it.
__device__ inline double far_wave_scan(double v) {
    v += dpp64<0x111>(v, 0.0);   // row_shr:1
    v += dpp64<0x112>(v, 0.0);   // row_shr:2
    v += dpp64<0x114>(v, 0.0);   // row_shr:4
    v += dpp64<0x118>(v, 0.0);   // row_shr:8
    v += dpp64<kDppBcast15, 0xA>(v, 0.0);
    v += dpp64<kDppBcast31, 0xC>(v, 0.0);
    return v;
}

constexpr double kLog2eD = 1.4426950408889634074;

// f64 dot product of two f32 rows of d floats (d a multiple of 4, 16-byte aligned).
// The float4s are loaded 8 at a time, every load of a batch issued before the first is used
// (one memory round trip per 32 elements instead of one per 4); the products are summed in
// element order either way.
__device__ inline double dot_f64(const float* a, const float* b, int d) {
    const float4* x = reinterpret_cast<const float4*>(a);
    const float4* y = reinterpret_cast<const float4*>(b);
    constexpr int U = 8;
    const int n4 = d / 4;
    double acc = 0.0;
    auto add4 = [&](const float4& u, const float4& v) {
        acc = fma((double)u.x, (double)v.x, acc);
        acc = fma((double)u.y, (double)v.y, acc);
        acc = fma((double)u.z, (double)v.z, acc);
        acc = fma((double)u.w, (double)v.w, acc);
    };
    int c = 0;
    for (; c + U <= n4; c += U) {
        float4 u[U], v[U];
#pragma unroll
        for (int k = 0; k < U; ++k) {
            u[k] = x[c + k];
            v[k] = y[c + k];
        }
#pragma unroll
        for (int k = 0; k < U; ++k) add4(u[k], v[k]);
    }
    for (; c < n4; ++c) add4(x[c], y[c]);
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
    ev.z = mass * ev.r + far_wave_scan(ev.e);
    return ev;
}

// Far-part modes: where a row's per-landmark far max, rescale, mass and eviction weights come
// from.
enum FarMode {
    kFarFromWorkspace = 0,   // the chunk's evictions, scored by far_evict_kernel
    kFarFusedOneRow = 1,     // one-row call: the row's own eviction is scored here
    kFarCurrent = 2,         // no evictions in the call: the state in mz is current
};

// The far partial of one (row i, head gh): a workgroup of 256 threads. Every operand is loaded
// in a few wide rounds (mu and t_hat are prefetched at the start), dot products and landmark
// sums are split across lanes, and the per-landmark scalars live in wave 0, lane b.
// DP = padded head width (64, 128, 256): the partial row has DP floats. DEV: the partial is
// read within the same launch by workgroups that may run on other XCDs, so it is stored with
// the device-scope cache policy (written through to the device-coherent level); the caller
// waits for those stores before it signals them.
template <int DP, int MODE, bool DEV = false>
__device__ __forceinline__ void far_part_block(const FarParams& p, const int bid) {
    constexpr int NT = 256;
    constexpr int D4P = DP / 4;             // float4 columns of a partial row
    constexpr int S = NT / D4P;             // column slices in the numerator phase
    constexpr int TH = (kFarMaxLandmarks + S - 1) / S;   // landmarks per slice, at most
    constexpr int EV = (kFarMaxRows + S - 1) / S;        // evicted rows per slice, at most
    constexpr int MU = kFarMaxLandmarks * kFarMaxLandmarks / NT;   // mu entries per thread
    __shared__ double s_fl[64], s_fe[64], s_ea[64], s_gn[64], s_gain[64];
    __shared__ double s_up[NT], s_cfp[NT];
    __shared__ double s_acc[NT * 4];
    __shared__ int s_have;
    __shared__ float s_pm, s_F;

    const int t = threadIdx.x, lane = t & 63;
    const int i = bid / p.nh, gh = bid % p.nh;
    const int g = gh / p.hpg, m = p.m, d4 = p.d / 4;
    const GroupState gs = group_state(p, g);
    const int j0 = MODE == kFarCurrent ? 0x7fffffff : gs.j0;

    // This (row, head)'s slot in the partial buffer.
    const int qi = i * p.hpg + gh % p.hpg;   // query index within the group, row-major
    const int blk = g * p.nqblocks + qi / p.qb;
    const size_t at = ((size_t)blk * p.slot_stride + p.far_slot) * p.qb + qi % p.qb;
    float4* acc_out = reinterpret_cast<float4*>(p.pacc + at * DP);
    auto put_acc = [&](int c, float4 v) {
        if constexpr (DEV) {
            const __amdgpu_buffer_rsrc_t r =
                __builtin_amdgcn_make_buffer_rsrc(acc_out, 0, DP * 4, kBufferWord3);
            __builtin_amdgcn_raw_buffer_store_b128(vu4{__float_as_uint(v.x), __float_as_uint(v.y),
                                                       __float_as_uint(v.z), __float_as_uint(v.w)},
                                                   r, c * 16, 0, kCachePolicyDevice);
        } else {
            acc_out[c] = v;
        }
    };
    auto put_ml = [&](float mv, float lv) {
        if constexpr (DEV) {
            store_dev(p.pm + at, mv);
            store_dev(p.pl + at, lv);
        } else {
            p.pm[at] = mv;
            p.pl[at] = lv;
        }
    };

    const long long farl = (long long)gs.far0 + (i >= j0 ? i - j0 + 1 : 0);
    if (farl <= 0) {   // empty far field: an empty partial
        if (t < D4P) put_acc(t, make_float4(0.f, 0.f, 0.f, 0.f));
        if (t == 0) put_ml(-INFINITY, 0.0f);
        return;
    }

    int mp = 4;
    while (mp < m) mp <<= 1;
    const int tpl = NT / mp;   // threads per landmark in the dot phase (4 .. 64)

    // Every operand is loaded up front from an address clamped into range, so that no load
    // sits behind a branch whose join would wait for it; the predicates apply where the values
    // are used. This thread's mu entries: landmark b = t % mp, rows a = t / mp + k tpl; t_hat
    // rows: column c = t % D4P, landmarks b = t / D4P + k S.
    const int bm = t % mp, am = t / mp;
    const int bmc = bm < m ? bm : m - 1;
    float mu_r[MU];
#pragma unroll
    for (int k = 0; k < MU; ++k) {
        const int a = min(am + k * tpl, m - 1);
        mu_r[k] = p.mu[((size_t)gh * m + a) * m + bmc];
    }
    const int cc = t % D4P, sl = t / D4P;
    const int ccc = cc < d4 ? cc : d4 - 1;
    float4 th_r[TH];
#pragma unroll
    for (int k = 0; k < TH; ++k) {
        const int b = min(sl + k * S, m - 1);
        th_r[k] = reinterpret_cast<const float4*>(p.t_hat + ((size_t)gh * m + b) * p.d)[ccc];
    }
    // Per-landmark state for wave 0, lane b (lanes b >= m load landmark m - 1 and ignore it).
    const size_t lb = (size_t)gh * m + (t < m ? t : m - 1);
    double MX, R = 1.0, Z, m_old = 0.0, mass = 0.0;
    if constexpr (MODE == kFarFromWorkspace) {
        MX = p.ev_mx[lb];
        R = p.ev_r[lb];
        Z = p.ev_z[lb * p.rows + i];
    } else {
        m_old = p.mz[(size_t)gh * 2 * m + (lb - (size_t)gh * m)];
        mass = p.mz[(size_t)gh * 2 * m + m + (lb - (size_t)gh * m)];
        MX = m_old;
        Z = mass;
    }
    const bool evicts1 = MODE == kFarFusedOneRow && j0 == 0;   // the one row evicts an entry
    // The one-row call's evicted value row, column cc (slice 0 uses it).
    const float* v1row = evicts1 ? evicted_row(p, gs, g, 0, true) : p.ring_v + (size_t)g * p.w * p.d;
    const float4 v_ev1 = reinterpret_cast<const float4*>(v1row)[ccc];

    // Landmark scores fl_a = scale <q, k_tilde_a> (and for the fused one-row mode the eviction
    // scores fe_a = scale <q_tilde_a, K_ev>): tpl consecutive lanes per landmark.
    {
        const int a = t / tpl, sp = t % tpl;
        double v = 0.0, v2 = 0.0;
        if (a < m) {
            const float4* qv = reinterpret_cast<const float4*>(p.q + ((size_t)i * p.nh + gh) * p.d);
            const float4* kt = reinterpret_cast<const float4*>(p.k_tilde + ((size_t)g * m + a) * p.d);
            for (int c = sp; c < d4; c += tpl) {
                const float4 x = qv[c], y = kt[c];
                v = fma((double)x.x, (double)y.x, v);
                v = fma((double)x.y, (double)y.y, v);
                v = fma((double)x.z, (double)y.z, v);
                v = fma((double)x.w, (double)y.w, v);
            }
            if (evicts1) {
                const float4* qt = reinterpret_cast<const float4*>(p.q_tilde + ((size_t)gh * m + a) * p.d);
                const float4* kv = reinterpret_cast<const float4*>(evicted_row(p, gs, g, 0, false));
                for (int c = sp; c < d4; c += tpl) {
                    const float4 x = qt[c], y = kv[c];
                    v2 = fma((double)x.x, (double)y.x, v2);
                    v2 = fma((double)x.y, (double)y.y, v2);
                    v2 = fma((double)x.z, (double)y.z, v2);
                    v2 = fma((double)x.w, (double)y.w, v2);
                }
            }
        }
        if (tpl == 4) {
            v = far_group_sum<4>(v);
            v2 = far_group_sum<4>(v2);
        } else if (tpl == 8) {
            v = far_group_sum<8>(v);
            v2 = far_group_sum<8>(v2);
        } else if (tpl == 16) {
            v = far_group_sum<16>(v);
            v2 = far_group_sum<16>(v2);
        } else {   // 32 or 64 threads per landmark (at most 8 landmarks)
            for (int k = tpl >> 1; k >= 1; k >>= 1) {
                v += __shfl_xor(v, k);
                v2 += __shfl_xor(v2, k);
            }
        }
        if (sp == 0 && a < m) {
            s_fl[a] = (double)p.scale * v;
            s_fe[a] = (double)p.scale * v2;
        }
    }
    __syncthreads();

    // Wave 0: f = max fl, exp(fl_a - f); the fused mode's eviction of landmark b.
    double f = 0.0, E = 0.0;
    if (t < 64) {
        const double fl = lane < m ? s_fl[lane] : -INFINITY;
        f = far_wave_max(fl);
        s_ea[lane] = lane < m ? exp(fl - f) : 0.0;
        if (evicts1 && lane < m) {
            const double fe = s_fe[lane];
            MX = fmax(m_old, fe);
            R = MX == m_old ? 1.0 : exp(m_old - MX);
            E = exp(fe - MX);
            Z = mass * R + E;
        }
    }
    __syncthreads();

    // Weights u_b = sum_a exp(fl_a - f) mu[a][b]: partial sums over this thread's rows a.
    {
        double u = 0.0;
#pragma unroll
        for (int k = 0; k < MU; ++k) {
            const int a = am + k * tpl;
            if (a < m) u = fma(s_ea[a], (double)mu_r[k], u);
        }
        s_up[t] = u;   // index am * mp + bm == t
    }
    __syncthreads();

    // Wave 0, lane b: u_b, the optional clamp, the gains against the partial's rounded max,
    // the far mass F, and (fused mode) the weight of the row's own eviction.
    if (t < 64) {
        double u = 0.0;
        if (lane < m)
            for (int a = 0; a < tpl; ++a) u += s_up[a * mp + lane];
        if (p.rect && u < 0.0) u = 0.0;
        const double Mb = lane < m ? f + MX : -INFINITY;   // lanes >= m hold landmark m - 1
        const float pm = (float)(far_wave_max(Mb) * kLog2eD);
        const double Mr = (double)pm / kLog2eD;
        const double gain = lane < m ? u * exp(Mb - Mr) : 0.0;
        const double F = far_wave_sum(lane < m ? gain * Z : 0.0);
        s_gain[lane] = gain;
        s_gn[lane] = lane < m ? gain * R : 0.0;
        if (MODE == kFarFusedOneRow) {
            const double cf0 = far_wave_sum(lane < m ? gain * E : 0.0);
            if (lane == 0) s_cfp[0] = cf0;
        }
        if (lane == 0) {
            s_have = F >= 0.0 && pm > -INFINITY;
            s_pm = pm;
            s_F = (float)F;
        }
    }
    __syncthreads();
    if (!s_have) {   // negative far mass: the far part is dropped
        if (t < D4P) put_acc(t, make_float4(0.f, 0.f, 0.f, 0.f));
        if (t == 0) put_ml(-INFINITY, 0.0f);
        return;
    }

    // Weights of the evicted rows j0 <= j <= i: cf_j = sum_b gain_b e_b(j), four partial sums
    // per row (wave w takes landmarks b = w mod 4).
    const int jlo = j0 > 0 ? j0 : 0;
    if constexpr (MODE == kFarFromWorkspace) {
        const int j = lane, w = t >> 6;
        const int jc = min(j, p.rows - 1);
        double e_r[kFarMaxLandmarks / 4];
#pragma unroll
        for (int k = 0; k < kFarMaxLandmarks / 4; ++k)
            e_r[k] = p.ev_e[((size_t)gh * m + min(w + 4 * k, m - 1)) * p.rows + jc];
        double cf = 0.0;
#pragma unroll
        for (int k = 0; k < kFarMaxLandmarks / 4; ++k)
            if (w + 4 * k < m) cf = fma(s_gain[w + 4 * k], e_r[k], cf);
        s_cfp[t] = j >= jlo && j <= i ? cf : 0.0;   // index w * 64 + j
        __syncthreads();
    }

    // Numerator, column cc, slice sl: landmarks b = sl + k S and evicted rows j = jlo + sl + k S.
    double ax = 0.0, ay = 0.0, az = 0.0, aw = 0.0;
#pragma unroll
    for (int k = 0; k < TH; ++k) {
        const int b = sl + k * S;
        const double gn = b < m ? s_gn[b] : 0.0;
        ax = fma(gn, (double)th_r[k].x, ax);
        ay = fma(gn, (double)th_r[k].y, ay);
        az = fma(gn, (double)th_r[k].z, az);
        aw = fma(gn, (double)th_r[k].w, aw);
    }
    if (MODE == kFarFusedOneRow && evicts1 && sl == 0) {
        const double cf = s_cfp[0];
        ax = fma(cf, (double)v_ev1.x, ax);
        ay = fma(cf, (double)v_ev1.y, ay);
        az = fma(cf, (double)v_ev1.z, az);
        aw = fma(cf, (double)v_ev1.w, aw);
    }
    if (MODE == kFarFromWorkspace && i >= jlo) {
        // rows past i load row i and are dropped at use
        float4 vr[EV];
#pragma unroll
        for (int k = 0; k < EV; ++k) {
            const int j = min(jlo + sl + k * S, i);
            vr[k] = reinterpret_cast<const float4*>(evicted_row(p, gs, g, j, true))[ccc];
        }
#pragma unroll
        for (int k = 0; k < EV; ++k) {
            const int j = jlo + sl + k * S;
            if (j <= i) {
                const double cf = s_cfp[j] + s_cfp[64 + j] + s_cfp[128 + j] + s_cfp[192 + j];
                ax = fma(cf, (double)vr[k].x, ax);
                ay = fma(cf, (double)vr[k].y, ay);
                az = fma(cf, (double)vr[k].z, az);
                aw = fma(cf, (double)vr[k].w, aw);
            }
        }
    }
    s_acc[4 * t + 0] = ax;
    s_acc[4 * t + 1] = ay;
    s_acc[4 * t + 2] = az;
    s_acc[4 * t + 3] = aw;
    __syncthreads();
    if (t < D4P) {
        double x = 0.0, y = 0.0, z = 0.0, w = 0.0;
        for (int k = 0; k < S; ++k) {
            const int u = 4 * (k * D4P + t);
            x += s_acc[u];
            y += s_acc[u + 1];
            z += s_acc[u + 2];
            w += s_acc[u + 3];
        }
        put_acc(t, t < d4 ? make_float4((float)x, (float)y, (float)z, (float)w)
                          : make_float4(0.f, 0.f, 0.f, 0.f));
    }
    if (t == 0) put_ml(s_pm, s_F);   // the merge works in the log2 domain
}

}  // namespace
}  // namespace winattn
