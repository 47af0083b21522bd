// Split-K windowed attention for decode-sized chunks (at most 8 query vectors per KV group per
// workgroup), computed entirely in registers.
//
// Prior art on the o1c page ("A sealed layer's attention for a chunk of rows, on Metal"): the
// token path `o1c_tok_near` gives each simdgroup a stripe of the window's keys, keeps the row's
// queries in registers and updates a running (max, sum, accumulator) per head, and
// `o1c_tok_merge` combines the partials. The gfx950 design:
//
//  - A lane group of TPK = D*NQ/32 adjacent lanes owns one key per pass: lane sl of the group
//    holds float4 columns sl, sl + TPK, ... of that key's K and V row (TPK lanes read TPK*16
//    consecutive bytes, so each load instruction is fully coalesced) and the same columns of
//    every query (32 floats per lane).
//  - Scores are partial dot products reduced across the group with DPP, which leaves the full
//    score in every lane of the group, exactly where the value update needs it.
//  - Each lane group is its own split: it keeps a running max, sum and accumulator per query
//    over the keys it owns. No LDS and no barrier inside the tile loop; the groups are merged
//    once at the end through LDS, and the workgroups' splits by the merge launch (or by the
//    last-arriving workgroup).
//  - The queries are requested before the key tiles, and every tile load is straight-line code,
//    so a tile's arithmetic waits only for that tile's loads. A split of up to three tiles has
//    all of them requested at once (straight-line instance); a longer split keeps two register
//    buffers, each refilled as soon as its tile has been consumed (loop instance).
#pragma once
#include <type_traits>

#include "winattn_dev.h"

namespace winattn {

template <int D, int NQ>
struct DecShape {
    static constexpr int TPK = D * NQ / 32;     // lanes per key
    static constexpr int F4 = D / (4 * TPK);    // float4 columns of a key per lane
    static constexpr int KPP = kThreads / TPK;  // keys per pass of the block = lane groups
    static constexpr int TK = 4096 / D;         // keys per tile: 4 float4 per lane per tensor
    static constexpr int PASSES = TK / KPP;
    static_assert(TPK >= 4 && TPK <= 64 && F4 >= 1 && PASSES >= 1, "unsupported shape");
    static_assert(PASSES * F4 == 4, "four float4 of K and of V per lane per tile");
};

// Given per-row sums (every lane of a 16-lane row holds its row's sum), the sum over the
// TPK = 32 or 64 lanes of the group, in every lane of the group: rows 0-1 and 2-3 meet by
// gfx950's row swap, the two halves of the wave by its half-wave swap (no lane reads through
// scalar registers).
template <int TPK>
__device__ inline float lane_group_sum_above16(float v) {
    static_assert(TPK == 32 || TPK == 64, "groups above 16 lanes are 32 or 64 wide");
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    if constexpr (TPK == 64) v = half_swap_sum(v);
    return v;
}

// Sum over the TPK lanes of a group of each of N values, result in every lane of the group.
// The DPP steps of the N values are interleaved level by level, so that no step waits on the
// one just before it.
template <int TPK, int N>
__device__ inline void lane_group_sum_n(float* v) {
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] += dpp<kDppXor1>(v[i], 0.0f);
    if constexpr (TPK >= 4) {
#pragma unroll
        for (int i = 0; i < N; ++i) v[i] += dpp<kDppXor2>(v[i], 0.0f);
    }
    if constexpr (TPK >= 8) {
#pragma unroll
        for (int i = 0; i < N; ++i) v[i] += dpp<kDppHalfMirror>(v[i], 0.0f);
    }
    if constexpr (TPK >= 16) {
#pragma unroll
        for (int i = 0; i < N; ++i) v[i] += dpp<kDppMirror>(v[i], 0.0f);
    }
    if constexpr (TPK > 16) {
#pragma unroll
        for (int i = 0; i < N; ++i) v[i] = lane_group_sum_above16<TPK>(v[i]);
    }
}

// One workgroup of the register kernel: split `split` of query block `qb` of group g. SHORT:
// every split of the launch has at most three tiles, run as straight-line code; otherwise a
// loop with two register buffers.
template <int D, int NQ, bool GATED, bool SHORT>
__device__ __forceinline__ void attn_dec_block(const AttnParams& p, const int split, const int qb,
                                               const int g) {
    using S = DecShape<D, NQ>;
    constexpr int TPK = S::TPK, F4 = S::F4, KPP = S::KPP, TK = S::TK, PASSES = S::PASSES;

    __shared__ __align__(16) float s_red[KPP * NQ * D];   // group accumulators at the end
    __shared__ float s_gm[KPP * NQ], s_gl[KPP * NQ];
    __shared__ float s_m[NQ], s_l[NQ];
    __shared__ int s_flag;
    static_assert(KPP * NQ * D >= kMergeScratch, "merge scratch reuses the reduction area");

    const int tid = threadIdx.x;
    const int gi = tid / TPK, sl = tid % TPK;   // lane group (key slot), lane within the group
    const int nq_tot = p.rows * p.hpg;
    const int q0 = qb * NQ;
    const int nq = min(NQ, nq_tot - q0);
    // ---- queries first: this lane's columns of every query, times scale*log2(e). They are
    // requested before the key tiles, so that the first tile's arithmetic waits only for that
    // tile and overlaps the arrival of the next one (vector loads return in issue order). The
    // addresses are clamped to a live element of the query and padding is scaled by 0.
    vf4 qr[NQ][F4];
    {
        const int d4q = p.d / 4;
#pragma unroll
        for (int j = 0; j < NQ; ++j) {
            const int qi = q0 + min(j, nq - 1);
            const int row = qi / p.hpg, gh = g * p.hpg + qi % p.hpg;
            const float* qp = p.q + ((size_t)row * p.nh + gh) * p.d;
#pragma unroll
            for (int f = 0; f < F4; ++f) {
                const int c = sl + TPK * f;
                const bool live = (j < nq) & (c < d4q);
                const vf4 v = *reinterpret_cast<const vf4*>(qp + 4 * (c < d4q ? c : 0));
                // a select on the loaded value lets the compiler move the load behind a branch
                // (and wait on it there); a factor of 0 keeps the load unconditional
                qr[j][f] = v * (live ? p.scale_log2 : 0.0f);
            }
        }
    }
    const GroupWin gw = resolve_group<GATED>(p, g);
    const int r_first = q0 / p.hpg, r_last = (q0 + nq - 1) / p.hpg;
    const int xlo = window_lo(gw.hi0 + r_first, gw.wcap);
    const int xhi = gw.hi0 + r_last;
    const Tiles tr = tile_range<TK>(p.ns, xlo, xhi, p.nsplit_grid, split);
    const int nsplit = tr.nsplit, nst = tr.nst;
    if (split >= nsplit) {
        mark_split_empty<NQ>(p, g * p.nqblocks + qb, split);
        return;
    }
    const int t_begin = tr.t_begin, t_end = tr.t_end;
    const int d4 = p.d / 4;

    // ---- tile loads: key of (pass, group) = tile base + pass * KPP + gi; columns sl + TPK f
    const KVBases b = kv_bases(p);
    const unsigned long long rk = b.rk + 4ull * (unsigned long long)((long long)g * p.ring_gs);
    const unsigned long long rv = b.rv + 4ull * (unsigned long long)((long long)g * p.ring_gs);
    const unsigned long long ck = b.ck + 4ull * (unsigned long long)((long long)g * p.chunk_gs);
    const unsigned long long cv = b.cv + 4ull * (unsigned long long)((long long)g * p.chunk_gs);
    const unsigned long long sk = b.sk + 4ull * (unsigned long long)((long long)g * p.ns * p.d);
    const unsigned long long sv = b.sv + 4ull * (unsigned long long)((long long)g * p.ns * p.d);
    const int ss = (int)p.ring_ss, crs = (int)p.chunk_rs;

    vf4 kA[PASSES][F4], vA[PASSES][F4], kB[PASSES][F4], vB[PASSES][F4];
    vf4 kC[PASSES][F4], vC[PASSES][F4];   // third buffer (straight-line instance only)
    // Every load reads a live row: a padding key (past the sinks, or past the block's stream
    // range) loads sink 0 or the block's last stream entry, and a column past d loads the key's
    // first columns. Its score is masked to -inf, so its weight is exactly 0 and 0 times finite
    // data adds nothing: no select on K, V or the accumulators is needed.
    // Sink and stream tiles share one set of loads: the base and row are selected, not
    // branched on, so each buffer's loads are straight-line code and the waits before a tile's
    // arithmetic count only the loads issued after it. Every key is read once per call, so the
    // loads are non-temporal: the stream does not displace the kernel's code, queries and
    // metadata from the caches (a 32768-slot decode: 56.8 -> 50.8 us per call).
    const unsigned long long dkc = ck - rk, dks = sk - rk, dvc = cv - rv, dvs = sv - rv;
    auto load_tile = [&](vf4 (&kr)[PASSES][F4], vf4 (&vr)[PASSES][F4], int t) {
        const bool sink_tile = t < nst;   // uniform over the block
        const int xt = xlo + (t - nst) * TK + gi;
#pragma unroll
        for (int ps = 0; ps < PASSES; ++ps) {
            const int si = t * TK + ps * KPP + gi;
            const int x = min(xt + ps * KPP, xhi - 1);
            const bool in_ring = x < gw.xsplit;
            int slot = gw.base + x;
            slot = slot >= gw.mod ? slot - gw.mod : slot;
            const int srow = si < p.ns ? si * p.d : 0;
            const int xrow = in_ring ? slot * ss : (x - gw.xsplit) * crs;
            const int row = sink_tile ? srow : xrow;
            // base = ring + (chunk - ring if a chunk row) + (sink - ring if a sink tile): two
            // independent selects of uniform differences (a select chain of the three bases
            // becomes a lookup table in private memory)
            const bool chunk_key = !in_ring & !sink_tile;
            const unsigned long long bk = rk + (chunk_key ? dkc : 0ull) + (sink_tile ? dks : 0ull);
            const unsigned long long bv = rv + (chunk_key ? dvc : 0ull) + (sink_tile ? dvs : 0ull);
#pragma unroll
            for (int f = 0; f < F4; ++f) {
                const int c = sl + TPK * f;
                const int off = c < d4 ? row + 4 * c : row;
                kr[ps][f] = __builtin_nontemporal_load(reinterpret_cast<gvf4p>(bk + 4ull * (unsigned)off));
                vr[ps][f] = __builtin_nontemporal_load(reinterpret_cast<gvf4p>(bv + 4ull * (unsigned)off));
            }
        }
    };
    // The second buffer is always filled (a one-tile split loads its tile twice), so that the
    // first tile's arithmetic waits only for the first tile's loads on every path.
    const int nt = t_end - t_begin;
    load_tile(kA, vA, t_begin);
    load_tile(kB, vB, min(t_begin + 1, t_end - 1));
    // A three-tile split (split 0 of a decode call: the sink tile and two stream tiles) has its
    // third tile requested up front too, so it does not queue behind the whole ring's traffic
    // after the first tile's arithmetic.
    if constexpr (SHORT) {
        if (nt == 3) load_tile(kC, vC, t_begin + 2);
    }

    // ---- window bounds of every query
    int qlo[NQ], qhi[NQ];
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
        const int hi = gw.hi0 + (q0 + min(j, nq - 1)) / p.hpg;
        qlo[j] = j < nq ? window_lo(hi, gw.wcap) : 0;
        qhi[j] = j < nq ? hi : 0;
    }

    float mrun[NQ], lrun[NQ];
    vf4 acc[NQ][F4];
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
        mrun[j] = -INFINITY;
        lrun[j] = 0.0f;
#pragma unroll
        for (int f = 0; f < F4; ++f) acc[j][f] = vf4{0.f, 0.f, 0.f, 0.f};
    }

    // ---- one tile: scores, online softmax of this lane group, value update
    auto step = [&](vf4 (&kr)[PASSES][F4], vf4 (&vr)[PASSES][F4], int t, auto refill) {
        // partial dot products over this lane's columns (q is zero past d), then summed over
        // the lane group
        float sc[PASSES * NQ];
#pragma unroll
        for (int ps = 0; ps < PASSES; ++ps)
#pragma unroll
            for (int j = 0; j < NQ; ++j) {
                float s = 0.0f;
#pragma unroll
                for (int f = 0; f < F4; ++f) {
                    float h = kr[ps][f].x * qr[j][f].x;
                    h = __builtin_fmaf(kr[ps][f].y, qr[j][f].y, h);
                    h = __builtin_fmaf(kr[ps][f].z, qr[j][f].z, h);
                    h = __builtin_fmaf(kr[ps][f].w, qr[j][f].w, h);
                    s = f == 0 ? h : s + h;
                }
                sc[ps * NQ + j] = s;
            }
        constexpr int kSumMax = 8;   // sums of 8 values interleaved level by level
        constexpr int kSumBlock = PASSES * NQ < kSumMax ? PASSES * NQ : kSumMax;
#pragma unroll
        for (int b = 0; b < PASSES * NQ; b += kSumBlock) lane_group_sum_n<TPK, kSumBlock>(sc + b);
        // Visibility, branch free: a stream key at entry x is visible to a query whose window
        // is [lo, hi) (padding queries have empty windows); a real sink to every real query.
        const int sink_tile = t < nst;   // uniform over the block
#pragma unroll
        for (int ps = 0; ps < PASSES; ++ps) {
            const int k = ps * KPP + gi;
            const int x = xlo + (t - nst) * TK + k;
            const int sink_real = sink_tile & (t * TK + k < p.ns);
#pragma unroll
            for (int j = 0; j < NQ; ++j) {
                const int in_win = (x >= qlo[j]) & (x < qhi[j]) & (sink_tile ^ 1);
                const int vis = in_win | (sink_real & (j < nq));
                sc[ps * NQ + j] = vis ? sc[ps * NQ + j] : -INFINITY;
            }
        }
#pragma unroll
        for (int j = 0; j < NQ; ++j) {
            float tmax = sc[j];
#pragma unroll
            for (int ps = 1; ps < PASSES; ++ps) tmax = fmaxf(tmax, sc[ps * NQ + j]);
            const float m_new = fmaxf(mrun[j], tmax);
            const float mu = safe_max(m_new);
            const float corr = __builtin_amdgcn_exp2f(mrun[j] - mu);
            mrun[j] = m_new;
            float lsum = 0.0f;
#pragma unroll
            for (int f = 0; f < F4; ++f) acc[j][f] *= corr;
#pragma unroll
            for (int ps = 0; ps < PASSES; ++ps) {
                const float pv = __builtin_amdgcn_exp2f(sc[ps * NQ + j] - mu);
                lsum += pv;
#pragma unroll
                for (int f = 0; f < F4; ++f) {
                    acc[j][f].x = __builtin_fmaf(pv, vr[ps][f].x, acc[j][f].x);
                    acc[j][f].y = __builtin_fmaf(pv, vr[ps][f].y, acc[j][f].y);
                    acc[j][f].z = __builtin_fmaf(pv, vr[ps][f].z, acc[j][f].z);
                    acc[j][f].w = __builtin_fmaf(pv, vr[ps][f].w, acc[j][f].w);
                }
            }
            lrun[j] = lrun[j] * corr + lsum;
        }
        if constexpr (decltype(refill)::value) {
            if (t + 2 < t_end) load_tile(kr, vr, t + 2);
        }
    };
    if constexpr (SHORT) {
        // Straight line for splits of up to three tiles (decode): no loop-carried buffers, so
        // the compiler has no register copies to make, and a copy would wait for every load.
        step(kA, vA, t_begin, std::false_type{});
        if (nt >= 2) step(kB, vB, t_begin + 1, std::false_type{});
        if (nt == 3) step(kC, vC, t_begin + 2, std::false_type{});
    } else {
        for (int t = t_begin; t < t_end; t += 2) {
            step(kA, vA, t, std::true_type{});
            if (t + 1 < t_end) step(kB, vB, t + 1, std::true_type{});
        }
    }

    // ---- merge the lane groups (each group's state is uniform across its lanes)
    if (sl == 0) {
#pragma unroll
        for (int j = 0; j < NQ; ++j) {
            s_gm[gi * NQ + j] = mrun[j];
            s_gl[gi * NQ + j] = lrun[j];
        }
    }
    __syncthreads();
    if (tid < NQ) {
        float m = -INFINITY;
        for (int u = 0; u < KPP; ++u) m = fmaxf(m, s_gm[u * NQ + tid]);
        const float mu = safe_max(m);
        float l = 0.0f;
        for (int u = 0; u < KPP; ++u) l += s_gl[u * NQ + tid] * __builtin_amdgcn_exp2f(s_gm[u * NQ + tid] - mu);
        s_m[tid] = m;
        s_l[tid] = l;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
        const float f = __builtin_amdgcn_exp2f(mrun[j] - safe_max(s_m[j]));
#pragma unroll
        for (int fc = 0; fc < F4; ++fc)
            *reinterpret_cast<vf4*>(s_red + (gi * NQ + j) * D + 4 * (sl + TPK * fc)) = acc[j][fc] * f;
    }
    __syncthreads();

    const int blk = g * p.nqblocks + qb;
    constexpr int D4 = D / 4;
    for (int item = tid; item < NQ * D4; item += kThreads) {
        const int j = item / D4, c = item % D4;
        if (j >= nq || c >= d4) continue;
        vf4 o = {0.f, 0.f, 0.f, 0.f};
        for (int u = 0; u < KPP; ++u) o += *reinterpret_cast<const vf4*>(s_red + (u * NQ + j) * D + 4 * c);
        if (nsplit == 1 && !p.merge_kernel) {
            o *= 1.0f / fmaxf(s_l[j], 1e-30f);
            store_out<GATED>(p, q0 + j, g, 4 * c, make_float4(o.x, o.y, o.z, o.w));
        } else {
            const size_t at = ((size_t)blk * p.slot_stride + split) * NQ + j;
            store_part4<NQ, D>(p, blk, split, j, 4 * c, make_float4(o.x, o.y, o.z, o.w));
            if (c == 0) {
                store_part(p, p.pm + at, s_m[j]);
                store_part(p, p.pl + at, s_l[j]);
            }
        }
    }
    if (nsplit > 1) {
        __syncthreads();   // s_red is reused as merge scratch
        merge_if_last<NQ, D, GATED>(p, blk, nsplit, q0, nq, g, &s_flag, s_red);
    }
}

}  // namespace winattn
