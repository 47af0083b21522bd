// Split-K windowed attention on the vector ALUs, for chunks with few query vectors per KV
// group (decode and short verify chunks: rows * hpg <= 16).
//
// Prior art on the o1c page ("A sealed layer's attention for a chunk of rows, on Metal"): the
// token path's flash-decoding partials (`o1c_tok_near`: a threadgroup per (group, key split),
// a running max, sum and accumulator per query, merged by `o1c_tok_merge`). On gfx950 the
// design differs: a 256-thread workgroup owns one (group, query block, key split); each key
// tile is read from HBM once, coalesced (a wave's 64 lanes read 1 KiB of consecutive rows),
// staged in LDS and shared by every query of the block; scores, the softmax step and the value
// sum each read the tile once from LDS. Splits merge in the last-arriving workgroup.
//
// Thread roles per tile of TK keys:
//   load   thread t loads float4 f = t + 256 j of the K and V tiles (key f / (D/4))
//   score  TPK adjacent lanes share a key, each a D/TPK slice of it, for all NQ queries,
//          then reduce across the TPK lanes
//   softmax wave w updates queries w, w+4, ... over the tile (lane = key)
//   value  thread t owns float4 column t % (D/4) of every query for key set t / (D/4);
//          the key sets are summed once, after the last tile
#include "winattn_dev.h"
#include "launch.h"

namespace winattn {

template <int D, int NQ>
struct ValuShape {
    static constexpr int TK = (D == 256) ? 32 : 64;   // keys per tile
    static constexpr int D4 = D / 4;
    static constexpr int TPK = kThreads / TK;         // lanes per key in the score phase
    static constexpr int SL = D / TPK;                // floats of a key per lane
    static constexpr int KS = kThreads / D4;          // key sets in the value phase
    static constexpr int KPT = TK / KS;               // keys per thread in the value phase
    static constexpr int KST = D + 4;                 // LDS row stride of K
    static constexpr int LPT = TK * D4 / kThreads;    // float4 loads per thread per tensor
    static constexpr int TILE_FLOATS = TK * KST + TK * D;
    static constexpr int RED_FLOATS = KS * NQ * D;
    static constexpr int UNION_FLOATS = TILE_FLOATS > RED_FLOATS ? TILE_FLOATS : RED_FLOATS;
    static_assert(SL % 4 == 0, "score slice must be whole float4s");
    static_assert(KS * D4 == kThreads && KPT * KS == TK, "value phase must tile the block");
    static_assert(NQ % 4 == 0, "four waves share the softmax");
    static_assert(TPK == 4 || TPK == 8, "a key's lanes reduce within a row");
    static_assert(UNION_FLOATS >= kMergeScratch, "merge scratch reuses the tile area");
};

template <int D, int NQ, bool GATED>
__global__ __launch_bounds__(kThreads) void attn_valu_kernel(const AttnParams p) {
    using S = ValuShape<D, NQ>;
    constexpr int TK = S::TK, D4 = S::D4, TPK = S::TPK, SL = S::SL, KS = S::KS, KPT = S::KPT;
    constexpr int KST = S::KST, LPT = S::LPT;

    __shared__ __align__(16) float s_union[S::UNION_FLOATS];   // K|V tile, later the reduction
    __shared__ __align__(16) float s_q[NQ * D];
    __shared__ __align__(16) float s_p[TK * NQ];               // scores, then weights: [key][q]
    __shared__ float s_corr[NQ], s_m[NQ], s_l[NQ];
    __shared__ int s_lo[NQ], s_hi[NQ], s_sink[NQ];
    __shared__ int s_flag;

    float* s_k = s_union;
    float* s_v = s_union + TK * KST;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int split = blockIdx.x, qb = blockIdx.y, g = blockIdx.z;
    const int nq_tot = p.rows * p.hpg;
    const int q0 = qb * NQ;
    const int nq = min(NQ, nq_tot - q0);
    const GroupWin gw = resolve_group<GATED>(p, g);

    // The block's stream range: from the first row's window start to the last row's end.
    const int r_first = q0 / p.hpg, r_last = (q0 + nq - 1) / p.hpg;
    const int hi_first = gw.hi0 + r_first;
    const int xlo = window_lo(hi_first, gw.wcap);
    const int xhi = gw.hi0 + r_last;
    const Tiles tr = tile_range<TK>(p.ns, xlo, xhi, p.nsplit_grid, split);
    const int nsplit = tr.nsplit, nst = tr.nst;
    if (split >= nsplit) {
        mark_split_empty<NQ>(p, g * p.nqblocks + qb, split);
        return;
    }
    const int t_begin = tr.t_begin, t_end = tr.t_end;
    const int d4 = p.d / 4;

    // Two register tile buffers: both of a split's first tiles are requested at once, and a
    // buffer is refilled as soon as its tile has been copied to LDS.
    float4 kA[LPT], vA[LPT], kB[LPT], vB[LPT];
    unsigned mA = 0u, mB = 0u;
    const KVBases kvb = kv_bases(p);
    auto load_tile = [&](float4 (&kr)[LPT], float4 (&vr)[LPT], unsigned& m, int t) {
        m = load_tile_regs<TK, D, LPT>(p, kvb, gw, g, xlo, xhi, nst, t, d4, kr, vr);
    };

    load_tile(kA, vA, mA, t_begin);   // first tiles in flight while the queries are staged
    if (t_begin + 1 < t_end) load_tile(kB, vB, mB, t_begin + 1);

    // Per-query window in key-index space, and the scaled queries.
    if (tid < NQ) {
        const int j = tid;
        if (j < nq) {
            const int row = (q0 + j) / p.hpg;
            const int hi = gw.hi0 + row;
            s_lo[j] = window_lo(hi, gw.wcap);
            s_hi[j] = hi;
            s_sink[j] = 1;
        } else {
            s_lo[j] = 0;
            s_hi[j] = 0;
            s_sink[j] = 0;
        }
    }
    for (int f = tid; f < NQ * D4; f += kThreads) {
        const int j = f / D4, c = f % D4;
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (j < nq && c < d4) {
            const int qi = q0 + j;
            const int row = qi / p.hpg, gh = g * p.hpg + qi % p.hpg;
            v = *reinterpret_cast<const float4*>(p.q + ((size_t)row * p.nh + gh) * p.d + 4 * c);
            v.x *= p.scale_log2; v.y *= p.scale_log2; v.z *= p.scale_log2; v.w *= p.scale_log2;
        }
        *reinterpret_cast<float4*>(s_q + j * D + 4 * c) = v;
    }

    float mrun[NQ / 4], lrun[NQ / 4];
#pragma unroll
    for (int m = 0; m < NQ / 4; ++m) {
        mrun[m] = -INFINITY;
        lrun[m] = 0.0f;
    }
    float4 pacc[NQ];
#pragma unroll
    for (int j = 0; j < NQ; ++j) pacc[j] = make_float4(0.f, 0.f, 0.f, 0.f);

    const int skey = tid / TPK, sl = tid % TPK;       // score role
    const int vc = tid % D4, vks = tid / D4;          // value role

    auto step = [&](float4 (&kr)[LPT], float4 (&vr)[LPT], unsigned& m, int t) {
        __syncthreads();   // the previous tile's readers are done with s_k, s_v, s_p
#pragma unroll
        for (int j = 0; j < LPT; ++j) {
            const int f = tid + kThreads * j;
            const int key = f / D4, c = f % D4;
            const bool keep = (m >> j) & 1u;
            *reinterpret_cast<float4*>(s_k + key * KST + 4 * c) = zero_unless(keep, kr[j]);
            *reinterpret_cast<float4*>(s_v + key * D + 4 * c) = zero_unless(keep, vr[j]);
        }
        __syncthreads();
        if (t + 2 < t_end) load_tile(kr, vr, m, t + 2);   // refill this buffer two tiles ahead

        // Scores: lanes sl of key skey hold slices; reduce over the TPK adjacent lanes.
        {
            float acc[NQ];
#pragma unroll
            for (int j = 0; j < NQ; ++j) acc[j] = 0.0f;
            const float* krow = s_k + skey * KST + sl * SL;
#pragma unroll
            for (int c = 0; c < SL / 4; ++c) {
                const float4 kv = *reinterpret_cast<const float4*>(krow + 4 * c);
#pragma unroll
                for (int j = 0; j < NQ; ++j) {
                    const float4 qv = *reinterpret_cast<const float4*>(s_q + j * D + sl * SL + 4 * c);
                    acc[j] = fmaf(kv.x, qv.x, acc[j]);
                    acc[j] = fmaf(kv.y, qv.y, acc[j]);
                    acc[j] = fmaf(kv.z, qv.z, acc[j]);
                    acc[j] = fmaf(kv.w, qv.w, acc[j]);
                }
            }
#pragma unroll
            for (int j = 0; j < NQ; ++j) acc[j] = group_sum<TPK>(acc[j]);
#pragma unroll
            for (int j = 0; j < NQ; ++j) {
                if (j % TPK == sl) {
                    const bool vis = key_visible<TK>(p.ns, xlo, nst, t, skey, s_lo[j], s_hi[j],
                                                     s_sink[j] != 0);
                    s_p[skey * NQ + j] = vis ? acc[j] : -INFINITY;
                }
            }
        }
        __syncthreads();

        // Online softmax over the tile, one wave per query (lane = key).
#pragma unroll
        for (int m = 0; m < NQ / 4; ++m) {
            const int j = wave + 4 * m;
            const float s = lane < TK ? s_p[lane * NQ + j] : -INFINITY;
            const float m_new = fmaxf(mrun[m], wave_max(s));
            const float mu = safe_max(m_new);
            const float corr = __builtin_amdgcn_exp2f(mrun[m] - mu);
            const float pv = __builtin_amdgcn_exp2f(s - mu);
            lrun[m] = lrun[m] * corr + wave_sum(pv);
            mrun[m] = m_new;
            if (lane < TK) s_p[lane * NQ + j] = pv;
            if (lane == 0) s_corr[j] = corr;
        }
        __syncthreads();

        // Value sum for this thread's key set.
#pragma unroll
        for (int j = 0; j < NQ; ++j) {
            const float c = s_corr[j];
            pacc[j].x *= c; pacc[j].y *= c; pacc[j].z *= c; pacc[j].w *= c;
        }
#pragma unroll
        for (int kk = 0; kk < KPT; ++kk) {
            const int key = vks + KS * kk;
            const float4 v = *reinterpret_cast<const float4*>(s_v + key * D + 4 * vc);
#pragma unroll
            for (int jj = 0; jj < NQ / 4; ++jj) {
                const float4 w4 = *reinterpret_cast<const float4*>(s_p + key * NQ + 4 * jj);
                const float wv[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    float4& a = pacc[4 * jj + u];
                    a.x = fmaf(wv[u], v.x, a.x);
                    a.y = fmaf(wv[u], v.y, a.y);
                    a.z = fmaf(wv[u], v.z, a.z);
                    a.w = fmaf(wv[u], v.w, a.w);
                }
            }
        }
    };
    for (int t = t_begin; t < t_end; t += 2) {
        step(kA, vA, mA, t);
        if (t + 1 < t_end) step(kB, vB, mB, t + 1);
    }

    // Sum the key sets through LDS, then write the output or this split's partial.
    __syncthreads();
    float* s_red = s_union;
#pragma unroll
    for (int j = 0; j < NQ; ++j)
        *reinterpret_cast<float4*>(s_red + (vks * NQ + j) * D + 4 * vc) = pacc[j];
    if (lane == 0) {
#pragma unroll
        for (int m = 0; m < NQ / 4; ++m) {
            s_m[wave + 4 * m] = mrun[m];
            s_l[wave + 4 * m] = lrun[m];
        }
    }
    __syncthreads();

    const int blk = g * p.nqblocks + qb;
    for (int item = tid; item < NQ * D4; item += kThreads) {
        const int j = item / D4, c = item % D4;
        if (j >= nq || c >= d4) continue;
        float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const float4 a = *reinterpret_cast<const float4*>(s_red + (ks * NQ + j) * D + 4 * c);
            o.x += a.x; o.y += a.y; o.z += a.z; o.w += a.w;
        }
        if (nsplit == 1 && !p.merge_kernel) {
            const float inv = 1.0f / fmaxf(s_l[j], 1e-30f);
            o.x *= inv; o.y *= inv; o.z *= inv; o.w *= inv;
            store_out<GATED>(p, q0 + j, g, 4 * c, o);
        } else {
            const size_t at = ((size_t)blk * p.slot_stride + split) * NQ + j;
            store_part4<NQ, D>(p, blk, split, j, 4 * c, o);
            if (c == 0) {
                store_part(p, p.pm + at, s_m[j]);
                store_part(p, p.pl + at, s_l[j]);
            }
        }
    }
    if (nsplit > 1) merge_if_last<NQ, D, GATED>(p, blk, nsplit, q0, nq, g, &s_flag, s_union);
}

template <int D, int NQ, bool GATED>
static hipError_t launch_valu_t(const AttnParams& p, dim3 grid, hipStream_t stream) {
    hipLaunchKernelGGL((attn_valu_kernel<D, NQ, GATED>), grid, dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

template <bool GATED>
static hipError_t launch_valu_g(const AttnParams& p, int dpad, int nq, dim3 grid, hipStream_t s) {
#define WINATTN_VALU_CASE(DD, QQ) \
    if (dpad == DD && nq == QQ) return launch_valu_t<DD, QQ, GATED>(p, grid, s);
    WINATTN_VALU_CASE(64, 4) WINATTN_VALU_CASE(64, 8) WINATTN_VALU_CASE(64, 16)
    WINATTN_VALU_CASE(128, 4) WINATTN_VALU_CASE(128, 8) WINATTN_VALU_CASE(128, 16)
    WINATTN_VALU_CASE(256, 4) WINATTN_VALU_CASE(256, 8) WINATTN_VALU_CASE(256, 16)
#undef WINATTN_VALU_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_valu(const AttnParams& p, bool gated, int dpad, int nq, dim3 grid,
                       hipStream_t stream) {
    return gated ? launch_valu_g<true>(p, dpad, nq, grid, stream)
                 : launch_valu_g<false>(p, dpad, nq, grid, stream);
}

int valu_tile_keys(int dpad) { return dpad == 256 ? 32 : 64; }

}  // namespace winattn
