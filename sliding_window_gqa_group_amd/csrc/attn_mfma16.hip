// Split-K windowed attention on v_mfma_f32_16x16x4f32, for wide heads (d = 256) and for
// chunks whose query count per KV group is too small to fill 128-query tiles.
//
// Same method as the 32x32 matrix-core kernel (o1c page's GEMM path: score and value products
// over the group's sinks, ring and chunk keys with live-column masks; K/V blocks staged once
// and shared by several query tiles, as in the egemma2 page's staged kernels), re-tiled so
// that a wave owns 16 query vectors instead of 32. Per lane that halves the query operand
// (d/4 registers) and the output accumulators (d/4), which keeps d = 256 out of scratch, and a
// workgroup covers 64 queries, so short chunks give four times as many workgroups.
//
// Layout on v_mfma_f32_16x16x4f32 (A 16x4, B 4x16, 4 accumulators per lane; lane l supplies
// A[l%16][l/16] and B[l/16][l%16]; accumulator r of lane l is element (4*(l/16) + r, l%16)):
//   scores    S^T = K . Q^T   A = K (16 keys x d, LDS), B = Q^T (registers)
//             -> lane l holds query l%16 against keys 16*kb + 4*(l/16) + r of key block kb
//   values    O^T = V^T . P^T A = V^T (LDS), B = P^T = the score registers after the softmax
//             -> lane l holds query l%16, output columns 16*db + 4*(l/16) + r
// The k-steps of the score product take d = 16m + 4*(l/16) + e (e = 0..3) in lane row l/16,
// so each lane reads its K and Q operands as float4s. The row max and sum of a query run over
// the lane's 8 scores of a 32-key tile and then across its 4 lane rows (two lane swaps).
#include "winattn_dev.h"
#include "launch.h"

namespace winattn {

typedef float floatx4 __attribute__((ext_vector_type(4)));

// s_waitcnt immediate that waits for every outstanding vector memory load of the wave
// (vmcnt = 0, expcnt and lgkmcnt at their maxima, i.e. not waited on).
constexpr int kVmcntZero = 0x0F70;

constexpr int kM16QB = 64;   // queries per workgroup (16 per wave)
constexpr int kM16TK = 32;   // keys per tile

// Max / sum of a lane's value with that of lane l ^ 16 (v_permlane16_swap with the same value
// in both operands: the two results are the lane's own value and its partner's).
__device__ inline float quarter_swap_max(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float quarter_swap_sum(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Everything the direct tile loads need, by value: the group's row bases (ring, chunk, sinks)
// and the block's key range. Passing values rather than capturing references keeps the base
// choice a select of registers (a select of two loaded references becomes a load through a
// selected address, which pins the referenced variables in private memory).
struct DirectSrc {
    unsigned long long rk, rv, ck, cv, sk, sv;
    int ns, d, ring_ss, chunk_rs, xlo, xhi, nst, base, mod, xsplit, wave;
    unsigned col;
};

template <bool GATED>
__device__ inline DirectSrc direct_src(const AttnParams& p, const KVBases& b, const GroupWin& gw,
                                       int g, int xlo, int xhi, int nst, int lane, int d4,
                                       int wave) {
    DirectSrc s;
    s.rk = b.rk + 4ull * (unsigned long long)((long long)g * p.ring_gs);
    s.rv = b.rv + 4ull * (unsigned long long)((long long)g * p.ring_gs);
    s.ck = b.ck + 4ull * (unsigned long long)((long long)g * p.chunk_gs);
    s.cv = b.cv + 4ull * (unsigned long long)((long long)g * p.chunk_gs);
    s.sk = b.sk + 4ull * (unsigned long long)((long long)g * p.ns * p.d);
    s.sv = b.sv + 4ull * (unsigned long long)((long long)g * p.ns * p.d);
    s.ns = p.ns;
    s.d = p.d;
    s.ring_ss = (int)p.ring_ss;
    s.chunk_rs = (int)p.chunk_rs;
    s.xlo = xlo;
    s.xhi = xhi;
    s.nst = nst;
    s.base = gw.base;
    s.mod = gw.mod;
    s.xsplit = gw.xsplit;
    s.wave = __builtin_amdgcn_readfirstlane(wave);   // uniform: row arithmetic stays scalar
    s.col = 4u * (unsigned)(lane < d4 ? lane : 0);
    return s;
}

// Wave w of NW loads rows w, w + NW, ... of key tile t straight into the LDS tile (kb, vb), one
// 64-lane row per instruction. Every row read is a live one (a padding key reads sink 0 or the
// block's last stream entry; lanes past d read the row's first columns), so no LDS slot holds
// non-finite padding: a masked key gets weight 0 and 0 times finite data adds nothing.
template <int TK, int KST, int VST, int NW>
__device__ __attribute__((always_inline)) inline void issue_direct(const DirectSrc s, int t,
                                                                   float* kb, float* vb) {
    static_assert(TK % NW == 0, "every wave loads the same number of rows");
    const bool sink_t = t < s.nst;
#pragma unroll
    for (int i = 0; i < TK / NW; ++i) {
        const int key = s.wave + NW * i;
        const int si = t * TK + key;
        const int x = min(s.xlo + (t - s.nst) * TK + key, s.xhi - 1);
        const bool in_ring = x < s.xsplit;
        int slot = s.base + x;
        slot = slot >= s.mod ? slot - s.mod : slot;
        const int off = sink_t ? (si < s.ns ? si : 0) * s.d
                               : (in_ring ? slot * s.ring_ss : (x - s.xsplit) * s.chunk_rs);
        const unsigned long long bk = sink_t ? s.sk : (in_ring ? s.rk : s.ck);
        const unsigned long long bv = sink_t ? s.sv : (in_ring ? s.rv : s.cv);
        const unsigned long long e = 4ull * (unsigned)off + 4ull * s.col;
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const float*>(bk + e), kb + key * KST, 16, 0, 0);
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const float*>(bv + e), vb + key * VST, 16, 0, 0);
    }
}

// d = 256: a key row is one wave-wide 16-byte-per-lane load, which gfx950 writes straight into
// LDS (global_load_lds_dwordx4); two LDS tile buffers then replace the register staging of the
// next tile, and the workgroup runs 8 waves, two per SIMD: waves w and w + 4 own the same 16
// queries and take one 16-key block of every tile each, so that one wave's softmax overlaps
// the other's matrix products. Their two online-softmax states are combined at the end.
// Narrower rows stage through registers with 4 waves.
template <int D>
constexpr int m16_key_split() { return D == 256 ? 2 : 1; }

template <int D, bool GATED>
__global__ __launch_bounds__(kThreads * m16_key_split<D>(), 1) void attn_mfma16_kernel(const AttnParams p) {
    constexpr int TK = kM16TK, QB = kM16QB;
    constexpr int KS = m16_key_split<D>();    // waves per query set (key blocks split among them)
    constexpr int NT = kThreads * KS;         // threads per workgroup
    constexpr int NW = NT / 64;
    constexpr int D4 = D / 4, KST = D + 4, VST = D + 4;
    constexpr int LPT = TK * D4 / kThreads;   // float4 loads per thread per tensor per tile
    constexpr int NDB = D / 16;               // 16-wide d blocks of the output
    constexpr int NKB = TK / 16;              // 16-key blocks of a tile
    constexpr int NKBW = NKB / KS;            // key blocks per wave
    constexpr bool DIRECT = D == 256;
    static_assert(LPT >= 1 && TK * D4 == LPT * kThreads, "tile load must cover the tile");
    static_assert(TK * KST >= 6 * NT, "merge scratch reuses the K tile area");
    static_assert(!DIRECT || D4 == 64, "direct loads move one 64-lane row per instruction");
    static_assert(KS == 1 || DIRECT, "the key split runs on the direct-load path");
    static_assert(NKBW * KS == NKB, "key blocks divide among the waves of a query set");

    // Each LDS tile buffer is its own array, so that the compiler sees that reading one buffer
    // never conflicts with the direct loads still filling the other, and leaves them in flight.
    __shared__ __align__(16) float s_k[TK * KST];
    __shared__ __align__(16) float s_v[TK * VST];
    __shared__ __align__(16) float s_k1[DIRECT ? TK * KST : 4];
    __shared__ __align__(16) float s_v1[DIRECT ? TK * VST : 4];
    __shared__ int s_flag;

    // Work item = (group, split, query block), query block fastest; the same two XCD orders
    // as the 32x32 kernel (contiguous eighths per XCD, or round-robin).
    const int n_items = p.nsplit_grid * p.nqblocks * p.ng;
    const int per_xcd = (n_items + 7) / 8;
    const int item = p.xcd_map ? (int)(blockIdx.x % 8u) * per_xcd + (int)(blockIdx.x / 8u)
                               : (int)blockIdx.x;
    if (item >= n_items) return;
    const int qb = item % p.nqblocks;
    const int split = (item / p.nqblocks) % p.nsplit_grid;
    const int g = item / (p.nqblocks * p.nsplit_grid);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int qw = wave & 3, kh = wave >> 2;   // query set of the wave, its part of the keys
    const int qcol = lane & 15, kr4 = lane >> 4;
    const int nq_tot = p.rows * p.hpg;
    const int q0 = qb * QB;
    const int nq = min(QB, nq_tot - q0);
    const GroupWin gw = resolve_group<GATED>(p, g);

    const int r_first = q0 / p.hpg, r_last = (q0 + nq - 1) / p.hpg;
    const int xlo = window_lo(gw.hi0 + r_first, gw.wcap);
    const int xhi = gw.hi0 + r_last;
    const Tiles tr = tile_range<TK>(p.ns, xlo, xhi, p.nsplit_grid, split);
    const int nsplit = tr.nsplit, nst = tr.nst;
    if (split >= nsplit) {
        mark_split_empty<QB>(p, g * p.nqblocks + qb, split);
        return;
    }
    const int t_begin = tr.t_begin, t_end = tr.t_end;
    const int d4 = p.d / 4;

    // This lane's query (column qcol of its wave's 16) and its window in key-index space.
    const int jq = qw * 16 + qcol;
    const bool qvalid = jq < nq;
    const int qi = q0 + (qvalid ? jq : nq - 1);
    const int row = qi / p.hpg, gh = g * p.hpg + qi % p.hpg;
    const int hi = gw.hi0 + row;
    const int lo = window_lo(hi, gw.wcap);

    constexpr int LPTR = DIRECT ? 1 : LPT;
    float4 kreg[LPTR], vreg[LPTR];
    unsigned kmask = 0u;
    const KVBases kvb = kv_bases(p);
    const DirectSrc dsrc = direct_src<GATED>(p, kvb, gw, g, xlo, xhi, nst, lane, d4, wave);
    auto load_tile = [&](int t) {
        if constexpr (!DIRECT)
            kmask = load_tile_regs<TK, D, LPT>(p, kvb, gw, g, xlo, xhi, nst, t, d4, kreg, vreg);
    };
    if constexpr (DIRECT)
        issue_direct<TK, KST, VST, NW>(dsrc, t_begin, s_k, s_v);
    else
        load_tile(t_begin);   // first tile in flight while the queries load

    // Q^T operand: qreg[4m + e] = scale*log2e * q[16m + 4*kr4 + e].
    float qreg[D / 4];
    {
        const float* qp = p.q + ((size_t)row * p.nh + gh) * p.d;
#pragma unroll
        for (int m = 0; m < D / 16; ++m) {
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            const int e = 16 * m + 4 * kr4;
            if (e < p.d) v = *reinterpret_cast<const float4*>(qp + e);
            qreg[4 * m + 0] = v.x * p.scale_log2;
            qreg[4 * m + 1] = v.y * p.scale_log2;
            qreg[4 * m + 2] = v.z * p.scale_log2;
            qreg[4 * m + 3] = v.w * p.scale_log2;
        }
    }

    floatx4 oacc[NDB];
#pragma unroll
    for (int b = 0; b < NDB; ++b) oacc[b] = floatx4{0.f, 0.f, 0.f, 0.f};
    float mrun = -INFINITY, lrun = 0.0f;

    // One tile of keys against the block's queries, from the LDS tile (tk_, tv_).
    auto compute_tile = [&](int t, const float* tk_, const float* tv_) __attribute__((always_inline)) {
        // This lane's visible keys of the tile as a range [klo, khi) of key indices.
        const int tx = xlo + (t - nst) * TK;   // first stream entry of a stream tile
        const bool sink_tile = t < nst;
        const int klo = sink_tile ? 0 : lo - tx;
        const int khi = sink_tile ? p.ns - t * TK : hi - tx;
        if (!__any(klo < TK && khi > 0 && khi > klo)) return;   // the whole wave misses it

        // This wave's key blocks of the tile: kb = kh * NKBW + kw. Software-pipelined: the K
        // fragments of step m + 2 are read while step m's products run (scheduling barriers
        // keep the compiler from moving the reads back next to their uses).
        constexpr int NM = D / 16;
        constexpr int PF = 2;
        floatx4 sacc[NKBW];
        float4 kbuf[PF + 1][NKBW];
#pragma unroll
        for (int kw = 0; kw < NKBW; ++kw) sacc[kw] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < PF; ++m)
#pragma unroll
            for (int kw = 0; kw < NKBW; ++kw)
                kbuf[m][kw] = *reinterpret_cast<const float4*>(
                    tk_ + (16 * (kh * NKBW + kw) + qcol) * KST + 4 * kr4 + 16 * m);
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            if (m + PF < NM) {
#pragma unroll
                for (int kw = 0; kw < NKBW; ++kw)
                    kbuf[(m + PF) % (PF + 1)][kw] = *reinterpret_cast<const float4*>(
                        tk_ + (16 * (kh * NKBW + kw) + qcol) * KST + 4 * kr4 + 16 * (m + PF));
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int kw = 0; kw < NKBW; ++kw) {
                const float4 k4 = kbuf[m % (PF + 1)][kw];
                sacc[kw] = __builtin_amdgcn_mfma_f32_16x16x4f32(k4.x, qreg[4 * m + 0], sacc[kw], 0, 0, 0);
                sacc[kw] = __builtin_amdgcn_mfma_f32_16x16x4f32(k4.y, qreg[4 * m + 1], sacc[kw], 0, 0, 0);
                sacc[kw] = __builtin_amdgcn_mfma_f32_16x16x4f32(k4.z, qreg[4 * m + 2], sacc[kw], 0, 0, 0);
                sacc[kw] = __builtin_amdgcn_mfma_f32_16x16x4f32(k4.w, qreg[4 * m + 3], sacc[kw], 0, 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // The first V^T operands of the value product, read now so that their latency hides
        // under the softmax (step st = 4 kw + kk covers keys 16 kb + 4 kr4 + kk).
        constexpr int NST = NKBW * 4;
        float vbuf[2][NDB];
#pragma unroll
        for (int b = 0; b < NDB; ++b)
            vbuf[0][b] = tv_[(16 * (kh * NKBW) + 4 * kr4) * VST + qcol + 16 * b];

        // Mask by select (never multiply: masked slots may hold anything), online softmax.
        float tmax = -INFINITY;
#pragma unroll
        for (int kw = 0; kw < NKBW; ++kw)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int k = 16 * (kh * NKBW + kw) + 4 * kr4 + r;
                sacc[kw][r] = (k >= klo && k < khi) ? sacc[kw][r] : -INFINITY;
                tmax = fmaxf(tmax, sacc[kw][r]);
            }
        tmax = half_swap_max(quarter_swap_max(tmax));
        // lazy rescaling against a reference max (kLazyRescale)
        const bool grow = tmax > mrun + kLazyRescale;
        if (__any(grow)) {
            const float m_new = grow ? tmax : mrun;
            const float corr = __builtin_amdgcn_exp2f(mrun - safe_max(m_new));
            lrun *= corr;
#pragma unroll
            for (int b = 0; b < NDB; ++b) oacc[b] *= corr;
            mrun = m_new;
        }
        const float mu = safe_max(mrun);
        float psum = 0.0f;
#pragma unroll
        for (int kw = 0; kw < NKBW; ++kw)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                sacc[kw][r] = __builtin_amdgcn_exp2f(sacc[kw][r] - mu);
                psum += sacc[kw][r];
            }
        lrun += half_swap_sum(quarter_swap_sum(psum));

#pragma unroll
        for (int st = 0; st < NST; ++st) {
            if (st + 1 < NST) {
                const int kw1 = (st + 1) / 4, kk1 = (st + 1) % 4;
                const float* vp = tv_ + (16 * (kh * NKBW + kw1) + 4 * kr4 + kk1) * VST + qcol;
#pragma unroll
                for (int b = 0; b < NDB; ++b) vbuf[(st + 1) & 1][b] = vp[16 * b];
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int b = 0; b < NDB; ++b)
                oacc[b] = __builtin_amdgcn_mfma_f32_16x16x4f32(vbuf[st & 1][b], sacc[st / 4][st % 4],
                                                               oacc[b], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    if constexpr (DIRECT) {
        // Wait for this wave's rows of tile t; the barrier makes every wave's rows visible and
        // tells that nobody still reads the other buffer (tile t - 1), which then takes t + 1.
        for (int t = t_begin; t < t_end; t += 2) {
            __builtin_amdgcn_s_waitcnt(kVmcntZero);
            __syncthreads();
            if (t + 1 < t_end) issue_direct<TK, KST, VST, NW>(dsrc, t + 1, s_k1, s_v1);
            compute_tile(t, s_k, s_v);
            if (t + 1 < t_end) {
                __builtin_amdgcn_s_waitcnt(kVmcntZero);
                __syncthreads();
                if (t + 2 < t_end) issue_direct<TK, KST, VST, NW>(dsrc, t + 2, s_k, s_v);
                compute_tile(t + 1, s_k1, s_v1);
            }
        }
    } else {
        for (int t = t_begin; t < t_end; ++t) {
            __syncthreads();
#pragma unroll
            for (int j = 0; j < LPT; ++j) {
                const int f = tid + kThreads * j;
                const int key = f / D4, c = f % D4;
                const bool keep = (kmask >> j) & 1u;
                *reinterpret_cast<float4*>(s_k + key * KST + 4 * c) = zero_unless(keep, kreg[j]);
                *reinterpret_cast<float4*>(s_v + key * VST + 4 * c) = zero_unless(keep, vreg[j]);
            }
            __syncthreads();
            if (t + 1 < t_end) load_tile(t + 1);
            compute_tile(t, s_k, s_v);
        }
    }

    if constexpr (KS == 2) {
        // Fold the second key half's (m, l, O) into the first: waves 4..7 publish theirs in the
        // (now free) tile buffers, waves 0..3 combine. O goes as [b][lane of the query set]
        // float4s, columns 0..127 in s_k and 128..255 in s_v.
        static_assert(NDB == 16 && 2 * 128 * 4 * 8 <= TK * KST, "combine area");
        __syncthreads();
        const int li = qw * 64 + lane;
        if (kh == 1) {
#pragma unroll
            for (int b = 0; b < NDB; ++b) {
                float* dst = (b < 8 ? s_k : s_v) + ((b & 7) * 256 + li) * 4;
                *reinterpret_cast<floatx4*>(dst) = oacc[b];
            }
            s_k1[li] = mrun;
            s_k1[256 + li] = lrun;
        }
        __syncthreads();
        if (kh == 0) {
            const float m1 = s_k1[li], l1 = s_k1[256 + li];
            const float mt = fmaxf(mrun, m1), mu = safe_max(mt);
            const float f0 = __builtin_amdgcn_exp2f(mrun - mu), f1 = __builtin_amdgcn_exp2f(m1 - mu);
            lrun = lrun * f0 + l1 * f1;
            mrun = mt;
#pragma unroll
            for (int b = 0; b < NDB; ++b) {
                const float* src = (b < 8 ? s_k : s_v) + ((b & 7) * 256 + li) * 4;
                oacc[b] = oacc[b] * f0 + *reinterpret_cast<const floatx4*>(src) * f1;
            }
        }
    }

    // Lane holds, for its query, d = 16b + 4*kr4 + (0..3) in oacc[b] (waves of key half 0).
    const int blk = g * p.nqblocks + qb;
    if (nsplit == 1 && !p.merge_kernel) {
        if (qvalid && kh == 0) {
            const float inv = 1.0f / fmaxf(lrun, 1e-30f);
#pragma unroll
            for (int b = 0; b < NDB; ++b) {
                const int e = 16 * b + 4 * kr4;
                if (e < p.d)
                    store_out<GATED>(p, qi, g, e,
                                     make_float4(oacc[b][0] * inv, oacc[b][1] * inv,
                                                 oacc[b][2] * inv, oacc[b][3] * inv));
            }
        }
        return;
    }
    if (qvalid && kh == 0) {
        const size_t at = ((size_t)blk * p.slot_stride + split) * QB + jq;
#pragma unroll
        for (int b = 0; b < NDB; ++b)
            store_part4<QB, D>(p, blk, split, jq, 16 * b + 4 * kr4,
                               make_float4(oacc[b][0], oacc[b][1], oacc[b][2], oacc[b][3]));
        if (kr4 == 0) {
            store_part(p, p.pm + at, mrun);
            store_part(p, p.pl + at, lrun);
        }
    }
    if constexpr (DIRECT) __syncthreads();   // no wave still reads the last tile's buffer
    merge_if_last<QB, D, GATED, NT>(p, blk, nsplit, q0, nq, g, &s_flag, s_k);
}

template <int D, bool GATED>
static hipError_t launch_mfma16_t(const AttnParams& p, hipStream_t stream) {
    const int n_items = p.nsplit_grid * p.nqblocks * p.ng;
    const int blocks = p.xcd_map ? 8 * ((n_items + 7) / 8) : n_items;
    hipLaunchKernelGGL((attn_mfma16_kernel<D, GATED>), dim3(blocks), dim3(kThreads * m16_key_split<D>()),
                       0, stream, p);
    return hipGetLastError();
}

hipError_t launch_mfma16(const AttnParams& p, bool gated, int dpad, hipStream_t stream) {
    if (gated) {
        if (dpad == 64) return launch_mfma16_t<64, true>(p, stream);
        if (dpad == 128) return launch_mfma16_t<128, true>(p, stream);
        if (dpad == 256) return launch_mfma16_t<256, true>(p, stream);
    } else {
        if (dpad == 64) return launch_mfma16_t<64, false>(p, stream);
        if (dpad == 128) return launch_mfma16_t<128, false>(p, stream);
        if (dpad == 256) return launch_mfma16_t<256, false>(p, stream);
    }
    return hipErrorInvalidValue;
}

// Layout probe of v_mfma_f32_16x16x4f32: A[i][k] = i for k = 0 and 1 otherwise, B[k][j] = 1
// for k = 0 and 64 j for k = 1, 0 for k > 1, so D[i][j] = i + 64 j names its own position.
// out[lane * 4 + r] receives accumulator r of lane `lane`.
__global__ __launch_bounds__(64) void mfma16_layout_probe_kernel(float* out) {
    const int lane = threadIdx.x, i = lane & 15, k = lane >> 4;
    const float a = k == 0 ? (float)i : 1.0f;
    const float b = k == 0 ? 1.0f : (k == 1 ? 64.0f * (float)i : 0.0f);
    floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
#pragma unroll
    for (int r = 0; r < 4; ++r) out[lane * 4 + r] = acc[r];
}

hipError_t launch_mfma16_probe(float* out, hipStream_t stream) {
    hipLaunchKernelGGL(mfma16_layout_probe_kernel, dim3(1), dim3(64), 0, stream, out);
    return hipGetLastError();
}

int mfma16_query_block() { return kM16QB; }
int mfma16_tile_keys() { return kM16TK; }

}  // namespace winattn
