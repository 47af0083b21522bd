// Split-K attention for decode-sized chunks (at most 8 query vectors per KV group) in one
// launch, streaming each group's ring in storage order.
//
// Prior art on the o1c page ("A sealed layer's attention for a chunk of rows, on Metal"): the
// token path `o1c_tok_near` gives each simdgroup a stripe of the window, keeps the row's queries
// in registers and updates a running (max, sum, accumulator) per head; `o1c_tok_merge` combines
// the stripes' partials in the last threadgroup to finish. What changes on gfx950:
//
//  - Key order. Softmax attention does not depend on the order of its keys, so a split takes a
//    fixed range of ring SLOTS (storage order) rather than a range of the window's entries.
//    Every K/V address of the call (ring slots, sinks, the chunk's rows) is then known before
//    the group's metadata arrives: all of a workgroup's loads are requested at once, at the
//    start, and the metadata (one more memory round trip) is read while they are in flight. It
//    only decides, per key and query, whether the key is visible: slot s holds entry
//    x = (s - head) mod wg, which row i sees when it is held (s < wg, x < len) and inside the
//    row's window (x >= lo_i). A slot outside every window may hold anything (never written,
//    NaN): its score is masked to -inf and its value zeroed by select, so it adds exactly 0.
//    The price: the whole w-slot ring of every group is read, however few of its slots are
//    live, so a call costs what a full ring costs.
//  - Split 0 also takes the group's extra keys: the sinks, then the chunk's rows (at most 8).
//  - Registers, no LDS in the key loop: a lane group of TPK = D*NQ/32 lanes owns one key per
//    pass (its lanes hold float4 columns of the key's K and V rows and of every query); scores
//    are partial dot products summed over the lane group with DPP; each lane group keeps a
//    running max, sum and accumulator per query, merged once through LDS at the end.
//  - One launch. Each split writes its partial (max, sum, accumulator per query) with
//    device-scope stores, waits for them to complete and raises ready flags; the group's last
//    few splits each wait for every flag, then read one column chunk of every partial in one
//    batch and fold it (the token path's merge rule), so no CU reads more than its share. No
//    second kernel, no kernel boundary, no read-modify-write.
//  - Work order: workgroup b takes group b mod ng, split b / ng. Workgroups are dealt to the 8
//    XCDs round-robin, so with 8 groups every split of a group runs on one XCD, next to the
//    partials its merge reads.
#include <type_traits>

#include "attn_dec_block.h"
#include "far_part.h"
#include "launch.h"

namespace winattn {

// Phase stamps, in timing builds only (compiled with WINATTN_PHASE_STAMPS; the library's normal
// build contains none of this code). Every wave reads the 100 MHz real-time counter at the
// kernel's phase boundaries, keeps the readings in registers and writes them once, at its end,
// with the number of the XCD it ran on, to g_phase_stamps[block * waves + wave][kStampWords]
// when the host has set that pointer (attn_phase_stamps_set); launches with a far part write
// none. The kernel's work is unchanged.
#ifdef WINATTN_PHASE_STAMPS
constexpr int kStampWords = 10;
__device__ unsigned long long* g_phase_stamps;
struct PhaseStamps {
    unsigned long long t[kStampWords - 1] = {};
    __device__ void mark(int k) { t[k] = __builtin_amdgcn_s_memrealtime(); }
    // the reading waits until `v` is available (the empty asm uses it)
    template <class V>
    __device__ void mark_after(int k, const V& v) {
        asm volatile("" : : "v"(v));
        mark(k);
    }
    // the reading waits until every memory access of the wave has completed
    __device__ void mark_drained(int k) {
        __builtin_amdgcn_s_waitcnt(0);
        mark(k);
    }
    __device__ void flush(int blk, int tid, int waves) {
        unsigned long long* o = g_phase_stamps;
        if (!o || blk < 0 || (tid & 63) != 0) return;
        o += ((size_t)blk * waves + tid / 64) * kStampWords;
        for (int k = 0; k < kStampWords - 1; ++k) o[k] = t[k];
        // hardware register 20 (XCC_ID), bits 0-3: the XCD of this wave
        o[kStampWords - 1] = __builtin_amdgcn_s_getreg(20 | (0 << 6) | (3 << 11));
    }
};
#else
struct PhaseStamps {
    __device__ void mark(int) {}
    template <class V>
    __device__ void mark_after(int, const V&) {}
    __device__ void mark_drained(int) {}
    __device__ void flush(int, int, int) {}
};
#endif

// A group's ring geometry from its metadata (len, head, far count, window override), clamped
// so that no access leaves the ring (as resolve_group clamps it): window wg, entries held len0,
// slot of the oldest entry head0.
struct RingGeom {
    int wg, len0, head0;
};

__device__ inline RingGeom ring_geom(vu4 m, int w) {
    const uint32_t wg = (m.w != 0u && m.w < (uint32_t)w) ? m.w : (uint32_t)w;
    const uint32_t len0 = m.x < wg ? m.x : wg;
    const uint32_t head0 = m.y >= wg ? m.y % wg : m.y;
    return RingGeom{(int)wg, (int)len0, (int)head0};
}


// Max / sum over the lane groups of a wave: lanes l, l ^ TPK, l ^ 2 TPK, ... (TPK = 8, 16, 32 or
// 64 lanes per group), result in every lane. Lanes l ^ 8 meet by a DPP rotation within a row of
// 16, lanes l ^ 16 and l ^ 32 by gfx950's row and half-wave swaps.
constexpr int kDppRowRor8 = 0x128;

template <int TPK>
__device__ inline float lane_groups_max(float v) {
    if constexpr (TPK <= 8) v = fmaxf(v, dpp<kDppRowRor8>(v, -INFINITY));
    if constexpr (TPK <= 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    }
    if constexpr (TPK <= 32) v = half_swap_max(v);
    return v;
}

template <int TPK>
__device__ inline float lane_groups_sum(float v) {
    if constexpr (TPK <= 8) v += dpp<kDppRowRor8>(v, 0.0f);
    if constexpr (TPK <= 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    if constexpr (TPK <= 32) v = half_swap_sum(v);
    return v;
}

// Max / sum over lanes l, l + span, l + 2 span, ... of the wave (span a power of two, 1 to 64,
// uniform over the wave), result in every lane: rotations within each row of 16 lanes by span,
// 2 span, ... 8, then the row and half-wave swaps.
__device__ inline float lanes_max_spaced(float v, int span) {
    if (span <= 1) v = fmaxf(v, dpp<0x121>(v, -INFINITY));
    if (span <= 2) v = fmaxf(v, dpp<0x122>(v, -INFINITY));
    if (span <= 4) v = fmaxf(v, dpp<0x124>(v, -INFINITY));
    if (span <= 8) v = fmaxf(v, dpp<kDppRowRor8>(v, -INFINITY));
    if (span <= 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    }
    if (span <= 32) v = half_swap_max(v);
    return v;
}

__device__ inline float lanes_sum_spaced(float v, int span) {
    if (span <= 1) v += dpp<0x121>(v, 0.0f);
    if (span <= 2) v += dpp<0x122>(v, 0.0f);
    if (span <= 4) v += dpp<0x124>(v, 0.0f);
    if (span <= 8) v += dpp<kDppRowRor8>(v, 0.0f);
    if (span <= 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    if (span <= 32) v = half_swap_sum(v);
    return v;
}

// The group's last `nk` splits are its gatherers (the last of the group's workgroups in dispatch
// order, so every split a gatherer waits for was dispatched before it, and the non-gatherers
// never wait). Gatherer k owns output columns [k, k + 1) * D / (4 nk) float4 of every query of
// the group: it reads only those columns of the group's nsplit partials and folds them:
// c = max_s m_s, out = sum_s acc_s 2^(m_s - c) / sum_s l_s 2^(m_s - c) (the token path's merge,
// `o1c_tok_merge`). One CU reads freshly written partials at only tens of GB/s, so the merge is
// spread over nk CUs, each reading a few KB.
//  - Every split raises one flag per gatherer (flags[k][s]), so each gatherer polls and clears
//    flags nobody else reads.
//  - Each wave owns ipw = NQ * D / (4 nk) / waves (query j, float4 column c) items. Lane
//    l = sub * ipw + item (ipw < 64) takes the splits s = sub (mod 64 / ipw) of its item, so the
//    lanes of one item differ only in the bits above ipw and meet by cross-lane reductions, with
//    no LDS and no barrier (ipw >= 64: a lane owns ipw / 64 items and every split of them).
//  - A wave first polls every flag of its gatherer (one flag read per lane and 64 splits) until
//    all are raised, then reads its splits' columns MB splits at a time, every load of a batch
//    issued before any is used. Reading each partial as its flag rises instead measured 1 us
//    slower per call: the bookkeeping of which splits are ready sits between seeing the last
//    flag and requesting its columns, and the columns are too few for the overlap to pay.
//  - The poll is bounded: after kGatherPolls rounds without every flag, a wave writes its items
//    as NaN rather than waiting longer (it cannot happen while every split runs).
//  - Each wave stores its items as soon as they are folded. After one barrier (every wave has
//    left its poll loop and said whether it saw every flag in `scratch`, NT / 64 words), the
//    gatherer's flags are cleared for the next call if every wave saw them all.
constexpr int kGatherPolls = 1 << 18;

template <int NQ, int D, int NT, bool GATED>
__device__ inline void gather_chunk(const AttnParams& p, int g, int nslot, int nflag, int nq, int nk,
                                    int k, unsigned int* flags, int* scratch) {
    constexpr int D4 = D / 4, NW = NT / 64;
    constexpr int MB = 8;                     // splits per lane per load round
    // items per lane at most: more than 64 per wave only for a single gatherer of 8 queries of
    // width 256
    constexpr int IPTM = NQ * D4 > NW * 64 ? NQ * D4 / (NW * 64) : 1;
    const int cpk = D4 / nk;                  // float4 columns per gatherer
    const int ipw = NQ * cpk / NW;            // items per wave (>= 2)
    const int span = ipw < 64 ? ipw : 64;     // lanes of one item are `span` apart
    const int nsub = 64 / span;               // lanes per item
    const int ipt = ipw / span;               // items per lane
    const int tid = threadIdx.x, lane = tid & 63, wave = tid / 64;
    const int sub = lane / span;
    const size_t grp = (size_t)g * nslot * NQ;   // first partial slot of the group
    const __amdgpu_buffer_rsrc_t racc =
        __builtin_amdgcn_make_buffer_rsrc(p.pacc + grp * D, 0, nslot * NQ * D * 4, kBufferWord3);
    const __amdgpu_buffer_rsrc_t rm =
        __builtin_amdgcn_make_buffer_rsrc(p.pm + grp, 0, nslot * NQ * 4, kBufferWord3);
    const __amdgpu_buffer_rsrc_t rl =
        __builtin_amdgcn_make_buffer_rsrc(p.pl + grp, 0, nslot * NQ * 4, kBufferWord3);

    float cm[IPTM], cl[IPTM];
    vf4 ca[IPTM];
    int jj[IPTM], cc[IPTM];
#pragma unroll
    for (int it = 0; it < IPTM; ++it) {
        const int item = wave * ipw + lane % span + span * (it < ipt ? it : 0);
        jj[it] = item / cpk;
        cc[it] = k * cpk + item % cpk;
        cm[it] = -INFINITY;
        cl[it] = 0.0f;
        ca[it] = vf4{0.f, 0.f, 0.f, 0.f};
    }
    // phase 1: every flag of this gatherer, polled until all are raised (pend: the flags not
    // yet seen, bit s of word s / 64 in lane s % 64 of every lane)
    unsigned long long pend[2] = {nflag >= 64 ? ~0ull : (1ull << nflag) - 1ull,
                                  nflag >= 128 ? ~0ull : (nflag > 64 ? (1ull << (nflag - 64)) - 1ull : 0ull)};
    const int nw = nflag > 64 ? 2 : 1;
    int polls = 0;
    bool complete = false;
    while (polls < kGatherPolls) {
        ++polls;
#pragma unroll
        for (int h = 0; h < 2; ++h)
            if (h < nw) pend[h] &= ~__builtin_amdgcn_ballot_w64(poll_flag(flags + min(h * 64 + lane, nflag - 1)) != 0u);
        if ((pend[0] | pend[1]) == 0ull) {   // wave-uniform (ballot results)
            complete = true;
            break;
        }
        __builtin_amdgcn_s_sleep(1);
    }
    // phase 2: this lane's slots s = sub + nsub i, MB at a time
    for (int s0 = sub; complete && s0 < nslot; s0 += MB * nsub) {
        float m[IPTM][MB], l[IPTM][MB];
        vf4 a[IPTM][MB];
#pragma unroll
        for (int it = 0; it < IPTM; ++it) {
#pragma unroll
            for (int u = 0; u < MB; ++u) {
                const int su = s0 + u * nsub;
                const int at = su * NQ + jj[it];
                m[it][u] = -INFINITY;   // past the lane's slots: no keys
                l[it][u] = 0.0f;
                a[it][u] = vf4{0.f, 0.f, 0.f, 0.f};
                if (su < nslot) {
                    m[it][u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rm, at * 4, 0, kCachePolicyDevice));
                    l[it][u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rl, at * 4, 0, kCachePolicyDevice));
                    a[it][u] = __builtin_bit_cast(
                        vf4, __builtin_amdgcn_raw_buffer_load_b128(racc, (at * D + 4 * cc[it]) * 4, 0, kCachePolicyDevice));
                }
            }
        }
#pragma unroll
        for (int it = 0; it < IPTM; ++it) {
            if (it >= ipt) break;
            float bm = -INFINITY;
#pragma unroll
            for (int u = 0; u < MB; ++u) bm = fmaxf(bm, m[it][u]);
            const float nm = fmaxf(cm[it], bm), mu = safe_max(nm);
            const float f0 = __builtin_amdgcn_exp2f(cm[it] - mu);
            cl[it] *= f0;
            ca[it] *= f0;
#pragma unroll
            for (int u = 0; u < MB; ++u) {
                const bool real = m[it][u] > -INFINITY;   // a split with no keys is -inf too
                const float f = __builtin_amdgcn_exp2f(m[it][u] - mu);
                cl[it] += (real ? l[it][u] : 0.0f) * f;
                ca[it] += (real ? a[it][u] : vf4{0.f, 0.f, 0.f, 0.f}) * f;
            }
            cm[it] = nm;
        }
    }

    // the lanes of each item meet: c = max over them, then the rescaled sums
#pragma unroll
    for (int it = 0; it < IPTM; ++it) {
        if (it >= ipt) break;
        const float c = lanes_max_spaced(cm[it], span);
        const float f = __builtin_amdgcn_exp2f(cm[it] - safe_max(c));
        cl[it] = lanes_sum_spaced(cl[it] * f, span);
        ca[it].x = lanes_sum_spaced(ca[it].x * f, span);
        ca[it].y = lanes_sum_spaced(ca[it].y * f, span);
        ca[it].z = lanes_sum_spaced(ca[it].z * f, span);
        ca[it].w = lanes_sum_spaced(ca[it].w * f, span);
    }
    // each wave stores its items at once (NaN if it gave up on a flag); the barrier only
    // guards the flag clearing below
    if (sub == 0) {
#pragma unroll
        for (int it = 0; it < IPTM; ++it) {
            if (it >= ipt || jj[it] >= nq || cc[it] >= p.d / 4) continue;
            vf4 o = ca[it] * (1.0f / fmaxf(cl[it], 1e-30f));
            if (!complete) o = vf4{NAN, NAN, NAN, NAN};
            store_out<GATED>(p, jj[it], g, 4 * cc[it], make_float4(o.x, o.y, o.z, o.w));
        }
    }
    if (lane == 0) scratch[wave] = complete ? 1 : 0;
    __syncthreads();   // every wave has left its poll loop
    bool bad = false;
#pragma unroll
    for (int w = 0; w < NW; ++w) bad |= scratch[w] == 0;
    // this gatherer's flags back to zero for the next call
    if (!bad && tid < 64) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int s = h * 64 + lane;
            if (s < nflag) __hip_atomic_store(flags + s, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// Lanes per key, float4 columns per lane, keys per pass and passes per tile of a workgroup of
// NT threads: TPK = D*NQ/32 lanes own a key (4 float4 of K and of V per lane per tile of
// TK = 4096 / D keys with 256 threads).
template <int D, int NQ, int NT>
struct DecodeShape {
    static constexpr int TPK = D * NQ / 32;
    static constexpr int F4 = D / (4 * TPK);
    static constexpr int KPP = NT / TPK;
    static constexpr int TK = 4096 / D;
    static constexpr int PASSES = TK / KPP;
    static_assert(TPK >= 4 && TPK <= 64 && F4 >= 1 && PASSES >= 1, "unsupported shape");
    // passes a split holds in registers without spilling (all requested up front)
    static constexpr int MAX_PASSES = 8;
    static constexpr int MAX_TILES = MAX_PASSES / PASSES;
};

// One split of the call: workgroup wg_index (counted from the first split's) takes group
// wg_index mod ng, split wg_index / ng. T: ring tiles per split (TK = 4096 / D slots each), all
// requested up front; NT threads. FAR: a one-row call with a far field; the group has one
// partial slot more, nsplit, which other workgroups of the launch fill (query j: head j's far
// partial), and each gatherer hpg flags more (nsplit + j for head j); the gatherers fold that
// slot with the splits' ones. GATED (with FAR): the gated one-row call (dory page, "Dory's token
// path": `dory_os` ... `dory_ogate`), whose ring already holds the row's own key: slots
// 0 .. len - 1 are its keys, all visible to the row, the extra keys are the sinks alone, and
// the outputs pass through the sigmoid gate.
template <int D, int NQ, int T, int NT, bool FAR, bool GATED>
__device__ __forceinline__ void decode_split(const AttnParams& p, const int wg_index) {
    static_assert(FAR || !GATED, "the gated call takes this kernel with its far part only");
    using S = DecodeShape<D, NQ, NT>;
    constexpr int TPK = S::TPK, F4 = S::F4, KPP = S::KPP, TK = S::TK, PASSES = S::PASSES;
    constexpr int NP = T * PASSES;   // ring passes of a split (one key per lane group each)
    static_assert(T <= S::MAX_TILES, "too many tiles for the registers");

    constexpr int NW = NT / 64;                           // waves
    // each wave's state at the end (then the gather's NW words)
    constexpr int kAccFloats = NW * NQ * D;
    __shared__ __align__(16) float s_acc[kAccFloats];
    __shared__ float s_wm[NW * NQ], s_wl[NW * NQ];

    const int tid = threadIdx.x;
    const int gi = tid / TPK, sl = tid % TPK;   // lane group (key slot), lane within the group
    const int g = wg_index % p.ng;
    const int split = wg_index / p.ng;
    const int nsplit = p.nsplit_grid;
    const int nslot = FAR ? nsplit + 1 : nsplit;          // partial slots of the group
    const int nflag = FAR ? nsplit + p.hpg : nsplit;      // ready flags of each gatherer
    const int nq = p.rows * p.hpg;              // every query of the group: one block
    const int d4 = p.d / 4;
    PhaseStamps ps_;
    ps_.mark(0);   // phase 0: start

    // ---- the group's metadata is requested first, ahead of the call's K/V traffic, as a
    // vector load: vector loads return in order, so waiting for it waits for nothing issued
    // after it, and it never holds up the scalar loads of the kernel's arguments (scalar loads
    // return out of order and are waited for all together). Nothing reads it until every load
    // of the split has been requested.
    vu4 meta_v = __builtin_amdgcn_raw_buffer_load_b128(
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(p.meta + 4 * g), 0, 16, kBufferWord3),
        0, 0, 0);

    // ---- queries: this lane's columns of every query, times scale*log2(e); addresses clamped
    // to a live element, padding scaled by 0 (a factor keeps the load unconditional)
    vf4 qr[NQ][F4];
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
        const int qi = min(j, nq - 1);
        const int row = qi / p.hpg, gh = g * p.hpg + qi % p.hpg;
        const float* qp = p.q + ((size_t)row * p.nh + gh) * p.d;
#pragma unroll
        for (int f = 0; f < F4; ++f) {
            const int c = sl + TPK * f;
            const bool live = (j < nq) & (c < d4);
            const vf4 v = *reinterpret_cast<const vf4*>(qp + 4 * (c < d4 ? c : 0));
            qr[j][f] = v * (live ? p.scale_log2 : 0.0f);
        }
    }

    const KVBases b = kv_bases(p);
    const unsigned long long rk = b.rk + 4ull * (unsigned long long)((long long)g * p.ring_gs);
    const unsigned long long rv = b.rv + 4ull * (unsigned long long)((long long)g * p.ring_gs);
    const unsigned long long ck = b.ck + 4ull * (unsigned long long)((long long)g * p.chunk_gs);
    const unsigned long long cv = b.cv + 4ull * (unsigned long long)((long long)g * p.chunk_gs);
    const unsigned long long sk = b.sk + 4ull * (unsigned long long)((long long)g * p.ns * p.d);
    const unsigned long long sv = b.sv + 4ull * (unsigned long long)((long long)g * p.ns * p.d);
    const int ss = (int)p.ring_ss, crs = (int)p.chunk_rs;
    const int nextra = p.ns + (GATED ? 0 : p.rows);

    // Extra key e of the group: sink e (e < ns), else chunk row e - ns; padding (e >= nextra)
    // loads the chunk's last row, a live address (the gated call, which has no chunk rows
    // here: the ring's slot 0).
    auto load_extra = [&](vf4 (&k)[F4], vf4 (&v)[F4], int e) {
        const bool sink = e < p.ns;
        const int crow = min(e - p.ns, p.rows - 1);
        const int row = sink ? e * p.d : (GATED ? 0 : crow * crs);
        const unsigned long long bk = sink ? sk : (GATED ? rk : ck), bv = sink ? sv : (GATED ? rv : cv);
#pragma unroll
        for (int f = 0; f < F4; ++f) {
            const int c = sl + TPK * f;
            const int off = c < d4 ? row + 4 * c : row;
            k[f] = *reinterpret_cast<gvf4p>(bk + 4ull * (unsigned)off);
            v[f] = *reinterpret_cast<gvf4p>(bv + 4ull * (unsigned)off);
        }
    };

    // ---- every load of the split, before the metadata: split 0's first pass of extra keys,
    // then the ring slots split*T*TK + i*KPP + gi of pass i (slots past w load slot w-1). The
    // ring is read once per call: its loads are non-temporal, so the stream does not push the
    // kernel's code, metadata and queries out of the caches (measured 3 % faster).
    vf4 kx[F4], vx[F4];
    if (split == 0) load_extra(kx, vx, gi);
    const int slot0 = split * (T * TK) + gi;
    vf4 kr[NP][F4], vr[NP][F4];
#pragma unroll
    for (int i = 0; i < NP; ++i) {
        const int slot = min(slot0 + i * KPP, p.w - 1);
#pragma unroll
        for (int f = 0; f < F4; ++f) {
            const int c = sl + TPK * f;
            const int off = slot * ss + (c < d4 ? 4 * c : 0);
            kr[i][f] = __builtin_nontemporal_load(reinterpret_cast<gvf4p>(rk + 4ull * (unsigned)off));
            vr[i][f] = __builtin_nontemporal_load(reinterpret_cast<gvf4p>(rv + 4ull * (unsigned)off));
        }
    }

    // ---- each query's window, from the metadata. The empty asm pins the first use of the
    // metadata here, after every load above (its memory clobber keeps them above it), so the
    // wait for the metadata cannot be scheduled ahead of them (all four words stay live until
    // then, so no register of the load in flight is reused before it lands).
    asm volatile("" : "+v"(meta_v.x), "+v"(meta_v.y), "+v"(meta_v.z), "+v"(meta_v.w) : : "memory");
    // (the gated call: slots 0 .. len - 1 hold the row's window, len clamped to w)
    const RingGeom rg = GATED ? RingGeom{p.w, (int)(meta_v.x < (uint32_t)p.w ? meta_v.x : (uint32_t)p.w), 0}
                              : ring_geom(meta_v, p.w);
    int qlo[NQ], qrow[NQ];
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
        const int row = min(j, nq - 1) / p.hpg;
        const int hi = rg.len0 + row + 1;
        qlo[j] = j < nq ? (GATED ? 0 : window_lo(hi, rg.wg)) : 0x7fffffff;   // padding sees nothing
        qrow[j] = j < nq ? row : -1;
    }
    ps_.mark_after(1, qlo[0]);   // phase 1: metadata arrived

    float mrun[NQ], lrun[NQ];
    vf4 acc[NQ][F4];
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
        mrun[j] = -INFINITY;
        lrun[j] = 0.0f;
#pragma unroll
        for (int f = 0; f < F4; ++f) acc[j][f] = vf4{0.f, 0.f, 0.f, 0.f};
    }

    // ---- NPS passes: scores, visibility (bit j of vis[ps]: query j sees the pass's key of this
    // lane group), online softmax of this lane group, value update
    auto step = [&](auto& kk, auto& vv, const auto& vis) {
        constexpr int NPS = std::extent<std::remove_reference_t<decltype(kk)>>::value;
        float sc[NPS * NQ];
#pragma unroll
        for (int ps = 0; ps < NPS; ++ps)
#pragma unroll
            for (int j = 0; j < NQ; ++j) {
                float s = 0.0f;
#pragma unroll
                for (int f = 0; f < F4; ++f) {
                    float h = kk[ps][f].x * qr[j][f].x;
                    h = __builtin_fmaf(kk[ps][f].y, qr[j][f].y, h);
                    h = __builtin_fmaf(kk[ps][f].z, qr[j][f].z, h);
                    h = __builtin_fmaf(kk[ps][f].w, qr[j][f].w, h);
                    s = f == 0 ? h : s + h;
                }
                sc[ps * NQ + j] = s;
            }
        constexpr int kSumMax = 8;   // sums of 8 values interleaved level by level
        constexpr int kSumBlock = NPS * NQ < kSumMax ? NPS * NQ : kSumMax;
#pragma unroll
        for (int bb = 0; bb < NPS * NQ; bb += kSumBlock) lane_group_sum_n<TPK, kSumBlock>(sc + bb);
#pragma unroll
        for (int ps = 0; ps < NPS; ++ps) {
#pragma unroll
            for (int j = 0; j < NQ; ++j)
                sc[ps * NQ + j] = (vis[ps] >> j) & 1u ? sc[ps * NQ + j] : -INFINITY;
            // a key no query sees may hold anything (a slot never written): 0 * NaN must not
            // reach the accumulators
            const bool any = vis[ps] != 0u;
#pragma unroll
            for (int f = 0; f < F4; ++f) {
                vv[ps][f].x = any ? vv[ps][f].x : 0.0f;
                vv[ps][f].y = any ? vv[ps][f].y : 0.0f;
                vv[ps][f].z = any ? vv[ps][f].z : 0.0f;
                vv[ps][f].w = any ? vv[ps][f].w : 0.0f;
            }
        }
#pragma unroll
        for (int j = 0; j < NQ; ++j) {
            float tmax = sc[j];
#pragma unroll
            for (int ps = 1; ps < NPS; ++ps) tmax = fmaxf(tmax, sc[ps * NQ + j]);
            const float m_new = fmaxf(mrun[j], tmax);
            const float mu = safe_max(m_new);
            const float corr = __builtin_amdgcn_exp2f(mrun[j] - mu);
            mrun[j] = m_new;
            float lsum = 0.0f;
#pragma unroll
            for (int f = 0; f < F4; ++f) acc[j][f] *= corr;
#pragma unroll
            for (int ps = 0; ps < NPS; ++ps) {
                const float pv = __builtin_amdgcn_exp2f(sc[ps * NQ + j] - mu);
                lsum += pv;
#pragma unroll
                for (int f = 0; f < F4; ++f) {
                    acc[j][f].x = __builtin_fmaf(pv, vv[ps][f].x, acc[j][f].x);
                    acc[j][f].y = __builtin_fmaf(pv, vv[ps][f].y, acc[j][f].y);
                    acc[j][f].z = __builtin_fmaf(pv, vv[ps][f].z, acc[j][f].z);
                    acc[j][f].w = __builtin_fmaf(pv, vv[ps][f].w, acc[j][f].w);
                }
            }
            lrun[j] = lrun[j] * corr + lsum;
        }
    };

    // Visibility of extra key e: a sink to every real query; chunk row c to the queries of
    // rows >= c whose window reaches back to it.
    auto extra_vis = [&](int e) {
        unsigned m = 0u;
        const int c = e - p.ns;
#pragma unroll
        for (int j = 0; j < NQ; ++j) {
            const bool v = e < p.ns ? j < nq
                                    : (e < nextra) & (c <= qrow[j]) & (rg.len0 + c >= qlo[j]);
            m |= v ? 1u << j : 0u;
        }
        return m;
    };

    // ---- split 0: its extra keys first (they arrived first), more passes of them if needed
    if (split == 0) {
        vf4 k1[1][F4], v1[1][F4];
#pragma unroll
        for (int f = 0; f < F4; ++f) {
            k1[0][f] = kx[f];
            v1[0][f] = vx[f];
        }
        unsigned vis1[1] = {extra_vis(gi)};
        step(k1, v1, vis1);
        for (int e0 = KPP; e0 < nextra; e0 += KPP) {   // more than one pass of sinks and rows
            load_extra(k1[0], v1[0], e0 + gi);
            vis1[0] = extra_vis(e0 + gi);
            step(k1, v1, vis1);
        }
    }

    // ---- the ring passes, one tile (PASSES passes) per online-softmax step
#pragma unroll
    for (int t = 0; t < T; ++t) {
        vf4 kt[PASSES][F4], vt[PASSES][F4];
        unsigned vis[PASSES];
#pragma unroll
        for (int ps = 0; ps < PASSES; ++ps) {
            const int i = t * PASSES + ps;
#pragma unroll
            for (int f = 0; f < F4; ++f) {
                kt[ps][f] = kr[i][f];
                vt[ps][f] = vr[i][f];
            }
            const int slot = slot0 + i * KPP;
            int x = slot - rg.head0;
            x = x < 0 ? x + rg.wg : x;
            const bool held = (slot < rg.wg) & (x < rg.len0);
            unsigned m = 0u;
#pragma unroll
            for (int j = 0; j < NQ; ++j) m |= (held & (x >= qlo[j])) ? 1u << j : 0u;
            vis[ps] = m;
        }
        step(kt, vt, vis);
        if (t == 0) ps_.mark_after(2, mrun[0]);   // phase 2: first ring tile done
    }
    ps_.mark_after(3, lrun[0]);   // phase 3: last ring tile done

    // ---- merge the lane groups of each wave with cross-lane swaps (every lane of a group
    // holds the group's state; groups of a wave differ in the lane bits above TPK), then the
    // waves through LDS
    const int wave = tid / 64;
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
        const float wm = lane_groups_max<TPK>(mrun[j]);
        const float f = __builtin_amdgcn_exp2f(mrun[j] - safe_max(wm));
        mrun[j] = wm;
        lrun[j] = lane_groups_sum<TPK>(lrun[j] * f);
#pragma unroll
        for (int fc = 0; fc < F4; ++fc) {
            acc[j][fc].x = lane_groups_sum<TPK>(acc[j][fc].x * f);
            acc[j][fc].y = lane_groups_sum<TPK>(acc[j][fc].y * f);
            acc[j][fc].z = lane_groups_sum<TPK>(acc[j][fc].z * f);
            acc[j][fc].w = lane_groups_sum<TPK>(acc[j][fc].w * f);
        }
    }
    if ((tid & 63) < TPK) {   // the wave's first lane group writes the wave's state
#pragma unroll
        for (int j = 0; j < NQ; ++j) {
#pragma unroll
            for (int fc = 0; fc < F4; ++fc)
                *reinterpret_cast<vf4*>(s_acc + (wave * NQ + j) * D + 4 * (sl + TPK * fc)) = acc[j][fc];
            if (sl == 0) {
                s_wm[wave * NQ + j] = mrun[j];
                s_wl[wave * NQ + j] = lrun[j];
            }
        }
    }
    __syncthreads();
    ps_.mark(4);   // phase 4: lane groups and waves merged into LDS

    // ---- this split's partial (or the output when the group has a single split), folded over
    // the waves per (query, float4 column) item. Partials are read within this launch by
    // workgroups that may run on other XCDs, whose L2 caches are not coherent with this one:
    // they are stored with the device-scope (sc1) cache policy, which writes them through to the
    // device-coherent level (16-byte buffer stores).
    constexpr int D4 = D / 4;
    const size_t at0 = ((size_t)g * nslot + split) * NQ;
    const __amdgpu_buffer_rsrc_t part =
        __builtin_amdgcn_make_buffer_rsrc(p.pacc + at0 * D, 0, NQ * D * 4, kBufferWord3);
    for (int item = tid; item < NQ * D4; item += NT) {
        const int j = item / D4, c = item % D4;
        float m = -INFINITY;
#pragma unroll
        for (int w = 0; w < NW; ++w) m = fmaxf(m, s_wm[w * NQ + j]);
        const float mu = safe_max(m);
        float l = 0.0f;
        vf4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const float f = __builtin_amdgcn_exp2f(s_wm[w * NQ + j] - mu);
            l += s_wl[w * NQ + j] * f;
            o += *reinterpret_cast<const vf4*>(s_acc + (w * NQ + j) * D + 4 * c) * f;
        }
        if (j >= nq || c >= d4) continue;
        if (!FAR && nsplit == 1) {
            o *= 1.0f / fmaxf(l, 1e-30f);
            store_out<GATED>(p, j, g, 4 * c, make_float4(o.x, o.y, o.z, o.w));
        } else {
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(vu4, o), part, (j * D + 4 * c) * 4,
                                                   0, kCachePolicyDevice);
            if (c == 0) {
                store_dev(p.pm + at0 + j, m);
                store_dev(p.pl + at0 + j, l);
            }
        }
    }
    ps_.mark(5);   // phase 5: partial (or output) stores issued
    if (!FAR && nsplit == 1) {
        ps_.flush(FAR ? -1 : wg_index, tid, NW);
        return;
    }

    // ---- every thread waits until its partial stores are acknowledged (complete at the
    // device-coherent level) before the barrier; then the split raises its ready flag for each
    // of the group's gatherers with device-scope stores
    const int nk = p.gather_k;
    unsigned int* flags = p.tickets + (size_t)g * nk * nflag;
    __builtin_amdgcn_s_waitcnt(0);
    ps_.mark(6);   // phase 6: partial stores acknowledged
    __syncthreads();
    if (tid < nk) __hip_atomic_store(flags + tid * nflag + split, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int k = split - (nsplit - nk);
    ps_.mark(7);   // phase 7: ready flags raised
    if (k < 0) {
        ps_.flush(FAR ? -1 : wg_index, tid, NW);
        return;
    }
    // the barrier above ended every read of the wave states: the gather reuses that LDS
    gather_chunk<NQ, D, NT, GATED>(p, g, nslot, nflag, nq, nk, k, flags + k * nflag, reinterpret_cast<int*>(s_acc));
    ps_.mark_drained(8);   // phase 8: column chunk gathered and its output stored
    ps_.flush(FAR ? -1 : wg_index, tid, NW);
}

template <int D, int NQ, int T, int NT>
__global__ __launch_bounds__(NT, 2) void attn_decode_kernel(const AttnParams p) {
    decode_split<D, NQ, T, NT, false, false>(p, (int)blockIdx.x);
}

// A one-row call with a far field: first the far partials of the nh heads (far_part.h, one
// workgroup each), so that their chain of dependent loads (group state, landmark keys, mixing
// matrix, far numerators, the evicted row) starts with the launch and runs while the splits
// stream the ring, then the splits. A far workgroup stores its partial at device scope, waits
// for those stores and raises its flag for each of its group's gatherers. (The same partials
// made by the group's first splits after their own work measured 18.2 against 14.8 us on the
// 4096-slot decode heads: the chain then starts only when the ring has been read.) GATED: the
// gated one-row call, whose far state is current (no eviction in the call).
template <int D, int NQ, int T, int NT, bool GATED>
__global__ __launch_bounds__(NT, 2) void attn_decode_far_kernel(const AttnParams p, const FarParams f) {
    static_assert(NT == 256, "the far part runs on 256 threads");
    const int bid = (int)blockIdx.x;
    if (bid < f.nh) {
        far_part_block<D, GATED ? kFarCurrent : kFarFusedOneRow, true>(f, bid);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        const int g = bid / p.hpg, nk = p.gather_k, nflag = p.nsplit_grid + p.hpg;
        if ((int)threadIdx.x < nk)
            __hip_atomic_store(p.tickets + ((size_t)g * nk + threadIdx.x) * nflag + p.nsplit_grid + bid % p.hpg,
                               1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
    }
    decode_split<D, NQ, T, NT, true, GATED>(p, bid - f.nh);
}

template <int D, int NQ, int T, int NT>
static hipError_t launch_decode_tt(const AttnParams& p, const FarParams* f, bool gated, hipStream_t stream) {
    const dim3 block(NT);
    if (f) {
        const dim3 grid((unsigned)(f->nh + p.nsplit_grid * p.ng));
        if (gated)
            hipLaunchKernelGGL((attn_decode_far_kernel<D, NQ, T, NT, true>), grid, block, 0, stream, p, *f);
        else
            hipLaunchKernelGGL((attn_decode_far_kernel<D, NQ, T, NT, false>), grid, block, 0, stream, p, *f);
    } else {
        const dim3 grid((unsigned)(p.nsplit_grid * p.ng));
        hipLaunchKernelGGL((attn_decode_kernel<D, NQ, T, NT>), grid, block, 0, stream, p);
    }
    return hipGetLastError();
}

// The instances: 1-4 ring tiles per split with 4 queries per block, 1-2 with 8.
template <int D, int NQ>
static hipError_t launch_decode_t(const AttnParams& p, const FarParams* f, bool gated, int tiles,
                                  hipStream_t stream) {
    constexpr int MT = DecodeShape<D, NQ, kThreads>::MAX_TILES;
    if (tiles == 1) return launch_decode_tt<D, NQ, 1, kThreads>(p, f, gated, stream);
    if (tiles == 2 && MT >= 2) return launch_decode_tt<D, NQ, (MT >= 2 ? 2 : 1), kThreads>(p, f, gated, stream);
    if (tiles == 3 && MT >= 3) return launch_decode_tt<D, NQ, (MT >= 3 ? 3 : 1), kThreads>(p, f, gated, stream);
    if (tiles == 4 && MT >= 4) return launch_decode_tt<D, NQ, (MT >= 4 ? 4 : 1), kThreads>(p, f, gated, stream);
    return hipErrorInvalidValue;
}

int decode_max_tiles(int dpad, int nq) {
    if (dpad == 64) return nq == 4 ? DecodeShape<64, 4, kThreads>::MAX_TILES : DecodeShape<64, 8, kThreads>::MAX_TILES;
    if (dpad == 128) return nq == 4 ? DecodeShape<128, 4, kThreads>::MAX_TILES : DecodeShape<128, 8, kThreads>::MAX_TILES;
    return nq == 4 ? DecodeShape<256, 4, kThreads>::MAX_TILES : DecodeShape<256, 8, kThreads>::MAX_TILES;
}

// f: the far part of a one-row call (its partial in slot nsplit of each group, p.hpg flags
// more per gatherer), or null; gated (with f): the gated one-row call.
hipError_t launch_decode(const AttnParams& p, const FarParams* f, bool gated, int dpad, int nq, int tiles,
                         hipStream_t stream) {
    if (gated && !f) return hipErrorInvalidValue;
    if (f && (f->rows != 1 || f->dpad != dpad || f->nh != p.nh || f->qb != nq || f->nqblocks != 1 ||
              f->far_slot != p.nsplit_grid || f->slot_stride != p.nsplit_grid + 1 || p.slot_stride != f->slot_stride))
        return hipErrorInvalidValue;
    if (dpad == 64 && nq == 4) return launch_decode_t<64, 4>(p, f, gated, tiles, stream);
    if (dpad == 64 && nq == 8) return launch_decode_t<64, 8>(p, f, gated, tiles, stream);
    if (dpad == 128 && nq == 4) return launch_decode_t<128, 4>(p, f, gated, tiles, stream);
    if (dpad == 128 && nq == 8) return launch_decode_t<128, 8>(p, f, gated, tiles, stream);
    if (dpad == 256 && nq == 4) return launch_decode_t<256, 4>(p, f, gated, tiles, stream);
    if (dpad == 256 && nq == 8) return launch_decode_t<256, 8>(p, f, gated, tiles, stream);
    return hipErrorInvalidValue;
}

}  // namespace winattn

#ifdef WINATTN_PHASE_STAMPS
// Timing builds: where the decode kernel writes its phase stamps (NULL: nowhere). The buffer
// holds kStampWords u64 per wave of the launch; each launch overwrites it.
extern "C" int attn_phase_stamps_set(void* device_ptr) {
    return hipMemcpyToSymbol(HIP_SYMBOL(winattn::g_phase_stamps), &device_ptr, sizeof(device_ptr)) == hipSuccess
               ? 0
               : -3;
}
#endif
