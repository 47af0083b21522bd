// Device-side pieces shared by the attention kernels: the launch parameters, the per-group
// window, key addressing over sinks / ring / chunk, wave reductions and the split merge.
//
// Window semantics (o1c page, "A sealed layer's attention for a chunk of rows, on Metal":
// `wgf`, `o1c_score`; dory page, "Dory's token path": `low_key`): every KV group has a logical
// key stream; row i sees the stream's entries x in [lo_i, hi_i) with hi_i = hi0 + i and
// lo_i = hi_i - min(wcap, hi_i), plus the group's ns sink keys. Entry x < xsplit lives in the
// ring at slot (base + x) mod mod; entry x >= xsplit is chunk row x - xsplit.
//   chunk call:  base = head0, mod = wg, xsplit = len0, hi0 = len0 + 1, wcap = wg
//   gated call:  positions from P0 = max(0, pos0 + 1 - window) on; base = P0 mod cap,
//                mod = cap, xsplit = never (the prep kernel wrote the chunk's rows into the
//                ring), hi0 = pos0 + 1 - P0, wcap = window.
// In both cases base < mod and every ring entry read has x < mod, so one conditional
// subtraction gives the slot.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace winattn {

typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kThreads = 256;

struct AttnParams {
    const float* ring_k;
    const float* ring_v;
    const uint32_t* meta;        // chunk calls, and the gated one-row call (else NULL)
    const float* sink_k;
    const float* sink_v;
    const float* q;              // [rows][nh][d]
    const float* chunk_k;
    const float* chunk_v;
    float* out;                  // [rows][nh][d]
    const float* gate;           // gated call only: [rows][nh*d]
    const float* gate_scale;     // gated call only: [nh*d]
    float* pacc;                 // split partials: [blocks][slot_stride][QB][D]
    float* pm;                   // [blocks][slot_stride][QB] running max (log2 domain)
    float* pl;                   // [blocks][slot_stride][QB] running sum
    unsigned int* tickets;       // [blocks]
    long long ring_gs, ring_ss;  // ring strides in floats: per group, per slot
    long long chunk_rs, chunk_gs;
    int rows, ng, hpg, nh, d, w, ns;
    int tps;                     // key tiles per split
    int nsplit_grid;             // splits reserved per query block
    int slot_stride;             // partial slots per query block: the splits, plus one for the
                                 // far field when the call has one
    int nqblocks;                // query blocks per group
    float scale_log2;            // scale * log2(e): scores live in the log2 domain
    int g_base, g_mod, g_hi0, g_wcap;   // gated call's ring descriptor
    int merge_kernel;            // 1: splits are merged by a separate kernel launch
    int xcd_map;                 // matrix-core kernel's work order (see attn_mfma.hip)
    int gather_k;                // slot-order kernel: gatherers (column chunks) per group
};

struct GroupWin {
    int base, mod, xsplit, hi0, wcap;
};

template <bool GATED>
__device__ inline GroupWin resolve_group(const AttnParams& p, int g) {
    GroupWin r;
    if constexpr (GATED) {
        if (p.meta) {
            // The gated one-row call: the row's own key is already in the ring, which holds
            // exactly the window, so ring slots 0 .. len-1 are the keys (storage order is
            // irrelevant to the softmax). len is clamped to w.
            const uint32_t len = p.meta[4 * g] < (uint32_t)p.w ? p.meta[4 * g] : (uint32_t)p.w;
            r.base = 0;
            r.mod = p.w;
            r.xsplit = (int)len;
            r.hi0 = (int)len;
            r.wcap = p.w;
        } else {
            r.base = p.g_base;
            r.mod = p.g_mod;
            r.xsplit = 0x7fffffff;
            r.hi0 = p.g_hi0;
            r.wcap = p.g_wcap;
        }
    } else {
        // Out-of-range meta is clamped so that no access leaves the group's ring.
        const uint32_t* m = p.meta + 4 * g;
        uint32_t ov = m[3];
        uint32_t wg = (ov != 0u && ov < (uint32_t)p.w) ? ov : (uint32_t)p.w;
        uint32_t len0 = m[0] < wg ? m[0] : wg;
        uint32_t head0 = m[1];
        if (head0 >= wg) head0 %= wg;
        r.base = (int)head0;
        r.mod = (int)wg;
        r.xsplit = (int)len0;
        r.hi0 = (int)len0 + 1;
        r.wcap = (int)wg;
    }
    return r;
}

// First visible stream entry of a row whose window ends (exclusive) at hi.
__device__ inline int window_lo(int hi, int wcap) { return hi - (wcap < hi ? wcap : hi); }

// Key tiles of a query block: first ceil(ns / TK) sink tiles (sink index t*TK + k), then stream
// tiles covering the block's stream range [xlo, xhi) (entry xlo + (t - nst)*TK + k). Sink tiles
// belong to split 0. The block's stream tiles (known only here: they depend on the ring's
// metadata) are divided evenly among the nsplit_grid splits the launch reserves per block, so
// every split gets the same work whatever the window's fill; with fewer tiles than splits the
// leading splits take one tile each and the rest are empty. The plan sizes nsplit_grid so that
// no split exceeds its tiles-per-split bound.
struct Tiles {
    int nst;       // sink tiles
    int nstream;   // stream tiles
    int nsplit;    // splits that have work (the leading ones)
    int t_begin, t_end;
};

template <int TK>
__device__ inline Tiles tile_range(int ns, int xlo, int xhi, int nsplit_grid, int split) {
    Tiles r;
    r.nst = (ns + TK - 1) / TK;
    r.nstream = (xhi - xlo + TK - 1) / TK;
    r.nsplit = min(nsplit_grid, r.nstream);
    const int div = max(r.nsplit, 1);   // no stream tiles: no split has work
    const int lo = (int)((long long)split * r.nstream / div);
    const int hi = (int)((long long)(split + 1) * r.nstream / div);
    r.t_begin = split == 0 ? 0 : r.nst + lo;
    r.t_end = r.nst + hi;
    return r;
}

// K and V rows of key k of tile t, chosen with selects rather than branches so that a thread's
// tile loads issue back to back. Padding keys (past the sinks or past the block's stream
// range) get the group ring's first row, a valid address, and `valid` = false: the caller
// loads unconditionally and zeroes the value by select.
// K/V base addresses held as integers in registers. Selecting between pointer fields of the
// argument struct makes the compiler fetch the chosen field from memory (or spill the choice
// to scratch) before every K/V load; integer selects plus an explicit global address space
// keep the loads as plain global loads that issue back to back.
typedef float vf4 __attribute__((ext_vector_type(4)));
typedef const vf4 __attribute__((address_space(1)))* gvf4p;

struct KVBases {
    unsigned long long rk, rv, sk, sv, ck, cv;
};

__device__ inline KVBases kv_bases(const AttnParams& p) {
    return KVBases{(unsigned long long)p.ring_k, (unsigned long long)p.ring_v,
                   (unsigned long long)p.sink_k, (unsigned long long)p.sink_v,
                   (unsigned long long)p.chunk_k, (unsigned long long)p.chunk_v};
}

__device__ inline float4 ld4(unsigned long long base, int off_floats) {
    const vf4 v = *reinterpret_cast<gvf4p>(base + 4ull * (unsigned int)off_floats);
    return make_float4(v.x, v.y, v.z, v.w);
}

__device__ inline float4 zero_unless(bool keep, float4 v) {
    return make_float4(keep ? v.x : 0.0f, keep ? v.y : 0.0f, keep ? v.z : 0.0f, keep ? v.w : 0.0f);
}

// Loads a K/V tile into registers: thread t takes float4 column t % (D/4) of keys
// t / (D/4) + j * (256 / (D/4)), j < LPT. Sink tiles and stream tiles take separate
// (tile-uniform) paths; within a stream tile a row is in the ring (slot (base + x) mod mod,
// one conditional subtraction) or in the chunk. Offsets within a group are 32-bit (the host
// keeps every tensor under 2^31 floats). Padding keys (past the sinks, past the block's stream
// range, or columns beyond d) load the group's first ring row, a valid address; the returned
// mask has bit j set for real keys, and the caller zeroes the others by select when it copies
// the tile to LDS, so the loads issue back to back with nothing waiting on them.
template <int TK, int D, int LPT>
__device__ inline unsigned load_tile_regs(const AttnParams& p, const KVBases b,
                                          const GroupWin& gw, int g, int xlo, int xhi, int nst,
                                          int t, int d4, float4 (&kr)[LPT], float4 (&vr)[LPT]) {
    static_assert(LPT <= 32, "validity mask holds 32 loads");
    unsigned mask = 0u;
    constexpr int D4 = D / 4;
    constexpr int KPP = kThreads / D4;   // keys per pass of the block
    const int key0 = threadIdx.x / D4, c = threadIdx.x % D4;
    const bool col_ok = c < d4;
    const unsigned long long rk = b.rk + 4ull * (unsigned long long)((long long)g * p.ring_gs);
    const unsigned long long rv = b.rv + 4ull * (unsigned long long)((long long)g * p.ring_gs);
    if (t < nst) {
        const unsigned long long sk = b.sk + 4ull * (unsigned long long)((long long)g * p.ns * p.d);
        const unsigned long long sv = b.sv + 4ull * (unsigned long long)((long long)g * p.ns * p.d);
#pragma unroll
        for (int j = 0; j < LPT; ++j) {
            const int si = t * TK + key0 + KPP * j;
            const bool valid = si < p.ns && col_ok;
            const int off = valid ? si * p.d + 4 * c : 0;
            kr[j] = ld4(valid ? sk : rk, off);
            vr[j] = ld4(valid ? sv : rv, off);
            mask |= valid ? 1u << j : 0u;
        }
    } else {
        const unsigned long long ck = b.ck + 4ull * (unsigned long long)((long long)g * p.chunk_gs);
        const unsigned long long cv = b.cv + 4ull * (unsigned long long)((long long)g * p.chunk_gs);
        const int ss = (int)p.ring_ss, crs = (int)p.chunk_rs;
        const int x0 = xlo + (t - nst) * TK + key0;
#pragma unroll
        for (int j = 0; j < LPT; ++j) {
            const int x = x0 + KPP * j;
            const bool valid = x < xhi && col_ok;
            const bool in_ring = x < gw.xsplit || !valid;
            int slot = gw.base + x;
            slot = slot >= gw.mod ? slot - gw.mod : slot;
            const int off = !valid ? 0 : (in_ring ? slot * ss : (x - gw.xsplit) * crs) + 4 * c;
            kr[j] = ld4(in_ring ? rk : ck, off);
            vr[j] = ld4(in_ring ? rv : cv, off);
            mask |= valid ? 1u << j : 0u;
        }
    }
    return mask;
}

// Whether key k of tile t is visible to a query whose stream window is [lo, hi); `sinks` is
// false for padding queries.
template <int TK>
__device__ inline bool key_visible(int ns, int xlo, int nst, int t, int k, int lo, int hi,
                                   bool sinks) {
    if (t < nst) return sinks && t * TK + k < ns;
    const int x = xlo + (t - nst) * TK + k;
    return x >= lo && x < hi;
}

// Cross-lane steps on DPP (data-parallel primitives: a VALU operand read from another lane of
// the same row of 16 or broadcast across rows), not on the LDS crossbar.
enum : int {
    kDppXor1 = 0xB1,          // quad_perm [1,0,3,2]
    kDppXor2 = 0x4E,          // quad_perm [2,3,0,1]
    kDppHalfMirror = 0x141,   // lane i <-> 7 - i within each half row
    kDppMirror = 0x140,       // lane i <-> 15 - i within each row
    kDppBcast15 = 0x142,      // lane 15 of each row to the whole next row
    kDppBcast31 = 0x143,      // lane 31 to rows 2 and 3
};

template <int CTRL, int ROW_MASK = 0xF>
__device__ inline float dpp(float v, float fill) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(fill), __float_as_int(v), CTRL,
                                                      ROW_MASK, 0xF, false));
}

// Max / sum over groups of N adjacent lanes (N in 2, 4, 8, 16), result in every lane of a group.
template <int N>
__device__ inline float group_max(float v) {
    if constexpr (N >= 2) v = fmaxf(v, dpp<kDppXor1>(v, -INFINITY));
    if constexpr (N >= 4) v = fmaxf(v, dpp<kDppXor2>(v, -INFINITY));
    if constexpr (N >= 8) v = fmaxf(v, dpp<kDppHalfMirror>(v, -INFINITY));
    if constexpr (N >= 16) v = fmaxf(v, dpp<kDppMirror>(v, -INFINITY));
    return v;
}

template <int N>
__device__ inline float group_sum(float v) {
    if constexpr (N >= 2) v += dpp<kDppXor1>(v, 0.0f);
    if constexpr (N >= 4) v += dpp<kDppXor2>(v, 0.0f);
    if constexpr (N >= 8) v += dpp<kDppHalfMirror>(v, 0.0f);
    if constexpr (N >= 16) v += dpp<kDppMirror>(v, 0.0f);
    return v;
}

// Max / sum of a lane's value with that of lane l ^ 32 (gfx950 v_permlane32_swap: with the
// same value in both operands, the two results hold the lane's own and its partner's value).
__device__ inline float half_swap_max(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float half_swap_sum(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Max / sum over the whole wave, returned uniform (every lane).
__device__ inline float wave_max(float v) {
    v = group_max<16>(v);
    v = fmaxf(v, dpp<kDppBcast15, 0xA>(v, -INFINITY));
    v = fmaxf(v, dpp<kDppBcast31, 0xC>(v, -INFINITY));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

__device__ inline float wave_sum(float v) {
    v = group_sum<16>(v);
    v += dpp<kDppBcast15, 0xA>(v, 0.0f);
    v += dpp<kDppBcast31, 0xC>(v, 0.0f);
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Numerically safe online-softmax step in the log2 domain. Given the running max m_old and the
// new candidate max, returns the max to subtract (0 while nothing is visible, so that
// exp2(-inf - m) = 0 instead of NaN).
__device__ inline float safe_max(float m_new) { return m_new == -INFINITY ? 0.0f : m_new; }

// Lazy rescaling of an online softmax: the running reference max moves only when a score
// exceeds it by more than this (log2 units), so every weight exp2(s - m) stays below 2^8 and
// the accumulators are rescaled rarely.
constexpr float kLazyRescale = 8.0f;

// Gate epilogue of the gated call (`dory_gate`): o / (1 + exp(-g * s)).
__device__ inline float4 gate4(const AttnParams& p, int row, int gh, int e, float4 o) {
    const size_t at = (size_t)gh * p.d + e;
    float4 gv = *reinterpret_cast<const float4*>(p.gate + (size_t)row * p.nh * p.d + at);
    float4 sv = *reinterpret_cast<const float4*>(p.gate_scale + at);
    o.x = o.x / (1.0f + expf(-(gv.x * sv.x)));
    o.y = o.y / (1.0f + expf(-(gv.y * sv.y)));
    o.z = o.z / (1.0f + expf(-(gv.z * sv.z)));
    o.w = o.w / (1.0f + expf(-(gv.w * sv.w)));
    return o;
}

template <bool GATED>
__device__ inline void store_out(const AttnParams& p, int qi, int g, int e, float4 o) {
    const int row = qi / p.hpg, gh = g * p.hpg + qi % p.hpg;
    if constexpr (GATED) o = gate4(p, row, gh, e, o);
    *reinterpret_cast<float4*>(p.out + ((size_t)row * p.nh + gh) * p.d + e) = o;
}

// Split partials merged inside the launch cross XCDs, whose L2 caches are not coherent with
// each other. The protocol (specific to gfx950's memory hierarchy):
//  - partials are stored with the device-scope (sc1) cache policy: agent-scope atomic stores for
//    scalars, 16-byte buffer stores with that policy for float4s; such stores are written
//    through to the device-coherent level and acknowledged from there;
//  - every thread waits for its stores' acknowledgements (vmcnt 0) before a barrier, so all of a
//    workgroup's partial stores are complete device-wide before its ticket or flag is set, which
//    is itself an agent-scope atomic;
//  - the reader acquires at agent scope (or reads with device-scope loads) after it saw the
//    ticket or flag.
// An agent-scope release fence per workgroup would do the same formally but writes back the
// whole L2 each time; hundreds of them serialise into tens of microseconds.
typedef unsigned int vu4 __attribute__((ext_vector_type(4)));
constexpr int kBufferWord3 = 0x00020000;    // raw (untyped) buffer resource word 3 on gfx9
constexpr int kCachePolicyDevice = 16;      // sc1: device (agent) scope

__device__ inline void store_dev(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A ready flag as a poll loop reads it: a relaxed agent-scope atomic load, coherent at device
// scope and, unlike a plain or buffer load, never hoisted out of the loop or merged with an
// earlier read of the same flag by the compiler.
__device__ inline unsigned poll_flag(const unsigned int* f) {
    return __hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// After every split of a query block has written its partial (m, l, acc), the last one to
// arrive combines them: c = max_s m_s, out = sum_s acc_s 2^(m_s - c) / sum_s l_s 2^(m_s - c)
// (the token path's partial merge, `o1c_tok_merge`). All threads of the block call it after
// writing their partials. `scratch` is free LDS of at least kMergeScratch floats.
//
// The merge is one CU reading every split's partial of the block, so it is laid out as one
// round of loads: each thread owns an item (query j, float4 column c) and a subset of the
// splits, issues all of that subset's loads together, folds them with the online rescaling,
// and the subsets meet in LDS.
constexpr int kMergeScratch = 6 * kThreads;
constexpr int kMergeUnroll = 16;

struct Part {
    float m, l;
    float4 a;
};

__device__ inline void part_fold(Part& x, float m, float l, float4 a) {
    const float mn = fmaxf(x.m, m), mu = safe_max(mn);
    const float cx = __builtin_amdgcn_exp2f(x.m - mu), cy = __builtin_amdgcn_exp2f(m - mu);
    x.l = x.l * cx + l * cy;
    x.a.x = x.a.x * cx + a.x * cy;
    x.a.y = x.a.y * cx + a.y * cy;
    x.a.z = x.a.z * cx + a.z * cy;
    x.a.w = x.a.w * cx + a.w * cy;
    x.m = mn;
}

// Fold splits s = s0, s0 + stride, ... < nsplit of item (j, c) into x, kMergeUnroll at a time.
template <int QB, int D>
__device__ inline void fold_splits(const AttnParams& p, size_t base, int j, int c, int s0,
                                   int stride, int nsplit, Part& x) {
    for (int s = s0; s < nsplit; s += kMergeUnroll * stride) {
        float m[kMergeUnroll], l[kMergeUnroll];
        float4 a[kMergeUnroll];
        // Unconditional loads (a split index past the end reads the last split again) so that
        // the whole batch issues back to back; the extra entries are dropped by select.
#pragma unroll
        for (int u = 0; u < kMergeUnroll; ++u) {
            const int su = min(s + u * stride, nsplit - 1);
            const size_t at = base + (size_t)su * QB + j;
            m[u] = p.pm[at];
            l[u] = p.pl[at];
            a[u] = *reinterpret_cast<const float4*>(p.pacc + at * D + 4 * c);
        }
#pragma unroll
        for (int u = 0; u < kMergeUnroll; ++u) {
            // past the end, or a split that marked its slot empty (m = -inf)
            const bool real = s + u * stride < nsplit && m[u] > -INFINITY;
            part_fold(x, real ? m[u] : -INFINITY, real ? l[u] : 0.0f,
                      real ? a[u] : make_float4(0.f, 0.f, 0.f, 0.f));
        }
    }
}

// Combines the nsplit partials of query block `blk` into the output (all NT threads of the
// block call it), for the DC columns starting at column 4 * c0 (DC = D: every column).
// `scratch` is free LDS of at least 6 * NT floats (kMergeScratch for 256 threads).
template <int QB, int D, bool GATED, int DC = D, int NT = kThreads>
__device__ inline void merge_block(const AttnParams& p, int blk, int nsplit, int q0, int nq, int g,
                                   float* scratch, int c0 = 0) {
    static_assert(DC % 4 == 0 && D % DC == 0, "column chunk must divide the padded width");
    constexpr int D4 = DC / 4;
    const int d4 = p.d / 4;
    const size_t base = (size_t)blk * p.slot_stride * QB;
    constexpr int ITEMS = QB * D4;
    if constexpr (ITEMS >= NT) {
        // Several items per thread, KG at a time: the loads of a group's items for a batch of U
        // splits issue together (storing one item's output before the next item's loads would
        // make each item a round trip of its own: the compiler cannot tell the output from the
        // partials).
        constexpr int IPT = ITEMS / NT;
        constexpr int KG = IPT < 4 ? IPT : 4;
        constexpr int U = 16 / KG;
        static_assert(IPT % KG == 0, "item groups");
#pragma unroll 1
        for (int k0 = 0; k0 < IPT; k0 += KG) {
            Part x[KG];
            int jj[KG], cc[KG];
#pragma unroll
            for (int k = 0; k < KG; ++k) {
                const int item = threadIdx.x + NT * (k0 + k);
                jj[k] = item / D4;
                cc[k] = c0 + item % D4;
                x[k] = Part{-INFINITY, 0.0f, make_float4(0.f, 0.f, 0.f, 0.f)};
            }
            for (int s = 0; s < nsplit; s += U) {
                float m[KG][U], l[KG][U];
                float4 a[KG][U];
#pragma unroll
                for (int k = 0; k < KG; ++k)
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        // unconditional (past the end: the last split again, dropped below)
                        const size_t at = base + (size_t)min(s + u, nsplit - 1) * QB + jj[k];
                        m[k][u] = p.pm[at];
                        l[k][u] = p.pl[at];
                        a[k][u] = *reinterpret_cast<const float4*>(p.pacc + at * D + 4 * cc[k]);
                    }
#pragma unroll
                for (int k = 0; k < KG; ++k)
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        // past the end, or a split that marked its slot empty (m = -inf)
                        const bool real = s + u < nsplit && m[k][u] > -INFINITY;
                        part_fold(x[k], real ? m[k][u] : -INFINITY, real ? l[k][u] : 0.0f,
                                  real ? a[k][u] : make_float4(0.f, 0.f, 0.f, 0.f));
                    }
            }
#pragma unroll
            for (int k = 0; k < KG; ++k) {
                if (jj[k] < nq && cc[k] < d4) {
                    const float inv = 1.0f / fmaxf(x[k].l, 1e-30f);
                    store_out<GATED>(p, q0 + jj[k], g, 4 * cc[k],
                                     make_float4(x[k].a.x * inv, x[k].a.y * inv, x[k].a.z * inv,
                                                 x[k].a.w * inv));
                }
            }
        }
    } else {
        constexpr int NSUB = NT / ITEMS;
        const int item = threadIdx.x % ITEMS, sub = threadIdx.x / ITEMS;
        const int j = item / D4, c = c0 + item % D4;
        Part x{-INFINITY, 0.0f, make_float4(0.f, 0.f, 0.f, 0.f)};
        fold_splits<QB, D>(p, base, j, c, sub, NSUB, nsplit, x);
        float* s_m = scratch;
        float* s_l = scratch + NT;
        float4* s_a = reinterpret_cast<float4*>(scratch + 2 * NT);
        s_m[threadIdx.x] = x.m;
        s_l[threadIdx.x] = x.l;
        s_a[threadIdx.x] = x.a;
        __syncthreads();
        if (threadIdx.x < ITEMS && j < nq && c < d4) {
            for (int u = 1; u < NSUB; ++u) {
                const int t = u * ITEMS + item;
                part_fold(x, s_m[t], s_l[t], s_a[t]);
            }
            const float inv = 1.0f / fmaxf(x.l, 1e-30f);
            store_out<GATED>(p, q0 + j, g, 4 * c,
                             make_float4(x.a.x * inv, x.a.y * inv, x.a.z * inv, x.a.w * inv));
        }
    }
}

// With a separate merge launch, a split that has no keys for its block marks the block's partial
// slots empty (m = -inf), and a block with a single split still writes a partial: the merge
// kernel then folds every split slot of the grid without resolving the group's window.
template <int QB>
__device__ inline void mark_split_empty(const AttnParams& p, int blk, int split) {
    if (p.merge_kernel && threadIdx.x < QB)
        p.pm[((size_t)blk * p.slot_stride + split) * QB + threadIdx.x] = -INFINITY;
}

// After every split of a query block has written its partial, the last one to arrive merges
// them. When the plan uses a separate merge kernel (p.merge_kernel), this returns at once.
template <int QB, int D, bool GATED, int NT = kThreads>
__device__ inline void merge_if_last(const AttnParams& p, int blk, int nsplit, int q0, int nq,
                                     int g, int* s_flag, float* scratch) {
    static_assert(QB <= NT && NT % QB == 0, "query block must divide the block");
    if (p.merge_kernel) return;
    // Every thread's device-scope partial stores are acknowledged before the counter moves.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned int prev =
            __hip_atomic_fetch_add(p.tickets + blk, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int last = (prev == (unsigned int)(nsplit - 1));
        if (last) __hip_atomic_store(p.tickets + blk, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *s_flag = last;
    }
    __syncthreads();
    if (!*s_flag) return;
    // Acquire at agent scope: drop this XCD's L2 copies of lines other XCDs have written, so the
    // plain vector loads below read the partials the other splits stored at device scope.
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    merge_block<QB, D, GATED, D, NT>(p, blk, nsplit, q0, nq, g, scratch);
}

// Partial stores: device scope for the in-kernel merge; plain when a separate merge kernel
// reads them after the kernel boundary.
__device__ inline void store_part(const AttnParams& p, float* dst, float v) {
    if (p.merge_kernel) *dst = v; else store_dev(dst, v);
}
// float4 column `col` of query j's accumulator in partial slot `split` of query block `blk`
// (QB queries of D floats per slot). The device-scope store is one 16-byte buffer store
// addressed from the slot's base, which is uniform over the workgroup.
template <int QB, int D>
__device__ inline void store_part4(const AttnParams& p, int blk, int split, int j, int col, float4 v) {
    float* slot = p.pacc + ((size_t)blk * p.slot_stride + split) * QB * D;
    if (p.merge_kernel) {
        *reinterpret_cast<float4*>(slot + (size_t)j * D + col) = v;
    } else {
        const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(slot, 0, QB * D * 4, kBufferWord3);
        __builtin_amdgcn_raw_buffer_store_b128(vu4{__float_as_uint(v.x), __float_as_uint(v.y),
                                                   __float_as_uint(v.z), __float_as_uint(v.w)},
                                               r, (j * D + col) * 4, 0, kCachePolicyDevice);
    }
}

}  // namespace winattn
