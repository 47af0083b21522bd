// The gated call in one launch for wide unit heads (head width in (128, 256], a multiple of 32):
// rotation and unit norms of the queries and of the chunk's keys, the ring write, attention over
// each row's window and the sigmoid gate (dory page, "Dory's token path": `dory_prep`,
// `low_key`, `dory_score`, `dory_soft`, `dory_sum`, `dory_gate`).
//
// Prior art on that page: a preparation dispatch writes the unit heads and the ring, then score,
// softmax, sum and gate dispatches run over the materialised scores. Here nothing is
// materialised and nothing waits for a separate preparation pass. Two forms share the plan:
//
// Register form (16 to 63 query vectors per KV head), attn_gated_kernel:
//  - A query set is 16 query vectors of one KV head (consecutive (row, head) pairs). The
//    workgroup rotates and normalises them once, from the raw heads, the table row and the
//    learned scale, into LDS, where every wave reads them as the B operand of
//    v_mfma_f32_16x16x4f32.
//  - The set's key positions are cut into 16-key blocks. A workgroup (4 waves, one per SIMD)
//    takes one split of them and its waves take every fourth block; each wave loads its blocks'
//    K and V straight from memory into registers in MFMA operand order (no LDS staging, no
//    barrier in the loop), two blocks ahead in two register buffers: a block's loads have the
//    products of the block before it to arrive.
//  - Keys at positions before the chunk come from the ring, which already holds unit keys; keys
//    of the chunk's own rows are rotated and normalised from the raw heads where they are used,
//    so no wave waits for another's ring write. The wave that owns a chunk row's block in the
//    row's own query set also writes that row's unit key and raw value into the ring. No reader
//    outside this call's own writers reads those slots (the ring holds more than
//    window + rows - 1 positions).
//  - The 4 waves of a workgroup meet in LDS; the splits of a set meet as in the decode kernel:
//    partials stored with the device-scope cache policy and acknowledged, then a ready flag;
//    the set's last split (dispatched after all the others) folds them, each wave a quarter of
//    the columns, and applies 1 / sum and the gate.
//
// Tile form (64 or more query vectors per KV head), attn_gated_tiles_kernel: blocks of 64
// queries, 32-key tiles staged in LDS, two waves per SIMD; described at the kernel.
//
// Layout on v_mfma_f32_16x16x4f32 (lane l supplies A[l%16][l/16] and B[l/16][l%16];
// accumulator r of lane l is element (4*(l/16) + r, l%16)):
//   scores  S^T = K . Q^T: A = K (key l%16, d = 16m + 4*(l/16) + e at step (m, e)),
//           B = Q^T (query l%16, same d); lane l holds query l%16 against keys 4*(l/16) + r
//   values  O^T = V^T . P^T: at step c (keys 4j + c, j = l/16) B = P^T is the lane's score r = c
//           and A = V^T with d-row l%16 of block db = 4q + e meaning d = 64q + 4*(l%16) + e,
//           so each lane reads V as float4s; accumulator r of block db holds
//           d = 64q + 16*(l/16) + 4r + e.
// Rotation pairs d and d + hd/2 sit in the same lane (hd/2 is a multiple of 16), and the sums
// of squares of a query or key run over the lane's values and its three partner lanes
// l ^ 16, l ^ 32, l ^ 48.
#include <type_traits>

#include "winattn_dev.h"
#include "launch.h"

namespace winattn {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kGatedPolls = 1 << 18;

// Max / sum over the four lanes of a column: l, l ^ 16, l ^ 32, l ^ 48.
__device__ inline float col_max(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return half_swap_max(fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1])));
}
__device__ inline float col_sum(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return half_swap_sum(__uint_as_float(r[0]) + __uint_as_float(r[1]));
}

__device__ inline f32x4 ldg4(const float* base, long long off) {
    return *reinterpret_cast<const f32x4*>(base + off);
}

__device__ inline f32x4 shfl4(f32x4 v, int src) {
    return f32x4{__shfl(v.x, src), __shfl(v.y, src), __shfl(v.z, src), __shfl(v.w, src)};
}

}  // namespace

// HM = hd / 32: the head width, 32 HM (5 to 8). NW waves per workgroup, one per SIMD; each keeps
// two blocks of K and V in flight (register buffers A and B), so that a block's loads have the
// products of the block before it to arrive.
template <int HM, int NW>
__global__ __launch_bounds__(64 * NW, 1) void attn_gated_kernel(const GatedFusedParams p) {
    constexpr int NT = 64 * NW;
    constexpr int QST = 256 + 4;          // LDS row of a query (padded: no bank conflicts)
    constexpr int CPW = 256 / NW;         // output columns each wave folds at the end
    constexpr int R = CPW / 16;           // float4s per lane of those columns
    static_assert(NT >= 256 && CPW % 16 == 0, "workgroup shape");
    __shared__ __align__(16) float s_q[16 * QST];         // the set's rotated unit queries
    __shared__ __align__(16) float s_o[NW * 16 * 256];    // each wave's (query, d) accumulators
    __shared__ float s_m[NW * 16], s_l[NW * 16];
    __shared__ int s_done[NW];

    // Block -> (split, query set), splits major: a set's last split (its gatherer) is dispatched
    // after every other split. Blocks go to the 8 XCDs round-robin; sets are dealt in contiguous
    // eighths of (KV head, set) order, so an XCD's sets share few KV heads (their K/V stay in its
    // L2) and every split of a set runs on one XCD.
    const int nqs_tot = p.nk * p.nqs;
    const int bid = (int)blockIdx.x;
    const int split = bid / nqs_tot;
    const int rr = bid % nqs_tot;
    const int qsg = nqs_tot % 8 == 0 ? (rr % 8) * (nqs_tot / 8) + rr / 8 : rr;
    const int kh = qsg / p.nqs, qs = qsg % p.nqs;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lr = lane >> 4;
    constexpr int hd = 32 * HM, half = 16 * HM;
    const int nqv = p.rows * p.hpg;              // query vectors of a KV head
    const int v0 = qs * 16;

    // This lane's query vector (column li of the set; padding repeats the last one) and window.
    const bool qvalid = v0 + li < nqv;
    const int vq = qvalid ? v0 + li : nqv - 1;
    const int qrow = vq / p.hpg, qhead = kh * p.hpg + vq % p.hpg;
    const int qpos = p.pos0 + qrow;
    const int qlo = max(0, qpos + 1 - p.window);
    // The set's key positions [plo, phi] in 16-key blocks; this split's blocks [b0, b1), of which
    // the wave takes b0 + wave, b0 + wave + NW, ...
    const int r_first = v0 / p.hpg, r_last = min(v0 + 15, nqv - 1) / p.hpg;
    const int plo = max(0, p.pos0 + r_first + 1 - p.window), phi = p.pos0 + r_last;
    const int nb = (phi - plo + 16) / 16;
    const int b0 = (int)((long long)nb * split / p.nsplit);
    const int b1 = (int)((long long)nb * (split + 1) / p.nsplit);

    // column offset of this lane's float4 for step m (d = 16m + 4 lr)
    auto dcol = [&](int m) { return 16 * m + 4 * lr; };

    // ---- key block loads (block kb: positions plo + 16 kb + 0..15; past phi: position phi).
    // Ring position pos: slot pos mod cap; chunk row c = pos - pos0: the raw heads (rotated and
    // normalised after the load).
    const long long ring_row = (long long)p.nk * hd;
    auto k_src = [&](int pos) -> const float* {
        return pos < p.pos0 ? p.ring_k + (long long)(pos % p.cap) * ring_row + (long long)kh * hd
                            : p.yk + ((long long)(pos - p.pos0) * p.nk + kh) * hd;
    };
    auto v_src = [&](int pos) -> const float* {
        return pos < p.pos0 ? p.ring_v + (long long)(pos % p.cap) * ring_row + (long long)kh * hd
                            : p.yv + ((long long)(pos - p.pos0) * p.nk + kh) * hd;
    };
    auto load_k = [&](f32x4 (&kf)[16], int kb) {
        const float* src = k_src(min(plo + 16 * kb + li, phi));
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            const bool in = dcol(m) < hd;
            kf[m] = in ? ldg4(src, dcol(m)) : f32x4{0.f, 0.f, 0.f, 0.f};
        }
    };
    auto load_v = [&](f32x4 (&vf)[16], int kb) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const float* src = v_src(min(plo + 16 * kb + 4 * lr + c, phi));
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int d = 64 * q + 4 * li;
                vf[4 * c + q] = d < hd ? ldg4(src, d) : f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
    };
    // Owner of chunk row c: the set holding the row's first query vector; there the row's block
    // belongs to exactly one (split, wave).
    auto owns_row = [&](int pos) {
        const int c = pos - p.pos0;
        return pos >= p.pos0 && pos <= phi && (c * p.hpg) / 16 == qs;
    };

    // The wave's first block is requested before the queries, so both round trips overlap.
    // Loads are never skipped: past the wave's last block they repeat that block (or the set's
    // first block when the wave has none), so every iteration has the same loads in flight and
    // the waits before the products name exactly the block they need.
    const int kb0 = b0 + wave;
    const int klast = max(0, b1 - 1);
    // DB: two register buffers per wave (one wave per SIMD); else one (two waves per SIMD, the
    // other wave's products cover a wave's waits)
    constexpr bool DB = NW == 4;
    f32x4 ka[16], va[16], kb_[DB ? 16 : 1], vb_[DB ? 16 : 1];
    load_k(ka, min(kb0, klast));
    load_v(va, min(kb0, klast));
    if constexpr (DB) {
        load_k(kb_, min(kb0 + NW, klast));
        load_v(vb_, min(kb0 + NW, klast));
    }

    // ---- the set's queries, once per workgroup: thread t < 512 takes query t / 32 and the
    // float4 pair (4j, 4j + hd/2), j = t % 32 < hd/8: rotation, unit norm over the query's 32
    // threads (half a wave), learned scale, scale * log2 e; columns past hd are zero
    for (int i = tid; i < 16 * QST / 4; i += NT)
        reinterpret_cast<f32x4*>(s_q)[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 512 / NT; ++k) {   // all loads of the queries in flight together
        const int t = tid + k * NT;
        const int q = t >> 5, j = t & 31;
        const bool on = 4 * j < half;
        const int vt = min(v0 + q, nqv - 1);
        const int row = vt / p.hpg, head = kh * p.hpg + vt % p.hpg;
        const int d = on ? 4 * j : 0;
        const float* yq = p.yq + ((long long)row * p.nh + head) * hd;
        const float* rope = p.rope + (long long)row * hd;
        const float* qsc = p.q_scale + (long long)head * hd;
        const f32x4 a = ldg4(yq, d), b = ldg4(yq, d + half), cs = ldg4(rope, d), sn = ldg4(rope, d + half);
        const f32x4 sa = ldg4(qsc, d), sb = ldg4(qsc, d + half);
        const f32x4 u = a * cs - b * sn, v = b * cs + a * sn;
        float ss = on ? (u.x * u.x + u.y * u.y) + (u.z * u.z + u.w * u.w) +
                            (v.x * v.x + v.y * v.y) + (v.z * v.z + v.w * v.w)
                      : 0.0f;
#pragma unroll
        for (int o = 1; o < 32; o <<= 1) ss += __shfl_xor(ss, o);
        const float f = p.scale_log2 / sqrtf(ss + p.eps);
        if (on) {
            *reinterpret_cast<f32x4*>(s_q + q * QST + d) = u * sa * f;
            *reinterpret_cast<f32x4*>(s_q + q * QST + d + half) = v * sb * f;
        }
    }
    __syncthreads();

    f32x4 oacc[16];
#pragma unroll
    for (int b = 0; b < 16; ++b) oacc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
    float mrun = -INFINITY, lrun = 0.0f;
    const float* qrowp = s_q + li * QST;   // B operand: query li, d = 16m + 4 lr + e

    // One block from the register buffers (kf, vf), which then take block kn. An inactive step
    // (past the wave's last block) skips the arithmetic but issues the same loads.
    auto step = [&](f32x4 (&kf)[16], f32x4 (&vf)[16], int kb, int kn, bool active)
                    __attribute__((always_inline)) {
      if (active) {
        const int base = plo + 16 * kb;
        // a block holding chunk rows: this lane's key (column li), where it is a chunk row, is
        // rotated and normalised in place with its table row (read here: such blocks are few)
        if (base + 15 >= p.pos0) {
            const int pos = min(base + li, phi);
            const bool chunk = pos >= p.pos0;
            const float* rope = p.rope + (long long)max(0, pos - p.pos0) * hd;
            float ss = 0.0f;
#pragma unroll
            for (int m = 0; m < HM; ++m) {
                const f32x4 cs = ldg4(rope, dcol(m)), sn = ldg4(rope, dcol(m + HM));
                const f32x4 a = kf[m], b = kf[m + HM];
                const f32x4 u = a * cs - b * sn, v = b * cs + a * sn;
                kf[m] = chunk ? u : a;
                kf[m + HM] = chunk ? v : b;
                ss += (u.x * u.x + u.y * u.y) + (u.z * u.z + u.w * u.w);
                ss += (v.x * v.x + v.y * v.y) + (v.z * v.z + v.w * v.w);
            }
            const float inv = chunk ? 1.0f / sqrtf(col_sum(ss) + p.eps) : 1.0f;
#pragma unroll
            for (int m = 0; m < 16; ++m) kf[m] *= inv;
            if (owns_row(base + li)) {
                float* dst = p.ring_k + (long long)((base + li) % p.cap) * ring_row + (long long)kh * hd;
#pragma unroll
                for (int m = 0; m < 16; ++m)
                    if (dcol(m) < hd) *reinterpret_cast<f32x4*>(dst + dcol(m)) = kf[m];
            }
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int vpos = base + 4 * lr + c;
                if (owns_row(vpos)) {
                    float* dst = p.ring_v + (long long)(vpos % p.cap) * ring_row + (long long)kh * hd;
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        if (64 * q + 4 * li < hd) *reinterpret_cast<f32x4*>(dst + 64 * q + 4 * li) = vf[4 * c + q];
                }
            }
        }

        // scores: four independent accumulation chains (one per float4 component). The queries
        // are read from LDS for every block: the empty asm keeps the compiler from hoisting
        // those reads out of the loop into 64 more live registers.
        asm volatile("" : : : "memory");
        f32x4 s4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) s4[e] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            const f32x4 q4 = *reinterpret_cast<const f32x4*>(qrowp + dcol(m));
            s4[0] = __builtin_amdgcn_mfma_f32_16x16x4f32(kf[m].x, q4.x, s4[0], 0, 0, 0);
            s4[1] = __builtin_amdgcn_mfma_f32_16x16x4f32(kf[m].y, q4.y, s4[1], 0, 0, 0);
            s4[2] = __builtin_amdgcn_mfma_f32_16x16x4f32(kf[m].z, q4.z, s4[2], 0, 0, 0);
            s4[3] = __builtin_amdgcn_mfma_f32_16x16x4f32(kf[m].w, q4.w, s4[3], 0, 0, 0);
        }
        f32x4 s = (s4[0] + s4[1]) + (s4[2] + s4[3]);
        load_k(kf, kn);   // K registers are free: a later block's keys

        // visibility (the query's window, inside the set's range) and the online softmax
        float tmax = -INFINITY;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int pos = base + 4 * lr + r;
            const bool vis = pos >= qlo && pos <= qpos && pos <= phi;
            s[r] = vis ? s[r] : -INFINITY;
            tmax = fmaxf(tmax, s[r]);
        }
        // The exponentials are taken against a reference max mrun that moves only when a score
        // exceeds it by more than kLazyRescale (a factor 2^8 at most on any weight): the
        // accumulators are then rescaled rarely after the first block. (m, l, O) stay
        // consistent with mrun, which is what the merges take.
        tmax = col_max(tmax);
        const bool grow = tmax > mrun + kLazyRescale;
        if (__any(grow)) {
            const float m_new = grow ? tmax : mrun;
            const float corr = __builtin_amdgcn_exp2f(mrun - safe_max(m_new));
            lrun *= corr;
#pragma unroll
            for (int b = 0; b < 16; ++b) oacc[b] *= corr;
            mrun = m_new;
        }
        const float mu = safe_max(mrun);
        float psum = 0.0f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            s[r] = __builtin_amdgcn_exp2f(s[r] - mu);
            psum += s[r];
        }
        lrun += col_sum(psum);

        // values
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f32x4 v = vf[4 * c + q];
                oacc[4 * q + 0] = __builtin_amdgcn_mfma_f32_16x16x4f32(v.x, s[c], oacc[4 * q + 0], 0, 0, 0);
                oacc[4 * q + 1] = __builtin_amdgcn_mfma_f32_16x16x4f32(v.y, s[c], oacc[4 * q + 1], 0, 0, 0);
                oacc[4 * q + 2] = __builtin_amdgcn_mfma_f32_16x16x4f32(v.z, s[c], oacc[4 * q + 2], 0, 0, 0);
                oacc[4 * q + 3] = __builtin_amdgcn_mfma_f32_16x16x4f32(v.w, s[c], oacc[4 * q + 3], 0, 0, 0);
            }
        load_v(vf, kn);   // V registers are free
      } else {
        load_k(kf, kn);
        load_v(vf, kn);
      }
    };
    if constexpr (DB) {
        for (int kb = kb0; kb < b1; kb += 2 * NW) {
            step(ka, va, kb, min(kb + 2 * NW, klast), true);
            step(kb_, vb_, kb + NW, min(kb + 3 * NW, klast), kb + NW < b1);
        }
    } else {
        for (int kb = kb0; kb < b1; kb += NW) step(ka, va, kb, min(kb + NW, klast), true);
    }

    // ---- the waves of the workgroup meet: each publishes (m, l, O) in LDS, then wave w folds
    // output columns [CPW w, CPW (w + 1)) of the 16 queries over the NW waves
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int d = 64 * q + 16 * lr + 4 * r;
            *reinterpret_cast<f32x4*>(s_o + (wave * 16 + li) * 256 + d) =
                f32x4{oacc[4 * q + 0][r], oacc[4 * q + 1][r], oacc[4 * q + 2][r], oacc[4 * q + 3][r]};
        }
    if (lr == 0) {
        s_m[wave * 16 + li] = mrun;
        s_l[wave * 16 + li] = lrun;
    }
    __syncthreads();
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, s_m[w * 16 + li]);
    float L = 0.0f;
    f32x4 O[R];
#pragma unroll
    for (int r = 0; r < R; ++r) O[r] = f32x4{0.f, 0.f, 0.f, 0.f};
    // this lane: query li, columns d = CPW wave + 4 R lr + 4 r
    const int dl = CPW * wave + 4 * R * lr;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const float f = __builtin_amdgcn_exp2f(s_m[w * 16 + li] - safe_max(M));
        L += s_l[w * 16 + li] * f;
#pragma unroll
        for (int r = 0; r < R; ++r)
            O[r] += *reinterpret_cast<const f32x4*>(s_o + (w * 16 + li) * 256 + dl + 4 * r) * f;
    }

    // the gate of this lane's output columns, requested before any wait for partials
    f32x4 gv[R], gsv[R];
    {
        const float* g = p.gate + (long long)qrow * p.nh * hd + (long long)qhead * hd;
        const float* gs = p.gate_scale + (long long)qhead * hd;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int d = dl + 4 * r;
            gv[r] = ldg4(g, d < hd ? d : 0);
            gsv[r] = ldg4(gs, d < hd ? d : 0);
        }
    }
    auto finish = [&](bool bad) {
        const float inv = 1.0f / fmaxf(L, 1e-30f);
        float* dst = p.out + ((long long)qrow * p.nh + qhead) * hd;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int d = dl + 4 * r;
            f32x4 o = O[r] * inv;
            o.x = o.x / (1.0f + expf(-(gv[r].x * gsv[r].x)));
            o.y = o.y / (1.0f + expf(-(gv[r].y * gsv[r].y)));
            o.z = o.z / (1.0f + expf(-(gv[r].z * gsv[r].z)));
            o.w = o.w / (1.0f + expf(-(gv[r].w * gsv[r].w)));
            if (bad) o = f32x4{NAN, NAN, NAN, NAN};
            if (qvalid && d < hd) *reinterpret_cast<f32x4*>(dst + d) = o;
        }
    };
    if (p.nsplit == 1) {
        finish(false);
        return;
    }

    // ---- splits of a set: partial (M, L, O) of item (set, split), written through to the
    // device-coherent level, acknowledged, then the split's ready flag
    const int last = p.nsplit - 1;
    unsigned int* flags = p.flags + (long long)qsg * p.nsplit;
    const long long item0 = (long long)qsg * p.nsplit;
    if (split < last) {
        const long long it = item0 + split;
        const __amdgpu_buffer_rsrc_t part =
            __builtin_amdgcn_make_buffer_rsrc(p.pacc + it * 16 * 256, 0, 16 * 256 * 4, kBufferWord3);
#pragma unroll
        for (int r = 0; r < R; ++r)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(vu4, O[r]), part,
                                                   (li * 256 + dl + 4 * r) * 4, 0, kCachePolicyDevice);
        if (wave == 0 && lr == 0) {
            store_dev(p.pm + it * 16 + li, M);
            store_dev(p.pl + it * 16 + li, L);
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (tid == 0) __hip_atomic_store(flags + split, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
    }

    // ---- the gatherer: each wave polls the set's flags and folds its columns
    const __amdgpu_buffer_rsrc_t racc =
        __builtin_amdgcn_make_buffer_rsrc(p.pacc + item0 * 16 * 256, 0, last * 16 * 256 * 4, kBufferWord3);
    const __amdgpu_buffer_rsrc_t rm = __builtin_amdgcn_make_buffer_rsrc(p.pm + item0 * 16, 0, last * 16 * 4, kBufferWord3);
    const __amdgpu_buffer_rsrc_t rl = __builtin_amdgcn_make_buffer_rsrc(p.pl + item0 * 16, 0, last * 16 * 4, kBufferWord3);
    unsigned long long pend = last >= 64 ? ~0ull : ((1ull << last) - 1ull);
    int polls = 0;
    while (pend != 0ull && polls < kGatedPolls) {
        ++polls;
        const unsigned f = poll_flag(flags + min(lane, last - 1));
        unsigned long long ready = __builtin_amdgcn_ballot_w64(f != 0u && lane < last) & pend;
        if (ready == 0ull) {
            __builtin_amdgcn_s_sleep(2);
            continue;
        }
        pend &= ~ready;
        while (ready != 0ull) {   // wave-uniform
            const int sp = __builtin_ctzll(ready);
            ready &= ready - 1ull;
            const int at = sp * 16 + li;
            const float m1 = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rm, at * 4, 0, kCachePolicyDevice));
            const float l1 = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rl, at * 4, 0, kCachePolicyDevice));
            f32x4 a[R];
#pragma unroll
            for (int r = 0; r < R; ++r)
                a[r] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                     racc, (at * 256 + dl + 4 * r) * 4, 0, kCachePolicyDevice));
            const float mn = fmaxf(M, m1), mu = safe_max(mn);
            const float f0 = __builtin_amdgcn_exp2f(M - mu), f1 = __builtin_amdgcn_exp2f(m1 - mu);
            L = L * f0 + l1 * f1;
#pragma unroll
            for (int r = 0; r < R; ++r) O[r] = O[r] * f0 + a[r] * f1;
            M = mn;
        }
    }
    if (lane == 0) s_done[wave] = pend == 0ull ? 1 : 0;
    __syncthreads();   // every wave has left its poll loop
    bool bad = false;
#pragma unroll
    for (int w = 0; w < NW; ++w) bad |= s_done[w] == 0;
    finish(bad);
    if (!bad && tid < last) __hip_atomic_store(flags + tid, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

constexpr int kGatedWaves = 4;

// ---- Tile form, for 64 or more query vectors per KV head. The same work in the layout of the
// 16x16 matrix-core kernel of the three-launch path: a block is 64 query vectors (four sets of
// 16) of one KV head; its positions are cut into 16-key blocks, shared among the block's
// splits; each split streams 32-key tiles into double-buffered LDS with direct global-to-LDS
// loads only, and runs 8 waves, two per SIMD: waves w and w + 4 own the same 16 queries and
// take the two 16-key halves of each tile, so that one wave's softmax overlaps the other's
// products.
//  - Prologue: the workgroup makes the block's 64 unit queries once (each wave 8 of them) and
//    passes them through LDS; tile 0 is in flight meanwhile.
//  - Chunk rows: a split whose range holds positions of the chunk first rotates and normalises
//    those rows' raw keys into the ring (several blocks may write one slot, always with the same
//    bytes; the raw value goes to the ring once, from the split that owns the row in the block
//    of its first query vector); its tiles then load them from there like any ring row, and
//    take chunk values straight from the raw heads. That split is counted one 16-key block
//    more than it streams, so that its extra work does not make it the last to finish.
//  - The two key halves of a query set fold in LDS (each wave keeps half of the columns); the
//    splits meet as in the decode kernel: partials with device-scope stores, acknowledged, one
//    ready flag per gatherer; the block's last gather_k splits wait for every flag, then each
//    reads its column chunk of all partials at once, folds them in split order, applies
//    1 / sum and the gate (read before the wait) and stores it.
constexpr int kGTK = 32;          // keys per tile
constexpr int kGKST = 256 + 4;    // LDS row stride (floats)

// Phase stamps of the tile form, in timing builds only (compiled with WINATTN_PHASE_STAMPS; the
// normal build contains none of this code): every wave reads the 100 MHz real-time counter at
// the phase boundaries below, keeps the readings in registers and writes them once, at its end,
// with its XCD number, to g_gated_stamps[block * 8 + wave][kGatedStampWords] when the host has
// set that pointer (attn_gated_stamps_set). The kernel's work is unchanged.
//   0 start, 1 queries in registers, 2 tile 0 in LDS, 3 tile 0 done, 4 tile 1 in LDS,
//   5 tile 1 done, 6 every tile done, 7 key halves folded, 8 flags raised (non-gatherers end),
//   9 every flag seen (gatherers), 10 outputs stored and drained (gatherers, single splits);
//   then the XCD, and the shader-clock counter at the start and when the stamps are written
#ifdef WINATTN_PHASE_STAMPS
constexpr int kGatedStampWords = 14;
__device__ unsigned long long* g_gated_stamps;
struct GatedStamps {
    unsigned long long t[11] = {};
    unsigned long long clk0 = __builtin_amdgcn_s_memtime();
    __device__ void mark(int k) { t[k] = __builtin_amdgcn_s_memrealtime(); }
    template <class V>
    __device__ void mark_after(int k, const V& v) {
        asm volatile("" : : "v"(v));
        mark(k);
    }
    __device__ void mark_drained(int k) {
        __builtin_amdgcn_s_waitcnt(0);
        mark(k);
    }
    __device__ void flush(int tid) {
        unsigned long long* o = g_gated_stamps;
        if (!o || (tid & 63) != 0) return;
        const unsigned long long clk1 = __builtin_amdgcn_s_memtime();
        o += ((size_t)blockIdx.x * 8 + tid / 64) * kGatedStampWords;
        for (int k = 0; k < 11; ++k) o[k] = t[k];
        o[11] = __builtin_amdgcn_s_getreg(20 | (0 << 6) | (3 << 11));   // XCC_ID
        o[12] = clk0;
        o[13] = clk1;
    }
};
#else
struct GatedStamps {
    __device__ void mark(int) {}
    template <class V>
    __device__ void mark_after(int, const V&) {}
    __device__ void mark_drained(int) {}
    __device__ void flush(int) {}
};
#endif

template <int HM>
__global__ __launch_bounds__(512, 1) void attn_gated_tiles_kernel(const GatedFusedParams p) {
    constexpr int NT = 512, NW = 8, TK = kGTK, KST = kGKST, QB = 64;
    constexpr int hd = 32 * HM, half = 16 * HM, d4 = hd / 4;
    // Each LDS tile buffer is its own array, so that the compiler sees that reading one buffer
    // never conflicts with the direct loads still filling the other, and leaves them in flight.
    __shared__ __align__(16) float s_k0[TK * KST];
    __shared__ __align__(16) float s_v0[TK * KST];
    __shared__ __align__(16) float s_k1[TK * KST];
    __shared__ __align__(16) float s_v1[TK * KST];
    __shared__ int s_done[NW];

    // Block -> (split, query block), splits major: every split that a gatherer waits for is
    // dispatched before the gatherers' splits, or is itself a gatherer (and raises its flags
    // before it gathers). Query blocks are dealt to the XCDs in contiguous eighths of
    // (KV head, block) order, so an XCD's blocks share few KV heads.
    const int nqb_tot = p.nk * p.nqs;
    const int bid = (int)blockIdx.x;
    const int split = bid / nqb_tot;
    const int rr = bid % nqb_tot;
    const int qbg = nqb_tot % 8 == 0 ? (rr % 8) * (nqb_tot / 8) + rr / 8 : rr;
    const int kvh = qbg / p.nqs, qb = qbg % p.nqs;
    const int S = p.nsplit;

    // the wave index as a scalar: row indices, pointer choices and branches derived from it
    // stay on the scalar unit
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int qw = wave & 3, kh = wave >> 2;          // query set, key half of each tile
    GatedStamps stamps;
    stamps.mark(0);
    const int qcol = lane & 15, kr4 = lane >> 4;
    const int nqv = p.rows * p.hpg;
    const int v0 = qb * QB;

    // This lane's query vector (column qcol of set qw; padding repeats the last) and window.
    const int jq = 16 * qw + qcol;
    const bool qvalid = v0 + jq < nqv;
    const int vq = qvalid ? v0 + jq : nqv - 1;
    const int qrow = vq / p.hpg;
    const int qpos = p.pos0 + qrow, qlo = max(0, qpos + 1 - p.window);
    // The block's positions [plo, phi], its 16-key blocks, this split's share [ks0, ks1)
    const int r_first = v0 / p.hpg, r_last = min(v0 + QB - 1, nqv - 1) / p.hpg;
    const int plo = max(0, p.pos0 + r_first + 1 - p.window), phi = p.pos0 + r_last;
    const int nb = (phi - plo + 16) / 16;
    // The last split also makes the chunk rows' unit keys: it is counted one 16-key block more
    // than it streams (nb + 1 shares). The larger shares go to the first splits, which gather
    // nothing, so that every gatherer is done with its own tiles early.
    const int shq = (nb + 1) / S, shr = (nb + 1) % S;
    const int bs0 = min(nb, split * shq + min(split, shr));
    const int bs1 = min(nb, (split + 1) * shq + min(split + 1, shr));
    const int ks0 = plo + 16 * bs0, ks1 = min(plo + 16 * bs1, phi + 1);
    const int ntile = (bs1 - bs0 + 1) / 2;

    // ---- tile t of the split (positions ks0 + 32 t + key) into LDS buffers (tkb, tvb), straight
    // from memory: wave w loads rows w, w + 8, w + 16, w + 24; positions past phi load position phi
    // (masked later). Keys always come from the ring: a chunk row's unit key is written there by
    // this workgroup before its first tile (see below); values of chunk rows come from the raw
    // heads. Nothing is waited for here, so the loads stay in flight under the current tile's
    // products.
    const long long ring_row = (long long)p.nk * hd;
    const unsigned col = 4u * (unsigned)(lane < d4 ? lane : 0);
    auto issue_tile = [&](int t, float* tkb, float* tvb) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < TK / NW; ++i) {
            const int key = wave + NW * i;
            const int pos = min(ks0 + TK * t + key, phi);
            const long long at = (long long)(pos % p.cap) * ring_row + (long long)kvh * hd + col;
            const long long cat = ((long long)max(0, pos - p.pos0) * p.nk + kvh) * hd + col;
            __builtin_amdgcn_global_load_lds(p.ring_k + at, tkb + key * KST, 16, 0, 0);
            __builtin_amdgcn_global_load_lds(pos < p.pos0 ? p.ring_v + at : p.yv + cat, tvb + key * KST, 16, 0, 0);
        }
    };
    // the split's chunk rows: positions [cs0, ks1) (empty for most splits)
    const int cs0 = max(ks0, p.pos0);
    auto tile_has_chunk = [&](int t) { return ks0 + TK * t + TK - 1 >= p.pos0; };

    // ---- chunk rows in the split's range: rotation and unit norm of the raw keys into the ring
    // (read back by the tile loads; every workgroup whose range holds the row writes the same
    // bytes), and the raw value into the ring by the one split that owns the row in the block
    // holding its first query vector. Wave w takes rows cs0 + w, cs0 + w + 8, ..., eight at a
    // time with all their loads in flight; lane l the float4 at d = 4l, its rotation partner
    // in lane l +- hd/8.
    auto make_chunk_keys = [&]() __attribute__((always_inline)) {
        const int pl_lane = lane < 4 * HM ? lane + 4 * HM : lane - 4 * HM;
        const int dm = 4 * (lane < 4 * HM ? lane : lane - 4 * HM);   // d mod hd/2
        const bool on = lane < d4;
        constexpr int PR = 8;
        for (int r0 = cs0 + wave; r0 < ks1; r0 += PR * NW) {
            f32x4 ka[PR], kc[PR], ksn[PR], va[PR];
#pragma unroll
            for (int i = 0; i < PR; ++i) {
                const int c = min(r0 + NW * i, ks1 - 1) - p.pos0;
                const long long cat = ((long long)c * p.nk + kvh) * hd;
                const float* rope = p.rope + (long long)c * hd;
                ka[i] = ldg4(p.yk + cat, col);
                va[i] = ldg4(p.yv + cat, col);
                kc[i] = ldg4(rope, on ? dm : 0);
                ksn[i] = ldg4(rope, on ? half + dm : 0);
            }
#pragma unroll
            for (int i = 0; i < PR; ++i) {
                const int pos = r0 + NW * i;
                const f32x4 a = ka[i], b = shfl4(a, pl_lane);
                f32x4 r = lane < 4 * HM ? a * kc[i] - b * ksn[i] : a * kc[i] + b * ksn[i];
                r = on ? r : f32x4{0.f, 0.f, 0.f, 0.f};
                const float ss = wave_sum((r.x * r.x + r.y * r.y) + (r.z * r.z + r.w * r.w));
                r *= 1.0f / sqrtf(ss + p.eps);
                if (pos < ks1 && on) {
                    const int c = pos - p.pos0;
                    const long long rat = (long long)(pos % p.cap) * ring_row + (long long)kvh * hd + col;
                    *reinterpret_cast<f32x4*>(p.ring_k + rat) = r;
                    if ((c * p.hpg) / QB == qb) *reinterpret_cast<f32x4*>(p.ring_v + rat) = va[i];
                }
            }
        }
        __builtin_amdgcn_s_waitcnt(0);   // the unit keys are written before any wave loads them
    };

    // ---- the block's 64 unit queries (times q_scale, scale and log2 e), made once per workgroup
    // into the second tile buffers (queries 0..31 in s_k1, 32..63 in s_v1), which tile 1 takes
    // only after the loop's first barrier: wave w makes queries 8w .. 8w + 7, lane 8 j + c the
    // float4 pairs (4 c', 4 c' + hd/2) for c' = c, c + 8, c + 16, c + 24 below hd/8. The query
    // loads are requested before tile 0's, so that waiting for them leaves the tile in flight
    // (tile 0 is requested on every path, so that the wait can name the query loads alone).
    {
        const int qj = 8 * wave + (lane >> 3), c8 = lane & 7;
        const int vt = min(v0 + qj, nqv - 1);
        const int row = vt / p.hpg, head = kvh * p.hpg + vt % p.hpg;
        const float* yq = p.yq + ((long long)row * p.nh + head) * hd;
        const float* rope = p.rope + (long long)row * hd;
        const float* qsc = p.q_scale + (long long)head * hd;
        f32x4 a[4], b[4], cs[4], sn[4], sa[4], sb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = c8 + 8 * i;
            const int d = 4 * c < half ? 4 * c : 0;
            a[i] = ldg4(yq, d);
            b[i] = ldg4(yq, d + half);
            cs[i] = ldg4(rope, d);
            sn[i] = ldg4(rope, d + half);
            sa[i] = ldg4(qsc, d);
            sb[i] = ldg4(qsc, d + half);
        }
        __builtin_amdgcn_sched_barrier(0);
        issue_tile(0, s_k0, s_v0);
        __builtin_amdgcn_sched_barrier(0);
        float ss = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const f32x4 u = a[i] * cs[i] - b[i] * sn[i], v = b[i] * cs[i] + a[i] * sn[i];
            a[i] = u;
            b[i] = v;
            if (4 * (c8 + 8 * i) < half)
                ss += ((u.x * u.x + u.y * u.y) + (u.z * u.z + u.w * u.w)) +
                      ((v.x * v.x + v.y * v.y) + (v.z * v.z + v.w * v.w));
        }
        ss += __shfl_xor(ss, 1);
        ss += __shfl_xor(ss, 2);
        ss += __shfl_xor(ss, 4);
        const float f = p.scale_log2 / sqrtf(ss + p.eps);
        // (a branch on the wave, not a pointer choice, names the array each store writes, so that
        // the compiler sees that they do not touch the buffers tile 0 is loading into)
        auto put = [&](float* qd) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int d = 4 * (c8 + 8 * i);
                if (d < half) {
                    *reinterpret_cast<f32x4*>(qd + d) = a[i] * sa[i] * f;
                    *reinterpret_cast<f32x4*>(qd + d + half) = b[i] * sb[i] * f;
                }
            }
        };
        if (wave < 4) put(s_k1 + qj * KST);
        else put(s_v1 + (qj - 32) * KST);
    }
    if (cs0 < ks1) make_chunk_keys();
    __syncthreads();
    // a first tile holding chunk rows of this split is loaded again now that their unit keys
    // are in the ring (the first load has landed: the chunk-key pass waited for it)
    if (cs0 < ks1 && tile_has_chunk(0)) issue_tile(0, s_k0, s_v0);
    // this wave's queries as the B operand: qreg[m] holds query jq at d = 16m + 4 kr4 (+ 0..3),
    // zero past hd
    f32x4 qreg[16];
    auto get_q = [&](const float* ql) __attribute__((always_inline)) {
#pragma unroll
        for (int m = 0; m < 16; ++m)
            qreg[m] = 16 * m + 4 * kr4 < hd ? *reinterpret_cast<const f32x4*>(ql + 16 * m)
                                            : f32x4{0.f, 0.f, 0.f, 0.f};
    };
    if (qw < 2) get_q(s_k1 + jq * KST + 4 * kr4);
    else get_q(s_v1 + (jq - 32) * KST + 4 * kr4);
    stamps.mark_after(1, qreg[15].w);

    f32x4 oacc[16];
#pragma unroll
    for (int b = 0; b < 16; ++b) oacc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
    float mrun = -INFINITY, lrun = 0.0f;
    // this lane's visible positions within the split
    const int vlo = max(qlo, ks0), vhi = min(qpos, ks1 - 1);

    // One tile: this wave's 16-key half (keys 16 kh .. 16 kh + 15 of the tile).
    auto compute_tile = [&](int t, const float* tk, const float* tv) __attribute__((always_inline)) {
        const int base = ks0 + TK * t + 16 * kh;
        if (base >= ks1) return;   // the split's last tile may have one half only
        const int klo = vlo - base, khi = vhi - base + 1;
        if (!__any(klo < 16 && khi > 0 && khi > klo)) return;
        constexpr int PF = 2;
        f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
        f32x4 kbuf[PF + 1];
        const float* krow = tk + (16 * kh + qcol) * KST + 4 * kr4;
#pragma unroll
        for (int m = 0; m < PF; ++m) kbuf[m] = *reinterpret_cast<const f32x4*>(krow + 16 * m);
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            if (m + PF < 16) kbuf[(m + PF) % (PF + 1)] = *reinterpret_cast<const f32x4*>(krow + 16 * (m + PF));
            __builtin_amdgcn_sched_barrier(0);
            const f32x4 k4 = kbuf[m % (PF + 1)];
            sacc = __builtin_amdgcn_mfma_f32_16x16x4f32(k4.x, qreg[m].x, sacc, 0, 0, 0);
            sacc = __builtin_amdgcn_mfma_f32_16x16x4f32(k4.y, qreg[m].y, sacc, 0, 0, 0);
            sacc = __builtin_amdgcn_mfma_f32_16x16x4f32(k4.z, qreg[m].z, sacc, 0, 0, 0);
            sacc = __builtin_amdgcn_mfma_f32_16x16x4f32(k4.w, qreg[m].w, sacc, 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        // the first V^T operands, read now so that their latency hides under the softmax
        float vbuf[2][16];
#pragma unroll
        for (int b = 0; b < 16; ++b) vbuf[0][b] = tv[(16 * kh + 4 * kr4) * KST + qcol + 16 * b];
        float tmax = -INFINITY;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int k = 4 * kr4 + r;
            sacc[r] = (k >= klo && k < khi) ? sacc[r] : -INFINITY;
            tmax = fmaxf(tmax, sacc[r]);
        }
        tmax = col_max(tmax);
        // lazy rescaling against a reference max (kLazyRescale)
        const bool grow = tmax > mrun + kLazyRescale;
        if (__any(grow)) {
            const float m_new = grow ? tmax : mrun;
            const float corr = __builtin_amdgcn_exp2f(mrun - safe_max(m_new));
            lrun *= corr;
#pragma unroll
            for (int b = 0; b < 16; ++b) oacc[b] *= corr;
            mrun = m_new;
        }
        const float mu = safe_max(mrun);
        float psum = 0.0f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            sacc[r] = __builtin_amdgcn_exp2f(sacc[r] - mu);
            psum += sacc[r];
        }
        lrun += col_sum(psum);
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            if (st + 1 < 4) {
                const float* vp = tv + (16 * kh + 4 * kr4 + st + 1) * KST + qcol;
#pragma unroll
                for (int b = 0; b < 16; ++b) vbuf[(st + 1) & 1][b] = vp[16 * b];
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int b = 0; b < 16; ++b)
                oacc[b] = __builtin_amdgcn_mfma_f32_16x16x4f32(vbuf[st & 1][b], sacc[st], oacc[b], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // Wait for this wave's rows of tile t; the barrier makes every wave's rows visible and tells
    // that nobody still reads the other buffer (tile t - 1), which then takes t + 1.
    for (int t = 0; t < ntile; t += 2) {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (t == 0) stamps.mark(2);
        if (t + 1 < ntile) issue_tile(t + 1, s_k1, s_v1);
        compute_tile(t, s_k0, s_v0);
        if (t == 0) stamps.mark_after(3, oacc[15].w);
        if (t + 1 < ntile) {
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            if (t == 0) stamps.mark(4);
            if (t + 2 < ntile) issue_tile(t + 2, s_k0, s_v0);
            compute_tile(t + 1, s_k1, s_v1);
            if (t == 0) stamps.mark_after(5, oacc[15].w);
        }
    }
    stamps.mark_after(6, oacc[15].w);

    // ---- the two key halves of each query set meet: wave w (key half kh) keeps the output
    // columns of blocks b in [8 kh, 8 kh + 8), publishes the other half and its (m, l) in the
    // tile buffers and folds in its partner's
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    const int li = qw * 64 + lane;
    // [b][query set][lane] float4s: columns 0..127 in s_k0, 128..255 in s_k1
    auto fo = [&](int b) { return (b < 8 ? s_k0 : s_k1) + ((b & 7) * 256 + li) * 4; };
    float* fm = s_v0;                        // [key half][m | l][query set][lane]
    // Each branch names its registers at compile time (H is the wave's key half).
    auto publish = [&](auto h_c) __attribute__((always_inline)) {
        constexpr int H = decltype(h_c)::value;
#pragma unroll
        for (int b = 8 * (1 - H); b < 8 * (1 - H) + 8; ++b) *reinterpret_cast<f32x4*>(fo(b)) = oacc[b];
    };
    if (kh == 0) publish(std::integral_constant<int, 0>{});
    else publish(std::integral_constant<int, 1>{});
    fm[kh * 512 + li] = mrun;
    fm[kh * 512 + 256 + li] = lrun;
    __syncthreads();
    {
        const float m1 = fm[(1 - kh) * 512 + li], l1 = fm[(1 - kh) * 512 + 256 + li];
        const float mt = fmaxf(mrun, m1), mu = safe_max(mt);
        const float f0 = __builtin_amdgcn_exp2f(mrun - mu), f1 = __builtin_amdgcn_exp2f(m1 - mu);
        lrun = lrun * f0 + l1 * f1;
        mrun = mt;
        auto fold = [&](auto h_c) __attribute__((always_inline)) {
            constexpr int H = decltype(h_c)::value;
#pragma unroll
            for (int b = 8 * H; b < 8 * H + 8; ++b)
                oacc[b] = oacc[b] * f0 + *reinterpret_cast<const f32x4*>(fo(b)) * f1;
        };
        if (kh == 0) fold(std::integral_constant<int, 0>{});
        else fold(std::integral_constant<int, 1>{});
    }
    // Wave w holds, for query jq, d = 16 b + 4 kr4 + (0..3) in oacc[b], b in [8 kh, 8 kh + 8).
    auto out_gated = [&](int v, int d, f32x4 o) {   // gate and store query vector v, column d
        const int row = v / p.hpg, head = kvh * p.hpg + v % p.hpg;
        const f32x4 gv = ldg4(p.gate + (long long)row * p.nh * hd + (long long)head * hd, d);
        const f32x4 sv = ldg4(p.gate_scale + (long long)head * hd, d);
        o.x = o.x / (1.0f + expf(-(gv.x * sv.x)));
        o.y = o.y / (1.0f + expf(-(gv.y * sv.y)));
        o.z = o.z / (1.0f + expf(-(gv.z * sv.z)));
        o.w = o.w / (1.0f + expf(-(gv.w * sv.w)));
        *reinterpret_cast<f32x4*>(p.out + ((long long)row * p.nh + head) * hd + d) = o;
    };
    stamps.mark_after(7, oacc[15].w);
    if (S == 1) {
        if (qvalid) {
            const float inv = 1.0f / fmaxf(lrun, 1e-30f);
            auto out_half = [&](auto h_c) __attribute__((always_inline)) {
                constexpr int H = decltype(h_c)::value;
#pragma unroll
                for (int b = 8 * H; b < 8 * H + 8; ++b) {
                    const int d = 16 * b + 4 * kr4;
                    if (d < hd) out_gated(vq, d, oacc[b] * inv);
                }
            };
            if (kh == 0) out_half(std::integral_constant<int, 0>{});
            else out_half(std::integral_constant<int, 1>{});
        }
        stamps.mark_drained(10);
        stamps.flush(tid);
        return;
    }

    // ---- partial of (block, split): written through to the device-coherent level, then one
    // ready flag per gatherer once every store is acknowledged
    const int G = p.gather_k;
    const long long it = (long long)qbg * S + split;
    {
        const __amdgpu_buffer_rsrc_t part =
            __builtin_amdgcn_make_buffer_rsrc(p.pacc + it * QB * 256, 0, QB * 256 * 4, kBufferWord3);
        auto store_half = [&](auto h_c) __attribute__((always_inline)) {
            constexpr int H = decltype(h_c)::value;
#pragma unroll
            for (int b = 8 * H; b < 8 * H + 8; ++b)
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(vu4, oacc[b]), part,
                                                       (jq * 256 + 16 * b + 4 * kr4) * 4, 0, kCachePolicyDevice);
        };
        if (kh == 0) store_half(std::integral_constant<int, 0>{});
        else store_half(std::integral_constant<int, 1>{});
        if (kh == 0 && kr4 == 0) {
            store_dev(p.pm + it * QB + jq, mrun);
            store_dev(p.pl + it * QB + jq, lrun);
        }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    unsigned int* flags = p.flags + (long long)qbg * G * S;   // [gatherer][split]
    if (tid < G) __hip_atomic_store(flags + tid * S + split, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    stamps.mark(8);
    const int k = split - (S - G);
    if (k < 0) {
        stamps.flush(tid);
        return;
    }

    // ---- gatherer k: columns [k CW, (k + 1) CW) of the block's 64 queries, CW = 256 / G; item
    // i = (query i / (CW / 4), float4 column i % (CW / 4)), IPT = 8 / G items per thread. The
    // waves first wait for every split's flag, then read the partials 16 (item, split) pairs at a
    // time, all requested before any is used, and fold them in split order.
    const int cw4 = 64 / G;                    // float4 columns per gatherer
    unsigned int* gflags = flags + k * S;
    const long long item0 = (long long)qbg * S;
    const __amdgpu_buffer_rsrc_t racc =
        __builtin_amdgcn_make_buffer_rsrc(p.pacc + item0 * QB * 256, 0, S * QB * 256 * 4, kBufferWord3);
    const __amdgpu_buffer_rsrc_t rm = __builtin_amdgcn_make_buffer_rsrc(p.pm + item0 * QB, 0, S * QB * 4, kBufferWord3);
    const __amdgpu_buffer_rsrc_t rl = __builtin_amdgcn_make_buffer_rsrc(p.pl + item0 * QB, 0, S * QB * 4, kBufferWord3);
    bool bad = false;
    auto gather = [&](auto ipt_c) __attribute__((always_inline)) {
        // SB splits per batch; with many items per thread, smaller batches and the gate read at
        // the end keep everything in registers
        constexpr int IPT = decltype(ipt_c)::value, SB = IPT <= 2 ? 16 / IPT : 8 / IPT;
        constexpr bool kGatePre = IPT <= 2;
        float gm[IPT], gl[IPT];
        f32x4 go[IPT], gg[IPT], gs[IPT];
        int gq[IPT], gc[IPT];
#pragma unroll
        for (int j = 0; j < IPT; ++j) {
            const int i = j * NT + tid;
            gq[j] = i / cw4;
            gc[j] = k * cw4 + i % cw4;
            gm[j] = -INFINITY;
            gl[j] = 0.0f;
            go[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        auto load_gate = [&](int j) {
            const int v = min(v0 + gq[j], nqv - 1), d = min(4 * gc[j], hd - 4);
            const int head = kvh * p.hpg + v % p.hpg;
            gg[j] = ldg4(p.gate + ((long long)(v / p.hpg) * p.nh + head) * hd, d);
            gs[j] = ldg4(p.gate_scale + (long long)head * hd, d);
        };
        if constexpr (kGatePre) {   // requested before the wait
#pragma unroll
            for (int j = 0; j < IPT; ++j) load_gate(j);
        }
        unsigned long long pend = S >= 64 ? ~0ull : ((1ull << S) - 1ull);
        int polls = 0;
        // One item per thread and at most 16 splits: each split's partial is requested as soon
        // as its flag is seen (so that only the last splits' loads remain after the last
        // flag), into registers of its own; the fold below still runs in split order.
        constexpr bool kEarly = IPT == 1;
        float em[kEarly ? 16 : 1], el[kEarly ? 16 : 1];
        f32x4 ea[kEarly ? 16 : 1];
        const bool early = kEarly && S <= 16;
        while (pend != 0ull && polls < kGatedPolls) {
            ++polls;
            const unsigned f = poll_flag(gflags + min(lane, S - 1));
            const unsigned long long ready = __builtin_amdgcn_ballot_w64(f != 0u && lane < S) & pend;
            pend &= ~ready;
            if constexpr (kEarly) {
                if (early) {
#pragma unroll
                    for (int u = 0; u < 16; ++u) {
                        if ((ready >> u) & 1ull) {
                            const int at = u * QB + gq[0];
                            em[u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rm, at * 4, 0, kCachePolicyDevice));
                            el[u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rl, at * 4, 0, kCachePolicyDevice));
                            ea[u] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                                  racc, (at * 256 + 4 * gc[0]) * 4, 0, kCachePolicyDevice));
                        }
                    }
                }
            }
            if (pend != 0ull) __builtin_amdgcn_s_sleep(2);
        }
        stamps.mark(9);
        if (lane == 0) s_done[wave] = pend == 0ull ? 1 : 0;
        __syncthreads();   // every wave has left its poll loop
#pragma unroll
        for (int w = 0; w < NW; ++w) bad |= s_done[w] == 0;
        if constexpr (kEarly) {
            if (early && !bad) {
#pragma unroll
                for (int u = 0; u < 16; ++u) {
                    if (u < S) {
                        const float mn = fmaxf(gm[0], em[u]), mu = safe_max(mn);
                        const float f0 = __builtin_amdgcn_exp2f(gm[0] - mu), f1 = __builtin_amdgcn_exp2f(em[u] - mu);
                        gl[0] = gl[0] * f0 + el[u] * f1;
                        go[0] = go[0] * f0 + ea[u] * f1;
                        gm[0] = mn;
                    }
                }
            }
        }
        for (int s0 = 0; s0 < S && !bad && !early; s0 += SB) {
            float m1[IPT][SB], l1[IPT][SB];
            f32x4 a1[IPT][SB];
#pragma unroll
            for (int j = 0; j < IPT; ++j)
#pragma unroll
                for (int u = 0; u < SB; ++u) {
                    const int at = min(s0 + u, S - 1) * QB + gq[j];
                    m1[j][u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rm, at * 4, 0, kCachePolicyDevice));
                    l1[j][u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rl, at * 4, 0, kCachePolicyDevice));
                    a1[j][u] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                             racc, (at * 256 + 4 * gc[j]) * 4, 0, kCachePolicyDevice));
                }
#pragma unroll
            for (int j = 0; j < IPT; ++j)
#pragma unroll
                for (int u = 0; u < SB; ++u) {
                    if (s0 + u < S) {
                        const float mn = fmaxf(gm[j], m1[j][u]), mu = safe_max(mn);
                        const float f0 = __builtin_amdgcn_exp2f(gm[j] - mu), f1 = __builtin_amdgcn_exp2f(m1[j][u] - mu);
                        gl[j] = gl[j] * f0 + l1[j][u] * f1;
                        go[j] = go[j] * f0 + a1[j][u] * f1;
                        gm[j] = mn;
                    }
                }
        }
#pragma unroll
        for (int j = 0; j < IPT; ++j) {
            const int v = v0 + gq[j], d = 4 * gc[j];
            if constexpr (!kGatePre) load_gate(j);
            if (v < nqv && d < hd) {
                f32x4 o = go[j] * (1.0f / fmaxf(gl[j], 1e-30f));
                o.x = o.x / (1.0f + expf(-(gg[j].x * gs[j].x)));
                o.y = o.y / (1.0f + expf(-(gg[j].y * gs[j].y)));
                o.z = o.z / (1.0f + expf(-(gg[j].z * gs[j].z)));
                o.w = o.w / (1.0f + expf(-(gg[j].w * gs[j].w)));
                if (bad) o = f32x4{NAN, NAN, NAN, NAN};
                const int head = kvh * p.hpg + v % p.hpg;
                *reinterpret_cast<f32x4*>(p.out + ((long long)(v / p.hpg) * p.nh + head) * hd + d) = o;
            }
        }
    };
    switch (G) {
        case 8: gather(std::integral_constant<int, 1>{}); break;
        case 4: gather(std::integral_constant<int, 2>{}); break;
        case 2: gather(std::integral_constant<int, 4>{}); break;
        default: gather(std::integral_constant<int, 8>{}); break;
    }
    if (!bad && tid < S) __hip_atomic_store(gflags + tid, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    stamps.mark_drained(10);
    stamps.flush(tid);
}

hipError_t launch_gated_fused(const GatedFusedParams& p, hipStream_t stream) {
    const long long blocks = (long long)p.nk * p.nqs * p.nsplit;
    if (blocks < 1 || blocks > 0x7fffffffLL || p.nsplit < 1 || p.nsplit > 64) return hipErrorInvalidValue;
    if (p.qb == 64) {
        if (p.gather_k < 1 || p.gather_k > 8 || p.gather_k > p.nsplit) return hipErrorInvalidValue;
        const dim3 grid((unsigned)blocks), block(512);
        switch (p.hd) {
            case 160: hipLaunchKernelGGL(attn_gated_tiles_kernel<5>, grid, block, 0, stream, p); break;
            case 192: hipLaunchKernelGGL(attn_gated_tiles_kernel<6>, grid, block, 0, stream, p); break;
            case 224: hipLaunchKernelGGL(attn_gated_tiles_kernel<7>, grid, block, 0, stream, p); break;
            case 256: hipLaunchKernelGGL(attn_gated_tiles_kernel<8>, grid, block, 0, stream, p); break;
            default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    constexpr int NW = kGatedWaves;
    const dim3 grid((unsigned)blocks), block(64 * NW);
    switch (p.hd) {
        case 160: hipLaunchKernelGGL((attn_gated_kernel<5, NW>), grid, block, 0, stream, p); break;
        case 192: hipLaunchKernelGGL((attn_gated_kernel<6, NW>), grid, block, 0, stream, p); break;
        case 224: hipLaunchKernelGGL((attn_gated_kernel<7, NW>), grid, block, 0, stream, p); break;
        case 256: hipLaunchKernelGGL((attn_gated_kernel<8, NW>), grid, block, 0, stream, p); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace winattn

#ifdef WINATTN_PHASE_STAMPS
// Timing builds: where the gated tile kernel writes its phase stamps (NULL: nowhere). The buffer
// holds kGatedStampWords u64 per wave of the launch (8 waves per workgroup); each launch
// overwrites it.
extern "C" int attn_gated_stamps_set(void* device_ptr) {
    return hipMemcpyToSymbol(HIP_SYMBOL(winattn::g_gated_stamps), &device_ptr, sizeof(device_ptr)) == hipSuccess
               ? 0
               : -3;
}
#endif
