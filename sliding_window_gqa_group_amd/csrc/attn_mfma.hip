// Split-K windowed attention on the f32 matrix cores, for chunks with many query vectors per
// KV group (prefill and wide verify chunks).
//
// Prior art: the o1c page's GEMM path (`o1c_gather`, `o1c_gmax`, `o1c_gsoft`, `o1c_gadd`:
// a per-group panel of sinks, ring and chunk keys, score and value GEMMs, live-column masks)
// and the staged flash kernels of the egemma2 page (K/V blocks in threadgroup memory shared by
// several query tiles). Here nothing is materialised: scores stay in registers, and K/V tiles
// are staged once per workgroup in LDS and shared by its four waves.
//
// Layout on v_mfma_f32_32x32x2f32 (A 32x2, B 2x32, 16 accumulators per lane; lane l supplies
// A[l%32][l/32] and B[l/32][l%32]; accumulator r of lane l is element
// (8*(r/4) + 4*(l/32) + r%4, l%32)):
//   scores    S^T = K . Q^T   A = K tile (32 keys x d, from LDS), B = Q^T (registers)
//             -> lane l holds query l%32 against keys 8*(r/4) + 4*(l/32) + r%4
//   values    O^T = V^T . P^T A = V^T (from LDS), B = P^T = exactly the score registers
//             after the softmax step, so P never leaves the lane
// Each k-step of the score product takes d indices {8c + r, 8c + 4 + r} from the two lane
// halves, which lets every lane read its K and Q operands as float4s.
//
// A workgroup owns 128 consecutive query vectors (row-major over (row, head) of one group),
// 32 per wave, and one split of the key tiles that the block's rows can see.
#include "winattn_dev.h"
#include "launch.h"

namespace winattn {

constexpr int kMfmaQB = 128;
constexpr int kMfmaTK = 32;

#ifdef WINATTN_PHASE_STAMPS
// Timing builds only: thread 0 of every workgroup records the 100 MHz real-time counter and the
// shader-clock counter when the workgroup starts and when its last tile is done, as
// g_mfma_clock[block][4] = {real0, clock0, real1, clock1} (attn_mfma_clock_set), from which
// the clock the matrix cores ran at follows.
__device__ unsigned long long* g_mfma_clock;
#endif

template <int D, bool GATED>
__global__ __launch_bounds__(kThreads, D == 256 ? 1 : 2) void attn_mfma_kernel(const AttnParams p) {
    constexpr int TK = kMfmaTK, QB = kMfmaQB;
    constexpr int D4 = D / 4, KST = D + 4, VST = D + 8;
    constexpr int LPT = TK * D4 / kThreads;   // float4 loads per thread per tensor per tile
    constexpr int NDB = D / 32;               // 32-wide d blocks of the output
    static_assert(LPT >= 1 && TK * D4 == LPT * kThreads, "tile load must cover the tile");
    static_assert(TK * KST >= kMergeScratch, "merge scratch reuses the K tile area");

    __shared__ __align__(16) float s_k[TK * KST];
    __shared__ __align__(16) float s_v[TK * VST];
    __shared__ int s_flag;

    // Work item = (group, split, query block), query block fastest. The hardware deals blocks
    // to the 8 XCDs round-robin (block b to XCD b % 8). Two orders:
    //  - xcd_map 1: XCD x takes the x-th contiguous eighth of the items, i.e. whole groups when
    //    the items divide evenly: all query blocks of a group share that XCD's L2, which holds
    //    the group's K/V when its window is short (a few MB);
    //  - xcd_map 0: item = b, every XCD gets a uniform mix of groups and splits, which balances
    //    groups of very different windows when their K/V cannot stay in L2 anyway.
    // Under xcd_map 1 the second half of an XCD's workgroups take their query blocks in reverse
    // order. An XCD hands its workgroups to its CUs breadth-first, so with two resident per CU
    // its j-th and (j + per_xcd/2)-th workgroups tend to share a CU; a chunk's later query blocks
    // see more keys (its own rows, causally), and the mirror pairs a heavy block with a light
    // one on each CU instead of two equal ones (512-row prefill: 264 -> 250 us per call).
    const int n_items = p.nsplit_grid * p.nqblocks * p.ng;
    const int per_xcd = (n_items + 7) / 8;
    int item = (int)blockIdx.x;
    if (p.xcd_map) {
        const int j = (int)(blockIdx.x / 8u), nqb = p.nqblocks;
        item = (int)(blockIdx.x % 8u) * per_xcd + j;
        // whole rows of nqb items on both halves, so the mirror stays a bijection
        if (2 * j >= per_xcd && per_xcd % (2 * nqb) == 0) item += nqb - 1 - 2 * (item % nqb);
    }
    if (item >= n_items) return;
    const int qb = item % p.nqblocks;
    const int split = (item / p.nqblocks) % p.nsplit_grid;
    const int g = item / (p.nqblocks * p.nsplit_grid);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int qcol = lane & 31, hb = lane >> 5;
#ifdef WINATTN_PHASE_STAMPS
    const unsigned long long ck_real0 = __builtin_amdgcn_s_memrealtime(), ck_clk0 = __builtin_amdgcn_s_memtime();
#endif
    const int nq_tot = p.rows * p.hpg;
    const int q0 = qb * QB;
    const int nq = min(QB, nq_tot - q0);
    const GroupWin gw = resolve_group<GATED>(p, g);

    const int r_first = q0 / p.hpg, r_last = (q0 + nq - 1) / p.hpg;
    const int hi_first = gw.hi0 + r_first;
    const int xlo = window_lo(hi_first, gw.wcap);
    const int xhi = gw.hi0 + r_last;
    const Tiles tr = tile_range<TK>(p.ns, xlo, xhi, p.nsplit_grid, split);
    const int nsplit = tr.nsplit, nst = tr.nst;
    if (split >= nsplit) {
        mark_split_empty<QB>(p, g * p.nqblocks + qb, split);
        return;
    }
    const int t_begin = tr.t_begin, t_end = tr.t_end;
    const int d4 = p.d / 4;

    // This lane's query (column qcol of its wave's 32) and its window in key-index space.
    const int jq = wave * 32 + qcol;
    const bool qvalid = jq < nq;
    const int qi = q0 + (qvalid ? jq : nq - 1);
    const int row = qi / p.hpg, gh = g * p.hpg + qi % p.hpg;
    const int hi = gw.hi0 + row;
    const int lo = window_lo(hi, gw.wcap);

    float4 kreg[LPT], vreg[LPT];
    unsigned kmask = 0u;
    const KVBases kvb = kv_bases(p);
    auto load_tile = [&](int t) {
        kmask = load_tile_regs<TK, D, LPT>(p, kvb, gw, g, xlo, xhi, nst, t, d4, kreg, vreg);
    };

    load_tile(t_begin);   // first tile in flight while the queries load

    // Q^T operand: qreg[4c + r] = scale*log2e * q[8c + 4*hb + r].
    float qreg[D / 2];
    {
        const float* qp = p.q + ((size_t)row * p.nh + gh) * p.d;
#pragma unroll
        for (int c = 0; c < D / 8; ++c) {
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            const int e = 8 * c + 4 * hb;
            if (e < p.d) v = *reinterpret_cast<const float4*>(qp + e);
            qreg[4 * c + 0] = v.x * p.scale_log2;
            qreg[4 * c + 1] = v.y * p.scale_log2;
            qreg[4 * c + 2] = v.z * p.scale_log2;
            qreg[4 * c + 3] = v.w * p.scale_log2;
        }
    }

    floatx16 oacc[NDB];
#pragma unroll
    for (int b = 0; b < NDB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[b][r] = 0.0f;
    float mrun = -INFINITY, lrun = 0.0f;

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

        // This lane's visible keys of the tile as a range [klo, khi) of key indices.
        const int tx = xlo + (t - nst) * TK;   // first stream entry of a stream tile
        const bool sink_tile = t < nst;
        const int klo = sink_tile ? 0 : lo - tx;
        const int khi = sink_tile ? p.ns - t * TK : hi - tx;
        if (!__any(klo < TK && khi > 0 && khi > klo)) continue;   // the whole wave misses it

        // Scores, software-pipelined: the K fragment of step c + 2 is read while step c's
        // products run (scheduling barriers keep the reads from sinking next to their uses).
        constexpr int NC = D / 8, PF = 2;
        floatx16 sacc;
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[r] = 0.0f;
        const float* kr = s_k + qcol * KST + 4 * hb;
        float4 kbuf[PF + 1];
#pragma unroll
        for (int c = 0; c < PF; ++c) kbuf[c] = *reinterpret_cast<const float4*>(kr + 8 * c);
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            if (c + PF < NC)
                kbuf[(c + PF) % (PF + 1)] = *reinterpret_cast<const float4*>(kr + 8 * (c + PF));
            __builtin_amdgcn_sched_barrier(0);
            const float4 k4 = kbuf[c % (PF + 1)];
            sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(k4.x, qreg[4 * c + 0], sacc, 0, 0, 0);
            sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(k4.y, qreg[4 * c + 1], sacc, 0, 0, 0);
            sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(k4.z, qreg[4 * c + 2], sacc, 0, 0, 0);
            sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(k4.w, qreg[4 * c + 3], sacc, 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        // The first V^T operands, read now so their latency hides under the softmax:
        // vbuf[r & 1][b] = V[8 (r / 4) + 4 hb + r % 4][32 b + qcol].
        float vbuf[2][NDB];
#pragma unroll
        for (int b = 0; b < NDB; ++b) vbuf[0][b] = s_v[(4 * hb) * VST + qcol + 32 * b];

        // Mask by select (never multiply: masked slots may hold anything), online softmax.
        float tmax = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int k = 8 * (r >> 2) + 4 * hb + (r & 3);
            sacc[r] = (k >= klo && k < khi) ? sacc[r] : -INFINITY;
            tmax = fmaxf(tmax, sacc[r]);
        }
        tmax = half_swap_max(tmax);
        // The exponentials are taken against a reference max that moves only when a score
        // exceeds it by more than kLazyRescale (so no weight exceeds 2^8): the accumulators are
        // rescaled rarely after the first tile. (m, l, O) stay consistent with it, which is
        // all the merges need.
        const bool grow = tmax > mrun + kLazyRescale;
        if (__any(grow)) {
            const float m_new = grow ? tmax : mrun;
            const float corr = __builtin_amdgcn_exp2f(mrun - safe_max(m_new));
            lrun *= corr;
#pragma unroll
            for (int b = 0; b < NDB; ++b)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[b][r] *= corr;
            mrun = m_new;
        }
        const float mu = safe_max(mrun);
        float psum = 0.0f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            sacc[r] = __builtin_amdgcn_exp2f(sacc[r] - mu);
            psum += sacc[r];
        }
        lrun += half_swap_sum(psum);

#pragma unroll
        for (int r = 0; r < 16; ++r) {
            if (r + 1 < 16) {
                const float* vr = s_v + (8 * ((r + 1) >> 2) + 4 * hb + ((r + 1) & 3)) * VST + qcol;
#pragma unroll
                for (int b = 0; b < NDB; ++b) vbuf[(r + 1) & 1][b] = vr[32 * b];
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int b = 0; b < NDB; ++b)
                oacc[b] = __builtin_amdgcn_mfma_f32_32x32x2f32(vbuf[r & 1][b], sacc[r], oacc[b], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

#ifdef WINATTN_PHASE_STAMPS
    if (g_mfma_clock && tid == 0) {
        asm volatile("" : : "v"(oacc[0][0]), "v"(lrun));
        const unsigned long long real1 = __builtin_amdgcn_s_memrealtime(), clk1 = __builtin_amdgcn_s_memtime();
        unsigned long long* o = g_mfma_clock + (size_t)blockIdx.x * 4;
        o[0] = ck_real0;
        o[1] = ck_clk0;
        o[2] = real1;
        o[3] = clk1;
    }
#endif
    // Lane holds, for its query, d = 32b + 8m + 4*hb + (0..3) in oacc[b][4m .. 4m+3].
    const int blk = g * p.nqblocks + qb;
    if (nsplit == 1 && !p.merge_kernel) {
        if (qvalid) {
            const float inv = 1.0f / fmaxf(lrun, 1e-30f);
#pragma unroll
            for (int b = 0; b < NDB; ++b)
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const int e = 32 * b + 8 * m + 4 * hb;
                    if (e < p.d) {
                        float4 o = make_float4(oacc[b][4 * m] * inv, oacc[b][4 * m + 1] * inv,
                                               oacc[b][4 * m + 2] * inv, oacc[b][4 * m + 3] * inv);
                        store_out<GATED>(p, qi, g, e, o);
                    }
                }
        }
        return;
    }
    if (qvalid) {
        const size_t at = ((size_t)blk * p.slot_stride + split) * QB + jq;
#pragma unroll
        for (int b = 0; b < NDB; ++b)
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int e = 32 * b + 8 * m + 4 * hb;
                store_part4<QB, D>(p, blk, split, jq, e,
                                   make_float4(oacc[b][4 * m], oacc[b][4 * m + 1], oacc[b][4 * m + 2],
                                               oacc[b][4 * m + 3]));
            }
        if (hb == 0) {
            store_part(p, p.pm + at, mrun);
            store_part(p, p.pl + at, lrun);
        }
    }
    merge_if_last<QB, D, GATED>(p, blk, nsplit, q0, nq, g, &s_flag, s_k);
}

template <int D, bool GATED>
static hipError_t launch_mfma_t(const AttnParams& p, hipStream_t stream) {
    const int n_items = p.nsplit_grid * p.nqblocks * p.ng;
    const int blocks = p.xcd_map ? 8 * ((n_items + 7) / 8) : n_items;
    hipLaunchKernelGGL((attn_mfma_kernel<D, GATED>), dim3(blocks), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_mfma(const AttnParams& p, bool gated, int dpad, hipStream_t stream) {
    if (gated) {
        if (dpad == 64) return launch_mfma_t<64, true>(p, stream);
        if (dpad == 128) return launch_mfma_t<128, true>(p, stream);
        if (dpad == 256) return launch_mfma_t<256, true>(p, stream);
    } else {
        if (dpad == 64) return launch_mfma_t<64, false>(p, stream);
        if (dpad == 128) return launch_mfma_t<128, false>(p, stream);
        if (dpad == 256) return launch_mfma_t<256, false>(p, stream);
    }
    return hipErrorInvalidValue;
}

// Layout probe of v_mfma_f32_32x32x2f32: A[i][0] = i, A[i][1] = 1, B[0][j] = 1,
// B[1][j] = 64 j, so D[i][j] = i + 64 j names its own position. out[lane * 16 + r] receives
// accumulator r of lane `lane`.
__global__ __launch_bounds__(64) void mfma_layout_probe_kernel(float* out) {
    const int lane = threadIdx.x;
    const float a = lane < 32 ? (float)lane : 1.0f;
    const float b = lane < 32 ? 1.0f : 64.0f * (float)(lane - 32);
    floatx16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc, 0, 0, 0);
#pragma unroll
    for (int r = 0; r < 16; ++r) out[lane * 16 + r] = acc[r];
}

hipError_t launch_mfma_probe(float* out, hipStream_t stream) {
    hipLaunchKernelGGL(mfma_layout_probe_kernel, dim3(1), dim3(64), 0, stream, out);
    return hipGetLastError();
}

int mfma_query_block() { return kMfmaQB; }
int mfma_tile_keys() { return kMfmaTK; }

}  // namespace winattn

#ifdef WINATTN_PHASE_STAMPS
// Timing builds: where the 32x32 matrix-core kernel records its clock readings (NULL: nowhere);
// 4 u64 per workgroup of the launch, each launch overwrites them.
extern "C" int attn_mfma_clock_set(void* device_ptr) {
    return hipMemcpyToSymbol(HIP_SYMBOL(winattn::g_mfma_clock), &device_ptr, sizeof(device_ptr)) == hipSuccess
               ? 0
               : -3;
}
#endif
