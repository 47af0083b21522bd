// Encoder attention over packed variable-length sequences on the f32 matrix cores.
//
// Defined by the egemma2 page ("EmbeddingGemma 2 encoder", `egemma2_msl.metal`):
// `eg_flash_body` / `eg_flash64` / `eg_flash64s` (flash attention over whole sequences, varlen
// segments [start, len], K/V heads shared by groups of query heads, f32 throughout) and
// `EgAtt` / `eg_softmax` (the symmetric window |i - j| <= window, 0 = the whole sequence).
// Non-causal: position i of a sequence sees positions max(0, i - w) .. min(len, i + w + 1) - 1.
//
// The design is the chunk path's matrix-core kernel without key splits: a workgroup owns 128
// consecutive (position, head) queries of one KV head in one sequence (four waves of 32), and
// streams the union of their windows through LDS in tiles of 32 keys shared by the four waves.
// Scores are S^T = K . Q^T on v_mfma_f32_32x32x2f32, so after the online softmax the score
// registers are exactly the B operand of O^T = V^T . P^T and P never leaves the lane (see
// attn_mfma.hip for the operand layout). Q, K, V and out rows are strided (the page's packed
// q|k|v rows are three offsets into one buffer).
#include "winattn_dev.h"
#include "launch.h"

namespace winattn {

namespace {

constexpr int kEncQB = 128;
constexpr int kEncTK = 32;

// Window of position i: [enc_lo, enc_hi); window 0 is the whole sequence.
__device__ inline int enc_lo(int i, int win) { return win > 0 ? max(0, i - win) : 0; }
__device__ inline int enc_hi(int i, int win, int len) { return win > 0 ? min(len, i + win + 1) : len; }

template <int D>
__global__ __launch_bounds__(kThreads, D == 256 ? 1 : 2) void enc_attn_kernel(const EncParams p) {
    constexpr int TK = kEncTK, QB = kEncQB;
    constexpr int D4 = D / 4, KST = D + 4, VST = D + 8;
    constexpr int LPT = TK * D4 / kThreads;   // float4 loads per thread per tensor per tile
    constexpr int NDB = D / 32;               // 32-wide d blocks of the output
    static_assert(LPT >= 1 && TK * D4 == LPT * kThreads, "tile load must cover the tile");

    __shared__ __align__(16) float s_k[TK * KST];
    __shared__ __align__(16) float s_v[TK * VST];

    // Work item = (sequence, KV head, query block), query block fastest. The hardware deals
    // blocks to the 8 XCDs round-robin. xcd_map 1: whole (sequence, KV head) runs of items go to
    // one XCD, whose L2 then serves their shared K/V stream (even work when the runs are alike);
    // xcd_map 0: item = block, every XCD gets a slice of every run (even work when sequence
    // lengths differ).
    const int n_items = p.nseg * p.nk * p.max_qblocks;
    const int per_xcd = (n_items + 7) / 8;
    const int item = p.xcd_map ? (int)(blockIdx.x % 8u) * per_xcd + (int)(blockIdx.x / 8u)
                               : (int)blockIdx.x;
    if (item >= n_items) return;
    const int qb = item % p.max_qblocks;
    const int kvh = (item / p.max_qblocks) % p.nk;
    const int seq = item / (p.max_qblocks * p.nk);
    const long long start = p.segs[2 * seq];
    const uint32_t len_raw = p.segs[2 * seq + 1];
    const int len = len_raw < (uint32_t)p.max_len ? (int)len_raw : p.max_len;   // rows past max_len: unwritten
    const int group = p.group;
    const int nq_tot = len * group;
    const int q0 = qb * QB;
    if (q0 >= nq_tot) return;
    const int nq = min(QB, nq_tot - q0);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int qcol = lane & 31, hb = lane >> 5;
    const int win = p.window;
    const int r_first = q0 / group, r_last = (q0 + nq - 1) / group;
    const int xlo = enc_lo(r_first, win), xhi = enc_hi(r_last, win, len);
    const int ntiles = (xhi - xlo + TK - 1) / TK;
    const int d4 = p.hd / 4;

    // This lane's query (column qcol of its wave's 32) and its window.
    const int jq = wave * 32 + qcol;
    const bool qvalid = jq < nq;
    const int qi = q0 + (qvalid ? jq : nq - 1);
    const int row = qi / group, h = kvh * group + qi % group;
    const int lo = enc_lo(row, win), hi = enc_hi(row, win, len);

    // Tile loads: thread tid takes float4 column c of keys key0 + j * (kThreads / D4). Keys past
    // the block's range and columns past hd load a valid row and column and are zeroed by select.
    const int key0 = tid / D4, col = tid % D4;
    const int colc = col < d4 ? col : d4 - 1;
    const float* kbase = p.k + start * p.ldk + (long long)kvh * p.hd + 4 * colc;
    const float* vbase = p.v + start * p.ldv + (long long)kvh * p.hd + 4 * colc;
    float4 kreg[LPT], vreg[LPT];
    unsigned kmask = 0u;
    auto load_tile = [&](int t) {
        kmask = 0u;
#pragma unroll
        for (int j = 0; j < LPT; ++j) {
            const int x = xlo + t * TK + key0 + j * (kThreads / D4);
            const bool ok = x < xhi && col < d4;
            const long long xr = x < xhi ? x : xhi - 1;
            kreg[j] = *reinterpret_cast<const float4*>(kbase + xr * p.ldk);
            vreg[j] = *reinterpret_cast<const float4*>(vbase + xr * p.ldv);
            kmask |= (ok ? 1u : 0u) << j;
        }
    };
    // At d = 256 the next tile's registers do not fit beside Q and O: each tile is loaded
    // right before it is stored to LDS instead of one tile ahead.
    constexpr bool PREFETCH = D != 256;
    if (PREFETCH && ntiles > 0) load_tile(0);

    // Q^T operand: qreg[4c + r] = scale*log2e * q[8c + 4*hb + r].
    float qreg[D / 2];
    {
        const float* qp = p.q + (start + row) * p.ldq + (long long)h * p.hd;
#pragma unroll
        for (int c = 0; c < D / 8; ++c) {
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            const int e = 8 * c + 4 * hb;
            if (e < p.hd) v = *reinterpret_cast<const float4*>(qp + e);
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

    for (int t = 0; t < ntiles; ++t) {
        __syncthreads();
        if (!PREFETCH) load_tile(t);
#pragma unroll
        for (int j = 0; j < LPT; ++j) {
            const int key = key0 + j * (kThreads / D4);
            const bool keep = (kmask >> j) & 1u;
            *reinterpret_cast<float4*>(s_k + key * KST + 4 * col) = zero_unless(keep, kreg[j]);
            *reinterpret_cast<float4*>(s_v + key * VST + 4 * col) = zero_unless(keep, vreg[j]);
        }
        __syncthreads();
        if (PREFETCH && t + 1 < ntiles) load_tile(t + 1);

        // This lane's visible keys of the tile as a range [klo, khi) of key indices.
        const int tx = xlo + t * TK;
        const int klo = lo - tx, khi = hi - tx;
        if (!__any(klo < TK && khi > 0)) continue;   // the whole wave misses this tile

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
        float vbuf[2][NDB];
#pragma unroll
        for (int b = 0; b < NDB; ++b) vbuf[0][b] = s_v[(4 * hb) * VST + qcol + 32 * b];

        // Mask by select, online softmax in the log2 domain.
        float tmax = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int k = 8 * (r >> 2) + 4 * hb + (r & 3);
            sacc[r] = (k >= klo && k < khi) ? sacc[r] : -INFINITY;
            tmax = fmaxf(tmax, sacc[r]);
        }
        tmax = half_swap_max(tmax);
        // lazy rescaling against a reference max (kLazyRescale)
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

    // Lane holds, for its query, d = 32b + 8m + 4*hb + (0..3) in oacc[b][4m .. 4m+3].
    if (!qvalid) return;
    const float inv = 1.0f / fmaxf(lrun, 1e-30f);
    float* op = p.out + (start + row) * p.ldo + (long long)h * p.hd;
#pragma unroll
    for (int b = 0; b < NDB; ++b)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int e = 32 * b + 8 * m + 4 * hb;
            if (e < p.hd)
                *reinterpret_cast<float4*>(op + e) =
                    make_float4(oacc[b][4 * m] * inv, oacc[b][4 * m + 1] * inv,
                                oacc[b][4 * m + 2] * inv, oacc[b][4 * m + 3] * inv);
        }
}

template <int D>
hipError_t launch_enc_t(const EncParams& p, hipStream_t stream) {
    const long long n_items = (long long)p.nseg * p.nk * p.max_qblocks;
    const int blocks = (int)(p.xcd_map ? 8 * ((n_items + 7) / 8) : n_items);
    hipLaunchKernelGGL((enc_attn_kernel<D>), dim3(blocks), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

int enc_query_block() { return kEncQB; }

hipError_t launch_enc_attn(const EncParams& p, int dpad, hipStream_t stream) {
    if (dpad == 64) return launch_enc_t<64>(p, stream);
    if (dpad == 128) return launch_enc_t<128>(p, stream);
    return launch_enc_t<256>(p, stream);
}

}  // namespace winattn
