// Split-K windowed attention for decode-sized chunks: the register kernel (its workgroup body
// is attn_dec_block.h), the separate split-merge launch and their launchers.
#include "attn_dec_block.h"
#include "launch.h"

namespace winattn {

// SHORT: every split of the launch has at most three tiles (the host picks it when the tiles per
// split plus the sink tiles are at most 3), run as straight-line code; otherwise a loop with two
// register buffers. Two instances rather than one with both paths: together they would not fit
// the register budget of two workgroups per CU.
template <int D, int NQ, bool GATED, bool SHORT>
__global__ __launch_bounds__(kThreads, 2) void attn_dec_kernel(const AttnParams p) {
    attn_dec_block<D, NQ, GATED, SHORT>(p, blockIdx.x, blockIdx.y, blockIdx.z);
}

// Separate merge launch: one workgroup per (query block, group, column chunk), so that the
// partials are read by many CUs at once rather than by one per block. The chunk is 32 columns
// (128 contiguous bytes of a partial row), except for 64-query blocks, where 16 columns give
// every thread exactly one (query, column) item (measured faster; for 128-query blocks the
// shorter 32-byte runs cost more than the extra workgroups gain).
template <int QB>
constexpr int merge_cols() { return QB == 64 ? 16 : 32; }

template <int QB, int D, bool GATED>
__global__ __launch_bounds__(kThreads) void split_merge_kernel(const AttnParams p) {
    __shared__ __align__(16) float scratch[kMergeScratch];
    const int qb = blockIdx.x, g = blockIdx.y;
    const int q0 = qb * QB;
    const int nq = min(QB, p.rows * p.hpg - q0);
    // Every slot of the block holds a partial or an empty mark (see mark_split_empty): the
    // splits, and the far field's partial when the call has one.
    constexpr int MC = merge_cols<QB>();
    merge_block<QB, D, GATED, MC>(p, g * p.nqblocks + qb, p.slot_stride, q0, nq, g, scratch,
                                  (int)blockIdx.z * (MC / 4));
}

template <int D, int NQ, bool GATED>
static hipError_t launch_dec_t(const AttnParams& p, dim3 grid, hipStream_t stream) {
    constexpr int TK = DecShape<D, NQ>::TK;
    const bool short_splits = p.tps + (p.ns + TK - 1) / TK <= 3;
    if (short_splits)
        hipLaunchKernelGGL((attn_dec_kernel<D, NQ, GATED, true>), grid, dim3(kThreads), 0, stream, p);
    else
        hipLaunchKernelGGL((attn_dec_kernel<D, NQ, GATED, false>), grid, dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

template <bool GATED>
static hipError_t launch_dec_g(const AttnParams& p, int dpad, int nq, dim3 grid, hipStream_t s) {
    if (dpad == 64 && nq == 4) return launch_dec_t<64, 4, GATED>(p, grid, s);
    if (dpad == 64 && nq == 8) return launch_dec_t<64, 8, GATED>(p, grid, s);
    if (dpad == 128 && nq == 4) return launch_dec_t<128, 4, GATED>(p, grid, s);
    if (dpad == 128 && nq == 8) return launch_dec_t<128, 8, GATED>(p, grid, s);
    if (dpad == 256 && nq == 4) return launch_dec_t<256, 4, GATED>(p, grid, s);
    if (dpad == 256 && nq == 8) return launch_dec_t<256, 8, GATED>(p, grid, s);
    return hipErrorInvalidValue;
}

template <bool GATED>
static hipError_t launch_merge_g(const AttnParams& p, int qb, int dpad, hipStream_t s) {
#define WINATTN_MERGE_CASE(QQ, DD)                                                               \
    if (qb == QQ && dpad == DD) {                                                                \
        const dim3 grid(p.nqblocks, p.ng, DD / merge_cols<QQ>());                                \
        hipLaunchKernelGGL((split_merge_kernel<QQ, DD, GATED>), grid, dim3(kThreads), 0, s, p);  \
        return hipGetLastError();                                                                \
    }
    WINATTN_MERGE_CASE(4, 64) WINATTN_MERGE_CASE(4, 128) WINATTN_MERGE_CASE(4, 256)
    WINATTN_MERGE_CASE(8, 64) WINATTN_MERGE_CASE(8, 128) WINATTN_MERGE_CASE(8, 256)
    WINATTN_MERGE_CASE(16, 64) WINATTN_MERGE_CASE(16, 128) WINATTN_MERGE_CASE(16, 256)
    WINATTN_MERGE_CASE(64, 64) WINATTN_MERGE_CASE(64, 128) WINATTN_MERGE_CASE(64, 256)
    WINATTN_MERGE_CASE(128, 64) WINATTN_MERGE_CASE(128, 128) WINATTN_MERGE_CASE(128, 256)
#undef WINATTN_MERGE_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_split_merge(const AttnParams& p, bool gated, int qb, int dpad,
                              hipStream_t stream) {
    return gated ? launch_merge_g<true>(p, qb, dpad, stream)
                 : launch_merge_g<false>(p, qb, dpad, stream);
}

hipError_t launch_dec(const AttnParams& p, bool gated, int dpad, int nq, dim3 grid,
                      hipStream_t stream) {
    return gated ? launch_dec_g<true>(p, dpad, nq, grid, stream)
                 : launch_dec_g<false>(p, dpad, nq, grid, stream);
}

int dec_tile_keys(int dpad) { return 4096 / dpad; }

}  // namespace winattn
