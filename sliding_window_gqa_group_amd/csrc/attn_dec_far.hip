// A one-row call with a far field in one launch: the far part of every head (far_part.h, one
// workgroup per head) and the near split-K register kernel (attn_dec_block.h) share a grid. Two
// forms: the chunk far call's one-row case (the row's own eviction scored in the far part) and
// the gated one-row far call (the far state is current; gated near descriptor and epilogue).
// The far workgroups come first in the grid, so their chain of dependent loads (group state,
// landmark keys, mixing matrix, far numerators) starts with the launch and runs while the near
// workgroups stream the ring; each writes its own partial slot, and the merge launch that follows
// folds them. Used when the register kernel takes the call with four queries per block and
// splits of at most three tiles (the decode shapes); other far calls launch the far part alone.
#include "attn_dec_block.h"
#include "far_part.h"
#include "launch.h"

namespace winattn {
namespace {

template <int D, bool GATED, int MODE>
__global__ __launch_bounds__(kThreads, 2) void attn_dec_far_kernel(const AttnParams p,
                                                                   const FarParams f) {
    const int nfar = f.rows * f.nh;
    const int bid = blockIdx.x;
    if (bid < nfar) {
        far_part_block<D, MODE>(f, bid);
        return;
    }
    const int b = bid - nfar;
    const int split = b % p.nsplit_grid, rest = b / p.nsplit_grid;
    attn_dec_block<D, 4, GATED, true>(p, split, rest % p.nqblocks, rest / p.nqblocks);
}

template <bool GATED, int MODE>
hipError_t launch_dec_far_t(const AttnParams& p, const FarParams& f, int dpad, dim3 grid,
                            hipStream_t stream) {
    const dim3 block(kThreads);
    if (dpad == 64)
        hipLaunchKernelGGL((attn_dec_far_kernel<64, GATED, MODE>), grid, block, 0, stream, p, f);
    else if (dpad == 128)
        hipLaunchKernelGGL((attn_dec_far_kernel<128, GATED, MODE>), grid, block, 0, stream, p, f);
    else if (dpad == 256)
        hipLaunchKernelGGL((attn_dec_far_kernel<256, GATED, MODE>), grid, block, 0, stream, p, f);
    else
        return hipErrorNotSupported;
    return hipGetLastError();
}

}  // namespace

hipError_t launch_dec_far(const AttnParams& p, const FarParams& f, int dpad, int qb, bool gated,
                          int mode, hipStream_t stream) {
    if (qb != 4 || f.rows != 1 || dpad != f.dpad) return hipErrorNotSupported;
    if (gated ? mode != kFarCurrent : mode != kFarFusedOneRow) return hipErrorNotSupported;
    const int tk = 4096 / dpad;   // the register kernel's keys per tile
    if (p.tps + (p.ns + tk - 1) / tk > 3) return hipErrorNotSupported;
    const long long near = (long long)p.nsplit_grid * p.nqblocks * p.ng;
    const long long blocks = (long long)f.rows * f.nh + near;
    if (blocks > 0x7fffffffLL) return hipErrorNotSupported;
    const dim3 grid((unsigned)blocks);
    return gated ? launch_dec_far_t<true, kFarCurrent>(p, f, dpad, grid, stream)
                 : launch_dec_far_t<false, kFarFusedOneRow>(p, f, dpad, grid, stream);
}

}  // namespace winattn
