// The C-ABI of winattn.h: argument validation, the launch plan (kernel, query block, key
// splits, workspace layout) and dispatch on the caller's stream. Nothing here allocates or
// synchronises.
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <cmath>
#include <mutex>

#include "launch.h"
#include "winattn.h"

// The kernels read ring metadata as four consecutive u32 per group.
static_assert(sizeof(attn_ring_meta) == 4 * sizeof(uint32_t) && alignof(attn_ring_meta) == alignof(uint32_t),
              "attn_ring_meta must be four packed u32");

namespace winattn {
namespace {

// Tuning knobs (attn_tuning_set); 0 = automatic.
int g_force_kernel = 0;     // 1 register, 2 MFMA 32x32, 3 LDS vector, 4 MFMA 16x16,
                            // 5 single-launch register kernel in slot order,
                            // 6 single-launch gated kernel (gated calls)
int g_tiles_per_split = 0;
int g_target_blocks = 0;
int g_merge_kernel = -1;    // -1 automatic, 0 merge in the last split, 1 separate merge launch
int g_xcd_map = -1;         // -1 automatic, else the matrix-core work order

constexpr int kMfma16MaxQ = 256;
// Split counters sit at the start of every workspace, at the same place for every plan, so
// that a workspace reused by calls of other shapes never finds partial sums where it expects
// counters. Plans with more query blocks than counters run unsplit (they fill the GPU anyway).
constexpr size_t kTicketBytes = 64 * 1024;
constexpr long long kMaxTickets = kTicketBytes / sizeof(unsigned int);

enum Kind { kKindDec = 1, kKindMfma = 2, kKindValu = 3, kKindMfma16 = 4, kKindDecode = 5, kKindGated = 6 };

// The single-launch slot-order kernel's last split gathers at most this many partials (two
// 64-bit masks of splits; its ring tiles per split, held in registers, are bounded by
// decode_max_tiles).
constexpr int kDecodeMaxSplits = 128;
constexpr int kDecodeTargetBlocks = 512;
constexpr int kDecodeMaxGatherers = 128;

struct Plan {
    int kind;
    bool mfma;
    int dpad;
    int qb;             // query vectors per block
    int nqblocks;
    int tk;             // keys per tile
    int tps;            // tiles per split (ring tiles per split for kKindDecode)
    int gather_k;       // gatherers per group (kKindDecode)
    int nsplit;         // splits reserved per block
    int slots;          // partial slots per block: nsplit plus extra (the far field's)
    bool merge_kernel;  // merge splits in a separate launch
    int xcd_map;        // matrix-core work order: 1 whole groups per XCD, 0 round-robin
    size_t off_q, off_pacc, off_pm, off_pl, off_tickets, bytes;
};

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
int cdiv(long long a, long long b) { return (int)((a + b - 1) / b); }

int pad_d(int d) { return d <= 64 ? 64 : (d <= 128 ? 128 : 256); }

// Plan of a plain chunk call on the single-launch slot-order kernel: every query of a group in
// one block, the group's w ring slots cut into splits of `tps` tiles, partials merged by the
// last split. `far`: a one-row chunk call with a far field, whose far partials (one workgroup
// per head, in the same launch) take one more partial slot per group and hpg more ready flags
// per gatherer. False if the shape is not one it takes.
bool decode_plan(int rows, int ng, int hpg, int d, int w, Plan& pl, bool far = false) {
    const long long nq_tot = (long long)rows * hpg;
    if (nq_tot > 8 || (g_force_kernel != 0 && g_force_kernel != kKindDecode && g_force_kernel != kKindGated))
        return false;
    if (far && rows != 1) return false;
    const int nfar = far ? hpg : 0;   // the far part's flags per gatherer
    pl.kind = kKindDecode;
    pl.mfma = false;
    pl.dpad = pad_d(d);
    pl.qb = nq_tot <= 4 ? 4 : 8;
    pl.nqblocks = 1;
    pl.tk = decode_tile_keys(pl.dpad);
    const int rt = cdiv(w, pl.tk);   // ring tiles of a group
    // tiles per split: the workgroups aim for two per CU (measured best for the decode shapes),
    // the far part's workgroups (one per head) included, so that every split, the gatherers
    // last among them, is resident from the start (the 4096-slot decode heads with a far field:
    // 43 splits of 3 tiles per group, 14.8 us; 64 of 2, with 32 workgroups waiting for a CU,
    // 15.5 us)
    const long long room = std::max<long long>(kDecodeTargetBlocks / 2, kDecodeTargetBlocks - (long long)ng * nfar);
    int tiles = cdiv((long long)rt * ng, room);
    // With a far part, splits of at least 64 KiB of ring (K and V): on small rings the far
    // workgroups and the gather of many small partials outweigh the extra parallelism (the gated
    // heads, 4 x 1024 slots of width 256, 8 MB: 1, 2 and 4 tiles of 32 KiB per split 15.9, 13.3
    // and 13.0 us against 14.4 us for the two-launch path)
    if (far) tiles = std::max(tiles, cdiv(64 << 10, (long long)pl.tk * pl.dpad * 8));
    if (g_tiles_per_split > 0) tiles = g_tiles_per_split;
    tiles = std::max(1, std::min(std::min(tiles, rt), decode_max_tiles(pl.dpad, pl.qb)));
    if (cdiv(rt, tiles) + nfar > kDecodeMaxSplits) return false;
    // Gatherers per group: up to 8 column chunks (a power of two dividing the d/4 columns and
    // at most the splits), while the waiting gatherers of all groups stay far below the
    // workgroups the GPU holds at once (they wait only for workgroups dispatched before them).
    const int nsp = cdiv(rt, tiles);
    int gk = 8;
    while (gk > 1 && (gk > nsp || (long long)ng * gk > kDecodeMaxGatherers)) gk /= 2;
    if ((long long)ng * gk > kDecodeMaxGatherers) return false;
    pl.gather_k = gk;
    // one ready flag per (gatherer, split or far head) of every group, in the counter region
    if ((long long)ng * gk * (nsp + nfar) > kMaxTickets) return false;
    pl.tps = tiles;
    pl.nsplit = cdiv(rt, tiles);
    pl.slots = pl.nsplit + (far ? 1 : 0);
    pl.merge_kernel = false;
    pl.xcd_map = 0;
    if (pl.slots == 1) {
        pl.bytes = 0;
        return true;
    }
    size_t off = kTicketBytes;
    const size_t slots = (size_t)ng * pl.slots * pl.qb;
    pl.off_tickets = 0;
    pl.off_q = off;
    pl.off_pacc = off;
    off = align_up(off + slots * pl.dpad * sizeof(float), 256);
    pl.off_pm = off;
    off = align_up(off + slots * sizeof(float), 256);
    pl.off_pl = off;
    off = align_up(off + slots * sizeof(float), 256);
    pl.bytes = off;
    return true;
}

// rows/hpg/d: the call's shape; wcap: the largest window any row can have; qbuf_floats: extra
// workspace for the gated call's prepared queries. `plain`: a plain chunk call (no far field,
// not gated), which the single-launch slot-order kernel may take; `far1`: a one-row call with a
// far field (extra_slots 1; the chunk call or the gated one), which it may take with the far
// part in its launch.
Plan make_plan(int rows, int ng, int hpg, int d, int wcap, int ns, size_t qbuf_floats,
               int extra_slots = 0, bool plain = false, bool far1 = false) {
    Plan pl{};
    if (plain && extra_slots == 0 && qbuf_floats == 0 && decode_plan(rows, ng, hpg, d, wcap, pl))
        return pl;
    pl = Plan{};
    if (far1 && extra_slots == 1 && qbuf_floats == 0 && decode_plan(rows, ng, hpg, d, wcap, pl, true))
        return pl;
    pl = Plan{};
    const long long nq_tot = (long long)rows * hpg;
    pl.dpad = pad_d(d);
    // Matrix cores above 8 query vectors per group. Up to 256 of them, 16x16 tiles in blocks of
    // 64 queries (16 per wave): more, smaller blocks, so the splits that fill the CUs each carry
    // less work (chunks of the decode heads: 4 rows 27 us against 42 us with the LDS vector
    // kernel, 32 rows 38 us against 50 us and 64 rows 62 us against 64 us on 32x32 tiles).
    // Beyond that 32x32 tiles in blocks of 128 (32 queries per wave: 96 rows 87 us against
    // 89 us), except at d = 256, where the 32-wide tiles would not fit in registers.
    pl.kind = nq_tot <= 8 ? kKindDec
                          : ((pl.dpad == 256 || nq_tot <= kMfma16MaxQ) ? kKindMfma16 : kKindMfma);
    if (g_force_kernel >= 1 && g_force_kernel <= 4) pl.kind = g_force_kernel;
    pl.mfma = pl.kind == kKindMfma || pl.kind == kKindMfma16;
    if (pl.kind == kKindMfma) {
        pl.qb = mfma_query_block();
        pl.tk = mfma_tile_keys();
    } else if (pl.kind == kKindMfma16) {
        pl.qb = mfma16_query_block();
        pl.tk = mfma16_tile_keys();
    } else if (pl.kind == kKindDec) {
        pl.qb = nq_tot <= 4 ? 4 : 8;
        pl.tk = dec_tile_keys(pl.dpad);
    } else {
        pl.qb = 16;
        pl.tk = valu_tile_keys(pl.dpad);
    }
    pl.nqblocks = cdiv(nq_tot, pl.qb);
    // A block of qb consecutive (row, head) queries spans at most this many rows.
    const long long span = std::min<long long>(rows, (pl.qb - 1) / hpg + 2);
    // Longest stream range a block can cover (sinks are extra tiles of split 0).
    const long long keys_max = (long long)wcap + span - 1;
    const int max_tiles = cdiv(keys_max, pl.tk);
    const long long blocks = (long long)pl.nqblocks * ng;
    // A matrix-core split should amortise its partial (qb x d floats) over a few tiles.
    const int tps_min = pl.kind == kKindMfma ? 4 : (pl.kind == kKindMfma16 ? 2 : 1);
    // Long windows: bound a split's work so the blocks of unequal groups balance.
    const int tps_cap = pl.mfma ? 128 : 64;
    // The merge is one CU reading every split's partial of a block: keep that under 2 MiB.
    const long long nsplit_cap = std::max<long long>(1, (2LL << 20) / ((long long)pl.qb * pl.dpad * 4));
    int tps;
    if (pl.mfma) {
        // Matrix-core kernels divide each block's real tiles evenly among its splits, so the
        // split count sets the work per workgroup, and the launch is as long as the busiest CU.
        // The splits fill the GPU's 256 CUs once: with one workgroup per CU when there are at
        // most 16 blocks (their workgroups stay short, and a second one per CU would mostly add
        // fixed costs and partials: a 64-row chunk of the decode heads measured 69 us at 13
        // splits against 76 us at 26), else two per CU for the 32x32 kernel (its waves then
        // share each SIMD, which keeps the matrix units busier: the 512-row prefill chunk
        // measured 269 us at 4 splits against 277 us at 8 and 284 us at 12); the 16x16 kernel
        // holds one per CU. Never more than 256 splits, nor fewer than long windows need.
        const long long per_cu = (pl.kind == kKindMfma && blocks > 16) ? 2 : 1;
        const long long slots = g_target_blocks > 0 ? g_target_blocks : 256 * per_cu;
        const long long s_hi = std::max<long long>(1, std::min<long long>(
                                   std::min<long long>(max_tiles / tps_min, nsplit_cap), 256));
        const long long s_lo = std::min<long long>(s_hi, cdiv(max_tiles, tps_cap));
        const long long s_pick = std::max(s_lo, std::min(s_hi, std::max<long long>(1, slots / blocks)));
        tps = cdiv(max_tiles, s_pick);
    } else {
        // Vector kernels: the register kernel runs two workgroups per CU, the LDS one one.
        const int target = g_target_blocks > 0 ? g_target_blocks : (pl.kind == kKindDec ? 512 : 256);
        int s_target = cdiv(target, blocks);
        if (s_target < 1) s_target = 1;
        if (s_target > max_tiles) s_target = max_tiles;
        tps = cdiv(max_tiles, s_target);
        if (tps < tps_min) tps = tps_min;
        if (tps > tps_cap) tps = tps_cap;
        if (cdiv(max_tiles, tps) > nsplit_cap) tps = cdiv(max_tiles, nsplit_cap);
    }
    if (g_tiles_per_split > 0) tps = g_tiles_per_split;
    if (blocks > kMaxTickets) tps = max_tiles;
    pl.tps = tps;
    pl.nsplit = cdiv(max_tiles, tps);
    // Splits merge in a separate launch by default: the kernel boundary makes the partials
    // visible, so the attention kernel stores them plainly, with no acknowledged device-scope
    // stores, counter or acquire, and no block's tail carries a merge (measured faster for the
    // decode, prefill and gated workloads). Merging in the last-arriving split stays available.
    pl.merge_kernel = g_merge_kernel >= 0 ? g_merge_kernel == 1 : true;
    // Whole groups per XCD when a group's K/V stream fits comfortably in an XCD's 4 MB L2
    // (twice that, since neighbouring blocks only touch the part of the window they share).
    const long long group_bytes = ((long long)wcap + span + ns) * d * 8;
    pl.xcd_map = g_xcd_map >= 0 ? g_xcd_map : (group_bytes <= (8LL << 20) ? 1 : 0);

    // Layout: [counters][prepared queries][partials], each region 256-byte aligned.
    pl.slots = pl.nsplit + extra_slots;
    if (extra_slots > 0) pl.merge_kernel = true;   // the extra partials merge in the merge launch
    const bool split = pl.nsplit > 1 || extra_slots > 0;
    if (!split && qbuf_floats == 0) {
        pl.bytes = 0;
        return pl;
    }
    size_t off = 0;
    pl.off_tickets = off;
    off += kTicketBytes;
    pl.off_q = off;
    off = align_up(off + qbuf_floats * sizeof(float), 256);
    if (split) {
        const size_t slots = (size_t)blocks * pl.slots * pl.qb;
        pl.off_pacc = off;
        off = align_up(off + slots * pl.dpad * sizeof(float), 256);
        pl.off_pm = off;
        off = align_up(off + slots * sizeof(float), 256);
        pl.off_pl = off;
        off = align_up(off + slots * sizeof(float), 256);
    }
    pl.bytes = off;
    return pl;
}

// Plan of the gated call in one launch (kernel 6): unit heads of width 160, 192, 224 or 256 and
// at least one full query set (16 query vectors) per KV head. From 64 query vectors per KV head
// on, the tile form (blocks of 64 queries, LDS-staged 32-key tiles, two waves per SIMD);
// below, the register form (sets of 16). Splits per block aim at one workgroup per CU.
struct GatedPlan {
    int qb, nqs, nsplit, gather_k;
    size_t off_pacc, off_pm, off_pl, bytes;
};

constexpr int kGatedTargetBlocks = 256;
constexpr int kGatedMaxSplits = 64;
constexpr int kGatedMaxGatherers = 128;   // waiting gatherers stay far below the CUs

bool gated_fused_plan(int rows, int nh, int nk, int hd, int window, GatedPlan& gp) {
    if (g_force_kernel != 0 && g_force_kernel != kKindGated) return false;
    if (hd <= 128 || hd > 256 || hd % 32 != 0) return false;
    const int hpg = nh / nk;
    const long long nqv = (long long)rows * hpg;
    if (nqv < 16 && g_force_kernel != kKindGated) return false;
    const int qb = nqv >= 64 ? 64 : 16;
    const long long nqs = (nqv + qb - 1) / qb;
    const long long blocks = nqs * nk;
    if (blocks > (1LL << 24)) return false;
    // positions a block can span: its rows' windows, at most window + rows spanned - 1
    const long long span = std::min<long long>(rows, (qb - 1) / hpg + 2);
    const long long nb = ((long long)window + span - 1 + 15) / 16;
    const int target = g_target_blocks > 0 ? g_target_blocks : kGatedTargetBlocks;
    long long ns = (target + blocks - 1) / blocks;
    // every wave of a split should keep at least one 16-key block (the tile form: one tile)
    ns = std::min<long long>(ns, std::max<long long>(1, nb / (qb == 64 ? 2 : 4)));
    ns = std::max<long long>(1, std::min<long long>(ns, kGatedMaxSplits));
    int gk = 1;
    if (qb == 64) {
        gk = 8;
        while (gk > 1 && (gk > ns || blocks * gk > kGatedMaxGatherers)) gk /= 2;
        while (ns > 1 && blocks * gk * ns > kMaxTickets) --ns;
        if (gk > ns) gk = 1;
    } else {
        while (ns > 1 && blocks * ns > kMaxTickets) --ns;
    }
    gp.qb = qb;
    gp.nqs = (int)nqs;
    gp.nsplit = (int)ns;
    gp.gather_k = gk;
    if (ns == 1) {
        gp.off_pacc = gp.off_pm = gp.off_pl = 0;
        gp.bytes = 0;
        return true;
    }
    const size_t items = (size_t)blocks * ns;
    size_t off = kTicketBytes;
    gp.off_pacc = off;
    off = align_up(off + items * qb * 256 * sizeof(float), 256);
    gp.off_pm = off;
    off = align_up(off + items * qb * sizeof(float), 256);
    gp.off_pl = off;
    off = align_up(off + items * qb * sizeof(float), 256);
    gp.bytes = off;
    return true;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// The kernels address rows within one group's ring, sinks or chunk with 32-bit offsets:
// every tensor of a call stays under 2^31 floats (8 GiB).
constexpr long long kMaxFloats = (1LL << 31) - 1;

bool chunk_shape_ok(int rows, int ng, int hpg, int d, int w, int ns) {
    if (rows < 1 || ng < 1 || hpg < 1 || w < 1 || ns < 0) return false;
    if (d < 4 || d > 256 || d % 4 != 0) return false;
    if (rows > (1 << 24) || w > (1 << 28) || ns > (1 << 20)) return false;
    if ((long long)ng * hpg > (1 << 16)) return false;
    const long long nh = (long long)ng * hpg;
    if ((long long)ng * w * d > kMaxFloats || (long long)ng * ns * d > kMaxFloats) return false;
    if ((long long)rows * nh * d > kMaxFloats || (long long)rows * ng * d > kMaxFloats) return false;
    return true;
}

bool gated_shape_ok(int rows, int pos0, int cap, int window, int nh, int nk, int hd) {
    if (rows < 1 || pos0 < 0 || cap < 1 || window < 1 || nh < 1 || nk < 1) return false;
    if (nh % nk != 0 || hd < 8 || hd > 256 || hd % 8 != 0) return false;
    if (rows > (1 << 24) || cap > (1 << 28) || window > (1 << 28) || nh > (1 << 16)) return false;
    if ((long long)pos0 + rows > 0x7ffffff0LL) return false;
    if ((long long)cap < (long long)window + rows - 1) return false;
    if ((long long)cap * nk * hd > kMaxFloats || (long long)rows * nh * hd > kMaxFloats) return false;
    return true;
}

// far1: a one-row far call's far part (far_mode 1 for the chunk call, 2 for the gated call),
// launched here: inside the register kernel's launch when that launch can carry it, else on
// its own before the near kernel.
int launch_attention(const Plan& pl, AttnParams& p, bool gated, char* ws, hipStream_t stream,
                     const FarParams* far1 = nullptr, int far_mode = 1) {
    p.xcd_map = pl.xcd_map;
    p.tps = pl.tps;
    p.nsplit_grid = pl.nsplit;
    p.slot_stride = pl.slots;
    p.nqblocks = pl.nqblocks;
    if (pl.slots > 1) {
        p.pacc = reinterpret_cast<float*>(ws + pl.off_pacc);
        p.pm = reinterpret_cast<float*>(ws + pl.off_pm);
        p.pl = reinterpret_cast<float*>(ws + pl.off_pl);
        p.tickets = reinterpret_cast<unsigned int*>(ws + pl.off_tickets);
    }
    p.merge_kernel = pl.merge_kernel && pl.slots > 1 ? 1 : 0;
    p.gather_k = pl.gather_k;
    hipError_t err = hipSuccess;
    const dim3 grid(pl.nsplit, pl.nqblocks, p.ng);
    if (pl.kind == kKindDecode) {   // merges in its last splits; the far part joins its launch
        if (gated ? (!far1 || far_mode != 2) : (far1 && far_mode != 1)) return WINATTN_ELAUNCH;
        err = launch_decode(p, far1, gated, pl.dpad, pl.qb, pl.tps, stream);
        return err == hipSuccess ? WINATTN_OK : WINATTN_ELAUNCH;
    }
    bool fused = false;
    if (far1) {
        if (pl.kind == kKindDec && p.merge_kernel) {
            err = launch_dec_far(p, *far1, pl.dpad, pl.qb, gated, far_mode, stream);
            if (err == hipSuccess)
                fused = true;
            else if (err != hipErrorNotSupported)
                return WINATTN_ELAUNCH;
        }
        if (!fused && launch_far_part(*far1, far_mode, stream) != hipSuccess) return WINATTN_ELAUNCH;
        err = hipSuccess;
    }
    if (fused)
        ;   // the near splits ran in the far part's launch
    else if (pl.kind == kKindMfma)
        err = launch_mfma(p, gated, pl.dpad, stream);
    else if (pl.kind == kKindMfma16)
        err = launch_mfma16(p, gated, pl.dpad, stream);
    else if (pl.kind == kKindDec)
        err = launch_dec(p, gated, pl.dpad, pl.qb, grid, stream);
    else
        err = launch_valu(p, gated, pl.dpad, pl.qb, grid, stream);
    if (err == hipSuccess && p.merge_kernel)
        err = launch_split_merge(p, gated, pl.qb, pl.dpad, stream);
    return err == hipSuccess ? WINATTN_OK : WINATTN_ELAUNCH;
}

}  // namespace
}  // namespace winattn

using namespace winattn;

extern "C" {

int attn_abi_version(void) { return WINATTN_ABI_VERSION; }

const char* attn_strerror(int code) {
    switch (code) {
        case WINATTN_OK: return "success";
        case WINATTN_EINVAL: return "invalid argument (size, pointer, alignment or constraint)";
        case WINATTN_EWORKSPACE: return "workspace missing or too small";
        case WINATTN_ELAUNCH: return "kernel launch failed";
        case WINATTN_EUNSUPPORTED: return "unsupported configuration";
        default: return "unknown error code";
    }
}

int attn_window_check_meta(const attn_ring_meta* host_meta, int ng, int w) {
    if (!host_meta || ng < 1 || w < 1) return WINATTN_EINVAL;
    for (int g = 0; g < ng; ++g) {
        const uint32_t len = host_meta[g].len, head = host_meta[g].head, ov = host_meta[g].window;
        if (ov > (uint32_t)w) return WINATTN_EINVAL;
        const uint32_t wg = ov != 0u ? ov : (uint32_t)w;
        if (len > wg) return WINATTN_EINVAL;
        if (len > 0 && head >= wg) return WINATTN_EINVAL;
    }
    return WINATTN_OK;
}

int attn_window_commit(float* ring_k, float* ring_v, attn_ring_meta* meta_, const float* chunk_k,
                       const float* chunk_v, int rows, int ng, int d, int w, void* stream) {
    uint32_t* meta = reinterpret_cast<uint32_t*>(meta_);
    if (!chunk_shape_ok(rows, ng, 1, d, w, 0)) return WINATTN_EINVAL;
    if (!ring_k || !ring_v || !meta || !chunk_k || !chunk_v) return WINATTN_EINVAL;
    if (!aligned16(ring_k) || !aligned16(ring_v) || !aligned16(chunk_k) || !aligned16(chunk_v) ||
        ((uintptr_t)meta & 3u) != 0)
        return WINATTN_EINVAL;
    const CommitParams p{ring_k, ring_v, meta, chunk_k, chunk_v, rows, ng, d, w};
    return launch_ring_commit(p, static_cast<hipStream_t>(stream)) == hipSuccess ? WINATTN_OK
                                                                                 : WINATTN_ELAUNCH;
}

size_t attn_window_chunk_workspace(int rows, int ng, int hpg, int d, int w, int ns) {
    if (!chunk_shape_ok(rows, ng, hpg, d, w, ns)) return 0;
    return make_plan(rows, ng, hpg, d, w, ns, 0, 0, true).bytes;
}

}  // extern "C"

namespace winattn {
namespace {

// attn_window_chunk with its workspace given: argument checks, the plan, the launches.
// `ws_cap` = 0 and `ws` = NULL ask only for the checks (the return is the plan's workspace
// bytes as a positive value, or a negative code), so a caller can size its scratch first.
long long chunk_call(const float* ring_k, const float* ring_v, const uint32_t* meta,
                     const float* sink_k, const float* sink_v, const float* q,
                     const float* chunk_k, const float* chunk_v, float* out, int rows, int ng,
                     int hpg, int d, int w, int ns, float scale, void* workspace,
                     size_t workspace_bytes, void* stream, bool check_only) {
    if (!chunk_shape_ok(rows, ng, hpg, d, w, ns) || !std::isfinite(scale)) return WINATTN_EINVAL;
    if (!ring_k || !ring_v || !meta || !q || !chunk_k || !chunk_v || !out) return WINATTN_EINVAL;
    if (ns > 0 && (!sink_k || !sink_v)) return WINATTN_EINVAL;
    if (!aligned16(ring_k) || !aligned16(ring_v) || !aligned16(q) || !aligned16(chunk_k) ||
        !aligned16(chunk_v) || !aligned16(out) || ((uintptr_t)meta & 3u) != 0)
        return WINATTN_EINVAL;
    if (ns > 0 && (!aligned16(sink_k) || !aligned16(sink_v))) return WINATTN_EINVAL;
    const Plan pl = make_plan(rows, ng, hpg, d, w, ns, 0, 0, true);
    if (check_only) return (long long)pl.bytes;
    if (pl.bytes > 0 && (!workspace || workspace_bytes < pl.bytes)) return WINATTN_EWORKSPACE;
    if (pl.bytes > 0 && !aligned16(workspace)) return WINATTN_EINVAL;

    AttnParams p{};
    p.ring_k = ring_k;
    p.ring_v = ring_v;
    p.meta = meta;
    p.sink_k = ns > 0 ? sink_k : nullptr;
    p.sink_v = ns > 0 ? sink_v : nullptr;
    p.q = q;
    p.chunk_k = chunk_k;
    p.chunk_v = chunk_v;
    p.out = out;
    p.ring_gs = (long long)w * d;
    p.ring_ss = d;
    p.chunk_rs = (long long)ng * d;
    p.chunk_gs = d;
    p.rows = rows;
    p.ng = ng;
    p.hpg = hpg;
    p.nh = ng * hpg;
    p.d = d;
    p.w = w;
    p.ns = ns;
    p.scale_log2 = scale * kLog2e;
    return launch_attention(pl, p, false, static_cast<char*>(workspace),
                            static_cast<hipStream_t>(stream));
}

}  // namespace
}  // namespace winattn

extern "C" {

int attn_window_chunk(const float* ring_k, const float* ring_v, const attn_ring_meta* meta_,
                      const float* sink_k, const float* sink_v, const float* q,
                      const float* chunk_k, const float* chunk_v, float* out, int rows, int ng,
                      int hpg, int d, int w, int ns, float scale, void* workspace,
                      size_t workspace_bytes, void* stream) {
    const uint32_t* meta = reinterpret_cast<const uint32_t*>(meta_);
    return (int)chunk_call(ring_k, ring_v, meta, sink_k, sink_v, q, chunk_k, chunk_v, out, rows,
                           ng, hpg, d, w, ns, scale, workspace, workspace_bytes, stream, false);
}

}  // extern "C"

// Scratch of attn_window_chunk_noalloc: split partials and split counters of the calls whose
// caller cannot allocate. Every GPU the library runs on holds its own copy, zero when the code
// object is loaded, for the life of the process. In host code `scratch` is only a handle for
// hipGetSymbolAddress: its device address is looked up once per device and used from then on.
static __device__ __align__(256) unsigned char scratch[WINATTN_NOALLOC_SCRATCH_BYTES];

namespace winattn {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch` per device, once looked up

// The current device's copy of `scratch`. On the first call on a device (that device current):
// hipGetSymbolAddress, then the split counters at its start are cleared by a fill kernel on
// `stream` (they must start at zero; every call leaves them at zero).
int scratch_on_current_device(void** ptr, hipStream_t stream) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return WINATTN_ELAUNCH;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return WINATTN_ELAUNCH;
        if (launch_fill_zero(p, kTicketBytes, stream) != hipSuccess) return WINATTN_ELAUNCH;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return WINATTN_OK;
}

}  // namespace
}  // namespace winattn

extern "C" {

int attn_window_chunk_noalloc(const float* ring_k, const float* ring_v, const attn_ring_meta* meta_,
                              const float* sink_k, const float* sink_v, const float* q,
                              const float* chunk_k, const float* chunk_v, float* out, int rows,
                              int ng, int hpg, int d, int w, int ns, float scale, void* stream) {
    const uint32_t* meta = reinterpret_cast<const uint32_t*>(meta_);
    const long long need = chunk_call(ring_k, ring_v, meta, sink_k, sink_v, q, chunk_k, chunk_v,
                                      out, rows, ng, hpg, d, w, ns, scale, nullptr, 0, stream, true);
    if (need < 0) return (int)need;
    if (need > (long long)WINATTN_NOALLOC_SCRATCH_BYTES) return WINATTN_EWORKSPACE;
    void* ws = nullptr;
    if (need > 0) {
        const int rc = scratch_on_current_device(&ws, static_cast<hipStream_t>(stream));
        if (rc != WINATTN_OK) return rc;
    }
    return (int)chunk_call(ring_k, ring_v, meta, sink_k, sink_v, q, chunk_k, chunk_v, out, rows,
                           ng, hpg, d, w, ns, scale, ws, WINATTN_NOALLOC_SCRATCH_BYTES, stream,
                           false);
}

namespace {

// Far-field workspace: the attention plan with one extra partial slot per query block, then the
// f64 eviction arrays [nh][m][rows] (weights, prefix masses) and [nh][m] (max, rescale).
struct FarPlan {
    Plan pl;
    size_t off_e, off_z, off_mx, off_r, bytes;
};

FarPlan make_far_plan(int rows, int ng, int hpg, int d, int w, int ns, int m) {
    FarPlan f{};
    f.pl = make_plan(rows, ng, hpg, d, w, ns, 0, 1, false, rows == 1);
    const size_t nhm = (size_t)ng * hpg * m;
    size_t off = f.pl.bytes;
    f.off_e = off;
    off = align_up(off + nhm * rows * sizeof(double), 256);
    f.off_z = off;
    off = align_up(off + nhm * rows * sizeof(double), 256);
    f.off_mx = off;
    off = align_up(off + nhm * sizeof(double), 256);
    f.off_r = off;
    off = align_up(off + nhm * sizeof(double), 256);
    f.bytes = off;
    return f;
}

bool far_shape_ok(int rows, int m) { return m >= 1 && m <= kFarMaxLandmarks && rows <= kFarMaxRows; }

}  // namespace

size_t attn_window_chunk_far_workspace(int rows, int ng, int hpg, int d, int w, int ns, int m) {
    if (!chunk_shape_ok(rows, ng, hpg, d, w, ns) || !far_shape_ok(rows, m)) return 0;
    return make_far_plan(rows, ng, hpg, d, w, ns, m).bytes;
}

int attn_window_chunk_far(const float* ring_k, const float* ring_v, const attn_ring_meta* meta_,
                          const float* sink_k, const float* sink_v, const float* q,
                          const float* chunk_k, const float* chunk_v, const float* k_tilde,
                          const float* q_tilde, const float* mu, const float* mz,
                          const float* t_hat, float* out, int rows, int ng, int hpg, int d, int w,
                          int ns, int m, float scale, void* workspace, size_t workspace_bytes,
                          void* stream) {
    const uint32_t* meta = reinterpret_cast<const uint32_t*>(meta_);
    if (!chunk_shape_ok(rows, ng, hpg, d, w, ns) || !std::isfinite(scale)) return WINATTN_EINVAL;
    if (m < 1) return WINATTN_EINVAL;
    if (!far_shape_ok(rows, m)) return WINATTN_EUNSUPPORTED;
    const void* ptrs[] = {ring_k, ring_v, q, chunk_k, chunk_v, k_tilde, q_tilde, mu, mz, t_hat, out};
    for (const void* ptr : ptrs)
        if (!ptr || !aligned16(ptr)) return WINATTN_EINVAL;
    if (!meta || ((uintptr_t)meta & 3u) != 0) return WINATTN_EINVAL;
    if (ns > 0 && (!sink_k || !sink_v || !aligned16(sink_k) || !aligned16(sink_v)))
        return WINATTN_EINVAL;
    if ((long long)ng * hpg * m * d > kMaxFloats) return WINATTN_EINVAL;
    const FarPlan fp = make_far_plan(rows, ng, hpg, d, w, ns, m);
    if (!workspace || workspace_bytes < fp.bytes) return WINATTN_EWORKSPACE;
    if (!aligned16(workspace)) return WINATTN_EINVAL;
    char* ws = static_cast<char*>(workspace);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const Plan& pl = fp.pl;

    FarParams f{};
    f.ring_k = ring_k;
    f.ring_v = ring_v;
    f.meta = meta;
    f.chunk_k = chunk_k;
    f.chunk_v = chunk_v;
    f.q = q;
    f.k_tilde = k_tilde;
    f.q_tilde = q_tilde;
    f.mu = mu;
    f.mz = const_cast<float*>(mz);        // read only on this path
    f.t_hat = const_cast<float*>(t_hat);
    f.ev_e = reinterpret_cast<double*>(ws + fp.off_e);
    f.ev_z = reinterpret_cast<double*>(ws + fp.off_z);
    f.ev_mx = reinterpret_cast<double*>(ws + fp.off_mx);
    f.ev_r = reinterpret_cast<double*>(ws + fp.off_r);
    f.pacc = reinterpret_cast<float*>(ws + pl.off_pacc);
    f.pm = reinterpret_cast<float*>(ws + pl.off_pm);
    f.pl = reinterpret_cast<float*>(ws + pl.off_pl);
    f.rows = rows;
    f.ng = ng;
    f.hpg = hpg;
    f.nh = ng * hpg;
    f.d = d;
    f.w = w;
    f.m = m;
    f.qb = pl.qb;
    f.nqblocks = pl.nqblocks;
    f.slot_stride = pl.slots;
    f.far_slot = pl.nsplit;
    f.dpad = pl.dpad;
    f.scale = scale;
    // A one-row call scores its own eviction inside the far-part kernel, which then rides in
    // the near kernel's launch where it can (launch_attention).
    if (rows > 1) {
        if (launch_far_evict(f, st) != hipSuccess) return WINATTN_ELAUNCH;
        if (launch_far_part(f, 0, st) != hipSuccess) return WINATTN_ELAUNCH;
    }

    AttnParams p{};
    p.ring_k = ring_k;
    p.ring_v = ring_v;
    p.meta = meta;
    p.sink_k = ns > 0 ? sink_k : nullptr;
    p.sink_v = ns > 0 ? sink_v : nullptr;
    p.q = q;
    p.chunk_k = chunk_k;
    p.chunk_v = chunk_v;
    p.out = out;
    p.ring_gs = (long long)w * d;
    p.ring_ss = d;
    p.chunk_rs = (long long)ng * d;
    p.chunk_gs = d;
    p.rows = rows;
    p.ng = ng;
    p.hpg = hpg;
    p.nh = ng * hpg;
    p.d = d;
    p.w = w;
    p.ns = ns;
    p.scale_log2 = scale * kLog2e;
    return launch_attention(pl, p, false, ws, st, rows == 1 ? &f : nullptr);
}

int attn_window_commit_far(float* ring_k, float* ring_v, attn_ring_meta* meta_, const float* chunk_k,
                           const float* chunk_v, const float* q_tilde, float* mz, float* t_hat,
                           int rows, int ng, int hpg, int d, int w, int m, float scale,
                           void* stream) {
    uint32_t* meta = reinterpret_cast<uint32_t*>(meta_);
    if (!chunk_shape_ok(rows, ng, hpg, d, w, 0) || !std::isfinite(scale)) return WINATTN_EINVAL;
    if (m < 1) return WINATTN_EINVAL;
    if (!far_shape_ok(rows, m)) return WINATTN_EUNSUPPORTED;
    const void* ptrs[] = {ring_k, ring_v, chunk_k, chunk_v, q_tilde, mz, t_hat};
    for (const void* ptr : ptrs)
        if (!ptr || !aligned16(ptr)) return WINATTN_EINVAL;
    if (!meta || ((uintptr_t)meta & 3u) != 0) return WINATTN_EINVAL;
    if ((long long)ng * hpg * m * d > kMaxFloats) return WINATTN_EINVAL;
    hipStream_t st = static_cast<hipStream_t>(stream);
    FarParams f{};
    f.ring_k = ring_k;
    f.ring_v = ring_v;
    f.meta = meta;
    f.chunk_k = chunk_k;
    f.chunk_v = chunk_v;
    f.q_tilde = q_tilde;
    f.mz = mz;
    f.t_hat = t_hat;
    f.rows = rows;
    f.ng = ng;
    f.hpg = hpg;
    f.nh = ng * hpg;
    f.d = d;
    f.w = w;
    f.m = m;
    f.scale = scale;
    if (launch_far_commit(f, st) != hipSuccess) return WINATTN_ELAUNCH;
    const CommitParams c{ring_k, ring_v, meta, chunk_k, chunk_v, rows, ng, d, w};
    return launch_ring_commit(c, st) == hipSuccess ? WINATTN_OK : WINATTN_ELAUNCH;
}

size_t attn_window_gated_far_workspace(int nh, int nk, int hd, int w, int ns, int m) {
    if (nh < 1 || nk < 1 || nh % nk != 0 || !chunk_shape_ok(1, nk, nh / nk, hd, w, ns) ||
        !far_shape_ok(1, m))
        return 0;
    return make_plan(1, nk, nh / nk, hd, w, ns, 0, 1, false, true).bytes;
}

int attn_window_gated_far(const float* q, const float* ring_k, const float* ring_v,
                          const attn_ring_meta* meta_, const float* sink_k, const float* sink_v,
                          const float* k_tilde, const float* mu, const float* mz,
                          const float* t_hat, const float* gate, const float* gate_scale,
                          float* out, int nh, int nk, int hd, int w, int ns, int m, float scale,
                          int rect, void* workspace, size_t workspace_bytes, void* stream) {
    const uint32_t* meta = reinterpret_cast<const uint32_t*>(meta_);
    if (nh < 1 || nk < 1 || nh % nk != 0 || !chunk_shape_ok(1, nk, nh / nk, hd, w, ns))
        return WINATTN_EINVAL;
    if (!std::isfinite(scale) || m < 1 || (rect != 0 && rect != 1)) return WINATTN_EINVAL;
    if (!far_shape_ok(1, m)) return WINATTN_EUNSUPPORTED;
    const void* ptrs[] = {q, ring_k, ring_v, k_tilde, mu, mz, t_hat, gate, gate_scale, out};
    for (const void* ptr : ptrs)
        if (!ptr || !aligned16(ptr)) return WINATTN_EINVAL;
    if (!meta || ((uintptr_t)meta & 3u) != 0) return WINATTN_EINVAL;
    if (ns > 0 && (!sink_k || !sink_v || !aligned16(sink_k) || !aligned16(sink_v)))
        return WINATTN_EINVAL;
    if ((long long)nh * m * hd > kMaxFloats) return WINATTN_EINVAL;
    const int hpg = nh / nk;
    const Plan pl = make_plan(1, nk, hpg, hd, w, ns, 0, 1, false, true);
    if (!workspace || workspace_bytes < pl.bytes) return WINATTN_EWORKSPACE;
    if (!aligned16(workspace)) return WINATTN_EINVAL;
    char* ws = static_cast<char*>(workspace);
    hipStream_t st = static_cast<hipStream_t>(stream);

    FarParams f{};
    f.ring_k = ring_k;
    f.ring_v = ring_v;
    f.meta = meta;
    f.q = q;
    f.k_tilde = k_tilde;
    f.mu = mu;
    f.mz = const_cast<float*>(mz);        // read only on this path
    f.t_hat = const_cast<float*>(t_hat);
    f.pacc = reinterpret_cast<float*>(ws + pl.off_pacc);
    f.pm = reinterpret_cast<float*>(ws + pl.off_pm);
    f.pl = reinterpret_cast<float*>(ws + pl.off_pl);
    f.rows = 1;
    f.ng = nk;
    f.hpg = hpg;
    f.nh = nh;
    f.d = hd;
    f.w = w;
    f.m = m;
    f.qb = pl.qb;
    f.nqblocks = pl.nqblocks;
    f.slot_stride = pl.slots;
    f.far_slot = pl.nsplit;
    f.dpad = pl.dpad;
    f.rect = rect;
    f.scale = scale;

    AttnParams p{};
    p.ring_k = ring_k;
    p.ring_v = ring_v;
    p.meta = meta;
    p.sink_k = ns > 0 ? sink_k : nullptr;
    p.sink_v = ns > 0 ? sink_v : nullptr;
    p.q = q;
    p.out = out;
    p.gate = gate;
    p.gate_scale = gate_scale;
    p.ring_gs = (long long)w * hd;
    p.ring_ss = hd;
    p.rows = 1;
    p.ng = nk;
    p.hpg = hpg;
    p.nh = nh;
    p.d = hd;
    p.w = w;
    p.ns = ns;
    p.scale_log2 = scale * kLog2e;
    return launch_attention(pl, p, true, ws, st, &f, 2);
}

int attn_encoder(const float* q, const float* k, const float* v, float* out,
                 const uint32_t* segs, int nseg, int max_len, int ldq, int ldk, int ldv, int ldo,
                 int nh, int nk, int hd, int window, float scale, void* stream) {
    if (nseg < 0 || max_len < 0 || nh < 1 || nk < 1 || nh % nk != 0 || window < 0)
        return WINATTN_EINVAL;
    if (hd < 4 || hd > 256 || hd % 4 != 0 || !std::isfinite(scale)) return WINATTN_EINVAL;
    if (ldq < nh * hd || ldk < nk * hd || ldv < nk * hd || ldo < nh * hd) return WINATTN_EINVAL;
    if (ldq % 4 || ldk % 4 || ldv % 4 || ldo % 4) return WINATTN_EINVAL;
    if (nseg == 0 || max_len == 0) return WINATTN_OK;
    const void* ptrs[] = {q, k, v, out};
    for (const void* ptr : ptrs)
        if (!ptr || !aligned16(ptr)) return WINATTN_EINVAL;
    if (!segs || ((uintptr_t)segs & 3u) != 0) return WINATTN_EINVAL;
    const int group = nh / nk;
    const long long qblocks = ((long long)max_len * group + enc_query_block() - 1) / enc_query_block();
    if ((long long)max_len > (1 << 28) || (long long)nseg * nk * qblocks > (1LL << 30))
        return WINATTN_EINVAL;
    EncParams p{};
    p.q = q;
    p.k = k;
    p.v = v;
    p.out = out;
    p.segs = segs;
    p.ldq = ldq;
    p.ldk = ldk;
    p.ldv = ldv;
    p.ldo = ldo;
    p.nh = nh;
    p.nk = nk;
    p.group = group;
    p.hd = hd;
    p.window = window;
    p.nseg = nseg;
    p.max_len = max_len;
    p.max_qblocks = (int)qblocks;
    // One sequence: its KV heads are alike, so whole heads per XCD; several sequences of
    // unknown (device-side) lengths: round-robin, so no XCD holds all the long ones.
    p.xcd_map = g_xcd_map >= 0 ? (g_xcd_map == 1 ? 1 : 0) : (nseg == 1 ? 1 : 0);
    p.scale_log2 = scale * kLog2e;
    return launch_enc_attn(p, pad_d(hd), static_cast<hipStream_t>(stream)) == hipSuccess
               ? WINATTN_OK
               : WINATTN_ELAUNCH;
}

size_t attn_window_gated_workspace(int rows, int nh, int nk, int hd, int window) {
    if (rows < 1 || nh < 1 || nk < 1 || window < 1 || nh % nk != 0 || hd < 8 || hd > 256 ||
        hd % 8 != 0)
        return 0;
    GatedPlan gp;
    if (gated_fused_plan(rows, nh, nk, hd, window, gp)) return gp.bytes;
    return make_plan(rows, nk, nh / nk, hd, window, 0, (size_t)rows * nh * hd).bytes;
}

int attn_window_gated(const float* yq, const float* yk, const float* yv, const float* rope,
                      const float* q_scale, const float* gate, const float* gate_scale,
                      float* ring_k, float* ring_v, float* out, int rows, int pos0, int cap,
                      int window, int nh, int nk, int hd, float scale, float eps,
                      void* workspace, size_t workspace_bytes, void* stream) {
    if (!gated_shape_ok(rows, pos0, cap, window, nh, nk, hd)) return WINATTN_EINVAL;
    if (!std::isfinite(scale) || !std::isfinite(eps) || eps < 0.0f) return WINATTN_EINVAL;
    const void* ptrs[] = {yq, yk, yv, rope, q_scale, gate, gate_scale, ring_k, ring_v, out};
    for (const void* ptr : ptrs)
        if (!ptr || !aligned16(ptr)) return WINATTN_EINVAL;
    const int hpg = nh / nk;
    hipStream_t st = static_cast<hipStream_t>(stream);
    GatedPlan gp;
    if (gated_fused_plan(rows, nh, nk, hd, window, gp)) {
        if (gp.bytes > 0 && (!workspace || workspace_bytes < gp.bytes)) return WINATTN_EWORKSPACE;
        if (gp.bytes > 0 && !aligned16(workspace)) return WINATTN_EINVAL;
        char* ws = static_cast<char*>(workspace);
        GatedFusedParams f{};
        f.yq = yq;
        f.yk = yk;
        f.yv = yv;
        f.rope = rope;
        f.q_scale = q_scale;
        f.gate = gate;
        f.gate_scale = gate_scale;
        f.ring_k = ring_k;
        f.ring_v = ring_v;
        f.out = out;
        if (gp.nsplit > 1) {
            f.flags = reinterpret_cast<unsigned int*>(ws);
            f.pacc = reinterpret_cast<float*>(ws + gp.off_pacc);
            f.pm = reinterpret_cast<float*>(ws + gp.off_pm);
            f.pl = reinterpret_cast<float*>(ws + gp.off_pl);
        }
        f.rows = rows;
        f.pos0 = pos0;
        f.cap = cap;
        f.window = window;
        f.nh = nh;
        f.nk = nk;
        f.hd = hd;
        f.hpg = hpg;
        f.qb = gp.qb;
        f.nqs = gp.nqs;
        f.nsplit = gp.nsplit;
        f.gather_k = gp.gather_k;
        f.scale_log2 = scale * kLog2e;
        f.eps = eps;
        return launch_gated_fused(f, st) == hipSuccess ? WINATTN_OK : WINATTN_ELAUNCH;
    }
    const Plan pl = make_plan(rows, nk, hpg, hd, window, 0, (size_t)rows * nh * hd);
    if (!workspace || workspace_bytes < pl.bytes) return WINATTN_EWORKSPACE;
    if (!aligned16(workspace)) return WINATTN_EINVAL;
    char* ws = static_cast<char*>(workspace);

    PrepParams pp{};
    pp.yq = yq;
    pp.yk = yk;
    pp.yv = yv;
    pp.rope = rope;
    pp.q_scale = q_scale;
    pp.qout = reinterpret_cast<float*>(ws + pl.off_q);
    pp.ring_k = ring_k;
    pp.ring_v = ring_v;
    pp.rows = rows;
    pp.pos0 = pos0;
    pp.cap = cap;
    pp.nh = nh;
    pp.nk = nk;
    pp.hd = hd;
    pp.eps = eps;
    if (launch_gated_prep(pp, st) != hipSuccess) return WINATTN_ELAUNCH;

    // Positions from p0 on, as a ring descriptor: entry x is position p0 + x at slot
    // (p0 + x) mod cap; row r's window ends at position pos0 + r.
    const long long p0 = std::max<long long>(0, (long long)pos0 + 1 - window);
    AttnParams p{};
    p.ring_k = ring_k;
    p.ring_v = ring_v;
    p.q = pp.qout;
    p.out = out;
    p.gate = gate;
    p.gate_scale = gate_scale;
    p.ring_gs = hd;
    p.ring_ss = (long long)nk * hd;
    p.rows = rows;
    p.ng = nk;
    p.hpg = hpg;
    p.nh = nh;
    p.d = hd;
    p.w = window;
    p.ns = 0;
    p.scale_log2 = scale * kLog2e;
    p.g_base = (int)(p0 % cap);
    p.g_mod = cap;
    p.g_hi0 = (int)((long long)pos0 + 1 - p0);
    p.g_wcap = window;
    return launch_attention(pl, p, true, ws, st);
}

int attn_workspace_init(void* workspace, size_t bytes, void* stream) {
    if (bytes == 0) return WINATTN_OK;
    if (!workspace || !aligned16(workspace)) return WINATTN_EINVAL;
    return launch_fill_zero(workspace, bytes, static_cast<hipStream_t>(stream)) == hipSuccess
               ? WINATTN_OK
               : WINATTN_ELAUNCH;
}

int attn_window_chunk_plan(int rows, int ng, int hpg, int d, int w, int ns, int* kernel,
                           int* query_block, int* splits, int* keys_per_split) {
    if (!chunk_shape_ok(rows, ng, hpg, d, w, ns)) return WINATTN_EINVAL;
    const Plan pl = make_plan(rows, ng, hpg, d, w, ns, 0, 0, true);
    if (kernel) *kernel = pl.kind;
    if (query_block) *query_block = pl.qb;
    if (splits) *splits = pl.nsplit;
    if (keys_per_split) *keys_per_split = pl.tps * pl.tk;
    return WINATTN_OK;
}

int attn_mfma_layout_probe(float* out, void* stream) {
    if (!out) return WINATTN_EINVAL;
    return launch_mfma_probe(out, static_cast<hipStream_t>(stream)) == hipSuccess ? WINATTN_OK
                                                                                  : WINATTN_ELAUNCH;
}

int attn_mfma16_layout_probe(float* out, void* stream) {
    if (!out) return WINATTN_EINVAL;
    return launch_mfma16_probe(out, static_cast<hipStream_t>(stream)) == hipSuccess
               ? WINATTN_OK
               : WINATTN_ELAUNCH;
}

int attn_read_probe(const void* src, size_t bytes, float* sink, void* stream) {
    if (!src || !sink || !aligned16(src) || bytes < 16 || bytes % 16 != 0) return WINATTN_EINVAL;
    return launch_read_probe(src, bytes, sink, static_cast<hipStream_t>(stream)) == hipSuccess
               ? WINATTN_OK
               : WINATTN_ELAUNCH;
}

int attn_tuning_set(int knob, int value) {
    if (value < 0) return WINATTN_EINVAL;
    switch (knob) {
        case WINATTN_TUNE_FORCE_KERNEL:
            if (value > 6) return WINATTN_EINVAL;
            g_force_kernel = value;
            return WINATTN_OK;
        case WINATTN_TUNE_TILES_PER_SPLIT:
            g_tiles_per_split = value;
            return WINATTN_OK;
        case WINATTN_TUNE_TARGET_BLOCKS:
            g_target_blocks = value;
            return WINATTN_OK;
        case WINATTN_TUNE_MERGE_KERNEL:
            if (value > 2) return WINATTN_EINVAL;
            g_merge_kernel = value - 1;
            return WINATTN_OK;
        case WINATTN_TUNE_XCD_MAP:
            if (value > 2) return WINATTN_EINVAL;
            g_xcd_map = value - 1;
            return WINATTN_OK;
        default:
            return WINATTN_EINVAL;
    }
}

}  // extern "C"
