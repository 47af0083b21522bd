// Host-side launchers of the attention kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>

#include "winattn_dev.h"

namespace winattn {

// Split-K VALU kernel; grid = (splits, query blocks, groups); dpad in {64, 128, 256};
// nq (query vectors per block) in {4, 8, 16}.
hipError_t launch_valu(const AttnParams& p, bool gated, int dpad, int nq, dim3 grid,
                       hipStream_t stream);
int valu_tile_keys(int dpad);

// Register-resident split-K kernel for <= 8 query vectors per block; grid as the VALU kernel;
// nq in {4, 8}.
hipError_t launch_dec(const AttnParams& p, bool gated, int dpad, int nq, dim3 grid,
                      hipStream_t stream);
int dec_tile_keys(int dpad);

struct FarParams;

// Single-launch register kernel for <= 8 query vectors per group (one block per group) that
// streams the ring in slot order; grid = nsplit_grid * ng workgroups; `tiles` ring tiles per
// split; the group's last gather_k splits merge its partials, a column chunk each. With `far`
// (a one-row call's far field, or null) the far part of every head runs in the same launch,
// ahead of the splits, and its partial (slot nsplit_grid) joins the gather; `gated` (with
// `far` only): the gated one-row call (ring slots 0 .. len-1, sinks, the sigmoid gate).
hipError_t launch_decode(const AttnParams& p, const FarParams* far, bool gated, int dpad, int nq,
                         int tiles, hipStream_t stream);
// Ring tiles per split the kernel holds in registers with nq queries per block.
int decode_max_tiles(int dpad, int nq);
// Keys per tile of that kernel.
inline int decode_tile_keys(int dpad) { return 4096 / dpad; }

// Separate launch that merges the split partials of every query block (qb query vectors per
// block); it reads only the partials, never the ring metadata.
hipError_t launch_split_merge(const AttnParams& p, bool gated, int qb, int dpad,
                              hipStream_t stream);

// Split-K MFMA kernel; 1-D grid over (group, split, query block) items, XCD-aware.
hipError_t launch_mfma(const AttnParams& p, bool gated, int dpad, hipStream_t stream);
int mfma_query_block();
int mfma_tile_keys();
hipError_t launch_mfma_probe(float* out, hipStream_t stream);

// Split-K MFMA kernel on 16x16x4 tiles (16 queries per wave) for d = 256 and short chunks;
// same grid and work order as launch_mfma.
hipError_t launch_mfma16(const AttnParams& p, bool gated, int dpad, hipStream_t stream);
int mfma16_query_block();
int mfma16_tile_keys();
hipError_t launch_mfma16_probe(float* out, hipStream_t stream);

struct PrepParams {
    const float* yq;
    const float* yk;
    const float* yv;
    const float* rope;
    const float* q_scale;
    float* qout;      // [rows][nh][hd] unit queries times the learned scale
    float* ring_k;    // [cap][nk][hd]
    float* ring_v;
    int rows, pos0, cap, nh, nk, hd;
    float eps;
};
hipError_t launch_gated_prep(const PrepParams& p, hipStream_t stream);

// The gated call in one launch (attn_gated.hip): head width in (128, 256], a multiple of 32.
struct GatedFusedParams {
    const float* yq;          // [rows][nh][hd] raw query heads
    const float* yk;          // [rows][nk][hd] raw key heads
    const float* yv;          // [rows][nk][hd]
    const float* rope;        // [rows][hd] cos | sin
    const float* q_scale;     // [nh][hd]
    const float* gate;        // [rows][nh * hd]
    const float* gate_scale;  // [nh * hd]
    float* ring_k;            // [cap][nk][hd]
    float* ring_v;
    float* out;               // [rows][nh][hd]
    float* pacc;              // split partials [block][split][QB][256] (nsplit > 1)
    float* pm;                // [block][split][QB]
    float* pl;
    unsigned int* flags;      // ready flags, zero between calls
    int rows, pos0, cap, window, nh, nk, hd, hpg;
    int qb;                   // query vectors per block: 16 (register form) or 64 (tile form)
    int nqs;                  // query blocks per KV head
    int nsplit;               // workgroups per query block, at most 64
    int gather_k;             // tile form: gatherers per block (the block's last splits)
    float scale_log2, eps;
};
hipError_t launch_gated_fused(const GatedFusedParams& p, hipStream_t stream);

hipError_t launch_fill_zero(void* ptr, size_t bytes, hipStream_t stream);

struct CommitParams {
    float* ring_k;          // [ng][w][d]
    float* ring_v;
    uint32_t* meta;         // [ng][4], updated in place
    const float* chunk_k;   // [rows][ng][d]
    const float* chunk_v;
    int rows, ng, d, w;
};
// Ring commit and meta advance after a chunk; one workgroup per group.
hipError_t launch_ring_commit(const CommitParams& p, hipStream_t stream);

struct FarParams {
    const float* ring_k;    // [ng][w][d]
    const float* ring_v;
    const uint32_t* meta;   // [ng][4], as before the chunk
    const float* chunk_k;   // [rows][ng][d]
    const float* chunk_v;
    const float* q;         // [rows][nh][d] (chunk call only)
    const float* k_tilde;   // [ng][m][d] landmark keys (chunk call only)
    const float* q_tilde;   // [nh][m][d] landmark queries
    const float* mu;        // [nh][m][m] mixing matrix (chunk call only)
    float* mz;              // [nh][2m] far maxima then far masses (written by the commit)
    float* t_hat;           // [nh][m][d] far numerators (written by the commit)
    double* ev_e;           // workspace [nh][m][rows]: eviction weights
    double* ev_z;           // workspace [nh][m][rows]: far mass as of each row
    double* ev_mx;          // workspace [nh][m]: far max after the chunk
    double* ev_r;           // workspace [nh][m]: rescale of the old state
    float* pacc;            // the attention's split partials; the far part is slot far_slot
    float* pm;
    float* pl;
    int rows, ng, hpg, nh, d, w, m;
    int qb, nqblocks, slot_stride, far_slot, dpad;
    int rect;               // clamp the landmark weights at zero (gated one-row form)
    float scale;
};
// Far field of a chunk (rows <= 64, m <= 64): eviction scores per (head, landmark), then the
// far partial of every (row, head) into the partial buffer, merged by the merge launch.
hipError_t launch_far_evict(const FarParams& p, hipStream_t stream);
// mode 0: evictions scored by launch_far_evict; 1: a one-row call that scores its own
// eviction; 2: no evictions in the call (the state is current).
hipError_t launch_far_part(const FarParams& p, int mode, hipStream_t stream);
// A one-row far call in one launch with the register kernel: the far part of every head (mode 1
// for the chunk call, 2 for the gated call) and the near splits. hipErrorNotSupported (nothing
// launched) unless the plan is the register kernel with 4 queries per block and splits of at
// most three tiles.
hipError_t launch_dec_far(const AttnParams& p, const FarParams& f, int dpad, int qb, bool gated,
                          int mode, hipStream_t stream);
// Far state after a chunk; runs before the ring commit, which overwrites the evicted rows.
hipError_t launch_far_commit(const FarParams& p, hipStream_t stream);
struct EncParams {
    const float* q;           // row t at t * ldq; head h's hd values at h * hd
    const float* k;           // row t at t * ldk; KV head kvh at kvh * hd
    const float* v;
    float* out;               // row t at t * ldo; head h at h * hd
    const uint32_t* segs;     // [nseg][2]: start, len
    int ldq, ldk, ldv, ldo;
    int nh, nk, group, hd;
    int window;               // 0: the whole sequence, else |i - j| <= window
    int nseg, max_len;        // sequences; the longest length the grid covers
    int max_qblocks;          // query blocks per (sequence, KV head) the grid reserves
    int xcd_map;              // work order: 1 whole (sequence, KV head) runs per XCD, 0 round-robin
    float scale_log2;
};
// Encoder attention over packed sequences on the f32 matrix cores; dpad in {64, 128, 256}.
hipError_t launch_enc_attn(const EncParams& p, int dpad, hipStream_t stream);
int enc_query_block();

// Plain streaming read of `bytes` (a multiple of 16) at `src`; `sink` ([256] floats) is written
// only if the data holds a NaN.
hipError_t launch_read_probe(const void* src, size_t bytes, float* sink, hipStream_t stream);

constexpr int kFarMaxRows = 64;
constexpr int kFarMaxLandmarks = 64;

}  // namespace winattn
