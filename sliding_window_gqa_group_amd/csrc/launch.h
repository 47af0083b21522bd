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

}  // namespace winattn
