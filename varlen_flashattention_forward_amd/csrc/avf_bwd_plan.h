// Launch arguments of the backward kernels, shared by the host planner and
// the gfx950 kernels (both sides of the library; nothing else uses them).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "avf_plan.h"

// Per-row reduction D[h, i] = sum_d out[i, h, d] * dout[i, h, d] over the
// rows [0, rows) and all heads.
struct AvfPreArgs {
    const void* o;
    const void* dout;
    float* delta;
    int64_t o_row, o_head, do_row, do_head, delta_head;  // element strides
    int64_t rows;
    int32_t num_heads;
};

// dK/dV (tiles of 32 * NW keys, streaming the segment's query rows) and dQ
// (tiles of query rows, streaming the segment's keys). One argument block
// serves both; `tile_start` counts the tiles of the kernel it is passed to.
struct AvfBwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* dout;
    const float* lse;    // natural-log LSE of the forward, [H, >= total_q]
    const float* delta;  // D of the preprocessing pass, [H, >= total_q]
    void* dq;
    void* dk;
    void* dv;
    // element strides (int64: offsets are formed in 64-bit arithmetic)
    int64_t q_row, q_head, k_row, k_head, v_row, v_head, do_row, do_head;
    int64_t dq_row, dq_head, dk_row, dk_head, dv_row, dv_head;
    int64_t lse_head, delta_head;
    float scale;        // softmax_scale
    float scale_log2e;  // softmax_scale * log2(e)
    int32_t causal;     // 1: query row r of a segment sees keys j <= r + Lk - Lq
    int32_t num_heads;
    int32_t num_segs;   // segments in this launch (1..AVF_SEGS_PER_LAUNCH)
    int32_t num_tiles;  // == gridDim.x, exact
    int32_t tile_start[AVF_SEGS_PER_LAUNCH + 1];
    int32_t q_start[AVF_SEGS_PER_LAUNCH + 1];  // absolute cu_seqlens_q entries
    int32_t k_start[AVF_SEGS_PER_LAUNCH + 1];  // absolute cu_seqlens_k entries
};

// Host-side launchers implemented next to the kernels. Block sizes: keys per
// dK/dV tile and query rows per dQ tile (-1 for an unsupported head_dim).
hipError_t avf_bwd_preprocess_launch(const AvfPreArgs& args, int32_t head_dim, hipStream_t stream);
hipError_t avf_bwd_dkdv_launch(const AvfBwdArgs& args, int32_t head_dim, hipStream_t stream);
// head_dim 64 and 96 (a separate compilation unit; called by avf_bwd_dkdv_launch)
hipError_t avf_bwd_dkdv_launch_small(const AvfBwdArgs& args, int32_t head_dim, hipStream_t stream);
hipError_t avf_bwd_dq_launch(const AvfBwdArgs& args, int32_t head_dim, hipStream_t stream);
int32_t avf_bwd_block_n(int32_t head_dim);
int32_t avf_bwd_block_m(int32_t head_dim);
