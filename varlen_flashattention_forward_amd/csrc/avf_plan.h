// Launch arguments and the tile map shared by the host planner and the gfx950
// kernel (both sides of the library; nothing here is used by anything else).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

// Segments handled by one launch. The plan of a launch (tile prefix and
// segment starts) travels in the kernel arguments, so no device workspace is
// needed; longer segment lists are split over several launches.
#define AVF_SEGS_PER_LAUNCH 128

// Chiplets (XCDs) of an MI355X. Workgroups are handed to XCDs round-robin in
// dispatch order; the tile map below gives each XCD a contiguous run of tiles
// so the workgroups sharing one XCD's L2 walk the same (segment, head) K/V.
#define AVF_NUM_XCD 8

struct AvfLaunchArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    // element strides (int64: offsets are formed in 64-bit arithmetic)
    int64_t q_row, q_head, k_row, k_head, v_row, v_head, o_row, o_head, lse_head;
    // per-segment base offsets (elements) for batched [W, S, H, D] tensors:
    // segment s (global index seg0 + local s) adds s * *_seg to its base;
    // all zero for packed varlen tensors
    int64_t q_seg, k_seg, v_seg, o_seg, lse_seg;
    int32_t seg0;       // global index of this launch's first segment
    int32_t causal;     // 1: query row r of a segment sees keys j <= r + Lk - Lq
    int32_t one_stage;  // 1: every segment has at most avf_one_stage_keys() keys (checked by
                        // the caller): the one-stage configuration, block_m avf_block_m_one
    int32_t short_stage;  // 1 (one_stage 0): at most avf_short_stage_keys() keys: 64-key
                          // stages, block_m avf_block_m_one
    // Device plan (sync-free entry): the planner's workspace (status, tile
    // count, tile prefix of all num_segs segments) and the caller's device
    // cu_seqlens; NULL for a host-planned launch, which uses the arrays below.
    const int32_t* dev_plan;
    const int32_t* cu_q;
    const int32_t* cu_k;
    // 8-bit score product: packed E4M3 codes of q and k ([tokens, H, D]
    // bytes) and their per-head amax (fp32 bits: H words for q, then H for
    // k); NULL for the bf16 path
    const uint8_t* q8;
    const uint8_t* k8;
    const uint32_t* amax8;
    float scale_log2e;  // softmax_scale * log2(e): logits in base-2 units
    float scale;        // softmax_scale: the LSE is reported in natural-log units
    int32_t num_heads;
    int32_t num_segs;   // segments in this launch (1..AVF_SEGS_PER_LAUNCH)
    int32_t num_tiles;  // == gridDim.x, exact
    // tile_start[s] = num_heads * sum_{s' < s} ceil(Lq_s' / BM); tile_start[num_segs] = num_tiles
    int32_t tile_start[AVF_SEGS_PER_LAUNCH + 1];
    // cu_seqlens entries of this launch's segments, absolute token indices
    int32_t q_start[AVF_SEGS_PER_LAUNCH + 1];
    int32_t k_start[AVF_SEGS_PER_LAUNCH + 1];
};

// Device-plan workspace: AVF_PLAN_HEADER_WORDS int32 words (status, tile
// count, two reserved), then tile_start[0..B] (tile_start[b] = H * sum over
// segments b' < b of ceil(L_b' / block)).
#define AVF_PLAN_HEADER_WORDS 4

struct AvfTile {
    int32_t seg, mblk, head;
};

// Workgroup index -> linear tile index. Linear tiles are ordered (segment,
// head, query block) with the query block fastest. Workgroup w runs on XCD
// w % 8 as its (w / 8)-th workgroup; XCD x owns the contiguous linear range
// [x*q + min(x, r), ...) of length q + (x < r) where T = 8q + r. This is a
// bijection of [0, T) for every T >= 1.
__host__ __device__ inline int32_t avf_linear_tile(int32_t wg, int32_t num_tiles) {
    const int32_t q = num_tiles / AVF_NUM_XCD;
    const int32_t r = num_tiles % AVF_NUM_XCD;
    const int32_t x = wg % AVF_NUM_XCD;
    const int32_t s = wg / AVF_NUM_XCD;
    return x * q + (x < r ? x : r) + s;
}

// Linear tile -> (segment, query block, head). `tile_start` is the launch's
// prefix array; empty segments have tile_start[s] == tile_start[s+1] and are
// never returned (the largest s with tile_start[s] <= L owns L).
template <typename Starts>
__host__ __device__ inline AvfTile avf_decode(int32_t linear, const Starts& tile_start,
                                              const Starts& q_start, int32_t num_segs,
                                              int32_t num_heads, int32_t block_m) {
    int32_t lo = 0, hi = num_segs - 1;
    while (lo < hi) {
        const int32_t mid = (lo + hi + 1) >> 1;
        if (tile_start[mid] <= linear)
            lo = mid;
        else
            hi = mid - 1;
    }
    const int32_t lq = q_start[lo + 1] - q_start[lo];
    const int32_t mtiles = (lq + block_m - 1) / block_m;
    const int32_t r = linear - tile_start[lo];
    AvfTile t;
    t.seg = lo;
    t.head = r / mtiles;
    t.mblk = r - t.head * mtiles;
    (void)num_heads;
    return t;
}

__host__ __device__ inline int64_t avf_elem_offset(int64_t row, int64_t row_stride, int64_t head,
                                                   int64_t head_stride) {
    return row * row_stride + head * head_stride;
}

// Host-side launchers implemented next to the kernels.
hipError_t avf_launch(const AvfLaunchArgs& args, int32_t head_dim, hipStream_t stream);
// Planner: validates cu_seqlens_q/k (B+1 device entries each) against the
// bounds and writes the workspace above for blocks of `block` rows of the
// `tiled` side (0: query rows, 1: key rows). Status: 0, or
// ATTN_VARLEN_ECU / ATTN_VARLEN_EMAXSEQ / ATTN_VARLEN_EUNSUPPORTED.
hipError_t avf_plan_launch(const int32_t* cu_q, const int32_t* cu_k, int32_t num_segs, int32_t num_heads,
                           int32_t block, int32_t tiled, int32_t max_q, int32_t max_k, int64_t q_tokens,
                           int64_t k_tokens, int32_t* workspace, hipStream_t stream);
// Query rows per tile of the general configuration and of the one-stage
// configuration (segments of at most avf_one_stage_keys() keys); -1 for an
// unsupported head_dim.
int32_t avf_block_m(int32_t head_dim);
int32_t avf_block_m_one(int32_t head_dim);
int32_t avf_one_stage_keys();
int32_t avf_short_stage_keys();
