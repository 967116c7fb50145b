// Device-side tile planner for the sync-free entry points: validates the
// caller's device cu_seqlens and writes the tile prefix the attention kernel
// decodes from, so no cu value ever travels to the host.
//
// The SM120 issue page ("Interpretation") shows what a host-sized grid over
// device cu_seqlens must not do: launch a bound on the tile count and let
// the surplus workgroups decode garbage coordinates. Here the grid is such a
// bound too, but every workgroup reads the planner's status and tile count
// first and forms no address for a tile at or past that count.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/attn_varlen.h"
#include "avf_plan.h"

namespace {

constexpr int kPlanThreads = 1024;

// One workgroup. Segments are taken in chunks of kPlanThreads, one per
// thread; an exclusive scan of the per-segment tile counts (Hillis-Steele in
// LDS, 64-bit) plus the running total of earlier chunks gives tile_start.
__global__ void __launch_bounds__(kPlanThreads) avf_plan_kernel(const int32_t* cu_q, const int32_t* cu_k, int32_t B,
                                                                int32_t H, int32_t block, int32_t tiled,
                                                                int32_t max_q, int32_t max_k, int64_t q_tokens,
                                                                int64_t k_tokens, int32_t* ws) {
    __shared__ int64_t scan[kPlanThreads];
    __shared__ int32_t bad;  // bit 0: cu order/extent, bit 1: over max_seqlen
    const int tid = threadIdx.x;
    if (tid == 0) bad = (cu_q[0] != 0 || cu_k[0] != 0) ? 1 : 0;
    __syncthreads();
    int64_t carry = 0;
    int32_t mine = 0;
    for (int64_t c0 = 0; c0 < B; c0 += kPlanThreads) {
        const int64_t b = c0 + tid;
        int64_t n = 0;
        if (b < B) {
            const int64_t lq = (int64_t)cu_q[b + 1] - cu_q[b];
            const int64_t lk = (int64_t)cu_k[b + 1] - cu_k[b];
            if (lq < 0 || lk < 0)
                mine |= 1;
            else if (lq > max_q || lk > max_k)
                mine |= 2;
            else
                n = ((tiled ? lk : lq) + block - 1) / block;
        }
        scan[tid] = n;
        __syncthreads();
        for (int off = 1; off < kPlanThreads; off <<= 1) {
            const int64_t add = tid >= off ? scan[tid - off] : 0;
            __syncthreads();
            scan[tid] += add;
            __syncthreads();
        }
        if (b < B) {
            const int64_t start = (carry + scan[tid] - n) * H;
            ws[AVF_PLAN_HEADER_WORDS + b] = (int32_t)(start < INT32_MAX ? start : INT32_MAX);
        }
        carry += scan[kPlanThreads - 1];
        __syncthreads();
    }
    if (mine) atomicOr(&bad, mine);
    __syncthreads();
    if (tid == 0) {
        if ((int64_t)cu_q[B] > q_tokens || (int64_t)cu_k[B] > k_tokens) bad |= 1;
        const int64_t total = carry * H;
        int32_t status = 0;
        if (bad & 1)
            status = ATTN_VARLEN_ECU;
        else if (bad & 2)
            status = ATTN_VARLEN_EMAXSEQ;
        else if (total > INT32_MAX)
            status = ATTN_VARLEN_EUNSUPPORTED;
        ws[AVF_PLAN_HEADER_WORDS + B] = (int32_t)(total < INT32_MAX ? total : INT32_MAX);
        ws[1] = status ? 0 : (int32_t)total;
        ws[2] = 0;
        ws[3] = 0;
        ws[0] = status;
    }
}

}  // namespace

hipError_t avf_plan_launch(const int32_t* cu_q, const int32_t* cu_k, int32_t num_segs, int32_t num_heads,
                           int32_t block, int32_t tiled, int32_t max_q, int32_t max_k, int64_t q_tokens,
                           int64_t k_tokens, int32_t* workspace, hipStream_t stream) {
    hipLaunchKernelGGL(avf_plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, cu_q, cu_k, num_segs, num_heads,
                       block, tiled, max_q, max_k, q_tokens, k_tokens, workspace);
    return hipGetLastError();
}
