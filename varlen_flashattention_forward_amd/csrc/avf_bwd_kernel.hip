// Backward of packed variable-length attention for gfx950 (MI355X, CDNA4).
//
// Gradients of O = softmax(scale * Q K^T) V for an upstream dO, given the
// forward's LSE (the backward of flash_attn_varlen_func on the "[FA4] cute
// varlen backward: int32 overflow in _bwd_preprocess ..." page). With
// P = exp(scale * S - LSE) recomputed from Q, K and the LSE:
//   D_i  = sum_d dO[i,d] * O[i,d]                   (preprocessing pass)
//   dP   = dO V^T,   dS = P * (dP - D_i)            (softmax Jacobian)
//   dV   = P^T dO,   dK = scale * dS^T Q,   dQ = scale * dS K
// Two tile kernels share no output: the dK/dV kernel owns a block of keys
// and streams the segment's query rows; the dQ kernel owns a block of query
// rows and streams the segment's keys. Every gradient element is written by
// one wave, once, with no atomics, so results are deterministic; the price
// is that S and dP are formed in both kernels.
//
// MFMA: v_mfma_f32_32x32x16_bf16 (wave64). A 32x32 result C[m][n] puts
// column n = lane % 32 in one lane pair and 16 rows m per lane; taken as a
// B operand it contracts over m. So:
//   dK/dV kernel: S = Q K^T and dP = dO V^T with queries as m and the wave's
//     32 keys as n; then dV^T += dO^T P and dK^T += Q^T dS contract over
//     queries, with A = dO^T and Q^T read by transposing LDS reads in the
//     row order of the C layout.
//   dQ kernel:    S^T = K Q^T and dP^T = V dO^T with keys as m and the wave's
//     32 query rows as n; then dQ^T += K^T dS^T contracts over keys, with
//     A = K^T read transposed from LDS.
// Rows streamed through LDS (Q and dO, or K and V) arrive by buffer loads
// that write LDS directly, double-buffered one stage ahead with one barrier
// per stage. Q/dO (and K) rows are read both as 16-byte row fragments and
// transposed, so their 16-byte chunks are permuted by a swizzle that keeps
// both read patterns free of bank conflicts on the 64-bank LDS (dual_swz).
// Offsets: tensor bases in int64 (row * row_stride + head * head_stride),
// the "Suggested kernel-side fix" of the _bwd_preprocess page; per-lane
// offsets inside a tile stay below 2^31 (checked on the host).

#include "avf_bwd_impl.h"

namespace {

template <int D>
hipError_t launch_pre(const AvfPreArgs& a, hipStream_t stream) {
    const int64_t items = a.rows * a.num_heads;
    const int64_t blocks = (items + 15) / 16;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL((avf_bwd_pre_kernel<D>), dim3((uint32_t)blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_dq(const AvfBwdArgs& a, hipStream_t stream) {
    if (a.causal)
        hipLaunchKernelGGL((avf_bwd_dq_kernel<D, kNW, kBK, true>), dim3((uint32_t)a.num_tiles), dim3(kNW * 64), 0,
                           stream, a);
    else
        hipLaunchKernelGGL((avf_bwd_dq_kernel<D, kNW, kBK, false>), dim3((uint32_t)a.num_tiles), dim3(kNW * 64), 0,
                           stream, a);
    return hipGetLastError();
}

}  // namespace

int32_t avf_bwd_block_n(int32_t head_dim) {
    return (head_dim == 64 || head_dim == 96 || head_dim == 128) ? 32 * kNW : -1;
}

int32_t avf_bwd_block_m(int32_t head_dim) {
    return (head_dim == 64 || head_dim == 96 || head_dim == 128) ? 32 * kNW : -1;
}

hipError_t avf_bwd_preprocess_launch(const AvfPreArgs& a, int32_t head_dim, hipStream_t stream) {
    switch (head_dim) {
        case 64: return launch_pre<64>(a, stream);
        case 96: return launch_pre<96>(a, stream);
        case 128: return launch_pre<128>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t avf_bwd_dkdv_launch(const AvfBwdArgs& a, int32_t head_dim, hipStream_t stream) {
    switch (head_dim) {
        case 64:
        case 96: return avf_bwd_dkdv_launch_small(a, head_dim, stream);
        case 128: return launch_dkdv<128, 1>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t avf_bwd_dq_launch(const AvfBwdArgs& a, int32_t head_dim, hipStream_t stream) {
    switch (head_dim) {
        case 64: return launch_dq<64>(a, stream);
        case 96: return launch_dq<96>(a, stream);
        case 128: return launch_dq<128>(a, stream);
        default: return hipErrorInvalidValue;
    }
}
