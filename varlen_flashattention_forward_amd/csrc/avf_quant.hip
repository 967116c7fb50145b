// Per-head E4M3 quantization of Q and K for the low-precision forward.
//
// For a bf16 tensor X [rows, H, D] (any row/head strides, contiguous D):
//   amax[h] = max |X[i, h, d]| over rows [0, rows) and d     (kernel 1, 2)
//   inv[h]  = 448 / amax[h] (fp32 division; 0 for an all-zero head)
//   code    = E4M3(X[i, h, d] * inv[h])  (fp32 product, hardware conversion:
//             round to nearest even, OCP E4M3FN)             (kernel 3)
// written as a packed [rows, H, D] byte tensor. The attention kernel
// dequantizes the products of codes with amax_q/448 * amax_k/448.
// This is the CDNA4 counterpart of the ffpa-attn page's quantized NVFP4
// forward ("ffpa-attn PR #387"): 8-bit operands for the score product, with
// every size and offset in 64-bit arithmetic (that page's fix: int64
// extents for anything that scales with the sequence length).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "avf_device.h"
#include "avf_quant.h"

namespace {

using namespace avf;

// kernel 1: clear the 2*H amax words (a kernel, not a memset, so a captured
// graph holds only kernels)
__global__ void avf_amax_clear(uint32_t* amax, int32_t n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) amax[i] = 0u;
}

// kernel 2: one workgroup per (chunk of kAmaxChunk rows, head). D/8 lanes
// per row, 16 bytes each; the workgroup's max by shuffles within each wave
// and LDS across waves, then ONE atomic max per workgroup on the float's bit
// pattern (non-negative floats order like their bits). All workgroups of a
// head update one word, so the atomics are kept few.
constexpr int kAmaxChunk = 1024;

template <int D>
__global__ void __launch_bounds__(256) avf_amax_kernel(const void* x, int64_t rows, int64_t row_stride,
                                                       int64_t head_stride, uint32_t* amax) {
    constexpr int LPR = D / 8;            // lanes per row
    constexpr int RPP = 256 / LPR;        // rows per pass
    __shared__ float wmax[4];
    const int64_t h = blockIdx.y;
    const int64_t r0 = (int64_t)blockIdx.x * kAmaxChunk;
    const int tid = threadIdx.x;
    const int c = tid % LPR;
    float m = 0.f;
    for (int p = tid / LPR; p < kAmaxChunk; p += RPP) {
        const int64_t r = r0 + p;
        if (r < rows) {
            const bf16x8 v = *reinterpret_cast<const bf16x8*>((const char*)x + 2 * (r * row_stride + h * head_stride) +
                                                             16 * c);
#pragma unroll
            for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf((float)v[e]));
        }
    }
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) m = fmaxf(m, __shfl_xor(m, s));
    if ((tid & 63) == 0) wmax[tid >> 6] = m;
    __syncthreads();
    if (tid == 0) {
        m = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
        atomicMax(amax + h, __float_as_uint(m));
    }
}

// kernel 3: codes. One thread per 8 elements (16 input bytes -> 8 codes).
template <int D>
__global__ void __launch_bounds__(256) avf_quant_kernel(const void* x, int64_t rows, int32_t H, int64_t row_stride,
                                                        int64_t head_stride, const uint32_t* amax, uint8_t* codes) {
    constexpr int LPR = D / 8;
    const int64_t item = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (row, head, chunk)
    const int64_t total = rows * H * LPR;
    if (item >= total) return;
    const int c = (int)(item % LPR);
    const int64_t rh = item / LPR;
    const int64_t h = rh % H;
    const int64_t r = rh / H;
    const float a = __uint_as_float(amax[h]);
    const float inv = a > 0.f ? 448.0f / a : 0.f;
    const bf16x8 v = *reinterpret_cast<const bf16x8*>((const char*)x + 2 * (r * row_stride + h * head_stride) + 16 * c);
    uint32_t w[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        int p = 0;
        p = __builtin_amdgcn_cvt_pk_fp8_f32((float)v[4 * i] * inv, (float)v[4 * i + 1] * inv, p, false);
        p = __builtin_amdgcn_cvt_pk_fp8_f32((float)v[4 * i + 2] * inv, (float)v[4 * i + 3] * inv, p, true);
        w[i] = (uint32_t)p;
    }
    *reinterpret_cast<uint2*>(codes + (r * H + h) * D + 8 * c) = make_uint2(w[0], w[1]);
}

template <int D>
hipError_t quantize(const void* x, int64_t rows, int32_t H, int64_t row_stride, int64_t head_stride, uint32_t* amax,
                    uint8_t* codes, hipStream_t s) {
    if (rows <= 0) return hipSuccess;
    // amax in row chunks of 2^24 rows per launch
    constexpr int64_t kAmaxRows = (int64_t)1 << 24;
    for (int64_t r0 = 0; r0 < rows; r0 += kAmaxRows) {
        const int64_t n = std::min(kAmaxRows, rows - r0);
        hipLaunchKernelGGL((avf_amax_kernel<D>), dim3((uint32_t)((n + kAmaxChunk - 1) / kAmaxChunk), (uint32_t)H),
                           dim3(256), 0, s,
                           (const char*)x + 2 * r0 * row_stride, n, row_stride, head_stride, amax);
    }
    // codes in row chunks of at most 2^30 threads per launch
    const int64_t per = std::max<int64_t>(1, ((int64_t)1 << 30) / ((int64_t)H * (D / 8)));
    for (int64_t r0 = 0; r0 < rows; r0 += per) {
        const int64_t n = std::min(per, rows - r0);
        const int64_t items = n * H * (D / 8);
        hipLaunchKernelGGL((avf_quant_kernel<D>), dim3((uint32_t)((items + 255) / 256)), dim3(256), 0, s,
                           (const char*)x + 2 * r0 * row_stride, n, H, row_stride, head_stride, amax,
                           codes + r0 * H * D);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t avf_fp8_quantize(const AvfQuantArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(avf_amax_clear, dim3((2 * a.num_heads + 255) / 256), dim3(256), 0, s, a.amax, 2 * a.num_heads);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    switch (a.head_dim) {
        case 64:
            e = quantize<64>(a.q, a.q_rows, a.num_heads, a.q_row, a.q_head, a.amax, a.q8, s);
            return e != hipSuccess ? e : quantize<64>(a.k, a.k_rows, a.num_heads, a.k_row, a.k_head, a.amax + a.num_heads, a.k8, s);
        case 128:
            e = quantize<128>(a.q, a.q_rows, a.num_heads, a.q_row, a.q_head, a.amax, a.q8, s);
            return e != hipSuccess ? e : quantize<128>(a.k, a.k_rows, a.num_heads, a.k_row, a.k_head, a.amax + a.num_heads, a.k8, s);
        default:
            return hipErrorInvalidValue;
    }
}
