// Roofline calibration kernel (not part of the attention ABI): the rate a
// plain stream of v_mfma_f32_32x32x16_bf16 instructions reaches on this GPU
// with given operand values. The MI355X dense bf16 figure (2.5 PFLOP/s)
// assumes 4096 flop/clk/CU at 2.4 GHz; under a power limit the clock drops
// with the switching activity of the operands, so the rate for random bf16
// operands is the ceiling an MFMA-bound kernel on random data can approach.
// Built into its own library (libavf_probe.so), used only by the benchmark.

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Each wave loads 4 A and 4 B operand fragments (8 x 1 KiB of `src`, wave
// w at fragments [8w, 8w + 8)) and runs `iters` rounds of 8 MFMAs on 8
// independent accumulators (no chain waits on its own result), alternating
// between two B pairs. The sums are written so the work is not removed.
__global__ void __launch_bounds__(256, 2) avf_probe_mfma_kernel(const bf16x8* __restrict__ src,
                                                                float* __restrict__ out, int32_t iters) {
    const int lane = threadIdx.x & 63;
    const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    bf16x8 a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        a[i] = src[(w * 8 + i) * 64 + lane];
        b[i] = src[(w * 8 + 4 + i) * 64 + lane];
    }
    f32x16 acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[c][e] = 0.f;
    for (int32_t it = 0; it < iters; it += 2) {
#pragma unroll
        for (int c = 0; c < 8; ++c)
            acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[c & 3], b[c >> 2], acc[c], 0, 0, 0);
#pragma unroll
        for (int c = 0; c < 8; ++c)
            acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[c & 3], b[2 + (c >> 2)], acc[c], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int e = 0; e < 16; ++e) s += acc[c][e];
    out[w * 64 + lane] = s;
}

}  // namespace

extern "C" {

// Bytes of bf16 operands (and of fp32 outputs) one launch of `workgroups`
// 256-thread workgroups reads (writes).
int64_t avf_probe_operand_bytes(int32_t workgroups) { return (int64_t)workgroups * 4 * 8 * 1024; }
int64_t avf_probe_output_bytes(int32_t workgroups) { return (int64_t)workgroups * 4 * 64 * 4; }

// Launches the probe: `operands` (device, 16-byte aligned) holds
// avf_probe_operand_bytes(workgroups) bytes of bf16 values, `out` (device)
// avf_probe_output_bytes(workgroups) bytes. iters must be even and > 0.
// The launch performs workgroups * 4 * iters * 8 MFMAs of 32768 flop each.
// Returns 0, -2 for bad arguments, -7 for a launch failure.
int32_t avf_probe_mfma(const void* operands, float* out, int32_t workgroups, int32_t iters, void* stream) {
    if (!operands || !out || workgroups <= 0 || iters <= 0 || (iters & 1) ||
        (reinterpret_cast<uintptr_t>(operands) & 15u))
        return -2;
    hipLaunchKernelGGL(avf_probe_mfma_kernel, dim3((uint32_t)workgroups), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<const bf16x8*>(operands), out, iters);
    return hipGetLastError() == hipSuccess ? 0 : -7;
}

}  // extern "C"
