// Roofline calibration kernel (not part of the attention ABI): the rate a
// plain stream of v_mfma_f32_32x32x16_bf16 instructions reaches on this GPU
// with given operand values. The MI355X dense bf16 figure (2.5 PFLOP/s)
// assumes 4096 flop/clk/CU at 2.4 GHz; under a power limit the clock drops
// with the switching activity of the operands, so the rate for random bf16
// operands is the ceiling an MFMA-bound kernel on random data can approach.
// A second kernel measures what VALU instructions next to the MFMAs cost
// the MFMA pipe (avf_probe_coissue). Built into its own library
// (libavf_probe.so), used only by the benchmark.

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

// Co-issue probe: each wave runs `iters` rounds of 8 slots; a slot is one
// v_mfma_f32_32x32x16_bf16 on zero operands (little switching, so the power
// limit hardly moves the clock) followed by NEXP v_exp_f32 and NFMA
// v_fma_f32 on registers the MFMAs do not touch, with a scheduling fence
// between slots. The time per slot against the MFMA-only variant is what the
// VALU instructions cost the MFMA pipe.
template <int NFMA, int NEXP>
__global__ void __launch_bounds__(256) avf_probe_coissue_kernel(float* __restrict__ out, int32_t iters) {
    bf16x8 a;
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = (__bf16)0.0f;
    f32x16 acc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[c][e] = 0.f;
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = 1e-3f * (float)(threadIdx.x + i);
    for (int32_t it = 0; it < iters; ++it) {
#pragma unroll
        for (int sl = 0; sl < 8; ++sl) {
            acc[sl & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, acc[sl & 3], 0, 0, 0);
#pragma unroll
            for (int i = 0; i < NEXP; ++i) x[i] = __builtin_amdgcn_exp2f(x[i]);
#pragma unroll
            for (int i = NEXP; i < NEXP + NFMA; ++i) x[i] = __builtin_fmaf(x[i], 0.999f, 0.001f);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    float sum = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int e = 0; e < 16; ++e) sum += acc[c][e];
#pragma unroll
    for (int i = 0; i < 16; ++i) sum += x[i];
    out[(int64_t)blockIdx.x * 256 + threadIdx.x] = sum;
}

template <int NFMA, int NEXP>
int32_t launch_coissue(float* out, int32_t workgroups, int32_t iters, hipStream_t s) {
    hipLaunchKernelGGL((avf_probe_coissue_kernel<NFMA, NEXP>), dim3((uint32_t)workgroups), dim3(256), 0, s, out,
                       iters);
    return hipGetLastError() == hipSuccess ? 0 : -7;
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

// Launches the co-issue probe with nfma v_fma_f32 and nexp v_exp_f32 per
// MFMA slot, (nfma, nexp) one of (0,0) (4,0) (8,0) (16,0) (0,1) (0,2) (0,4)
// (3,1) (4,2). `out` (device) holds workgroups * 256 floats; each
// 256-thread workgroup runs iters * 8 slots per wave. Returns 0, -2 for bad
// arguments, -7 for a launch failure.
int32_t avf_probe_coissue(int32_t nfma, int32_t nexp, float* out, int32_t workgroups, int32_t iters, void* stream) {
    if (!out || workgroups <= 0 || iters <= 0) return -2;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    switch (nfma * 16 + nexp) {
        case 0: return launch_coissue<0, 0>(out, workgroups, iters, s);
        case 4 * 16: return launch_coissue<4, 0>(out, workgroups, iters, s);
        case 8 * 16: return launch_coissue<8, 0>(out, workgroups, iters, s);
        case 16 * 16: return launch_coissue<16, 0>(out, workgroups, iters, s);
        case 1: return launch_coissue<0, 1>(out, workgroups, iters, s);
        case 2: return launch_coissue<0, 2>(out, workgroups, iters, s);
        case 4: return launch_coissue<0, 4>(out, workgroups, iters, s);
        case 3 * 16 + 1: return launch_coissue<3, 1>(out, workgroups, iters, s);
        case 4 * 16 + 2: return launch_coissue<4, 2>(out, workgroups, iters, s);
        default: return -2;
    }
}

}  // extern "C"
