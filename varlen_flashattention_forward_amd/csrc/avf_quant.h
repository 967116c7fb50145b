// Per-head E4M3 quantization of Q and K (host launcher next to the kernels).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

struct AvfQuantArgs {
    const void* q;
    const void* k;
    int64_t q_rows, k_rows;  // rows [0, n) of each tensor are quantized
    int64_t q_row, q_head, k_row, k_head;  // element strides
    int32_t num_heads, head_dim;           // head_dim 64 or 128
    uint32_t* amax;  // 2 * num_heads words: amax of q per head, then of k (fp32 bits)
    uint8_t* q8;     // packed [q_rows, H, D] codes
    uint8_t* k8;     // packed [k_rows, H, D] codes
};

// Clears amax, then for q and k: per-head amax, then the codes.
hipError_t avf_fp8_quantize(const AvfQuantArgs& args, hipStream_t stream);
