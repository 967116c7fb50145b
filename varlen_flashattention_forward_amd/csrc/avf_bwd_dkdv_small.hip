// dK/dV kernel instantiations for head_dim 64 and 96: compiled with MFMA
// results in architectural registers, so the softmax reads S and dP without
// AGPR copies, and cut for two workgroups per CU (two waves per SIMD, which
// overlap one wave's softmax with the other's MFMAs). Their registers fit
// 256 per lane; head_dim 128 does not and lives in avf_bwd_kernel.hip.

#include "avf_bwd_impl.h"

hipError_t avf_bwd_dkdv_launch_small(const AvfBwdArgs& a, int32_t head_dim, hipStream_t stream) {
    switch (head_dim) {
        case 64: return launch_dkdv<64, 2>(a, stream);
        case 96: return launch_dkdv<96, 2>(a, stream);
        default: return hipErrorInvalidValue;
    }
}
