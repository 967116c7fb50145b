// Device helpers shared by the gfx950 attention kernels: vector types, buffer
// resources, the direct-to-LDS buffer load, and the transposing LDS fragment
// read. Included only by the HIP kernel sources of this library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace avf {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

// gfx9 raw buffer descriptor word 3: 32-bit data format, no swizzle, no
// index stride; records are bytes and out-of-range loads return 0.
constexpr int kBufWord3 = 0x00020000;

// s_waitcnt immediate (gfx9 encoding) that waits for vmcnt <= n and leaves the
// export and LGKM counters untouched.
__host__ __device__ constexpr int vmcnt_imm(int n) {
    return (n & 15) | ((n >> 4) << 14) | 0x70 | 0xF00;
}

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             kBufWord3);
}

// 16-byte buffer load written straight to LDS: lane l of the wave fills LDS
// bytes [lds_addr + 16*l, +16) (lds_addr in M0, wave-uniform) with the record at
// `voffset` of the buffer resource `rsrc`. It is issued as inline assembly on
// purpose: the compiler then does not track it, so it adds no vector-memory
// waits of its own before later LDS reads (it would otherwise make every
// transposing read wait for the loads of later stages, which write other
// buffers of the ring). Completion is awaited explicitly with s_waitcnt vmcnt
// and a barrier before the stage is read. Vector-memory loads complete in
// order, so the compiler's own waits on older loads stay correct.
__device__ inline void load_lds16(i32x4 rsrc, uint32_t lds_addr, uint32_t voffset) {
#if defined(__HIP_DEVICE_COMPILE__)
    asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(voffset), "s"(rsrc), "{m0}"(__builtin_amdgcn_readfirstlane(lds_addr))
                 : "memory");
#endif
}

// load_lds16 with a wave-uniform byte offset `soffset` (an SGPR) added to the
// lane's `voffset`, so that loads of one lane that differ by a uniform stride
// share one offset register and need no per-load vector arithmetic.
__device__ inline void load_lds16_so(i32x4 rsrc, uint32_t lds_addr, uint32_t voffset, uint32_t soffset) {
#if defined(__HIP_DEVICE_COMPILE__)
    asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds"
                 :
                 : "v"(voffset), "s"(rsrc), "s"(__builtin_amdgcn_readfirstlane(soffset)),
                   "{m0}"(__builtin_amdgcn_readfirstlane(lds_addr))
                 : "memory");
#endif
}

// Marks `x` as read and rewritten at this point of the instruction stream
// (emits nothing). Between scheduling fences this keeps a pure arithmetic
// result where the source computes it instead of letting the optimizer sink
// it to its first use.
template <typename V>
__device__ inline void pin(V& x) {
    asm volatile("" : "+v"(x));
}

// Buffer resource words (gfx9 layout) for the inline-assembly loads.
__device__ inline i32x4 rsrc_words(const void* base, uint32_t bytes) {
    const uint64_t b = (uint64_t)(uintptr_t)base;
    i32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)b);
    r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32) & 0xffff);  // stride 0
    r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
    r[3] = kBufWord3;
    return r;
}

// Two transposing 8-byte LDS reads (ds_read_b64_tr_b16) at p0 and p1 joined
// into one 8 x bf16 MFMA operand (p0 gives elements 0..3, p1 elements 4..7).
__device__ inline bf16x8 read_tr8(const char* p0, const char* p1) {
    const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p0);
    const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p1);
    const i16x8 both = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    return __builtin_bit_cast(bf16x8, both);
}

}  // namespace avf
