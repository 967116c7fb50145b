// Packed variable-length attention forward for gfx950 (MI355X, CDNA4).
//
// One workgroup computes one tile: BM query rows of one head of one segment,
// streaming that segment's K/V in blocks of BN keys through double-buffered
// LDS. The operation is the flash-attention varlen forward with its LSE
// (the (out, lse) return of flash_attn_varlen_func on the "[FA4] cute varlen
// backward: int32 overflow in _bwd_preprocess ..." page); the online softmax
// keeps a running row maximum m and sum l and rescales the accumulator when m
// grows, so the result equals softmax(scale * Q K^T) V exactly up to rounding.
//
// Matrix layout on the MFMA (v_mfma_f32_32x32x16_bf16, wave64):
//   S^T = K * Q^T:  A = 32 keys x 16 dims of K (from LDS, one 16-byte read per
//                   lane), B = Q^T (kept in registers for the whole tile).
//                   The 32x32 result puts ONE query row per lane pair
//                   (lane l and l+32, 16 keys each), so the row max needs one
//                   cross-half exchange and the row sum none until the end.
//   O^T += V^T P^T: A = 32 dims x 16 keys of V^T (LDS), B = P^T, which is the
//                   S^T result itself, rounded to bf16 in place: the key order
//                   of the MFMA result is matched by storing V^T in LDS with
//                   key bits 2 and 3 swapped inside every 16-key group.
//   O^T accumulates with one query row per lane pair too, so the rescale by
//   exp2(m_old - m_new) is a per-lane scalar.
// Offsets: every tensor base is formed in int64 (row * row_stride + head *
// head_stride, as the "Suggested kernel-side fix" of the _bwd_preprocess page
// asks) and rebased per tile; the per-lane buffer offsets inside a tile are
// bounded by BM * row_stride bytes < 2^31, checked on the host. Buffer
// resources clip every load and store to the tile's valid rows, so a tail
// tile reads zeros past the segment instead of a neighbour's or unmapped memory.
// Validity: the grid is exactly the tile count, so every workgroup decodes to a
// real tile before it forms any address (the SM120 page's memcheck findings
// show the opposite order, prefetching from garbage coordinates).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "avf_plan.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

// Largest per-lane partial row sum of softmax weights accepted before the
// reference max is moved (bounds every weight by 2^16).
constexpr float kPsumMax = 65536.0f;

// gfx9 raw buffer descriptor word 3: 32-bit data format, no swizzle, no
// index stride; records are bytes and out-of-range loads return 0.
constexpr int kBufWord3 = 0x00020000;

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             kBufWord3);
}

// Position of key k (0..BN-1) inside a V^T row in LDS: bits 2 and 3 swapped.
__device__ constexpr int vt_pos(int k) {
    return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1);
}

template <int D, int QB, int NW, int BN>
struct Tile {
    static constexpr int NT = NW * 64;          // threads per workgroup
    static constexpr int BM = QB * 32 * NW;     // query rows per tile
    static constexpr int KS = D / 16;           // MFMA k-steps over D
    static constexpr int DB = D / 32;           // 32-wide column blocks of O
    static constexpr int KB = BN / 32;          // 32-key sub-blocks per K/V tile
    static constexpr int KP = D * 2 + 16;       // K row pitch in LDS, bytes (padded)
    static constexpr int VP = BN * 2 + 16;      // V^T row pitch in LDS, bytes (padded)
    static constexpr int KBYTES = BN * KP;
    static constexpr int VBYTES = D * VP;
    static constexpr int STAGE = KBYTES + VBYTES;
    static constexpr int KCH = BN * D / 8;      // 16-byte chunks per K tile
    static constexpr int KPT = (KCH + NT - 1) / NT;
    static constexpr int VTASK = (BN / 4) * (D / 8);  // 4 keys x 8 dims per task
    static constexpr int VPT = (VTASK + NT - 1) / NT;
    static_assert(D % 32 == 0 && BN % 32 == 0, "tile shape");
};

template <int D, int QB, int NW, int BN>
__global__ void __launch_bounds__(NW * 64, 1) avf_fwd_kernel(const AvfLaunchArgs a) {
    using T = Tile<D, QB, NW, BN>;
    constexpr int BM = T::BM;
    __shared__ __attribute__((aligned(16))) char lds[2 * T::STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;
    const int hf = lane >> 5;

    // ---- tile decode (the grid is exact: every workgroup owns a real tile) ----
    const int32_t linear = avf_linear_tile((int32_t)blockIdx.x, a.num_tiles);
    const AvfTile tile = avf_decode(linear, a.tile_start, a.q_start, a.num_segs, a.num_heads, BM);
    const int32_t seg = tile.seg;
    const int32_t h = tile.head;
    const int32_t lq = a.q_start[seg + 1] - a.q_start[seg];
    const int32_t lk = a.k_start[seg + 1] - a.k_start[seg];
    const int32_t row0 = tile.mblk * BM;
    const int32_t rows_here = min(BM, lq - row0);
    const int64_t q_tok0 = (int64_t)a.q_start[seg] + row0;
    const int64_t k_tok0 = (int64_t)a.k_start[seg];

    // ---- Q^T fragments (B operand), resident for the whole tile ----
    const uint32_t q_rs = (uint32_t)(a.q_row * 2);
    const char* qptr = (const char*)a.q + 2 * avf_elem_offset(q_tok0, a.q_row, h, a.q_head);
    const auto qrs = make_rsrc(qptr, (uint32_t)(rows_here - 1) * q_rs + 2 * D);
    const int wrow0 = wave * QB * 32;
    bf16x8 qf[QB][T::KS];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int ks = 0; ks < T::KS; ++ks) {
            const uint32_t off = (uint32_t)(wrow0 + qb * 32 + l32) * q_rs + (ks * 16 + hf * 8) * 2;
            qf[qb][ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(qrs, off, 0, 0));
        }

    f32x16 o[QB][T::DB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int db = 0; db < T::DB; ++db)
#pragma unroll
            for (int e = 0; e < 16; ++e) o[qb][db][e] = 0.f;
    float m_i[QB], mc_i[QB], l_i[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        m_i[qb] = -INFINITY;
        mc_i[qb] = -INFINITY;
        l_i[qb] = 0.f;
    }
    const float c = a.scale_log2e;

    // ---- K/V staging: global -> registers (prefetch) -> LDS ----
    const int32_t nkt = (lk + BN - 1) / BN;
    const uint32_t k_rs = (uint32_t)(a.k_row * 2);
    const uint32_t v_rs = (uint32_t)(a.v_row * 2);
    i32x4 kst[T::KPT];
    i32x4 vst[T::VPT][4];

    auto load_tile = [&](int32_t j) {
        const int32_t key0 = j * BN;
        const int32_t nk = min(BN, lk - key0);
        const char* kp = (const char*)a.k + 2 * avf_elem_offset(k_tok0 + key0, a.k_row, h, a.k_head);
        const char* vp = (const char*)a.v + 2 * avf_elem_offset(k_tok0 + key0, a.v_row, h, a.v_head);
        const auto krs = make_rsrc(kp, (uint32_t)(nk - 1) * k_rs + 2 * D);
        const auto vrs = make_rsrc(vp, (uint32_t)(nk - 1) * v_rs + 2 * D);
#pragma unroll
        for (int cI = 0; cI < T::KPT; ++cI) {
            const int id = tid + cI * T::NT;
            if (T::KCH % T::NT == 0 || id < T::KCH) {
                const int key = id / (D / 8), dc = id % (D / 8);
                kst[cI] = __builtin_amdgcn_raw_buffer_load_b128(krs, key * k_rs + dc * 16, 0, 0);
            }
        }
#pragma unroll
        for (int cI = 0; cI < T::VPT; ++cI) {
            const int id = tid + cI * T::NT;
            if (T::VTASK % T::NT == 0 || id < T::VTASK) {
                const int kq = id % (BN / 4), dc = id / (BN / 4);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    vst[cI][r] = __builtin_amdgcn_raw_buffer_load_b128(vrs, (4 * kq + r) * v_rs + dc * 16, 0, 0);
            }
        }
    };

    auto store_tile = [&](int buf) {
        char* kl = lds + buf * T::STAGE;
        char* vl = kl + T::KBYTES;
#pragma unroll
        for (int cI = 0; cI < T::KPT; ++cI) {
            const int id = tid + cI * T::NT;
            if (T::KCH % T::NT == 0 || id < T::KCH) {
                const int key = id / (D / 8), dc = id % (D / 8);
                *reinterpret_cast<i32x4*>(kl + key * T::KP + dc * 16) = kst[cI];
            }
        }
#pragma unroll
        for (int cI = 0; cI < T::VPT; ++cI) {
            const int id = tid + cI * T::NT;
            if (T::VTASK % T::NT == 0 || id < T::VTASK) {
                const int kq = id % (BN / 4), dc = id / (BN / 4);
                const int pos = vt_pos(4 * kq);
#pragma unroll
                for (int cc = 0; cc < 8; ++cc) {
                    const int e = cc >> 1;
                    const uint32_t sel = (cc & 1) ? 0x07060302u : 0x05040100u;
                    i32x2 w;
                    w[0] = (int)__builtin_amdgcn_perm((uint32_t)vst[cI][1][e], (uint32_t)vst[cI][0][e], sel);
                    w[1] = (int)__builtin_amdgcn_perm((uint32_t)vst[cI][3][e], (uint32_t)vst[cI][2][e], sel);
                    *reinterpret_cast<i32x2*>(vl + (dc * 8 + cc) * T::VP + pos * 2) = w;
                }
            }
        }
    };

    if (nkt > 0) {
        load_tile(0);
        store_tile(0);
    }
    __syncthreads();
    // Every global load issued so far (Q fragments, first K/V tile) is complete
    // here; saying so keeps the compiler's wait counters inside the loop from
    // holding the MFMAs until the next tile's prefetch has landed.
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), other counters untouched

    for (int32_t j = 0; j < nkt; ++j) {
        const int buf = j & 1;
        const bool more = j + 1 < nkt;
        if (more) load_tile(j + 1);
        const char* kl = lds + buf * T::STAGE;
        const char* vl = kl + T::KBYTES;
        const int32_t nk = min(BN, lk - j * BN);

#pragma unroll
        for (int kb = 0; kb < T::KB; ++kb) {
            if (kb * 32 >= nk) break;
            // S^T for 32 keys x (QB*32) query rows
            f32x16 s[QB];
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
#pragma unroll
                for (int e = 0; e < 16; ++e) s[qb][e] = 0.f;
            bf16x8 ka[T::KS];
#pragma unroll
            for (int ks = 0; ks < T::KS; ++ks)
                ka[ks] = *reinterpret_cast<const bf16x8*>(kl + (kb * 32 + l32) * T::KP + (ks * 16 + hf * 8) * 2);
#pragma unroll
            for (int ks = 0; ks < T::KS; ++ks)
#pragma unroll
                for (int qb = 0; qb < QB; ++qb)
                    s[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks], qf[qb][ks], s[qb], 0, 0, 0);
            if (nk < (kb + 1) * 32) {
                // keys past the segment end: element e holds key kb*32 + 8*(e/4) + 4*hf + e%4
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int key = kb * 32 + 8 * (e >> 2) + 4 * hf + (e & 3);
                    if (key >= nk)
#pragma unroll
                        for (int qb = 0; qb < QB; ++qb) s[qb][e] = -INFINITY;
                }
            }
            // Online softmax against a lazily moved reference max m_i: the
            // weights are p = exp2(c*s - c*m_i). Every p is bounded by its row's
            // partial sum, so while each lane's sum stays <= kPsumMax nothing
            // can overflow and the reference may stay where it is. Otherwise
            // (first block, m_i = -inf; or a row max that grew by more than
            // log2(kPsumMax)) the wave takes this block's row max, rescales O and
            // l by exp2(c*(m_old - m_new)) and recomputes p. Same softmax; the
            // common path has neither a max reduction nor an accumulator rescale.
            bf16x8 pk[QB][2];
            float psum[QB];
            auto weights = [&]() {
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) {
                    float acc = 0.f;
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qb][e], c, -mc_i[qb]));
                        acc += p;
                        pk[qb][e >> 3][e & 7] = (__bf16)p;
                    }
                    psum[qb] = acc;
                }
            };
            weights();
            bool over = false;
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) over |= !(psum[qb] <= kPsumMax);  // NaN counts as over
            if (__builtin_amdgcn_ballot_w64(over) != 0) {
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) {
                    float v = s[qb][0];
#pragma unroll
                    for (int e = 1; e < 16; ++e) v = fmaxf(v, s[qb][e]);
                    const float mnew = fmaxf(m_i[qb], fmaxf(v, __shfl_xor(v, 32)));
                    const float alpha = __builtin_amdgcn_exp2f((m_i[qb] - mnew) * c);
                    l_i[qb] *= alpha;
#pragma unroll
                    for (int db = 0; db < T::DB; ++db)
#pragma unroll
                        for (int e = 0; e < 16; ++e) o[qb][db][e] *= alpha;
                    m_i[qb] = mnew;
                    mc_i[qb] = mnew * c;
                }
                weights();
            }
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) l_i[qb] += psum[qb];
            // O^T += V^T P^T over the 32 keys, two 16-key MFMA steps
#pragma unroll
            for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
                for (int db = 0; db < T::DB; ++db) {
                    const bf16x8 va = *reinterpret_cast<const bf16x8*>(vl + (db * 32 + l32) * T::VP + (kb * 32 + k2 * 16 + hf * 8) * 2);
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb)
                        o[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pk[qb][k2], o[qb][db], 0, 0, 0);
                }
        }
        if (more) store_tile(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: O = O_acc / l (bf16), LSE = m*scale + ln l ----
    const uint32_t o_rs = (uint32_t)(a.o_row * 2);
    char* optr = (char*)a.o + 2 * avf_elem_offset(q_tok0, a.o_row, h, a.o_head);
    const auto ors = make_rsrc(optr, (uint32_t)(rows_here - 1) * o_rs + 2 * D);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const float l_tot = l_i[qb] + __shfl_xor(l_i[qb], 32);
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        const int row = wrow0 + qb * 32 + l32;
        if (row < rows_here) {
#pragma unroll
            for (int db = 0; db < T::DB; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    bf16x4 ov;
#pragma unroll
                    for (int e = 0; e < 4; ++e) ov[e] = (__bf16)(o[qb][db][4 * g + e] * inv);
                    const uint32_t off = (uint32_t)row * o_rs + (db * 32 + 8 * g + 4 * hf) * 2;
                    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(i32x2, ov), ors, off, 0, 0);
                }
            if (hf == 0 && a.lse != nullptr) {
                const float lse = l_tot > 0.f ? m_i[qb] * a.scale + __logf(l_tot) : -INFINITY;
                a.lse[(int64_t)h * a.lse_head + q_tok0 + row] = lse;
            }
        }
    }
}

template <int D, int QB, int NW, int BN>
hipError_t launch_cfg(const AvfLaunchArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL((avf_fwd_kernel<D, QB, NW, BN>), dim3((uint32_t)a.num_tiles), dim3(NW * 64), 0,
                       stream, a);
    return hipGetLastError();
}

// Per head_dim tile configuration: (QB query blocks of 32 rows per wave,
// NW waves, BN keys per K/V stage). BM = QB * 32 * NW. Overridable at build
// time (-DAVF_CFG_D128=QB,NW,BN) for tuning sweeps.
#ifndef AVF_CFG_D64
#define AVF_CFG_D64 1, 8, 64
#endif
#ifndef AVF_CFG_D96
#define AVF_CFG_D96 1, 8, 64
#endif
#ifndef AVF_CFG_D128
#define AVF_CFG_D128 1, 8, 64
#endif
template <int QB_, int NW_, int BN_>
struct CfgOf { static constexpr int QB = QB_, NW = NW_, BN = BN_; };
template <int D> struct Cfg;
template <> struct Cfg<64> : CfgOf<AVF_CFG_D64> {};
template <> struct Cfg<96> : CfgOf<AVF_CFG_D96> {};
template <> struct Cfg<128> : CfgOf<AVF_CFG_D128> {};

template <int D>
constexpr int block_m_of() { return Cfg<D>::QB * 32 * Cfg<D>::NW; }

}  // namespace

int32_t avf_block_m(int32_t head_dim) {
    switch (head_dim) {
        case 64: return block_m_of<64>();
        case 96: return block_m_of<96>();
        case 128: return block_m_of<128>();
        default: return -1;
    }
}

hipError_t avf_launch(const AvfLaunchArgs& a, int32_t head_dim, hipStream_t stream) {
    switch (head_dim) {
        case 64: return launch_cfg<64, Cfg<64>::QB, Cfg<64>::NW, Cfg<64>::BN>(a, stream);
        case 96: return launch_cfg<96, Cfg<96>::QB, Cfg<96>::NW, Cfg<96>::BN>(a, stream);
        case 128: return launch_cfg<128, Cfg<128>::QB, Cfg<128>::NW, Cfg<128>::BN>(a, stream);
        default: return hipErrorInvalidValue;
    }
}
