// Backward kernels of packed variable-length attention (gfx950), as
// templates: included by the two sources that instantiate them (the dK/dV
// kernel for head_dim 64 and 96 is compiled with MFMA results in
// architectural registers and two workgroups per CU, head_dim 128 with
// AGPR accumulators and one). See avf_bwd_kernel.hip for the algorithm.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "avf_bwd_plan.h"
#include "avf_device.h"

namespace {

using namespace avf;

constexpr float kLog2e = 1.4426950408889634f;

// Chunk permutation of a 2*D-byte LDS row read both ways:
//  row fragments (ds_read_b128): each 16-lane phase reads one chunk of 16
//    consecutive rows, so f must separate those rows over all 64 banks;
//  transposed fragments (ds_read_b64_tr_b16): each 32-lane phase reads 4
//    chunks (aligned to 4) of 4 consecutive rows (aligned to 4), so f must
//    give those 4 rows different groups of 4 chunks.
//  D = 128 (16 chunks, 256-byte rows): the two 2-bit fields of row % 16 swapped;
//  D = 64 (8 chunks, two rows per 256 bytes): bit 1 of the row to chunk bit 2,
//    bits 2-3 to chunk bits 0-1;
//  D = 96 (12 chunks, 192-byte rows cycle through 4 bank offsets): (row / 4) % 4.
// All three are checked against the 64-bank model for both patterns; f depends
// on the row only modulo 16 and never leaves the row.
template <int D>
__device__ constexpr int dual_swz(int row) {
    if constexpr (D == 128)
        return ((row & 3) << 2) | ((row >> 2) & 3);
    else if constexpr (D == 64)
        return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
    else
        return (row >> 2) & 3;
}

// ---------------------------------------------------------------------------
// Preprocessing: D[h, i] = sum_d O[i,h,d] * dO[i,h,d] in fp32. 16 lanes per
// (row, head) item, each reading 16 bytes of both rows; 16 items per
// 256-thread workgroup. HBM bound: it reads O and dO once.
template <int D>
__global__ void __launch_bounds__(256) avf_bwd_pre_kernel(const AvfPreArgs a) {
    const int64_t item = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
    const int c = threadIdx.x & 15;
    const int64_t items = a.rows * a.num_heads;
    float acc = 0.f;
    int64_t row = 0, h = 0;
    if (item < items) {
        row = item / a.num_heads;
        h = item - row * a.num_heads;
        if (c < D / 8) {
            const char* op = (const char*)a.o + 2 * (row * a.o_row + h * a.o_head) + 16 * c;
            const char* gp = (const char*)a.dout + 2 * (row * a.do_row + h * a.do_head) + 16 * c;
            const bf16x8 ov = *reinterpret_cast<const bf16x8*>(op);
            const bf16x8 gv = *reinterpret_cast<const bf16x8*>(gp);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc = __builtin_fmaf((float)ov[e], (float)gv[e], acc);
        }
    }
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 16);
    if (item < items && c == 0) a.delta[h * a.delta_head + row] = acc;
}

// ---------------------------------------------------------------------------
// Row staging shared by both tile kernels: `nrows` valid rows (row r of the
// stage at element offset r * row_stride from `base`) copied into an LDS
// block of BR rows x 2*D bytes with dual_swz, by NW waves issuing 1 KiB
// direct loads. Rows past nrows re-read the last valid row (finite data;
// the kernels mask them out).
template <int D, int BR, int NW>
__device__ inline void stage_rows(const void* base, int64_t row_stride, int32_t nrows, uint32_t lds_dst,
                                  int wave, int lane) {
    constexpr int ROWB = 2 * D;
    constexpr int NI = BR * ROWB / 1024;
    static_assert(NI % NW == 0, "every wave issues the same number of loads");
    const uint32_t rs = (uint32_t)(row_stride * 2);
    const i32x4 rsrc = rsrc_words(base, (uint32_t)(nrows - 1) * rs + ROWB);
#pragma unroll
    for (int m = 0; m < NI / NW; ++m) {
        const int i = wave + NW * m;
        const int pos = i * 1024 + 16 * lane;
        const int row = pos / ROWB;
        const int slot = (pos % ROWB) >> 4;
        const uint32_t rc = (uint32_t)min(row, nrows - 1);
        load_lds16(rsrc, lds_dst + i * 1024, rc * rs + ((slot ^ dual_swz<D>(row)) << 4));
    }
}

// Per-lane LDS byte offsets (within a staged block, relative to a 32-row
// sub-block) of the two fragment kinds read from dual_swz rows.
template <int D>
struct FragOffsets {
    static constexpr int KS = D / 16, DB = D / 32, ROWB = 2 * D;
    int row[KS];     // row fragment ks: row l32, chunk 2*ks + hf
    int tr[2][DB];   // transposed fragment half r, dims [db*32, +32)
    __device__ FragOffsets(int lane) {
        const int l32 = lane & 31, hf = lane >> 5;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) row[ks] = l32 * ROWB + (((2 * ks + hf) ^ dual_swz<D>(l32)) << 4);
        // In each 16-lane group, lane j of a transposing read receives
        // element j % 4 of the 8-byte rows read by lanes 4t + j / 4: reading
        // row 8r + 4*hf + (lane/4) % 4 at dims db*32 + 16*((lane/16) % 2) +
        // 4*(lane % 4) hands lane l the dims l % 32 of exactly the rows its
        // B-operand slots 4r..4r+3 hold in the 32x32 C layout.
        const int trow = 4 * hf + ((lane >> 2) & 3);
        const int tdim = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const int row8 = 8 * r + trow, d = db * 32 + tdim;
                tr[r][db] = row8 * ROWB + (((d >> 3) ^ dual_swz<D>(row8)) << 4) + (d & 4) * 2;
            }
    }
};

// MFMA B-operand fragments of 32 rows (lane: row l32, dims ks*16 + hf*8 .. +8)
// loaded straight from global memory; rows at or past nrows read 0.
template <int D>
__device__ inline void load_b_frags(const void* base, int64_t row_stride, int32_t nrows, int lane,
                                    bf16x8 (&f)[D / 16]) {
    const uint32_t rs = (uint32_t)(row_stride * 2);
    const auto rsrc = make_rsrc(base, nrows > 0 ? (uint32_t)(nrows - 1) * rs + 2 * D : 0u);
    const int l32 = lane & 31, hf = lane >> 5;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
        const uint32_t off = (uint32_t)l32 * rs + (ks * 16 + hf * 8) * 2;
        f[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rsrc, off, 0, 0));
    }
}

// Store a transposed 32-row block acc[db] (C[m = dim][n = row], row = l32)
// scaled by `mul` as bf16 rows [0, nrows) of a [rows, D] tensor at `base`.
template <int D>
__device__ inline void store_rows_t(void* base, int64_t row_stride, int32_t nrows, int lane,
                                    const f32x16 (&acc)[D / 32], float mul) {
    const int l32 = lane & 31, hf = lane >> 5;
    if (nrows <= 0 || l32 >= nrows) return;
    const uint32_t rs = (uint32_t)(row_stride * 2);
    const auto rsrc = make_rsrc(base, (uint32_t)(nrows - 1) * rs + 2 * D);
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            bf16x4 w;
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = (__bf16)(acc[db][4 * g + e] * mul);
            const uint32_t off = (uint32_t)l32 * rs + (db * 32 + 8 * g + 4 * hf) * 2;
            __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(i32x2, w), rsrc, off, 0, 0);
        }
}

// f(std::integral_constant<int, i>) for i = B .. E-1, in order
template <int B, int E, typename F>
__device__ inline void static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// dK/dV sub-block slots (KS = D/16 MFMA slots per product, DB = D/32): the
// scaled exponent of element e (its exp2 and, for a pair, the bf16 packing
// follow one slot apart), and the product dS = P (dP - D) (the packing
// follows one slot later). Elements 0-7 feed the first 16-row half of the P
// and dS operands, 8-15 the second.
constexpr int dkdv_p_slot(int e, int KS, int DB) {
    return e < 8 ? KS + 1 + e * (KS - 3) / 8 : 2 * KS - 2 + (e - 8) * DB / 8;
}
constexpr int dkdv_ds_slot(int e, int KS, int DB) {
    return e < 8 ? 2 * KS + 1 + e * (KS - 3) / 8 : 3 * KS - 2 + (e - 8) * DB / 8;
}

// ---------------------------------------------------------------------------
// dK/dV: one workgroup per (segment, head, block of 32*NW keys); wave w owns
// keys [w*32, +32) of the block with their K and V rows in registers and
// dK^T, dV^T accumulators. Query rows stream in stages of BQ rows: Q, dO,
// LSE and D of the stage in one LDS buffer, two buffers.
// MINB: workgroups per CU the register budget is cut for (1: up to 512
// registers per lane with AGPRs; 2: up to 256).
template <int D, int NW, int BQ, bool CAUSAL, int MINB>
__global__ void __launch_bounds__(NW * 64, MINB) avf_bwd_dkdv_kernel(const AvfBwdArgs a) {
    constexpr int KS = D / 16, DB = D / 32, ROWB = 2 * D;
    constexpr int BN = 32 * NW;
    constexpr int SB = BQ / 32;
    constexpr int RBYTES = BQ * ROWB;                  // Q (or dO) rows of a stage
    constexpr int OFF_DO = RBYTES;
    // LSE and D rows arrive at OFF_RAW and OFF_RAWD; before the stage's
    // barrier wave 0 stores them at OFF_LSE as -LSE * log2(e), the offset the
    // weights' exponent takes, and at OFF_DEL as -D, the initial value of the
    // dP accumulator (so the MFMA yields dP - D), so no wave spends a VALU
    // instruction per element on either
    constexpr int OFF_LSE = 2 * RBYTES;
    constexpr int OFF_DEL = 2 * RBYTES + 4 * BQ;
    constexpr int OFF_RAW = 2 * RBYTES + 8 * BQ;
    constexpr int OFF_RAWD = 2 * RBYTES + 12 * BQ;
    constexpr int STAGE = 2 * RBYTES + 16 * BQ;
    static_assert(STAGE % 16 == 0 && BQ % 32 == 0 && BQ <= 64, "stage layout");
    __shared__ __attribute__((aligned(16))) char lds[2 * STAGE];
    const uint32_t lds_addr = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;
    const int hf = lane >> 5;

    const int32_t linear = avf_linear_tile((int32_t)blockIdx.x, a.num_tiles);
    const AvfTile tile = avf_decode(linear, a.tile_start, a.k_start, a.num_segs, a.num_heads, BN);
    const int32_t seg = tile.seg;
    const int64_t h = tile.head;
    const int32_t lq = a.q_start[seg + 1] - a.q_start[seg];
    const int32_t lk = a.k_start[seg + 1] - a.k_start[seg];
    const int32_t key0 = tile.mblk * BN;
    const int32_t wkey0 = key0 + wave * 32;            // the wave's first key
    const int32_t wkeys = max(0, min(32, lk - wkey0));  // its valid keys
    const int64_t q_tok0 = a.q_start[seg];
    const int64_t k_tok = (int64_t)a.k_start[seg] + wkey0;
    const int32_t coff = lk - lq;  // causal: row r sees keys j <= r + coff

    bf16x8 kf[KS], vf[KS];
    load_b_frags<D>((const char*)a.k + 2 * (k_tok * a.k_row + h * a.k_head), a.k_row, wkeys, lane, kf);
    load_b_frags<D>((const char*)a.v + 2 * (k_tok * a.v_row + h * a.v_head), a.v_row, wkeys, lane, vf);
    f32x16 dk[DB], dv[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) dk[db][e] = dv[db][e] = 0.f;

    // Query rows that see any key of the block: all, or with the causal mask
    // rows r >= key0 - coff. Stages from jfull on see every key of the block.
    const int32_t nst = (lq + BQ - 1) / BQ;
    const int32_t js = CAUSAL ? min(nst, max(0, key0 - coff) / BQ) : 0;
    const int32_t jfull = CAUSAL ? min(nst, max(js, (key0 + BN - 1 - coff + BQ - 1) / BQ)) : 0;

    const FragOffsets<D> fo(lane);
    const float c = a.scale_log2e;

    auto load_stage = [&](int32_t j, int buf) {
        const int32_t q0 = j * BQ;
        const int32_t nrows = min(BQ, lq - q0);
        const int64_t tok = q_tok0 + q0;
        const uint32_t dst = lds_addr + buf * STAGE;
        stage_rows<D, BQ, NW>((const char*)a.q + 2 * (tok * a.q_row + h * a.q_head), a.q_row, nrows, dst, wave,
                              lane);
        stage_rows<D, BQ, NW>((const char*)a.dout + 2 * (tok * a.do_row + h * a.do_head), a.do_row, nrows,
                              dst + OFF_DO, wave, lane);
        // LSE and D of the stage's rows: 4 * BQ bytes each, 16-byte lanes of wave 0
        if (wave == 0 && lane < BQ / 4) {
            const i32x4 lr = rsrc_words(a.lse + h * a.lse_head + tok, (uint32_t)nrows * 4);
            const i32x4 dr = rsrc_words(a.delta + h * a.delta_head + tok, (uint32_t)nrows * 4);
            load_lds16(lr, dst + OFF_RAW, 16 * lane);
            load_lds16(dr, dst + OFF_RAWD, 16 * lane);
        }
    };

    // One stage: for each 32-row sub-block, S and dP (queries x the wave's
    // keys), P and dS, then dV^T += dO^T P and dK^T += Q^T dS.
    // MASKED (compile-time): rows past the segment end, and with the causal
    // mask keys past the row's limit, get P = dS = 0 (selected, so garbage
    // LSE/D of padding rows never enters).
    // A sub-block is written slot by slot, one MFMA per slot, with a
    // scheduling fence between slots: S (KS slots), dP (KS), dV from the
    // weights of rows 0-15 and 16-31 of the 32x32 result (DB each), then dK
    // the same way. Each slot reads the A operand of the MFMA two slots on,
    // and carries a share of the VALU work, placed after the MFMA whose
    // result it needs has had a slot to finish and before the first MFMA
    // that takes it: the weights P of the lane's rows 0-7 (elements 0-7)
    // during dP and of rows 8-15 early in dV, dS likewise one group later.
    // The per-accumulator MFMA order is unchanged (t = 0 before t = 1).
    auto stage = [&](int32_t j, int buf, auto masked) {
        constexpr bool MASKED = decltype(masked)::value;
        constexpr int NSL = 4 * KS;
        const char* sbase = lds + buf * STAGE;
#pragma unroll
        for (int sb = 0; sb < SB; ++sb) {
            const char* qrows = sbase + sb * 32 * ROWB;
            const char* grows = sbase + OFF_DO + sb * 32 * ROWB;
            // A operand of MFMA slot m: Q rows, dO rows, then dO^T and Q^T
            // (transposed reads) for t = 0, 1
            auto read_a = [&](auto mc) -> bf16x8 {
                constexpr int m = decltype(mc)::value;
                if constexpr (m < KS) {
                    return *reinterpret_cast<const bf16x8*>(qrows + fo.row[m]);
                } else if constexpr (m < 2 * KS) {
                    return *reinterpret_cast<const bf16x8*>(grows + fo.row[m - KS]);
                } else {
                    constexpr int grp = (m - 2 * KS) / DB, d = (m - 2 * KS) % DB;
                    const char* b = (grp < 2 ? grows : qrows) + (grp & 1) * 16 * ROWB;
                    return read_tr8(b + fo.tr[0][d], b + fo.tr[1][d]);
                }
            };
            // element e of the lane: row sb*32 + 8*(e/4) + 4*hf + e%4 of the stage
            auto row_ok = [&](int e) {
                const int32_t row = j * BQ + sb * 32 + 8 * (e >> 2) + 4 * hf + (e & 3);
                bool ok = row < lq;
                if constexpr (CAUSAL) ok = ok && (wkey0 + l32 <= row + coff);
                return ok;
            };
            f32x16 sacc, dpacc, dinit;
            float4 lse4[4];
            float x[16], pw[16], dsv[16];
            bf16x8 pb[2], db16[2];
            bf16x8 abuf[3];
            static_for<-2, NSL>([&](auto tc) {
                constexpr int t = decltype(tc)::value;
                if constexpr (t + 2 < NSL) abuf[(t + 2) % 3] = read_a(std::integral_constant<int, t + 2>{});
                if constexpr (t == -2) {
#pragma unroll
                    for (int g = 0; g < 4; ++g)
                        lse4[g] = *reinterpret_cast<const float4*>(sbase + OFF_LSE + 4 * (sb * 32 + 8 * g + 4 * hf));
                }
                // -D of the lane's 16 rows: the dP accumulator's initial value
                if constexpr (t == KS - 3) {
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const float4 v = *reinterpret_cast<const float4*>(sbase + OFF_DEL + 4 * (sb * 32 + 8 * g + 4 * hf));
                        dinit[4 * g] = v.x;
                        dinit[4 * g + 1] = v.y;
                        dinit[4 * g + 2] = v.z;
                        dinit[4 * g + 3] = v.w;
                    }
                }
                if constexpr (t >= 0) {
                    const bf16x8 A = abuf[t % 3];
                    const f32x16 zero = {};
                    if constexpr (t < KS) {
                        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, kf[t], t == 0 ? zero : sacc, 0, 0, 0);
                    } else if constexpr (t < 2 * KS) {
                        dpacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, vf[t - KS], t == KS ? dinit : dpacc, 0, 0, 0);
                    } else {
                        constexpr int grp = (t - 2 * KS) / DB, d = (t - 2 * KS) % DB;
                        if constexpr (grp < 2)
                            dv[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, pb[grp], dv[d], 0, 0, 0);
                        else
                            dk[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, db16[grp - 2], dk[d], 0, 0, 0);
                    }
                }
                static_for<0, 16>([&](auto ec) {
                    constexpr int e = decltype(ec)::value;
                    constexpr int pf = dkdv_p_slot(e, KS, DB), dsub = dkdv_ds_slot(e, KS, DB);
                    if constexpr (t == pf) {
                        const float4 v = lse4[e >> 2];  // -LSE * log2(e) of the element's row
                        x[e] = __builtin_fmaf(sacc[e], c,
                                              (e & 3) == 0 ? v.x : (e & 3) == 1 ? v.y : (e & 3) == 2 ? v.z : v.w);
                        pin(x[e]);
                    } else if constexpr (t == pf + 1) {
                        pw[e] = __builtin_amdgcn_exp2f(x[e]);
                        pin(pw[e]);
                    } else if constexpr (t == pf + 2 && (e & 1)) {
                        float p0 = pw[e - 1], p1 = pw[e];
                        if constexpr (MASKED) {
                            p0 = row_ok(e - 1) ? p0 : 0.f;
                            p1 = row_ok(e) ? p1 : 0.f;
                        }
                        bf16x2 w = {(__bf16)p0, (__bf16)p1};
                        pin(w);
                        pb[e >> 3][(e & 7) - 1] = w[0];
                        pb[e >> 3][e & 7] = w[1];
                    }
                    if constexpr (t == dsub) {
                        dsv[e] = pw[e] * dpacc[e];  // dpacc holds dP - D
                        if constexpr (MASKED) dsv[e] = row_ok(e) ? dsv[e] : 0.f;
                        pin(dsv[e]);
                    } else if constexpr (t == dsub + 1 && (e & 1)) {
                        bf16x2 w = {(__bf16)dsv[e - 1], (__bf16)dsv[e]};
                        pin(w);
                        db16[e >> 3][(e & 7) - 1] = w[0];
                        db16[e >> 3][e & 7] = w[1];
                    }
                });
                __builtin_amdgcn_sched_barrier(0);
            });
        }
    };

    if (js < nst) {
        load_stage(js, 0);
        int buf = 0;
        auto next = [&](int32_t j) {
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
            if (wave == 0 && lane < BQ / 4) {
                char* sb = lds + buf * STAGE;
                const float4 r = *reinterpret_cast<const float4*>(sb + OFF_RAW + 16 * lane);
                const float4 d = *reinterpret_cast<const float4*>(sb + OFF_RAWD + 16 * lane);
                *reinterpret_cast<float4*>(sb + OFF_LSE + 16 * lane) =
                    float4{-r.x * kLog2e, -r.y * kLog2e, -r.z * kLog2e, -r.w * kLog2e};
                *reinterpret_cast<float4*>(sb + OFF_DEL + 16 * lane) = float4{-d.x, -d.y, -d.z, -d.w};
            }
            __syncthreads();
            if (j + 1 < nst) load_stage(j + 1, buf ^ 1);
        };
        int32_t j = js;
        // stages crossing the causal diagonal of the block
        if constexpr (CAUSAL) {
            for (; j < jfull; ++j) {
                next(j);
                stage(j, buf, std::true_type{});
                buf ^= 1;
            }
        }
        // stages every row of which sees every key of the block
        for (; j + 1 < nst; ++j) {
            next(j);
            stage(j, buf, std::false_type{});
            buf ^= 1;
        }
        if (j < nst) {
            next(j);
            stage(j, buf, std::true_type{});
        }
    }

    store_rows_t<D>((char*)a.dk + 2 * (k_tok * a.dk_row + h * a.dk_head), a.dk_row, wkeys, lane, dk, a.scale);
    store_rows_t<D>((char*)a.dv + 2 * (k_tok * a.dv_row + h * a.dv_head), a.dv_row, wkeys, lane, dv, 1.f);
}

// ---------------------------------------------------------------------------
// dQ: one workgroup per (segment, head, block of 32*NW query rows); wave w
// owns rows [w*32, +32) with their Q and dO rows in registers, one LSE and
// one D per lane, and a dQ^T accumulator. Keys stream in stages of BK: K and
// V rows of the stage in one LDS buffer, two buffers.
template <int D, int NW, int BK, bool CAUSAL>
__global__ void __launch_bounds__(NW * 64, 2) avf_bwd_dq_kernel(const AvfBwdArgs a) {
    constexpr int KS = D / 16, DB = D / 32, ROWB = 2 * D;
    constexpr int BM = 32 * NW;
    constexpr int SB = BK / 32;
    constexpr int RBYTES = BK * ROWB;
    constexpr int STAGE = 2 * RBYTES;  // K rows, then V rows
    static_assert(BK % 32 == 0, "stage layout");
    __shared__ __attribute__((aligned(16))) char lds[2 * STAGE];
    const uint32_t lds_addr = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;
    const int hf = lane >> 5;

    const int32_t linear = avf_linear_tile((int32_t)blockIdx.x, a.num_tiles);
    const AvfTile tile = avf_decode(linear, a.tile_start, a.q_start, a.num_segs, a.num_heads, BM);
    const int32_t seg = tile.seg;
    const int64_t h = tile.head;
    const int32_t lq = a.q_start[seg + 1] - a.q_start[seg];
    const int32_t lk = a.k_start[seg + 1] - a.k_start[seg];
    // causal: later row blocks see more keys, so they are dispatched first
    const int32_t mblk = CAUSAL ? (lq + BM - 1) / BM - 1 - tile.mblk : tile.mblk;
    const int32_t row0 = mblk * BM;
    const int32_t rows_here = min(BM, lq - row0);
    const int32_t wrow0 = row0 + wave * 32;
    const int32_t wrows = max(0, min(32, lq - wrow0));
    const int64_t q_tok = (int64_t)a.q_start[seg] + wrow0;
    const int64_t k_tok0 = a.k_start[seg];
    const int32_t coff = lk - lq;
    // keys the block needs, and the first key some row of it does not see
    const int32_t k_end = CAUSAL ? max(0, min(lk, row0 + rows_here + coff)) : lk;
    const int32_t kfull = CAUSAL ? max(0, min(k_end, row0 + 1 + coff)) : k_end;

    bf16x8 qf[KS], gf[KS];
    load_b_frags<D>((const char*)a.q + 2 * (q_tok * a.q_row + h * a.q_head), a.q_row, wrows, lane, qf);
    load_b_frags<D>((const char*)a.dout + 2 * (q_tok * a.do_row + h * a.do_head), a.do_row, wrows, lane, gf);
    // this lane's row l32: LSE in base-2 units and D (0 past the segment)
    float lse2 = 0.f, del = 0.f;
    if (l32 < wrows) {
        lse2 = a.lse[h * a.lse_head + q_tok + l32] * kLog2e;
        del = a.delta[h * a.delta_head + q_tok + l32];
    }
    f32x16 dq[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) dq[db][e] = 0.f;
    // -D of the lane's row in every slot: the dP accumulator's initial value,
    // so the MFMA yields dP - D
    f32x16 negd;
#pragma unroll
    for (int e = 0; e < 16; ++e) negd[e] = -del;

    const FragOffsets<D> fo(lane);
    const float c = a.scale_log2e;
    const int32_t nst = (k_end + BK - 1) / BK;
    const int32_t jmask = kfull / BK;  // first stage with a per-row limit

    auto load_stage = [&](int32_t j, int buf) {
        const int32_t k0 = j * BK;
        const int32_t nk = min(BK, k_end - k0);
        const int64_t tok = k_tok0 + k0;
        const uint32_t dst = lds_addr + buf * STAGE;
        stage_rows<D, BK, NW>((const char*)a.k + 2 * (tok * a.k_row + h * a.k_head), a.k_row, nk, dst, wave, lane);
        stage_rows<D, BK, NW>((const char*)a.v + 2 * (tok * a.v_row + h * a.v_head), a.v_row, nk, dst + RBYTES,
                              wave, lane);
    };

    // One stage: per 32-key sub-block, S^T and dP^T (keys x the wave's rows),
    // P and dS, then dQ^T += K^T dS^T. MASKED: keys at or past the lane's
    // limit (segment or block end, causal limit of its row) get P = dS = 0.
    auto stage = [&](int32_t j, int buf, auto masked) {
        constexpr bool MASKED = decltype(masked)::value;
        const char* sbase = lds + buf * STAGE;
        int32_t lim = BK;
        if constexpr (MASKED) {
            lim = min(BK, k_end - j * BK);
            if constexpr (CAUSAL) lim = min(lim, wrow0 + l32 + coff + 1 - j * BK);
        }
#pragma unroll
        for (int sb = 0; sb < SB; ++sb) {
            const char* krows = sbase + sb * 32 * ROWB;
            const char* vrows = sbase + RBYTES + sb * 32 * ROWB;
            f32x16 s = {}, dp = negd;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8 ka = *reinterpret_cast<const bf16x8*>(krows + fo.row[ks]);
                s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[ks], s, 0, 0, 0);
            }
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8 va = *reinterpret_cast<const bf16x8*>(vrows + fo.row[ks]);
                dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, gf[ks], dp, 0, 0, 0);
            }
            bf16x8 db16[2];
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[e], c, -lse2));
                float ds = p * dp[e];  // dp holds dP - D
                if constexpr (MASKED) {
                    const int key = sb * 32 + 8 * (e >> 2) + 4 * hf + (e & 3);
                    ds = key < lim ? ds : 0.f;
                }
                db16[e >> 3][e & 7] = (__bf16)ds;
            }
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const char* kt = krows + t * 16 * ROWB;
#pragma unroll
                for (int d = 0; d < DB; ++d) {
                    const bf16x8 ka = read_tr8(kt + fo.tr[0][d], kt + fo.tr[1][d]);
                    dq[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, db16[t], dq[d], 0, 0, 0);
                }
            }
        }
    };

    if (nst > 0) {
        load_stage(0, 0);
        int buf = 0;
        auto next = [&](int32_t j) {
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
            __syncthreads();
            if (j + 1 < nst) load_stage(j + 1, buf ^ 1);
        };
        int32_t j = 0;
        const int32_t nfree = min(jmask, nst - 1);
        for (; j < nfree; ++j) {
            next(j);
            stage(j, buf, std::false_type{});
            buf ^= 1;
        }
        for (; j < nst; ++j) {
            next(j);
            stage(j, buf, std::true_type{});
            buf ^= 1;
        }
    }

    store_rows_t<D>((char*)a.dq + 2 * (q_tok * a.dq_row + h * a.dq_head), a.dq_row, wrows, lane, dq, a.scale);
}

// Tile shapes: dK/dV 4 waves x 32 keys, 64 query rows per stage; dQ 4 waves
// x 32 rows, 64 keys per stage.
constexpr int kNW = 4, kBQ = 64, kBK = 64;

template <int D, int MINB>
hipError_t launch_dkdv(const AvfBwdArgs& a, hipStream_t stream) {
    if (a.causal)
        hipLaunchKernelGGL((avf_bwd_dkdv_kernel<D, kNW, kBQ, true, MINB>), dim3((uint32_t)a.num_tiles), dim3(kNW * 64),
                           0, stream, a);
    else
        hipLaunchKernelGGL((avf_bwd_dkdv_kernel<D, kNW, kBQ, false, MINB>), dim3((uint32_t)a.num_tiles),
                           dim3(kNW * 64), 0, stream, a);
    return hipGetLastError();
}

}  // namespace
